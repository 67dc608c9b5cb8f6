"""ctypes binding of libcausal_attn.so (argument marshalling only).

Every step of the attention path runs in the library's HIP kernels; this module only checks
tensor shapes/dtypes, allocates outputs and workspaces with PyTorch (device memory) and
passes raw pointers plus the current HIP stream to the C ABI declared in include/attn.h.
If the library is missing, every entry point raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import functools
import os
from dataclasses import dataclass

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libcausal_attn.so")

ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EWORKSPACE, ATTN_ELAUNCH = 0, -1, -2, -3, -4
ATTN_ESCRATCH = -5
DECODE_NOALLOC_MAX_BYTES = 8 << 20
ATTN_F32, ATTN_BF16 = 0, 1

EXPORTED = [
    "attn_fwd_workspace_bytes", "attn_bwd_workspace_bytes", "attn_decode_workspace_bytes",
    "attn_fwd_packed_workspace_bytes", "attn_bwd_packed_workspace_bytes",
    "attn_check_cfg", "attn_check_decode_cfg", "attn_check_extend_cfg", "attn_fwd", "attn_bwd",
    "attn_fwd_packed", "attn_bwd_packed", "attn_decode", "attn_extend", "attn_status_str",
    "attn_trace_enable", "attn_trace_read", "attn_dropout_mask_bytes", "attn_dropout_mask",
    "attn_fwd_dropout", "attn_bwd_dropout", "attn_decode_leftpad", "attn_extend_leftpad",
    "attn_bwd_khat", "attn_device_info", "attn_decode_ticket_bytes", "attn_decode_noalloc",
    "attn_bwd_split", "attn_bwd_split_workspace_bytes",
]


class AttnCfg(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32), ("window", ctypes.c_int32),
                ("softcap", ctypes.c_float), ("scale", ctypes.c_float), ("rope", ctypes.c_int32),
                ("rope_base", ctypes.c_float), ("qk_norm", ctypes.c_int32),
                ("norm_eps", ctypes.c_float), ("dtype", ctypes.c_int32)]


class AttnDecodeCfg(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("D", ctypes.c_int32), ("Lmax", ctypes.c_int32), ("softcap", ctypes.c_float),
                ("scale", ctypes.c_float), ("rope", ctypes.c_int32), ("rope_base", ctypes.c_float),
                ("qk_norm", ctypes.c_int32), ("norm_eps", ctypes.c_float),
                ("split_len", ctypes.c_int32)]


class AttnExtendCfg(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("S", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32), ("Lmax", ctypes.c_int32),
                ("window", ctypes.c_int32), ("softcap", ctypes.c_float),
                ("scale", ctypes.c_float), ("rope", ctypes.c_int32), ("rope_base", ctypes.c_float),
                ("qk_norm", ctypes.c_int32), ("norm_eps", ctypes.c_float)]


class AttnTraceEntry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double)]


class AttnDeviceInfo(ctypes.Structure):
    _fields_ = [("compute_units", ctypes.c_int32), ("clock_khz", ctypes.c_int32),
                ("mem_clock_khz", ctypes.c_int32), ("mem_bus_bits", ctypes.c_int32),
                ("bf16_dense_tflops", ctypes.c_double)]


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} ({status})")
        self.status = status


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libcausal_attn.so once; raise if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m causal_attention_02_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        cfgp, dcfgp = ctypes.POINTER(AttnCfg), ctypes.POINTER(AttnDecodeCfg)
        ecfgp = ctypes.POINTER(AttnExtendCfg)
        L.attn_fwd_workspace_bytes.argtypes = [cfgp]
        L.attn_fwd_workspace_bytes.restype = sz
        L.attn_bwd_workspace_bytes.argtypes = [cfgp]
        L.attn_bwd_workspace_bytes.restype = sz
        L.attn_fwd_packed_workspace_bytes.argtypes = [cfgp]
        L.attn_fwd_packed_workspace_bytes.restype = sz
        L.attn_bwd_packed_workspace_bytes.argtypes = [cfgp]
        L.attn_bwd_packed_workspace_bytes.restype = sz
        L.attn_decode_workspace_bytes.argtypes = [dcfgp]
        L.attn_decode_workspace_bytes.restype = sz
        L.attn_decode_ticket_bytes.argtypes = [dcfgp]
        L.attn_decode_ticket_bytes.restype = sz
        L.attn_check_cfg.argtypes = [cfgp, ctypes.c_int]
        L.attn_check_cfg.restype = ctypes.c_int
        L.attn_check_decode_cfg.argtypes = [dcfgp]
        L.attn_check_decode_cfg.restype = ctypes.c_int
        L.attn_check_extend_cfg.argtypes = [ecfgp]
        L.attn_check_extend_cfg.restype = ctypes.c_int
        L.attn_fwd.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.attn_fwd.restype = ctypes.c_int
        L.attn_bwd.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.attn_bwd_khat.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.attn_bwd_khat.restype = ctypes.c_int
        L.attn_bwd_split.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.attn_bwd_split.restype = ctypes.c_int
        L.attn_bwd_split_workspace_bytes.argtypes = [cfgp]
        L.attn_bwd_split_workspace_bytes.restype = sz
        L.attn_bwd.restype = ctypes.c_int
        L.attn_fwd_packed.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.attn_fwd_packed.restype = ctypes.c_int
        L.attn_bwd_packed.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.attn_bwd_packed.restype = ctypes.c_int
        f32, u64 = ctypes.c_float, ctypes.c_uint64
        L.attn_dropout_mask_bytes.argtypes = [cfgp]
        L.attn_dropout_mask_bytes.restype = sz
        L.attn_dropout_mask.argtypes = [cfgp, f32, u64, u64, vp, sz, vp]
        L.attn_dropout_mask.restype = ctypes.c_int
        L.attn_fwd_dropout.argtypes = [cfgp, vp, vp, vp, f32, vp, sz, vp, vp, vp, sz, vp]
        L.attn_fwd_dropout.restype = ctypes.c_int
        L.attn_bwd_dropout.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, f32, vp, sz, vp, vp, vp, vp,
                                       sz, vp]
        L.attn_bwd_dropout.restype = ctypes.c_int
        L.attn_decode.argtypes = [dcfgp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.attn_decode.restype = ctypes.c_int
        L.attn_decode_noalloc.argtypes = [dcfgp, vp, vp, vp, vp, vp, vp]
        L.attn_decode_noalloc.restype = ctypes.c_int
        L.attn_extend.argtypes = [ecfgp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.attn_extend.restype = ctypes.c_int
        L.attn_decode_leftpad.argtypes = [dcfgp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.attn_decode_leftpad.restype = ctypes.c_int
        L.attn_extend_leftpad.argtypes = [ecfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.attn_extend_leftpad.restype = ctypes.c_int
        L.attn_status_str.argtypes = [ctypes.c_int]
        L.attn_status_str.restype = ctypes.c_char_p
        L.attn_device_info.argtypes = [ctypes.c_int, ctypes.POINTER(AttnDeviceInfo)]
        L.attn_device_info.restype = ctypes.c_int
        L.attn_trace_enable.argtypes = [ctypes.c_int]
        L.attn_trace_enable.restype = ctypes.c_int
        L.attn_trace_read.argtypes = [ctypes.POINTER(AttnTraceEntry), ctypes.c_int]
        L.attn_trace_read.restype = ctypes.c_int
        _LIB = L
    return _LIB


def status_str(status: int) -> str:
    return lib().attn_status_str(int(status)).decode()


def _check(status: int, what: str):
    if status != ATTN_OK:
        raise AttnError(status, what)


@dataclass
class AttnOptions:
    """Variant flags shared by forward and backward (see attn_cfg in include/attn.h)."""
    window: int = 0
    softcap: float = 0.0
    scale: float = 0.0
    rope: bool = False
    rope_base: float = 10000.0
    qk_norm: bool = False
    norm_eps: float = 1e-6


def make_cfg(B, T, Hq, Hkv, D, opts: AttnOptions, dtype: int) -> AttnCfg:
    return AttnCfg(B, T, Hq, Hkv, D, int(opts.window), float(opts.softcap), float(opts.scale),
                   int(bool(opts.rope)), float(opts.rope_base), int(bool(opts.qk_norm)),
                   float(opts.norm_eps), int(dtype))


def make_decode_cfg(B, Hq, Hkv, D, Lmax, opts: AttnOptions, split_len: int = 0) -> AttnDecodeCfg:
    return AttnDecodeCfg(B, Hq, Hkv, D, Lmax, float(opts.softcap), float(opts.scale),
                         int(bool(opts.rope)), float(opts.rope_base), int(bool(opts.qk_norm)),
                         float(opts.norm_eps), int(split_len))


def make_extend_cfg(B, S, Hq, Hkv, D, Lmax, opts: AttnOptions) -> AttnExtendCfg:
    return AttnExtendCfg(B, S, Hq, Hkv, D, Lmax, int(opts.window), float(opts.softcap),
                         float(opts.scale), int(bool(opts.rope)), float(opts.rope_base),
                         int(bool(opts.qk_norm)), float(opts.norm_eps))


# ---------------------------------------------------------------------------------------------
# torch-facing wrappers
# ---------------------------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None and t.numel() > 0 else 0)


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(fn):
    """Run a wrapper with `stream` (when given) as torch's current stream, so that the outputs
    and the workspace it allocates belong to the stream the kernels are enqueued on.  The
    caching allocator then reuses a freed workspace block only in that stream's order, after
    the kernels that read it.  Buffers the caller passes in stay the caller's to order."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, stream=None, **kw)
        with _torch().cuda.stream(stream):
            return fn(*args, stream=stream, **kw)
    return wrapper


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t, shape, dtype, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: must be a contiguous GPU tensor")


def _workspace(nbytes, device, ws):
    torch = _torch()
    if nbytes == 0:
        return None
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace of {ws.numel() * ws.element_size()} bytes < {nbytes} needed")
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def decode_workspace(B, Hq, Hkv, D, Lmax, opts: AttnOptions | None = None, split_len: int = 0,
                     device="cuda"):
    """A zero-filled decode workspace for these sizes (its ticket counters must start at zero;
    every attn_decode call leaves them zero, so it can be reused by later calls)."""
    torch = _torch()
    cfg = make_decode_cfg(B, Hq, Hkv, D, Lmax, opts or AttnOptions(), split_len)
    _check(lib().attn_check_decode_cfg(ctypes.byref(cfg)), "decode_workspace")
    n = int(lib().attn_decode_workspace_bytes(ctypes.byref(cfg)))
    return torch.zeros(max(n, 1), dtype=torch.uint8, device=device)


def fwd_workspace_bytes(B, T, Hq, Hkv, D, opts: AttnOptions, dtype=ATTN_BF16) -> int:
    return int(lib().attn_fwd_workspace_bytes(ctypes.byref(make_cfg(B, T, Hq, Hkv, D, opts, dtype))))


def bwd_workspace_bytes(B, T, Hq, Hkv, D, opts: AttnOptions) -> int:
    return int(lib().attn_bwd_workspace_bytes(ctypes.byref(make_cfg(B, T, Hq, Hkv, D, opts, ATTN_BF16))))


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def dropout_mask_bytes(B, T, Hq, Hkv, D, opts: AttnOptions | None = None) -> int:
    cfg = make_cfg(B, T, Hq, Hkv, D, opts or AttnOptions(), ATTN_BF16)
    return int(lib().attn_dropout_mask_bytes(ctypes.byref(cfg)))


@_on_stream
def attn_dropout_mask(q, k, p: float, seed: int, offset: int = 0, opts: AttnOptions | None = None,
                      *, out=None, stream=None):
    """Keep mask (uint8 buffer of dropout_mask_bytes) for dropout rate p on the attention weights
    of q [B,Hq,T,D] against k [B,Hkv,T,D]; pass it with the same p to attn_fwd / attn_bwd."""
    torch = _torch()
    opts = opts or AttnOptions()
    B, Hq, T, D = q.shape
    cfg = make_cfg(B, T, Hq, k.shape[1], D, opts, ATTN_BF16)
    _check(lib().attn_check_cfg(ctypes.byref(cfg), 0), "attn_dropout_mask")
    n = int(lib().attn_dropout_mask_bytes(ctypes.byref(cfg)))
    m = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device) if out is None else out
    if _nbytes(m) < n or not m.is_cuda or not m.is_contiguous():
        raise ValueError(f"dropout mask: need a contiguous GPU buffer of {n} bytes")
    st = lib().attn_dropout_mask(ctypes.byref(cfg), ctypes.c_float(p), ctypes.c_uint64(seed),
                                 ctypes.c_uint64(offset), _ptr(m), ctypes.c_size_t(_nbytes(m)),
                                 _stream(stream))
    _check(st, "attn_dropout_mask")
    return m


@_on_stream
def attn_fwd(q, k, v, opts: AttnOptions | None = None, *, out=None, lse=None, workspace=None,
             stream=None, segment_ids=None, dropout_p=0.0, dropout_mask=None):
    """Forward: q [B,Hq,T,D], k/v [B,Hkv,T,D] (bf16 or fp32) -> (o, lse fp32 [B,Hq,T]).

    segment_ids (int32 [B,T], optional): packed rows; attention stays inside each run of equal
    ids (bf16 only).  dropout_mask (from attn_dropout_mask with rate dropout_p, optional):
    dropout on the attention weights (bf16 only)."""
    torch = _torch()
    opts = opts or AttnOptions()
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    dt = _dtype_code(q)
    _need(q, (B, Hq, T, D), q.dtype, "q")
    _need(k, (B, Hkv, T, D), q.dtype, "k")
    _need(v, (B, Hkv, T, D), q.dtype, "v")
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(o, q.shape, q.dtype, "out")
    _need(lse_t, (B, Hq, T), torch.float32, "lse")
    cfg = make_cfg(B, T, Hq, Hkv, D, opts, dt)
    st = lib().attn_check_cfg(ctypes.byref(cfg), 0)
    _check(st, "attn_fwd")
    if dropout_mask is not None:
        if segment_ids is not None:
            raise ValueError("dropout with segment ids is not supported")
        ws = _workspace(int(lib().attn_fwd_workspace_bytes(ctypes.byref(cfg))), q.device, workspace)
        st = lib().attn_fwd_dropout(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v),
                                    ctypes.c_float(dropout_p), _ptr(dropout_mask),
                                    ctypes.c_size_t(_nbytes(dropout_mask)), _ptr(o), _ptr(lse_t),
                                    _ptr(ws), ctypes.c_size_t(_nbytes(ws)), _stream(stream))
        _check(st, "attn_fwd_dropout")
        return o, lse_t
    if segment_ids is not None:
        _need(segment_ids, (B, T), torch.int32, "segment_ids")
        ws = _workspace(int(lib().attn_fwd_packed_workspace_bytes(ctypes.byref(cfg))), q.device,
                        workspace)
        st = lib().attn_fwd_packed(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(segment_ids),
                                   _ptr(o), _ptr(lse_t), _ptr(ws),
                                   ctypes.c_size_t(0 if ws is None else ws.numel() * ws.element_size()),
                                   _stream(stream))
        _check(st, "attn_fwd_packed")
        return o, lse_t
    ws = _workspace(int(lib().attn_fwd_workspace_bytes(ctypes.byref(cfg))), q.device, workspace)
    st = lib().attn_fwd(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), _ptr(ws),
                        ctypes.c_size_t(0 if ws is None else ws.numel() * ws.element_size()),
                        _stream(stream))
    _check(st, "attn_fwd")
    return o, lse_t


@_on_stream
def attn_bwd(q, k, v, o, dO, lse, opts: AttnOptions | None = None, *, dq=None, dk=None, dv=None,
             workspace=None, stream=None, segment_ids=None, dropout_p=0.0, dropout_mask=None,
             khat=None, split=False):
    """Backward (bf16): returns (dq, dk, dv) with respect to the raw q, k, v (packed rows with
    segment_ids, dropout with the forward's dropout_mask and dropout_p, as in attn_fwd).

    khat (optional): the forward's workspace (or any buffer starting with k after RoPE /
    QK-norm, bf16 [B,Hkv,T,D]); the backward then skips its own pass over k.
    split: attn_bwd_split (dS stored by the dK/dV pass, dQ from it); plain rows only."""
    torch = _torch()
    opts = opts or AttnOptions()
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    bf = torch.bfloat16
    for t, shp, name in ((q, (B, Hq, T, D), "q"), (k, (B, Hkv, T, D), "k"), (v, (B, Hkv, T, D), "v"),
                         (o, (B, Hq, T, D), "o"), (dO, (B, Hq, T, D), "dO")):
        _need(t, shp, bf, name)
    _need(lse, (B, Hq, T), torch.float32, "lse")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, q.shape, bf, "dq")
    _need(dk, k.shape, bf, "dk")
    _need(dv, v.shape, bf, "dv")
    cfg = make_cfg(B, T, Hq, Hkv, D, opts, ATTN_BF16)
    _check(lib().attn_check_cfg(ctypes.byref(cfg), 1), "attn_bwd")
    if split:
        if segment_ids is not None or dropout_mask is not None or khat is not None:
            raise ValueError("the split backward takes plain rows only")
        ws = _workspace(int(lib().attn_bwd_split_workspace_bytes(ctypes.byref(cfg))), q.device,
                        workspace)
        st = lib().attn_bwd_split(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO),
                                  _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                                  ctypes.c_size_t(_nbytes(ws)), _stream(stream))
        _check(st, "attn_bwd_split")
        return dq, dk, dv
    if khat is not None:
        if segment_ids is not None or dropout_mask is not None:
            raise ValueError("khat is taken by the plain backward only")
        if _nbytes(khat) < B * Hkv * T * D * 2 or not khat.is_cuda or not khat.is_contiguous():
            raise ValueError("khat: need a contiguous GPU buffer of k's bf16 size")
        ws = _workspace(int(lib().attn_bwd_workspace_bytes(ctypes.byref(cfg))), q.device, workspace)
        st = lib().attn_bwd_khat(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO),
                                 _ptr(lse), _ptr(khat), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                                 ctypes.c_size_t(_nbytes(ws)), _stream(stream))
        _check(st, "attn_bwd_khat")
        return dq, dk, dv
    if dropout_mask is not None:
        if segment_ids is not None:
            raise ValueError("dropout with segment ids is not supported")
        ws = _workspace(int(lib().attn_bwd_workspace_bytes(ctypes.byref(cfg))), q.device, workspace)
        st = lib().attn_bwd_dropout(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO),
                                    _ptr(lse), ctypes.c_float(dropout_p), _ptr(dropout_mask),
                                    ctypes.c_size_t(_nbytes(dropout_mask)), _ptr(dq), _ptr(dk),
                                    _ptr(dv), _ptr(ws), ctypes.c_size_t(_nbytes(ws)),
                                    _stream(stream))
        _check(st, "attn_bwd_dropout")
        return dq, dk, dv
    if segment_ids is not None:
        _need(segment_ids, (B, T), torch.int32, "segment_ids")
        ws = _workspace(int(lib().attn_bwd_packed_workspace_bytes(ctypes.byref(cfg))), q.device,
                        workspace)
        st = lib().attn_bwd_packed(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO),
                                   _ptr(lse), _ptr(segment_ids), _ptr(dq), _ptr(dk), _ptr(dv),
                                   _ptr(ws),
                                   ctypes.c_size_t(0 if ws is None else ws.numel() * ws.element_size()),
                                   _stream(stream))
        _check(st, "attn_bwd_packed")
        return dq, dk, dv
    ws = _workspace(int(lib().attn_bwd_workspace_bytes(ctypes.byref(cfg))), q.device, workspace)
    st = lib().attn_bwd(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse),
                        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                        ctypes.c_size_t(0 if ws is None else ws.numel() * ws.element_size()),
                        _stream(stream))
    _check(st, "attn_bwd")
    return dq, dk, dv


@_on_stream
def attn_decode(q, k_cache, v_cache, cache_len, opts: AttnOptions | None = None, *, split_len=0,
                out=None, workspace=None, stream=None, cache_start=None):
    """Decode (bf16): q [B,Hq,D], caches [B,Hkv,Lmax,D], cache_len int32 [B] -> o [B,Hq,D].

    cache_start (int32 [B], optional): left-padded batches, rows below it are padding."""
    torch = _torch()
    opts = opts or AttnOptions()
    B, Hq, D = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    bf = torch.bfloat16
    _need(q, (B, Hq, D), bf, "q")
    _need(k_cache, (B, Hkv, Lmax, D), bf, "k_cache")
    _need(v_cache, (B, Hkv, Lmax, D), bf, "v_cache")
    _need(cache_len, (B,), torch.int32, "cache_len")
    o = torch.empty_like(q) if out is None else out
    _need(o, q.shape, bf, "out")
    cfg = make_decode_cfg(B, Hq, Hkv, D, Lmax, opts, split_len)
    _check(lib().attn_check_decode_cfg(ctypes.byref(cfg)), "attn_decode")
    nws = int(lib().attn_decode_workspace_bytes(ctypes.byref(cfg)))
    if workspace is None:
        # The ticket counters at its start must be zero (a caller-owned workspace keeps them
        # zero from call to call; see decode_workspace).
        ws = torch.zeros(max(nws, 1), dtype=torch.uint8, device=q.device)
    else:
        ws = _workspace(nws, q.device, workspace)
    if cache_start is not None:
        _need(cache_start, (B,), torch.int32, "cache_start")
        st = lib().attn_decode_leftpad(ctypes.byref(cfg), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(cache_start), _ptr(cache_len), _ptr(o), _ptr(ws),
                                       ctypes.c_size_t(_nbytes(ws)), _stream(stream))
        _check(st, "attn_decode_leftpad")
        return o
    st = lib().attn_decode(ctypes.byref(cfg), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len),
                           _ptr(o), _ptr(ws),
                           ctypes.c_size_t(0 if ws is None else ws.numel() * ws.element_size()),
                           _stream(stream))
    _check(st, "attn_decode")
    return o


def attn_decode_noalloc(q, k_cache, v_cache, cache_len, out, opts: AttnOptions | None = None, *,
                        split_len=0, stream=None):
    """attn_decode into a caller-given `out` with the library's static scratch as workspace:
    nothing is allocated (no torch allocation either).  Same shapes as attn_decode."""
    torch = _torch()
    opts = opts or AttnOptions()
    B, Hq, D = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    bf = torch.bfloat16
    _need(q, (B, Hq, D), bf, "q")
    _need(k_cache, (B, Hkv, Lmax, D), bf, "k_cache")
    _need(v_cache, (B, Hkv, Lmax, D), bf, "v_cache")
    _need(cache_len, (B,), torch.int32, "cache_len")
    _need(out, q.shape, bf, "out")
    cfg = make_decode_cfg(B, Hq, Hkv, D, Lmax, opts, split_len)
    st = lib().attn_decode_noalloc(ctypes.byref(cfg), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(cache_len), _ptr(out), _stream(stream))
    _check(st, "attn_decode_noalloc")
    return out


@_on_stream
def attn_extend(q, k_new, v_new, k_cache, v_cache, cache_len, opts: AttnOptions | None = None, *,
                out=None, stream=None, cache_start=None):
    """S new tokens against a KV cache (bf16): q [B,Hq,S,D], k_new/v_new [B,Hkv,S,D], caches
    [B,Hkv,Lmax,D] (rows cache_len[b] .. cache_len[b]+S-1 are written), cache_len int32 [B]
    (not modified) -> o [B,Hq,S,D].  cache_start (int32 [B], optional): left-padded batches."""
    torch = _torch()
    opts = opts or AttnOptions()
    B, Hq, S, D = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    bf = torch.bfloat16
    _need(q, (B, Hq, S, D), bf, "q")
    _need(k_new, (B, Hkv, S, D), bf, "k_new")
    _need(v_new, (B, Hkv, S, D), bf, "v_new")
    _need(k_cache, (B, Hkv, Lmax, D), bf, "k_cache")
    _need(v_cache, (B, Hkv, Lmax, D), bf, "v_cache")
    _need(cache_len, (B,), torch.int32, "cache_len")
    o = torch.empty_like(q) if out is None else out
    _need(o, q.shape, bf, "out")
    cfg = make_extend_cfg(B, S, Hq, Hkv, D, Lmax, opts)
    if cache_start is not None:
        _need(cache_start, (B,), torch.int32, "cache_start")
        st = lib().attn_extend_leftpad(ctypes.byref(cfg), _ptr(q), _ptr(k_new), _ptr(v_new),
                                       _ptr(k_cache), _ptr(v_cache), _ptr(cache_start),
                                       _ptr(cache_len), _ptr(o), _stream(stream))
        _check(st, "attn_extend_leftpad")
        return o
    st = lib().attn_extend(ctypes.byref(cfg), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                           _ptr(v_cache), _ptr(cache_len), _ptr(o), _stream(stream))
    _check(st, "attn_extend")
    return o


def device_info(device: int = 0) -> dict:
    """Compute units, clocks, memory bus width and the dense bf16 MFMA peak of a HIP device."""
    info = AttnDeviceInfo()
    _check(lib().attn_device_info(int(device), ctypes.byref(info)), "attn_device_info")
    return {f: getattr(info, f) for f, _ in AttnDeviceInfo._fields_}


def trace_enable(on: bool = True):
    _check(lib().attn_trace_enable(1 if on else 0), "attn_trace_enable")


def trace_read() -> dict:
    """{kernel name: (launches, total_ms)} recorded since trace_enable(True)."""
    L = lib()
    n = L.attn_trace_read(None, 0)
    if n < 0:
        raise AttnError(n, "attn_trace_read")
    buf = (AttnTraceEntry * max(n, 1))()
    n = L.attn_trace_read(buf, n)
    if n < 0:
        raise AttnError(n, "attn_trace_read")
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(n)}
