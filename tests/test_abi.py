"""The C ABI library loads, exports every symbol include/attn.h declares, and rejects bad
arguments on the host before anything is enqueued.  No GPU is needed: every call here
either touches no HIP API at all or returns before the first one."""
import ctypes
import os
import re

import pytest

from causal_attention_02_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return bd.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert sorted(bd.EXPORTED) == names


def cfg(**kw):
    base = dict(B=2, T=128, Hq=8, Hkv=4, D=96, opts=bd.AttnOptions(softcap=50.0, rope=True,
                                                                     qk_norm=True),
                dtype=bd.ATTN_BF16)
    base.update(kw)
    return bd.make_cfg(base["B"], base["T"], base["Hq"], base["Hkv"], base["D"], base["opts"],
                       base["dtype"])


def test_config_validation(L):
    ok = cfg()
    assert L.attn_check_cfg(ctypes.byref(ok), 0) == bd.ATTN_OK
    assert L.attn_check_cfg(ctypes.byref(ok), 1) == bd.ATTN_OK
    assert L.attn_check_cfg(None, 0) == bd.ATTN_EINVAL
    bad = [cfg(Hq=6, Hkv=4), cfg(B=-1), cfg(T=-3), cfg(Hkv=0),
           cfg(opts=bd.AttnOptions(window=-1)), cfg(opts=bd.AttnOptions(softcap=-1.0)),
           cfg(opts=bd.AttnOptions(softcap=float("nan"))), cfg(opts=bd.AttnOptions(scale=float("inf"))),
           cfg(opts=bd.AttnOptions(rope=True, rope_base=0.0)),
           cfg(opts=bd.AttnOptions(qk_norm=True, norm_eps=0.0)), cfg(dtype=7), cfg(D=0)]
    for c in bad:
        assert L.attn_check_cfg(ctypes.byref(c), 0) == bd.ATTN_EINVAL
    for D in (16, 48, 80, 256):
        assert L.attn_check_cfg(ctypes.byref(cfg(D=D)), 0) == bd.ATTN_EUNSUPPORTED
    f32 = cfg(dtype=bd.ATTN_F32)
    assert L.attn_check_cfg(ctypes.byref(f32), 0) == bd.ATTN_OK
    assert L.attn_check_cfg(ctypes.byref(f32), 1) == bd.ATTN_EUNSUPPORTED


def test_workspace_sizes(L):
    c = cfg(B=16, T=2048)
    rows = 16 * 8 * 2048
    q_elems, k_elems = rows * 96, 16 * 4 * 2048 * 96
    assert L.attn_fwd_workspace_bytes(ctypes.byref(c)) == k_elems * 2
    assert L.attn_fwd_workspace_bytes(ctypes.byref(cfg(B=16, T=2048, dtype=bd.ATTN_F32))) == \
        (q_elems + k_elems) * 4
    assert L.attn_bwd_workspace_bytes(ctypes.byref(c)) == 2 * rows * 4 + (q_elems + k_elems) * 2
    plain = cfg(B=16, T=2048, opts=bd.AttnOptions())
    assert L.attn_fwd_workspace_bytes(ctypes.byref(plain)) == 0
    assert L.attn_bwd_workspace_bytes(ctypes.byref(plain)) == 2 * rows * 4
    # Split backward: the same regions, then the dS fragments: per (b, h) the triangle of 64
    # 32-query blocks x their 16-key blocks, 64 * 65 fragments of 1 KB.
    ds = 16 * 8 * 64 * 65 * 1024
    assert L.attn_bwd_split_workspace_bytes(ctypes.byref(c)) == \
        L.attn_bwd_workspace_bytes(ctypes.byref(c)) + ds
    # A window of 512 keeps a band: blocks i >= 16 span 33 or 34 key blocks, stride 34.
    win = cfg(B=16, T=2048, opts=bd.AttnOptions(window=512))
    assert L.attn_bwd_split_workspace_bytes(ctypes.byref(win)) == \
        L.attn_bwd_workspace_bytes(ctypes.byref(win)) + 16 * 8 * 64 * 34 * 1024
    assert L.attn_fwd_workspace_bytes(ctypes.byref(cfg(Hq=5))) == 0  # invalid -> 0
    # Decode: [tickets, one uint32 per (b, kv head, head subset)][partials B*Hq*nsplit*(D+2)
    # f32], each region 256-byte aligned.
    al = lambda x: (x + 255) // 256 * 256
    # 64 x 4 units fill the GPU: one chunk per cache.
    d = bd.make_decode_cfg(64, 8, 4, 96, 2048, bd.AttnOptions(softcap=50.0, rope=True))
    assert L.attn_decode_ticket_bytes(ctypes.byref(d)) == al(64 * 4 * 4)
    assert L.attn_decode_workspace_bytes(ctypes.byref(d)) == al(64 * 4 * 4) + 64 * 8 * 1 * 98 * 4
    # One sequence, 4 units: 64-row chunks (64 over a 4096-row cache).
    d = bd.make_decode_cfg(1, 8, 4, 96, 4096, bd.AttnOptions())
    assert L.attn_decode_workspace_bytes(ctypes.byref(d)) == al(4 * 4) + 1 * 8 * 64 * 98 * 4
    # 16 sequences x 4 units: 64 units, chunks of ceil(2048 * 64 / 1024) = 128 rows.
    d = bd.make_decode_cfg(16, 8, 4, 96, 2048, bd.AttnOptions())
    assert L.attn_decode_workspace_bytes(ctypes.byref(d)) == al(64 * 4) + 16 * 8 * 16 * 98 * 4
    # A 256-row cache of one sequence, 12 units: 64-row chunks, so 48 workgroups.
    d = bd.make_decode_cfg(1, 12, 12, 64, 256, bd.AttnOptions())
    assert L.attn_decode_workspace_bytes(ctypes.byref(d)) == al(12 * 4) + al(1 * 12 * 4 * 66 * 4)
    d = bd.make_decode_cfg(64, 8, 4, 96, 2048, bd.AttnOptions(), split_len=128)
    assert L.attn_decode_workspace_bytes(ctypes.byref(d)) == al(64 * 4 * 4) + 64 * 8 * 16 * 98 * 4
    assert L.attn_decode_ticket_bytes(None) == 0


def test_packed_workspace_and_validation(L):
    c = cfg(B=16, T=2048)
    rows = 16 * 2048
    extra = 2 * ((rows * 4 + 255) // 256 * 256)
    assert L.attn_fwd_packed_workspace_bytes(ctypes.byref(c)) == \
        L.attn_fwd_workspace_bytes(ctypes.byref(c)) + extra
    assert L.attn_bwd_packed_workspace_bytes(ctypes.byref(c)) == \
        L.attn_bwd_workspace_bytes(ctypes.byref(c)) + extra
    fake, null, s = ctypes.c_void_p(0x1000), ctypes.c_void_p(0), ctypes.c_void_p(0)
    small = cfg()
    # segment ids are required when there is work
    assert L.attn_fwd_packed(ctypes.byref(small), fake, fake, fake, null, fake, fake, fake,
                             1 << 40, s) == -1
    assert L.attn_bwd_packed(ctypes.byref(small), fake, fake, fake, fake, fake, fake, null, fake,
                             fake, fake, fake, 1 << 40, s) == -1
    f32 = cfg(dtype=bd.ATTN_F32)
    assert L.attn_fwd_packed(ctypes.byref(f32), fake, fake, fake, fake, fake, fake, fake,
                             1 << 40, s) == -2
    # the packed workspace is checked against the packed figure
    need = L.attn_fwd_packed_workspace_bytes(ctypes.byref(small))
    assert L.attn_fwd_packed(ctypes.byref(small), fake, fake, fake, fake, fake, fake, fake,
                             need - 1, s) == -3
    empty = cfg(T=0)
    assert L.attn_fwd_packed(ctypes.byref(empty), null, null, null, null, null, null, null, 0, s) == 0


def test_dropout_mask_bytes_and_validation(L):
    c = cfg(B=16, T=2048)
    pitch = 2 * ((2048 + 63) // 64)
    half = (16 * 8 * 2048 * pitch * 4 + 255) // 256 * 256
    assert L.attn_dropout_mask_bytes(ctypes.byref(c)) == 2 * half
    odd = cfg(B=3, T=65)  # two 64-column word pairs per row
    assert L.attn_dropout_mask_bytes(ctypes.byref(odd)) == \
        2 * ((3 * 8 * 65 * 4 * 4 + 255) // 256 * 256)
    fake, null, s = ctypes.c_void_p(0x1000), ctypes.c_void_p(0), ctypes.c_void_p(0)
    small = cfg()
    need = L.attn_dropout_mask_bytes(ctypes.byref(small))
    u64 = ctypes.c_uint64
    # rate out of range, missing or short mask: rejected before anything is enqueued
    for p in (-0.1, 1.0, 1.0 - 2.0 ** -18, float("nan"), float("inf")):
        assert L.attn_dropout_mask(ctypes.byref(small), p, u64(1), u64(0), fake, need, s) == -1
        assert L.attn_fwd_dropout(ctypes.byref(small), fake, fake, fake, p, fake, need, fake, fake,
                                  fake, 1 << 40, s) == -1
        assert L.attn_bwd_dropout(ctypes.byref(small), fake, fake, fake, fake, fake, fake, p, fake,
                                  need, fake, fake, fake, fake, 1 << 40, s) == -1
    assert L.attn_dropout_mask(ctypes.byref(small), 0.1, u64(1), u64(0), null, need, s) == -1
    assert L.attn_dropout_mask(ctypes.byref(small), 0.1, u64(1), u64(0), fake, need - 1, s) == -1
    assert L.attn_fwd_dropout(ctypes.byref(small), fake, fake, fake, 0.1, fake, need - 1, fake,
                              fake, fake, 1 << 40, s) == -1
    assert L.attn_bwd_dropout(ctypes.byref(small), fake, fake, fake, fake, fake, fake, 0.1, null,
                              need, fake, fake, fake, fake, 1 << 40, s) == -1
    f32 = cfg(dtype=bd.ATTN_F32)
    assert L.attn_fwd_dropout(ctypes.byref(f32), fake, fake, fake, 0.1, fake, 1 << 40, fake, fake,
                              fake, 1 << 40, s) == -2
    empty = cfg(T=0)
    assert L.attn_dropout_mask_bytes(ctypes.byref(empty)) == 0
    assert L.attn_dropout_mask(ctypes.byref(empty), 0.1, u64(1), u64(0), null, 0, s) == 0
    assert L.attn_fwd_dropout(ctypes.byref(empty), null, null, null, 0.1, null, 0, null, null,
                              null, 0, s) == 0


def test_leftpad_entry_points_validation(L):
    fake, null, s = ctypes.c_void_p(0x1000), ctypes.c_void_p(0), ctypes.c_void_p(0)
    d = bd.make_decode_cfg(4, 8, 4, 96, 256, bd.AttnOptions(softcap=50.0, rope=True))
    need = L.attn_decode_workspace_bytes(ctypes.byref(d))
    # cache_start is required when there is work; the rest is checked as for attn_decode
    assert L.attn_decode_leftpad(ctypes.byref(d), fake, fake, fake, null, fake, fake, fake, need,
                                 s) == -1
    assert L.attn_decode_leftpad(ctypes.byref(d), fake, fake, fake, fake, null, fake, fake, need,
                                 s) == -1
    assert L.attn_decode_leftpad(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake,
                                 need - 1, s) == -3
    e = bd.make_extend_cfg(4, 16, 8, 4, 96, 256, bd.AttnOptions(rope=True))
    assert L.attn_extend_leftpad(ctypes.byref(e), fake, fake, fake, fake, fake, null, fake, fake,
                                 s) == -1
    assert L.attn_extend_leftpad(ctypes.byref(e), fake, fake, fake, fake, fake, fake, null, fake,
                                 s) == -1
    bad = bd.make_extend_cfg(4, 16, 8, 3, 96, 256, bd.AttnOptions())
    assert L.attn_extend_leftpad(ctypes.byref(bad), fake, fake, fake, fake, fake, fake, fake,
                                 fake, s) == -1
    nothing = bd.make_decode_cfg(0, 8, 4, 96, 256, bd.AttnOptions())
    assert L.attn_decode_leftpad(ctypes.byref(nothing), null, null, null, null, null, null, null,
                                 0, s) == 0
    e0 = bd.make_extend_cfg(4, 0, 8, 4, 96, 256, bd.AttnOptions())
    assert L.attn_extend_leftpad(ctypes.byref(e0), null, null, null, null, null, null, null, null,
                                 s) == 0


def test_bwd_khat_validation(L):
    fake, null, s = ctypes.c_void_p(0x1000), ctypes.c_void_p(0), ctypes.c_void_p(0)
    c = cfg()  # RoPE and QK-norm on: khat is required
    need = L.attn_bwd_workspace_bytes(ctypes.byref(c))
    assert L.attn_bwd_khat(ctypes.byref(c), fake, fake, fake, fake, fake, fake, null, fake, fake,
                           fake, fake, need, s) == -1
    assert L.attn_bwd_khat(ctypes.byref(c), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                           fake, fake, need - 1, s) == -3
    plain = cfg(opts=bd.AttnOptions())  # neither: khat unused, the usual checks apply
    assert L.attn_bwd_khat(ctypes.byref(plain), fake, fake, fake, fake, fake, fake, null, null,
                           fake, fake, fake, 1 << 40, s) == -1
    empty = cfg(T=0)
    assert L.attn_bwd_khat(ctypes.byref(empty), null, null, null, null, null, null, null, null,
                           null, null, null, 0, s) == 0


def test_decode_config_validation(L):
    o = bd.AttnOptions(softcap=50.0, rope=True)
    assert L.attn_check_decode_cfg(ctypes.byref(bd.make_decode_cfg(64, 8, 4, 96, 2048, o))) == 0
    assert L.attn_check_decode_cfg(ctypes.byref(bd.make_decode_cfg(64, 8, 3, 96, 2048, o))) == -1
    assert L.attn_check_decode_cfg(ctypes.byref(bd.make_decode_cfg(64, 8, 4, 96, -1, o))) == -1
    assert L.attn_check_decode_cfg(ctypes.byref(bd.make_decode_cfg(64, 8, 4, 96, 2048, o, 100))) == -1
    assert L.attn_check_decode_cfg(ctypes.byref(bd.make_decode_cfg(64, 8, 4, 80, 2048, o))) == -2


def test_extend_config_validation(L):
    o = bd.AttnOptions(softcap=50.0, rope=True, qk_norm=True)
    ok = bd.make_extend_cfg(4, 16, 8, 4, 96, 2048, o)
    assert L.attn_check_extend_cfg(ctypes.byref(ok)) == bd.ATTN_OK
    assert L.attn_check_extend_cfg(None) == bd.ATTN_EINVAL
    bad = [bd.make_extend_cfg(4, -1, 8, 4, 96, 2048, o), bd.make_extend_cfg(4, 16, 8, 3, 96, 2048, o),
           bd.make_extend_cfg(4, 16, 8, 4, 96, -1, o), bd.make_extend_cfg(-2, 16, 8, 4, 96, 64, o),
           bd.make_extend_cfg(4, 16, 8, 4, 96, 64, bd.AttnOptions(window=-3)),
           bd.make_extend_cfg(4, 16, 8, 4, 96, 64, bd.AttnOptions(qk_norm=True, norm_eps=0.0))]
    for c in bad:
        assert L.attn_check_extend_cfg(ctypes.byref(c)) == bd.ATTN_EINVAL
    assert L.attn_check_extend_cfg(ctypes.byref(bd.make_extend_cfg(4, 16, 8, 4, 80, 64, o))) == \
        bd.ATTN_EUNSUPPORTED
    fake, null, s = ctypes.c_void_p(0x1000), ctypes.c_void_p(0), ctypes.c_void_p(0)
    assert L.attn_extend(ctypes.byref(bad[1]), fake, fake, fake, fake, fake, fake, fake, s) == -1
    assert L.attn_extend(ctypes.byref(ok), fake, fake, fake, fake, fake, null, fake, s) == -1
    empty = bd.make_extend_cfg(4, 0, 8, 4, 96, 2048, o)
    assert L.attn_extend(ctypes.byref(empty), null, null, null, null, null, null, null, s) == 0


def test_entry_points_reject_before_launch(L):
    """Invalid configs, null pointers and short workspaces return an error status without
    any HIP call (this process has no GPU, so reaching one would fail differently)."""
    c = cfg()
    fake = ctypes.c_void_p(0x1000)
    null = ctypes.c_void_p(0)
    s = ctypes.c_void_p(0)
    bad = cfg(Hq=6, Hkv=4)
    assert L.attn_fwd(ctypes.byref(bad), fake, fake, fake, fake, fake, fake, 1 << 40, s) == -1
    assert L.attn_fwd(ctypes.byref(c), null, fake, fake, fake, fake, fake, 1 << 40, s) == -1
    assert L.attn_fwd(ctypes.byref(c), fake, fake, fake, fake, fake, null, 0, s) == -3
    assert L.attn_fwd(ctypes.byref(c), fake, fake, fake, fake, fake, fake, 16, s) == -3
    assert L.attn_bwd(ctypes.byref(c), fake, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                      16, s) == -3
    assert L.attn_bwd(ctypes.byref(c), fake, fake, fake, fake, null, fake, fake, fake, fake, fake,
                      1 << 40, s) == -1
    f32 = cfg(dtype=bd.ATTN_F32)
    assert L.attn_bwd(ctypes.byref(f32), fake, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                      1 << 40, s) == -2
    d = bd.make_decode_cfg(4, 8, 4, 96, 64, bd.AttnOptions())
    assert L.attn_decode(ctypes.byref(d), fake, fake, fake, fake, fake, null, 0, s) == -3
    assert L.attn_decode(ctypes.byref(d), fake, fake, fake, null, fake, fake, 1 << 40, s) == -1
    # Empty problems are valid and enqueue nothing.
    assert L.attn_fwd(ctypes.byref(cfg(T=0)), null, null, null, null, null, null, 0, s) == 0
    assert L.attn_bwd(ctypes.byref(cfg(B=0)), null, null, null, null, null, null, null, null, null,
                      null, 0, s) == 0
    d0 = bd.make_decode_cfg(0, 8, 4, 96, 64, bd.AttnOptions())
    assert L.attn_decode(ctypes.byref(d0), null, null, null, null, null, null, 0, s) == 0


def test_status_strings_and_trace(L):
    assert bd.status_str(0) == "ok"
    assert "workspace" in bd.status_str(-3)
    assert bd.status_str(12345) == "unknown status"
    bd.trace_enable(True)
    assert bd.trace_read() == {}
    bd.trace_enable(False)


def test_device_info_rejects_null(L):
    """Host-only: a null output is rejected before the runtime is asked anything."""
    assert L.attn_device_info(0, None) == bd.ATTN_EINVAL


def test_noalloc_decode_rejects_oversized_before_any_device_call(L):
    """The static-scratch decode checks its size on the host: a configuration needing more
    than the scratch returns ATTN_ESCRATCH (null pointers are never reached)."""
    d = bd.make_decode_cfg(64, 8, 4, 96, 8192, bd.AttnOptions(), split_len=64)
    assert L.attn_decode_workspace_bytes(ctypes.byref(d)) > bd.DECODE_NOALLOC_MAX_BYTES
    assert L.attn_decode_noalloc(ctypes.byref(d), None, None, None, None, None, None) == \
        bd.ATTN_ESCRATCH
    assert L.attn_decode_noalloc(None, None, None, None, None, None, None) == bd.ATTN_EINVAL
