"""Plain fp64 CPU oracle for causal self-attention: forward, backward and KV-cache decode.

TEST INFRASTRUCTURE ONLY.  This module is the checker, not the product: only the
test-suite (``tests/``), the smoke check in ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with the
HIP library, and imports nothing from it.

What it computes (sources, by page title and section):

* The attention definition, softmax(Q K^T / sqrt(d_k)) V, applied per head, and the
  causal rule that scores of future positions are set to -inf before the softmax --
  "GPT pretraining" page (dekermanjian, llm_gpt_pretrain), section "Multihead
  Attention" (the definition and the MultiHeadAttention listing).  The mask there is
  "upper triangle above the diagonal is masked"; the MiniGPT page ("Build and Train
  a MiniGPT with JAX", section "Model Architecture") states the same rule as
  "lower triangle including the diagonal is allowed".
* Heads laid out as [B, H, T, d] (the ``_split_heads`` reshape/transpose in the same
  listing).
* Grouped-query attention (8 query heads over 4 KV heads), RoPE, parameter-free
  RMSNorm QK-norm ("no learnable scale") and logit soft-capping -- nanoGPT-JAX 181M
  model card, section "Architecture" (table and "Design choices worth naming");
  the same features and the sliding window are named on the flaxchat page, section
  "Core Features".
* KV-cache decode -- "GPT pretraining" page, section "Bonus: KV Caching": the causal rule
  measured from the cached length, i.e. new query i sits at position (rows cached
  before the step) + i and may see cache row j iff j is not after that position; with
  one new query whose key is already stored, every cached row is visible.  The same
  step with several new tokens, storing their keys and values first, is
  ``attention_extend``.

Readings of what the pages leave open (each also listed with its reason in the
project's design notes):

* RoPE pairs element i with element i + d/2 (half split), rotates by +p*w_i with
  w_i = base^(-2i/d), and is applied to the whole head dimension.
* RMSNorm: x / sqrt(mean(x^2) + eps), eps passed in (default 1e-6), applied to the
  RoPE-rotated row (the two commute: RoPE is a rotation and keeps mean(x^2)).
* The soft-cap acts on the scaled scores before the mask: s <- c * tanh(s / c).
* Query head h reads KV head floor(h / (Hq / Hkv)) (contiguous groups).
* Sliding window W > 0: key j is visible to query i iff i - W < j <= i.
* Decode: the cache already holds the new token's (rotated) key/value, so the query
  sits at position L_b - 1 and sees all L_b cached keys; a sequence with L_b = 0
  yields an all-zero output row.
* Packed rows (segment_ids): a segment is a maximal run of equal ids in a row; a token
  attends only to keys of its own run, and its RoPE position is its offset from the start
  of the run (nanoGPT-JAX 181M model card, SFT notes: packed rows with segment ids, RoPE
  from packed segment positions).  Scores see RoPE only through position differences and
  RMSNorm commutes with the rotation, so restarting positions at each run changes no
  output or gradient here; it matters for keys that are stored rotated (a KV cache).
* Extend: cache_len counts the rows present before the step; new token i sits at
  position L_b + i, its key is rotated at that position (and normalised) before it
  is stored, and rows that would land at or past Lmax are not stored (their queries
  return zero rows).
* Left-padded batches (181M model card, inference notes: left-padded prompts with
  right-aligned generation through a KV cache, attending only the compact active slice):
  cache_start[b] = S_b rows of padding precede sequence b's first token, so row r holds
  the token at position r - S_b; only rows S_b .. (the query's row) are attended, and a
  query whose own row is below S_b (a padding token) returns a zero row.  Without
  cache_start, S_b = 0.
* Attention dropout ("GPT pretraining" page, section "Multihead Attention": dropout on the
  attention weights after the softmax, before they multiply V; rate 0.1 in the page's GPT
  configuration): inverted dropout, as the page's dropout layer does -- a weight is kept
  with probability 1 - p and then scaled by 1 / (1 - p), or set to zero.  The keep
  decision for query i and key j of head (b, h) compares a 16-bit random field with
  t = round(65536 p); the rate actually applied is t / 65536 and the scale is
  65536 / (65536 - t).  The fields come from the counter-based generator Philox4x64-10
  (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011)
  with key (seed, 0) and counter (floor(j / 16), i, b * H + h, offset): field j mod 16 of
  that 256-bit block, counting 16-bit fields from the low end of output word 0.  The
  log-sum-exp returned by the forward stays that of the softmax before dropout.

Everything is computed densely per (batch, head) in float64 with numpy; there is
no tiling, fusion or reordering beyond the definitions above.  numpy's own Philox
bit generator supplies the Philox blocks.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rope_rotate",
    "rope_unrotate",
    "rms_normalize",
    "visible_mask",
    "segment_starts",
    "attention_forward",
    "attention_backward",
    "attention_decode",
    "attention_extend",
    "dropout_threshold",
    "dropout_fields",
    "dropout_keep",
]


# --------------------------------------------------------------------------------------
# Q/K prologue pieces (nanoGPT-JAX 181M model card, "Architecture": RoPE, QK-norm)
# --------------------------------------------------------------------------------------
def _rope_angles(positions: np.ndarray, d: int, base: float) -> np.ndarray:
    """Angles a[t, i] = p_t * base^(-2i/d) for i < d/2 (float64, shape [len(positions), d/2])."""
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    omega = np.power(float(base), -2.0 * i / d)
    return np.asarray(positions, dtype=np.float64)[:, None] * omega[None, :]


def rope_rotate(x: np.ndarray, positions: np.ndarray, base: float = 10000.0) -> np.ndarray:
    """Rotate each pair (x_i, x_{i+d/2}) of the rows of x[..., T, d] by the angle p_t * w_i.

    (x_i, x_{i+d/2}) -> (x_i cos a - x_{i+d/2} sin a,  x_i sin a + x_{i+d/2} cos a).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("RoPE needs an even head dimension")
    a = _rope_angles(positions, d, base)
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def rope_unrotate(y: np.ndarray, positions: np.ndarray, base: float = 10000.0) -> np.ndarray:
    """The transpose (= inverse) of :func:`rope_rotate`: rotate every pair by -p_t * w_i.

    Because the rotation is orthogonal, this is also the map that carries a gradient
    with respect to the rotated row back to the raw row.
    """
    y = np.asarray(y, dtype=np.float64)
    d = y.shape[-1]
    a = _rope_angles(positions, d, base)
    c, s = np.cos(a), np.sin(a)
    y1, y2 = y[..., : d // 2], y[..., d // 2:]
    return np.concatenate([y1 * c + y2 * s, -y1 * s + y2 * c], axis=-1)


def rms_normalize(x: np.ndarray, eps: float = 1e-6):
    """Parameter-free RMSNorm of every row: returns (x / r, r) with r = sqrt(mean(x^2) + eps)."""
    x = np.asarray(x, dtype=np.float64)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x / r, r


def _prologue(x, positions, rope, rope_base, qk_norm, norm_eps):
    """Raw rows -> the rows that enter the score product; also returns what the backward needs."""
    y = rope_rotate(x, positions, rope_base) if rope else np.asarray(x, dtype=np.float64)
    if qk_norm:
        yhat, r = rms_normalize(y, norm_eps)
    else:
        yhat, r = y, None
    return yhat, r


def _prologue_backward(dyhat, yhat, r, positions, rope, rope_base, qk_norm):
    """Gradient through the prologue: RMSNorm backward, then RoPE backward.

    For yhat = y / r with r = sqrt(mean(y^2) + eps):  dy = (dyhat - yhat * mean(dyhat * yhat)) / r.
    For y = R(a) x:  dx = R(a)^T dy = R(-a) dy.
    """
    if qk_norm:
        dy = (dyhat - yhat * np.mean(dyhat * yhat, axis=-1, keepdims=True)) / r
    else:
        dy = dyhat
    return rope_unrotate(dy, positions, rope_base) if rope else dy


# --------------------------------------------------------------------------------------
# Mask ("GPT pretraining" page, "Multihead Attention"; flaxchat "Core Features" window)
# --------------------------------------------------------------------------------------
def visible_mask(T: int, window: int = 0) -> np.ndarray:
    """Boolean [T, T]: True where key j is visible to query i (j <= i, and i - j < window if window > 0)."""
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    m = j <= i
    if window > 0:
        m &= (i - j) < window
    return m


def segment_starts(ids) -> np.ndarray:
    """Index of the first token of each token's segment (a maximal run of equal ids)."""
    ids = np.asarray(ids)
    start = np.zeros(len(ids), dtype=np.int64)
    for i in range(1, len(ids)):
        start[i] = i if ids[i] != ids[i - 1] else start[i - 1]
    return start


def _row_layout(T, window, segment_ids, b):
    """Positions and visibility of row b: absolute positions and the causal (window) mask,
    or, for packed rows, offsets within each segment and the mask restricted to the segment."""
    allowed = visible_mask(T, window)
    if segment_ids is None:
        return np.arange(T), allowed
    start = segment_starts(segment_ids[b])
    return np.arange(T) - start, allowed & (np.arange(T)[None, :] >= start[:, None])


def _scores(qh, kh, scale, softcap):
    """Scaled scores and their soft-capped version for one (b, h): both [Tq, Tk]."""
    s_pre = scale * (qh @ kh.T)
    if softcap > 0:
        return s_pre, softcap * np.tanh(s_pre / softcap)
    return s_pre, s_pre


def _softmax_rows(s, allowed):
    """Row softmax over the allowed entries (masked entries are -inf); also the natural-log LSE."""
    s = np.where(allowed, s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=-1, keepdims=True)
    return e / l, (m + np.log(l))[..., 0]


# --------------------------------------------------------------------------------------
# Attention dropout ("GPT pretraining" page, "Multihead Attention")
# --------------------------------------------------------------------------------------
def dropout_threshold(p: float):
    """(t, scale): the 16-bit threshold t = round(65536 p) and the kept-weight scale 65536 / (65536 - t).

    A weight is kept iff its random field is >= t, so the rate applied is t / 65536.
    Requires 0 <= p and t < 65536.
    """
    p = float(p)
    if not p >= 0.0:
        raise ValueError("dropout rate must be >= 0")
    t = int(np.floor(p * 65536.0 + 0.5))
    if t >= 65536:
        raise ValueError("dropout rate rounds to 1")
    return t, 65536.0 / (65536 - t)


def dropout_fields(b: int, h: int, H: int, i: int, T: int, seed: int, offset: int) -> np.ndarray:
    """The 16-bit random fields of keys 0..T-1 for query i of head (b, h), as uint16 [T].

    Block n (keys 16 n .. 16 n + 15) is Philox4x64-10 with key (seed, 0) applied to the
    counter (n, i, b H + h, offset); key 16 n + 4 w + f takes bits 16 f .. 16 f + 15 of the
    block's output word w.  numpy's Philox encrypts the counter after incrementing it, so it
    is started one below the first block's counter.
    """
    nb = (T + 15) // 16
    c = (int(i) << 64) | (int(b * H + h) << 128) | (int(offset) << 192)
    gen = np.random.Philox(key=np.array([int(seed), 0], dtype=np.uint64),
                           counter=(c - 1) % (1 << 256))
    words = gen.random_raw(4 * nb).astype(np.uint64)  # block n: words 4 n .. 4 n + 3
    shifts = np.arange(0, 64, 16, dtype=np.uint64)
    fields = (words[:, None] >> shifts[None, :]) & np.uint64(0xFFFF)
    return fields.reshape(-1)[:T].astype(np.uint16)


def dropout_keep(B: int, H: int, T: int, p: float, seed: int, offset: int = 0) -> np.ndarray:
    """Keep mask [B, H, T, T] (bool): entry (b, h, i, j) is True iff dropout keeps weight P_ij."""
    t, _ = dropout_threshold(p)
    keep = np.empty((B, H, T, T), dtype=bool)
    for b in range(B):
        for h in range(H):
            for i in range(T):
                keep[b, h, i] = dropout_fields(b, h, H, i, T, seed, offset) >= t
    return keep


def _dropout_factor(keep, p, b, h):
    """Per-entry factor keep / (1 - rate) for head (b, h), or None without dropout."""
    if keep is None:
        return None
    _, scale = dropout_threshold(p)
    return np.where(keep[b, h], scale, 0.0)


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, T, d]")
    B, Hq, T, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != T or k.shape[3] != d:
        raise ValueError("k and v must be [B, Hkv, T, d] matching q")
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, T, d


def attention_forward(q, k, v, *, window=0, softcap=0.0, scale=None, rope=False,
                      rope_base=10000.0, qk_norm=False, norm_eps=1e-6, segment_ids=None,
                      dropout_p=0.0, dropout_keep=None):
    """Causal attention forward for q [B,Hq,T,d], k/v [B,Hkv,T,d]; returns (O [B,Hq,T,d], LSE [B,Hq,T]).

    Per (b, h):  q^ = prologue(q), k^ = prologue(k);  S = scale * q^ k^T;  S <- c tanh(S / c)
    if capped;  masked entries -> -inf;  P = row softmax(S);  O = P V;  LSE = ln sum_j exp(S_ij).
    segment_ids [B, T] (optional): packed rows, see the module notes.
    dropout_keep [B, Hq, T, T] (optional, with rate dropout_p): O = (P * Z) V with
    Z = keep / (1 - rate); the LSE is unchanged.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, T, d = _check_shapes(q, k, v)
    if scale is None or scale == 0:
        scale = 1.0 / np.sqrt(d)
    group = Hq // Hkv
    O = np.empty((B, Hq, T, d))
    LSE = np.empty((B, Hq, T))
    for b in range(B):
        pos, allowed = _row_layout(T, window, segment_ids, b)
        khat = [_prologue(k[b, g], pos, rope, rope_base, qk_norm, norm_eps)[0] for g in range(Hkv)]
        for h in range(Hq):
            g = h // group
            qh, _ = _prologue(q[b, h], pos, rope, rope_base, qk_norm, norm_eps)
            _, s = _scores(qh, khat[g], scale, softcap)
            P, lse = _softmax_rows(s, allowed)
            Z = _dropout_factor(dropout_keep, dropout_p, b, h)
            O[b, h] = (P if Z is None else P * Z) @ v[b, g]
            LSE[b, h] = lse
    return O, LSE


def attention_backward(q, k, v, dO, *, window=0, softcap=0.0, scale=None, rope=False,
                       rope_base=10000.0, qk_norm=False, norm_eps=1e-6, segment_ids=None,
                       dropout_p=0.0, dropout_keep=None, o_stored=None):
    """Analytic gradients (dQ, dK, dV) of <O, dO> with respect to the RAW q, k, v.

    Per (b, h) with g = kv head of h:
      dV_g += P^T dO;  dP = dO V_g^T;  D_i = sum_d dO_i O_i;  dS = P * (dP - D);
    with dropout (Z = keep / (1 - rate), O = (P * Z) V):  dV_g += (P * Z)^T dO and
    dP = Z * (dO V_g^T), D unchanged (it equals sum_j P_ij dP_ij either way);
      dS_pre = dS * (1 - tanh(S_pre / c)^2) if capped;
      dq^ = scale dS_pre k^;  dk^_g += scale dS_pre^T q^;
    then each of dq^, dk^ goes back through RMSNorm and RoPE.
    o_stored [B, Hq, T, d] (optional): the output from which D is formed, e.g. the forward's
    output as it is stored (rounded to bf16); by default the exact O.  Only D changes.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    B, Hq, Hkv, T, d = _check_shapes(q, k, v)
    if dO.shape != q.shape:
        raise ValueError("dO must have q's shape")
    if scale is None or scale == 0:
        scale = 1.0 / np.sqrt(d)
    group = Hq // Hkv
    dQ = np.empty_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    for b in range(B):
        pos, allowed = _row_layout(T, window, segment_ids, b)
        kpro = [_prologue(k[b, g], pos, rope, rope_base, qk_norm, norm_eps) for g in range(Hkv)]
        dkhat = [np.zeros((T, d)) for _ in range(Hkv)]
        for h in range(Hq):
            g = h // group
            qhat, rq = _prologue(q[b, h], pos, rope, rope_base, qk_norm, norm_eps)
            khat = kpro[g][0]
            s_pre, s = _scores(qhat, khat, scale, softcap)
            P, _ = _softmax_rows(s, allowed)
            Z = _dropout_factor(dropout_keep, dropout_p, b, h)
            Pz = P if Z is None else P * Z
            O = Pz @ v[b, g]
            dV[b, g] += Pz.T @ dO[b, h]
            dP = dO[b, h] @ v[b, g].T
            if Z is not None:
                dP = dP * Z
            Od = O if o_stored is None else np.asarray(o_stored, dtype=np.float64)[b, h]
            D = np.sum(dO[b, h] * Od, axis=-1, keepdims=True)
            dS = P * (dP - D)
            if softcap > 0:
                dS = dS * (1.0 - np.tanh(s_pre / softcap) ** 2)
            dqhat = scale * (dS @ khat)
            dkhat[g] += scale * (dS.T @ qhat)
            dQ[b, h] = _prologue_backward(dqhat, qhat, rq, pos, rope, rope_base, qk_norm)
        for g in range(Hkv):
            khat, rk = kpro[g]
            dK[b, g] = _prologue_backward(dkhat[g], khat, rk, pos, rope, rope_base, qk_norm)
    return dQ, dK, dV


def attention_decode(q, k_cache, v_cache, cache_len, *, softcap=0.0, scale=None, rope=False,
                     rope_base=10000.0, qk_norm=False, norm_eps=1e-6, cache_start=None):
    """One-token decode: q [B,Hq,d] attends over rows S_b .. L_b - 1 of k/v_cache [B,Hkv,Lmax,d].

    The cached keys are taken as already rotated (and normalised, when QK-norm is on); only
    the query is rotated, at position L_b - 1 - S_b, and normalised.  cache_len is clamped to
    [0, Lmax] and cache_start (S_b, default 0) to [0, L_b]; an empty range gives a zero
    output row.  Returns o [B,Hq,d].
    """
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    B, Hq, d = q.shape
    if kc.ndim != 4 or kc.shape != vc.shape or kc.shape[0] != B or kc.shape[3] != d:
        raise ValueError("caches must be [B, Hkv, Lmax, d] matching q")
    Hkv, Lmax = kc.shape[1], kc.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if scale is None or scale == 0:
        scale = 1.0 / np.sqrt(d)
    group = Hq // Hkv
    o = np.zeros((B, Hq, d))
    for b in range(B):
        L = int(min(max(int(cache_len[b]), 0), Lmax))
        S0 = 0 if cache_start is None else int(min(max(int(cache_start[b]), 0), L))
        if L == S0:
            continue
        qhat, _ = _prologue(q[b][:, None, :], np.array([L - 1 - S0]), rope, rope_base, qk_norm,
                            norm_eps)
        for h in range(Hq):
            g = h // group
            _, s = _scores(qhat[h], kc[b, g, S0:L], scale, softcap)
            P, _ = _softmax_rows(s, np.ones_like(s, dtype=bool))
            o[b, h] = (P @ vc[b, g, S0:L])[0]
    return o


def attention_extend(q, k_new, v_new, k_cache, v_cache, cache_len, *, window=0, softcap=0.0,
                     scale=None, rope=False, rope_base=10000.0, qk_norm=False, norm_eps=1e-6,
                     cache_start=None):
    """S new tokens per sequence against a KV cache ("GPT pretraining" page, "Bonus: KV Caching").

    q [B,Hq,S,d], k_new/v_new [B,Hkv,S,d] are raw (before RoPE / QK-norm); the caches
    [B,Hkv,Lmax,d] hold rotated (and normalised) keys in rows < cache_len[b].  Token i of
    sequence b sits at position p = L_b + i: its key (rotated at p, normalised) and value are
    stored in row p, and its query (rotated at p, normalised) attends over keys j <= p (and
    j > p - window with a window) -- the page's offset rule with offset = L_b.
    cache_len is clamped to [0, Lmax]; tokens with p >= Lmax are not stored and give zero
    output rows.  Returns (o [B,Hq,S,d], k_cache', v_cache'); the inputs are not modified.
    With cache_start (S_b, clamped to [0, Lmax]) the rows below S_b are left padding: the
    token in row r sits at position r - S_b (its key is rotated there), only rows >= S_b are
    attended, and new tokens whose row is below S_b (padding) are stored but give zero rows.
    """
    q = np.asarray(q, dtype=np.float64)
    kn = np.asarray(k_new, dtype=np.float64)
    vn = np.asarray(v_new, dtype=np.float64)
    kc = np.array(k_cache, dtype=np.float64)
    vc = np.array(v_cache, dtype=np.float64)
    if q.ndim != 4 or kn.ndim != 4 or kn.shape != vn.shape:
        raise ValueError("q must be [B,Hq,S,d] and k_new/v_new [B,Hkv,S,d]")
    B, Hq, S, d = q.shape
    if kn.shape[0] != B or kn.shape[2] != S or kn.shape[3] != d:
        raise ValueError("k_new/v_new must match q in B, S and d")
    if kc.ndim != 4 or kc.shape != vc.shape or kc.shape[0] != B or kc.shape[1] != kn.shape[1] \
            or kc.shape[3] != d:
        raise ValueError("caches must be [B, Hkv, Lmax, d] matching k_new")
    Hkv, Lmax = kc.shape[1], kc.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if scale is None or scale == 0:
        scale = 1.0 / np.sqrt(d)
    group = Hq // Hkv
    o = np.zeros((B, Hq, S, d))
    for b in range(B):
        L = int(min(max(int(cache_len[b]), 0), Lmax))
        S0 = 0 if cache_start is None else int(min(max(int(cache_start[b]), 0), Lmax))
        n = min(S, Lmax - L)  # tokens that fit in the cache
        if n <= 0:
            continue
        rows = L + np.arange(n)
        pos = rows - S0
        khat, _ = _prologue(kn[b][:, :n], pos, rope, rope_base, qk_norm, norm_eps)
        kc[b, :, L:L + n] = khat
        vc[b, :, L:L + n] = vn[b][:, :n]
        qhat, _ = _prologue(q[b][:, :n], pos, rope, rope_base, qk_norm, norm_eps)
        j = np.arange(L + n)[None, :]
        allowed = (j <= rows[:, None]) & (j >= S0)
        if window > 0:
            allowed &= (rows[:, None] - j) < window
        real = rows >= S0  # padding tokens (rows below S_b) give zero rows
        for h in range(Hq):
            g = h // group
            _, sc = _scores(qhat[h][real], kc[b, g, :L + n], scale, softcap)
            P, _ = _softmax_rows(sc, allowed[real])
            o[b, h, :n][real] = P @ vc[b, g, :L + n]
    return o, kc, vc
