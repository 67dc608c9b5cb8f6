"""Seeded synthetic inputs and the named workload shapes.

This module holds no attention arithmetic: it only draws N(0, 1) numbers from a seeded
generator, rounds them to bfloat16 (round-to-nearest-even) when asked, and records
the workload shapes.  Both the HIP path (through its binding) and the fp64 oracle
consume exactly these host arrays, so the two sides see bit-identical inputs.

The shapes come from the pages' models (see ``WORKLOADS``); the pages train on
token corpora that this library never sees -- the attention kernel only ever reads
the projected q/k/v activations, for which N(0, 1) draws of the same shape stand in.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

SEED_BASE = 42  # the pages seed their loaders and models with 42; workload i uses 42 + i


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are already bfloat16-representable (uint16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclass(frozen=True)
class Workload:
    """One named attention workload: shapes [B, H, T, d] and the variant flags."""
    name: str
    B: int
    T: int
    Hq: int
    Hkv: int
    D: int
    dtype: str = "bf16"          # "f32" or "bf16"
    window: int = 0              # 0 = plain causal
    softcap: float = 0.0         # 0 = off
    rope: bool = False
    rope_base: float = 10000.0
    qk_norm: bool = False
    norm_eps: float = 1e-6
    backward: bool = True
    decode: bool = False         # single-token KV-cache decode instead of fwd/bwd
    len_lo: int = 0              # decode: cache lengths ~ U{len_lo .. T}
    seg_lo: int = 0              # packed rows: run lengths ~ U{seg_lo .. seg_hi} (0 = unpacked)
    seg_hi: int = 0
    new_tokens: int = 0          # extend: tokens appended per sequence (cache lengths ~
                                 # U{len_lo .. T - new_tokens}, T = allocated rows)
    leftpad: bool = False        # decode: left-padded batch, right-aligned in T cache rows
    dropout: float = 0.0         # dropout rate on the attention weights (0 = none); the keep
                                 # mask is drawn with generator seed `seed`, offset 0
    seed: int = SEED_BASE
    note: str = field(default="", compare=False)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# Shapes from the pages (see tests/golden/page_shapes.json for the cited values).
WORKLOADS = {
    # MiniGPT: maxlen 128, embed 192 over 6 heads -> d = 32; fp32 forward only.
    "minigpt_fwd_f32": Workload("minigpt_fwd_f32", B=2, T=128, Hq=6, Hkv=6, D=32, dtype="f32",
                                backward=False, seed=SEED_BASE + 0),
    # MiniGPT training batch (batch 32), bf16 forward + backward.
    "minigpt_train_bf16": Workload("minigpt_train_bf16", B=32, T=128, Hq=6, Hkv=6, D=32,
                                   seed=SEED_BASE + 1),
    # nanoGPT-JAX 181M: 8 query / 4 KV heads, head dim 96, sequence 2048, RoPE, QK-norm,
    # soft-cap 50.
    "gqa181m_train": Workload("gqa181m_train", B=16, T=2048, Hq=8, Hkv=4, D=96, softcap=50.0,
                              rope=True, qk_norm=True, seed=SEED_BASE + 2),
    # flaxchat depth 12: 768 dims over 6 heads -> d = 128, GQA 3 KV heads; global layer ...
    "flaxchat_full": Workload("flaxchat_full", B=16, T=2048, Hq=6, Hkv=3, D=128, rope=True,
                              qk_norm=True, seed=SEED_BASE + 3),
    # ... and the sliding-window layers (window 512).
    "flaxchat_w512": Workload("flaxchat_w512", B=16, T=2048, Hq=6, Hkv=3, D=128, window=512,
                              rope=True, qk_norm=True, seed=SEED_BASE + 3),
    # KV-cache decode: 64 sequences, cache lengths U{256..2048}, 8/4 heads, d 96, RoPE, cap 50.
    "gqa181m_decode": Workload("gqa181m_decode", B=64, T=2048, Hq=8, Hkv=4, D=96, softcap=50.0,
                               rope=True, backward=False, decode=True, len_lo=256,
                               seed=SEED_BASE + 4),
    # Batched generation from left-padded prompts (181M model card, inference notes): every
    # cache is right-aligned at 2048 rows and holds U{256..2048} real rows after its padding.
    "gqa181m_decode_leftpad": Workload("gqa181m_decode_leftpad", B=64, T=2048, Hq=8, Hkv=4, D=96,
                                       softcap=50.0, rope=True, backward=False, decode=True,
                                       len_lo=256, leftpad=True, seed=SEED_BASE + 11),
    # SFT-style packed rows on the 181M shapes: each row holds sequences of U{64..1024} tokens.
    "gqa181m_sft_packed": Workload("gqa181m_sft_packed", B=16, T=2048, Hq=8, Hkv=4, D=96,
                                   softcap=50.0, rope=True, qk_norm=True, seg_lo=64, seg_hi=1024,
                                   seed=SEED_BASE + 9),
    # A multi-token step on the decode caches: 128 new tokens per sequence (chunked prefill or
    # speculative verification) against cache lengths U{256..1920}.
    "gqa181m_extend": Workload("gqa181m_extend", B=64, T=2048, Hq=8, Hkv=4, D=96, softcap=50.0,
                               rope=True, backward=False, len_lo=256, new_tokens=128,
                               seed=SEED_BASE + 8),
    # GPT pretraining page: 768 dims over 12 heads -> d = 64, context 256, batch 128; plain
    # causal multi-head attention (learned position embeddings, no RoPE / QK-norm / cap).
    "gpt_pretrain_train": Workload("gpt_pretrain_train", B=128, T=256, Hq=12, Hkv=12, D=64,
                                   seed=SEED_BASE + 5),
    # The same with the page's attention dropout (rate 0.1 on the weights) in training.
    "gpt_pretrain_train_dropout": Workload("gpt_pretrain_train_dropout", B=128, T=256, Hq=12,
                                           Hkv=12, D=64, dropout=0.1, seed=SEED_BASE + 10),
    # Instruction tuning on GPT-2 XL: 1600 dims over 25 heads -> d = 64, context 256, batch 8.
    "gpt2xl_instruct_train": Workload("gpt2xl_instruct_train", B=8, T=256, Hq=25, Hkv=25, D=64,
                                      seed=SEED_BASE + 6),
    # The GPT pretraining page's KV-cache run: one sequence, full 256-token context, 12 heads.
    "gpt_pretrain_decode": Workload("gpt_pretrain_decode", B=1, T=256, Hq=12, Hkv=12, D=64,
                                    backward=False, decode=True, len_lo=256, seed=SEED_BASE + 7),
}


def _normal(rng: np.random.Generator, shape, bf16: bool) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return round_to_bf16(x) if bf16 else x


def make_train_inputs(w: Workload, seed: int | None = None, q_gain: float = 1.0):
    """q [B,Hq,T,D], k/v [B,Hkv,T,D], dO [B,Hq,T,D] as float32 host arrays (bf16-exact if bf16).

    ``q_gain`` scales q before rounding (a sharper-attention stress input); 1 by default.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    bf16 = w.dtype == "bf16"
    q = rng.standard_normal(size=(w.B, w.Hq, w.T, w.D), dtype=np.float32) * np.float32(q_gain)
    q = round_to_bf16(q) if bf16 else q
    k = _normal(rng, (w.B, w.Hkv, w.T, w.D), bf16)
    v = _normal(rng, (w.B, w.Hkv, w.T, w.D), bf16)
    dO = _normal(rng, (w.B, w.Hq, w.T, w.D), bf16) if w.backward else None
    return q, k, v, dO


def make_decode_inputs(w: Workload, seed: int | None = None):
    """q [B,Hq,D], k/v caches [B,Hkv,Lmax,D] (float32, bf16-exact), cache_len int32 [B].

    Lmax = w.T; every cache row is drawn, also those at or beyond a sequence's length.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    cache_len = rng.integers(w.len_lo, w.T, size=w.B, endpoint=True).astype(np.int32)
    q = _normal(rng, (w.B, w.Hq, w.D), True)
    kc = _normal(rng, (w.B, w.Hkv, w.T, w.D), True)
    vc = _normal(rng, (w.B, w.Hkv, w.T, w.D), True)
    return q, kc, vc, cache_len


def make_segment_ids(w: Workload, seed: int | None = None) -> np.ndarray:
    """int32 [B, T] segment ids: each row is cut into runs of U{seg_lo .. seg_hi} tokens (the
    last run takes what is left), numbered 0, 1, 2, ... within the row."""
    rng = np.random.default_rng((w.seed if seed is None else seed) + 1000)
    ids = np.empty((w.B, w.T), dtype=np.int32)
    for b in range(w.B):
        a, n = 0, 0
        while a < w.T:
            L = int(rng.integers(w.seg_lo, w.seg_hi, endpoint=True))
            ids[b, a:a + L] = n
            a, n = a + L, n + 1
    return ids


def packed_flops(w: Workload, ids) -> float:
    """14 d flops per visible pair; runs of length n have n (n + 1) / 2 pairs per head."""
    pairs = 0
    for row in np.asarray(ids):
        cuts = np.flatnonzero(np.diff(row)) + 1
        for n in np.diff(np.concatenate([[0], cuts, [len(row)]])):
            pairs += int(n) * (int(n) + 1) // 2
    return 14.0 * w.D * w.Hq * pairs


def make_leftpad_decode_inputs(w: Workload, seed: int | None = None):
    """make_decode_inputs for a left-padded batch: (q, k_cache, v_cache, cache_start,
    cache_len) with cache_len = Lmax = w.T for every sequence and cache_start = T - (real rows),
    real rows ~ U{len_lo .. T}."""
    q, kc, vc, real = make_decode_inputs(w, seed)
    lens = np.full(w.B, w.T, dtype=np.int32)
    return q, kc, vc, (lens - real).astype(np.int32), lens


def make_extend_inputs(w: Workload, seed: int | None = None):
    """q [B,Hq,S,D], k_new/v_new [B,Hkv,S,D], caches [B,Hkv,Lmax,D] (float32, bf16-exact) and
    cache_len int32 [B] ~ U{len_lo .. Lmax - S}; S = w.new_tokens, Lmax = w.T."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    S = w.new_tokens
    cache_len = rng.integers(w.len_lo, w.T - S, size=w.B, endpoint=True).astype(np.int32)
    q = _normal(rng, (w.B, w.Hq, S, w.D), True)
    kn = _normal(rng, (w.B, w.Hkv, S, w.D), True)
    vn = _normal(rng, (w.B, w.Hkv, S, w.D), True)
    kc = _normal(rng, (w.B, w.Hkv, w.T, w.D), True)
    vc = _normal(rng, (w.B, w.Hkv, w.T, w.D), True)
    return q, kn, vn, kc, vc, cache_len


def extend_flops(w: Workload, cache_len) -> float:
    """4 d flops per visible (new query, key) pair: query i of sequence b sees L_b + i + 1 keys."""
    S = w.new_tokens
    pairs = sum(S * int(L) + S * (S + 1) // 2 for L in cache_len)
    return 4.0 * w.D * w.Hq * pairs


def visible_pairs(T: int, window: int = 0) -> int:
    """Number of (query, key) pairs a causal (optionally windowed) mask lets through per head."""
    if window <= 0 or window >= T:
        return T * (T + 1) // 2
    return window * (window + 1) // 2 + (T - window) * window


def train_flops(w: Workload, backward: bool | None = None) -> float:
    """Algorithmic FLOPs: 4d per visible pair forward, 10d backward (recomputed QK^T included)."""
    bwd = w.backward if backward is None else backward
    per_pair = 4 * w.D + (10 * w.D if bwd else 0)
    return float(per_pair) * visible_pairs(w.T, w.window) * w.B * w.Hq


def decode_bytes(w: Workload, cache_len: np.ndarray) -> float:
    """Algorithmic HBM bytes of one decode call: active K and V rows (bf16), once per KV head,
    plus q, o (bf16) and cache_len."""
    active = float(np.clip(cache_len, 0, w.T).astype(np.int64).sum())
    return 2 * active * w.Hkv * w.D * 2 + 2 * w.B * w.Hq * w.D * 2 + 4 * w.B
