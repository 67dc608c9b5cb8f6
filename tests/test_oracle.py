"""Pins for the fp64 oracle, independent of the oracle's own code.

Each test checks the oracle against something other than itself: a per-query brute
force written with scalar loops and complex-number RoPE, central finite differences,
exact invariants of the attention definition, or special cases with a textbook answer.
No GPU is needed.
"""
import cmath
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import (attention_backward, attention_decode, attention_extend, attention_forward,
                    dropout_fields, dropout_keep, dropout_threshold, rms_normalize, rope_rotate,
                    rope_unrotate, segment_starts, visible_mask)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(rng, *shape):
    return rng.standard_normal(shape)


# ------------------------------------------------------------------------------------
# Brute force: one query at a time, scalar Python, RoPE as complex multiplication.
# ------------------------------------------------------------------------------------
def _bf_prologue(row, pos, rope, base, qk_norm, eps):
    d = len(row)
    half = d // 2
    out = list(row)
    if rope:
        for i in range(half):
            z = complex(row[i], row[i + half]) * cmath.exp(1j * pos * base ** (-2.0 * i / d))
            out[i], out[i + half] = z.real, z.imag
    if qk_norm:
        ms = sum(x * x for x in out) / d
        out = [x / math.sqrt(ms + eps) for x in out]
    return out


def brute_force_forward(q, k, v, window, softcap, rope, qk_norm, base=10000.0, eps=1e-6):
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d)
    O = np.zeros((B, Hq, T, d))
    L = np.zeros((B, Hq, T))
    for b, h, i in itertools.product(range(B), range(Hq), range(T)):
        g = h * Hkv // Hq
        qi = _bf_prologue(q[b, h, i], i, rope, base, qk_norm, eps)
        keys = [j for j in range(T) if j <= i and (window == 0 or i - j < window)]
        scores = []
        for j in keys:
            kj = _bf_prologue(k[b, g, j], j, rope, base, qk_norm, eps)
            s = scale * sum(a * c for a, c in zip(qi, kj))
            if softcap:
                s = softcap * math.tanh(s / softcap)
            scores.append(s)
        mx = max(scores)
        w = [math.exp(s - mx) for s in scores]
        tot = sum(w)
        for jj, j in enumerate(keys):
            O[b, h, i] += (w[jj] / tot) * v[b, g, j]
        L[b, h, i] = mx + math.log(tot)
    return O, L


FLAG_SETS = [
    dict(window=0, softcap=0.0, rope=False, qk_norm=False),
    dict(window=0, softcap=0.5, rope=False, qk_norm=False),
    dict(window=0, softcap=50.0, rope=True, qk_norm=True),
    dict(window=2, softcap=0.0, rope=True, qk_norm=False),
    dict(window=1, softcap=0.0, rope=False, qk_norm=True),
    dict(window=3, softcap=0.5, rope=True, qk_norm=True),
]


@pytest.mark.parametrize("heads", [(1, 1), (2, 1), (4, 2), (3, 3)])
@pytest.mark.parametrize("flags", FLAG_SETS)
def test_forward_matches_brute_force(heads, flags):
    rng = np.random.default_rng(7)
    Hq, Hkv = heads
    for T, d in [(1, 2), (5, 4), (9, 8)]:
        q, k, v = rnd(rng, 2, Hq, T, d), rnd(rng, 2, Hkv, T, d), rnd(rng, 2, Hkv, T, d)
        O, L = attention_forward(q, k, v, **flags)
        Ob, Lb = brute_force_forward(q, k, v, **flags)
        np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------------
# Finite differences for the analytic backward.
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("flags", FLAG_SETS)
def test_backward_matches_finite_differences(flags):
    rng = np.random.default_rng(11)
    B, Hq, Hkv, T, d = 1, 2, 1, 7, 8
    q, k, v = rnd(rng, B, Hq, T, d), rnd(rng, B, Hkv, T, d), rnd(rng, B, Hkv, T, d)
    dO = rnd(rng, B, Hq, T, d)
    dQ, dK, dV = attention_backward(q, k, v, dO, **flags)

    def loss(q_, k_, v_):
        return float(np.sum(attention_forward(q_, k_, v_, **flags)[0] * dO))

    h = 1e-6
    for name, x, grad in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (loss(**{f"{n}_": a for n, a in args_p.items()})
                        - loss(**{f"{n}_": a for n, a in args_m.items()})) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=0, atol=2e-7, err_msg=name)


# ------------------------------------------------------------------------------------
# Exact invariants of the definition.
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("flags", FLAG_SETS)
def test_rows_of_p_sum_to_one(flags):
    rng = np.random.default_rng(3)
    q, k = rnd(rng, 2, 4, 33, 8), rnd(rng, 2, 2, 33, 8)
    O, _ = attention_forward(q, k, np.ones((2, 2, 33, 8)), **flags)
    np.testing.assert_allclose(O, 1.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("flags", FLAG_SETS)
def test_causal_invariant(flags):
    """Output row t does not change when tokens after t are perturbed."""
    rng = np.random.default_rng(5)
    T = 24
    q, k, v = rnd(rng, 1, 2, T, 8), rnd(rng, 1, 1, T, 8), rnd(rng, 1, 1, T, 8)
    O, L = attention_forward(q, k, v, **flags)
    for t in (0, 5, 17):
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        q2[:, :, t + 1:] += rnd(rng, 1, 2, T - t - 1, 8)
        k2[:, :, t + 1:] *= 3.0
        v2[:, :, t + 1:] -= 7.0
        O2, L2 = attention_forward(q2, k2, v2, **flags)
        np.testing.assert_allclose(O2[:, :, : t + 1], O[:, :, : t + 1], rtol=0, atol=1e-14)
        np.testing.assert_allclose(L2[:, :, : t + 1], L[:, :, : t + 1], rtol=0, atol=1e-14)
        assert np.abs(O2[:, :, t + 1:] - O[:, :, t + 1:]).max() > 1e-3


@pytest.mark.parametrize("flags", FLAG_SETS)
def test_gradient_sum_identities(flags):
    """sum_j dV_j = sum_i dO_i per (b, kv head) over the group (rows of P sum to 1), and
    <Q, dQ> = <K, dK> per (b, kv head) (scores are invariant to Q -> aQ, K -> K/a;
    only exact without QK-norm, which breaks that scaling)."""
    rng = np.random.default_rng(9)
    B, Hq, Hkv, T, d = 2, 4, 2, 13, 8
    q, k, v = rnd(rng, B, Hq, T, d), rnd(rng, B, Hkv, T, d), rnd(rng, B, Hkv, T, d)
    dO = rnd(rng, B, Hq, T, d)
    dQ, dK, dV = attention_backward(q, k, v, dO, **flags)
    g = Hq // Hkv
    np.testing.assert_allclose(dV.sum(axis=2),
                               dO.reshape(B, Hkv, g, T, d).sum(axis=(2, 3)), rtol=0, atol=1e-12)
    if not flags["qk_norm"]:
        lhs = (q * dQ).reshape(B, Hkv, g, T, d).sum(axis=(2, 3, 4))
        rhs = (k * dK).sum(axis=(2, 3))
        np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-12)
    else:
        # QK-norm: each normalised row is scale-invariant, so <x_row, dx_row> = O(eps).
        assert np.abs((q * dQ).sum(-1)).max() < 1e-4
        assert np.abs((k * dK).sum(-1)).max() < 1e-4


def test_stored_output_enters_only_through_d():
    """o_stored replaces the exact O in D_i = dO_i . O_i only.  Plain attention, closed form: a
    change dD_i of D changes dS_ij by -P_ij dD_i, so dQ_i by -scale dD_i sum_j P_ij k_j and dK_j
    by -scale sum_i P_ij dD_i q_i, and leaves dV.  With every flag set the change is still
    linear in dD (twice the perturbation, twice the change) and dV is untouched."""
    rng = np.random.default_rng(31)
    B, H, T, d = 1, 2, 7, 6
    q, k, v, dO = rnd(rng, B, H, T, d), rnd(rng, B, H, T, d), rnd(rng, B, H, T, d), rnd(rng, B, H, T, d)
    O, _ = attention_forward(q, k, v)
    base = attention_backward(q, k, v, dO)
    for a, b in zip(attention_backward(q, k, v, dO, o_stored=O), base):
        np.testing.assert_allclose(a, b, atol=1e-15)
    dlt = 1e-3 * rnd(rng, B, H, T, d)
    dQ, dK, dV = attention_backward(q, k, v, dO, o_stored=O + dlt)
    np.testing.assert_array_equal(dV, base[2])
    scale = 1.0 / math.sqrt(d)
    for h in range(H):
        P = np.zeros((T, T))
        for i in range(T):
            sc = [scale * float(q[0, h, i] @ k[0, h, j]) for j in range(i + 1)]
            m = max(sc)
            e = [math.exp(x - m) for x in sc]
            P[i, :i + 1] = np.array(e) / sum(e)
        dD = (dO[0, h] * dlt[0, h]).sum(-1)
        np.testing.assert_allclose(dQ[0, h] - base[0][0, h], -scale * dD[:, None] * (P @ k[0, h]),
                                   atol=1e-13)
        np.testing.assert_allclose(dK[0, h] - base[1][0, h], -scale * P.T @ (dD[:, None] * q[0, h]),
                                   atol=1e-13)
    for flags in FLAG_SETS:
        O, _ = attention_forward(q, k, v, **flags)
        b0 = attention_backward(q, k, v, dO, **flags)
        b1 = attention_backward(q, k, v, dO, o_stored=O + dlt, **flags)
        b2 = attention_backward(q, k, v, dO, o_stored=O + 2 * dlt, **flags)
        np.testing.assert_array_equal(b1[2], b0[2])
        for x0, x1, x2 in zip(b0[:2], b1[:2], b2[:2]):
            np.testing.assert_allclose(x2 - x0, 2 * (x1 - x0), atol=1e-13)


def test_plain_attention_dk_sums_to_zero():
    """Without RoPE/cap/norm, adding a constant vector to every key shifts each score row by a
    constant, which softmax ignores: sum_j dK_j = 0."""
    rng = np.random.default_rng(10)
    q, k, v, dO = rnd(rng, 1, 2, 11, 4), rnd(rng, 1, 1, 11, 4), rnd(rng, 1, 1, 11, 4), rnd(rng, 1, 2, 11, 4)
    _, dK, _ = attention_backward(q, k, v, dO)
    np.testing.assert_allclose(dK.sum(axis=2), 0.0, atol=1e-13)


# ------------------------------------------------------------------------------------
# Special cases with textbook answers.
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("flags", FLAG_SETS)
def test_single_token_returns_value(flags):
    rng = np.random.default_rng(1)
    q, k, v = rnd(rng, 3, 2, 1, 8), rnd(rng, 3, 1, 1, 8), rnd(rng, 3, 1, 1, 8)
    O, _ = attention_forward(q, k, v, **flags)
    np.testing.assert_allclose(O, np.repeat(v, 2, axis=1), atol=1e-15)


def test_window_one_is_identity():
    rng = np.random.default_rng(2)
    q, k, v, dO = rnd(rng, 2, 2, 9, 8), rnd(rng, 2, 2, 9, 8), rnd(rng, 2, 2, 9, 8), rnd(rng, 2, 2, 9, 8)
    for rope, norm, cap in itertools.product([0, 1], [0, 1], [0.0, 2.0]):
        kw = dict(window=1, rope=bool(rope), qk_norm=bool(norm), softcap=cap)
        O, L = attention_forward(q, k, v, **kw)
        np.testing.assert_allclose(O, v, atol=1e-15)
        dQ, dK, dV = attention_backward(q, k, v, dO, **kw)
        np.testing.assert_allclose(dQ, 0.0, atol=1e-14)
        np.testing.assert_allclose(dK, 0.0, atol=1e-14)
        np.testing.assert_allclose(dV, dO, atol=1e-14)


def test_zero_query_gives_prefix_mean():
    """q = 0 makes every visible score equal, so row t is the mean of v_0..v_t (window: of the
    last W rows)."""
    rng = np.random.default_rng(4)
    T = 10
    q, k, v = np.zeros((1, 2, T, 4)), rnd(rng, 1, 2, T, 4), rnd(rng, 1, 2, T, 4)
    for window, rope, norm in [(0, False, False), (0, True, True), (3, True, False)]:
        O, L = attention_forward(q, k, v, window=window, rope=rope, qk_norm=norm, softcap=5.0)
        for t in range(T):
            lo = 0 if window == 0 else max(0, t - window + 1)
            np.testing.assert_allclose(O[0, :, t], v[0, :, lo: t + 1].mean(axis=1), atol=1e-14)
            np.testing.assert_allclose(L[0, :, t], math.log(t + 1 - lo), atol=1e-14)


def test_two_token_closed_form():
    """T = 2, d = 2, plain attention: row 1 is the logistic mix of v_0 and v_1."""
    q = np.array([[[[0.3, -1.2], [0.8, 0.5]]]])
    k = np.array([[[[1.5, 0.25], [-0.5, 2.0]]]])
    v = np.array([[[[1.0, -2.0], [4.0, 3.0]]]])
    O, L = attention_forward(q, k, v)
    s0 = (0.8 * 1.5 + 0.5 * 0.25) / math.sqrt(2)
    s1 = (0.8 * -0.5 + 0.5 * 2.0) / math.sqrt(2)
    p1 = 1.0 / (1.0 + math.exp(s0 - s1))
    np.testing.assert_allclose(O[0, 0, 0], v[0, 0, 0], atol=1e-15)
    np.testing.assert_allclose(O[0, 0, 1], (1 - p1) * v[0, 0, 0] + p1 * v[0, 0, 1], atol=1e-15)
    np.testing.assert_allclose(L[0, 0, 1], math.log(math.exp(s0) + math.exp(s1)), atol=1e-15)


def test_large_window_equals_causal_and_large_cap_equals_none():
    rng = np.random.default_rng(6)
    q, k, v, dO = rnd(rng, 1, 2, 12, 8), rnd(rng, 1, 1, 12, 8), rnd(rng, 1, 1, 12, 8), rnd(rng, 1, 2, 12, 8)
    base = attention_forward(q, k, v, rope=True)
    for a, b in zip(attention_forward(q, k, v, rope=True, window=12), base):
        np.testing.assert_array_equal(a, b)
    for a, b in zip(attention_forward(q, k, v, rope=True, window=40), base):
        np.testing.assert_array_equal(a, b)
    for a, b in zip(attention_forward(q, k, v, rope=True, softcap=1e7), base):
        np.testing.assert_allclose(a, b, atol=1e-12)
    for a, b in zip(attention_backward(q, k, v, dO, rope=True, softcap=1e7),
                    attention_backward(q, k, v, dO, rope=True)):
        np.testing.assert_allclose(a, b, atol=1e-12)


@pytest.mark.parametrize("flags", FLAG_SETS)
def test_gqa_equals_mha_with_repeated_kv(flags):
    rng = np.random.default_rng(8)
    B, Hq, Hkv, T, d = 2, 6, 2, 9, 4
    q, k, v, dO = rnd(rng, B, Hq, T, d), rnd(rng, B, Hkv, T, d), rnd(rng, B, Hkv, T, d), rnd(rng, B, Hq, T, d)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    Og, Lg = attention_forward(q, k, v, **flags)
    Om, Lm = attention_forward(q, kr, vr, **flags)
    np.testing.assert_allclose(Og, Om, atol=1e-14)
    np.testing.assert_allclose(Lg, Lm, atol=1e-14)
    dQg, dKg, dVg = attention_backward(q, k, v, dO, **flags)
    dQm, dKm, dVm = attention_backward(q, kr, vr, dO, **flags)
    np.testing.assert_allclose(dQg, dQm, atol=1e-13)
    np.testing.assert_allclose(dKg, dKm.reshape(B, Hkv, 3, T, d).sum(axis=2), atol=1e-13)
    np.testing.assert_allclose(dVg, dVm.reshape(B, Hkv, 3, T, d).sum(axis=2), atol=1e-13)


# ------------------------------------------------------------------------------------
# Prologue pieces: RoPE and RMSNorm.
# ------------------------------------------------------------------------------------
def test_rope_properties():
    rng = np.random.default_rng(12)
    d, T = 16, 50
    x = rnd(rng, T, d)
    pos = np.arange(T)
    y = rope_rotate(x, pos)
    np.testing.assert_allclose(y[0], x[0], atol=0)                                # p = 0
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)
    np.testing.assert_allclose(rope_unrotate(y, pos), x, atol=1e-14)
    # First pair turns by exactly p radians, the last by p * base^(-(d-2)/d).
    e = np.zeros((1, d))
    e[0, 0] = 1.0
    for p in (1, 7, 2047):
        r = rope_rotate(e, np.array([p]))[0]
        assert abs(r[0] - math.cos(p)) < 1e-12 and abs(r[d // 2] - math.sin(p)) < 1e-12
    e = np.zeros((1, d))
    e[0, d // 2 - 1] = 1.0
    w = 10000.0 ** (-(d - 2) / d)
    r = rope_rotate(e, np.array([3]))[0]
    assert abs(r[d // 2 - 1] - math.cos(3 * w)) < 1e-14 and abs(r[d - 1] - math.sin(3 * w)) < 1e-14
    # Scores depend only on the offset between positions.
    a, b = rnd(rng, 1, d), rnd(rng, 1, d)
    for p1, p2, shift in [(5, 2, 11), (40, 0, 3), (9, 9, 100)]:
        s = (rope_rotate(a, np.array([p1])) @ rope_rotate(b, np.array([p2])).T)[0, 0]
        s2 = (rope_rotate(a, np.array([p1 + shift])) @ rope_rotate(b, np.array([p2 + shift])).T)[0, 0]
        assert abs(s - s2) < 1e-12


def test_rope_and_norm_commute_and_norm_value():
    rng = np.random.default_rng(13)
    x = rnd(rng, 30, 8) * 3.0
    pos = np.arange(30)
    eps = 1e-6
    a, _ = rms_normalize(rope_rotate(x, pos), eps)
    b = rope_rotate(rms_normalize(x, eps)[0], pos)
    np.testing.assert_allclose(a, b, atol=1e-14)
    y, r = rms_normalize(x, eps)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), ms / (ms + eps), rtol=1e-14)
    np.testing.assert_allclose(r[:, 0], np.sqrt(ms + eps), rtol=1e-15)


def test_mask_matches_page_conventions():
    """MiniGPT builds the allowed set as the lower triangle of ones; the GPT pretraining page masks
    the strict upper triangle; the KV-cache offset mask with q_len == k_len is the same mask."""
    T = 7
    m = visible_mask(T)
    np.testing.assert_array_equal(m, np.tril(np.ones((T, T))).astype(bool))
    np.testing.assert_array_equal(~m, np.triu(np.ones((T, T), dtype=bool), 1))
    rows, cols = np.arange(T)[:, None], np.arange(T)[None, :]
    np.testing.assert_array_equal(~m, cols > (0 + rows))
    for W in (1, 2, 5):
        np.testing.assert_array_equal(visible_mask(T, W).sum(axis=1), np.minimum(np.arange(T) + 1, W))


# ------------------------------------------------------------------------------------
# Decode.
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("flags", [dict(softcap=0.0, rope=False, qk_norm=False),
                                   dict(softcap=50.0, rope=True, qk_norm=False),
                                   dict(softcap=2.0, rope=True, qk_norm=True)])
def test_decode_equals_last_row_of_forward(flags):
    rng = np.random.default_rng(14)
    B, Hq, Hkv, T, d = 3, 4, 2, 15, 8
    q, k, v = rnd(rng, B, Hq, T, d), rnd(rng, B, Hkv, T, d), rnd(rng, B, Hkv, T, d)
    pos = np.arange(T)
    kc = rope_rotate(k, pos) if flags["rope"] else k.copy()
    if flags["qk_norm"]:
        kc = rms_normalize(kc)[0]
    Lmax = T + 4
    kcache = np.full((B, Hkv, Lmax, d), np.nan)
    vcache = np.full((B, Hkv, Lmax, d), np.nan)
    lens = np.array([T, 1, 9])
    for b in range(B):
        kcache[b, :, :T] = kc[b]
        vcache[b, :, :T] = v[b]
    assert attention_decode(q[:, :, -1], kcache, vcache, lens, **flags).shape == (B, Hq, d)
    for b in range(B):
        L = lens[b]
        O, _ = attention_forward(q[b:b + 1, :, :L], k[b:b + 1, :, :L], v[b:b + 1, :, :L], **flags)
        ob = attention_decode(q[b:b + 1, :, L - 1], kcache[b:b + 1], vcache[b:b + 1], lens[b:b + 1], **flags)
        np.testing.assert_allclose(ob[0], O[0, :, L - 1], atol=1e-14)


def test_decode_zero_length_and_clamp():
    rng = np.random.default_rng(15)
    q, kc, vc = rnd(rng, 3, 2, 4), rnd(rng, 3, 1, 6, 4), rnd(rng, 3, 1, 6, 4)
    o = attention_decode(q, kc, vc, np.array([0, -5, 99]))
    np.testing.assert_array_equal(o[0], 0.0)
    np.testing.assert_array_equal(o[1], 0.0)
    o_full = attention_decode(q[2:], kc[2:], vc[2:], np.array([6]))
    np.testing.assert_allclose(o[2], o_full[0], atol=0)


# ------------------------------------------------------------------------------------
# Packed rows: segment ids restrict attention to a token's own run; RoPE restarts per run.
# ------------------------------------------------------------------------------------
def test_segment_starts_examples():
    np.testing.assert_array_equal(segment_starts([7, 7, 3, 3, 3, 7]), [0, 0, 2, 2, 2, 5])
    np.testing.assert_array_equal(segment_starts([1]), [0])
    np.testing.assert_array_equal(segment_starts([0, 1, 2]), [0, 1, 2])
    np.testing.assert_array_equal(segment_starts([4, 4, 4]), [0, 0, 0])


def _packed_case(rng, B, Hq, Hkv, lengths, d):
    T = sum(lengths)
    q, k, v, dO = rnd(rng, B, Hq, T, d), rnd(rng, B, Hkv, T, d), rnd(rng, B, Hkv, T, d), rnd(rng, B, Hq, T, d)
    ids = np.concatenate([np.full(n, i % 3) for i, n in enumerate(lengths)])  # runs of 0,1,2,0,..
    return q, k, v, dO, np.tile(ids, (B, 1))


@pytest.mark.parametrize("flags", FLAG_SETS)
def test_packed_rows_equal_separate_sequences(flags):
    """A packed row is block-diagonal: each run gives what the same tokens give alone."""
    rng = np.random.default_rng(31)
    lengths = [5, 1, 7, 3]
    q, k, v, dO, ids = _packed_case(rng, 2, 4, 2, lengths, 8)
    O, L = attention_forward(q, k, v, segment_ids=ids, **flags)
    dQ, dK, dV = attention_backward(q, k, v, dO, segment_ids=ids, **flags)
    a = 0
    for n in lengths:
        sl = slice(a, a + n)
        Os, Ls = attention_forward(q[:, :, sl], k[:, :, sl], v[:, :, sl], **flags)
        gs = attention_backward(q[:, :, sl], k[:, :, sl], v[:, :, sl], dO[:, :, sl], **flags)
        np.testing.assert_allclose(O[:, :, sl], Os, atol=1e-13)
        np.testing.assert_allclose(L[:, :, sl], Ls, atol=1e-13)
        for g, r in zip((dQ, dK, dV), gs):
            np.testing.assert_allclose(g[:, :, sl], r, atol=1e-12)
        a += n


def test_packed_rows_match_brute_force():
    rng = np.random.default_rng(32)
    q, k, v, _, ids = _packed_case(rng, 1, 2, 1, [3, 4, 2], 6)
    flags = dict(window=3, softcap=2.0, rope=True, qk_norm=True)
    O, _ = attention_forward(q, k, v, segment_ids=ids, **flags)
    T, d = q.shape[2], q.shape[3]
    start = [0, 0, 0, 3, 3, 3, 3, 7, 7]
    for h, i in itertools.product(range(2), range(T)):
        qi = _bf_prologue(q[0, h, i], i - start[i], True, 10000.0, True, 1e-6)
        keys = [j for j in range(start[i], i + 1) if i - j < 3]
        sc = []
        for j in keys:
            kj = _bf_prologue(k[0, 0, j], j - start[j], True, 10000.0, True, 1e-6)
            s_ = sum(a * c for a, c in zip(qi, kj)) / math.sqrt(d)
            sc.append(2.0 * math.tanh(s_ / 2.0))
        w = [math.exp(x - max(sc)) for x in sc]
        ref = sum(wj / sum(w) * v[0, 0, j] for wj, j in zip(w, keys))
        np.testing.assert_allclose(O[0, h, i], ref, atol=1e-12)


def test_packed_gradients_match_finite_differences():
    rng = np.random.default_rng(33)
    q, k, v, dO, ids = _packed_case(rng, 1, 2, 1, [2, 3, 2], 4)
    flags = dict(window=0, softcap=1.5, rope=True, qk_norm=True)
    grads = attention_backward(q, k, v, dO, segment_ids=ids, **flags)
    f = lambda qq, kk, vv: float(np.sum(attention_forward(qq, kk, vv, segment_ids=ids, **flags)[0] * dO))
    eps = 1e-6
    for which, x in enumerate((q, k, v)):
        for idx in [(0, 0, 1, 2), (0, 0, 4, 0), (0, 0, 6, 3)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num = (f(*args_p) - f(*args_m)) / (2 * eps)
            np.testing.assert_allclose(grads[which][idx], num, rtol=1e-6, atol=1e-8)


def test_single_run_is_plain_attention():
    rng = np.random.default_rng(34)
    q, k, v, dO = rnd(rng, 2, 2, 9, 8), rnd(rng, 2, 1, 9, 8), rnd(rng, 2, 1, 9, 8), rnd(rng, 2, 2, 9, 8)
    ids = np.full((2, 9), 5)
    flags = dict(softcap=3.0, rope=True, qk_norm=True)
    np.testing.assert_allclose(attention_forward(q, k, v, segment_ids=ids, **flags)[0],
                               attention_forward(q, k, v, **flags)[0], atol=0)
    for a, b in zip(attention_backward(q, k, v, dO, segment_ids=ids, **flags),
                    attention_backward(q, k, v, dO, **flags)):
        np.testing.assert_allclose(a, b, atol=0)


# ------------------------------------------------------------------------------------
# Extend: S new tokens against a KV cache (append, then attend with the offset mask).
# ------------------------------------------------------------------------------------
def brute_force_extend(q, kn, vn, kc, vc, lens, window, softcap, rope, qk_norm, base=10000.0,
                       eps=1e-6, starts=None):
    B, Hq, S, d = q.shape
    Hkv, Lmax = kc.shape[1], kc.shape[2]
    scale = 1.0 / math.sqrt(d)
    O = np.zeros((B, Hq, S, d))
    K, V = kc.copy(), vc.copy()
    for b in range(B):
        L = min(max(int(lens[b]), 0), Lmax)
        s0 = 0 if starts is None else min(max(int(starts[b]), 0), Lmax)  # left padding rows
        for g, i in itertools.product(range(Hkv), range(S)):
            if L + i < Lmax:
                K[b, g, L + i] = _bf_prologue(kn[b, g, i], L + i - s0, rope, base, qk_norm, eps)
                V[b, g, L + i] = vn[b, g, i]
        for h, i in itertools.product(range(Hq), range(S)):
            p = L + i
            if p >= Lmax or p < s0:
                continue
            g = h * Hkv // Hq
            qi = _bf_prologue(q[b, h, i], p - s0, rope, base, qk_norm, eps)
            keys = [j for j in range(s0, p + 1) if window == 0 or p - j < window]
            sc = []
            for j in keys:
                s_ = scale * sum(a * c for a, c in zip(qi, K[b, g, j]))
                sc.append(softcap * math.tanh(s_ / softcap) if softcap else s_)
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            for jj, j in enumerate(keys):
                O[b, h, i] += w[jj] / sum(w) * V[b, g, j]
    return O, K, V


@pytest.mark.parametrize("flags", FLAG_SETS)
def test_extend_matches_brute_force(flags):
    rng = np.random.default_rng(21)
    B, Hq, Hkv, S, d, Lmax = 3, 4, 2, 3, 6, 8
    q, kn, vn = rnd(rng, B, Hq, S, d), rnd(rng, B, Hkv, S, d), rnd(rng, B, Hkv, S, d)
    kc, vc = rnd(rng, B, Hkv, Lmax, d), rnd(rng, B, Hkv, Lmax, d)
    lens = np.array([2, 0, 6])  # the last sequence overflows: only 2 of its 3 tokens fit
    O, K, V = attention_extend(q, kn, vn, kc, vc, lens, **flags)
    Ob, Kb, Vb = brute_force_extend(q, kn, vn, kc, vc, lens, **flags)
    np.testing.assert_allclose(O, Ob, atol=1e-12)
    np.testing.assert_allclose(K, Kb, atol=1e-12)
    np.testing.assert_allclose(V, Vb, atol=0)
    np.testing.assert_array_equal(O[2, :, 2], 0.0)


@pytest.mark.parametrize("flags", FLAG_SETS)
def test_extend_on_empty_cache_is_the_forward(flags):
    rng = np.random.default_rng(22)
    B, Hq, Hkv, T, d = 2, 4, 2, 9, 8
    q, k, v = rnd(rng, B, Hq, T, d), rnd(rng, B, Hkv, T, d), rnd(rng, B, Hkv, T, d)
    kc, vc = rnd(rng, B, Hkv, T + 3, d), rnd(rng, B, Hkv, T + 3, d)
    O, K, V = attention_extend(q, k, v, kc, vc, np.zeros(B, int), **flags)
    Of, _ = attention_forward(q, k, v, **flags)
    np.testing.assert_allclose(O, Of, atol=1e-13)
    kr = rope_rotate(k, np.arange(T)) if flags["rope"] else k
    kr = rms_normalize(kr)[0] if flags["qk_norm"] else kr
    np.testing.assert_allclose(K[:, :, :T], kr, atol=1e-14)
    np.testing.assert_array_equal(V[:, :, :T], v)
    np.testing.assert_array_equal(K[:, :, T:], kc[:, :, T:])  # rows past the new ones untouched


@pytest.mark.parametrize("flags", FLAG_SETS[:3])
def test_extend_one_token_is_decode(flags):
    rng = np.random.default_rng(23)
    B, Hq, Hkv, d, Lmax = 3, 4, 2, 8, 12
    q, kn, vn = rnd(rng, B, Hq, 1, d), rnd(rng, B, Hkv, 1, d), rnd(rng, B, Hkv, 1, d)
    kc, vc = rnd(rng, B, Hkv, Lmax, d), rnd(rng, B, Hkv, Lmax, d)
    lens = np.array([0, 5, 11])
    O, K, V = attention_extend(q, kn, vn, kc, vc, lens, **flags)
    dec = attention_decode(q[:, :, 0], K, V, lens + 1,
                           **{a: b for a, b in flags.items() if a != "window"})
    np.testing.assert_allclose(O[:, :, 0], dec, atol=1e-13)


@pytest.mark.parametrize("flags", FLAG_SETS)
def test_extend_chunks_compose(flags):
    rng = np.random.default_rng(24)
    B, Hq, Hkv, S1, S2, d, Lmax = 2, 2, 1, 3, 4, 8, 16
    q, kn, vn = rnd(rng, B, Hq, S1 + S2, d), rnd(rng, B, Hkv, S1 + S2, d), rnd(rng, B, Hkv, S1 + S2, d)
    kc, vc = rnd(rng, B, Hkv, Lmax, d), rnd(rng, B, Hkv, Lmax, d)
    lens = np.array([4, 1])
    O, K, V = attention_extend(q, kn, vn, kc, vc, lens, **flags)
    O1, K1, V1 = attention_extend(q[:, :, :S1], kn[:, :, :S1], vn[:, :, :S1], kc, vc, lens, **flags)
    O2, K2, V2 = attention_extend(q[:, :, S1:], kn[:, :, S1:], vn[:, :, S1:], K1, V1, lens + S1,
                                  **flags)
    np.testing.assert_allclose(O, np.concatenate([O1, O2], axis=2), atol=1e-13)
    np.testing.assert_allclose(K, K2, atol=0)
    np.testing.assert_allclose(V, V2, atol=0)


@pytest.mark.parametrize("flags", FLAG_SETS)
def test_extend_is_the_forward_suffix(flags):
    """A cache filled with the first L prepared keys, then S more tokens: the outputs are the
    last S rows of the forward over the whole sequence."""
    rng = np.random.default_rng(25)
    B, Hq, Hkv, T, d = 3, 4, 2, 11, 8
    q, k, v = rnd(rng, B, Hq, T, d), rnd(rng, B, Hkv, T, d), rnd(rng, B, Hkv, T, d)
    Of, _ = attention_forward(q, k, v, **flags)
    kr = rope_rotate(k, np.arange(T)) if flags["rope"] else k
    kr = rms_normalize(kr)[0] if flags["qk_norm"] else kr
    for L in (0, 4, T - 1):
        kc = np.full((B, Hkv, T, d), np.nan)
        vc = np.full((B, Hkv, T, d), np.nan)
        kc[:, :, :L], vc[:, :, :L] = kr[:, :, :L], v[:, :, :L]
        O, K, V = attention_extend(q[:, :, L:], k[:, :, L:], v[:, :, L:], kc, vc,
                                   np.full(B, L), **flags)
        np.testing.assert_allclose(O, Of[:, :, L:], atol=1e-13)
        np.testing.assert_allclose(K, kr, atol=1e-14)


def test_extend_clamps_and_leaves_inputs():
    rng = np.random.default_rng(26)
    q, kn, vn = rnd(rng, 2, 2, 3, 4), rnd(rng, 2, 1, 3, 4), rnd(rng, 2, 1, 3, 4)
    kc, vc = rnd(rng, 2, 1, 5, 4), rnd(rng, 2, 1, 5, 4)
    kc0, vc0 = kc.copy(), vc.copy()
    O, K, V = attention_extend(q, kn, vn, kc, vc, np.array([-4, 99]))
    np.testing.assert_array_equal(kc, kc0)
    np.testing.assert_array_equal(vc, vc0)
    Oz, _, _ = attention_extend(q[:1], kn[:1], vn[:1], kc[:1], vc[:1], np.array([0]))
    np.testing.assert_allclose(O[0], Oz[0], atol=0)  # negative length counts as 0
    np.testing.assert_array_equal(O[1], 0.0)  # a full cache stores nothing and attends nothing
    np.testing.assert_array_equal(K[1], kc[1])


# ------------------------------------------------------------------------------------
# Workload shapes come from the pages.
# ------------------------------------------------------------------------------------
def test_workload_shapes_match_pages():
    from causal_attention_02_amd.inputs import WORKLOADS
    ps = json.load(open(os.path.join(GOLDEN, "page_shapes.json")))
    mg, nano, fc = ps["minigpt"], ps["nanogpt_181m"], ps["flaxchat_depth12"]
    w = WORKLOADS["minigpt_fwd_f32"]
    assert (w.T, w.Hq, w.D) == (mg["maxlen"], mg["num_heads"], mg["embed_dim"] // mg["num_heads"])
    w = WORKLOADS["minigpt_train_bf16"]
    assert (w.B, w.T, w.Hq, w.D) == (mg["batch_size"], mg["maxlen"], mg["num_heads"], 32)
    for name in ("gqa181m_train", "gqa181m_decode"):
        w = WORKLOADS[name]
        assert (w.Hq, w.Hkv, w.D, w.T) == (nano["query_heads"], nano["kv_heads"], nano["head_dim"],
                                           nano["sequence_length"])
    for name in ("flaxchat_full", "flaxchat_w512"):
        w = WORKLOADS[name]
        assert (w.Hq, w.Hkv, w.D) == (fc["heads"], fc["kv_heads"], fc["model_dim"] // fc["heads"])
    gp, g2 = ps["gpt_pretrain"], ps["gpt2_family"]
    w = WORKLOADS["gpt_pretrain_train"]
    assert (w.B, w.T, w.Hq, w.Hkv, w.D) == (gp["batch_size"], gp["context_length"], gp["num_heads"],
                                            gp["num_heads"], gp["d_model"] // gp["num_heads"])
    w = WORKLOADS["gpt_pretrain_train_dropout"]
    assert (w.B, w.T, w.Hq, w.Hkv, w.D, w.dropout) == (
        gp["batch_size"], gp["context_length"], gp["num_heads"], gp["num_heads"],
        gp["d_model"] // gp["num_heads"], gp["mha_dropout_rate"])
    w = WORKLOADS["gpt_pretrain_decode"]
    demo = gp["kv_cache_demo"]
    assert (w.B, w.T, w.len_lo, w.Hq, w.D) == (demo["batch"], demo["context_length"],
                                               demo["context_length"], gp["num_heads"], 64)
    w = WORKLOADS["gpt2xl_instruct_train"]
    d_model, heads = g2["sizes"][-1]
    assert (w.B, w.T, w.Hq, w.Hkv, w.D) == (g2["batch_size"], g2["context_length"], heads, heads,
                                            d_model // heads)
    assert all(dm // h == 64 for dm, h in g2["sizes"])


# ------------------------------------------------------------------------------------
# Attention dropout ("GPT pretraining" page, "Multihead Attention").
# ------------------------------------------------------------------------------------
_M64 = (1 << 64) - 1


def philox4x64_10(ctr, key):
    """Philox4x64-10 from its published definition (Salmon et al., SC 2011), scalar Python.

    Round: (hi0, lo0) = M0 * x0, (hi1, lo1) = M1 * x2 (128-bit products);
    x <- (hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0); the key is bumped by the Weyl
    constants between rounds.
    """
    m0, m1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157
    w0, w1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B
    x = [int(c) & _M64 for c in ctr]
    k0, k1 = int(key[0]) & _M64, int(key[1]) & _M64
    for r in range(10):
        if r:
            k0, k1 = (k0 + w0) & _M64, (k1 + w1) & _M64
        p0, p1 = m0 * x[0], m1 * x[2]
        x = [(p1 >> 64) ^ x[1] ^ k0, p1 & _M64, (p0 >> 64) ^ x[3] ^ k1, p0 & _M64]
    return x


def test_philox_definition_matches_numpy():
    # The scalar definition above against numpy's Philox bit generator (which encrypts the
    # counter after incrementing it).
    rng = np.random.default_rng(40)
    for n in range(50):
        ctr = [int(c) for c in rng.integers(0, 2 ** 63, 4, dtype=np.int64)]
        key = [int(c) for c in rng.integers(0, 2 ** 63, 2, dtype=np.int64)]
        if n < 3:
            ctr = [n, 0, 0, 0]
        c = sum(v << (64 * i) for i, v in enumerate(ctr))
        gen = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=(c - 1) % (1 << 256))
        assert [int(w) for w in gen.random_raw(4)] == philox4x64_10(ctr, key)


def test_dropout_fields_follow_the_counter_layout():
    # Field of key j for query i of head (b, h): block (j // 16, i, b H + h, offset) under key
    # (seed, 0), word (j % 16) // 4, bits 16 (j % 4) ...
    for (b, h, H, i, T, seed, offset) in [(0, 0, 1, 0, 5, 0, 0), (1, 2, 3, 7, 40, 42, 5),
                                          (3, 11, 12, 255, 256, 2 ** 63 + 9, 2 ** 40)]:
        got = dropout_fields(b, h, H, i, T, seed, offset)
        want = []
        for j in range(T):
            blk = philox4x64_10([j // 16, i, b * H + h, offset], [seed, 0])
            want.append((blk[(j % 16) // 4] >> (16 * (j % 4))) & 0xFFFF)
        assert got.tolist() == want


def test_dropout_threshold_values():
    assert dropout_threshold(0.0) == (0, 1.0)
    assert dropout_threshold(0.5) == (32768, 2.0)
    t, sc = dropout_threshold(0.1)
    assert t == 6554 and sc == 65536.0 / (65536 - 6554)
    assert dropout_threshold(1.0 - 2.0 ** -16)[0] == 65535
    for bad in (-0.1, 1.0, 0.99999999):
        with pytest.raises(ValueError):
            dropout_threshold(bad)


def test_dropout_keep_rate_and_independence():
    B, H, T = 2, 3, 96
    for p in (0.1, 0.5):
        keep = dropout_keep(B, H, T, p, seed=42, offset=0)
        t, _ = dropout_threshold(p)
        q = t / 65536.0
        n = keep.size
        assert abs((1.0 - keep.mean()) - q) < 5 * math.sqrt(q * (1 - q) / n)
        # Another seed, another offset, another head: agreement as for independent draws.
        for other in (dropout_keep(B, H, T, p, seed=43, offset=0),
                      dropout_keep(B, H, T, p, seed=42, offset=1)):
            agree = np.mean(keep == other)
            e = q * q + (1 - q) * (1 - q)
            assert abs(agree - e) < 5 * math.sqrt(e * (1 - e) / n)
        assert not np.array_equal(keep[0, 0], keep[0, 1])
        assert not np.array_equal(keep[0, 0], keep[1, 0])
    assert dropout_keep(1, 2, 33, 0.0, seed=1).all()


def brute_force_dropout_forward(q, k, v, keep, scale_d):
    """Plain causal attention with the weights multiplied by keep * scale_d; scalar loops."""
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    O = np.zeros((B, Hq, T, d))
    for b, h, i in itertools.product(range(B), range(Hq), range(T)):
        g = h * Hkv // Hq
        s = [sum(q[b, h, i, c] * k[b, g, j, c] for c in range(d)) / math.sqrt(d) for j in range(i + 1)]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        tot = sum(w)
        for j in range(i + 1):
            if keep[b, h, i, j]:
                O[b, h, i] += (w[j] / tot) * scale_d * v[b, g, j]
    return O


def test_dropout_forward_matches_brute_force():
    rng = np.random.default_rng(41)
    for (Hq, Hkv, T, d, p) in [(2, 1, 7, 4, 0.3), (3, 3, 18, 2, 0.1), (4, 2, 33, 8, 0.5)]:
        q, k, v = rnd(rng, 2, Hq, T, d), rnd(rng, 2, Hkv, T, d), rnd(rng, 2, Hkv, T, d)
        keep = dropout_keep(2, Hq, T, p, seed=7, offset=3)
        O, L = attention_forward(q, k, v, dropout_p=p, dropout_keep=keep)
        _, sc = dropout_threshold(p)
        np.testing.assert_allclose(O, brute_force_dropout_forward(q, k, v, keep, sc), atol=1e-12)
        np.testing.assert_allclose(L, attention_forward(q, k, v)[1], atol=0)


@pytest.mark.parametrize("flags", FLAG_SETS)
def test_dropout_special_cases(flags):
    rng = np.random.default_rng(42)
    q, k, v, dO = rnd(rng, 1, 2, 9, 4), rnd(rng, 1, 1, 9, 4), rnd(rng, 1, 1, 9, 4), rnd(rng, 1, 2, 9, 4)
    plain = attention_forward(q, k, v, **flags)
    # Rate 0 keeps everything at scale 1.
    keep0 = dropout_keep(1, 2, 9, 0.0, seed=3)
    np.testing.assert_array_equal(attention_forward(q, k, v, dropout_p=0.0, dropout_keep=keep0,
                                                    **flags)[0], plain[0])
    # Everything kept at rate 1/2: twice the output, twice the gradients of <O, dO>.
    allk = np.ones((1, 2, 9, 9), dtype=bool)
    np.testing.assert_allclose(attention_forward(q, k, v, dropout_p=0.5, dropout_keep=allk,
                                                 **flags)[0], 2 * plain[0], atol=1e-14)
    for a, b in zip(attention_backward(q, k, v, dO, dropout_p=0.5, dropout_keep=allk, **flags),
                    attention_backward(q, k, v, dO, **flags)):
        np.testing.assert_allclose(a, 2 * b, atol=1e-12)
    # Nothing kept: zero output and zero gradients.
    nok = np.zeros((1, 2, 9, 9), dtype=bool)
    assert not attention_forward(q, k, v, dropout_p=0.5, dropout_keep=nok, **flags)[0].any()
    for a in attention_backward(q, k, v, dO, dropout_p=0.5, dropout_keep=nok, **flags):
        np.testing.assert_allclose(a, 0, atol=1e-15)


@pytest.mark.parametrize("flags", FLAG_SETS[:3])
def test_dropout_gradients_match_finite_differences(flags):
    rng = np.random.default_rng(43)
    B, Hq, Hkv, T, d, p = 1, 2, 1, 7, 4, 0.3
    q, k, v, dO = rnd(rng, B, Hq, T, d), rnd(rng, B, Hkv, T, d), rnd(rng, B, Hkv, T, d), rnd(rng, B, Hq, T, d)
    keep = dropout_keep(B, Hq, T, p, seed=11, offset=0)
    kw = dict(dropout_p=p, dropout_keep=keep, **flags)
    grads = attention_backward(q, k, v, dO, **kw)
    f = lambda qq, kk, vv: float(np.sum(attention_forward(qq, kk, vv, **kw)[0] * dO))
    eps = 1e-6
    for which, x in enumerate((q, k, v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p, args_m = [q, k, v], [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (f(*args_p) - f(*args_m)) / (2 * eps)
        np.testing.assert_allclose(grads[which], num, rtol=0, atol=2e-7)


def test_dropout_is_unbiased():
    # Inverted dropout: the mean output over independent masks tends to the plain output.
    rng = np.random.default_rng(44)
    q, k, v = rnd(rng, 1, 1, 6, 4), rnd(rng, 1, 1, 6, 4), rnd(rng, 1, 1, 6, 4)
    plain = attention_forward(q, k, v)[0]
    p, n = 0.3, 600
    outs = np.stack([attention_forward(q, k, v, dropout_p=p,
                                       dropout_keep=dropout_keep(1, 1, 6, p, seed=s))[0]
                     for s in range(n)])
    se = outs.std(axis=0) / math.sqrt(n)
    assert np.all(np.abs(outs.mean(axis=0) - plain) <= 5 * se + 1e-12)


# ------------------------------------------------------------------------------------
# Left-padded batches (181M model card, inference notes): rows below cache_start[b] are padding.
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("flags", FLAG_SETS)
def test_leftpad_extend_matches_brute_force(flags):
    rng = np.random.default_rng(50)
    B, Hq, Hkv, S, d, Lmax = 4, 2, 1, 6, 4, 12
    q, kn, vn = rnd(rng, B, Hq, S, d), rnd(rng, B, Hkv, S, d), rnd(rng, B, Hkv, S, d)
    kc, vc = rnd(rng, B, Hkv, Lmax, d), rnd(rng, B, Hkv, Lmax, d)
    lens, starts = np.array([0, 3, 5, 9]), np.array([2, 1, 5, 11])
    got = attention_extend(q, kn, vn, kc, vc, lens, cache_start=starts, **flags)
    want = brute_force_extend(q, kn, vn, kc, vc, lens, starts=starts, **flags)
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, b, atol=1e-12)


@pytest.mark.parametrize("flags", FLAG_SETS[:3])
def test_leftpad_decode_equals_compact_slice(flags):
    # Padding rows (filled with large garbage) change nothing; the query sits at position
    # L - 1 - S of the compact sequence.
    flags = {k: v for k, v in flags.items() if k != "window"}
    rng = np.random.default_rng(51)
    B, Hq, Hkv, d, Lmax = 4, 4, 2, 8, 20
    q = rnd(rng, B, Hq, d)
    compact = rnd(rng, B, Hkv, Lmax, d), rnd(rng, B, Hkv, Lmax, d)
    lens = np.array([5, 1, 20, 7])
    starts = np.array([3, 0, 0, 13])
    kc, vc = 1e3 * rnd(rng, B, Hkv, Lmax, d), 1e3 * rnd(rng, B, Hkv, Lmax, d)
    for b in range(B):
        n = min(lens[b], Lmax - starts[b])
        kc[b, :, starts[b]:starts[b] + n] = compact[0][b, :, :n]
        vc[b, :, starts[b]:starts[b] + n] = compact[1][b, :, :n]
    got = attention_decode(q, kc, vc, np.minimum(starts + lens, Lmax), cache_start=starts, **flags)
    want = attention_decode(q, compact[0], compact[1], np.minimum(lens, Lmax - starts), **flags)
    np.testing.assert_allclose(got, want, atol=1e-12)
    # start at or past the length: an empty slice, a zero row
    z = attention_decode(q, kc, vc, np.array([3, 0, 4, 2]), cache_start=np.array([3, 0, 9, 2]),
                         **flags)
    assert not z.any()


@pytest.mark.parametrize("flags", FLAG_SETS)
def test_leftpad_prefill_equals_forward_of_each_prompt(flags):
    # A left-padded batch prefilled in one extend step: each prompt's rows equal the causal
    # forward of that prompt alone, padding rows are zero, and the stored keys are the
    # prompt's own (rotated from position 0).
    rng = np.random.default_rng(52)
    B, Hq, Hkv, S, d = 3, 2, 1, 9, 4
    pads = np.array([0, 4, 8])
    q, kn, vn = rnd(rng, B, Hq, S, d), rnd(rng, B, Hkv, S, d), rnd(rng, B, Hkv, S, d)
    kc, vc = np.zeros((B, Hkv, S, d)), np.zeros((B, Hkv, S, d))
    o, K, V = attention_extend(q, kn, vn, kc, vc, np.zeros(B, dtype=int), cache_start=pads,
                               **flags)
    for b in range(B):
        P = pads[b]
        ref, _ = attention_forward(q[b:b + 1, :, P:], kn[b:b + 1, :, P:], vn[b:b + 1, :, P:],
                                   **flags)
        np.testing.assert_allclose(o[b, :, P:], ref[0], atol=1e-12)
        assert not o[b, :, :P].any()
        _, Kc, _ = attention_extend(q[b:b + 1, :, P:], kn[b:b + 1, :, P:], vn[b:b + 1, :, P:],
                                    kc[b:b + 1, :, :S - P], vc[b:b + 1, :, :S - P], [0], **flags)
        np.testing.assert_allclose(K[b, :, P:], Kc[0], atol=1e-12)
