// Host-side interface between the C ABI (attn_api.hip) and the kernel files.
// Every launcher enqueues on the given stream and returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "device_common.h"

namespace attn {

// Kernel tracing: brackets each launch by a pair of events while enabled.
struct TraceScope {
  TraceScope(const char* name, hipStream_t stream);
  ~TraceScope();
  int slot;
  hipStream_t stream;
};

// ---- score mode selection ---------------------------------------------------------------
// With QK-norm every normalised row has |x^| <= sqrt(D), so |S_pre| <= scale * D.  When that
// bound is small the softmax can use it as a fixed shift (exact: softmax is shift invariant,
// and exp2(y - shift) stays far above the fp32 underflow threshold), and the soft-cap's tanh
// argument is small enough for its Taylor polynomial.
struct ScoreSetup {
  int mode;          // kScoreScale / kScoreCapExp / kScoreCapPoly
  int fixed_shift;   // 1: use `shift` instead of a running maximum (forward)
  float shift;       // log2 units
  ScoreCoef coef;
};

inline ScoreSetup make_score_setup(float scale, float softcap, int D, int qk_norm) {
  ScoreSetup s{};
  const double log2e = 1.4426950408889634;
  // Bound with slack for the bf16 rounding of q^ and k^ (relative 2^-8 each).
  const double bound = qk_norm ? (double)scale * D * (1.0 + 1.0 / 64) : INFINITY;
  s.fixed_shift = bound <= 30.0;
  s.shift = s.fixed_shift ? (float)(bound * log2e) : 0.f;
  if (softcap <= 0.f) {
    s.mode = kScoreScale;
    s.coef.k0 = (float)(scale * log2e);
  } else if (s.fixed_shift && bound / softcap <= 0.25) {
    // y = c log2e tanh(a scale / c) = a * sum_k t_k (scale/c)^(2k+1) c log2e a^(2k)
    const double x = (double)scale / softcap, k1 = (double)softcap * log2e;
    const double xm = bound / softcap;  // largest |S_pre / c|
    // First dropped terms of the degree-5 cut: tanh's x^7 term (in y units) and sech^2's
    // x^6 term (relative); the series alternate with shrinking terms for |x| < pi/2.
    const double tail_y = k1 * (17.0 / 315) * pow(xm, 7), tail_g = (17.0 / 45) * pow(xm, 6);
    const double tol = 1.0 / 4096;
    s.mode = (tail_y <= tol && tail_g <= tol) ? kScoreCapPoly5 : kScoreCapPoly;
    const double t[5] = {1.0, -1.0 / 3, 2.0 / 15, -17.0 / 315, 62.0 / 2835};
    double pw = x;
    float* p[5] = {&s.coef.p1, &s.coef.p3, &s.coef.p5, &s.coef.p7, &s.coef.p9};
    for (int i = 0; i < 5; ++i) {
      *p[i] = (float)(t[i] * pw * k1);
      pw *= x * x;
    }
    s.coef.k1 = (float)k1;
    s.coef.inv_k1_sq = (float)(1.0 / (k1 * k1));
    s.coef.g2 = (float)(-x * x);
    s.coef.g4 = (float)(2.0 / 3 * x * x * x * x);
  } else {
    s.mode = kScoreCapExp;
  }
  // The raw score that stands in for a masked entry of an edge tile, so that masked and
  // unmasked tiles share one body (set before the score transform).  Without a bound on the
  // shift (plain scores), -1e30.  The polynomial modes run under the QK-norm bound, so a row's
  // shift lies within about +-60 (log2 units); their transform is a * q(a^2) with q >= 0.72 p1
  // for every a (both truncations of tanh(x)/x stay above 0.72), so a = -1024 / (0.72 p1)
  // gives y <= -1024: a weight of exactly 0 under any such shift, with the slope factor of the
  // backward still finite.  Checked below with the kernels' own float formulas.
  if (s.mode == kScoreScale) {
    s.coef.mask_acc = -1.0e30f;
  } else if (s.mode != kScoreCapExp) {
    const float m = (float)(-1024.0 / (0.72 * (double)s.coef.p1));
    const float a2 = m * m;
    bool ok;
    if (s.mode == kScoreCapPoly5) {
      const float y = m * fmaf(a2, fmaf(a2, s.coef.p5, s.coef.p3), s.coef.p1);
      const float g = fmaf(a2, fmaf(a2, s.coef.g4, s.coef.g2), 1.f);
      ok = isfinite(y) && y <= -1024.f && isfinite(g);
    } else {
      float q = fmaf(a2, s.coef.p9, s.coef.p7);
      q = fmaf(a2, q, s.coef.p5);
      q = fmaf(a2, q, s.coef.p3);
      q = fmaf(a2, q, s.coef.p1);
      const float u = m * q;
      ok = isfinite(u) && u <= -1024.f && isfinite(u * u * s.coef.inv_k1_sq);
    }
    if (ok) s.coef.mask_acc = m;
    else s.mode = kScoreCapExp;  // the general form (masks after the transform)
  }
  if (s.mode == kScoreCapExp) {
    s.coef.k0 = (float)(2.0 * scale * log2e / softcap);
    s.coef.k1 = (float)(softcap * log2e);
    s.coef.inv_k1_sq = (float)(1.0 / ((double)s.coef.k1 * s.coef.k1));
  }
  return s;
}

inline RowPrologue make_row_prologue(int rope, float rope_base, int qk_norm, float eps, int D) {
  RowPrologue r{};
  r.rope = rope;
  r.qk_norm = qk_norm;
  r.eps = eps;
  const double two_pi = 6.283185307179586;
  for (int i = 0; i < D / 2 && i < 64; ++i)
    r.omega_rev[i] = rope ? pow((double)rope_base, -2.0 * i / D) / two_pi : 0.0;
  return r;
}

// ---- row passes (rowops.hip) -------------------------------------------------------------
// y = N(R(x)) for rows of length D; row r sits at position r % T.  elt = 2 (bf16) or 4 (f32).
// segment ids [B, T] -> first / last token index of every token's run (packed rows).
hipError_t launch_segment_bounds(const int32_t* ids, int32_t* start, int32_t* end, int B, int T,
                                 hipStream_t s);
// k_new/v_new [B, Hkv, S, D] -> cache rows cache_len[b] + i (RoPE at that row minus
// cache_start[b], or at the row itself when cache_start is null; QK-norm); rows at or past
// Lmax are not written.
hipError_t launch_append_kv(const void* kn, const void* vn, void* kc, void* vc,
                            const int32_t* cache_len, const int32_t* cache_start, int B, int Hkv,
                            int S, int Lmax, int D, int rope, float rope_base, int qk_norm,
                            float eps, hipStream_t s);
hipError_t launch_prologue(const void* x, void* y, int64_t rows, int T, int D, int elt, int rope,
                           float rope_base, int qk_norm, float eps, hipStream_t s);
// Backward preparation over the [B, Hq, T] query rows: nD = -rowsum(dO * O), L2 = LSE * log2(e)
// and, when qh is not null, qh = N(R(q)) (bf16).
hipError_t launch_bwd_prep(const void* q, const void* o, const void* dO, const float* lse,
                           void* qh, float* nD, float* L2, int64_t rows, int T, int D, int rope,
                           float rope_base, int qk_norm, float eps, hipStream_t s);

// ---- attention dropout (dropout.hip) ------------------------------------------------------
// Keep masks, one bit per (query, key): 32-bit words, `dropout_pitch(T)` words per row (an even
// count, so the attention kernels' 64-wide tiles always read whole word pairs).
inline int dropout_pitch(int T) { return 2 * ((T + 63) / 64); }
// rows [B, H, T, pitch]: bit c of word w of row i keeps (i, 32 w + c); cols [B, H, T, pitch]:
// bit c of word w of row j keeps (32 w + c, j).  Only words of 32 x 32 tiles that meet the
// causal / window band are written.  Keep iff the element's 16-bit Philox field >= thr.
hipError_t launch_dropout_mask(uint32_t* rows, uint32_t* cols, int B, int H, int T, int window,
                               uint32_t thr, uint64_t seed, uint64_t offset, hipStream_t s);

// ---- forward (fwd.hip) -------------------------------------------------------------------
struct FwdParams {
  const void* q;  // [B, Hq, T, D] raw q (bf16: RoPE/QK-norm applied in the kernel)
  const void* k;  // [B, Hkv, T, D] k^ (already through the prologue)
  const void* v;
  void* o;
  float* lse;
  int B, T, Hq, Hkv, D, window;
  float scale, softcap;
  int rope;
  float rope_base;
  int qk_norm;
  float eps;
  // Extend mode: q holds T new tokens per sequence, k/v are caches of Lmax rows per head
  // (already holding the new keys), query i sits at position cache_len[b] + i.
  const int32_t* cache_len = nullptr;
  int Lmax = 0;
  // Left-padded batches (extend only): rows below cache_start[b] are padding, positions count
  // from there, and new tokens in padding rows get zero output rows (null: no padding).
  const int32_t* cache_start = nullptr;
  // Packed rows: first token index of every token's run, [B, T] (null: one run per row).
  const int32_t* seg_start = nullptr;
  // Dropout on the weights: row-layout keep mask (null: none) and the kept-weight scale.
  const uint32_t* drop_rows = nullptr;
  float drop_scale = 1.f;
};
hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t s);
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t s);  // q, k already prologued

// ---- dS fragments (split backward) ----------------------------------------------------------
// The dK/dV pass stores dS (bf16) of every (32-query block i, 16-key block j) that holds a
// visible pair as one 1 KB fragment: 64 lanes x 8 values in the B-operand layout of
// v_mfma_f32_32x32x16_bf16 (lane l: query 32 i + l % 32, keys 16 j + 8 (l / 32) + 0..7).
// Block i spans key blocks lo_i .. hi_i with hi_i = min(2 i + 1, nkb - 1) and lo_i =
// floor(max(0, 32 i - W + 1) / 16) (0 without a window).  Without a window (or W >= T) the
// fragments of a head are packed as a triangle, index i (i + 1) + j; with one, as a band of
// `stride` fragments per block, index i stride + j - lo_i.
struct DsBand {
  int nqb, nkb;     // 32-query blocks, 16-key blocks
  int window;       // W when 0 < W < T, else 0
  int stride;       // 0: triangle; else fragments per query block
  int64_t frags;    // fragments per (b, h)
};
inline DsBand make_ds_band(int T, int window) {
  DsBand d{};
  d.nqb = (T + 31) / 32;
  d.nkb = (T + 15) / 16;
  d.window = (window > 0 && window < T) ? window : 0;
  if (d.window == 0) {
    d.stride = 0;
    d.frags = (int64_t)d.nqb * (d.nqb + 1);
  } else {
    int S = 1;
    for (int i = 0; i < d.nqb; ++i) {
      const int hi = 2 * i + 1 < d.nkb - 1 ? 2 * i + 1 : d.nkb - 1;
      const int lo = (32 * i - d.window + 1 > 0 ? 32 * i - d.window + 1 : 0) / 16;
      if (hi - lo + 1 > S) S = hi - lo + 1;
    }
    d.stride = S;
    d.frags = (int64_t)d.nqb * S;
  }
  return d;
}

// ---- backward (bwd.hip) ------------------------------------------------------------------
struct BwdParams {
  const void* q;     // raw q (bf16) [B, Hq, T, D]
  const void* k;     // raw k (bf16) [B, Hkv, T, D]
  const void* kh;    // k^ (bf16) for the dq pass (== k without RoPE/QK-norm)
  void* qh;          // q^ (bf16) written by the dq pass for the dkdv pass (== q without them)
  const void* v;
  const void* o;
  const void* dO;
  const float* lse;  // [B, Hq, T]
  float* Dvec;       // [B, Hq, T] -rowsum(dO * O), written by the dq pass
  float* L2;         // [B, Hq, T] LSE * log2(e), written by the dq pass
  void* dq;
  void* dk;
  void* dv;
  int B, T, Hq, Hkv, D, window;
  float scale, softcap;
  int rope;
  float rope_base;
  int qk_norm;
  float eps;
  // Packed rows: first / last token index of every token's run, [B, T] (null: one run).
  const int32_t* seg_start = nullptr;
  const int32_t* seg_end = nullptr;
  // Dropout on the weights: keep masks in both layouts (null: none), kept-weight scale.
  const uint32_t* drop_rows = nullptr;
  const uint32_t* drop_cols = nullptr;
  float drop_scale = 1.f;
  // Split backward: dS fragments [B * Hq, band.frags, 512] bf16 written by the dK/dV pass and
  // read by launch_bwd_dq_ds (null: the dq pass recomputes dS instead).
  void* ds = nullptr;
  DsBand band{};
};
hipError_t launch_bwd_dq(const BwdParams& p, hipStream_t s);
hipError_t launch_bwd_dkdv(const BwdParams& p, hipStream_t s);
// dQ from the dS fragments the dK/dV pass exported (p.ds): no recomputation of S or dP.
hipError_t launch_bwd_dq_ds(const BwdParams& p, hipStream_t s);



// ---- decode (decode.hip) -----------------------------------------------------------------
// Query heads handled by one decode workgroup: the largest of 4, 3, 2, 1 that divides the
// group size and keeps heads x D <= 256 (the per-lane state fits in registers), so each
// workgroup streams its KV head's cache once for all of them.
inline int decode_heads_per_block(int group, int D) {
  for (int h = 4; h > 1; --h)
    if (group % h == 0 && h * D <= 256) return h;
  return 1;
}
struct DecodeParams {
  const void* q;        // [B, Hq, D]
  const void* kc;       // [B, Hkv, Lmax, D]
  const void* vc;
  const int32_t* cache_len;
  const int32_t* cache_start;  // left padding rows per sequence (null: none)
  void* o;              // [B, Hq, D]
  float* part;          // [B, Hq, nsplit, D + 2]
  unsigned* count;      // [B * Hkv * head subsets], zero on entry and on exit
  int B, Hq, Hkv, D, Lmax, split_len, nsplit;
  float scale, softcap;
  int rope;
  float rope_base;
  int qk_norm;
  float eps;
};
hipError_t launch_decode(const DecodeParams& p, hipStream_t s);

}  // namespace attn
