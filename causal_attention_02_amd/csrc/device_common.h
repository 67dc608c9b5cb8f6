// Device-side helpers shared by the gfx950 attention kernels: vector types, the bf16
// MFMA wrappers, LDS transpose reads, cross-lane reductions and bf16 conversion.
//
// Lane layouts used throughout (CDNA4, wave64), as checked on the hardware:
//  * v_mfma_f32_32x32x16_bf16  C[32x32] += A[32x16] * B[16x32]:
//      A: lane l holds A[l % 32][8 * (l / 32) + p],  p = 0..7
//      B: lane l holds B[8 * (l / 32) + p][l % 32]
//      C: lane l, register r holds C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
//  * ds_read_b64_tr_b16 (per group of 16 lanes): result lane j, element e is element
//      j % 4 of the 8 bytes loaded by lane 4 * e + j / 4 of the same group.  So if lane L
//      of a group loads row (k0 + L / 4), columns (n0 + 4 * (L % 4)) .. +3 of a row-major
//      [k][n] bf16 matrix, lane j receives column n0 + j, rows k0 .. k0 + 3.
//  * v_permlane32_swap(x, x): lane l < 32 gets (x[l], x[l + 32]); lane l >= 32 gets
//      (x[l - 32], x[l]) -- both halves of a lane pair (l, l ^ 32) in one instruction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite stand-in for -inf in the running maximum: exp2(kNegBig - m) is exactly 0 for any
// finite score m, and exp2(kNegBig - kNegBig) = 1 only while a row has seen no visible key,
// a state that a later visible key multiplies away (its rescale factor is 0).
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Round-to-nearest-even float -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }
__device__ __forceinline__ float from_bf16(bf16 x) { return (float)x; }

__device__ __forceinline__ bf16x8 pack8(const f32x16& v, int base) {
  bf16x8 r;
#pragma unroll
  for (int p = 0; p < 8; ++p) r[p] = (bf16)v[base + p];
  return r;
}

// ---- dropout keep bits -----------------------------------------------------------------
// A lane's 16 accumulator elements of a 32-wide block sit at offsets 8 (r / 4) + r % 4 + 4 gl
// of the block; `mw` is the block's keep word shifted right by 4 gl, so element r's bit is
// keep_bit(r).
__device__ __forceinline__ constexpr int keep_bit(int r) { return 8 * (r >> 2) + (r & 3); }

// All ones if bit `bit` of mw is set, else zero (v_bfe_i32).
__device__ __forceinline__ uint32_t keep_all(uint32_t mw, int bit) {
  return (uint32_t)((int32_t)(mw << (31 - bit)) >> 31);
}

// x where element r is kept, +0 where it is dropped.
__device__ __forceinline__ float keep_only(float x, uint32_t mw, int r) {
  return __uint_as_float(__float_as_uint(x) & keep_all(mw, keep_bit(r)));
}

// Zero the dropped weights of a packed half block (elements 8 h .. 8 h + 7, two per dword).
__device__ __forceinline__ bf16x8 keep_packed(bf16x8 v, uint32_t mw, int h) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 u = __builtin_bit_cast(u32x4, v);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int bit = keep_bit(8 * h + 2 * d);  // the pair's second element is bit + 1
    u[d] &= (keep_all(mw, bit) & 0xFFFFu) | (keep_all(mw, bit + 1) & 0xFFFF0000u);
  }
  return __builtin_bit_cast(bf16x8, u);
}

// Sum of the 8 bf16 values with fp32 accumulation (v_dot2_f32_bf16 against (1, 1)).
__device__ __forceinline__ float sum_bf16x8(bf16x8 v) {
  const bf16x2 one = {(bf16)1.f, (bf16)1.f};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 pr = {v[2 * i], v[2 * i + 1]};
    s = __builtin_amdgcn_fdot2_f32_bf16(pr, one, s, false);
  }
  return s;
}

// Two transposing LDS reads (rows k0..k0+3 and k1..k1+3) glued into one MFMA operand.
__device__ __forceinline__ bf16x8 tr_read_pair(const bf16* p0, const bf16* p1) {
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
  union {
    struct { i16x4 lo, hi; } s;
    bf16x8 v;
  } u;
  u.s.lo = a;
  u.s.hi = b;
  return u.v;
}

// max / sum over the lane pair (l, l ^ 32).
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <typename T>
__device__ __forceinline__ T ld16(const void* p) {
  return *reinterpret_cast<const T*>(p);
}

// Angle p * base^(-2i/D) reduced to [-pi, pi] in double precision, then its cosine and sine
// in single precision.
__device__ __forceinline__ void rope_cos_sin(int pos, int i, int D, double log2_base, float* c,
                                            float* s) {
  const double w = exp2(-(2.0 * i / D) * log2_base);
  double a = (double)pos * w;
  const double two_pi = 6.283185307179586;
  a -= two_pi * rint(a / two_pi);
  sincosf((float)a, s, c);
}

// ---- score transform -------------------------------------------------------------------
// The kernels work with y = S * log2(e) so that softmax weights are exp2(y - shift).
//   kScoreScale: y = acc * scale * log2(e)
//   kScoreCapExp: soft-cap through tanh(x) = 1 - 2 / (exp(2x) + 1) (any argument range)
//   kScoreCapPoly: soft-cap through the odd Taylor polynomial of tanh up to x^9, used only
//     when the host has shown |S_pre / c| <= 1/4 (QK-norm bounds |S_pre| <= scale * D);
//     there its truncation error is below 1e-8 relative, under fp32 rounding.
//   kScoreCapPoly5: the same series cut after x^5, used only where the host has shown that
//     the dropped terms move y by at most 2^-12 (a relative change of 2^-12 in a softmax
//     weight, an eighth of bf16's rounding step) and that the derivative series
//     sech^2(x) = 1 - x^2 + (2/3) x^4 cut the same way is within 2^-12 relative.
enum { kScoreScale = 0, kScoreCapExp = 1, kScoreCapPoly = 2, kScoreCapPoly5 = 3 };

struct ScoreCoef {
  float k0;          // kScoreScale: scale*log2e;  kScoreCapExp: 2*scale*log2e/c
  float k1;          // kScoreCapExp: c*log2e
  float p1, p3, p5, p7, p9;  // polynomial modes: y = a * (p1 + a^2 (p3 + a^2 (p5 + ...)))
  float inv_k1_sq;   // 1 / (c log2e)^2 : tanh^2 = (y / (c log2e))^2
  float g2, g4;      // kScoreCapPoly5: sech^2 = 1 + a^2 (g2 + a^2 g4)
  float mask_acc;    // raw score standing in for a masked entry (not kScoreCapExp): weight 0,
                     // finite slope factor
};

// Returns y - shift (log2 units).  With T2 also *t2 = tanh^2(S_pre / c) (exp / degree-9
// modes only).
template <int MODE, bool T2>
__device__ __forceinline__ float score_y(float acc, const ScoreCoef& c, float shift, float* t2) {
  if constexpr (MODE == kScoreScale) {
    if constexpr (T2) *t2 = 0.f;
    return fmaf(acc, c.k0, -shift);
  } else if constexpr (MODE == kScoreCapExp) {
    const float e = exp2_fast(acc * c.k0);
    const float r = rcp_fast(e + 1.f);  // tanh = 1 - 2 r
    if constexpr (T2) {
      const float th = fmaf(r, -2.f, 1.f);
      *t2 = th * th;
    }
    return fmaf(r, -2.f * c.k1, c.k1 - shift);
  } else if constexpr (MODE == kScoreCapPoly5) {
    static_assert(!T2, "degree-5 mode gives the derivative through score_grad");
    const float a2 = acc * acc;
    const float q = fmaf(a2, fmaf(a2, c.p5, c.p3), c.p1);
    return fmaf(acc, q, -shift);
  } else {
    const float a2 = acc * acc;
    float q = fmaf(a2, c.p9, c.p7);
    q = fmaf(a2, q, c.p5);
    q = fmaf(a2, q, c.p3);
    q = fmaf(a2, q, c.p1);
    if constexpr (T2) {
      const float u = acc * q;
      *t2 = u * u * c.inv_k1_sq;
      return u - shift;
    } else {
      return fmaf(acc, q, -shift);
    }
  }
}

// Backward form: returns y - shift and sets *g to d(capped score)/d(raw score) relative to
// the uncapped slope, i.e. 1 - tanh^2(S_pre / c) (left unset for kScoreScale).
template <int MODE>
__device__ __forceinline__ float score_grad(float acc, const ScoreCoef& c, float shift, float* g) {
  if constexpr (MODE == kScoreScale) {
    return fmaf(acc, c.k0, -shift);
  } else if constexpr (MODE == kScoreCapPoly5) {
    const float a2 = acc * acc;
    const float q = fmaf(a2, fmaf(a2, c.p5, c.p3), c.p1);
    *g = fmaf(a2, fmaf(a2, c.g4, c.g2), 1.f);
    return fmaf(acc, q, -shift);
  } else {
    float t2;
    const float y = score_y<MODE, true>(acc, c, shift, &t2);
    *g = 1.f - t2;
    return y;
  }
}

// Visibility of key j to query i as one unsigned compare: 0 <= i - j < wlim, with
// wlim = W for a sliding window and 2^31 - 1 for plain causal attention.
__device__ __forceinline__ bool visible(int i_minus_j, unsigned wlim) {
  return (unsigned)i_minus_j < wlim;
}

// ---- RoPE / RMSNorm on register-resident rows ------------------------------------------
// Rows are held as x[NC][W]: chunk c, element e covers head-dim index d(c, e).  A lane pair
// (l, l ^ 32) holds one full row; RoPE partners d and d + D/2 always sit in the same lane
// (both MFMA layouts put them at chunk c and c + NC/2), so the rotation needs no exchange
// and the RMSNorm mean is a per-lane sum plus one pair_sum.
// omega_rev[i] = base^(-2i/D) / (2 pi): the rotation in revolutions per position.
__device__ __forceinline__ void rope_pair(float& x1, float& x2, int pos, double omega_rev,
                                          bool inverse) {
  double r = (double)pos * omega_rev;
  r -= floor(r);
  const float rf = (float)r;
  const float c = __builtin_amdgcn_cosf(rf);
  const float s = inverse ? -__builtin_amdgcn_sinf(rf) : __builtin_amdgcn_sinf(rf);
  const float y1 = x1 * c - x2 * s;
  const float y2 = x1 * s + x2 * c;
  x1 = y1;
  x2 = y2;
}

struct RowPrologue {
  int rope, qk_norm;
  float eps;
  double omega_rev[64];
};

// Prologue (RoPE at `pos`, then RMSNorm) of a row held in the MFMA operand layout: chunk s,
// element p is head-dim index 16 s + 8 (lane / 32) + p; partner chunks are s and s + NS/2.
template <int NS>
__device__ __forceinline__ void prologue_oplayout(float (&x)[NS][8], int pos, int gl,
                                                  const RowPrologue& rp, int D) {
  if (rp.rope) {
#pragma unroll
    for (int s = 0; s < NS / 2; ++s)
#pragma unroll
      for (int p = 0; p < 8; ++p)
        rope_pair(x[s][p], x[s + NS / 2][p], pos, rp.omega_rev[16 * s + 8 * gl + p], false);
  }
  if (rp.qk_norm) {
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int p = 0; p < 8; ++p) ss = fmaf(x[s][p], x[s][p], ss);
    ss = pair_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)D + rp.eps);
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int p = 0; p < 8; ++p) x[s][p] *= inv;
  }
}

// Gradient through the prologue for a row held in the MFMA accumulator layout: entry
// (e, j) is head-dim index 8 e + 4 (lane / 32) + j, e < D/8; partners are e and e + D/16.
// g holds dL/d(x^) on entry and dL/dx on exit; xr is the raw input row in the same layout.
template <int NE>
__device__ __forceinline__ void prologue_backward_acclayout(float (&g)[NE][4], float (&xr)[NE][4],
                                                            int pos, int gl,
                                                            const RowPrologue& rp, int D) {
  if (rp.rope) {
#pragma unroll
    for (int e = 0; e < NE / 2; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        rope_pair(xr[e][j], xr[e + NE / 2][j], pos, rp.omega_rev[8 * e + 4 * gl + j], false);
  }
  if (rp.qk_norm) {
    // y = rotated row, y^ = y / r, dy = (dy^ - y^ mean(dy^ y^)) / r
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) ss = fmaf(xr[e][j], xr[e][j], ss);
    ss = pair_sum(ss);
    const float inv_r = 1.0f / sqrtf(ss / (float)D + rp.eps);
    float md = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) md = fmaf(g[e][j], xr[e][j] * inv_r, md);
    md = pair_sum(md) / (float)D;
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) g[e][j] = (g[e][j] - xr[e][j] * inv_r * md) * inv_r;
  }
  if (rp.rope) {
#pragma unroll
    for (int e = 0; e < NE / 2; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        rope_pair(g[e][j], g[e + NE / 2][j], pos, rp.omega_rev[8 * e + 4 * gl + j], true);
  }
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// ---- workgroup order ---------------------------------------------------------------------
// Workgroups are dealt to the 8 XCDs (each with its own L2) round-robin by index.  Within one
// rank of a (rank, head) grid, index i runs on XCD i % 8; this returns the head for index i
// such that each XCD gets a contiguous range of nbh / 8 heads, i.e. whole GQA groups whose
// query heads share one K/V stream, instead of every 8th head.  The rank order (heaviest
// tiles first) is untouched.  Identity when nbh is not a multiple of 8.
__device__ __forceinline__ int xcd_local_head(int i, int nbh) {
  return (nbh & 7) ? i : (i & 7) * (nbh >> 3) + (i >> 3);
}

// ---- tile staging ------------------------------------------------------------------------
// Direct global -> LDS copies of 64-row bf16 tiles into LDS rows of pitch D + 8 elements
// (the pad keeps the row-per-lane MFMA operand reads free of bank conflicts).  The LDS image
// is cut into 1 KB chunks, one wave-wide 16-byte load each: lane l of chunk c carries image
// granule p = 64 c + l, which is granule p % G of padded row p / G (G = D/8 + 1).  The
// source tile is contiguous (rows r0 .. r0 + 63 of one head), so that granule sits
// p - p / G granules past the tile start; sources are clamped to the head's last granule
// (rows past the end and the pad granules read real, finite data that is never used).
// Chunks are dealt round-robin to the NW waves; a wave keeps one offset per chunk it owns.
template <int D, int NW>
struct TileDma {
  static constexpr int G = D / 8 + 1;
  static constexpr int NC = (G + NW - 1) / NW;  // chunks per wave (the last may be absent)
  uint32_t off[NC];  // byte offset of the chunk's source granule from the tile start
  __device__ __forceinline__ TileDma(int w, int l) {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int pg = 64 * (w + NW * i) + l;
      off[i] = 16u * (uint32_t)(pg - pg / G);
    }
  }
  // Copy rows r0.. of the head starting at src (T rows) into lds (w: this wave's index).
  __device__ __forceinline__ void copy(bf16* lds, const bf16* src, int r0, int T, int w) const {
    w = __builtin_amdgcn_readfirstlane(w);  // the LDS targets and chunk ownership are uniform
    if (r0 + 64 < T) {
      // Every source granule, the last row's pad included, lies inside the head: a uniform
      // base plus the lane's 32-bit offset, which the hardware adds itself (no clamp and no
      // per-lane 64-bit address arithmetic).
      // The base is uniform; reading it from the first lane places it in scalar registers
      // once per copy instead of once per load.
      const uint64_t bv = reinterpret_cast<uint64_t>(src + (int64_t)r0 * D);
      const uint32_t blo = __builtin_amdgcn_readfirstlane((uint32_t)bv);
      const uint32_t bhi = __builtin_amdgcn_readfirstlane((uint32_t)(bv >> 32));
      const char* base = reinterpret_cast<const char*>(((uint64_t)bhi << 32) | blo);
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int c = w + NW * i;
        if (c < G) {
          // The empty asm keeps the offset a 32-bit value here (not a widened copy hoisted
          // out of the loop), so the load takes the base-register-plus-offset form.
          uint32_t o = off[i];
          asm volatile("" : "+v"(o));
          __builtin_amdgcn_global_load_lds(base + o, lds + 512 * c, 16, 0, 0);
        }
      }
      return;
    }
    const int first = r0 * (D / 8), last = T * (D / 8) - 1;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = w + NW * i;
      if (c < G) {
        const bf16* from = src + 8 * (int64_t)min(first + (int)(off[i] >> 4), last);
        __builtin_amdgcn_global_load_lds(from, lds + 512 * c, 16, 0, 0);
      }
    }
  }
};

// The same copies for a kernel with no register to spare: the per-lane byte offsets (each
// below 2^16: at most 64 G granules of 16 bytes) are held two to a register and extracted
// with one instruction per chunk.
template <int D, int NW>
struct TileDma16 {
  static constexpr int G = D / 8 + 1;
  static constexpr int NC = (G + NW - 1) / NW;
  static_assert(64 * G * 16 <= 65536, "offsets must fit 16 bits");
  uint32_t off2[(NC + 1) / 2];
  __device__ __forceinline__ TileDma16(int w, int l) {
#pragma unroll
    for (int i = 0; i < (NC + 1) / 2; ++i) off2[i] = 0u;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int pg = 64 * (w + NW * i) + l;
      off2[i / 2] |= (16u * (uint32_t)(pg - pg / G)) << (16 * (i & 1));
    }
  }
  __device__ __forceinline__ uint32_t off(int i) const {
    uint32_t o = (i & 1) ? off2[i / 2] >> 16 : off2[i / 2] & 0xffffu;
    asm volatile("" : "+v"(o));  // extracted here, not hoisted out of the loop
    return o;
  }
  // Copy rows r0.. of the head starting at src (T rows) into lds.  Rows below `lo` (left
  // padding of a cache) read row lo instead, so that whatever those rows hold (they are
  // masked, but a NaN times a zero weight would still be NaN) never enters the tile.
  __device__ __forceinline__ void copy(bf16* lds, const bf16* src, int r0, int T, int w,
                                       int lo) const {
    w = __builtin_amdgcn_readfirstlane(w);
    if (r0 + 64 < T && r0 >= lo) {
      // Every source granule lies inside the head: uniform base plus 32-bit lane offset.
      const uint64_t bv = reinterpret_cast<uint64_t>(src + (int64_t)r0 * D);
      const uint32_t blo = __builtin_amdgcn_readfirstlane((uint32_t)bv);
      const uint32_t bhi = __builtin_amdgcn_readfirstlane((uint32_t)(bv >> 32));
      const char* base = reinterpret_cast<const char*>(((uint64_t)bhi << 32) | blo);
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int c = w + NW * i;
        if (c < G) {
          const uint32_t o = off(i);
          __builtin_amdgcn_global_load_lds(base + o, lds + 512 * c, 16, 0, 0);
        }
      }
      return;
    }
    const int first = r0 * (D / 8), last = T * (D / 8) - 1, lo_g = lo * (D / 8);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = w + NW * i;
      if (c < G) {
        const int gsrc = max(min(first + (int)(off(i) >> 4), last), lo_g);
        __builtin_amdgcn_global_load_lds(src + 8 * (int64_t)gsrc, lds + 512 * c, 16, 0, 0);
      }
    }
  }
};

}  // namespace attn
