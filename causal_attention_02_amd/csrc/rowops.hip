// Stand-alone prologue pass: RoPE then parameter-free RMSNorm of k (and, on the fp32 path,
// q) rows (nanoGPT-JAX 181M model card, "Architecture": RoPE, QK-norm, "parameter-free
// RMSNorm (no learnable scale)").  HBM-bound.  The bf16 attention kernels apply the same
// prologue to their own q rows in registers; keys are visited by many query tiles, so they
// are prepared once here.
//
// RoPE pairs element i with element i + D/2 and turns the pair by p * base^(-2i/D).
#include "device_common.h"
#include "launch.h"

namespace attn {

template <typename T>
__device__ __forceinline__ float load_elt(const T* p);
template <>
__device__ __forceinline__ float load_elt<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_elt<bf16>(const bf16* p) { return from_bf16(*p); }

template <typename T>
__device__ __forceinline__ void store_elt(T* p, float x);
template <>
__device__ __forceinline__ void store_elt<float>(float* p, float x) { *p = x; }
template <>
__device__ __forceinline__ void store_elt<bf16>(bf16* p, float x) { *p = to_bf16(x); }

// 4 waves per block, one row per wave.
template <typename T>
__global__ __launch_bounds__(256) void prologue_kernel(const T* __restrict__ x, T* __restrict__ y,
                                                       int64_t rows, int Tlen, int D, int rope,
                                                       double log2_base, int qk_norm, float eps) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int half = D >> 1;
  const bool act = lane < half;
  const T* xr = x + row * D;
  float x1 = act ? load_elt(xr + lane) : 0.f;
  float x2 = act ? load_elt(xr + lane + half) : 0.f;
  if (rope && act) {
    float c, s;
    rope_cos_sin((int)(row % Tlen), lane, D, log2_base, &c, &s);
    const float r1 = x1 * c - x2 * s;
    const float r2 = x1 * s + x2 * c;
    x1 = r1;
    x2 = r2;
  }
  if (qk_norm) {
    const float ss = wave_sum(x1 * x1 + x2 * x2);
    const float inv = 1.0f / sqrtf(ss / (float)D + eps);
    x1 *= inv;
    x2 *= inv;
  }
  if (act) {
    T* yr = y + row * D;
    store_elt(yr + lane, x1);
    store_elt(yr + lane + half, x2);
  }
}

// bf16 rows: 8 lanes per row, each owning 8 RoPE pairs (16-byte loads of both halves); each
// thread takes kPrologueRows rows 32 apart, all loaded before any is computed (more bytes in
// flight per thread: 14.5 against 15.6 us for the 181M keys; four rows were slower).
constexpr int kPrologueRows = 2;
__global__ __launch_bounds__(256) void prologue_bf16_kernel(const bf16* __restrict__ x,
                                                            bf16* __restrict__ y, int64_t rows,
                                                            int Tlen, int D, RowPrologue rp) {
  const int u = threadIdx.x & 7;
  const int half = D / 2;
  float x1[kPrologueRows][8], x2[kPrologueRows][8];
  int64_t row[kPrologueRows];
  bool act[kPrologueRows];
#pragma unroll
  for (int k = 0; k < kPrologueRows; ++k) {
    row[k] = (int64_t)blockIdx.x * (32 * kPrologueRows) + 32 * k + (threadIdx.x >> 3);
    act[k] = row[k] < rows && u < D / 16;
    const bf16* xr = x + (row[k] < rows ? row[k] : 0) * D;
    bf16x8 a, c;
    if (act[k]) {
      a = ld16<bf16x8>(xr + 8 * u);
      c = ld16<bf16x8>(xr + half + 8 * u);
    } else {
#pragma unroll
      for (int p = 0; p < 8; ++p) a[p] = c[p] = to_bf16(0.f);
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      x1[k][p] = (float)a[p];
      x2[k][p] = (float)c[p];
    }
  }
#pragma unroll
  for (int k = 0; k < kPrologueRows; ++k) {
    if (rp.rope && act[k]) {
      const int pos = (int)(row[k] % Tlen);
#pragma unroll
      for (int p = 0; p < 8; ++p) rope_pair(x1[k][p], x2[k][p], pos, rp.omega_rev[8 * u + p], false);
    }
    if (rp.qk_norm) {
      float ss = 0.f;
#pragma unroll
      for (int p = 0; p < 8; ++p) ss += x1[k][p] * x1[k][p] + x2[k][p] * x2[k][p];
      ss += __shfl_xor(ss, 1, 8);
      ss += __shfl_xor(ss, 2, 8);
      ss += __shfl_xor(ss, 4, 8);
      const float inv = 1.0f / sqrtf(ss / (float)D + rp.eps);
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        x1[k][p] *= inv;
        x2[k][p] *= inv;
      }
    }
    if (act[k]) {
      bf16x8 a, c;
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        a[p] = to_bf16(x1[k][p]);
        c[p] = to_bf16(x2[k][p]);
      }
      bf16* yr = y + row[k] * D;
      *reinterpret_cast<bf16x8*>(yr + 8 * u) = a;
      *reinterpret_cast<bf16x8*>(yr + half + 8 * u) = c;
    }
  }
}

// Append S new tokens to a KV cache ("GPT pretraining" page, "Bonus: KV Caching": compute
// the new keys and values, append them, then attend).  Token i of sequence b lands in cache
// row p = cache_len[b] + i (cache_len clamped to [0, Lmax]); its key is rotated at position
// p - cache_start[b] (left padding rows; 0 without) and normalised first, its value copied.
// Rows with p >= Lmax are not written.  Same lane layout
// as prologue_bf16_kernel: 8 lanes per row, each owning 8 RoPE pairs.
__global__ __launch_bounds__(256) void append_kv_kernel(const bf16* __restrict__ kn,
                                                        const bf16* __restrict__ vn,
                                                        bf16* __restrict__ kc, bf16* __restrict__ vc,
                                                        const int32_t* __restrict__ cache_len,
                                                        const int32_t* __restrict__ cache_start,
                                                        int64_t rows, int S, int Hkv, int Lmax, int D,
                                                        RowPrologue rp) {
  const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);  // (b, g, i) row-major
  const int u = threadIdx.x & 7;
  const bool in_range = row < rows;
  const int64_t bg = in_range ? row / S : 0;
  const int i = in_range ? (int)(row - bg * S) : 0;
  const int b = (int)(bg / Hkv);
  const int L = in_range ? min(max(cache_len[b], 0), Lmax) : 0;
  const int pos = L + i;  // cache row; the RoPE position counts from the first real row
  const int first = (in_range && cache_start) ? min(max(cache_start[b], 0), Lmax) : 0;
  const bool act = in_range && pos < Lmax && u < D / 16;
  const int half = D / 2;
  float x1[8], x2[8];
  const bf16* xr = kn + (in_range ? row : 0) * D;
  if (act) {
    const bf16x8 a = ld16<bf16x8>(xr + 8 * u);
    const bf16x8 c = ld16<bf16x8>(xr + half + 8 * u);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      x1[p] = (float)a[p];
      x2[p] = (float)c[p];
    }
  } else {
#pragma unroll
    for (int p = 0; p < 8; ++p) x1[p] = x2[p] = 0.f;
  }
  if (rp.rope && act) {
#pragma unroll
    for (int p = 0; p < 8; ++p)
      rope_pair(x1[p], x2[p], pos - first, rp.omega_rev[8 * u + p], false);
  }
  if (rp.qk_norm) {
    float ss = 0.f;
#pragma unroll
    for (int p = 0; p < 8; ++p) ss += x1[p] * x1[p] + x2[p] * x2[p];
    ss += __shfl_xor(ss, 1, 8);
    ss += __shfl_xor(ss, 2, 8);
    ss += __shfl_xor(ss, 4, 8);
    const float inv = 1.0f / sqrtf(ss / (float)D + rp.eps);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      x1[p] *= inv;
      x2[p] *= inv;
    }
  }
  if (act) {
    bf16x8 a, c;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      a[p] = to_bf16(x1[p]);
      c[p] = to_bf16(x2[p]);
    }
    const int64_t dst = (bg * Lmax + pos) * D;
    *reinterpret_cast<bf16x8*>(kc + dst + 8 * u) = a;
    *reinterpret_cast<bf16x8*>(kc + dst + half + 8 * u) = c;
    const bf16* vr = vn + row * D;
    *reinterpret_cast<bf16x8*>(vc + dst + 8 * u) = ld16<bf16x8>(vr + 8 * u);
    *reinterpret_cast<bf16x8*>(vc + dst + half + 8 * u) = ld16<bf16x8>(vr + half + 8 * u);
  }
}

hipError_t launch_append_kv(const void* kn, const void* vn, void* kc, void* vc,
                            const int32_t* cache_len, const int32_t* cache_start, int B, int Hkv,
                            int S, int Lmax, int D, int rope, float rope_base, int qk_norm,
                            float eps, hipStream_t s) {
  const int64_t rows = (int64_t)B * Hkv * S;
  if (rows <= 0) return hipSuccess;
  TraceScope t("append_kv", s);
  hipLaunchKernelGGL(append_kv_kernel, dim3((unsigned)((rows + 31) / 32)), dim3(256), 0, s,
                     (const bf16*)kn, (const bf16*)vn, (bf16*)kc, (bf16*)vc, cache_len, cache_start,
                     rows, S, Hkv, Lmax, D, make_row_prologue(rope, rope_base, qk_norm, eps, D));
  return hipGetLastError();
}

// Packed rows (nanoGPT-JAX 181M model card, SFT notes: rows packed with segment ids): a
// segment is a maximal run of equal ids.  For every token, start = index of the first token
// of its run and end = index of the last; attention stays inside [start, end].  One
// workgroup per row: each thread scans a contiguous span, then the spans' boundaries are
// combined with a prefix maximum (starts) and a suffix minimum (ends) over the threads.
__global__ __launch_bounds__(1024) void segment_bounds_kernel(const int32_t* __restrict__ ids,
                                                             int32_t* __restrict__ st,
                                                             int32_t* __restrict__ en, int T) {
  __shared__ int smax[1024], smin[1024];
  const int64_t base = (int64_t)blockIdx.x * T;
  const int t = threadIdx.x;
  const int span = (T + 1023) / 1024;
  const int a = min(t * span, T), z = min(a + span, T);
  int lmax = -1, lmin = 0x7fffffff;
  for (int i = a; i < z; ++i) {
    const int id = ids[base + i];
    if (i == 0 || id != ids[base + i - 1]) lmax = i;                      // a run starts at i
    if (lmin == 0x7fffffff && (i == T - 1 || id != ids[base + i + 1])) lmin = i;  // first run end
  }
  smax[t] = lmax;
  smin[t] = lmin;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive prefix max / suffix min
    const int vmax = t >= off ? smax[t - off] : -1;
    const int vmin = t + off < 1024 ? smin[t + off] : 0x7fffffff;
    __syncthreads();
    smax[t] = max(smax[t], vmax);
    smin[t] = min(smin[t], vmin);
    __syncthreads();
  }
  int run = t > 0 ? smax[t - 1] : -1;
  for (int i = a; i < z; ++i) {
    if (i == 0 || ids[base + i] != ids[base + i - 1]) run = i;
    st[base + i] = run;
  }
  int runm = t < 1023 ? smin[t + 1] : 0x7fffffff;
  for (int i = z - 1; i >= a; --i) {
    if (i == T - 1 || ids[base + i] != ids[base + i + 1]) runm = i;
    en[base + i] = runm;
  }
}

hipError_t launch_segment_bounds(const int32_t* ids, int32_t* start, int32_t* end, int B, int T,
                                 hipStream_t s) {
  if (B <= 0 || T <= 0) return hipSuccess;
  TraceScope t("segment_bounds", s);
  hipLaunchKernelGGL(segment_bounds_kernel, dim3((unsigned)B), dim3(1024), 0, s, ids, start, end,
                     T);
  return hipGetLastError();
}

// Backward preparation, one pass over the query rows (same lane layout as
// prologue_bf16_kernel: 8 lanes per row, each owning elements 8u..8u+7 of both halves):
//   nD[r] = -sum_d dO[r, d] O[r, d]   (the softmax-gradient row term, negated)
//   L2[r] = LSE[r] * log2(e)          (the backward works in log2 units)
//   qh[r] = N(R(q[r]))                (when qh is not null: RoPE at position r % T, RMSNorm)
__global__ __launch_bounds__(256) void bwd_prep_kernel(const bf16* __restrict__ q,
                                                       const bf16* __restrict__ o,
                                                       const bf16* __restrict__ dO,
                                                       const float* __restrict__ lse,
                                                       bf16* __restrict__ qh, float* __restrict__ nD,
                                                       float* __restrict__ L2, int64_t rows,
                                                       int Tlen, int D, RowPrologue rp) {
  const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int u = threadIdx.x & 7;
  const bool act = row < rows && u < D / 16;
  const int half = D / 2;
  const int64_t off = (row < rows ? row : 0) * D;
  float dsum = 0.f;
  if (act) {
    const bf16x8 o1 = ld16<bf16x8>(o + off + 8 * u), o2 = ld16<bf16x8>(o + off + half + 8 * u);
    const bf16x8 g1 = ld16<bf16x8>(dO + off + 8 * u), g2 = ld16<bf16x8>(dO + off + half + 8 * u);
#pragma unroll
    for (int p = 0; p < 8; ++p)
      dsum = fmaf((float)g1[p], (float)o1[p], fmaf((float)g2[p], (float)o2[p], dsum));
  }
  dsum += __shfl_xor(dsum, 1, 8);
  dsum += __shfl_xor(dsum, 2, 8);
  dsum += __shfl_xor(dsum, 4, 8);
  if (row < rows && u == 0) {
    nD[row] = -dsum;
    L2[row] = lse[row] * kLog2e;
  }
  if (!qh) return;
  float x1[8], x2[8];
  if (act) {
    const bf16x8 a = ld16<bf16x8>(q + off + 8 * u);
    const bf16x8 c = ld16<bf16x8>(q + off + half + 8 * u);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      x1[p] = (float)a[p];
      x2[p] = (float)c[p];
    }
  } else {
#pragma unroll
    for (int p = 0; p < 8; ++p) x1[p] = x2[p] = 0.f;
  }
  if (rp.rope && act) {
    const int pos = (int)(row % Tlen);
#pragma unroll
    for (int p = 0; p < 8; ++p) rope_pair(x1[p], x2[p], pos, rp.omega_rev[8 * u + p], false);
  }
  if (rp.qk_norm) {
    float ss = 0.f;
#pragma unroll
    for (int p = 0; p < 8; ++p) ss += x1[p] * x1[p] + x2[p] * x2[p];
    ss += __shfl_xor(ss, 1, 8);
    ss += __shfl_xor(ss, 2, 8);
    ss += __shfl_xor(ss, 4, 8);
    const float inv = 1.0f / sqrtf(ss / (float)D + rp.eps);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      x1[p] *= inv;
      x2[p] *= inv;
    }
  }
  if (act) {
    bf16x8 a, c;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      a[p] = to_bf16(x1[p]);
      c[p] = to_bf16(x2[p]);
    }
    *reinterpret_cast<bf16x8*>(qh + off + 8 * u) = a;
    *reinterpret_cast<bf16x8*>(qh + off + half + 8 * u) = c;
  }
}

hipError_t launch_bwd_prep(const void* q, const void* o, const void* dO, const float* lse,
                           void* qh, float* nD, float* L2, int64_t rows, int T, int D, int rope,
                           float rope_base, int qk_norm, float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  TraceScope t("bwd_prep", s);
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((rows + 31) / 32)), dim3(256), 0, s,
                     (const bf16*)q, (const bf16*)o, (const bf16*)dO, lse, (bf16*)qh, nD, L2, rows,
                     T, D, make_row_prologue(rope, rope_base, qk_norm, eps, D));
  return hipGetLastError();
}

hipError_t launch_prologue(const void* x, void* y, int64_t rows, int T, int D, int elt, int rope,
                           float rope_base, int qk_norm, float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (elt == 2) {
    TraceScope t("prologue_bf16", s);
    const int64_t per_block = 32 * kPrologueRows;
    hipLaunchKernelGGL(prologue_bf16_kernel, dim3((unsigned)((rows + per_block - 1) / per_block)),
                       dim3(256), 0, s,
                       (const bf16*)x, (bf16*)y, rows, T, D,
                       make_row_prologue(rope, rope_base, qk_norm, eps, D));
  } else {
    const double log2_base = rope ? log2((double)rope_base) : 0.0;
    TraceScope t("prologue_f32", s);
    hipLaunchKernelGGL(prologue_kernel<float>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s,
                       (const float*)x, (float*)y, rows, T, D, rope, log2_base, qk_norm, eps);
  }
  return hipGetLastError();
}

}  // namespace attn
