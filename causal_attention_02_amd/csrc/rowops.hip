// Row-wise passes around the attention core (all HBM-bound, one wave per row):
//  * prologue: RoPE then parameter-free RMSNorm of q/k rows (nanoGPT-JAX 181M model card,
//    "Architecture": RoPE, QK-norm, "parameter-free RMSNorm (no learnable scale)").
//  * epilogue: the gradient through those two maps, carrying dL/d(q^) back to dL/dq.
//  * rowdot:   D_i = sum_d dO_id * O_id, the per-row term of the softmax backward.
//
// RoPE pairs element i with element i + D/2 and turns the pair by p * base^(-2i/D);
// lane i of the wave owns pair i, so the rotation needs no data exchange and the RMSNorm
// mean is one wave reduction.
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

__global__ __launch_bounds__(256) void epilogue_kernel(const float* __restrict__ dyhat,
                                                       const bf16* __restrict__ x,
                                                       bf16* __restrict__ dx, int64_t rows,
                                                       int Tlen, int D, int rope, double log2_base,
                                                       int qk_norm, float eps) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int half = D >> 1;
  const bool act = lane < half;
  float c = 1.f, s = 0.f;
  if (rope && act) rope_cos_sin((int)(row % Tlen), lane, D, log2_base, &c, &s);
  float g1 = act ? dyhat[row * D + lane] : 0.f;
  float g2 = act ? dyhat[row * D + lane + half] : 0.f;
  if (qk_norm) {
    // Recompute the rotated row y and its normalised form y^ = y / r.
    const bf16* xr = x + row * D;
    const float x1 = act ? from_bf16(xr[lane]) : 0.f;
    const float x2 = act ? from_bf16(xr[lane + half]) : 0.f;
    const float y1 = x1 * c - x2 * s;
    const float y2 = x1 * s + x2 * c;
    const float ms = wave_sum(y1 * y1 + y2 * y2) / (float)D;
    const float inv_r = 1.0f / sqrtf(ms + eps);
    const float h1 = y1 * inv_r, h2 = y2 * inv_r;
    // dy = (dy^ - y^ * mean(dy^ * y^)) / r
    const float mdot = wave_sum(g1 * h1 + g2 * h2) / (float)D;
    g1 = (g1 - h1 * mdot) * inv_r;
    g2 = (g2 - h2 * mdot) * inv_r;
  }
  if (act) {
    // dx = R^T dy: turn the pair back by -angle.
    const float d1 = g1 * c + g2 * s;
    const float d2 = -g1 * s + g2 * c;
    dx[row * D + lane] = to_bf16(d1);
    dx[row * D + lane + half] = to_bf16(d2);
  }
}

// 16 lanes per row, 16 rows per 256-thread block; each lane reads bf16 pairs.
__global__ __launch_bounds__(256) void rowdot_kernel(const bf16x2* __restrict__ dO,
                                                     const bf16x2* __restrict__ O,
                                                     float* __restrict__ Dvec, int64_t rows,
                                                     int D) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  float acc = 0.f;
  if (row < rows) {
    const int pairs = D >> 1;
    const bf16x2* a = dO + row * pairs;
    const bf16x2* b = O + row * pairs;
    for (int p = sub; p < pairs; p += 16) {
      const bf16x2 u = a[p], w = b[p];
      acc += (float)u[0] * (float)w[0] + (float)u[1] * (float)w[1];
    }
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (row < rows && sub == 0) Dvec[row] = acc;
}

hipError_t launch_prologue(const void* x, void* y, int64_t rows, int T, int D, int elt, int rope,
                           float rope_base, int qk_norm, float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const double log2_base = rope ? log2((double)rope_base) : 0.0;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (elt == 2) {
    TraceScope t("prologue_bf16", s);
    hipLaunchKernelGGL(prologue_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)x, (bf16*)y,
                       rows, T, D, rope, log2_base, qk_norm, eps);
  } else {
    TraceScope t("prologue_f32", s);
    hipLaunchKernelGGL(prologue_kernel<float>, grid, dim3(256), 0, s, (const float*)x, (float*)y,
                       rows, T, D, rope, log2_base, qk_norm, eps);
  }
  return hipGetLastError();
}

hipError_t launch_epilogue(const float* dyhat, const void* x, void* dx, int64_t rows, int T, int D,
                           int rope, float rope_base, int qk_norm, float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const double log2_base = rope ? log2((double)rope_base) : 0.0;
  TraceScope t("epilogue_bf16", s);
  hipLaunchKernelGGL(epilogue_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, dyhat,
                     (const bf16*)x, (bf16*)dx, rows, T, D, rope, log2_base, qk_norm, eps);
  return hipGetLastError();
}

hipError_t launch_rowdot(const void* dO, const void* O, float* Dvec, int64_t rows, int D,
                         hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  TraceScope t("rowdot_bf16", s);
  hipLaunchKernelGGL(rowdot_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s,
                     (const bf16x2*)dO, (const bf16x2*)O, Dvec, rows, D);
  return hipGetLastError();
}

}  // namespace attn
