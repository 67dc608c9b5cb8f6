// Attention-dropout keep masks ("GPT pretraining" page, section "Multihead Attention": dropout
// on the attention weights).  One pass writes the keep bits of every 32 x 32 (query, key)
// tile that the causal / window band touches, in two layouts:
//   rows[b, h, i, w]  bit c = keep(i, 32 w + c)   -- read by the forward and dQ kernels
//   cols[b, h, j, w]  bit c = keep(32 w + c, j)   -- read by the dK/dV kernel
// so that each attention kernel loads one 32-bit word per lane per 32-element block instead
// of running the generator itself.  Words of tiles outside the band are not written.
//
// The keep decision for query i, key j of head (b, h): the 16-bit field j mod 16 of the
// Philox4x64-10 block for counter (floor(j / 16), i, b H + h, offset) under key (seed, 0)
// (field f of the block is bits 16 (f mod 4) .. of output word f / 4) is >= thr.
// Philox4x64-10 is the counter-based generator of Salmon, Moraes, Dror and Shaw, "Parallel
// Random Numbers: As Easy as 1, 2, 3" (SC 2011): ten rounds of two 64 x 64 -> 128-bit
// multiplications and xors, with the key advanced by two Weyl constants between rounds.
#include "launch.h"

namespace attn {
namespace {

struct DropArgs {
  uint32_t* rows;
  uint32_t* cols;
  int T, window, pitch, nqt, nch;
  uint32_t thr;
  uint64_t seed, offset;
};

// Full 64 x 64 -> 128-bit product m * x from four 32 x 32 -> 64 products (v_mad_u64_u32);
// none of the partial sums can overflow 64 bits.
template <uint64_t M>
__device__ __forceinline__ void mulhilo64(uint64_t x, uint64_t& lo, uint64_t& hi) {
  constexpr uint32_t ml = (uint32_t)M, mh = (uint32_t)(M >> 32);
  const uint32_t xl = (uint32_t)x, xh = (uint32_t)(x >> 32);
  const uint64_t p0 = (uint64_t)xl * ml;
  const uint64_t p1 = (uint64_t)xl * mh + (uint32_t)(p0 >> 32);
  const uint64_t p2 = (uint64_t)xh * ml + (uint32_t)p1;
  hi = (uint64_t)xh * mh + (uint32_t)(p1 >> 32) + (uint32_t)(p2 >> 32);
  lo = (p2 << 32) | (uint32_t)p0;
}

__device__ __forceinline__ void philox4x64_10(uint64_t (&x)[4], uint64_t k0, uint64_t k1) {
  constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull, kM1 = 0xCA5A826395121157ull;
  constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull, kW1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t lo0, hi0, lo1, hi1;
    mulhilo64<kM0>(x[0], lo0, hi0);
    mulhilo64<kM1>(x[2], lo1, hi1);
    const uint64_t y0 = hi1 ^ x[1] ^ k0, y2 = hi0 ^ x[3] ^ k1;
    x[0] = y0;
    x[1] = lo1;
    x[2] = y2;
    x[3] = lo0;
    k0 += kW0;
    k1 += kW1;
  }
}

// Keep bits of the 16 keys of one block: bit n <=> field n >= thr.
__device__ __forceinline__ uint32_t keep16(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                           const DropArgs& a) {
  uint64_t x[4] = {c0, c1, c2, c3};
  philox4x64_10(x, a.seed, 0);
  uint32_t bits = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = (uint32_t)x[w], hi = (uint32_t)(x[w] >> 32);
    bits |= (uint32_t)((lo & 0xFFFFu) >= a.thr) << (4 * w);
    bits |= (uint32_t)((lo >> 16) >= a.thr) << (4 * w + 1);
    bits |= (uint32_t)((hi & 0xFFFFu) >= a.thr) << (4 * w + 2);
    bits |= (uint32_t)((hi >> 16) >= a.thr) << (4 * w + 3);
  }
  return bits;
}

// One step of the 32 x 32 bit transpose across the 32 lanes of a half-wave (row r in lane r):
// the off-diagonal m x m blocks of every 2m x 2m block trade places.
template <int M, uint32_t MASK>
__device__ __forceinline__ uint32_t transpose_step(uint32_t x, int r) {
  const uint32_t p = (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, (M << 10) | 0x1F);  // lane r ^ M
  return (r & M) ? ((x & ~MASK) | ((p >> M) & MASK)) : ((x & MASK) | ((p << M) & ~MASK));
}

// Workgroup: one 32-query tile qt of one head and 8 consecutive 32-key tiles; each half-wave
// (32 lanes, one query row per lane) makes one tile.
__global__ __launch_bounds__(256) void dropout_mask_kernel(DropArgs a) {
  const int ch = blockIdx.x % a.nch;
  const int rest = blockIdx.x / a.nch;
  const int qt = rest % a.nqt;
  const int bh = rest / a.nqt;
  const int l = threadIdx.x & 63, r = l & 31;
  const int kt = ch * 8 + 2 * (threadIdx.x >> 6) + (l >> 5);
  const int kt_lo = a.window > 0 ? max(0, qt * 32 - a.window + 1) / 32 : 0;
  if (kt > qt || kt < kt_lo) return;  // whole half-waves leave together
  const int i = qt * 32 + r;
  const uint64_t jb = 2 * (uint64_t)kt;
  const uint32_t row = keep16(jb, (uint64_t)i, (uint64_t)bh, a.offset, a) |
                       (keep16(jb + 1, (uint64_t)i, (uint64_t)bh, a.offset, a) << 16);
  if (i < a.T) a.rows[((int64_t)bh * a.T + i) * a.pitch + kt] = row;
  uint32_t x = row;
  x = transpose_step<16, 0x0000FFFFu>(x, r);
  x = transpose_step<8, 0x00FF00FFu>(x, r);
  x = transpose_step<4, 0x0F0F0F0Fu>(x, r);
  x = transpose_step<2, 0x33333333u>(x, r);
  x = transpose_step<1, 0x55555555u>(x, r);
  const int j = kt * 32 + r;
  if (j < a.T) a.cols[((int64_t)bh * a.T + j) * a.pitch + qt] = x;
}

}  // namespace

hipError_t launch_dropout_mask(uint32_t* rows, uint32_t* cols, int B, int H, int T, int window,
                               uint32_t thr, uint64_t seed, uint64_t offset, hipStream_t s) {
  DropArgs a;
  a.rows = rows;
  a.cols = cols;
  a.T = T;
  a.window = window;
  a.pitch = dropout_pitch(T);
  a.nqt = (T + 31) / 32;
  a.nch = (a.nqt + 7) / 8;
  a.thr = thr;
  a.seed = seed;
  a.offset = offset;
  TraceScope t("dropout_mask", s);
  hipLaunchKernelGGL(dropout_mask_kernel, dim3((unsigned)((int64_t)B * H * a.nqt * a.nch)),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace attn
