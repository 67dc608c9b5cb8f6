// Causal attention backward on gfx950: gradients of sum(O * dO) with respect to q^, k^, v.
//
// With P = exp(S - LSE) recomputed from the forward's log-sum-exp (so no T x T matrix is
// stored), the softmax backward is
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D) with D_i = sum_d dO_id O_id,
//     dS_pre = dS * (1 - tanh^2(S_pre / c)) when soft-capped,
//     dq^ = scale dS_pre k^,   dk^ = scale dS_pre^T q^.
// (The pages differentiate the attention forward of the "GPT pretraining" page, section
// "Multihead Attention", by autodiff inside their training step; these are the same
// derivatives written out.)
//
// Two kernels, no atomics:
//  * dkdv: one workgroup per (b, kv head, 128 keys), 4 waves x 32 keys.  K^ and V of the
//    wave's keys live in registers as MFMA B operands; the loop runs over every query head
//    of the GQA group and every query tile that can see the keys (causal: at or below the
//    diagonal; window: up to key + W - 1).  Q^ and dO tiles are staged row-major in LDS;
//    S = Q^ K^T and dP = dO V^T land with one KEY per lane (lane % 32), which is the layout
//    dV^T += dO^T P and dK^T += Q^T dS need for their B operands, and the transposed
//    A operands come from ds_read_b64_tr_b16.  dK and dV of a KV head are summed over its
//    query group inside the workgroup.
//  * dq: one workgroup per (b, h, 128 queries), the forward's layout (one QUERY per lane):
//    S^T and dP^T are recomputed, and dQ^T += K^T dS^T.
#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

struct BwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dO;
  const float* lse;
  const float* Dvec;
  void* dq;
  void* dk;
  bf16* dv;
  int grad_f32;
  int B, T, Hq, Hkv, window, ntiles;
  float scale, scale_log2, cap_k1, cap_k2;
};

// Scaled score in log2 units; with the cap also returns t = tanh(S_pre / c).
template <bool CAP>
__device__ __forceinline__ float score_log2(float x, const BwdArgs& a, float* t) {
  if constexpr (CAP) {
    const float e = exp2_fast(x * a.cap_k1);
    const float th = 1.f - 2.f * rcp_fast(e + 1.f);
    *t = th;
    return a.cap_k2 * th;
  } else {
    *t = 0.f;
    return x * a.scale_log2;
  }
}

template <int D>
__device__ __forceinline__ void store_grad_rowpart(void* base, int64_t row, int D_, int col,
                                                  const float* v4, bool f32) {
  if (f32) {
    float* p = reinterpret_cast<float*>(base) + row * D_ + col;
    *reinterpret_cast<f32x4*>(p) = f32x4{v4[0], v4[1], v4[2], v4[3]};
  } else {
    bf16* p = reinterpret_cast<bf16*>(base) + row * D_ + col;
    bf16x4 b4;
#pragma unroll
    for (int j = 0; j < 4; ++j) b4[j] = to_bf16(v4[j]);
    *reinterpret_cast<bf16x4*>(p) = b4;
  }
}

// ------------------------------------------------------------------------------------------
// dQ
// ------------------------------------------------------------------------------------------
constexpr int kBMq = 128;  // queries per dq workgroup
constexpr int kBNk = 64;   // keys per dq tile

template <int D, bool CAP>
__global__ __launch_bounds__(256, (D >= 128 ? 1 : 2)) void bwd_dq_kernel(BwdArgs a) {
  constexpr int LD = D + 8;
  constexpr int NS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int CPR = D / 8;
  constexpr int CPT = kBNk * CPR / 256;
  __shared__ __attribute__((aligned(16))) bf16 sK[2][kBNk * LD];
  __shared__ __attribute__((aligned(16))) bf16 sV[2][kBNk * LD];

  const int T = a.T;
  const int nbh = a.B * a.Hq;
  const int rank = blockIdx.x / nbh;
  const int bh = blockIdx.x - rank * nbh;
  const int qt = a.ntiles - 1 - rank;
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, gl = l >> 5, lr = l & 31;
  const int q0 = qt * kBMq, qw0 = q0 + 32 * w;
  const int qi = qw0 + lr;
  const int qrow = min(qi, T - 1);
  const int window = a.window;
  const bf16* kbase = a.k + (int64_t)(b * a.Hkv + g) * T * D;
  const bf16* vbase = a.v + (int64_t)(b * a.Hkv + g) * T * D;

  bf16x8 bq[NS], bdo[NS];
  {
    const int64_t off = ((int64_t)bh * T + qrow) * D + 8 * gl;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      bq[s] = ld16<bf16x8>(a.q + off + 16 * s);
      bdo[s] = ld16<bf16x8>(a.dO + off + 16 * s);
    }
  }
  const float lse2 = a.lse[(int64_t)bh * T + qrow] * kLog2e;
  const float Di = a.Dvec[(int64_t)bh * T + qrow];

  const int k_end = min(T, q0 + kBMq);
  const int k_begin = window > 0 ? max(0, q0 - window + 1) : 0;
  const int kt0 = k_begin / kBNk, kt1 = (k_end - 1) / kBNk;

  uint4 rk[CPT], rv[CPT];
  auto gload = [&](int kt) {
    const int k0 = kt * kBNk;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + 256 * c;
      const int row = idx / CPR, col = (idx - row * CPR) * 8;
      const int key = k0 + row;
      if (key < T) {
        rk[c] = ld16<uint4>(kbase + (int64_t)key * D + col);
        rv[c] = ld16<uint4>(vbase + (int64_t)key * D + col);
      } else {
        rk[c] = make_uint4(0, 0, 0, 0);
        rv[c] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + 256 * c;
      const int row = idx / CPR, col = (idx - row * CPR) * 8;
      *reinterpret_cast<uint4*>(&sK[buf][row * LD + col]) = rk[c];
      *reinterpret_cast<uint4*>(&sV[buf][row * LD + col]) = rv[c];
    }
  };

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[db][r] = 0.f;

  const bool wave_active = qw0 < T;
  const int qw_last = min(qw0 + 31, T - 1);
  const int trow = 4 * gl + ((l & 15) >> 2);
  const int tcol = 16 * ((l >> 4) & 1) + 4 * (l & 3);

  gload(kt0);
  sstore(0);
  __syncthreads();
  int cur = 0;
  for (int kt = kt0; kt <= kt1; ++kt) {
    const bool has_next = kt < kt1;
    if (has_next) gload(kt + 1);
    const int k0 = kt * kBNk;
    const bool skip = !wave_active || k0 > qw_last ||
                      (window > 0 && k0 + kBNk - 1 < qw0 - window + 1);
    if (!skip) {
      const bool need_mask = (k0 + kBNk - 1 > qw0) || (window > 0 && k0 < qw_last - window + 1);
      const bf16* sk = sK[cur];
      const bf16* sv = sV[cur];
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[kb][r] = 0.f;
          pacc[kb][r] = 0.f;
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int off = (kb * 32 + lr) * LD + 16 * s + 8 * gl;
          sacc[kb] = mfma32(ld16<bf16x8>(sk + off), bq[s], sacc[kb]);
          pacc[kb] = mfma32(ld16<bf16x8>(sv + off), bdo[s], pacc[kb]);
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float th;
          float y = score_log2<CAP>(sacc[kb][r], a, &th);
          if (need_mask) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * gl + (r & 3);
            if (key > qi || (window > 0 && qi - key >= window)) y = kNegBig;
          }
          const float p = exp2_fast(y - lse2);
          float ds = p * (pacc[kb][r] - Di);
          if constexpr (CAP) ds *= (1.f - th * th);
          sacc[kb][r] = ds;
        }
      bf16x8 dsb[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        dsb[kb][0] = pack8(sacc[kb], 0);
        dsb[kb][1] = pack8(sacc[kb], 8);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const bf16* p0 = sk + (kb * 32 + 16 * t + trow) * LD + 32 * db + tcol;
            dqacc[db] = mfma32(tr_read_pair(p0, p0 + 8 * LD), dsb[kb][t], dqacc[db]);
          }
    }
    if (has_next) sstore(cur ^ 1);
    __syncthreads();
    cur ^= 1;
  }

  if (qi < T) {
    const int64_t row = (int64_t)bh * T + qi;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float v4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v4[j] = dqacc[db][4 * i4 + j] * a.scale;
        store_grad_rowpart<D>(a.dq, row, D, 32 * db + 8 * i4 + 4 * gl, v4, a.grad_f32 != 0);
      }
  }
}

// ------------------------------------------------------------------------------------------
// dK, dV
// ------------------------------------------------------------------------------------------
constexpr int kBNkv = 128;  // keys per dkdv workgroup
constexpr int kBMt = 64;    // queries per dkdv tile

template <int D, bool CAP>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int LD = D + 8;
  constexpr int NS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int CPR = D / 8;
  constexpr int CPT = kBMt * CPR / 256;
  __shared__ __attribute__((aligned(16))) bf16 sQ[2][kBMt * LD];
  __shared__ __attribute__((aligned(16))) bf16 sO[2][kBMt * LD];  // dO tile
  __shared__ __attribute__((aligned(16))) float sL[2][kBMt];      // LSE * log2(e)
  __shared__ __attribute__((aligned(16))) float sD[2][kBMt];      // D = rowsum(dO * O)

  const int T = a.T;
  const int nbg = a.B * a.Hkv;
  const int kt = blockIdx.x / nbg;  // key tile 0 sees the most queries: heaviest first
  const int bg = blockIdx.x - kt * nbg;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, gl = l >> 5, lr = l & 31;
  const int kwg0 = kt * kBNkv;
  const int kw0 = kwg0 + 32 * w;
  const int kj = kw0 + lr;
  const int window = a.window;

  bf16x8 bk[NS], bv[NS];
  {
    const int64_t off = ((int64_t)bg * T + min(kj, T - 1)) * D + 8 * gl;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      bk[s] = ld16<bf16x8>(a.k + off + 16 * s);
      bv[s] = ld16<bf16x8>(a.v + off + 16 * s);
    }
  }

  const int kwg_last = min(kwg0 + kBNkv - 1, T - 1);
  const int q_begin = kwg0;
  const int q_end = window > 0 ? min(T, kwg_last + window) : T;
  const int qt0 = q_begin / kBMt, qt1 = (q_end - 1) / kBMt;
  const int nq = qt1 - qt0 + 1;
  const int nit = G * nq;

  uint4 rq[CPT], ro[CPT];
  float rl = 0.f, rd = 0.f;
  auto gload = [&](int it) {
    const int hh = it / nq;
    const int q0 = (qt0 + it - hh * nq) * kBMt;
    const int h = g * G + hh;
    const int64_t hbase = (int64_t)(b * a.Hq + h) * T;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + 256 * c;
      const int row = idx / CPR, col = (idx - row * CPR) * 8;
      const int qq = q0 + row;
      if (qq < T) {
        rq[c] = ld16<uint4>(a.q + (hbase + qq) * D + col);
        ro[c] = ld16<uint4>(a.dO + (hbase + qq) * D + col);
      } else {
        rq[c] = make_uint4(0, 0, 0, 0);
        ro[c] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < kBMt) {
      const int qq = q0 + tid;
      rl = qq < T ? a.lse[hbase + qq] * kLog2e : -kNegBig;  // rows past T: P = 0
    } else if (tid < 2 * kBMt) {
      const int qq = q0 + tid - kBMt;
      rd = qq < T ? a.Dvec[hbase + qq] : 0.f;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + 256 * c;
      const int row = idx / CPR, col = (idx - row * CPR) * 8;
      *reinterpret_cast<uint4*>(&sQ[buf][row * LD + col]) = rq[c];
      *reinterpret_cast<uint4*>(&sO[buf][row * LD + col]) = ro[c];
    }
    if (tid < kBMt)
      sL[buf][tid] = rl;
    else if (tid < 2 * kBMt)
      sD[buf][tid - kBMt] = rd;
  };

  f32x16 dvacc[NDB], dkacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dvacc[db][r] = 0.f;
      dkacc[db][r] = 0.f;
    }

  const bool wave_active = kw0 < T;
  const int kw_last = min(kw0 + 31, T - 1);
  const int trow = 4 * gl + ((l & 15) >> 2);
  const int tcol = 16 * ((l >> 4) & 1) + 4 * (l & 3);

  gload(0);
  sstore(0);
  __syncthreads();
  int cur = 0;
  for (int it = 0; it < nit; ++it) {
    const bool has_next = it + 1 < nit;
    if (has_next) gload(it + 1);
    const int hh = it / nq;
    const int q0 = (qt0 + it - hh * nq) * kBMt;
    const int q_last = min(q0 + kBMt - 1, T - 1);
    const bool skip = !wave_active || q_last < kw0 ||
                      (window > 0 && q0 > kw_last + window - 1);
    if (!skip) {
      const bool need_mask = (q0 < kw_last) || (window > 0 && q_last - kw0 >= window);
      const bf16* sq = sQ[cur];
      const bf16* so = sO[cur];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x16 sacc, pacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[r] = 0.f;
          pacc[r] = 0.f;
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int off = (qb * 32 + lr) * LD + 16 * s + 8 * gl;
          sacc = mfma32(ld16<bf16x8>(sq + off), bk[s], sacc);
          pacc = mfma32(ld16<bf16x8>(so + off), bv[s], pacc);
        }
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int qloc = qb * 32 + 8 * i4 + 4 * gl;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sL[cur][qloc]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sD[cur][qloc]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 4 * i4 + j;
            float th;
            float y = score_log2<CAP>(sacc[r], a, &th);
            if (need_mask) {
              const int iq = q0 + qloc + j;
              if (kj > iq || (window > 0 && iq - kj >= window)) y = kNegBig;
            }
            const float p = exp2_fast(y - l4[j]);
            float ds = p * (pacc[r] - d4[j]);
            if constexpr (CAP) ds *= (1.f - th * th);
            sacc[r] = p;
            pacc[r] = ds;
          }
        }
        bf16x8 pb[2], dsb[2];
        pb[0] = pack8(sacc, 0);
        pb[1] = pack8(sacc, 8);
        dsb[0] = pack8(pacc, 0);
        dsb[1] = pack8(pacc, 8);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int off = (qb * 32 + 16 * t + trow) * LD + 32 * db + tcol;
            dvacc[db] = mfma32(tr_read_pair(so + off, so + off + 8 * LD), pb[t], dvacc[db]);
            dkacc[db] = mfma32(tr_read_pair(sq + off, sq + off + 8 * LD), dsb[t], dkacc[db]);
          }
      }
    }
    if (has_next) sstore(cur ^ 1);
    __syncthreads();
    cur ^= 1;
  }

  if (kj < T) {
    const int64_t row = (int64_t)bg * T + kj;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float k4[4], v4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          k4[j] = dkacc[db][4 * i4 + j] * a.scale;
          v4[j] = dvacc[db][4 * i4 + j];
        }
        const int col = 32 * db + 8 * i4 + 4 * gl;
        store_grad_rowpart<D>(a.dk, row, D, col, k4, a.grad_f32 != 0);
        store_grad_rowpart<D>(a.dv, row, D, col, v4, false);
      }
  }
}

BwdArgs make_args(const BwdParams& p) {
  BwdArgs a;
  a.q = (const bf16*)p.q;
  a.k = (const bf16*)p.k;
  a.v = (const bf16*)p.v;
  a.dO = (const bf16*)p.dO;
  a.lse = p.lse;
  a.Dvec = p.Dvec;
  a.dq = p.dq;
  a.dk = p.dk;
  a.dv = (bf16*)p.dv;
  a.grad_f32 = p.grad_f32;
  a.B = p.B;
  a.T = p.T;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.window = p.window;
  a.ntiles = 0;
  a.scale = p.scale;
  a.scale_log2 = p.scale * kLog2e;
  const bool cap = p.softcap > 0.f;
  a.cap_k1 = cap ? 2.f * p.scale * kLog2e / p.softcap : 0.f;
  a.cap_k2 = cap ? p.softcap * kLog2e : 0.f;
  return a;
}

template <int D>
hipError_t launch_dq_d(const BwdParams& p, hipStream_t s) {
  BwdArgs a = make_args(p);
  a.ntiles = (p.T + kBMq - 1) / kBMq;
  const dim3 grid((unsigned)(a.ntiles * p.B * p.Hq));
  static const char* names[4] = {"bwd_dq_d32", "bwd_dq_d64", "bwd_dq_d96", "bwd_dq_d128"};
  TraceScope t(names[D / 32 - 1], s);
  if (p.softcap > 0.f)
    hipLaunchKernelGGL((bwd_dq_kernel<D, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dkdv_d(const BwdParams& p, hipStream_t s) {
  BwdArgs a = make_args(p);
  a.ntiles = (p.T + kBNkv - 1) / kBNkv;
  const dim3 grid((unsigned)(a.ntiles * p.B * p.Hkv));
  static const char* names[4] = {"bwd_dkdv_d32", "bwd_dkdv_d64", "bwd_dkdv_d96", "bwd_dkdv_d128"};
  TraceScope t(names[D / 32 - 1], s);
  if (p.softcap > 0.f)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dq(const BwdParams& p, hipStream_t s) {
  switch (p.D) {
    case 32: return launch_dq_d<32>(p, s);
    case 64: return launch_dq_d<64>(p, s);
    case 96: return launch_dq_d<96>(p, s);
    case 128: return launch_dq_d<128>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dkdv(const BwdParams& p, hipStream_t s) {
  switch (p.D) {
    case 32: return launch_dkdv_d<32>(p, s);
    case 64: return launch_dkdv_d<64>(p, s);
    case 96: return launch_dkdv_d<96>(p, s);
    case 128: return launch_dkdv_d<128>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace attn
