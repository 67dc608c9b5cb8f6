// Causal attention backward on gfx950: gradients of sum(O * dO) with respect to the raw
// q, k, v (before RoPE and QK-norm).
//
// With P = exp(S - LSE) recomputed from the forward's log-sum-exp (so no T x T matrix is
// stored), the softmax backward is
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D) with D_i = sum_d dO_id O_id,
//     dS_pre = dS * (1 - tanh^2(S_pre / c)) when soft-capped,
//     dq^ = scale dS_pre k^,   dk^ = scale dS_pre^T q^,
// and dq^, dk^ go back through RMSNorm (dy = (dy^ - y^ mean(dy^ y^)) / r) and RoPE (rotate
// by -angle).  (The pages differentiate the attention forward of the "GPT pretraining" page,
// section "Multihead Attention", by autodiff inside their training step; these are the
// same derivatives written out.)
//
// Two kernels, no atomics, launched dq then dkdv:
//  * dq: one workgroup per (b, h, 128 queries), the forward's layout (one QUERY per lane).
//    It applies the q prologue in registers (and writes q^ for dkdv), computes D_i from
//    the dO and O rows it holds, recomputes S^T and dP^T per key tile and accumulates
//    dQ^T += K^T dS^T; the prologue backward runs on the accumulators before the store.
//  * dkdv: one workgroup per (b, kv head, 128 keys), 4 waves x 32 keys.  k^ (prologue in
//    registers) and V of the wave's keys are MFMA B operands; the loop runs over every query
//    head of the GQA group and every query tile that can see the keys (causal: at or below
//    the diagonal; window: up to key + W - 1).  q^ and dO tiles are staged row-major in LDS;
//    S = q^ k^T and dP = dO V^T land with one KEY per lane (lane % 32), which is the layout
//    dV^T += dO^T P and dK^T += q^T dS need for their B operands; the transposed A operands
//    come from ds_read_b64_tr_b16.  dK and dV of a KV head are summed over its query group
//    inside the workgroup.
//
// Within a tile each wave issues one 32-row block's (or half block's) MFMAs beside another
// block's gradient arithmetic, so its matrix and vector units work at once; how far that goes
// depends on the registers the instantiation has (see the step and run variants).
//
// Dropout on the weights (O = (P * Z) V, Z = keep / (1 - rate)): dV = (P * Z)^T dO and
// dS = P * (Z * (dO V^T) - D) with the same D.  The DROP instantiations stage each tile's
// keep words in LDS beside it (row layout for dq, column layout for dkdv), start dP at 0
// instead of -D, and scale dV once at the end.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

struct BwdArgs {
  const bf16* q;    // raw q
  const bf16* k;    // raw k
  const bf16* kh;   // k^ (dq pass)
  bf16* qh;         // q^ (written by dq, read by dkdv)
  const bf16* v;
  const bf16* o;
  const bf16* dO;
  const float* lse;
  float* Dvec;
  float* L2;  // LSE * log2(e) per query row (written by dq for dkdv)
  const int32_t* seg_start;  // packed rows: first / last index of each token's run, [B, T]
  const int32_t* seg_end;    // (null: one run per row)
  const uint32_t* drop_rows; // dropout keep masks, row and column layouts (or null)
  const uint32_t* drop_cols;
  int drop_pitch;
  float drop_scale;          // kept-weight scale 1 / (1 - rate)
  bf16* dq;
  bf16* dk;
  bf16* dv;
  int B, T, Hq, Hkv, window, ntiles;
  int pro;  // RoPE or QK-norm on
  float scale;
  ScoreCoef sc;
  RowPrologue rp;
  bf16* ds;    // split backward: dS fragments (null: not exported / not used)
  DsBand band;
};

// ---- dS fragments ----------------------------------------------------------------------------
// Key blocks lo .. hi of 32-query block i, and the fragment index of (i, j) within a head.
__device__ __forceinline__ int ds_lo(int i, const DsBand& d) {
  return d.window > 0 ? max(0, 32 * i - d.window + 1) >> 4 : 0;
}
__device__ __forceinline__ int ds_hi(int i, const DsBand& d) { return min(2 * i + 1, d.nkb - 1); }
__device__ __forceinline__ int64_t ds_frag(int i, int j, const DsBand& d) {
  return d.stride == 0 ? (int64_t)i * (i + 1) + j : (int64_t)i * d.stride + (j - ds_lo(i, d));
}

// Store 4 consecutive values of a row (accumulator layout) as bf16.
__device__ __forceinline__ void store4(bf16* p, const float* v) {
  bf16x4 b4;
#pragma unroll
  for (int j = 0; j < 4; ++j) b4[j] = to_bf16(v[j]);
  *reinterpret_cast<bf16x4*>(p) = b4;
}

// Write a gradient row held as accumulators acc[db][16] (layout: d = 32 db + 8 (r/4) + 4 gl
// + r%4) after scaling and, when RoPE/QK-norm are on, the prologue backward against the raw
// input row xraw (at position pos).  Must be called by all lanes; stores only if `store`.
template <int D>
__device__ __forceinline__ void finish_grad_row(const f32x16 (&acc)[D / 32], float scale,
                                                const bf16* xraw, bf16* out, int pos, int gl,
                                                bool pro, const RowPrologue& rp, bool store) {
  constexpr int NE = D / 8;
  float g[NE][4];
#pragma unroll
  for (int e = 0; e < NE; ++e)
#pragma unroll
    for (int j = 0; j < 4; ++j) g[e][j] = acc[e / 4][4 * (e % 4) + j] * scale;
  if (pro) {
    float xr[NE][4];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const bf16x4 v4 = *reinterpret_cast<const bf16x4*>(xraw + 8 * e + 4 * gl);
#pragma unroll
      for (int j = 0; j < 4; ++j) xr[e][j] = (float)v4[j];
    }
    prologue_backward_acclayout<NE>(g, xr, pos, gl, rp, D);
  }
  if (store) {
#pragma unroll
    for (int e = 0; e < NE; ++e) store4(out + 8 * e + 4 * gl, g[e]);
  }
}

// ------------------------------------------------------------------------------------------
// dQ
// ------------------------------------------------------------------------------------------
constexpr int kBMq = 128;  // queries per dq workgroup
constexpr int kBNk = 64;   // keys per dq tile

// Two waves per SIMD where the registers fit (all D <= 96; D = 128 without a soft-cap).
template <int D, int MODE, bool DROP>
__global__ __launch_bounds__(256, (D <= 96 || MODE == kScoreScale) ? 2 : 1) void bwd_dq_kernel(BwdArgs a) {
  constexpr int LD = D + 8;
  constexpr int NS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TILE = kBNk * LD;
  static_assert(kBNk == 64 && TILE % 512 == 0, "tiles are 64 padded rows, whole 1 KB chunks");
  __shared__ __attribute__((aligned(16))) bf16 sK0[TILE];
  __shared__ __attribute__((aligned(16))) bf16 sK1[TILE];
  __shared__ __attribute__((aligned(16))) bf16 sV0[TILE];
  __shared__ __attribute__((aligned(16))) bf16 sV1[TILE];
  // Dropout keep words of the tile's two 32-key blocks for the 128 queries: [block][query].
  __shared__ __attribute__((aligned(16))) uint32_t sM0[DROP ? 2 * kBMq : 1];
  __shared__ __attribute__((aligned(16))) uint32_t sM1[DROP ? 2 * kBMq : 1];

  const int T = a.T;
  const int nbh = a.B * a.Hq;
  const int rank = blockIdx.x / nbh;
  const int bh = xcd_local_head(blockIdx.x - rank * nbh, nbh);
  const int qt = a.ntiles - 1 - rank;
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const int tid = threadIdx.x, l = tid & 63, gl = l >> 5, lr = l & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int q0 = qt * kBMq, qw0 = q0 + 32 * w;
  const int qi = qw0 + lr;
  const int qrow = min(qi, T - 1);
  const int window = a.window;
  const unsigned wlim = window > 0 ? (unsigned)window : 0x7fffffffu;
  // Packed rows: this lane's query sees keys back to the start of its run only.
  const int32_t* sst = a.seg_start ? a.seg_start + (int64_t)b * T : nullptr;
  const unsigned lim = sst ? min(wlim, (unsigned)(qrow - sst[qrow] + 1)) : wlim;
  const bf16* kbase = a.kh + (int64_t)(b * a.Hkv + g) * T * D;
  const bf16* vbase = a.v + (int64_t)(b * a.Hkv + g) * T * D;
  const int64_t rowoff = ((int64_t)bh * T + qrow) * D;

  bf16x8 bq[NS], bdo[NS];
  float Di;
  {
    const int64_t off = rowoff + 8 * gl;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      bq[s] = ld16<bf16x8>(a.q + off + 16 * s);
      bdo[s] = ld16<bf16x8>(a.dO + off + 16 * s);
    }
    if (a.pro) {
      float x[NS][8];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int p = 0; p < 8; ++p) x[s][p] = (float)bq[s][p];
      prologue_oplayout<NS>(x, qrow, gl, a.rp, D);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int p = 0; p < 8; ++p) bq[s][p] = to_bf16(x[s][p]);
        if (qi < T) *reinterpret_cast<bf16x8*>(a.qh + off + 16 * s) = bq[s];
      }
    }
    // D_i = dO_i . O_i from the rows this lane pair holds.
    float dsum = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 ov = ld16<bf16x8>(a.o + off + 16 * s);
#pragma unroll
      for (int p = 0; p < 8; ++p) dsum = fmaf((float)bdo[s][p], (float)ov[p], dsum);
    }
    Di = pair_sum(dsum);
    if (gl == 0 && qi < T) a.Dvec[(int64_t)bh * T + qi] = -Di;
  }
  const float lse2 = a.lse[(int64_t)bh * T + qrow] * kLog2e;
  if (gl == 0 && qi < T) a.L2[(int64_t)bh * T + qi] = lse2;

  const int k_end = min(T, q0 + kBMq);
  const int k_begin = max(window > 0 ? max(0, q0 - window + 1) : 0, sst ? sst[q0] : 0);
  const int kt0 = k_begin / kBNk, kt1 = (k_end - 1) / kBNk;

  // Rows past T read clamped, finite data that the causal mask removes.
  const TileDma<D, 4> tdma(w, l);
  auto dma = [&](int kt, int buf) {
    tdma.copy(buf ? sK1 : sK0, kbase, kt * kBNk, T, w);
    tdma.copy(buf ? sV1 : sV0, vbase, kt * kBNk, T, w);
    if constexpr (DROP) {
      // Wave w: keep word of block (w & 1) for queries q0 + 64 (w >> 1) + lane.
      const int row = min(q0 + 64 * (w >> 1) + l, T - 1);
      __builtin_amdgcn_global_load_lds(
          a.drop_rows + ((int64_t)bh * T + row) * a.drop_pitch + 2 * kt + (w & 1),
          (buf ? sM1 : sM0) + (w & 1) * kBMq + 64 * (w >> 1), 4, 0, 0);
    }
  };

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[db][r] = 0.f;

  const bool wave_active = qw0 < T;
  const int qw_last = min(qw0 + 31, T - 1);
  // Earliest and latest run start among the wave's queries (packed rows).
  const int s_lo = sst ? sst[min(qw0, T - 1)] : 0, s_hi = sst ? sst[qw_last] : 0;
  const int trow = 4 * gl + ((l & 15) >> 2);
  const int tcol = 16 * ((l >> 4) & 1) + 4 * (l & 3);

  // One key tile, two 32-key blocks.  For each block: S^T = K q^T and dP^T = V dO^T, then
  // dS = P (dP - D) and dQ^T += K^T dS^T.
  // The wave's instruction stream pairs the matrix work of one block with the elementwise
  // work of the other, so the wave keeps its matrix and vector units busy at once: block 0's
  // products; block 1's products beside block 0's dS; block 0's dQ products beside block 1's
  // dS; block 1's dQ products.
  auto run_paired = [&](int kt, const bf16* sk, const bf16* sv,
                      const uint32_t* sm) __attribute__((always_inline)) {
    const int k0 = kt * kBNk;
    const bool skip = !wave_active || k0 > qw_last || k0 + kBNk - 1 < s_lo ||
                      (window > 0 && k0 + kBNk - 1 < qw0 - window + 1);
    if (skip) return;
    uint32_t mw[2] = {0u, 0u};
    if constexpr (DROP) {
      mw[0] = sm[qi - q0] >> (4 * gl);
      mw[1] = sm[kBMq + qi - q0] >> (4 * gl);
    }
    const bool need_mask = (k0 + kBNk - 1 > qw0) || k0 < s_hi ||
                           (window > 0 && k0 < qw_last - window + 1);
    // qi - key for element (kb, r) is qd - (32 kb + 8 (r / 4) + r % 4).
    const int qd = qi - k0 - 4 * gl;

    // Score modes other than the exp form mask in place of the raw score (a.sc.mask_acc, right
    // after a block's score MFMAs, in a uniform branch), so masked and unmasked tiles share one
    // body: two bodies would join with the dQ accumulators in different registers, and the
    // moves that reconcile them cost more than the selects.  The exp form's capped scores are
    // bounded, so it keeps a masked body that masks after the transform.
    constexpr bool kAccMask = MODE != kScoreCapExp;
    auto body = [&](auto masked) {
      f32x16 sacc[2], pacc[2];
      bf16x8 dsb[2][2];
      auto mask_block = [&](int kb) {
        if constexpr (kAccMask) {
          if (need_mask) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
              sacc[kb][r] = visible(qd - (32 * kb + 8 * (r >> 2) + (r & 3)), lim) ? sacc[kb][r]
                                                                                   : a.sc.mask_acc;
          }
        }
      };
      // dS for element r of block kb, in place of its score.
      auto grad = [&](int kb, int r) {
        float gf;
        float y = score_grad<MODE>(sacc[kb][r], a.sc, lse2, &gf);
        if constexpr (decltype(masked)::value)
          y = visible(qd - (32 * kb + 8 * (r >> 2) + (r & 3)), lim) ? y : kNegBig;
        float p = exp2_fast(y);
        if constexpr (MODE != kScoreScale) p *= gf;
        if constexpr (DROP)
          sacc[kb][r] = p * fmaf(keep_only(a.drop_scale, mw[kb], r), pacc[kb][r], -Di);
        else
          sacc[kb][r] = p * (pacc[kb][r] - Di);
        // Pins the element's arithmetic to the step that asks for it (the scheduling fences
        // alone leave free arithmetic to drift towards its first use).
        asm volatile("" : "+v"(sacc[kb][r]));
      };
      auto kv_off = [&](int kb, int s) { return (kb * 32 + lr) * LD + 16 * s + 8 * gl; };
      auto kt_ptr = [&](int kb, int i) {  // step i = NDB t + db of block kb's dQ products
        return sk + (kb * 32 + 16 * (i / NDB) + trow) * LD + 32 * (i % NDB) + tcol;
      };
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[kb][r] = 0.f;  // zero accumulators need no vector instructions before the MFMA
          pacc[kb][r] = 0.f;
        }
      // Operand reads run PF steps ahead of their MFMAs (one where dropout's keep words leave
      // no registers for a second set).
      constexpr int PF = (DROP && D >= 96) ? 1 : 2;
      // Both blocks' S / dP products as one stream of 2 NS steps (step j: block j / NS, slice
      // j % NS); block 1's steps each carry a share of block 0's dS.
      bf16x8 ka[PF], va[PF];
#pragma unroll
      for (int j = 0; j < PF; ++j) {
        ka[j] = ld16<bf16x8>(sk + kv_off(j / NS, j % NS));
        va[j] = ld16<bf16x8>(sv + kv_off(j / NS, j % NS));
      }
#pragma unroll
      for (int j = 0; j < 2 * NS; ++j) {
        const int kb = j / NS, s = j % NS;
        if (j == NS) mask_block(0);
        sacc[kb] = mfma32(ka[j % PF], bq[s], sacc[kb]);
        pacc[kb] = mfma32(va[j % PF], bdo[s], pacc[kb]);
        if (j + PF < 2 * NS) {
          ka[j % PF] = ld16<bf16x8>(sk + kv_off((j + PF) / NS, (j + PF) % NS));
          va[j % PF] = ld16<bf16x8>(sv + kv_off((j + PF) / NS, (j + PF) % NS));
        }
        if (kb == 1) {
#pragma unroll
          for (int r = 16 * s / NS; r < 16 * (s + 1) / NS; ++r) grad(0, r);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      mask_block(1);
      dsb[0][0] = pack8(sacc[0], 0);
      dsb[0][1] = pack8(sacc[0], 8);
      // Both blocks' dQ products as one stream of 4 NDB steps (step i: block i / (2 NDB),
      // product i % (2 NDB) = NDB t + db).  Block 1's dS shares them out by halves: elements
      // 0-7 beside block 0's products, elements 8-15 beside block 1's first-half products,
      // which need only elements 0-7.
      auto kt_at = [&](int i) {
        const bf16* p0 = kt_ptr(i / (2 * NDB), i % (2 * NDB));
        return tr_read_pair(p0, p0 + 8 * LD);
      };
      bf16x8 kt_[PF];
#pragma unroll
      for (int i = 0; i < PF; ++i) kt_[i] = kt_at(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4 * NDB; ++i) {
        const int kb = i / (2 * NDB), k = i % (2 * NDB);
        if (i == 2 * NDB) dsb[1][0] = pack8(sacc[1], 0);
        if (i == 3 * NDB) dsb[1][1] = pack8(sacc[1], 8);
        dqacc[k % NDB] = mfma32(kt_[i % PF], dsb[kb][k / NDB], dqacc[k % NDB]);
        if (i + PF < 4 * NDB) kt_[i % PF] = kt_at(i + PF);
        if (i < 3 * NDB) {
          const int h = i / (2 * NDB) == 0 ? i : i - 2 * NDB;  // step within its share
          const int n = i < 2 * NDB ? 2 * NDB : NDB;          // steps in the share
          const int r0 = i < 2 * NDB ? 0 : 8;
#pragma unroll
          for (int r = r0 + 8 * h / n; r < r0 + 8 * (h + 1) / n; ++r) grad(1, r);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if constexpr (kAccMask)
      body(std::false_type{});
    else if (need_mask)
      body(std::true_type{});
    else
      body(std::false_type{});
  };

  // The same tile in phases: S^T and dP^T for both blocks (dP^T accumulates on top of -D_i,
  // so it comes out as dP - D), then per half block dS and dQ^T += K^T dS^T.  The phase
  // fences keep one phase's registers live at a time.
  auto run_phased = [&](int kt, const bf16* sk, const bf16* sv,
                      const uint32_t* sm) __attribute__((always_inline)) {
    const int k0 = kt * kBNk;
    const bool skip = !wave_active || k0 > qw_last || k0 + kBNk - 1 < s_lo ||
                      (window > 0 && k0 + kBNk - 1 < qw0 - window + 1);
    if (skip) return;
    uint32_t mw[2] = {0u, 0u};
    if constexpr (DROP) {
      mw[0] = sm[qi - q0] >> (4 * gl);
      mw[1] = sm[kBMq + qi - q0] >> (4 * gl);
    }
    const bool need_mask = (k0 + kBNk - 1 > qw0) || k0 < s_hi ||
                           (window > 0 && k0 < qw_last - window + 1);
    // qi - key for element (kb, r) is qd - (32 kb + 8 (r / 4) + r % 4).
    const int qd = qi - k0 - 4 * gl;
    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[kb][r] = 0.f;
        pacc[kb][r] = DROP ? 0.f : -Di;
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int off = (kb * 32 + lr) * LD + 16 * s + 8 * gl;
        const bf16x8 ka = ld16<bf16x8>(sk + off);
        const bf16x8 va = ld16<bf16x8>(sv + off);
        sacc[kb] = mfma32(ka, bq[s], sacc[kb]);
        pacc[kb] = mfma32(va, bdo[s], pacc[kb]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // Half t: elements 8t .. 8t + 7 (keys 16t .. 16t + 15 of the block).
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        auto grads = [&](auto masked) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 8 * t + e;
            float gf;
            float y = score_grad<MODE>(sacc[kb][r], a.sc, lse2, &gf);
            if constexpr (decltype(masked)::value)
              y = visible(qd - (32 * kb + 8 * (r >> 2) + (r & 3)), lim) ? y : kNegBig;
            float p = exp2_fast(y);
            if constexpr (MODE != kScoreScale) p *= gf;
            if constexpr (DROP)
              sacc[kb][r] = p * fmaf(keep_only(a.drop_scale, mw[kb], r), pacc[kb][r], -Di);
            else
              sacc[kb][r] = p * pacc[kb][r];
          }
        };
        if (need_mask)
          grads(std::true_type{});
        else
          grads(std::false_type{});
        const bf16x8 dsb = pack8(sacc[kb], 8 * t);
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 kt_[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16* p0 = sk + (kb * 32 + 16 * t + trow) * LD + 32 * db + tcol;
          kt_[db] = tr_read_pair(p0, p0 + 8 * LD);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) dqacc[db] = mfma32(kt_[db], dsb, dqacc[db]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // The paired order holds about twenty more registers than the phased one; at d = 128
  // without a soft-cap (two waves per SIMD, 256 registers each) that would spill.
  auto run = [&](int kt, const bf16* sk, const bf16* sv,
               const uint32_t* sm) __attribute__((always_inline)) {
    if constexpr (D >= 128 && MODE == kScoreScale)
      run_phased(kt, sk, sv, sm);
    else
      run_paired(kt, sk, sv, sm);
  };

  // Two-deep pipeline over key tiles, unrolled by two so each LDS buffer is a distinct
  // array: the loads into one buffer never wait on reads of the other.
  dma(kt0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kt = kt0; kt <= kt1; kt += 2) {
    if (kt + 1 <= kt1) dma(kt + 1, 1);
    run(kt, sK0, sV0, sM0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 1 > kt1) break;
    if (kt + 2 <= kt1) dma(kt + 2, 0);
    run(kt + 1, sK1, sV1, sM1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  finish_grad_row<D>(dqacc, a.scale, a.q + rowoff, a.dq + rowoff, qrow, gl, a.pro != 0, a.rp,
                     qi < T);
}

// ------------------------------------------------------------------------------------------
// dK, dV
// ------------------------------------------------------------------------------------------
constexpr int kBNkv = 128;  // keys per dkdv workgroup
constexpr int kBMt = 64;    // queries per dkdv tile

// Two waves per SIMD for D <= 64, and for D = 96 without dropout (its keep words and -D
// values no longer fit the 256 registers two waves allow); one otherwise.
// EXPORT: also store this pass's dS as fragments for bwd_dq_ds_kernel (the split backward).
template <int D, int MODE, bool DROP, bool EXPORT>
__global__ __launch_bounds__(256, (D >= 128 || (DROP && D >= 96)) ? 1 : 2) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int LD = D + 8;
  constexpr int NS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TILE = kBMt * LD;  // elements of one padded tile (a whole number of 1 KB)
  static_assert(TILE % 512 == 0, "tile image must be whole 1 KB chunks");
  __shared__ __attribute__((aligned(16))) bf16 sQ0[TILE];
  __shared__ __attribute__((aligned(16))) bf16 sQ1[TILE];
  __shared__ __attribute__((aligned(16))) bf16 sO0[TILE];  // dO tiles
  __shared__ __attribute__((aligned(16))) bf16 sO1[TILE];
  __shared__ __attribute__((aligned(16))) float sL[2][kBMt];  // LSE * log2(e)
  __shared__ __attribute__((aligned(16))) float sD[2][kBMt];  // -D, D = rowsum(dO * O)
  // Dropout keep words of the tile's two 32-query blocks for the 128 keys: [block][key].
  __shared__ __attribute__((aligned(16))) uint32_t sM0[DROP ? 2 * kBNkv : 1];
  __shared__ __attribute__((aligned(16))) uint32_t sM1[DROP ? 2 * kBNkv : 1];
  // Split backward: each wave's dS of the current tile, [32 keys][64 queries + 8] bf16, written
  // in the accumulator layout and read back transposed into fragments (wave-private: no barrier).
  constexpr int DSP = kBMt + 8;
  __shared__ __attribute__((aligned(16))) bf16 sDS[EXPORT ? 4 * 32 * DSP : 1];

  const int T = a.T;
  const int nbg = a.B * a.Hkv;
  const int kt = blockIdx.x / nbg;  // key tile 0 sees the most queries: heaviest first
  // Contiguous (b, kv head) ranges per XCD, as the dq grid places its heads: a group's q^ rows
  // were written through the L2 this workgroup reads from.
  const int bg = xcd_local_head(blockIdx.x - kt * nbg, nbg);
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int tid = threadIdx.x, l = tid & 63, gl = l >> 5, lr = l & 31;
  const int w = tid >> 6;
  const int kwg0 = kt * kBNkv;
  const int kw0 = kwg0 + 32 * w;
  const int kj = kw0 + lr;
  const int krow = min(kj, T - 1);
  const int window = a.window;
  // Query i sees this lane's key j iff 0 <= i - j < lim: the causal / window rule, i < T
  // (query rows past T are clamped copies of row T - 1 and must get P = 0) and, for packed
  // rows, i <= the last index of the key's run.
  const int32_t* sen = a.seg_end ? a.seg_end + (int64_t)b * T : nullptr;
  const unsigned lim = (unsigned)min(min(window > 0 ? window : 0x7fffffff, max(T - kj, 0)),
                                     sen ? max(sen[krow] - kj + 1, 0) : 0x7fffffff);
  const int64_t krowoff = ((int64_t)bg * T + krow) * D;
  const bf16* qsrc = a.pro ? a.qh : a.q;

  bf16x8 bk[NS], bv[NS];
  {
    const int64_t off = krowoff + 8 * gl;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      bk[s] = ld16<bf16x8>(a.k + off + 16 * s);
      bv[s] = ld16<bf16x8>(a.v + off + 16 * s);
    }
    if (a.pro) {
      float x[NS][8];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int p = 0; p < 8; ++p) x[s][p] = (float)bk[s][p];
      prologue_oplayout<NS>(x, krow, gl, a.rp, D);
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int p = 0; p < 8; ++p) bk[s][p] = to_bf16(x[s][p]);
    }
  }

  const int kwg_last = min(kwg0 + kBNkv - 1, T - 1);
  const int q_begin = kwg0;
  const int q_end = min(window > 0 ? min(T, kwg_last + window) : T, sen ? sen[kwg_last] + 1 : T);
  const int qt0 = q_begin / kBMt, qt1 = (q_end - 1) / kBMt;
  const int nq = qt1 - qt0 + 1;
  const int nit = G * nq;

  // Query tile of iteration it (query head hh = it / nq).  Without a window and with at least
  // 8 tiles per head, from the last tile back to the diagonal: every key block of a KV group
  // then starts at the same tile and walks in step with the others, so the workgroups on one
  // XCD read each q^ / dO tile at about the same time and the L2 serves all but the first
  // (a third fewer fetches beyond L2 at T = 2048, in the same time).  Otherwise from the
  // diagonal down (the reversed walk was slower with a window or short ranges).
  const bool walk_down = window == 0 && nq >= 8;
  auto q_tile = [&](int it, int hh) {
    const int u = it - hh * nq;
    return (walk_down ? qt1 - u : qt0 + u) * kBMt;
  };
  const TileDma<D, 4> tdma(w, l);
  // Issue the direct loads of iteration it's q^ / dO tiles and LSE / D vectors into
  // buffer `buf`; they are waited for at the end of the iteration that issues them.
  auto dma = [&](int it, int buf) {
    const int hh = it / nq;
    const int q0 = q_tile(it, hh);
    const int64_t hbase = (int64_t)(b * a.Hq + g * G + hh) * T;
    tdma.copy(buf ? sQ1 : sQ0, qsrc + hbase * D, q0, T, w);
    tdma.copy(buf ? sO1 : sO0, a.dO + hbase * D, q0, T, w);
    const int64_t qc = hbase + min(q0 + l, T - 1);
    if (w == 2) __builtin_amdgcn_global_load_lds(a.L2 + qc, &sL[buf][0], 4, 0, 0);
    if (w == 3) __builtin_amdgcn_global_load_lds(a.Dvec + qc, &sD[buf][0], 4, 0, 0);
    if constexpr (DROP) {
      // Wave w: keep word of query block (w & 1) for keys kwg0 + 64 (w >> 1) + lane.
      const int key = min(kwg0 + 64 * (w >> 1) + l, T - 1);
      __builtin_amdgcn_global_load_lds(
          a.drop_cols + (hbase + key) * a.drop_pitch + q0 / 32 + (w & 1),
          (buf ? sM1 : sM0) + (w & 1) * kBNkv + 64 * (w >> 1), 4, 0, 0);
    }
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
  // Earliest and latest run end among the wave's keys (packed rows; run ends grow with the
  // token index).
  const int e_lo = sen ? sen[min(kw0, T - 1)] : T, e_hi = sen ? sen[kw_last] : T;
  const int trow = 4 * gl + ((l & 15) >> 2);
  const int tcol = 16 * ((l >> 4) & 1) + 4 * (l & 3);

  // dS export.  stash(qb, t, v): v = dS of block qb, half t packed as bf16 (elements 0-3:
  // queries 16 t + 4 gl + 0..3 of the block, 4-7: 16 t + 8 + 4 gl + 0..3) into this wave's
  // [key][query] buffer.  export_ds(q0): after the tile, the transposing reads turn it into
  // the fragments of (32-query block, 16-key block) pairs inside the band, stored whole.
  static_assert(!(EXPORT && DROP), "dS export is for the plain backward");
  // The lane's offsets into the buffer are recomputed from a fresh lane id at each use (the
  // empty asm keeps them from being held in registers across the tile loop).
  auto lane_id = []() __attribute__((always_inline)) {
    int t = (int)__builtin_amdgcn_workitem_id_x();
    asm volatile("" : "+v"(t));
    return t;
  };
  auto stash = [&](int qb, int t, const bf16x8& v) __attribute__((always_inline)) {
    if constexpr (EXPORT) {
      const int id = lane_id(), ll = id & 63;
      bf16* row = sDS + ((id >> 6) * 32 + (ll & 31)) * DSP + 4 * (ll >> 5) + 32 * qb + 16 * t;
      *reinterpret_cast<bf16x4*>(row) = bf16x4{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<bf16x4*>(row + 8) = bf16x4{v[4], v[5], v[6], v[7]};
    }
  };
  auto export_ds = [&](int hh, int q0) __attribute__((always_inline)) {
    if constexpr (EXPORT) {
      const int id = lane_id(), ll = id & 63, gq = ll >> 4, L = ll & 15;
      // Loader role of this lane: key row 8 (gq / 2) + L / 4 (+ 4), query columns
      // 16 (gq % 2) + 4 (L % 4) .. + 3 of the fragment's 16 x 32 window.
      const bf16* src = sDS + ((id >> 6) * 32 + 8 * (gq >> 1) + (L >> 2)) * DSP +
                        16 * (gq & 1) + 4 * (L & 3);
      bf16* dst = a.ds + ((int64_t)(b * a.Hq + g * G + hh) * a.band.frags) * 512 + 8 * ll;
#pragma unroll
      for (int qf = 0; qf < 2; ++qf) {
        const int i = (q0 >> 5) + qf;
        if (i >= a.band.nqb) continue;
        const int lo = ds_lo(i, a.band), hi = ds_hi(i, a.band);
#pragma unroll
        for (int kf = 0; kf < 2; ++kf) {
          const int j = (kw0 >> 4) + kf;
          if (j < lo || j > hi) continue;
          const bf16* p0 = src + 16 * kf * DSP + 32 * qf;
          const bf16x8 v = tr_read_pair(p0, p0 + 4 * DSP);
          // Streamed past the L2, where this pass keeps its q^ / dO tiles.
          __builtin_nontemporal_store(v, reinterpret_cast<bf16x8*>(dst + ds_frag(i, j, a.band) * 512));
        }
      }
    }
  };

  // One q tile against this wave's 32 keys, operands in (sq, so, sl, sd), keep words in sm:
  // the two 32-query blocks one after the other.
  auto step_split = [&](int it, const bf16* sq, const bf16* so, const float* sl,
                        const float* sd, const uint32_t* sm) __attribute__((always_inline)) {
    const int hh = it / nq;
    const int q0 = q_tile(it, hh);
    const int q_last = min(q0 + kBMt - 1, T - 1);
    const bool skip = !wave_active || q_last < kw0 || q0 > e_hi ||
                      (window > 0 && q0 > kw_last + window - 1);
    if (skip) return;
    const bool need_mask = (q0 < kw_last) || (q0 + kBMt > T) || q_last > e_lo ||
                           (window > 0 && q_last - kw0 >= window);
    // iq - kj for element (qb, r) is kd + 32 qb + 8 (r / 4) + r % 4.
    const int kd = q0 + 4 * gl - kj;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // S = q^ k^T and dP = dO V^T for 32 queries x this wave's 32 keys; dP accumulates on
      // top of -D (element r belongs to query offset 8 (r / 4) + r % 4 of the block), so it
      // comes out as dP - D.
      f32x16 sacc, pacc;
      uint32_t mw = 0u;
      if constexpr (DROP) {
        mw = sm[qb * kBNkv + kj - kwg0] >> (4 * gl);
#pragma unroll
        for (int r = 0; r < 16; ++r) pacc[r] = 0.f;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 nd = *reinterpret_cast<const float4*>(sd + qb * 32 + 4 * gl + 8 * i);
          pacc[4 * i] = nd.x;
          pacc[4 * i + 1] = nd.y;
          pacc[4 * i + 2] = nd.z;
          pacc[4 * i + 3] = nd.w;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int off = (qb * 32 + lr) * LD + 16 * s + 8 * gl;
        const bf16x8 qa = ld16<bf16x8>(sq + off);
        const bf16x8 oa = ld16<bf16x8>(so + off);
        sacc = mfma32(qa, bk[s], sacc);
        pacc = mfma32(oa, bv[s], pacc);
      }
      // Phase fences: with two waves per SIMD the other wave fills one wave's MFMA, VALU
      // and LDS phases, so each wave keeps only one phase's registers live.
      __builtin_amdgcn_sched_barrier(0);
      // The exp-form soft-cap's gradient holds a few more registers; at d >= 96 pairing the
      // halves would spill, so there they run one after the other.
      if constexpr (MODE != kScoreCapExp || D < 96) {
        // Half t covers elements 8t .. 8t + 7 (queries 16t .. 16t + 15 of the block): the
        // softmax gradient, then that half's share of dV^T += dO^T P and dK^T += q^T dS.  Half
        // 0's products are issued beside half 1's gradient, so the wave's matrix and vector
        // units work at once.
        float4 lq[2][2], nq[2][2];  // LSE and -D (dropout only) of each half's queries
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            lq[t][j] = *reinterpret_cast<const float4*>(sl + qb * 32 + 4 * gl + 16 * t + 8 * j);
            if constexpr (DROP)
              nq[t][j] = *reinterpret_cast<const float4*>(sd + qb * 32 + 4 * gl + 16 * t + 8 * j);
          }
        auto grad = [&](auto masked, int r) {
          const int t = r >> 3, e = r & 7;
          const int qo = 8 * (r >> 2) + (r & 3);
          const float4 l4 = lq[t][e >> 2];
          const float lse = (e & 3) == 0 ? l4.x : (e & 3) == 1 ? l4.y : (e & 3) == 2 ? l4.z : l4.w;
          float gf;
          float y = score_grad<MODE>(sacc[r], a.sc, lse, &gf);
          if constexpr (decltype(masked)::value) y = visible(kd + 32 * qb + qo, lim) ? y : kNegBig;
          const float p = exp2_fast(y);
          float ds;
          if constexpr (DROP) {
            const float4 n4 = nq[t][e >> 2];
            const float nd = (e & 3) == 0 ? n4.x : (e & 3) == 1 ? n4.y : (e & 3) == 2 ? n4.z : n4.w;
            ds = p * fmaf(keep_only(a.drop_scale, mw, r), pacc[r], nd);
            sacc[r] = keep_only(p, mw, r);  // dV takes the kept weights; scaled at the end
          } else {
            ds = p * pacc[r];
            sacc[r] = p;
          }
          if constexpr (MODE != kScoreScale) ds *= gf;
          pacc[r] = ds;
          // Pins the element's arithmetic to the step that asks for it.
          asm volatile("" : "+v"(sacc[r]), "+v"(pacc[r]));
        };
        auto tr_off = [&](int i) {  // product step i = NDB t + db
          return (qb * 32 + 16 * (i / NDB) + trow) * LD + 32 * (i % NDB) + tcol;
        };
        auto half = [&](auto masked) {
#pragma unroll
          for (int r = 0; r < 8; ++r) grad(masked, r);
          bf16x8 pb[2], dsb[2];
          pb[0] = pack8(sacc, 0);
          dsb[0] = pack8(pacc, 0);
          stash(qb, 0, dsb[0]);
          bf16x8 ot = tr_read_pair(so + tr_off(0), so + tr_off(0) + 8 * LD);
          bf16x8 qt_ = tr_read_pair(sq + tr_off(0), sq + tr_off(0) + 8 * LD);
          __builtin_amdgcn_sched_barrier(0);
          // Half 0's products, each followed by the next operands' reads and a share of half
          // 1's gradient; then half 1's products.
#pragma unroll
          for (int i = 0; i < NDB; ++i) {
            dvacc[i] = mfma32(ot, pb[0], dvacc[i]);
            dkacc[i] = mfma32(qt_, dsb[0], dkacc[i]);
            ot = tr_read_pair(so + tr_off(i + 1), so + tr_off(i + 1) + 8 * LD);
            qt_ = tr_read_pair(sq + tr_off(i + 1), sq + tr_off(i + 1) + 8 * LD);
#pragma unroll
            for (int r = 8 + 8 * i / NDB; r < 8 + 8 * (i + 1) / NDB; ++r) grad(masked, r);
            __builtin_amdgcn_sched_barrier(0);
          }
          pb[1] = pack8(sacc, 8);
          dsb[1] = pack8(pacc, 8);
          stash(qb, 1, dsb[1]);
#pragma unroll
          for (int i = NDB; i < 2 * NDB; ++i) {
            dvacc[i - NDB] = mfma32(ot, pb[1], dvacc[i - NDB]);
            dkacc[i - NDB] = mfma32(qt_, dsb[1], dkacc[i - NDB]);
            if (i + 1 < 2 * NDB) {
              ot = tr_read_pair(so + tr_off(i + 1), so + tr_off(i + 1) + 8 * LD);
              qt_ = tr_read_pair(sq + tr_off(i + 1), sq + tr_off(i + 1) + 8 * LD);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        };
        if (need_mask)
          half(std::true_type{});
        else
          half(std::false_type{});
      } else {
        // Half t covers elements 8t .. 8t + 7 (queries 16t .. 16t + 15 of the block): the
        // softmax gradient, then that half's share of dV^T += dO^T P and dK^T += q^T dS.
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float* lrow = sl + qb * 32 + 4 * gl + 16 * t;
          const float4 lq[2] = {*reinterpret_cast<const float4*>(lrow),
                                *reinterpret_cast<const float4*>(lrow + 8)};
          float4 nq[2];  // -D of the half's queries (dropout: dP starts at 0)
          if constexpr (DROP) {
            nq[0] = *reinterpret_cast<const float4*>(sd + qb * 32 + 4 * gl + 16 * t);
            nq[1] = *reinterpret_cast<const float4*>(sd + qb * 32 + 4 * gl + 16 * t + 8);
          }
          auto grads = [&](auto masked) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int r = 8 * t + e;
              const int qo = 8 * (r >> 2) + (r & 3);
              float gf;
              float y = score_grad<MODE>(sacc[r], a.sc, lq[e >> 2][e & 3], &gf);
              if constexpr (decltype(masked)::value)
                y = visible(kd + 32 * qb + qo, lim) ? y : kNegBig;
              const float p = exp2_fast(y);
              float ds;
              if constexpr (DROP) {
                const float4 n4 = nq[e >> 2];
                const float nd =
                    (e & 3) == 0 ? n4.x : (e & 3) == 1 ? n4.y : (e & 3) == 2 ? n4.z : n4.w;
                ds = p * fmaf(keep_only(a.drop_scale, mw, r), pacc[r], nd);
                sacc[r] = keep_only(p, mw, r);  // dV takes the kept weights; scaled at the end
              } else {
                ds = p * pacc[r];
                sacc[r] = p;
              }
              if constexpr (MODE != kScoreScale) ds *= gf;
              pacc[r] = ds;
            }
          };
          if (need_mask)
            grads(std::true_type{});
          else
            grads(std::false_type{});
          const bf16x8 pb = pack8(sacc, 8 * t), dsb = pack8(pacc, 8 * t);
          stash(qb, t, dsb);
          __builtin_amdgcn_sched_barrier(0);
          bf16x8 ot[NDB], qt_[NDB];
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const int off = (qb * 32 + 16 * t + trow) * LD + 32 * db + tcol;
            ot[db] = tr_read_pair(so + off, so + off + 8 * LD);
            qt_[db] = tr_read_pair(sq + off, sq + off + 8 * LD);
          }
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            dvacc[db] = mfma32(ot[db], pb, dvacc[db]);
            dkacc[db] = mfma32(qt_[db], dsb, dkacc[db]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };

  // The same q tile in quarters (block qb, half t) at two waves per SIMD and d = 96 (at
  // d <= 64 the steps are too short for it to pay; measured slower), where registers hold
  // only one block's scores plus a half block: block 0's S / dP products; block 0's first
  // half gradient and its dV / dK products; block 1's S / dP products beside block 0's second
  // half gradient; block 0's second-half products beside block 1's first-half gradient;
  // block 1's first-half products beside its second-half gradient; block 1's second-half
  // products.
  auto step_quarters = [&](int it, const bf16* sq, const bf16* so, const float* sl,
                           const float* sd, const uint32_t* sm) __attribute__((always_inline)) {
    const int hh = it / nq;
    const int q0 = q_tile(it, hh);
    const int q_last = min(q0 + kBMt - 1, T - 1);
    const bool skip = !wave_active || q_last < kw0 || q0 > e_hi ||
                      (window > 0 && q0 > kw_last + window - 1);
    if (skip) return;
    const bool need_mask = (q0 < kw_last) || (q0 + kBMt > T) || q_last > e_lo ||
                           (window > 0 && q_last - kw0 >= window);
    // iq - kj for element (qb, r) is kd + 32 qb + 8 (r / 4) + r % 4.
    const int kd = q0 + 4 * gl - kj;
    auto body = [&](auto masked) {
      f32x16 sacc[2], pacc[2];
      uint32_t mw[2] = {0u, 0u};
      auto pick = [](const float4& v, int c) {
        return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
      };
      // S accumulates from 0; dP from -D (dropout: from 0, -D joins in the gradient).
      auto setup = [&](int qb) {
        if constexpr (DROP) mw[qb] = sm[qb * kBNkv + kj - kwg0] >> (4 * gl);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 nd = *reinterpret_cast<const float4*>(sd + qb * 32 + 4 * gl + 8 * j);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            sacc[qb][4 * j + c] = 0.f;
            pacc[qb][4 * j + c] = DROP ? 0.f : pick(nd, c);
          }
        }
      };
      // Gradient of element r of block qb: P (dV operand) into sacc, dS into pacc.
      // LSE log2(e) of half h of block qb (elements 8h .. 8h + 7: two runs of four rows), read
      // as two 16-byte loads ahead of the gradients that use them.
      auto lse_half = [&](int qb, int h, float4 (&lv)[2]) {
        lv[0] = *reinterpret_cast<const float4*>(sl + qb * 32 + 4 * gl + 16 * h);
        lv[1] = *reinterpret_cast<const float4*>(sl + qb * 32 + 4 * gl + 16 * h + 8);
      };
      auto grad = [&](int qb, int r, const float4 (&lv)[2]) {
        const int qo = 8 * (r >> 2) + (r & 3);
        const float lse = pick(lv[(r >> 2) & 1], r & 3);
        float gf;
        float y = score_grad<MODE>(sacc[qb][r], a.sc, lse, &gf);
        if constexpr (decltype(masked)::value)
          y = visible(kd + 32 * qb + qo, lim) ? y : kNegBig;
        const float p = exp2_fast(y);
        float ds;
        if constexpr (DROP) {
          const float nd = sd[qb * 32 + 4 * gl + 8 * (r >> 2) + (r & 3)];
          ds = p * fmaf(keep_only(a.drop_scale, mw[qb], r), pacc[qb][r], nd);
          sacc[qb][r] = keep_only(p, mw[qb], r);  // dV takes the kept weights; scaled at the end
        } else {
          ds = p * pacc[qb][r];
          sacc[qb][r] = p;
        }
        if constexpr (MODE != kScoreScale) ds *= gf;
        pacc[qb][r] = ds;
        asm volatile("" : "+v"(sacc[qb][r]), "+v"(pacc[qb][r]));
      };
      auto qk_off = [&](int qb, int s) { return (qb * 32 + lr) * LD + 16 * s + 8 * gl; };
      auto tr_off = [&](int qb, int t, int db) {
        return (qb * 32 + 16 * t + trow) * LD + 32 * db + tcol;
      };
      bf16x8 pb[2][2], dsb[2][2];
      auto pack = [&](int qb, int t) {
        pb[qb][t] = pack8(sacc[qb], 8 * t);
        dsb[qb][t] = pack8(pacc[qb], 8 * t);
        stash(qb, t, dsb[qb][t]);
      };
      // dV / dK products of quarter (qb, t), step db carrying gradient elements
      // [g0 + 8 db / NDB, g0 + 8 (db + 1) / NDB) of block gq (none when gq < 0).
      auto quarter = [&](int qb, int t, int gq, int g0) {
        float4 lv[2];
        if (gq >= 0) lse_half(gq, g0 / 8, lv);
        bf16x8 ot = tr_read_pair(so + tr_off(qb, t, 0), so + tr_off(qb, t, 0) + 8 * LD);
        bf16x8 qt_ = tr_read_pair(sq + tr_off(qb, t, 0), sq + tr_off(qb, t, 0) + 8 * LD);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          dvacc[db] = mfma32(ot, pb[qb][t], dvacc[db]);
          dkacc[db] = mfma32(qt_, dsb[qb][t], dkacc[db]);
          if (db + 1 < NDB) {
            ot = tr_read_pair(so + tr_off(qb, t, db + 1), so + tr_off(qb, t, db + 1) + 8 * LD);
            qt_ = tr_read_pair(sq + tr_off(qb, t, db + 1), sq + tr_off(qb, t, db + 1) + 8 * LD);
          }
          if (gq >= 0) {
#pragma unroll
            for (int r = g0 + 8 * db / NDB; r < g0 + 8 * (db + 1) / NDB; ++r) grad(gq, r, lv);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      // Block 0's products, scheduled by the compiler.
      setup(0);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 qa = ld16<bf16x8>(sq + qk_off(0, s));
        const bf16x8 oa = ld16<bf16x8>(so + qk_off(0, s));
        sacc[0] = mfma32(qa, bk[s], sacc[0]);
        pacc[0] = mfma32(oa, bv[s], pacc[0]);
      }
      __builtin_amdgcn_sched_barrier(0);
      {
        float4 lv[2];
        lse_half(0, 0, lv);
#pragma unroll
        for (int r = 0; r < 8; ++r) grad(0, r, lv);
      }
      pack(0, 0);
      quarter(0, 0, -1, 0);
      // Block 1's products beside block 0's second-half gradient.
      setup(1);
      bf16x8 qa = ld16<bf16x8>(sq + qk_off(1, 0));
      bf16x8 oa = ld16<bf16x8>(so + qk_off(1, 0));
      float4 lv1[2];
      lse_half(0, 1, lv1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        sacc[1] = mfma32(qa, bk[s], sacc[1]);
        pacc[1] = mfma32(oa, bv[s], pacc[1]);
        if (s + 1 < NS) {
          qa = ld16<bf16x8>(sq + qk_off(1, s + 1));
          oa = ld16<bf16x8>(so + qk_off(1, s + 1));
        }
#pragma unroll
        for (int r = 8 + 8 * s / NS; r < 8 + 8 * (s + 1) / NS; ++r) grad(0, r, lv1);
        __builtin_amdgcn_sched_barrier(0);
      }
      pack(0, 1);
      quarter(0, 1, 1, 0);
      pack(1, 0);
      quarter(1, 0, 1, 8);
      pack(1, 1);
      quarter(1, 1, -1, 0);
    };
    if (need_mask)
      body(std::true_type{});
    else
      body(std::false_type{});
  };

  // The same q tile with the two query blocks overlapped, for one wave per SIMD (the wave
  // has no partner to fill its idle units, and 512 registers hold both blocks' scores):
  // block 0's S / dP products; block 1's products beside block 0's gradient; block 0's dV /
  // dK products beside block 1's gradient; block 1's dV / dK products.  Steps are fenced by
  // scheduling barriers, the gradient pinned to its step, LDS operands read two steps ahead.
  auto step_full = [&](int it, const bf16* sq, const bf16* so, const float* sl,
                       const float* sd, const uint32_t* sm) __attribute__((always_inline)) {
    const int hh = it / nq;
    const int q0 = q_tile(it, hh);
    const int q_last = min(q0 + kBMt - 1, T - 1);
    const bool skip = !wave_active || q_last < kw0 || q0 > e_hi ||
                      (window > 0 && q0 > kw_last + window - 1);
    if (skip) return;
    const bool need_mask = (q0 < kw_last) || (q0 + kBMt > T) || q_last > e_lo ||
                           (window > 0 && q_last - kw0 >= window);
    // iq - kj for element (qb, r) is kd + 32 qb + 8 (r / 4) + r % 4.
    const int kd = q0 + 4 * gl - kj;
    auto body = [&](auto masked) {
      f32x16 sacc[2], pacc[2];
      uint32_t mw[2] = {0u, 0u};
      // Per block and element group j = r / 4: LSE and -D of queries 8 j + 4 gl .. + 3.
      float4 lq[2][4], nq4[2][4];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lq[qb][j] = *reinterpret_cast<const float4*>(sl + qb * 32 + 4 * gl + 8 * j);
          nq4[qb][j] = *reinterpret_cast<const float4*>(sd + qb * 32 + 4 * gl + 8 * j);
        }
        if constexpr (DROP) mw[qb] = sm[qb * kBNkv + kj - kwg0] >> (4 * gl);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[qb][r] = 0.f;  // zero accumulators need no vector instructions before the MFMA
          pacc[qb][r] = 0.f;
        }
      }
      auto pick = [](const float4& v, int c) {
        return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
      };
      // Gradient of element r of block qb: P (dV operand) into sacc, dS into pacc.
      auto grad = [&](int qb, int r) {
        const int qo = 8 * (r >> 2) + (r & 3);
        float gf;
        float y = score_grad<MODE>(sacc[qb][r], a.sc, pick(lq[qb][r >> 2], r & 3), &gf);
        if constexpr (decltype(masked)::value)
          y = visible(kd + 32 * qb + qo, lim) ? y : kNegBig;
        const float p = exp2_fast(y);
        const float nd = pick(nq4[qb][r >> 2], r & 3);
        float ds;
        if constexpr (DROP) {
          ds = p * fmaf(keep_only(a.drop_scale, mw[qb], r), pacc[qb][r], nd);
          sacc[qb][r] = keep_only(p, mw[qb], r);  // dV takes the kept weights; scaled at the end
        } else {
          ds = p * (pacc[qb][r] + nd);
          sacc[qb][r] = p;
        }
        if constexpr (MODE != kScoreScale) ds *= gf;
        pacc[qb][r] = ds;
        asm volatile("" : "+v"(sacc[qb][r]), "+v"(pacc[qb][r]));
      };
      auto qk_off = [&](int qb, int s) { return (qb * 32 + lr) * LD + 16 * s + 8 * gl; };
      auto tr_off = [&](int qb, int i) {  // product step i = NDB t + db
        return (qb * 32 + 16 * (i / NDB) + trow) * LD + 32 * (i % NDB) + tcol;
      };
      // S / dP products of both blocks as one stream of 2 NS steps (step j: block j / NS,
      // slice j % NS); block 1's steps each carry a share of block 0's gradient.
      bf16x8 qa[2], oa[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        qa[j] = ld16<bf16x8>(sq + qk_off(j / NS, j % NS));
        oa[j] = ld16<bf16x8>(so + qk_off(j / NS, j % NS));
      }
#pragma unroll
      for (int j = 0; j < 2 * NS; ++j) {
        const int qb = j / NS, s = j % NS;
        sacc[qb] = mfma32(qa[j & 1], bk[s], sacc[qb]);
        pacc[qb] = mfma32(oa[j & 1], bv[s], pacc[qb]);
        if (j + 2 < 2 * NS) {
          qa[j & 1] = ld16<bf16x8>(sq + qk_off((j + 2) / NS, (j + 2) % NS));
          oa[j & 1] = ld16<bf16x8>(so + qk_off((j + 2) / NS, (j + 2) % NS));
        }
        if (qb == 1) {
#pragma unroll
          for (int r = 16 * s / NS; r < 16 * (s + 1) / NS; ++r) grad(0, r);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // dV^T += dO^T P and dK^T += q^T dS of both blocks as one stream of 4 NDB steps (step
      // i: block i / (2 NDB), product i % (2 NDB)); block 0's steps carry block 1's gradient.
      bf16x8 pb[2][2], dsb[2][2];
      pb[0][0] = pack8(sacc[0], 0);
      pb[0][1] = pack8(sacc[0], 8);
      dsb[0][0] = pack8(pacc[0], 0);
      dsb[0][1] = pack8(pacc[0], 8);
      stash(0, 0, dsb[0][0]);
      stash(0, 1, dsb[0][1]);
      bf16x8 ot[2], qt_[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        ot[i] = tr_read_pair(so + tr_off(0, i), so + tr_off(0, i) + 8 * LD);
        qt_[i] = tr_read_pair(sq + tr_off(0, i), sq + tr_off(0, i) + 8 * LD);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4 * NDB; ++i) {
        const int qb = i / (2 * NDB), k = i % (2 * NDB), db = k % NDB, t = k / NDB;
        if (i == 2 * NDB) {
          pb[1][0] = pack8(sacc[1], 0);
          pb[1][1] = pack8(sacc[1], 8);
          dsb[1][0] = pack8(pacc[1], 0);
          dsb[1][1] = pack8(pacc[1], 8);
          stash(1, 0, dsb[1][0]);
          stash(1, 1, dsb[1][1]);
        }
        dvacc[db] = mfma32(ot[i & 1], pb[qb][t], dvacc[db]);
        dkacc[db] = mfma32(qt_[i & 1], dsb[qb][t], dkacc[db]);
        if (i + 2 < 4 * NDB) {
          const int o = tr_off((i + 2) / (2 * NDB), (i + 2) % (2 * NDB));
          ot[i & 1] = tr_read_pair(so + o, so + o + 8 * LD);
          qt_[i & 1] = tr_read_pair(sq + o, sq + o + 8 * LD);
        }
        if (qb == 0) {
#pragma unroll
          for (int r = 16 * k / (2 * NDB); r < 16 * (k + 1) / (2 * NDB); ++r) grad(1, r);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (need_mask)
      body(std::true_type{});
    else
      body(std::false_type{});
  };

  auto step = [&](int it, const bf16* sq, const bf16* so, const float* sl, const float* sd,
                  const uint32_t* sm) __attribute__((always_inline)) {
    if constexpr (D >= 128 || (DROP && D >= 96))
      step_full(it, sq, so, sl, sd, sm);
    else if constexpr (D == 96 && MODE != kScoreCapExp)
      step_quarters(it, sq, so, sl, sd, sm);
    else
      step_split(it, sq, so, sl, sd, sm);
  };

  // The fragments of iteration it's dS, stored after the barrier that ends the iteration: the
  // wait before that barrier counts stores too, so stores issued inside the step would hold it
  // for a write round trip; issued here they overlap the next iteration's work.  A wave whose
  // step skipped the tile has nothing to store.
  auto export_after = [&](int it) __attribute__((always_inline)) {
    const int hh = it / nq;
    const int q0 = q_tile(it, hh);
    const int q_last = min(q0 + kBMt - 1, T - 1);
    const bool skip = !wave_active || q_last < kw0 || q0 > e_hi ||
                      (window > 0 && q0 > kw_last + window - 1);
    if constexpr (EXPORT)
      if (!skip) export_ds(hh, q0);
  };

  // Two-deep pipeline over the (query head, query tile) iterations, unrolled by two so each
  // LDS buffer is a distinct array: the loads into one buffer never wait on reads of the other.
  dma(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int it = 0; it < nit; it += 2) {
    if (it + 1 < nit) dma(it + 1, 1);
    step(it, sQ0, sO0, sL[0], sD[0], sM0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    export_after(it);
    if (it + 1 >= nit) break;
    if (it + 2 < nit) dma(it + 2, 0);
    step(it + 1, sQ1, sO1, sL[1], sD[1], sM1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    export_after(it + 1);
  }

  finish_grad_row<D>(dkacc, a.scale, a.k + krowoff, a.dk + krowoff, krow, gl, a.pro != 0, a.rp,
                     kj < T);
  if (kj < T) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float v4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v4[j] = dvacc[db][4 * i4 + j] * (DROP ? a.drop_scale : 1.f);
        store4(a.dv + krowoff + 32 * db + 8 * i4 + 4 * gl, v4);
      }
  }
}

// ------------------------------------------------------------------------------------------
// dQ from exported dS (split backward)
// ------------------------------------------------------------------------------------------
// One workgroup per (b, h, 128 queries), 4 waves x 32 queries, the dq pass's grid order.  Per
// 64-key tile: k^ staged in LDS (double buffered), the wave's four dS fragments (16 keys each)
// loaded straight into MFMA B operands, and dQ^T += K^T dS^T with K^T read transposed from
// LDS.  The fragments of the next tile are in flight while the current one multiplies.  No
// score, exponential or dP is recomputed; the epilogue is the dq pass's (scale, RMSNorm and
// RoPE backward).
template <int D>
__global__ __launch_bounds__(256, D <= 96 ? 4 : 3) void bwd_dq_ds_kernel(BwdArgs a) {
  constexpr int LD = D + 8;
  constexpr int NDB = D / 32;
  constexpr int TILE = kBNk * LD;
  __shared__ __attribute__((aligned(16))) bf16 sK0[TILE];
  __shared__ __attribute__((aligned(16))) bf16 sK1[TILE];

  const int T = a.T;
  const int nbh = a.B * a.Hq;
  const int rank = blockIdx.x / nbh;
  const int bh = xcd_local_head(blockIdx.x - rank * nbh, nbh);
  const int qt = a.ntiles - 1 - rank;
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const int tid = threadIdx.x, l = tid & 63, gl = l >> 5, lr = l & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q0 = qt * kBMq, qw0 = q0 + 32 * w;
  const int qi = qw0 + lr;
  const int qrow = min(qi, T - 1);
  const bf16* kbase = a.kh + (int64_t)(b * a.Hkv + g) * T * D;
  const int64_t rowoff = ((int64_t)bh * T + qrow) * D;
  const bool wave_active = qw0 < T;
  // This wave's 32-query block and its key blocks.
  const int iq = qw0 >> 5;
  const int jlo = ds_lo(iq, a.band), jhi = ds_hi(iq, a.band);
  const bf16* dsh = a.ds + ((int64_t)bh * a.band.frags) * 512 + 8 * l;

  const int window = a.window;
  const int k_end = min(T, q0 + kBMq);
  const int k_begin = window > 0 ? max(0, q0 - window + 1) : 0;
  const int kt0 = k_begin / kBNk, kt1 = (k_end - 1) / kBNk;

  const TileDma<D, 4> tdma(w, l);
  // Fragment f of tile kt (key block 4 kt + f), or zeros outside this wave's band.
  auto frag_in = [&](int kt, int f) {
    const int j = 4 * kt + f;
    return wave_active && j >= jlo && j <= jhi;
  };
  auto load_frags = [&](bf16x8 (&fr)[4], int kt) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      if (frag_in(kt, f))
        fr[f] = __builtin_nontemporal_load(
            reinterpret_cast<const bf16x8*>(dsh + ds_frag(iq, 4 * kt + f, a.band) * 512));
    }
  };

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[db][r] = 0.f;

  // K^T operand of key block f, head-dim block db: lane (group gq, L) loads key row
  // 16 f + 8 (gq / 2) + L / 4 (+ 4) at columns 32 db + 16 (gq % 2) + 4 (L % 4).
  const int gq = l >> 4, L = l & 15;
  const int aoff = (8 * (gq >> 1) + (L >> 2)) * LD + 16 * (gq & 1) + 4 * (L & 3);
  auto run = [&](int kt, const bf16* sk, const bf16x8 (&fr)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      if (!frag_in(kt, f)) continue;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16* p0 = sk + 16 * f * LD + 32 * db + aoff;
        dqacc[db] = mfma32(tr_read_pair(p0, p0 + 4 * LD), fr[f], dqacc[db]);
      }
    }
  };

  bf16x8 fr0[4], fr1[4];
  tdma.copy(sK0, kbase, kt0 * kBNk, T, w);
  load_frags(fr0, kt0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kt = kt0; kt <= kt1; kt += 2) {
    if (kt + 1 <= kt1) {
      tdma.copy(sK1, kbase, (kt + 1) * kBNk, T, w);
      load_frags(fr1, kt + 1);
    }
    run(kt, sK0, fr0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 1 > kt1) break;
    if (kt + 2 <= kt1) {
      tdma.copy(sK0, kbase, (kt + 2) * kBNk, T, w);
      load_frags(fr0, kt + 2);
    }
    run(kt + 1, sK1, fr1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  finish_grad_row<D>(dqacc, a.scale, a.q + rowoff, a.dq + rowoff, qrow, gl, a.pro != 0, a.rp,
                     qi < T);
}

BwdArgs make_args(const BwdParams& p, int D) {
  BwdArgs a;
  a.q = (const bf16*)p.q;
  a.k = (const bf16*)p.k;
  a.kh = (const bf16*)p.kh;
  a.qh = (bf16*)p.qh;
  a.v = (const bf16*)p.v;
  a.o = (const bf16*)p.o;
  a.dO = (const bf16*)p.dO;
  a.lse = p.lse;
  a.Dvec = p.Dvec;
  a.L2 = p.L2;
  a.seg_start = p.seg_start;
  a.seg_end = p.seg_end;
  a.drop_rows = p.drop_rows;
  a.drop_cols = p.drop_cols;
  a.drop_pitch = dropout_pitch(p.T);
  a.drop_scale = p.drop_scale;
  a.dq = (bf16*)p.dq;
  a.dk = (bf16*)p.dk;
  a.dv = (bf16*)p.dv;
  a.B = p.B;
  a.T = p.T;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.window = p.window;
  a.ntiles = 0;
  a.pro = (p.rope || p.qk_norm) ? 1 : 0;
  a.scale = p.scale;
  a.sc = make_score_setup(p.scale, p.softcap, D, p.qk_norm).coef;
  a.rp = make_row_prologue(p.rope, p.rope_base, p.qk_norm, p.eps, D);
  a.ds = (bf16*)p.ds;
  a.band = p.band;
  return a;
}

template <int D>
hipError_t launch_dq_ds_d(const BwdParams& p, hipStream_t s) {
  BwdArgs a = make_args(p, D);
  a.ntiles = (p.T + kBMq - 1) / kBMq;
  const dim3 grid((unsigned)(a.ntiles * p.B * p.Hq));
  static const char* names[4] = {"bwd_dq_ds_d32", "bwd_dq_ds_d64", "bwd_dq_ds_d96",
                                 "bwd_dq_ds_d128"};
  TraceScope t(names[D / 32 - 1], s);
  hipLaunchKernelGGL((bwd_dq_ds_kernel<D>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dq_d(const BwdParams& p, hipStream_t s) {
  BwdArgs a = make_args(p, D);
  a.ntiles = (p.T + kBMq - 1) / kBMq;
  const int mode = make_score_setup(p.scale, p.softcap, D, p.qk_norm).mode;
  const dim3 grid((unsigned)(a.ntiles * p.B * p.Hq));
  static const char* names[4] = {"bwd_dq_d32", "bwd_dq_d64", "bwd_dq_d96", "bwd_dq_d128"};
  TraceScope t(names[D / 32 - 1], s);
  if (a.drop_rows) {
    if (mode == kScoreScale)
      hipLaunchKernelGGL((bwd_dq_kernel<D, kScoreScale, true>), grid, dim3(256), 0, s, a);
    else if (mode == kScoreCapPoly5)
      hipLaunchKernelGGL((bwd_dq_kernel<D, kScoreCapPoly5, true>), grid, dim3(256), 0, s, a);
    else if (mode == kScoreCapPoly)
      hipLaunchKernelGGL((bwd_dq_kernel<D, kScoreCapPoly, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, kScoreCapExp, true>), grid, dim3(256), 0, s, a);
  } else {
    if (mode == kScoreScale)
      hipLaunchKernelGGL((bwd_dq_kernel<D, kScoreScale, false>), grid, dim3(256), 0, s, a);
    else if (mode == kScoreCapPoly5)
      hipLaunchKernelGGL((bwd_dq_kernel<D, kScoreCapPoly5, false>), grid, dim3(256), 0, s, a);
    else if (mode == kScoreCapPoly)
      hipLaunchKernelGGL((bwd_dq_kernel<D, kScoreCapPoly, false>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, kScoreCapExp, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <int D, bool DROP, bool EXPORT>
void launch_dkdv_mode(const BwdArgs& a, int mode, dim3 grid, hipStream_t s) {
  if (mode == kScoreScale)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, kScoreScale, DROP, EXPORT>), grid, dim3(256), 0, s, a);
  else if (mode == kScoreCapPoly5)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, kScoreCapPoly5, DROP, EXPORT>), grid, dim3(256), 0, s, a);
  else if (mode == kScoreCapPoly)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, kScoreCapPoly, DROP, EXPORT>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, kScoreCapExp, DROP, EXPORT>), grid, dim3(256), 0, s, a);
}

template <int D>
hipError_t launch_dkdv_d(const BwdParams& p, hipStream_t s) {
  BwdArgs a = make_args(p, D);
  a.ntiles = (p.T + kBNkv - 1) / kBNkv;
  const int mode = make_score_setup(p.scale, p.softcap, D, p.qk_norm).mode;
  const dim3 grid((unsigned)(a.ntiles * p.B * p.Hkv));
  static const char* names[4] = {"bwd_dkdv_d32", "bwd_dkdv_d64", "bwd_dkdv_d96", "bwd_dkdv_d128"};
  static const char* xnames[4] = {"bwd_dkdv_export_d32", "bwd_dkdv_export_d64",
                                  "bwd_dkdv_export_d96", "bwd_dkdv_export_d128"};
  TraceScope t((a.ds ? xnames : names)[D / 32 - 1], s);
  if (a.drop_cols)
    launch_dkdv_mode<D, true, false>(a, mode, grid, s);
  else if (a.ds)
    launch_dkdv_mode<D, false, true>(a, mode, grid, s);
  else
    launch_dkdv_mode<D, false, false>(a, mode, grid, s);
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

hipError_t launch_bwd_dq_ds(const BwdParams& p, hipStream_t s) {
  switch (p.D) {
    case 32: return launch_dq_ds_d<32>(p, s);
    case 64: return launch_dq_ds_d<64>(p, s);
    case 96: return launch_dq_ds_d<96>(p, s);
    case 128: return launch_dq_ds_d<128>(p, s);
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
