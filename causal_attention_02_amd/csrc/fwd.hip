// Causal attention forward on gfx950.
//
// Definition ("GPT pretraining" page, section "Multihead Attention"):
//   O = softmax(S) V with S = scale * Q K^T, future positions set to -inf before the
//   softmax; optional soft-cap S <- c tanh(S / c) and sliding window (flaxchat page,
//   "Core Features"; nanoGPT-JAX 181M model card, "Architecture").
// The result is reached exactly (up to rounding) by the flash formulation: key tiles are
// visited once, a running row maximum m and row sum l rescale the partial output, and
// LSE = m + ln(l) is kept for the backward.
//
// bf16 kernel layout (one workgroup = (b, h, 128 queries), 4 waves x 32 queries):
//   * Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 so that a lane holds 16
//     scores of ONE query (lane % 32) per 32-key block: the row max / sum is a per-lane
//     reduction plus one permlane32 swap with the partner lane l ^ 32.
//   * Q stays in registers as the MFMA B operand for the whole kernel.
//   * K and V tiles (64 keys) are staged row-major in LDS, double buffered.  K feeds the
//     A operand directly; V^T is read with ds_read_b64_tr_b16, and P goes from the score
//     accumulators straight into the B operand of O^T += V^T P^T (no LDS round trip).
//   * Key tiles wholly above the diagonal or outside the window are never visited; only
//     tiles that straddle a mask edge evaluate the element mask.
//   * Within a tile (two 32-key blocks) each wave issues one block's MFMAs beside the other
//     block's weight arithmetic, so its matrix and vector units work at once.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

struct FwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;                // may be null (extend: no LSE output)
  const int32_t* cache_len;  // extend: rows already cached per sequence (null in training)
  const int32_t* cache_start;  // extend, left-padded batches: padding rows per sequence (or null)
  const int32_t* seg_start;  // packed rows: first index of each token's run, [B, T] (or null)
  const uint32_t* drop_rows; // dropout: row-layout keep mask [B, Hq, T, drop_pitch] (or null)
  int drop_pitch;
  float drop_scale;          // kept-weight scale 1 / (1 - rate)
  int B, T, Hq, Hkv, window, nqt;
  int Tk;                    // rows per head of k/v (T in training, Lmax for a cache)
  float shift;  // fixed softmax shift (log2 units) when the score bound allows one
  ScoreCoef sc;
  RowPrologue rp;
};

constexpr int kBM = 128;  // queries per workgroup
constexpr int kBN = 64;   // keys per tile

// O^T[d][q] += V^T[d][key] P^T[key][q] for one 32-key block of the LDS tile; lane L of each
// 16-lane group reads 4 values of key row (16 t + L / 4) at columns 4 (L % 4) of its half.
template <int D>
__device__ __forceinline__ void pv_block(f32x16 (&oacc)[D / 32], const bf16* sv, int kb,
                                         const bf16x8 (&pb)[2], int trow, int tcol) {
  constexpr int LD = D + 8;
  constexpr int NDB = D / 32;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    bf16x8 va[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const bf16* p0 = sv + (kb * 32 + 16 * t + trow) * LD + 32 * db + tcol;
      va[db] = tr_read_pair(p0, p0 + 8 * LD);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(va[db], pb[t], oacc[db]);
  }
}

// Largest factor (log2) a row's running maximum may grow by before the accumulators are
// rescaled (running-maximum forward only).
constexpr float kRescaleSlack = 8.f;

// Kernel variants: plain rows; packed rows (segment ids); dropout on the weights.
constexpr int kVarPlain = 0, kVarPacked = 1, kVarDrop = 2;

// MODE: score transform (kScore*); FIXED: fixed shift instead of a running maximum.
// Three waves per SIMD for D <= 96 (registers and 52 KB of LDS per workgroup fit), else two.
// VAR: kVarPacked -- rows carry several runs (segment ids); a compile-time switch so the plain
// kernels keep the window limit in a scalar register.  kVarDrop -- dropout: the keep words of
// each key tile are staged in LDS with the tile, the PV product takes the kept weights, the
// row sum all of them, and the output is scaled by 1 / (1 - rate).  Both run two waves per SIMD.
template <int D, int MODE, bool FIXED, int VAR>
__global__ __launch_bounds__(256, (D <= 96 && VAR == kVarPlain) ? 3 : 2) void fwd_bf16_kernel(FwdArgs a) {
  constexpr bool PACKED = VAR == kVarPacked;
  constexpr bool DROP = VAR == kVarDrop;
  constexpr int LD = D + 8;          // LDS row pitch (elements)
  constexpr int NS = D / 16;         // MFMA k-steps over the head dimension
  constexpr int NDB = D / 32;        // 32-wide blocks of the head dimension
  constexpr int TILE = kBN * LD;
  static_assert(kBN == 64 && TILE % 512 == 0, "tiles are 64 padded rows, whole 1 KB chunks");
  __shared__ __attribute__((aligned(16))) bf16 sK0[TILE];
  __shared__ __attribute__((aligned(16))) bf16 sK1[TILE];
  __shared__ __attribute__((aligned(16))) bf16 sV0[TILE];
  __shared__ __attribute__((aligned(16))) bf16 sV1[TILE];
  // Dropout keep words of the tile's two 32-key blocks for the workgroup's 128 queries:
  // [block][query].
  __shared__ __attribute__((aligned(16))) uint32_t sM0[DROP ? 2 * kBM : 1];
  __shared__ __attribute__((aligned(16))) uint32_t sM1[DROP ? 2 * kBM : 1];

  const int T = a.T;  // query rows per head
  const int nbh = a.B * a.Hq;
  const int rank = blockIdx.x / nbh;  // heaviest (last) query tiles first
  const int bh = xcd_local_head(blockIdx.x - rank * nbh, nbh);
  const int qt = a.nqt - 1 - rank;
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  const int g = h / (a.Hq / a.Hkv);

  const int tid = threadIdx.x, l = tid & 63, gl = l >> 5, lr = l & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int q0 = qt * kBM, qw0 = q0 + 32 * w;
  const int qi = qw0 + lr;
  // Extend (a KV cache): query i sits at position off + i and the cache holds off + nq keys
  // after the append; queries that did not fit (off + i >= Lmax) get zero rows.  Training:
  // off = 0 and nq = nk = T.
  const int Tk = a.Tk;
  const int off = a.cache_len ? min(max(a.cache_len[b], 0), Tk) : 0;
  const int nq = min(T, Tk - off);
  const int nk = off + nq;
  if (q0 >= nq) {
    for (int t = tid; t < kBM * D; t += 256) {
      const int r = q0 + t / D;
      if (r < T) a.o[((int64_t)bh * T + r) * D + t % D] = to_bf16(0.f);
    }
    return;
  }
  const int qrow = min(qi, nq - 1);
  const int window = a.window;
  const unsigned wlim = window > 0 ? (unsigned)window : 0x7fffffffu;
  // Packed rows: this lane's query sees keys back to the start of its run only.  A left-padded
  // cache (extend) takes the same path with one run per sequence, from row cache_start[b]:
  // positions count from there, and queries in padding rows get zero rows.
  const int S0 = PACKED && a.cache_start ? min(max(a.cache_start[b], 0), Tk) : 0;
  const int32_t* sst = PACKED && !a.cache_start ? a.seg_start + (int64_t)b * T : nullptr;
  auto run_start = [&](int x) { return sst ? sst[x] : S0; };
  const unsigned lim =
      PACKED ? min(wlim, (unsigned)max(off + qrow - run_start(qrow) + 1, 0)) : wlim;

  const bf16* kbase = a.k + (int64_t)(b * a.Hkv + g) * Tk * D;
  const bf16* vbase = a.v + (int64_t)(b * a.Hkv + g) * Tk * D;

  // Q operand: lane holds q^[qi][16 s + 8 gl .. +7]; RoPE and RMSNorm are applied here.
  bf16x8 bq[NS];
  {
    const bf16* qp = a.q + ((int64_t)bh * T + qrow) * D + 8 * gl;
#pragma unroll
    for (int s = 0; s < NS; ++s) bq[s] = ld16<bf16x8>(qp + 16 * s);
    if (a.rp.rope | a.rp.qk_norm) {
      float x[NS][8];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int p = 0; p < 8; ++p) x[s][p] = (float)bq[s][p];
      prologue_oplayout<NS>(x, off + qrow - S0, gl, a.rp, D);
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int p = 0; p < 8; ++p) bq[s][p] = to_bf16(x[s][p]);
    }
  }

  const int k_end = min(nk, off + q0 + kBM);
  const int k_begin =
      max(window > 0 ? max(0, off + q0 - window + 1) : 0, PACKED ? run_start(q0) : 0);
  const int kt0 = k_begin / kBN, kt1 = (k_end - 1) / kBN;

  // Tile loads: rows past T read clamped, finite data whose scores the causal mask removes
  // (such keys lie after every query).
  const TileDma16<D, 4> tdma(w, l);
  auto dma = [&](int kt, int buf) {
    tdma.copy(buf ? sK1 : sK0, kbase, kt * kBN, nk, w, PACKED ? S0 : 0);
    tdma.copy(buf ? sV1 : sV0, vbase, kt * kBN, nk, w, PACKED ? S0 : 0);
    if constexpr (DROP) {
      // Wave w: keep word of block (w & 1) for queries q0 + 64 (w >> 1) + lane.
      const int row = min(q0 + 64 * (w >> 1) + l, T - 1);
      __builtin_amdgcn_global_load_lds(
          a.drop_rows + ((int64_t)bh * T + row) * a.drop_pitch + 2 * kt + (w & 1),
          (buf ? sM1 : sM0) + (w & 1) * kBM + 64 * (w >> 1), 4, 0, 0);
    }
  };

  float m_run = FIXED ? a.shift : kNegBig, l_run = 0.f;
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;

  // Positions of the wave's first and last existing query.
  const bool wave_active = qw0 < nq;
  const int pw0 = off + qw0, pw_last = off + min(qw0 + 31, nq - 1);
  // Earliest and latest run start among the wave's queries (packed rows; run starts grow
  // with the token index).
  const int s_lo = PACKED ? run_start(min(qw0, nq - 1)) : 0;
  const int s_hi = PACKED ? run_start(min(qw0 + 31, nq - 1)) : 0;
  const int trow = 4 * gl + ((l & 15) >> 2);
  const int tcol = 16 * ((l >> 4) & 1) + 4 * (l & 3);

  // One key tile against this wave's 32 queries, operands in (sk, sv), keep words in sm.
  auto run = [&](int kt, const bf16* sk, const bf16* sv, const uint32_t* sm) {
    const int k0 = kt * kBN;
    const bool skip = !wave_active || k0 > pw_last || k0 + kBN - 1 < s_lo ||
                      (window > 0 && k0 + kBN - 1 < pw0 - window + 1);
    if (!skip) {
      uint32_t mw[2] = {0u, 0u};
      if constexpr (DROP) {
        mw[0] = sm[qi - q0] >> (4 * gl);
        mw[1] = sm[kBM + qi - q0] >> (4 * gl);
      }
      const bool need_mask = (k0 + kBN - 1 > pw0) || k0 < s_hi ||
                             (window > 0 && k0 < pw_last - window + 1);
      // position - key for element (kb, r) is qd - (32 kb + 8 (r / 4) + r % 4).
      const int qd = off + qi - k0 - 4 * gl;
      if constexpr (FIXED) {
        // One straight-line body per mask variant, software-pipelined over the two 32-key
        // blocks in steps fenced by scheduling barriers: block 1's score MFMAs each followed
        // by a share of block 0's weights, then block 0's PV MFMAs each followed by a share
        // of block 1's weights.  LDS operands are read two steps ahead of their MFMA.
        // One body for masked and unmasked tiles: an edge tile's invisible scores are replaced
        // in place by kNegBig right after their MFMAs (a uniform branch around the selects),
        // which the score transforms of this path send to -inf.  Two separate bodies would
        // join with the output accumulators in different registers, and the copies that
        // reconcile them cost more than the selects.
        auto body = [&]() {
          // Steps an LDS operand read runs ahead of its MFMA (V: one at three waves per SIMD).
          constexpr int KPF = 2, VPF = (D <= 96 && VAR == kVarPlain) ? 1 : 2;
          // Three waves per SIMD leave no register to spare: there the fences hold only the
          // MFMA and memory instructions and let scalar and vector work cross (the weights are
          // still held to their step by the asm pins), which lets the allocator fit.
          constexpr int kFence = (D <= 96 && VAR == kVarPlain) ? 0x6 : 0;
          f32x16 sacc[2];
          auto mask_block = [&](int kb) {
            if (need_mask) {
#pragma unroll
              for (int r = 0; r < 16; ++r)
                sacc[kb][r] = visible(qd - (32 * kb + 8 * (r >> 2) + (r & 3)), lim) ? sacc[kb][r] : kNegBig;
            }
          };
          auto weight = [&](int kb, int r) {
            const float y = score_y<MODE, false>(sacc[kb][r], a.sc, m_run, nullptr);
            sacc[kb][r] = exp2_fast(y);
            // Pins the element's arithmetic to the step that asks for it.
            asm volatile("" : "+v"(sacc[kb][r]));
          };
          // Half t of a block's weights rounded to bf16 in MFMA operand order; the row sum is taken
          // over the rounded values, the ones the PV product uses, so the normalisation
          // matches the numerator exactly (a single visible key returns V).
          auto pack = [&](int kb, int t, bf16x8& pb) {
            pb = pack8(sacc[kb], 8 * t);
            l_run += sum_bf16x8(pb);
            if constexpr (DROP) pb = keep_packed(pb, mw[kb], t);
          };
          auto k_ptr = [&](int kb, int s) { return sk + (kb * 32 + lr) * LD + 16 * s + 8 * gl; };
          auto v_ptr = [&](int kb, int i) {  // PV step i = NDB t + db
            return sv + (kb * 32 + 16 * (i / NDB) + trow) * LD + 32 * (i % NDB) + tcol;
          };
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
          // Both blocks' score MFMAs as one stream of 2 NS steps (step j: block j / NS, slice
          // j % NS); block 1's steps each carry a share of block 0's weights.
          bf16x8 kr[KPF];
#pragma unroll
          for (int j = 0; j < KPF; ++j) kr[j] = ld16<bf16x8>(k_ptr(j / NS, j % NS));
#pragma unroll
          for (int j = 0; j < 2 * NS; ++j) {
            const int kb = j / NS, s = j % NS;
            if (j == NS) mask_block(0);
            sacc[kb] = mfma32(kr[j % KPF], bq[s], sacc[kb]);
            if (j + KPF < 2 * NS)
              kr[j % KPF] = ld16<bf16x8>(k_ptr((j + KPF) / NS, (j + KPF) % NS));
            if (kb == 1) {
#pragma unroll
              for (int r = 16 * s / NS; r < 16 * (s + 1) / NS; ++r) weight(0, r);
            }
            __builtin_amdgcn_sched_barrier(kFence);
          }
          // Both blocks' PV MFMAs as one stream of 4 NDB steps (step i: block i / (2 NDB),
          // product i % (2 NDB) = NDB t + db).  Block 1's weights share them out by halves:
          // elements 0-7 beside block 0's products, 8-15 beside block 1's first-half
          // products, which need only elements 0-7.
          mask_block(1);
          bf16x8 pb[2][2];
          pack(0, 0, pb[0][0]);
          pack(0, 1, pb[0][1]);
          auto v_at = [&](int i) {
            const bf16* p0 = v_ptr(i / (2 * NDB), i % (2 * NDB));
            return tr_read_pair(p0, p0 + 8 * LD);
          };
          bf16x8 vr[VPF];
#pragma unroll
          for (int i = 0; i < VPF; ++i) vr[i] = v_at(i);
          __builtin_amdgcn_sched_barrier(kFence);
#pragma unroll
          for (int i = 0; i < 4 * NDB; ++i) {
            const int kb = i / (2 * NDB), k = i % (2 * NDB);
            if (i == 2 * NDB) pack(1, 0, pb[1][0]);
            if (i == 3 * NDB) pack(1, 1, pb[1][1]);
            oacc[k % NDB] = mfma32(vr[i % VPF], pb[kb][k / NDB], oacc[k % NDB]);
            if (i + VPF < 4 * NDB) vr[i % VPF] = v_at(i + VPF);
            if (i < 3 * NDB) {
              const int h = i < 2 * NDB ? i : i - 2 * NDB;  // step within its share
              const int n = i < 2 * NDB ? 2 * NDB : NDB;    // steps in the share
              const int r0 = i < 2 * NDB ? 0 : 8;
#pragma unroll
              for (int r = r0 + 8 * h / n; r < r0 + 8 * (h + 1) / n; ++r) weight(1, r);
            }
            __builtin_amdgcn_sched_barrier(kFence);
          }
        };
        body();
      } else {
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          bf16x8 ka[NS];
#pragma unroll
          for (int s = 0; s < NS; ++s)
            ka[s] = ld16<bf16x8>(sk + (kb * 32 + lr) * LD + 16 * s + 8 * gl);
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
          for (int s = 0; s < NS; ++s) sacc[kb] = mfma32(ka[s], bq[s], sacc[kb]);
        }
        auto scores = [&](auto masked) {
          float mx = kNegBig;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              float y = score_y<MODE, false>(sacc[kb][r], a.sc, 0.f, nullptr);
              if constexpr (decltype(masked)::value)
                y = visible(qd - (32 * kb + 8 * (r >> 2) + (r & 3)), lim) ? y : kNegBig;
              sacc[kb][r] = y;
              mx = fmaxf(mx, y);
            }
          return mx;
        };
        float mx = need_mask ? scores(std::true_type{}) : scores(std::false_type{});
        mx = pair_max(mx);
        // Lazy rescaling: the reference maximum moves (and the accumulators are rescaled) only
        // when a row's maximum exceeds it by more than 2^8, decided for the whole wave; else
        // the weights are taken against the old reference, at most 2^8.  Numerator and
        // denominator share the reference, so the result is the same softmax.
        const bool grow = mx > m_run + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
          const float m_new = grow ? mx : m_run;
          const float alpha = exp2_fast(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb][r] = exp2_fast(sacc[kb][r] - m_run);
          bf16x8 pb[2] = {pack8(sacc[kb], 0), pack8(sacc[kb], 8)};
          l_run += sum_bf16x8(pb[0]) + sum_bf16x8(pb[1]);
          if constexpr (DROP) {
            pb[0] = keep_packed(pb[0], mw[kb], 0);
            pb[1] = keep_packed(pb[1], mw[kb], 1);
          }
          pv_block<D>(oacc, sv, kb, pb, trow, tcol);
        }
      }
    }
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

  const float l_tot = pair_sum(l_run);
  if (qi < nq && off + qi >= S0) {
    const float inv = (DROP ? a.drop_scale : 1.f) / l_tot;
    bf16* op = a.o + ((int64_t)bh * T + qi) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 v4;
#pragma unroll
        for (int j = 0; j < 4; ++j) v4[j] = to_bf16(oacc[db][4 * i4 + j] * inv);
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * i4 + 4 * gl) = v4;
      }
    if (gl == 0 && a.lse) a.lse[(int64_t)bh * T + qi] = (m_run + log2_fast(l_tot)) * kLn2;
  } else if (qi < T) {
    bf16* op = a.o + ((int64_t)bh * T + qi) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 z;
#pragma unroll
        for (int j = 0; j < 4; ++j) z[j] = to_bf16(0.f);
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * i4 + 4 * gl) = z;
      }
  }
}

// ---- fp32 forward: 16 lanes per query, exact online softmax in fp32 ----------------------
// A workgroup takes 16 consecutive queries of one (b, h); the 16 lanes of a query split its
// visible keys (lane t takes keys k0 + t, k0 + t + 16, ...), each keeping a running (max,
// sum, output row) with exact expf, and the 16 states are merged across the lanes at the end
// (LSE-weighted).  The dot products run in four independent partial sums, so the latency of
// one fused multiply-add chain does not set the pace.  This is the fp32 parity path of small
// shapes; the bf16 kernels above carry the large workloads.
struct FwdF32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int B, T, Hq, Hkv, window, nqt;
  float scale, softcap;
};

constexpr int kF32Queries = 16;  // queries per workgroup (16 lanes each: 256 threads)

template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdF32Args a) {
  static_assert(D % 4 == 0, "rows are read as float4");
  const int T = a.T;
  const int nbh = a.B * a.Hq;
  const int rank = blockIdx.x / nbh;
  const int bh = blockIdx.x - rank * nbh;
  const int qt = a.nqt - 1 - rank;  // heaviest query tiles first
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const int r = threadIdx.x >> 4, t = threadIdx.x & 15;
  const int q0 = qt * kF32Queries, qi = q0 + r;
  const int qrow = min(qi, T - 1);
  const float* kb = a.k + (int64_t)(b * a.Hkv + g) * T * D;
  const float* vb = a.v + (int64_t)(b * a.Hkv + g) * T * D;
  float qv[D];
  {
    const float4* qp = reinterpret_cast<const float4*>(a.q + ((int64_t)bh * T + qrow) * D);
#pragma unroll
    for (int c = 0; c < D / 4; ++c) {
      const float4 x = qp[c];
      qv[4 * c] = x.x;
      qv[4 * c + 1] = x.y;
      qv[4 * c + 2] = x.z;
      qv[4 * c + 3] = x.w;
    }
  }
  // Keys [lo, qrow] are visible (lo from the window), as in the oracle's mask.
  const int lo = a.window > 0 ? max(0, qrow - a.window + 1) : 0;
  float m = -INFINITY, l = 0.f;
  float ov[D];
#pragma unroll
  for (int d = 0; d < D; ++d) ov[d] = 0.f;
  for (int j = lo + t; j <= qrow; j += 16) {
    const float4* kp = reinterpret_cast<const float4*>(kb + (int64_t)j * D);
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 4; ++c) {
      const float4 x = kp[c];
      float& acc = part[c & 3];
      acc = fmaf(qv[4 * c], x.x, acc);
      acc = fmaf(qv[4 * c + 1], x.y, acc);
      acc = fmaf(qv[4 * c + 2], x.z, acc);
      acc = fmaf(qv[4 * c + 3], x.w, acc);
    }
    float s = ((part[0] + part[1]) + (part[2] + part[3])) * a.scale;
    if (a.softcap > 0.f) s = a.softcap * tanhf(s / a.softcap);
    if (s > m) {
      const float alpha = expf(m - s);  // 0 for the first key (m = -inf)
      l *= alpha;
#pragma unroll
      for (int d = 0; d < D; ++d) ov[d] *= alpha;
      m = s;
    }
    const float p = expf(s - m);
    l += p;
    const float4* vp = reinterpret_cast<const float4*>(vb + (int64_t)j * D);
#pragma unroll
    for (int c = 0; c < D / 4; ++c) {
      const float4 x = vp[c];
      ov[4 * c] = fmaf(p, x.x, ov[4 * c]);
      ov[4 * c + 1] = fmaf(p, x.y, ov[4 * c + 1]);
      ov[4 * c + 2] = fmaf(p, x.z, ov[4 * c + 2]);
      ov[4 * c + 3] = fmaf(p, x.w, ov[4 * c + 3]);
    }
  }
  // Merge the 16 lanes of the query: M = max m, l = sum l_t e^(m_t - M), o likewise.  A lane
  // without keys holds m = -inf and l = 0 and contributes nothing.
#pragma unroll
  for (int x = 1; x < 16; x <<= 1) {
    const float m2 = __shfl_xor(m, x, 64);
    const float l2 = __shfl_xor(l, x, 64);
    const float mn = fmaxf(m, m2);
    const float fa = m == -INFINITY ? 0.f : expf(m - mn);
    const float fb = m2 == -INFINITY ? 0.f : expf(m2 - mn);
    l = l * fa + l2 * fb;
#pragma unroll
    for (int d = 0; d < D; ++d) ov[d] = ov[d] * fa + __shfl_xor(ov[d], x, 64) * fb;
    m = mn;
  }
  if (qi < T && t == 0) {
    float4* op = reinterpret_cast<float4*>(a.o + ((int64_t)bh * T + qi) * D);
    const float inv = 1.f / l;
#pragma unroll
    for (int c = 0; c < D / 4; ++c)
      op[c] = make_float4(ov[4 * c] * inv, ov[4 * c + 1] * inv, ov[4 * c + 2] * inv, ov[4 * c + 3] * inv);
    a.lse[(int64_t)bh * T + qi] = m + logf(l);
  }
}

// Launch the plain, packed-rows or dropout instantiation.
template <int D, int MODE, bool FIXED>
void launch_k(dim3 grid, hipStream_t s, const FwdArgs& a) {
  if (a.seg_start || a.cache_start)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, MODE, FIXED, kVarPacked>), grid, dim3(256), 0, s, a);
  else if (a.drop_rows)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, MODE, FIXED, kVarDrop>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, MODE, FIXED, kVarPlain>), grid, dim3(256), 0, s, a);
}

template <int D>
hipError_t launch_fwd_bf16_d(const FwdParams& p, hipStream_t s) {
  FwdArgs a;
  a.q = (const bf16*)p.q;
  a.k = (const bf16*)p.k;
  a.v = (const bf16*)p.v;
  a.o = (bf16*)p.o;
  a.lse = p.lse;
  a.cache_len = p.cache_len;
  a.cache_start = p.cache_start;
  a.seg_start = p.seg_start;
  a.drop_rows = p.drop_rows;
  a.drop_pitch = dropout_pitch(p.T);
  a.drop_scale = p.drop_scale;
  a.B = p.B;
  a.T = p.T;
  a.Tk = p.cache_len ? p.Lmax : p.T;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.window = p.window;
  a.nqt = (p.T + kBM - 1) / kBM;
  const ScoreSetup ss = make_score_setup(p.scale, p.softcap, D, p.qk_norm);
  a.shift = ss.shift;
  a.sc = ss.coef;
  a.rp = make_row_prologue(p.rope, p.rope_base, p.qk_norm, p.eps, D);
  const dim3 grid((unsigned)(a.nqt * p.B * p.Hq));
  static const char* names[4] = {"fwd_bf16_d32", "fwd_bf16_d64", "fwd_bf16_d96", "fwd_bf16_d128"};
  TraceScope t(names[D / 32 - 1], s);
  if (ss.mode == kScoreScale && ss.fixed_shift)
    launch_k<D, kScoreScale, true>(grid, s, a);
  else if (ss.mode == kScoreScale)
    launch_k<D, kScoreScale, false>(grid, s, a);
  else if (ss.mode == kScoreCapPoly5 && ss.fixed_shift)
    launch_k<D, kScoreCapPoly5, true>(grid, s, a);
  else if (ss.mode == kScoreCapPoly && ss.fixed_shift)
    launch_k<D, kScoreCapPoly, true>(grid, s, a);
  else
    launch_k<D, kScoreCapExp, false>(grid, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_f32_d(const FwdParams& p, hipStream_t s) {
  FwdF32Args a;
  a.q = (const float*)p.q;
  a.k = (const float*)p.k;
  a.v = (const float*)p.v;
  a.o = (float*)p.o;
  a.lse = p.lse;
  a.B = p.B;
  a.T = p.T;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.window = p.window;
  a.nqt = (p.T + kF32Queries - 1) / kF32Queries;
  a.scale = p.scale;
  a.softcap = p.softcap;
  TraceScope t("fwd_f32", s);
  hipLaunchKernelGGL((fwd_f32_kernel<D>), dim3((unsigned)(a.nqt * p.B * p.Hq)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t s) {
  switch (p.D) {
    case 32: return launch_fwd_bf16_d<32>(p, s);
    case 64: return launch_fwd_bf16_d<64>(p, s);
    case 96: return launch_fwd_bf16_d<96>(p, s);
    case 128: return launch_fwd_bf16_d<128>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t s) {
  switch (p.D) {
    case 32: return launch_fwd_f32_d<32>(p, s);
    case 64: return launch_fwd_f32_d<64>(p, s);
    case 96: return launch_fwd_f32_d<96>(p, s);
    case 128: return launch_fwd_f32_d<128>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace attn
