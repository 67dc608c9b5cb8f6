// Single-token KV-cache decode on gfx950 ("GPT pretraining" page, section "Bonus: KV
// Caching"): the cache of sequence b holds L = cache_len[b] rows, the newest token's key and
// value among them, and that token's query sits at position L - 1, so no cached row is in its
// future and all L are scored.  The nanoGPT-JAX 181M model card's inference notes ask that only
// the compact active part of the cache be attended; rows at or past L are never read.
// With left-padded batches (the same notes: left-padded prompts, right-aligned generation)
// rows below cache_start[b] are padding and are not read either; positions count from there.
//
// The work is HBM-bound (about 2 flops per byte), so it runs on the vector ALUs with
// coalesced 16-byte loads, not on MFMA:
//  * split kernel: one 4-wave workgroup per (chunk of split_len cache rows, b, kv head, head
//    subset).  LPR lanes share one row, each owning D/LPR elements in 8- or 16-byte granules
//    interleaved so that each load instruction reads one contiguous span of every row it
//    touches; the chunk is streamed in passes of NW * 2 * 64 / LPR rows through a two-stage
//    register pipeline (the loads of the next pass are in flight while the current one
//    computes).  A whole cache per workgroup (the batch fills the GPU) uses four lanes per
//    row and 16-byte loads.  Chunked caches use eight lanes per row: the per-lane buffers
//    halve, four workgroups fit per CU, and the memory latency that starts each chunk (cache
//    length, then the first rows) hides behind the other workgroups' streams.  Each lane keeps a
//    running (max, sum, output) for every query head of the GQA group (K and V are read once
//    per KV head); lanes and waves are merged (LSE-weighted) into one partial per chunk.
//  * merge, in the same kernel: a sequence's active rows span n chunks (fixed split_len, so
//    every workgroup streams about the same number of rows whatever the cache lengths).  With
//    n = 1 the chunk writes the output itself.  Otherwise each chunk stores its partial
//    (m, l, o), publishes it (agent-scope release) and takes a ticket from the (b, kv head,
//    head subset) counter; the chunk that draws the last ticket reads the n partials
//    (acquire), merges them -- with M = max m_s, o = sum_s o_s 2^(m_s - M) / sum_s l_s
//    2^(m_s - M), an exact identity of softmax -- writes the output and sets the counter back
//    to zero for the next call.
#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

struct DecArgs {
  const bf16* q;
  const bf16* kc;
  const bf16* vc;
  const int32_t* cache_len;
  const int32_t* cache_start;  // left padding rows per sequence (or null: none)
  bf16* o;
  float* part;      // [B, Hq, nsplit, D + 2] partials (m, l, o) of multi-chunk sequences
  unsigned* count;  // [B * Hkv * head subsets] tickets; zero between calls
  int B, Hq, Hkv, Lmax, split_len, nsplit;
  ScoreCoef sc;    // score transform (mode chosen on the host)
  float scale;
  RowPrologue rp;  // query RoPE (position L - 1 - start) and RMSNorm
};

// Active rows [first, L) of sequence b: L = cache_len clamped to [0, Lmax], first = the
// left padding clamped to [0, L].
__device__ __forceinline__ int active_end(const DecArgs& a, int b) {
  return min(max(a.cache_len[b], 0), a.Lmax);
}
__device__ __forceinline__ int active_first(const DecArgs& a, int b, int L) {
  return a.cache_start ? min(max(a.cache_start[b], 0), L) : 0;
}

// Device-coherent (agent-scope) store and load of a partial: performed where every compute
// unit sees them, without the cache-wide write-back a release fence costs.
__device__ __forceinline__ void coherent_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waves per split workgroup: four, with two workgroups resident per CU, so one streams while
// the other starts up or drains (measured faster than one 8-wave workgroup per CU).
constexpr int kDecWaves = 4;
// Largest factor a running maximum may grow by before the accumulators are rescaled (log2).
constexpr float kRescaleSlack = 8.f;

// Running softmax state of one lane for one query head: maximum (log2 units), weight sum
// and the weighted sum of its value-row elements.
template <int NE>
struct RunState {
  float m, l, o[NE];
};

// A DPP lane permutation of x (CTRL: the dpp_ctrl encoding).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Lane map of one cache row: LPR lanes (4 or 8), lane j owning granules j, j + LPR, ... of GB
// bytes (16 when the row's 16-byte granules divide evenly among the lanes, else 8), so granule
// k of all LPR lanes is one contiguous span of the row.  Element e of granule k of lane j is
// head-dim index (j + LPR k) EPG + e.  Four lanes per row give 16-byte loads; eight halve the
// per-lane buffers (more workgroups per CU).
template <int D, int LPR>
struct RowMap {
  static constexpr int GB = ((D * 2 / 16) % LPR == 0) ? 16 : 8;
  static constexpr int EPG = GB / 2;        // elements per granule
  static constexpr int NG = D / EPG / LPR;  // granules per lane
  static constexpr int NE = NG * EPG;       // elements per lane (D / LPR)
  typedef __bf16 G __attribute__((ext_vector_type(EPG)));
  static __device__ __forceinline__ int dim(int j, int k, int e) { return (j + LPR * k) * EPG + e; }
  static_assert(LPR * NG * EPG == D, "the LPR lanes' granules tile the row exactly");
  static_assert(LPR == 4 || LPR == 8, "the score sums cover quads or half rows of lanes");
};

// Workgroups resident per CU: two with four lanes per row; with eight, four (three when the
// group's heads hold 256 or more output elements per row).
template <int D, int HPB, int LPR>
constexpr int dec_min_blocks() { return LPR == 4 ? 2 : (HPB * D >= 256 ? 3 : 4); }

template <int D, int HPB, int MODE, int LPR>
__global__ __launch_bounds__(64 * kDecWaves, (dec_min_blocks<D, HPB, LPR>())) void decode_split_kernel(DecArgs a) {
  constexpr int NW = kDecWaves;
  typedef RowMap<D, LPR> RM;
  constexpr int NG = RM::NG, EPG = RM::EPG;
  constexpr int NE = RM::NE;      // output elements per lane and head
  constexpr int NSTEP = 2;        // rows per lane per pass (a pair: one dot2 per element)
  constexpr int kRowsPerStep = 64 / LPR;  // rows a wave covers per step
  constexpr int kRowsPerWave = kRowsPerStep * NSTEP;
  constexpr int kPass = NW * kRowsPerWave;  // rows per workgroup pass
  constexpr int RL = 64 / LPR;  // row groups of lanes per wave
  // Rescaled states of every row group for the merge: [wave][row group] rows of HPB x D, the
  // row stride padded to 4 banks mod 64 so that the 16-byte writes of a wave's row groups
  // fall on distinct banks.
  constexpr int kRowStride = HPB * D + (4 - (HPB * D) % 64 + 64) % 64;
  __shared__ float sq[HPB][D];
  __shared__ float sm[NW][HPB];
  __shared__ float sl[NW][HPB];
  __shared__ __attribute__((aligned(16))) float so[NW * RL * kRowStride];

  const int G = a.Hq / a.Hkv;
  const int nsub = G / HPB;
  // Workgroup i runs on XCD i % 8.  Chunk `split` of unit y is placed so that every XCD gets
  // each chunk index of an eighth of the units, and a unit's chunks rotate over the XCDs:
  // the first chunks (active for every sequence) and the last ones (active only for long
  // caches) are spread evenly instead of landing on a few XCDs.
  const int units = a.B * a.Hkv * nsub;
  int split, y;
  if ((units & 7) == 0) {
    const int xcd = blockIdx.x & 7, k = blockIdx.x >> 3;
    split = k % a.nsplit;
    y = 8 * (k / a.nsplit) + ((xcd + split) & 7);
  } else {
    y = blockIdx.x % units;
    split = blockIdx.x / units;
  }
  const int hs = y % nsub;
  const int bg = y / nsub;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int h0 = g * G + hs * HPB;
  // The raw query pair of this lane (wave hh < HPB holds head h0 + hh), loaded before anything
  // waits on the cache length, so its latency overlaps that of the length.
  const int half = D / 2;
  const bool qact = w < HPB && lane < half;
  float x1 = 0.f, x2 = 0.f;
  if (qact) {
    const bf16* qr = a.q + ((int64_t)b * a.Hq + h0 + w) * D;
    x1 = from_bf16(qr[lane]);
    x2 = from_bf16(qr[lane + half]);
  }
  const int L = active_end(a, b);
  const int first = active_first(a, b, L);
  const int c0 = split * a.split_len;  // this chunk's rows: [c0, c0 + split_len) & [first, L)
  const int start = max(c0, first);
  const int stop = min(L, c0 + a.split_len);
  // Chunks s_first .. s_first + nact - 1 hold the active rows [first, L) (none if first == L).
  const int s_first = first / a.split_len;
  const int nact = first < L ? (L - 1) / a.split_len - s_first + 1 : 0;
  if (start >= stop) {
    // No active row in this chunk.  For an empty active range the first chunk writes the
    // output row: zeros.
    if (nact == 0 && split == 0)
      for (int t = tid; t < HPB * D; t += 64 * NW)
        a.o[((int64_t)b * a.Hq + h0 + t / D) * D + t % D] = to_bf16(0.f);
    return;
  }
  const int npass = (stop - start + kPass - 1) / kPass;

  const int j8 = lane % LPR;  // this lane's part of a row
  const int rq = lane / LPR;  // row within a step
  const bf16* kb = a.kc + (int64_t)bg * a.Lmax * D;
  const bf16* vb = a.vc + (int64_t)bg * a.Lmax * D;
  const int row0 = start + kRowsPerWave * w + rq;  // this lane's row in pass 0, step 0

  // Loads of one pass.  Rows past `stop` read row stop - 1 (in bounds, weight 0); this also
  // covers the prefetch issued past the last pass, so every load is unconditional and the
  // compiler waits for exactly the older pass.
  typedef typename RM::G Gv;
  struct Buf {
    Gv k[NSTEP][NG], v[NSTEP][NG];
  };
  // The loads address a uniform base (scalar registers) plus one 32-bit byte offset per lane
  // and step (below Lmax * 2D <= 2^32, checked on the host), with the granule's position as an
  // immediate.  The offsets of the next pass are computed as soon as the previous pass has been
  // issued, so they sit in registers of their own: an address register that had been a load
  // target would make the next pass wait for the loads still in flight.
  auto uniform = [](const bf16* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const __attribute__((address_space(1))) char*)(((uint64_t)hi << 32) | lo);
  };
  const auto kbase = uniform(kb);
  const auto vbase = uniform(vb);
  const uint32_t lane_byte = 2u * (uint32_t)RM::dim(j8, 0, 0);
  auto offsets = [&](uint32_t (&o)[NSTEP], int pass) {
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      o[st] = (uint32_t)min(row0 + kPass * pass + kRowsPerStep * st, stop - 1) * (uint32_t)(2 * D) +
              lane_byte;
      asm volatile("" : "+v"(o[st]));
    }
  };
  uint32_t onext[NSTEP];
  offsets(onext, 0);
  // Passes are loaded in order 0, 1, 2, ...; each call issues the pass `onext` points at.
  auto load = [&](Buf& bu, int pass) {
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
#pragma unroll
      for (int u = 0; u < NG; ++u) {
        // Granule u of this lane: elements RM::dim(j8, u, 0) .. + EPG - 1 of the row (< D).
        const int gb = 2 * RM::dim(0, u, 0);  // bytes past the lane's first granule
        bu.k[st][u] = *(const __attribute__((address_space(1))) Gv*)(kbase + onext[st] + gb);
        bu.v[st][u] = *(const __attribute__((address_space(1))) Gv*)(vbase + onext[st] + gb);
      }
    }
    offsets(onext, pass + 1);
  };

  Buf b0, b1;
  load(b0, 0);

  // Query prologue while the first loads are in flight: wave hh rotates (position
  // L - 1 - first) and normalises head h0 + hh.
  if (w < HPB) {
    if (a.rp.rope && qact) rope_pair(x1, x2, L - 1 - first, a.rp.omega_rev[lane], false);
    if (a.rp.qk_norm) {
      const float inv = 1.0f / sqrtf(wave_sum(x1 * x1 + x2 * x2) / (float)D + a.rp.eps);
      x1 *= inv;
      x2 *= inv;
    }
    if (qact) {
      sq[w][lane] = x1;
      sq[w][lane + half] = x2;
    }
  }
  __syncthreads();
  // q^ of this lane's eighth of a row, as bf16 pairs for v_dot2_f32_bf16 against the keys.
  bf16x2 qv[HPB][NE / 2];
#pragma unroll
  for (int hh = 0; hh < HPB; ++hh)
#pragma unroll
    for (int u = 0; u < NG; ++u)
#pragma unroll
      for (int e = 0; e < EPG / 2; ++e) {
        qv[hh][u * EPG / 2 + e][0] = to_bf16(sq[hh][RM::dim(j8, u, 2 * e)]);
        qv[hh][u * EPG / 2 + e][1] = to_bf16(sq[hh][RM::dim(j8, u, 2 * e + 1)]);
      }

  RunState<NE> st_[HPB];
#pragma unroll
  for (int hh = 0; hh < HPB; ++hh) {
    st_[hh].m = kNegBig;
    st_[hh].l = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) st_[hh].o[e] = 0.f;
  }

  // One pass: scores of this lane's two rows for every head, then the weights as a bf16 pair
  // and o += p0 v0 + p1 v1 as one dot2 per element.  The accumulators are rescaled only when
  // the maximum grows by more than 2^8 (the result is the same: numerator and denominator
  // share the reference maximum).
  auto compute = [&](const Buf& bu, int pass) {
    float yv[NSTEP][HPB];
#pragma unroll
    for (int stp = 0; stp < NSTEP; ++stp) {
      const bool valid = row0 + kPass * pass + kRowsPerStep * stp < stop;
#pragma unroll
      for (int hh = 0; hh < HPB; ++hh) {
        float dot = 0.f;
#pragma unroll
        for (int u = 0; u < NG; ++u)
#pragma unroll
          for (int e = 0; e < EPG / 2; ++e) {
            const bf16x2 kp = {bu.k[stp][u][2 * e], bu.k[stp][u][2 * e + 1]};
            dot = __builtin_amdgcn_fdot2_f32_bf16(qv[hh][u * EPG / 2 + e], kp, dot, false);
          }
        // Sum over the LPR lanes of the row: DPP quad permutations (xor 1, xor 2), then, for
        // eight lanes, the mirror inside each half row of 8.
        dot += dpp_f<0xB1>(dot);
        dot += dpp_f<0x4E>(dot);
        if constexpr (LPR == 8) dot += dpp_f<0x141>(dot);
        const float yy = score_y<MODE, false>(dot, a.sc, 0.f, nullptr);
        yv[stp][hh] = valid ? yy : kNegBig;
      }
    }
    // Value pairs (row 0, row 1) per element, shared by all heads.
    bf16x2 vp[NE];
#pragma unroll
    for (int u = 0; u < NG; ++u)
#pragma unroll
      for (int e = 0; e < EPG; ++e) vp[EPG * u + e] = bf16x2{bu.v[0][u][e], bu.v[1][u][e]};
#pragma unroll
    for (int hh = 0; hh < HPB; ++hh) {
      RunState<NE>& S = st_[hh];
      const float mx = fmaxf(yv[0][hh], yv[1][hh]);
      if (mx > S.m + kRescaleSlack) {
        const float alpha = exp2_fast(S.m - mx);
        S.l *= alpha;
#pragma unroll
        for (int e = 0; e < NE; ++e) S.o[e] *= alpha;
        S.m = mx;
      }
      const bf16x2 pp = {to_bf16(exp2_fast(yv[0][hh] - S.m)), to_bf16(exp2_fast(yv[1][hh] - S.m))};
      S.l += (float)pp[0] + (float)pp[1];
#pragma unroll
      for (int e = 0; e < NE; ++e) S.o[e] = __builtin_amdgcn_fdot2_f32_bf16(vp[e], pp, S.o[e], false);
    }
  };

  // Two-stage register pipeline: the loads of pass p + 1 are in flight while pass p computes.
  for (int pass = 0; pass < npass; pass += 2) {
    load(b1, pass + 1);
    compute(b0, pass);
    if (pass + 1 >= npass) break;
    load(b0, pass + 2);
    compute(b1, pass + 1);
  }

  // Merge all row groups at once.  The lanes of a row group share its scores, so they hold the
  // same (m, l) and split its output elements.  First the workgroup's largest reference per
  // head (DPP and lane swaps inside each wave, then the waves through LDS); each lane rescales
  // its own (l, o) to it; then every thread sums one output element over the row groups
  // through LDS: no exp or maximum per merge step.
  // All-lane reduction of a wave: DPP inside rows of 16 lanes, then lane swaps across rows.
  auto wave_reduce = [lane](float x, auto op) {
    x = op(x, dpp_f<0xB1>(x));   // xor 1
    x = op(x, dpp_f<0x4E>(x));   // xor 2
    x = op(x, dpp_f<0x141>(x));  // mirror inside 8 lanes
    x = op(x, dpp_f<0x140>(x));  // mirror inside 16 lanes
    {
      auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
      x = op(x, __uint_as_float(((lane >> 4) & 1) ? r[0] : r[1]));
    }
    {
      auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
      x = op(x, __uint_as_float(lane >= 32 ? r[0] : r[1]));
    }
    return x;
  };
  auto fmax_op = [](float x, float y) { return fmaxf(x, y); };
  auto add_op = [](float x, float y) { return x + y; };
#pragma unroll
  for (int hh = 0; hh < HPB; ++hh) {
    const float wm = wave_reduce(st_[hh].m, fmax_op);
    if (lane == 0) sm[w][hh] = wm;
  }
  __syncthreads();
  {
    float* row = so + (w * RL + rq) * kRowStride;
#pragma unroll
    for (int hh = 0; hh < HPB; ++hh) {
      float M = sm[0][hh];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, sm[ww][hh]);
      // A row group that saw no active row holds m = kNegBig, l = 0, o = 0: factor 0.
      const float f = exp2_fast(st_[hh].m - M);
      // The wave's rescaled weight sum (one lane per row group carries its l).
      const float lw = wave_reduce(j8 == 0 ? st_[hh].l * f : 0.f, add_op);
      if (lane == 0) sl[w][hh] = lw;
#pragma unroll
      for (int u = 0; u < NG; ++u)
#pragma unroll
        for (int e = 0; e < EPG; ++e) row[hh * D + RM::dim(j8, u, e)] = st_[hh].o[EPG * u + e] * f;
    }
  }
  __syncthreads();
  for (int t = tid; t < HPB * D; t += 64 * NW) {
    const int hh = t / D, d = t - hh * D;
    float M = sm[0][hh];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, sm[ww][hh]);
    float lt = 0.f, ot = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) lt += sl[ww][hh];
#pragma unroll
    for (int g2 = 0; g2 < NW * RL; ++g2) ot += so[g2 * kRowStride + hh * D + d];
    if (nact == 1) {
      // The only chunk of this sequence: write the normalised output directly.
      a.o[((int64_t)b * a.Hq + h0 + hh) * D + d] = to_bf16(ot / lt);
    } else {
      float* pp = a.part + (((int64_t)b * a.Hq + h0 + hh) * a.nsplit + split) * (D + 2);
      coherent_store(pp + 2 + d, ot);
      if (d == 0) {
        coherent_store(pp, M);
        coherent_store(pp + 1, lt);
      }
    }
  }
  if (nact == 1) return;
  // Publish the partial, then take a ticket; the last of the nact chunks merges.  The partials
  // travel only through device-coherent stores and loads, so publishing them needs no
  // cache-wide write-back: each wave waits until its stores are performed, the barrier joins
  // the waves, and only then is the ticket drawn.
  __shared__ unsigned ticket;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  unsigned* cnt = a.count + y;
  if (tid == 0) ticket = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (ticket != (unsigned)(nact - 1)) return;
  // Merge in batches of MB chunks: a batch's loads are all issued before any is used (indices
  // past the last chunk re-read it with weight 0), so the merge waits for one memory round
  // trip per batch, not per chunk.
  constexpr int MB = 8;
  for (int t = tid; t < HPB * D; t += 64 * NW) {
    const int hh = t / D, d = t - hh * D;
    const float* pp = a.part + (((int64_t)b * a.Hq + h0 + hh) * a.nsplit + s_first) * (D + 2);
    float M = kNegBig, lt = 0.f, ot = 0.f;
    for (int s0 = 0; s0 < nact; s0 += MB) {
      float mv[MB], lv[MB], ov[MB];
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const float* ps = pp + min(s0 + j, nact - 1) * (D + 2);
        mv[j] = coherent_load(ps);
        lv[j] = coherent_load(ps + 1);
        ov[j] = coherent_load(ps + 2 + d);
      }
      float mb = M;
#pragma unroll
      for (int j = 0; j < MB; ++j) mb = fmaxf(mb, mv[j]);
      const float r = exp2_fast(M - mb);
      lt *= r;
      ot *= r;
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const float f = s0 + j < nact ? exp2_fast(mv[j] - mb) : 0.f;
        lt = fmaf(lv[j], f, lt);
        ot = fmaf(ov[j], f, ot);
      }
      M = mb;
    }
    a.o[((int64_t)b * a.Hq + h0 + hh) * D + d] = to_bf16(ot / lt);
  }
  // Every chunk of this sequence has drawn its ticket: ready for the next call.
  if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int HPB, int MODE, int LPR>
hipError_t launch_split(const DecArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const dim3 grid((unsigned)(a.nsplit * a.B * a.Hkv * (G / HPB)));
  static const char* names[4] = {"decode_split_d32", "decode_split_d64", "decode_split_d96",
                                 "decode_split_d128"};
  TraceScope t(names[D / 32 - 1], s);
  hipLaunchKernelGGL((decode_split_kernel<D, HPB, MODE, LPR>), grid, dim3(64 * kDecWaves), 0, s, a);
  return hipGetLastError();
}

// One chunk per cache: four lanes per row (16-byte loads; measured faster when each
// workgroup streams a whole cache).  Chunked caches: eight lanes per row (four workgroups per
// CU hide each chunk's start-up latency behind the others' streams).
template <int D, int HPB, int MODE>
hipError_t launch_split_lanes(const DecArgs& a, hipStream_t s) {
  return a.nsplit == 1 ? launch_split<D, HPB, MODE, 4>(a, s) : launch_split<D, HPB, MODE, 8>(a, s);
}

template <int D, int HPB>
hipError_t launch_split_mode(const DecArgs& a, int mode, hipStream_t s) {
  if (mode == kScoreScale) return launch_split_lanes<D, HPB, kScoreScale>(a, s);
  if (mode == kScoreCapPoly5) return launch_split_lanes<D, HPB, kScoreCapPoly5>(a, s);
  if (mode == kScoreCapPoly) return launch_split_lanes<D, HPB, kScoreCapPoly>(a, s);
  return launch_split_lanes<D, HPB, kScoreCapExp>(a, s);
}

template <int D>
hipError_t launch_decode_d(const DecArgs& a, int mode, hipStream_t s) {
  hipError_t e;
  // decode_heads_per_block keeps heads x D <= 256, so only those instantiations exist.
  switch (decode_heads_per_block(a.Hq / a.Hkv, D)) {
    case 4:
      if constexpr (4 * D <= 256) e = launch_split_mode<D, 4>(a, mode, s);
      else e = hipErrorInvalidValue;
      break;
    case 3:
      if constexpr (3 * D <= 256) e = launch_split_mode<D, 3>(a, mode, s);
      else e = hipErrorInvalidValue;
      break;
    case 2: e = launch_split_mode<D, 2>(a, mode, s); break;
    default: e = launch_split_mode<D, 1>(a, mode, s); break;
  }
  return e;
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t s) {
  DecArgs a;
  a.q = (const bf16*)p.q;
  a.kc = (const bf16*)p.kc;
  a.vc = (const bf16*)p.vc;
  a.cache_len = p.cache_len;
  a.cache_start = p.cache_start;
  a.o = (bf16*)p.o;
  a.part = p.part;
  a.count = p.count;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.Lmax = p.Lmax;
  a.split_len = p.split_len;
  a.nsplit = p.nsplit;
  a.scale = p.scale;
  // Scores use the same transform as training; the decode keeps a running maximum, so the
  // fixed-shift option of the forward is not needed here.
  const ScoreSetup ss = make_score_setup(p.scale, p.softcap, p.D, p.qk_norm);
  a.sc = ss.coef;
  a.rp = make_row_prologue(p.rope, p.rope_base, p.qk_norm, p.eps, p.D);
  switch (p.D) {
    case 32: return launch_decode_d<32>(a, ss.mode, s);
    case 64: return launch_decode_d<64>(a, ss.mode, s);
    case 96: return launch_decode_d<96>(a, ss.mode, s);
    case 128: return launch_decode_d<128>(a, ss.mode, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace attn
