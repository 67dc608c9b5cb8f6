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
//    subset), two resident per CU.  Four lanes share one row (each owns D/4 elements: 64
//    contiguous bytes per quad and load); a wave covers 16 rows per step, and the chunk is
//    streamed in passes
//    through a two-stage register pipeline (the loads of the next pass are in flight while
//    the current one computes).  Each quad keeps a running (max, sum, output) for every
//    query head of the GQA group (K and V are read once per KV head); quads and waves are
//    merged (LSE-weighted) into one partial (m, l, o) per chunk.
//  * combine kernel: merges the chunks of each (b, h): with M = max m_s,
//    o = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M)  -- an exact identity of softmax.
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
  float* part;
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

// Merge two states: both are rescaled to the larger maximum (exact softmax identity).
template <int NE>
__device__ __forceinline__ void merge_state(RunState<NE>& s, float mp, float lp, const float* op) {
  const float mn = fmaxf(s.m, mp);
  const float fa = exp2_fast(s.m - mn), fb = exp2_fast(mp - mn);
  s.l = s.l * fa + lp * fb;
#pragma unroll
  for (int e = 0; e < NE; ++e) s.o[e] = s.o[e] * fa + op[e] * fb;
  s.m = mn;
}

__device__ __forceinline__ float dpp_ror(float x, int ctrl_is_8) {
  const int v = __float_as_int(x);
  return __int_as_float(ctrl_is_8 ? __builtin_amdgcn_update_dpp(0, v, 0x128, 0xf, 0xf, false)
                                  : __builtin_amdgcn_update_dpp(0, v, 0x124, 0xf, 0xf, false));
}

// All-reduce of the states over the 16 lanes that share (lane & 3): two DPP row rotations
// (by 4 and 8 lanes) inside each row of 16, then swaps across rows (xor 16, xor 32).
template <int NE>
__device__ __forceinline__ void merge_quads(RunState<NE>& s) {
#pragma unroll
  for (int r8 = 0; r8 < 2; ++r8) {
    float op[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) op[e] = dpp_ror(s.o[e], r8);
    merge_state<NE>(s, dpp_ror(s.m, r8), dpp_ror(s.l, r8), op);
  }
  const int lane = threadIdx.x & 63;
  {
    // v_permlane16_swap(x, x): a lane in an even row of 16 gets (x[l], x[l + 16]), one in an
    // odd row (x[l - 16], x[l]); the partner's value is the other half.
    const bool odd = (lane >> 4) & 1;
    auto sw = [odd](float x) {
      auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
      return __uint_as_float(odd ? r[0] : r[1]);
    };
    float op[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) op[e] = sw(s.o[e]);
    merge_state<NE>(s, sw(s.m), sw(s.l), op);
  }
  {
    const bool hi = lane >= 32;
    auto sw = [hi](float x) {
      auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
      return __uint_as_float(hi ? r[0] : r[1]);
    };
    float op[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) op[e] = sw(s.o[e]);
    merge_state<NE>(s, sw(s.m), sw(s.l), op);
  }
}

template <int D, int HPB, int MODE>
__global__ __launch_bounds__(64 * kDecWaves, 2) void decode_split_kernel(DecArgs a) {
  constexpr int NW = kDecWaves;
  constexpr int NU = D / 32;      // 16-byte chunks per lane per row
  constexpr int NE = NU * 8;      // output elements per lane and head
  constexpr int NSTEP = 2;        // rows per lane per pass (a pair: one dot2 per element)
  constexpr int kRowsPerWave = 16 * NSTEP;
  constexpr int kPass = NW * kRowsPerWave;  // rows per workgroup pass
  __shared__ float sq[HPB][D];
  __shared__ float sm[NW][HPB], sl[NW][HPB];
  __shared__ float so[NW][HPB][D];

  const int G = a.Hq / a.Hkv;
  const int nsub = G / HPB;
  const int split = blockIdx.x;
  const int y = blockIdx.y;
  const int hs = y % nsub;
  const int bg = y / nsub;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int L = active_end(a, b);
  const int first = active_first(a, b, L);
  const int c0 = split * a.split_len;  // this chunk's rows: [c0, c0 + split_len) & [first, L)
  const int start = max(c0, first);
  const int stop = min(L, c0 + a.split_len);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int h0 = g * G + hs * HPB;
  if (start >= stop) {
    // No active row in this chunk.  With a single chunk per sequence (an empty active
    // range) the output row is written here: zeros.
    if (a.nsplit == 1)
      for (int t = tid; t < HPB * D; t += 64 * NW)
        a.o[((int64_t)b * a.Hq + h0 + t / D) * D + t % D] = to_bf16(0.f);
    return;
  }
  const int npass = (stop - start + kPass - 1) / kPass;

  const int s4 = lane & 3;   // this lane's quarter of a row
  const int rq = lane >> 2;  // row within a 16-row step
  const bf16* kb = a.kc + (int64_t)bg * a.Lmax * D + 8 * s4;
  const bf16* vb = a.vc + (int64_t)bg * a.Lmax * D + 8 * s4;
  const int row0 = start + kRowsPerWave * w + rq;  // this lane's row in pass 0, step 0

  // Loads of one pass.  Rows past `stop` read row stop - 1 (in bounds, weight 0); this also
  // covers the prefetch issued past the last pass, so every load is unconditional and the
  // compiler waits for exactly the older pass.
  struct Buf {
    bf16x8 k[NSTEP][NU], v[NSTEP][NU];
  };
  auto load = [&](Buf& bu, int pass) {
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      const int64_t off = (int64_t)min(row0 + kPass * pass + 16 * st, stop - 1) * D;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        bu.k[st][u] = ld16<bf16x8>(kb + off + 32 * u);
        bu.v[st][u] = ld16<bf16x8>(vb + off + 32 * u);
      }
    }
  };

  Buf b0, b1;
  load(b0, 0);

  // Query prologue while the first loads are in flight: wave hh rotates (position
  // L - 1 - first) and normalises head h0 + hh.
  if (w < HPB) {
    const int half = D / 2;
    const bool act = lane < half;
    const bf16* qr = a.q + ((int64_t)b * a.Hq + h0 + w) * D;
    float x1 = act ? from_bf16(qr[lane]) : 0.f;
    float x2 = act ? from_bf16(qr[lane + half]) : 0.f;
    if (a.rp.rope && act) rope_pair(x1, x2, L - 1 - first, a.rp.omega_rev[lane], false);
    if (a.rp.qk_norm) {
      const float inv = 1.0f / sqrtf(wave_sum(x1 * x1 + x2 * x2) / (float)D + a.rp.eps);
      x1 *= inv;
      x2 *= inv;
    }
    if (act) {
      sq[w][lane] = x1;
      sq[w][lane + half] = x2;
    }
  }
  __syncthreads();
  // q^ of this lane's row quarter, as bf16 pairs for v_dot2_f32_bf16 against the cached keys.
  bf16x2 qv[HPB][NU * 4];
#pragma unroll
  for (int hh = 0; hh < HPB; ++hh)
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qv[hh][4 * u + e][0] = to_bf16(sq[hh][32 * u + 8 * s4 + 2 * e]);
        qv[hh][4 * u + e][1] = to_bf16(sq[hh][32 * u + 8 * s4 + 2 * e + 1]);
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
      const bool valid = row0 + kPass * pass + 16 * stp < stop;
#pragma unroll
      for (int hh = 0; hh < HPB; ++hh) {
        float dot = 0.f;
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bf16x2 kp = {bu.k[stp][u][2 * e], bu.k[stp][u][2 * e + 1]};
            dot = __builtin_amdgcn_fdot2_f32_bf16(qv[hh][4 * u + e], kp, dot, false);
          }
        dot += __shfl_xor(dot, 1, 64);
        dot += __shfl_xor(dot, 2, 64);
        const float yy = score_y<MODE, false>(dot, a.sc, 0.f, nullptr);
        yv[stp][hh] = valid ? yy : kNegBig;
      }
    }
    // Value pairs (row 0, row 1) per element, shared by all heads.
    bf16x2 vp[NE];
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) vp[8 * u + e] = bf16x2{bu.v[0][u][e], bu.v[1][u][e]};
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

  // Merge the 16 lanes of each wave that own the same quarter of the rows, then the waves.
#pragma unroll
  for (int hh = 0; hh < HPB; ++hh) merge_quads<NE>(st_[hh]);
  if (lane < 4) {
#pragma unroll
    for (int hh = 0; hh < HPB; ++hh) {
      if (lane == 0) {
        sm[w][hh] = st_[hh].m;
        sl[w][hh] = st_[hh].l;
      }
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) so[w][hh][32 * u + 8 * s4 + e] = st_[hh].o[8 * u + e];
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
    for (int ww = 0; ww < NW; ++ww) {
      const float f = exp2_fast(sm[ww][hh] - M);
      lt += sl[ww][hh] * f;
      ot += so[ww][hh][d] * f;
    }
    if (a.nsplit == 1) {
      // The only chunk of this sequence: write the normalised output directly.
      a.o[((int64_t)b * a.Hq + h0 + hh) * D + d] = to_bf16(ot / lt);
    } else {
      float* pp = a.part + (((int64_t)b * a.Hq + h0 + hh) * a.nsplit + split) * (D + 2);
      pp[2 + d] = ot;
      if (d == 0) {
        pp[0] = M;
        pp[1] = lt;
      }
    }
  }
}

// One wave per (b, h), four per block.  Lanes read the chunks' (m, l) in parallel and the
// wave reduces them; then each lane sums two output columns over the chunks.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecArgs a) {
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= a.B * a.Hq) return;
  const int lane = threadIdx.x & 63;
  const int b = wid / a.Hq;
  const int L = active_end(a, b);
  const int first = active_first(a, b, L);
  // Chunks s0 .. n - 1 hold active rows (none when first == L); only they wrote partials.
  const int n = (L + a.split_len - 1) / a.split_len;
  const int s_first = first < L ? first / a.split_len : n;
  const float* pp = a.part + ((int64_t)wid * a.nsplit + s_first) * (D + 2);
  const int nact = n - s_first;
  const bool act = 2 * lane < D;
  float M = kNegBig;
  for (int s = lane; s < nact; s += 64) M = fmaxf(M, pp[s * (D + 2)]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  float lt = 0.f, o0 = 0.f, o1 = 0.f;
  for (int s0 = 0; s0 < nact; s0 += 64) {
    const int cnt = min(64, nact - s0);
    const float* ps = pp + (s0 + lane) * (D + 2);
    const float f = lane < cnt ? exp2_fast(ps[0] - M) : 0.f;
    if (lane < cnt) lt = fmaf(ps[1], f, lt);
#pragma unroll 4
    for (int s = 0; s < cnt; ++s) {
      const float fs = __shfl(f, s, 64);
      if (act) {
        const float2 v = *reinterpret_cast<const float2*>(pp + (s0 + s) * (D + 2) + 2 + 2 * lane);
        o0 = fmaf(v.x, fs, o0);
        o1 = fmaf(v.y, fs, o1);
      }
    }
  }
  lt = wave_sum(lt);
  const float inv = nact > 0 ? 1.f / lt : 0.f;
  if (act) {
    bf16x2 r;
    r[0] = to_bf16(o0 * inv);
    r[1] = to_bf16(o1 * inv);
    *reinterpret_cast<bf16x2*>(a.o + (int64_t)wid * D + 2 * lane) = r;
  }
}

template <int D, int HPB, int MODE>
hipError_t launch_split(const DecArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const dim3 grid((unsigned)a.nsplit, (unsigned)(a.B * a.Hkv * (G / HPB)));
  static const char* names[4] = {"decode_split_d32", "decode_split_d64", "decode_split_d96",
                                 "decode_split_d128"};
  TraceScope t(names[D / 32 - 1], s);
  hipLaunchKernelGGL((decode_split_kernel<D, HPB, MODE>), grid, dim3(64 * kDecWaves), 0, s, a);
  return hipGetLastError();
}

template <int D, int HPB>
hipError_t launch_split_mode(const DecArgs& a, int mode, hipStream_t s) {
  if (mode == kScoreScale) return launch_split<D, HPB, kScoreScale>(a, s);
  if (mode == kScoreCapPoly5) return launch_split<D, HPB, kScoreCapPoly5>(a, s);
  if (mode == kScoreCapPoly) return launch_split<D, HPB, kScoreCapPoly>(a, s);
  return launch_split<D, HPB, kScoreCapExp>(a, s);
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
  if (e != hipSuccess || a.nsplit == 1) return e;
  TraceScope t("decode_combine", s);
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)((a.B * a.Hq + 3) / 4)), dim3(256),
                     0, s, a);
  return hipGetLastError();
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
