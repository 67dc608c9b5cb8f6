// Single-token KV-cache decode on gfx950 ("GPT pretraining" page, section "Bonus: KV
// Caching": the new token's key and value are appended to the cache and its one query
// attends over the entire cached history; with offset = k_len - q_len = L - 1 every cached
// key is visible).  The nanoGPT-JAX 181M model card's inference notes ask that only the
// compact active part of the cache be attended; rows at or past cache_len[b] are never read.
//
// The work is HBM-bound (about 2 flops per byte), so it runs on the vector ALUs with
// coalesced 16-byte loads, not on MFMA:
//  * split kernel: one workgroup per (chunk of split_len keys, b, kv head, head subset).
//    Four lanes share one cache row (each owns D/4 elements, 64 contiguous bytes per load
//    instruction and quad), a wave covers 16 rows per step and the workgroup 64.  Each
//    quad keeps a running (max, sum, output) over its rows for every query head of the
//    GQA group, so K and V are streamed once per KV head.  The quads and waves are then
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
  bf16* o;
  float* part;
  int B, Hq, Hkv, Lmax, split_len, nsplit;
  float scale, cap_k1, cap_k2;  // cap_k1 = 2 log2(e) / c, cap_k2 = c log2(e)
  int rope;
  double log2_base;
  int qk_norm;
  float eps;
};

template <int D, int HPB, bool CAP>
__global__ __launch_bounds__(256) void decode_split_kernel(DecArgs a) {
  constexpr int NU = D / 32;  // 16-byte chunks per lane per row
  __shared__ float sq[HPB][D];
  __shared__ float sm[4][HPB], sl[4][HPB];
  __shared__ float so[4][HPB][D];

  const int G = a.Hq / a.Hkv;
  const int nsub = G / HPB;
  const int split = blockIdx.x;
  const int y = blockIdx.y;
  const int hs = y % nsub;
  const int bg = y / nsub;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int L = min(max(a.cache_len[b], 0), a.Lmax);
  const int start = split * a.split_len;
  if (start >= L) return;  // whole workgroup: this chunk holds no active row
  const int stop = min(L, start + a.split_len);
  const int h0 = g * G + hs * HPB;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  // Query prologue: wave hh rotates (position L - 1) and normalises head h0 + hh.
  if (w < HPB) {
    const int half = D / 2;
    const bool act = lane < half;
    const bf16* qr = a.q + ((int64_t)b * a.Hq + h0 + w) * D;
    float x1 = act ? from_bf16(qr[lane]) : 0.f;
    float x2 = act ? from_bf16(qr[lane + half]) : 0.f;
    if (a.rope && act) {
      float c, s;
      rope_cos_sin(L - 1, lane, D, a.log2_base, &c, &s);
      const float r1 = x1 * c - x2 * s, r2 = x1 * s + x2 * c;
      x1 = r1;
      x2 = r2;
    }
    if (a.qk_norm) {
      const float inv = 1.0f / sqrtf(wave_sum(x1 * x1 + x2 * x2) / (float)D + a.eps);
      x1 *= inv;
      x2 *= inv;
    }
    if (act) {
      sq[w][lane] = x1 * a.scale;
      sq[w][lane + half] = x2 * a.scale;
    }
  }
  __syncthreads();

  const int s4 = lane & 3;     // this lane's part of the row
  const int rq = lane >> 2;    // row within the wave's 16
  float qv[HPB][NU * 8];
#pragma unroll
  for (int hh = 0; hh < HPB; ++hh)
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[hh][8 * u + e] = sq[hh][32 * u + 8 * s4 + e];

  float m[HPB], ls[HPB], ov[HPB][NU * 8];
#pragma unroll
  for (int hh = 0; hh < HPB; ++hh) {
    m[hh] = kNegBig;
    ls[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < NU * 8; ++e) ov[hh][e] = 0.f;
  }

  const bf16* kb = a.kc + (int64_t)bg * a.Lmax * D + 8 * s4;
  const bf16* vb = a.vc + (int64_t)bg * a.Lmax * D + 8 * s4;
  for (int base = start; base < stop; base += 64) {
    const int j = base + 16 * w + rq;
    const bool valid = j < stop;
    bf16x8 kr[NU], vr[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      if (valid) {
        kr[u] = ld16<bf16x8>(kb + (int64_t)j * D + 32 * u);
        vr[u] = ld16<bf16x8>(vb + (int64_t)j * D + 32 * u);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kr[u][e] = (bf16)0.f;
          vr[u][e] = (bf16)0.f;
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < HPB; ++hh) {
      float dot = 0.f;
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) dot = fmaf(qv[hh][8 * u + e], (float)kr[u][e], dot);
      dot += __shfl_xor(dot, 1, 64);
      dot += __shfl_xor(dot, 2, 64);
      float yv;
      if constexpr (CAP) {
        const float ex = exp2_fast(dot * a.cap_k1);
        yv = a.cap_k2 * (1.f - 2.f * rcp_fast(ex + 1.f));
      } else {
        yv = dot * kLog2e;
      }
      const float m_new = valid ? fmaxf(m[hh], yv) : m[hh];
      const float alpha = exp2_fast(m[hh] - m_new);
      const float p = valid ? exp2_fast(yv - m_new) : 0.f;
      m[hh] = m_new;
      ls[hh] = ls[hh] * alpha + p;
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) ov[hh][8 * u + e] = fmaf(p, (float)vr[u][e], ov[hh][8 * u + e] * alpha);
    }
  }

  // Merge the 16 quads of the wave (lanes with the same s4).
#pragma unroll
  for (int off = 4; off < 64; off <<= 1) {
#pragma unroll
    for (int hh = 0; hh < HPB; ++hh) {
      const float mp = __shfl_xor(m[hh], off, 64);
      const float lp = __shfl_xor(ls[hh], off, 64);
      const float mn = fmaxf(m[hh], mp);
      const float fa = exp2_fast(m[hh] - mn), fb = exp2_fast(mp - mn);
      ls[hh] = ls[hh] * fa + lp * fb;
#pragma unroll
      for (int e = 0; e < NU * 8; ++e) {
        const float op = __shfl_xor(ov[hh][e], off, 64);
        ov[hh][e] = ov[hh][e] * fa + op * fb;
      }
      m[hh] = mn;
    }
  }
  if (lane < 4) {
#pragma unroll
    for (int hh = 0; hh < HPB; ++hh) {
      if (lane == 0) {
        sm[w][hh] = m[hh];
        sl[w][hh] = ls[hh];
      }
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) so[w][hh][32 * u + 8 * s4 + e] = ov[hh][8 * u + e];
    }
  }
  __syncthreads();
  // Merge the 4 waves and write this chunk's partial (m, l, o[D]) for each head.
  for (int t = tid; t < HPB * D; t += 256) {
    const int hh = t / D, d = t - hh * D;
    float M = sm[0][hh];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, sm[ww][hh]);
    float lt = 0.f, ot = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = exp2_fast(sm[ww][hh] - M);
      lt += sl[ww][hh] * f;
      ot += so[ww][hh][d] * f;
    }
    float* pp = a.part + (((int64_t)b * a.Hq + h0 + hh) * a.nsplit + split) * (D + 2);
    pp[2 + d] = ot;
    if (d == 0) {
      pp[0] = M;
      pp[1] = lt;
    }
  }
}

// One wave per (b, h); 4 per block.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecArgs a) {
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= a.B * a.Hq) return;
  const int lane = threadIdx.x & 63;
  const int b = wid / a.Hq;
  const int L = min(max(a.cache_len[b], 0), a.Lmax);
  const int n = (L + a.split_len - 1) / a.split_len;
  const float* pp = a.part + (int64_t)wid * a.nsplit * (D + 2);
  float M = kNegBig;
  for (int s = 0; s < n; ++s) M = fmaxf(M, pp[s * (D + 2)]);
  float lt = 0.f, o0 = 0.f, o1 = 0.f;
  for (int s = 0; s < n; ++s) {
    const float* ps = pp + s * (D + 2);
    const float f = exp2_fast(ps[0] - M);
    lt += ps[1] * f;
    if (lane < D) o0 += ps[2 + lane] * f;
    if (lane + 64 < D) o1 += ps[2 + lane + 64] * f;
  }
  const float inv = n > 0 ? 1.f / lt : 0.f;
  bf16* op = a.o + (int64_t)wid * D;
  if (lane < D) op[lane] = to_bf16(o0 * inv);
  if (lane + 64 < D) op[lane + 64] = to_bf16(o1 * inv);
}

template <int D, int HPB>
hipError_t launch_split(const DecArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const dim3 grid((unsigned)a.nsplit, (unsigned)(a.B * a.Hkv * (G / HPB)));
  static const char* names[4] = {"decode_split_d32", "decode_split_d64", "decode_split_d96",
                                 "decode_split_d128"};
  TraceScope t(names[D / 32 - 1], s);
  if (a.cap_k2 > 0.f)
    hipLaunchKernelGGL((decode_split_kernel<D, HPB, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, HPB, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  hipError_t e;
  if (G % 4 == 0)
    e = launch_split<D, 4>(a, s);
  else if (G % 3 == 0)
    e = launch_split<D, 3>(a, s);
  else if (G % 2 == 0)
    e = launch_split<D, 2>(a, s);
  else
    e = launch_split<D, 1>(a, s);
  if (e != hipSuccess) return e;
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
  a.o = (bf16*)p.o;
  a.part = p.part;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.Lmax = p.Lmax;
  a.split_len = p.split_len;
  a.nsplit = p.nsplit;
  a.scale = p.scale;
  const bool cap = p.softcap > 0.f;
  a.cap_k1 = cap ? 2.f * kLog2e / p.softcap : 0.f;
  a.cap_k2 = cap ? p.softcap * kLog2e : 0.f;
  a.rope = p.rope;
  a.log2_base = p.rope ? log2((double)p.rope_base) : 0.0;
  a.qk_norm = p.qk_norm;
  a.eps = p.eps;
  switch (p.D) {
    case 32: return launch_decode_d<32>(a, s);
    case 64: return launch_decode_d<64>(a, s);
    case 96: return launch_decode_d<96>(a, s);
    case 128: return launch_decode_d<128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace attn
