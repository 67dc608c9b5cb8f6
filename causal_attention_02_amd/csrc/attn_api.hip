// C ABI of the attention library: argument validation, workspace layout, launch order and
// the optional kernel trace.  Nothing here allocates device memory or synchronises.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/attn.h"
#include "launch.h"

namespace attn {

// ---------------------------------------------------------------------------------------
// Kernel trace
// ---------------------------------------------------------------------------------------
namespace {
struct TraceRec {
  const char* name;
  hipEvent_t start, stop;
};
struct Tracer {
  std::mutex mu;
  bool on = false;  // guarded by mu
  std::vector<TraceRec> recs;
};
Tracer& tracer() {
  static Tracer t;
  return t;
}
// Read without a lock by every launch: while tracing is off (the default) a launch performs
// this one relaxed load and touches no other shared state.
std::atomic<bool> g_trace_on{false};
void trace_clear_locked(Tracer& t) {
  for (auto& r : t.recs) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  t.recs.clear();
}
}  // namespace

TraceScope::TraceScope(const char* name, hipStream_t s) : slot(-1), stream(s) {
  if (!g_trace_on.load(std::memory_order_relaxed)) return;
  Tracer& t = tracer();
  std::lock_guard<std::mutex> lk(t.mu);
  if (!t.on) return;
  TraceRec r{name, nullptr, nullptr};
  if (hipEventCreate(&r.start) != hipSuccess) return;
  if (hipEventCreate(&r.stop) != hipSuccess) {
    (void)hipEventDestroy(r.start);
    return;
  }
  (void)hipEventRecord(r.start, s);
  t.recs.push_back(r);
  slot = (int)t.recs.size() - 1;
}

TraceScope::~TraceScope() {
  if (slot < 0) return;
  Tracer& t = tracer();
  std::lock_guard<std::mutex> lk(t.mu);
  if (slot < (int)t.recs.size()) (void)hipEventRecord(t.recs[slot].stop, stream);
}

}  // namespace attn

using namespace attn;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool supported_d(int D) { return D == 32 || D == 64 || D == 96 || D == 128; }

int check_cfg(const attn_cfg* c, int bwd) {
  if (!c) return ATTN_EINVAL;
  if (c->B < 0 || c->T < 0 || c->Hq < 1 || c->Hkv < 1 || c->Hq % c->Hkv != 0) return ATTN_EINVAL;
  if (c->window < 0) return ATTN_EINVAL;
  if (!(c->softcap >= 0.f) || !isfinite(c->softcap)) return ATTN_EINVAL;
  if (!(c->scale >= 0.f) || !isfinite(c->scale)) return ATTN_EINVAL;
  if (c->rope != 0 && c->rope != 1) return ATTN_EINVAL;
  if (c->rope && (!(c->rope_base > 0.f) || !isfinite(c->rope_base))) return ATTN_EINVAL;
  if (c->qk_norm != 0 && c->qk_norm != 1) return ATTN_EINVAL;
  if (c->qk_norm && (!(c->norm_eps > 0.f) || !isfinite(c->norm_eps))) return ATTN_EINVAL;
  if (c->dtype != ATTN_F32 && c->dtype != ATTN_BF16) return ATTN_EINVAL;
  if (c->D <= 0) return ATTN_EINVAL;
  if (!supported_d(c->D)) return ATTN_EUNSUPPORTED;
  if (bwd && c->dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
  // Element offsets are 64-bit; row indices inside a (b, h) slice are 32-bit.
  if ((int64_t)c->T * c->D > INT32_MAX) return ATTN_EUNSUPPORTED;
  if ((int64_t)c->B * c->Hq > INT32_MAX / 64) return ATTN_EUNSUPPORTED;
  return ATTN_OK;
}

int check_dcfg(const attn_decode_cfg* c) {
  if (!c) return ATTN_EINVAL;
  if (c->B < 0 || c->Lmax < 0 || c->Hq < 1 || c->Hkv < 1 || c->Hq % c->Hkv != 0) return ATTN_EINVAL;
  if (!(c->softcap >= 0.f) || !isfinite(c->softcap)) return ATTN_EINVAL;
  if (!(c->scale >= 0.f) || !isfinite(c->scale)) return ATTN_EINVAL;
  if (c->rope != 0 && c->rope != 1) return ATTN_EINVAL;
  if (c->rope && (!(c->rope_base > 0.f) || !isfinite(c->rope_base))) return ATTN_EINVAL;
  if (c->qk_norm != 0 && c->qk_norm != 1) return ATTN_EINVAL;
  if (c->qk_norm && (!(c->norm_eps > 0.f) || !isfinite(c->norm_eps))) return ATTN_EINVAL;
  if (c->split_len < 0 || c->split_len % 64 != 0) return ATTN_EINVAL;
  if (c->D <= 0) return ATTN_EINVAL;
  if (!supported_d(c->D)) return ATTN_EUNSUPPORTED;
  if ((int64_t)c->Lmax * c->D > INT32_MAX) return ATTN_EUNSUPPORTED;
  if ((int64_t)c->B * c->Hkv * c->Hq > (int64_t)UINT16_MAX * 1024) return ATTN_EUNSUPPORTED;
  return ATTN_OK;
}

int check_ecfg(const attn_extend_cfg* c) {
  if (!c) return ATTN_EINVAL;
  if (c->B < 0 || c->S < 0 || c->Lmax < 0 || c->window < 0) return ATTN_EINVAL;
  if (c->Hq < 1 || c->Hkv < 1 || c->Hq % c->Hkv != 0) return ATTN_EINVAL;
  if (!(c->softcap >= 0.f) || !isfinite(c->softcap)) return ATTN_EINVAL;
  if (!(c->scale >= 0.f) || !isfinite(c->scale)) return ATTN_EINVAL;
  if (c->rope != 0 && c->rope != 1) return ATTN_EINVAL;
  if (c->rope && (!(c->rope_base > 0.f) || !isfinite(c->rope_base))) return ATTN_EINVAL;
  if (c->qk_norm != 0 && c->qk_norm != 1) return ATTN_EINVAL;
  if (c->qk_norm && (!(c->norm_eps > 0.f) || !isfinite(c->norm_eps))) return ATTN_EINVAL;
  if (c->D <= 0) return ATTN_EINVAL;
  if (!supported_d(c->D)) return ATTN_EUNSUPPORTED;
  if ((int64_t)c->Lmax * c->D > INT32_MAX || (int64_t)c->S * c->D > INT32_MAX)
    return ATTN_EUNSUPPORTED;
  // Forward grid: one workgroup per (128 new tokens, b, query head).
  if ((int64_t)((c->S + 127) / 128) * c->B * c->Hq > INT32_MAX) return ATTN_EUNSUPPORTED;
  return ATTN_OK;
}

float eff_scale(float scale, int D) { return scale > 0.f ? scale : 1.0f / sqrtf((float)D); }

// (b, kv head, head subset) units of a decode call: each owns one ticket counter.
long decode_units(const attn_decode_cfg* c) {
  return (long)c->B * c->Hkv * (c->Hq / c->Hkv / decode_heads_per_block(c->Hq / c->Hkv, c->D));
}

// Default chunking.  A batch whose units alone give a workgroup to every compute unit streams
// each cache in one chunk: every chunk pays the latency of its cache length and first rows
// before it streams, and measured at 64 sequences of U{256..2048} rows, any split (64 to 1024
// rows) was slower than none.  Smaller batches are cut into chunks (64 rows at least) so that
// full caches would give about four workgroups per compute unit.
int decode_split_len(const attn_decode_cfg* c) {
  if (c->split_len > 0) return c->split_len;
  const long units = decode_units(c);
  if (units >= 256 || c->Lmax <= 64) return c->Lmax > 0 ? (c->Lmax + 63) / 64 * 64 : 64;
  const long len = ((long)c->Lmax * units + 1023) / 1024;
  return (int)std::max(64L, (len + 63) / 64 * 64);
}

int decode_nsplit(const attn_decode_cfg* c) {
  const int sl = decode_split_len(c);
  return c->Lmax > 0 ? (c->Lmax + sl - 1) / sl : 1;
}

// The decode grid is one dimension of nsplit * units workgroups.
bool decode_grid_fits(const attn_decode_cfg* c) {
  return (int64_t)decode_nsplit(c) * decode_units(c) <= INT32_MAX;
}

// Workspace layouts (each region 256-byte aligned), when RoPE or QK-norm is on:
//   fwd bf16: [k^ B*Hkv*T*D bf16]       (q gets its prologue inside the forward kernel)
//   fwd f32:  [q^ B*Hq*T*D f32][k^ B*Hkv*T*D f32]
//   bwd:      [D B*Hq*T f32][LSE*log2e B*Hq*T f32][q^ bf16][k^ bf16]
//             (without RoPE/QK-norm only the two f32 rows)
size_t fwd_ws(const attn_cfg* c) {
  if (!(c->rope || c->qk_norm)) return 0;
  const size_t nq = (size_t)c->B * c->Hq * c->T * c->D, nk = (size_t)c->B * c->Hkv * c->T * c->D;
  if (c->dtype == ATTN_BF16) return align_up(nk * 2);
  return align_up(nq * 4) + align_up(nk * 4);
}

// Backward workspace without the dS fragments (packed rows and dropout recompute dS in the
// dq pass).
size_t bwd_ws_base(const attn_cfg* c) {
  const size_t rows = (size_t)c->B * c->Hq * c->T;
  size_t s = 2 * align_up(rows * 4);
  if (c->rope || c->qk_norm) {
    const size_t nq = rows * c->D, nk = (size_t)c->B * c->Hkv * c->T * c->D;
    s += align_up(nq * 2) + align_up(nk * 2);
  }
  return s;
}

size_t bwd_ws(const attn_cfg* c) { return bwd_ws_base(c); }

// Split backward (attn_bwd_split): the base regions, then the dS fragments (bf16, the band of
// the causal / window mask, 1 KB per 32 x 16 block).
size_t ds_bytes(const attn_cfg* c) {
  return align_up((size_t)c->B * c->Hq * (size_t)make_ds_band(c->T, c->window).frags * 1024);
}
size_t bwd_split_ws(const attn_cfg* c) { return bwd_ws_base(c) + ds_bytes(c); }

// Packed rows: run starts and ends, [B, T] int32 each.
size_t seg_ws(const attn_cfg* c) { return 2 * align_up((size_t)c->B * c->T * 4); }

// Dropout keep masks: row layout then column layout, B * Hq * T rows of dropout_pitch(T)
// words each.
size_t drop_half(const attn_cfg* c) {
  return align_up((size_t)c->B * c->Hq * c->T * dropout_pitch(c->T) * 4);
}
size_t drop_bytes(const attn_cfg* c) { return 2 * drop_half(c); }

// 16-bit keep threshold round(65536 p) and the kept-weight scale, or false if p is out of range.
bool drop_params(float p, uint32_t* thr, float* scale) {
  if (!(p >= 0.f) || !isfinite(p)) return false;
  const double t = floor((double)p * 65536.0 + 0.5);
  if (t >= 65536.0) return false;
  *thr = (uint32_t)t;
  *scale = (float)(65536.0 / (65536.0 - t));
  return true;
}

// Decode workspace: [tickets: one uint32 per unit][partials B*Hq*nsplit*(D+2) f32].  The
// ticket region must hold zeros before the first call; every call leaves it zero.
size_t dec_count_bytes(const attn_decode_cfg* c) { return align_up((size_t)decode_units(c) * 4); }
size_t dec_ws(const attn_decode_cfg* c) {
  return dec_count_bytes(c) + align_up((size_t)c->B * c->Hq * decode_nsplit(c) * (c->D + 2) * 4);
}

int launch_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ELAUNCH; }

}  // namespace

extern "C" {

const char* attn_status_str(int s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_EINVAL: return "invalid argument";
    case ATTN_EUNSUPPORTED: return "unsupported configuration";
    case ATTN_EWORKSPACE: return "workspace missing or too small";
    case ATTN_ELAUNCH: return "kernel launch failed";
    case ATTN_ESCRATCH: return "needs more than the static decode scratch";
  }
  return "unknown status";
}

int attn_check_cfg(const attn_cfg* cfg, int for_backward) { return check_cfg(cfg, for_backward); }
int attn_check_decode_cfg(const attn_decode_cfg* cfg) { return check_dcfg(cfg); }
int attn_check_extend_cfg(const attn_extend_cfg* cfg) { return check_ecfg(cfg); }

size_t attn_fwd_workspace_bytes(const attn_cfg* cfg) {
  return check_cfg(cfg, 0) == ATTN_OK ? fwd_ws(cfg) : 0;
}
size_t attn_bwd_workspace_bytes(const attn_cfg* cfg) {
  return check_cfg(cfg, 1) == ATTN_OK ? bwd_ws(cfg) : 0;
}
size_t attn_fwd_packed_workspace_bytes(const attn_cfg* cfg) {
  return check_cfg(cfg, 0) == ATTN_OK ? fwd_ws(cfg) + seg_ws(cfg) : 0;
}
size_t attn_bwd_packed_workspace_bytes(const attn_cfg* cfg) {
  return check_cfg(cfg, 1) == ATTN_OK ? bwd_ws_base(cfg) + seg_ws(cfg) : 0;
}
size_t attn_bwd_split_workspace_bytes(const attn_cfg* cfg) {
  return check_cfg(cfg, 1) == ATTN_OK ? bwd_split_ws(cfg) : 0;
}
size_t attn_decode_workspace_bytes(const attn_decode_cfg* cfg) {
  return check_dcfg(cfg) == ATTN_OK ? dec_ws(cfg) : 0;
}
size_t attn_decode_ticket_bytes(const attn_decode_cfg* cfg) {
  return check_dcfg(cfg) == ATTN_OK ? dec_count_bytes(cfg) : 0;
}

// Forward and backward bodies; `ids` (segment ids [B, T], or null) selects packed rows, whose
// run starts (and ends) go to a region after the plain workspace.
// Dropout: `drop` points to a keep-mask buffer (row layout, then column layout) and dscale
// is the kept-weight scale.
static int fwd_impl(const attn_cfg* c, const void* q, const void* k, const void* v,
                    const int32_t* ids, void* o, float* lse, void* ws, size_t ws_bytes,
                    void* stream, const void* drop = nullptr, float dscale = 1.f) {
  int st = check_cfg(c, 0);
  if (st != ATTN_OK) return st;
  if ((ids || drop) && c->dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
  if (c->B == 0 || c->T == 0) return ATTN_OK;
  if (!q || !k || !v || !o || !lse) return ATTN_EINVAL;
  const size_t need = fwd_ws(c) + (ids ? seg_ws(c) : 0);
  if (need > 0 && (!ws || ws_bytes < need)) return ATTN_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const bool pro = c->rope || c->qk_norm;
  const int64_t qrows = (int64_t)c->B * c->Hq * c->T, krows = (int64_t)c->B * c->Hkv * c->T;
  FwdParams p{q, k, v, o, lse, c->B, c->T, c->Hq, c->Hkv, c->D, c->window,
              eff_scale(c->scale, c->D), c->softcap, c->rope, c->rope_base, c->qk_norm,
              c->norm_eps};
  p.drop_rows = (const uint32_t*)drop;
  p.drop_scale = dscale;
  hipError_t e = hipSuccess;
  if (ids) {
    int32_t* sst = (int32_t*)((char*)ws + fwd_ws(c));
    int32_t* sen = (int32_t*)((char*)sst + align_up((size_t)c->B * c->T * 4));
    e = launch_segment_bounds(ids, sst, sen, c->B, c->T, s);
    p.seg_start = sst;
  }
  if (e == hipSuccess && c->dtype == ATTN_BF16) {
    if (pro) {
      e = launch_prologue(k, ws, krows, c->T, c->D, 2, c->rope, c->rope_base, c->qk_norm,
                          c->norm_eps, s);
      p.k = ws;
    }
    if (e == hipSuccess) e = launch_fwd_bf16(p, s);
  } else if (e == hipSuccess) {
    if (pro) {
      char* w = (char*)ws;
      void* kw = w + align_up((size_t)qrows * c->D * 4);
      e = launch_prologue(q, w, qrows, c->T, c->D, 4, c->rope, c->rope_base, c->qk_norm,
                          c->norm_eps, s);
      if (e == hipSuccess)
        e = launch_prologue(k, kw, krows, c->T, c->D, 4, c->rope, c->rope_base, c->qk_norm,
                            c->norm_eps, s);
      p.q = w;
      p.k = kw;
    }
    if (e == hipSuccess) e = launch_fwd_f32(p, s);
  }
  return launch_status(e);
}

// khat: k after RoPE / QK-norm as the forward used it (null: computed here).
// split: the split backward (dS stored by the dK/dV pass, dQ from it); plain rows, no dropout.
static int bwd_impl(const attn_cfg* c, const void* q, const void* k, const void* v,
                    const void* o, const void* dO, const float* lse, const int32_t* ids,
                    void* dq, void* dk, void* dv, void* ws, size_t ws_bytes, void* stream,
                    const void* drop = nullptr, float dscale = 1.f,
                    const void* khat = nullptr, bool split = false) {
  int st = check_cfg(c, 1);
  if (st != ATTN_OK) return st;
  if (c->B == 0 || c->T == 0) return ATTN_OK;
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return ATTN_EINVAL;
  const size_t need = split ? bwd_split_ws(c) : ids ? bwd_ws(c) + seg_ws(c) : bwd_ws(c);
  if (!ws || ws_bytes < need) return ATTN_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int64_t qrows = (int64_t)c->B * c->Hq * c->T, krows = (int64_t)c->B * c->Hkv * c->T;
  char* w = (char*)ws;
  float* Dvec = (float*)w;
  w += align_up((size_t)qrows * 4);
  float* L2 = (float*)w;
  w += align_up((size_t)qrows * 4);
  const bool pro = c->rope || c->qk_norm;
  void* qh = const_cast<void*>(q);
  const void* kh = k;
  hipError_t e = hipSuccess;
  if (pro) {
    qh = w;
    w += align_up((size_t)qrows * c->D * 2);
    if (khat) {
      kh = khat;
    } else {
      void* kw = w;
      e = launch_prologue(k, kw, krows, c->T, c->D, 2, c->rope, c->rope_base, c->qk_norm,
                          c->norm_eps, s);
      kh = kw;
    }
  }
  BwdParams p{q, k, kh, qh, v, o, dO, lse, Dvec, L2, dq, dk, dv, c->B, c->T, c->Hq, c->Hkv, c->D,
              c->window, eff_scale(c->scale, c->D), c->softcap, c->rope, c->rope_base,
              c->qk_norm, c->norm_eps};
  if (drop) {
    p.drop_rows = (const uint32_t*)drop;
    p.drop_cols = (const uint32_t*)((const char*)drop + drop_half(c));
    p.drop_scale = dscale;
  }
  if (ids && e == hipSuccess) {
    int32_t* sst = (int32_t*)((char*)ws + bwd_ws(c));
    int32_t* sen = (int32_t*)((char*)sst + align_up((size_t)c->B * c->T * 4));
    e = launch_segment_bounds(ids, sst, sen, c->B, c->T, s);
    p.seg_start = sst;
    p.seg_end = sen;
  }
  if (split) {
    // -D, LSE log2(e) and q^ in one pass; dK, dV with dS stored as fragments; dQ from them.
    p.ds = (char*)ws + bwd_ws_base(c);
    p.band = make_ds_band(c->T, c->window);
    if (e == hipSuccess)
      e = launch_bwd_prep(q, o, dO, lse, pro ? qh : nullptr, Dvec, L2, qrows, c->T, c->D, c->rope,
                          c->rope_base, c->qk_norm, c->norm_eps, s);
    if (e == hipSuccess) e = launch_bwd_dkdv(p, s);
    if (e == hipSuccess) e = launch_bwd_dq_ds(p, s);
    return launch_status(e);
  }
  if (e == hipSuccess) e = launch_bwd_dq(p, s);
  if (e == hipSuccess) e = launch_bwd_dkdv(p, s);
  return launch_status(e);
}

int attn_fwd(const attn_cfg* c, const void* q, const void* k, const void* v, void* o, float* lse,
             void* ws, size_t ws_bytes, void* stream) {
  return fwd_impl(c, q, k, v, nullptr, o, lse, ws, ws_bytes, stream);
}

int attn_bwd(const attn_cfg* c, const void* q, const void* k, const void* v, const void* o,
             const void* dO, const float* lse, void* dq, void* dk, void* dv, void* ws,
             size_t ws_bytes, void* stream) {
  return bwd_impl(c, q, k, v, o, dO, lse, nullptr, dq, dk, dv, ws, ws_bytes, stream);
}

int attn_bwd_khat(const attn_cfg* c, const void* q, const void* k, const void* v, const void* o,
                  const void* dO, const float* lse, const void* khat, void* dq, void* dk,
                  void* dv, void* ws, size_t ws_bytes, void* stream) {
  if (c && (c->rope || c->qk_norm) && c->B > 0 && c->T > 0 && !khat) return ATTN_EINVAL;
  return bwd_impl(c, q, k, v, o, dO, lse, nullptr, dq, dk, dv, ws, ws_bytes, stream, nullptr,
                  1.f, khat);
}

int attn_bwd_split(const attn_cfg* c, const void* q, const void* k, const void* v, const void* o,
                   const void* dO, const float* lse, void* dq, void* dk, void* dv, void* ws,
                   size_t ws_bytes, void* stream) {
  return bwd_impl(c, q, k, v, o, dO, lse, nullptr, dq, dk, dv, ws, ws_bytes, stream, nullptr,
                  1.f, nullptr, true);
}

int attn_fwd_packed(const attn_cfg* c, const void* q, const void* k, const void* v,
                    const int32_t* segment_ids, void* o, float* lse, void* ws, size_t ws_bytes,
                    void* stream) {
  if (!segment_ids && c && c->B > 0 && c->T > 0) return ATTN_EINVAL;
  return fwd_impl(c, q, k, v, segment_ids, o, lse, ws, ws_bytes, stream);
}

int attn_bwd_packed(const attn_cfg* c, const void* q, const void* k, const void* v,
                    const void* o, const void* dO, const float* lse, const int32_t* segment_ids,
                    void* dq, void* dk, void* dv, void* ws, size_t ws_bytes, void* stream) {
  if (!segment_ids && c && c->B > 0 && c->T > 0) return ATTN_EINVAL;
  return bwd_impl(c, q, k, v, o, dO, lse, segment_ids, dq, dk, dv, ws, ws_bytes, stream);
}

size_t attn_dropout_mask_bytes(const attn_cfg* cfg) {
  return check_cfg(cfg, 0) == ATTN_OK ? drop_bytes(cfg) : 0;
}

int attn_dropout_mask(const attn_cfg* c, float p, uint64_t seed, uint64_t offset, void* mask,
                      size_t mask_bytes, void* stream) {
  int st = check_cfg(c, 0);
  if (st != ATTN_OK) return st;
  uint32_t thr;
  float scale;
  if (!drop_params(p, &thr, &scale)) return ATTN_EINVAL;
  if (c->B == 0 || c->T == 0) return ATTN_OK;
  if (!mask || mask_bytes < drop_bytes(c)) return ATTN_EINVAL;
  uint32_t* rows = (uint32_t*)mask;
  uint32_t* cols = (uint32_t*)((char*)mask + drop_half(c));
  return launch_status(launch_dropout_mask(rows, cols, c->B, c->Hq, c->T, c->window, thr, seed,
                                           offset, (hipStream_t)stream));
}

int attn_fwd_dropout(const attn_cfg* c, const void* q, const void* k, const void* v, float p,
                     const void* mask, size_t mask_bytes, void* o, float* lse, void* ws,
                     size_t ws_bytes, void* stream) {
  int st = check_cfg(c, 0);
  if (st != ATTN_OK) return st;
  uint32_t thr;
  float scale;
  if (!drop_params(p, &thr, &scale)) return ATTN_EINVAL;
  if (c->dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
  if (c->B == 0 || c->T == 0) return ATTN_OK;
  if (!mask || mask_bytes < drop_bytes(c)) return ATTN_EINVAL;
  return fwd_impl(c, q, k, v, nullptr, o, lse, ws, ws_bytes, stream, mask, scale);
}

int attn_bwd_dropout(const attn_cfg* c, const void* q, const void* k, const void* v,
                     const void* o, const void* dO, const float* lse, float p, const void* mask,
                     size_t mask_bytes, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                     void* stream) {
  int st = check_cfg(c, 1);
  if (st != ATTN_OK) return st;
  uint32_t thr;
  float scale;
  if (!drop_params(p, &thr, &scale)) return ATTN_EINVAL;
  if (c->B == 0 || c->T == 0) return ATTN_OK;
  if (!mask || mask_bytes < drop_bytes(c)) return ATTN_EINVAL;
  return bwd_impl(c, q, k, v, o, dO, lse, nullptr, dq, dk, dv, ws, ws_bytes, stream, mask, scale);
}

// Decode and extend bodies; `start` (left padding rows per sequence, device int32 [B]) may be
// null.
static int decode_impl(const attn_decode_cfg* c, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* start, const int32_t* cache_len,
                       void* o, void* ws, size_t ws_bytes, void* stream) {
  int st = check_dcfg(c);
  if (st != ATTN_OK) return st;
  if (c->B == 0) return ATTN_OK;
  if (!q || !o || !cache_len) return ATTN_EINVAL;
  if (c->Lmax > 0 && (!k_cache || !v_cache)) return ATTN_EINVAL;
  if (!decode_grid_fits(c)) return ATTN_EUNSUPPORTED;
  const size_t need = dec_ws(c);
  if (!ws || ws_bytes < need) return ATTN_EWORKSPACE;
  DecodeParams p{q, k_cache, v_cache, cache_len, start, o,
                 (float*)((char*)ws + dec_count_bytes(c)), (unsigned*)ws, c->B, c->Hq, c->Hkv,
                 c->D, c->Lmax, decode_split_len(c), decode_nsplit(c),
                 eff_scale(c->scale, c->D), c->softcap, c->rope, c->rope_base, c->qk_norm,
                 c->norm_eps};
  return launch_status(launch_decode(p, (hipStream_t)stream));
}

static int extend_impl(const attn_extend_cfg* c, const void* q, const void* k_new,
                       const void* v_new, void* k_cache, void* v_cache, const int32_t* start,
                       const int32_t* cache_len, void* o, void* stream) {
  int st = check_ecfg(c);
  if (st != ATTN_OK) return st;
  if (c->B == 0 || c->S == 0) return ATTN_OK;
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !cache_len || !o) return ATTN_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  // 1. Store the new tokens' keys (RoPE at their positions, QK-norm) and values.
  hipError_t e = launch_append_kv(k_new, v_new, k_cache, v_cache, cache_len, start, c->B, c->Hkv,
                                  c->S, c->Lmax, c->D, c->rope, c->rope_base, c->qk_norm,
                                  c->norm_eps, s);
  // 2. The forward kernel in cache mode: queries at rows cache_len[b] + i over the cache.
  if (e == hipSuccess) {
    FwdParams p{q, k_cache, v_cache, o, nullptr, c->B, c->S, c->Hq, c->Hkv, c->D, c->window,
                eff_scale(c->scale, c->D), c->softcap, c->rope, c->rope_base, c->qk_norm,
                c->norm_eps};
    p.cache_len = cache_len;
    p.cache_start = start;
    p.Lmax = c->Lmax;
    e = launch_fwd_bf16(p, s);
  }
  return launch_status(e);
}

int attn_decode(const attn_decode_cfg* c, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* cache_len, void* o, void* ws, size_t ws_bytes, void* stream) {
  return decode_impl(c, q, k_cache, v_cache, nullptr, cache_len, o, ws, ws_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------------------
// Allocation-free decode: the workspace is a statically sized device array.  The loader
// zero-fills it, and every call leaves its ticket region zero again, so it starts each call
// as attn_decode requires.  In host code `scratch` only names the symbol; its device address
// is looked up once per device (hipGetSymbolAddress, with that device current) and only that
// address is passed to kernels.
// ---------------------------------------------------------------------------------------
namespace {
constexpr int kScratchDevices = 64;
static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_NOALLOC_MAX_BYTES];
std::once_flag g_scratch_once[kScratchDevices];
void* g_scratch_ptr[kScratchDevices];
hipError_t g_scratch_err[kScratchDevices];

// This device's copy of `scratch` (null with the runtime's error when the lookup failed).
void* scratch_for_device(int dev, hipError_t* err) {
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_err[dev] = e;
    g_scratch_ptr[dev] = e == hipSuccess ? p : nullptr;
  });
  *err = g_scratch_err[dev];
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

int attn_decode_noalloc(const attn_decode_cfg* c, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* cache_len, void* o, void* stream) {
  const int st = check_dcfg(c);
  if (st != ATTN_OK) return st;
  if (c->B == 0) return ATTN_OK;
  if (dec_ws(c) > (size_t)ATTN_DECODE_NOALLOC_MAX_BYTES) return ATTN_ESCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_ELAUNCH;
  if (dev >= kScratchDevices) return ATTN_EUNSUPPORTED;
  hipError_t e = hipSuccess;
  void* ws = scratch_for_device(dev, &e);
  if (!ws) return ATTN_ELAUNCH;
  return decode_impl(c, q, k_cache, v_cache, nullptr, cache_len, o, ws,
                     (size_t)ATTN_DECODE_NOALLOC_MAX_BYTES, stream);
}

int attn_decode_leftpad(const attn_decode_cfg* c, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* cache_start, const int32_t* cache_len,
                        void* o, void* ws, size_t ws_bytes, void* stream) {
  if (!cache_start && c && c->B > 0) return ATTN_EINVAL;
  return decode_impl(c, q, k_cache, v_cache, cache_start, cache_len, o, ws, ws_bytes, stream);
}

int attn_extend(const attn_extend_cfg* c, const void* q, const void* k_new, const void* v_new,
                void* k_cache, void* v_cache, const int32_t* cache_len, void* o, void* stream) {
  return extend_impl(c, q, k_new, v_new, k_cache, v_cache, nullptr, cache_len, o, stream);
}

int attn_extend_leftpad(const attn_extend_cfg* c, const void* q, const void* k_new,
                        const void* v_new, void* k_cache, void* v_cache,
                        const int32_t* cache_start, const int32_t* cache_len, void* o,
                        void* stream) {
  if (!cache_start && c && c->B > 0 && c->S > 0) return ATTN_EINVAL;
  return extend_impl(c, q, k_new, v_new, k_cache, v_cache, cache_start, cache_len, o, stream);
}

int attn_device_info(int device, attn_device_info_t* out) {
  if (!out) return ATTN_EINVAL;
  int cu = 0, clk = 0, mclk = 0, bus = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      hipDeviceGetAttribute(&clk, hipDeviceAttributeClockRate, device) != hipSuccess ||
      hipDeviceGetAttribute(&mclk, hipDeviceAttributeMemoryClockRate, device) != hipSuccess ||
      hipDeviceGetAttribute(&bus, hipDeviceAttributeMemoryBusWidth, device) != hipSuccess)
    return ATTN_ELAUNCH;
  out->compute_units = cu;
  out->clock_khz = clk;
  out->mem_clock_khz = mclk;
  out->mem_bus_bits = bus;
  out->bf16_dense_tflops = (double)cu * 4096.0 * clk * 1e3 / 1e12;
  return ATTN_OK;
}

int attn_trace_enable(int on) {
  Tracer& t = tracer();
  std::lock_guard<std::mutex> lk(t.mu);
  if (on) trace_clear_locked(t);
  t.on = on != 0;
  g_trace_on.store(t.on, std::memory_order_relaxed);
  return ATTN_OK;
}

int attn_trace_read(attn_trace_entry* out, int max_entries) {
  if (max_entries < 0 || (max_entries > 0 && !out)) return ATTN_EINVAL;
  Tracer& t = tracer();
  std::lock_guard<std::mutex> lk(t.mu);
  std::vector<attn_trace_entry> agg;
  for (auto& r : t.recs) {
    if (hipEventSynchronize(r.stop) != hipSuccess) return ATTN_ELAUNCH;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return ATTN_ELAUNCH;
    attn_trace_entry* e = nullptr;
    for (auto& x : agg)
      if (strncmp(x.name, r.name, sizeof(x.name)) == 0) e = &x;
    if (!e) {
      attn_trace_entry n;
      memset(&n, 0, sizeof(n));
      strncpy(n.name, r.name, sizeof(n.name) - 1);
      agg.push_back(n);
      e = &agg.back();
    }
    e->launches += 1;
    e->total_ms += ms;
  }
  const int n = (int)agg.size();
  for (int i = 0; i < n && i < max_entries; ++i) out[i] = agg[i];
  return n;
}

}  // extern "C"
