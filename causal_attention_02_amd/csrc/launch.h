// Host-side interface between the C ABI (attn_api.hip) and the kernel files.
// Every launcher enqueues on the given stream and returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// Kernel tracing: brackets each launch by a pair of events while enabled.
struct TraceScope {
  TraceScope(const char* name, hipStream_t stream);
  ~TraceScope();
  int slot;
  hipStream_t stream;
};

// ---- prologue / epilogue / row reductions (rowops.hip) ----------------------------------
// y = N(R(x)) for rows of length D; row r sits at position r % T.  elt = 2 (bf16) or 4 (f32).
hipError_t launch_prologue(const void* x, void* y, int64_t rows, int T, int D, int elt, int rope,
                           float rope_base, int qk_norm, float eps, hipStream_t s);
// dx = R^T(N'(dyhat)) from the fp32 gradient dyhat and the raw bf16 row x.
hipError_t launch_epilogue(const float* dyhat, const void* x, void* dx, int64_t rows, int T, int D,
                           int rope, float rope_base, int qk_norm, float eps, hipStream_t s);
// Dvec[r] = sum_d dO[r, d] * O[r, d]   (bf16 rows)
hipError_t launch_rowdot(const void* dO, const void* O, float* Dvec, int64_t rows, int D,
                         hipStream_t s);

// ---- forward (fwd.hip) -------------------------------------------------------------------
struct FwdParams {
  const void* q;  // [B, Hq, T, D]
  const void* k;  // [B, Hkv, T, D]
  const void* v;
  void* o;
  float* lse;
  int B, T, Hq, Hkv, D, window;
  float scale, softcap;
};
hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t s);
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t s);

// ---- backward (bwd.hip) ------------------------------------------------------------------
struct BwdParams {
  const void* q;     // Q^ (bf16) [B, Hq, T, D]
  const void* k;     // K^ (bf16) [B, Hkv, T, D]
  const void* v;
  const void* dO;
  const float* lse;  // [B, Hq, T]
  const float* Dvec; // [B, Hq, T]
  void* dq;          // bf16, or fp32 when grad_f32
  void* dk;          // bf16, or fp32 when grad_f32
  void* dv;          // bf16
  int grad_f32;
  int B, T, Hq, Hkv, D, window;
  float scale, softcap;
};
hipError_t launch_bwd_dq(const BwdParams& p, hipStream_t s);
hipError_t launch_bwd_dkdv(const BwdParams& p, hipStream_t s);

// ---- decode (decode.hip) -----------------------------------------------------------------
struct DecodeParams {
  const void* q;        // [B, Hq, D]
  const void* kc;       // [B, Hkv, Lmax, D]
  const void* vc;
  const int32_t* cache_len;
  void* o;              // [B, Hq, D]
  float* part;          // [B, Hq, nsplit, D + 2]
  int B, Hq, Hkv, D, Lmax, split_len, nsplit;
  float scale, softcap;
  int rope;
  float rope_base;
  int qk_norm;
  float eps;
};
hipError_t launch_decode(const DecodeParams& p, hipStream_t s);

}  // namespace attn
