/*
 * attn.h -- C ABI of the MI355X (gfx950) causal self-attention library (libcausal_attn.so).
 *
 * What is computed.  For every batch b and query head h (KV head g = h / (Hq / Hkv),
 * contiguous groups -- grouped-query attention as on the nanoGPT-JAX 181M model card,
 * "Architecture": 8 query heads over 4 KV heads):
 *
 *     q^ = N(R(q)),  k^ = N(R(k))                     (prologue, each optional)
 *     S  = scale * q^ k^T                             (scale = 1/sqrt(D) by default)
 *     S  = c * tanh(S / c)                            (logit soft-cap, optional)
 *     S_ij = -inf unless j <= i and (W == 0 or i - j < W)
 *     O  = softmax_rows(S) V,   LSE_i = ln sum_j exp(S_ij)
 *
 * The definition softmax(Q K^T / sqrt(d_k)) V and the causal rule (future scores set to
 * -inf before the softmax) are those of the "GPT pretraining" page (llm_gpt_pretrain),
 * section "Multihead Attention"; heads are laid out [B, H, T, D] as that page's
 * _split_heads produces.  R is RoPE (pairs (x_i, x_{i+D/2}) rotated by p * base^(-2i/D)),
 * N the parameter-free RMSNorm x / sqrt(mean(x^2) + eps) -- both named on the nanoGPT-JAX
 * 181M model card ("Design choices worth naming") and on the flaxchat page ("Core
 * Features"), which also names the sliding window.  The KV-cache decode is the step of the
 * "Bonus: KV Caching" section of the GPT pretraining page: the newest token's key and value
 * are already stored at row L - 1 of its cache, and its query (position L - 1) is scored
 * against rows 0 .. L - 1; attn_extend is the same step for S new tokens, including storing
 * their keys and values.
 *
 * Conventions for every entry point below.
 *  - Pointers marked "device" are device memory owned by the caller; the library never
 *    allocates, frees or keeps them.  Tensors are dense and row-major in the stated shape.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the null stream).  No call
 *    synchronises the host.  Calls keep no state between them and may run concurrently on
 *    different streams with different buffers: with the kernel trace off (the default), a
 *    call reads one process-wide flag and writes no shared host or device state.
 *  - Argument errors are reported by a negative status BEFORE anything is enqueued.
 *    A failed launch is reported as ATTN_ELAUNCH.  Faults inside kernels surface at the
 *    caller's next synchronisation.
 *  - One element type (cfg->dtype) is used for q, k, v, o, dO, dq, dk, dv; LSE is always
 *    float32 natural-log, shape [B, Hq, T].
 */
#ifndef CAUSAL_ATTN_H
#define CAUSAL_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_EINVAL = -1,       /* a null pointer, a negative or inconsistent size, Hq % Hkv != 0 ... */
  ATTN_EUNSUPPORTED = -2, /* valid but not implemented: D not in {32,64,96,128}, fp32 backward ... */
  ATTN_EWORKSPACE = -3,   /* workspace missing or smaller than the *_workspace_bytes() figure   */
  ATTN_ELAUNCH = -4,      /* the HIP runtime refused a launch                                   */
  ATTN_ESCRATCH = -5      /* attn_decode_noalloc: the call needs more than its static scratch   */
} attn_status;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

/* Training forward/backward configuration. */
typedef struct {
  int32_t B, T;        /* batch, sequence length (>= 0; 0 means nothing to do)                 */
  int32_t Hq, Hkv;     /* query heads, KV heads; Hq % Hkv == 0                                  */
  int32_t D;           /* head dimension: 32, 64, 96 or 128                                     */
  int32_t window;      /* 0 = plain causal; W > 0: key j visible to query i iff i - W < j <= i  */
  float softcap;       /* 0 = off; c > 0: S <- c * tanh(S / c) on the scaled scores             */
  float scale;         /* 0 = 1/sqrt(D)                                                         */
  int32_t rope;        /* 1 = rotate q and k rows at positions 0..T-1                           */
  float rope_base;     /* RoPE base (10000 on the pages' models); > 0 when rope = 1             */
  int32_t qk_norm;     /* 1 = parameter-free RMSNorm of every q and k row (after RoPE)          */
  float norm_eps;      /* RMSNorm epsilon (> 0 when qk_norm = 1)                                */
  int32_t dtype;       /* attn_dtype: ATTN_BF16 for everything, ATTN_F32 for the forward only   */
} attn_cfg;

/* Single-token KV-cache decode configuration (bfloat16 only). */
typedef struct {
  int32_t B;           /* sequences (>= 0)                                                      */
  int32_t Hq, Hkv, D;  /* as in attn_cfg                                                        */
  int32_t Lmax;        /* allocated cache rows per (b, kv head), >= 0                           */
  float softcap;       /* as in attn_cfg                                                        */
  float scale;         /* 0 = 1/sqrt(D)                                                         */
  int32_t rope;        /* 1 = rotate the query at position cache_len[b] - 1                    */
  float rope_base;
  int32_t qk_norm;     /* 1 = RMSNorm the query (cached keys are stored already normalised)     */
  float norm_eps;
  int32_t split_len;   /* keys per split-K chunk: 0 = library default, else a multiple of 64    */
} attn_decode_cfg;

/* Multi-token step against a KV cache (bfloat16 only): append, then attend. */
typedef struct {
  int32_t B;           /* sequences (>= 0)                                                      */
  int32_t S;           /* new tokens per sequence (>= 0)                                        */
  int32_t Hq, Hkv, D;  /* as in attn_cfg                                                        */
  int32_t Lmax;        /* allocated cache rows per (b, kv head), >= 0                           */
  int32_t window;      /* 0 = plain causal; W > 0: key j visible to position p iff p - W < j    */
  float softcap;       /* as in attn_cfg                                                        */
  float scale;         /* 0 = 1/sqrt(D)                                                         */
  int32_t rope;        /* 1 = rotate the new queries and keys at their positions                */
  float rope_base;
  int32_t qk_norm;     /* 1 = RMSNorm the new queries and keys (cached keys are normalised)     */
  float norm_eps;
} attn_extend_cfg;

/* Bytes of device workspace that attn_fwd / attn_bwd / attn_decode need for this
 * configuration (0 if none).  Host-only; returns 0 for an invalid configuration.  The
 * split backward's (attn_bwd_split_workspace_bytes) adds the dS fragments its dK/dV pass
 * stores for the dQ pass: 1 KB per (32-query, 16-key) block in the causal / window band,
 * e.g. 545 MB at B = 16, T = 2048, 8 query heads. */
size_t attn_fwd_workspace_bytes(const attn_cfg* cfg);
size_t attn_bwd_workspace_bytes(const attn_cfg* cfg);
size_t attn_decode_workspace_bytes(const attn_decode_cfg* cfg);
/* The same for attn_fwd_packed / attn_bwd_packed (the plain figure plus 8 * B * T bytes, each
 * region 256-byte aligned). */
size_t attn_fwd_packed_workspace_bytes(const attn_cfg* cfg);
size_t attn_bwd_packed_workspace_bytes(const attn_cfg* cfg);
size_t attn_bwd_split_workspace_bytes(const attn_cfg* cfg);

/* Host-only validation of a configuration; the status attn_fwd would return for it
 * (before pointer and workspace checks).  for_backward = 1 applies the backward's rules. */
int attn_check_cfg(const attn_cfg* cfg, int for_backward);
int attn_check_decode_cfg(const attn_decode_cfg* cfg);
int attn_check_extend_cfg(const attn_extend_cfg* cfg);

/*
 * attn_fwd -- flash-style forward.
 *   q   [B, Hq,  T, D] device, dtype      k, v [B, Hkv, T, D] device, dtype
 *   o   [B, Hq,  T, D] device, dtype (written)
 *   lse [B, Hq,  T]    device, float32 natural-log log-sum-exp of each score row (written);
 *                      the backward consumes it.
 *   ws  device workspace of ws_bytes >= attn_fwd_workspace_bytes(cfg) (may be NULL if 0).
 * Returns ATTN_OK or a negative attn_status.
 */
int attn_fwd(const attn_cfg* cfg, const void* q, const void* k, const void* v, void* o,
             float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * attn_bwd -- gradients of sum(O * dO) with respect to the RAW q, k, v (before RoPE and
 * QK-norm).  bfloat16 only.  q, k, v, o, lse are exactly what attn_fwd consumed/produced.
 *   dO [B, Hq, T, D] device, bf16;  dq [B, Hq, T, D], dk, dv [B, Hkv, T, D] device, bf16
 *   (written; dk/dv hold the sums over each KV head's query group).
 *   ws device workspace of ws_bytes >= attn_bwd_workspace_bytes(cfg).
 * The result is deterministic (no atomics).
 */
int attn_bwd(const attn_cfg* cfg, const void* q, const void* k, const void* v, const void* o,
             const void* dO, const float* lse, void* dq, void* dk, void* dv, void* ws,
             size_t ws_bytes, void* stream);

/*
 * attn_bwd_split -- attn_bwd computed another way (same arguments, same results up to fp32
 * rounding order, deterministic): the dK/dV pass also stores dS (bf16, the value the dQ product
 * uses in attn_bwd as well) for every 32 x 16 (query, key) block of the mask's band, and dQ is
 * then a product of those blocks with k^, instead of a pass that recomputes S, P and dP per
 * query tile.  It moves about twice the backward's other HBM traffic through memory
 * (545 MB written and read at B = 16, T = 2048, 8 query heads) and measured slower than
 * attn_bwd on MI355X; it is kept as a checked alternative.  Workspace:
 * attn_bwd_split_workspace_bytes(cfg).  Plain rows without dropout only.
 */
int attn_bwd_split(const attn_cfg* cfg, const void* q, const void* k, const void* v,
                   const void* o, const void* dO, const float* lse, void* dq, void* dk, void* dv,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * attn_bwd_khat -- attn_bwd without its own pass over k: khat is k after RoPE / QK-norm,
 * bf16 [B, Hkv, T, D], exactly as the forward used it.  A bfloat16 attn_fwd with RoPE or
 * QK-norm on leaves it at the start of its workspace, so a caller that keeps that workspace
 * from the forward to the backward passes it here (every other argument as for attn_bwd).
 * With neither RoPE nor QK-norm khat is not read (k is used) and may be NULL.
 */
int attn_bwd_khat(const attn_cfg* cfg, const void* q, const void* k, const void* v,
                  const void* o, const void* dO, const float* lse, const void* khat, void* dq,
                  void* dk, void* dv, void* ws, size_t ws_bytes, void* stream);

/*
 * attn_fwd_packed, attn_bwd_packed -- attn_fwd / attn_bwd for rows that pack several
 * sequences (the nanoGPT-JAX 181M model card's SFT data: rows packed with segment ids).
 *   segment_ids [B, T] device, int32 -- a segment is a maximal run of equal ids in a row;
 *             token i attends to key j iff j <= i, j is in i's run (and i - j < W with a
 *             window).  Any id values are allowed; equal ids in separate runs are separate.
 * Every other argument is as for attn_fwd / attn_bwd (the backward consumes the packed
 * forward's o and lse); the workspaces are attn_fwd_packed_workspace_bytes /
 * attn_bwd_packed_workspace_bytes.  RoPE positions stay the row positions: scores see RoPE
 * only through position differences, so restarting them per run would change nothing.
 * Packed rows are bfloat16 only.  segment_ids may be NULL only when there is nothing to do.
 */
int attn_fwd_packed(const attn_cfg* cfg, const void* q, const void* k, const void* v,
                    const int32_t* segment_ids, void* o, float* lse, void* ws, size_t ws_bytes,
                    void* stream);
int attn_bwd_packed(const attn_cfg* cfg, const void* q, const void* k, const void* v,
                    const void* o, const void* dO, const float* lse, const int32_t* segment_ids,
                    void* dq, void* dk, void* dv, void* ws, size_t ws_bytes, void* stream);

/*
 * Attention dropout -- the "GPT pretraining" page, section "Multihead Attention", applies
 * dropout to the attention weights (after the softmax, before they multiply V; rate 0.1 in
 * its GPT configuration).  Inverted dropout: a weight is kept with probability 1 - p and
 * scaled by 1 / (1 - p), else zeroed.  The decision for query i, key j of head (b, h) takes
 * the 16-bit field j mod 16 of the Philox4x64-10 block (Salmon et al., "Parallel Random
 * Numbers: As Easy as 1, 2, 3", SC 2011) for counter (floor(j / 16), i, b * Hq + h, offset)
 * under key (seed, 0) -- field f is bits 16 (f mod 4) .. 16 (f mod 4) + 15 of output word
 * f / 4 -- and keeps the weight iff field >= t = round(65536 p).  The rate applied is
 * therefore t / 65536 and the scale 65536 / (65536 - t); p must satisfy 0 <= p and t < 65536.
 *
 * attn_dropout_mask_bytes -- size of the keep-mask buffer for cfg: two bit matrices of
 *   B * Hq * T rows of 2 * ceil(T / 64) 32-bit words (one row-major over keys, one over
 *   queries).  0 for an invalid configuration.
 * attn_dropout_mask -- fill `mask` (device, >= attn_dropout_mask_bytes(cfg) bytes, owned by
 *   the caller) with the keep bits of (p, seed, offset).  Only the words of 32 x 32 tiles that
 *   meet the causal / window band are written; the rest of the buffer is left as it was.
 *   A fresh (seed, offset) pair gives an independent mask.
 * attn_fwd_dropout, attn_bwd_dropout -- attn_fwd / attn_bwd with the weights multiplied by
 *   keep / (1 - rate): O = (P * Z) V, and the gradients of sum(O * dO) for that O.  `mask` is
 *   the buffer attn_dropout_mask filled for the same cfg and p (the backward must see the
 *   forward's mask); lse stays the log-sum-exp of the undropped scores.  Workspaces are those
 *   of attn_fwd / attn_bwd.  bfloat16 only; one run per row (no segment ids).
 */
size_t attn_dropout_mask_bytes(const attn_cfg* cfg);
int attn_dropout_mask(const attn_cfg* cfg, float p, uint64_t seed, uint64_t offset, void* mask,
                      size_t mask_bytes, void* stream);
int attn_fwd_dropout(const attn_cfg* cfg, const void* q, const void* k, const void* v, float p,
                     const void* mask, size_t mask_bytes, void* o, float* lse, void* ws,
                     size_t ws_bytes, void* stream);
int attn_bwd_dropout(const attn_cfg* cfg, const void* q, const void* k, const void* v,
                     const void* o, const void* dO, const float* lse, float p, const void* mask,
                     size_t mask_bytes, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * attn_decode -- one new query per sequence against its KV cache (split-K over the cache
 * length in chunks of cfg->split_len rows, then an LSE-weighted merge of a sequence's chunks
 * by the last of them to finish).  bfloat16 only.
 *   q         [B, Hq, D] device, bf16 -- raw (un-rotated) query of the newest token
 *   k_cache   [B, Hkv, Lmax, D] device, bf16 -- keys already rotated (and normalised when
 *             qk_norm = 1); the newest token's key is already appended
 *   v_cache   [B, Hkv, Lmax, D] device, bf16
 *   cache_len [B] device, int32 -- active rows L_b; only rows 0..L_b-1 are read.  Values
 *             are clamped to [0, Lmax] in the kernel; L_b = 0 yields a zero output row.
 *   o         [B, Hq, D] device, bf16 (written)
 *   ws        device workspace of ws_bytes >= attn_decode_workspace_bytes(cfg).  Its first
 *             attn_decode_ticket_bytes(cfg) bytes are ticket counters that must be ZERO before
 *             the workspace is first used (e.g. allocated zero-filled); every call leaves them
 *             zero again.  Calls that share a workspace must not overlap.
 */
size_t attn_decode_ticket_bytes(const attn_decode_cfg* cfg);
int attn_decode(const attn_decode_cfg* cfg, const void* q, const void* k_cache,
                const void* v_cache, const int32_t* cache_len, void* o, void* ws,
                size_t ws_bytes, void* stream);

/*
 * attn_decode_noalloc -- attn_decode for callers that cannot allocate device memory (code
 * recorded into a HIP graph, tight serving loops, harnesses that forbid allocation): the
 * workspace is a static device array of ATTN_DECODE_NOALLOC_MAX_BYTES per GPU, held until the
 * process ends, instead of a caller buffer.  Every other argument and rule is attn_decode's.
 * Configurations whose attn_decode_workspace_bytes exceeds that size return ATTN_ESCRATCH
 * before anything is enqueued.  The call allocates nothing (its first call on a device looks
 * up that device's copy of the array once).  All calls on one GPU share the array: calls that
 * overlap in time on one GPU (concurrent streams, or a graph replayed while another call
 * runs) race and must not be issued.  The current device must be the stream's device.
 */
#define ATTN_DECODE_NOALLOC_MAX_BYTES (8u << 20)
int attn_decode_noalloc(const attn_decode_cfg* cfg, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* cache_len, void* o, void* stream);

/*
 * attn_extend -- S new tokens per sequence against its KV cache (the multi-token form of the
 * step in the "Bonus: KV Caching" section of the GPT pretraining page).  New token i of
 * sequence b sits at position p = cache_len[b] + i: its key and value are stored at cache row
 * p, and its query is scored against cache rows j <= p.  With cache_len = 0 this is the
 * causal forward of the S tokens (prefill); with S = 1 it is attn_decode plus the store.
 * bfloat16 only; no workspace.
 *   q         [B, Hq, S, D] device, bf16 -- raw queries of the new tokens
 *   k_new, v_new [B, Hkv, S, D] device, bf16 -- raw keys and values of the new tokens
 *   k_cache, v_cache [B, Hkv, Lmax, D] device, bf16 -- rows < cache_len[b] hold the earlier
 *             tokens' keys (rotated, and normalised when qk_norm = 1) and values.  Rows
 *             cache_len[b] .. cache_len[b] + S - 1 are WRITTEN with the new tokens' keys
 *             (rotated at their positions, normalised) and values; no other row is touched.
 *   cache_len [B] device, int32 -- rows present before the call; not modified (the caller
 *             adds S).  Values are clamped to [0, Lmax] in the kernels.
 *   o         [B, Hq, S, D] device, bf16 (written) -- token i of sequence b sits at
 *             position p = cache_len[b] + i and attends over rows j <= p (and j > p - W for
 *             window = W > 0).  Tokens with p >= Lmax are neither stored nor attended:
 *             their output rows are zero.
 * q, k_new, v_new and o must not overlap the caches.
 */
int attn_extend(const attn_extend_cfg* cfg, const void* q, const void* k_new, const void* v_new,
                void* k_cache, void* v_cache, const int32_t* cache_len, void* o, void* stream);

/*
 * attn_decode_leftpad, attn_extend_leftpad -- attn_decode / attn_extend for left-padded
 * batches (the nanoGPT-JAX 181M model card's inference notes: left-padded prompts with
 * right-aligned generation through a KV cache, attending only the compact active slice).
 *   cache_start [B] device, int32 -- rows 0 .. cache_start[b] - 1 of sequence b's cache are
 *             padding: they are never read, and the token in row r sits at position
 *             r - cache_start[b] (keys stored by attn_extend_leftpad are rotated there; the
 *             decode query sits at position cache_len[b] - 1 - cache_start[b]).  Clamped in
 *             the kernels to [0, cache_len[b]] (decode) or [0, Lmax] (extend).
 * Decode attends rows cache_start[b] .. cache_len[b] - 1 (an empty range gives a zero row).
 * Extend attends rows cache_start[b] .. p for the token in row p; tokens whose row is below
 * cache_start[b] (padding, e.g. the pad tokens of a left-padded prompt prefilled with
 * cache_len = 0) are stored but their output rows are zero.  Every other argument and rule is
 * that of attn_decode / attn_extend; cache_start may be NULL only when there is nothing to do.
 */
int attn_decode_leftpad(const attn_decode_cfg* cfg, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* cache_start, const int32_t* cache_len,
                        void* o, void* ws, size_t ws_bytes, void* stream);
int attn_extend_leftpad(const attn_extend_cfg* cfg, const void* q, const void* k_new,
                        const void* v_new, void* k_cache, void* v_cache,
                        const int32_t* cache_start, const int32_t* cache_len, void* o,
                        void* stream);

/* Static, human-readable name of a status code. */
const char* attn_status_str(int status);

/*
 * attn_device_info -- host-only query of the figures a roofline needs, for HIP device
 * `device` (no allocation, nothing enqueued).  bf16_dense_tflops = compute_units * clock *
 * 4096 flops: gfx950's dense bf16 MFMA rate is 2048 multiply-adds per clock per compute unit.
 * The memory clock and bus width are reported as the runtime gives them.  Returns ATTN_OK,
 * ATTN_EINVAL for a null `out`, or ATTN_ELAUNCH if the runtime query fails.
 */
typedef struct {
  int32_t compute_units;
  int32_t clock_khz;       /* peak engine clock */
  int32_t mem_clock_khz;   /* peak memory clock */
  int32_t mem_bus_bits;    /* memory bus width */
  double bf16_dense_tflops;
} attn_device_info_t;

int attn_device_info(int device, attn_device_info_t* out);

/*
 * Kernel tracing (a measurement aid, off by default).  While enabled, every kernel the
 * library enqueues is bracketed by a pair of HIP events on its stream; attn_trace_read
 * synchronises those events and reports, per kernel name, the number of launches and
 * their summed device time.  The trace is the library's only process-wide state (a flag,
 * plus a mutex-guarded event list that only enabled tracing touches): enable/read/disable
 * from one thread while no other thread calls the library.
 */
typedef struct {
  char name[48];       /* kernel family, e.g. "fwd_bf16_d128"                                   */
  int64_t launches;    /* launches recorded since the last reset                                */
  double total_ms;     /* summed event-to-event time of those launches                          */
} attn_trace_entry;

int attn_trace_enable(int on);                       /* on = 1 starts (and clears), 0 stops    */
int attn_trace_read(attn_trace_entry* out, int max_entries);  /* returns the entry count (>= 0)
                                                                 or a negative attn_status     */

#ifdef __cplusplus
}
#endif

#endif /* CAUSAL_ATTN_H */
