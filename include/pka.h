/*
 * pka.h -- prefix-KV chunk attention for context-frozen training (MI355X, gfx950).
 *
 * The method (pages cited by title and section):
 *  - "Context-Frozen Training", The Solution: a no-grad forward of the context builds
 *    its KV cache (Phase 1); the decision tokens then run forward and backward against
 *    that frozen cache (Phase 2); gradients flow through the decision tokens only.
 *  - "train: walk the window" (llama.cpp), What it is / Contents: a window is trained
 *    one chunk at a time; each chunk reads the earlier tokens from a KV cache that is
 *    held fixed (F16 or q8_0 storage), and after its step the chunk's own K/V are
 *    written into that cache for the chunks after it. Approval comment: V is kept in
 *    token-major order, not transposed, which is what lets it be block-quantised, and
 *    the storage type is whatever the serving side uses, so here it is an argument.
 *  - "stop-gradient through context tokens" (prime-rl), Known gaps: an attention
 *    backward that produces gradient for the kept (chunk) queries only.
 *
 * Shapes: B windows, Hq query heads, Hkv KV heads (G = Hq/Hkv query heads share KV
 * head h/G), head_dim D, prefix (cached context) length P, chunk length C. Chunk
 * query i (token P+i of the window) attends to prefix keys 0..P-1 and chunk keys
 * 0..i (causal attention offset by P). The prefix gets no gradient: it is a constant.
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library
 *    allocates nothing and keeps no state between calls, except the opt-in
 *    profiling counters at the end of this file and the fixed per-GPU device array
 *    that pka_chunk_attn_bwd_noalloc uses as its workspace.
 *  - Layouts are dense row-major with the innermost dimension contiguous:
 *      q, o, dO, dq        bf16 [B][Hq][C][D]
 *      k, v, dk, dv        bf16 [B][Hkv][C][D]     (the chunk's own keys/values)
 *      lse, delta          f32  [B][Hq][C]
 *      cache k, v          F16/BF16: u16 [B][Hkv][capacity][D]
 *                          Q8_0:     int8 [B][Hkv][capacity][D]
 *      cache k/v scales    Q8_0 only: f16 [B][Hkv][capacity][D/32]
 *    Every base pointer must be 16-byte aligned.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null stream)
 *    and never synchronises the host.
 *  - Arguments are validated on the host before any HIP call; on failure nothing is
 *    launched and a non-zero pka_status is returned (never an abort or exception),
 *    mirroring the walk's failure exit in "train: walk the window" (rebase comment:
 *    a failed chunk step returns false, like a refused graph). A launch failure
 *    returns PKA_ERR_HIP. pka_last_error() gives a message for the calling thread.
 *  - Calls that overlap on one stream are ordered; calls on different streams that
 *    share output buffers race (the caller orders them).
 *  - Limits: D in {64, 128}; 1 <= C <= 65536; 0 <= P; P + C <= 2^31 - 1;
 *    B * Hq * C <= 2^31 - 1. The backward calls (pka_chunk_attn_bwd,
 *    pka_chunk_attn_bwd_noalloc, pka_prefix_kv_grad) also need the query rows of one
 *    KV head below 4 GiB: (Hq / Hkv) * C * D * 2 <= 2^32 - 2^20 bytes, else
 *    PKA_ERR_DIMS.
 */
#ifndef PKA_H
#define PKA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* pka_stream_t; /* identical to hipStream_t */

typedef enum {
  PKA_OK = 0,
  PKA_ERR_NULL = 1,        /* a required pointer is NULL                        */
  PKA_ERR_DIMS = 2,        /* inconsistent or out-of-range dimensions           */
  PKA_ERR_UNSUPPORTED = 3, /* head_dim or cache type this library does not serve */
  PKA_ERR_CAPACITY = 4,    /* the cache is too short for the rows addressed     */
  PKA_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned                  */
  PKA_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required        */
  PKA_ERR_HIP = 7          /* a HIP launch failed                               */
} pka_status;

typedef enum {
  PKA_CACHE_F16 = 0,  /* IEEE half; read as bf16 (round to nearest even)          */
  PKA_CACHE_BF16 = 1, /* bf16, read as is                                         */
  PKA_CACHE_Q8_0 = 2  /* blocks of 32 int8 codes along D + one fp16 scale per block:
                         value = f32(scale) * code, read as bf16 (RNE)            */
} pka_cache_type;

/* One chunk step of B windows. Every window has the same chunk length; the prefix
 * length is the same for all windows unless prefix_lens is given (ragged windows:
 * a batch of windows walked to different depths, the longest one setting the
 * work, as in "train: walk the window", Contents: the longest window's step). */
typedef struct {
  int32_t batch;       /* B >= 1                                    */
  int32_t n_heads_q;   /* Hq >= 1, a multiple of n_heads_kv         */
  int32_t n_heads_kv;  /* Hkv >= 1                                  */
  int32_t head_dim;    /* D: 64 or 128                              */
  int64_t prefix_len;  /* P >= 0: cached context rows 0..P-1 are read; with
                          prefix_lens, the largest prefix of the batch          */
  int64_t chunk_len;   /* C >= 1                                    */
  float softmax_scale; /* > 0 and finite; usually 1/sqrt(D)         */
  const int32_t* prefix_lens; /* optional DEVICE array int32[B] (4-byte aligned):
                          window b's own prefix length P_b; chunk row i of window
                          b then attends to cache rows 0..P_b-1 and chunk rows
                          0..i, and appends write rows [P_b, P_b + C). Entries are
                          clamped to [0, prefix_len] (never read past prefix_len).
                          NULL: every window has prefix_len.                     */
} pka_dims;

/* The frozen prefix cache of B windows x Hkv heads x capacity token rows. */
typedef struct {
  int32_t type;      /* pka_cache_type                                         */
  int32_t head_dim;  /* must equal pka_dims.head_dim                           */
  int64_t capacity;  /* rows per (window, KV head)                             */
  void* k;           /* F16/BF16: u16[B][Hkv][cap][D]; Q8_0: int8[B][Hkv][cap][D] */
  void* v;
  void* k_scale;     /* Q8_0: f16[B][Hkv][cap][D/32]; NULL for F16/BF16          */
  void* v_scale;
} pka_cache;

/* Workspace (bytes) the calls below need for this shape; 0 means none. The amount
 * depends only on the dims (the split of the prefix over workgroups is planned for
 * the 256 compute units of an MI355X). */
size_t pka_fwd_workspace_bytes(const pka_dims* dims);
size_t pka_bwd_workspace_bytes(const pka_dims* dims);

/* Forward of chunk attention against the frozen prefix ("Context-Frozen Training",
 * The Solution, Phase 2; "train: walk the window", What it is).
 *   o[b][h][i]   = sum_j softmax_j(scale * q[b][h][i] . K_j) V_j over allowed j
 *   lse[b][h][i] = ln sum_j exp(scale * q[b][h][i] . K_j) over allowed j (natural log)
 * where K_j, V_j (j < P) are cache rows of KV head h/G and K_{P+t}, V_{P+t} = k, v
 * rows t of the chunk; row i allows j <= P + i. Reads cache rows [0, P) only.
 * ws: pka_fwd_workspace_bytes(dims) bytes of device memory (may be NULL if 0). */
pka_status pka_chunk_attn_fwd(const pka_dims* dims, const void* q, const void* k,
                              const void* v, const pka_cache* cache, void* o,
                              float* lse, void* ws, size_t ws_bytes,
                              pka_stream_t stream);

/* The forward above fused with the re-decode of the chunk into the cache: one launch
 * computes o and lse exactly as pka_chunk_attn_fwd (the chunk's own keys are the
 * bf16 k, v) and writes rows [P_b, P_b + C) of the cache from k, v exactly as the
 * pka_kv_append_* call of the cache's type would. This is the no-grad forward of a
 * context piece that builds the cache chunk by chunk ("Context-Frozen Training", The
 * Solution, Phase 1: a forward without gradients fills the KV cache; "train: walk the
 * window", What it is: the chunk is re-decoded into the cache so the next one sees
 * it). Requires prefix_len + C <= capacity. The rows written are never read by the
 * same launch, so the fusion changes no value. */
pka_status pka_chunk_attn_fwd_append(const pka_dims* dims, const void* q, const void* k,
                                     const void* v, const pka_cache* cache, void* o,
                                     float* lse, void* ws, size_t ws_bytes,
                                     pka_stream_t stream);

/* Backward of the forward above from the upstream gradient d_o on the chunk rows.
 * Computes delta = rowsum(d_o * o), then
 *   dq = scale * dS K      over prefix and chunk keys,
 *   dk = scale * dS^T q,  dv = P^T d_o   for the chunk's own C keys only,
 * with P = exp(scale q K^T - lse) (masked) and dS = P * (d_o V^T - delta); dk, dv
 * are summed over the G query heads of each KV head. The prefix gets no gradient:
 * its rows are fixed inputs of the step ("train: walk the window", Why it's a draft;
 * "stop-gradient through context tokens", Known gaps: gradient for the kept queries
 * alone).
 * o and lse are the forward's outputs. delta (f32 [B][Hq][C]) is written if not
 * NULL. ws: pka_bwd_workspace_bytes(dims) bytes (always > 0). */
pka_status pka_chunk_attn_bwd(const pka_dims* dims, const void* q, const void* k,
                              const void* v, const pka_cache* cache, const void* o,
                              const float* lse, const void* d_o, void* dq, void* dk,
                              void* dv, float* delta, void* ws, size_t ws_bytes,
                              pka_stream_t stream);

/* pka_chunk_attn_bwd without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture, tight
 * training loops, harnesses that forbid hipMalloc. The workspace is a fixed array of
 * PKA_BWD_NOALLOC_MAX_WORKSPACE bytes inside the library, one per GPU, held by that GPU
 * from the first call on it until the process ends. Outputs and every other argument
 * are as in pka_chunk_attn_bwd (same kernels, same results bit for bit).
 * Errors: PKA_ERR_WORKSPACE (nothing launched) when pka_bwd_workspace_bytes(dims)
 * exceeds that size; the other statuses as pka_chunk_attn_bwd.
 * Concurrency: all calls on one GPU share its array, so two of them in flight at the
 * same time (on different streams, or from different threads without ordering) race
 * and give wrong results; order them on one stream. The array keeps what the last
 * call left in it; no call depends on its contents. */
#define PKA_BWD_NOALLOC_MAX_WORKSPACE ((size_t)96 << 20)
pka_status pka_chunk_attn_bwd_noalloc(const pka_dims* dims, const void* q, const void* k,
                                      const void* v, const pka_cache* cache, const void* o,
                                      const float* lse, const void* d_o, void* dq, void* dk,
                                      void* dv, float* delta, pka_stream_t stream);

/* Gradient of the chunk's loss with respect to the last `horizon` cached prefix rows
 * of every window, from the chunk's queries only: the part of the exact reverse pass
 * that a stop-gradient prefix drops ("train: walk the window", Why it's a draft: an
 * exact reverse pass with horizon H = 0 ... all; "stop-gradient through context
 * tokens", Mechanism: kept queries attend to the context's k/v, so context dK/dV
 * are nonzero and feed the k/v weight gradients). With P_b the window's prefix:
 *   dk_prefix[b][kv][h] = scale * sum_{g, i} dS[i][j] q[b][kv*G+g][i]
 *   dv_prefix[b][kv][h] = sum_{g, i} P[i][j] d_o[b][kv*G+g][i],   j = P_b - H + h,
 * with P and dS as in pka_chunk_attn_bwd, taken against the cache rows as the
 * attention reads them (F16 / q8_0 dequantised to bf16); rows with j < 0 (P_b < H)
 * are written as 0. Outputs are f32 [B][Hkv][H][D]. Inputs: the chunk's q and d_o,
 * the forward's lse and the backward's delta (pka_chunk_attn_bwd with delta != NULL).
 * 0 <= horizon <= prefix_len; horizon = 0 writes nothing. ws:
 * pka_prefix_kv_grad_workspace_bytes(dims, horizon) bytes (may be NULL if 0). */
size_t pka_prefix_kv_grad_workspace_bytes(const pka_dims* dims, int64_t horizon);
pka_status pka_prefix_kv_grad(const pka_dims* dims, int64_t horizon, const void* q,
                              const pka_cache* cache, const float* lse, const void* d_o,
                              const float* delta, float* dk_prefix, float* dv_prefix,
                              void* ws, size_t ws_bytes, pka_stream_t stream);

/* Re-decode of the chunk into the cache ("train: walk the window", What it is and
 * Contents): writes cache rows [P, P+C) of every (window, KV head) from k, v
 * (bf16 [B][Hkv][C][D]). Uses batch, n_heads_kv, head_dim, prefix_len, chunk_len of
 * dims (rows [P_b, P_b+C) with prefix_lens); requires prefix_len + C <= capacity
 * and a cache of the matching type.
 *  q8_0: per block of 32 values along D: amax = max|x|, d = amax/127 (IEEE fp32
 *        division), scale = fp16(d) (RNE), code = clamp(round_half_away(x/d), +-127)
 *        with the fp32 d; an all-zero block stores scale 0 and codes 0.
 *  f16:  fp16(x) with round to nearest even.      bf16: a copy. */
pka_status pka_kv_append_q8_0(const pka_dims* dims, const void* k, const void* v,
                              const pka_cache* cache, pka_stream_t stream);
pka_status pka_kv_append_f16(const pka_dims* dims, const void* k, const void* v,
                             const pka_cache* cache, pka_stream_t stream);
pka_status pka_kv_append_bf16(const pka_dims* dims, const void* k, const void* v,
                              const pka_cache* cache, pka_stream_t stream);

/* Row-sparse linear backward of the projections next to attention ("stop-gradient
 * through context tokens", Mechanism): q/o and the MLP keep their full-row forward
 * y = x W^T, and their backward runs only on the K token rows that some loss term
 * reads (the other rows' upstream gradient is zero by then):
 *   dw = dy[keep]^T x[keep]                          f32 [out][in]
 *   dx[keep[r]] = dy[keep[r]] W;  dx[other rows] = 0  bf16 [N][in]
 * This equals the dense backward with dy zeroed outside the kept rows. x is bf16
 * [N][in], w bf16 [out][in], dy bf16 [N][out], all row-major; keep is a DEVICE
 * int32 [K] array of distinct rows of x (any order; entries outside [0, N) are
 * skipped: they add nothing and write nothing). in_features and out_features are
 * multiples of 128. dw or dx may be NULL, and that product is skipped; 0 <= K <= N
 * (K = 0 writes dw = 0 and dx = 0). x, w, dy, dw, dx and ws 16-byte aligned, keep
 * 4-byte aligned; all are caller-owned device memory.
 * ws: pka_row_sparse_linear_bwd_workspace_bytes(dims) bytes (may be NULL if 0; not used
 * when dx is NULL): when few kept rows make few output tiles, the dX product is split
 * over the output features and its fp32 partials go there. Results are deterministic.
 * Errors (nothing launched): PKA_ERR_DIMS (N < 1, K outside [0, N], a grid too large),
 * PKA_ERR_UNSUPPORTED (features not multiples of 128), PKA_ERR_NULL / PKA_ERR_ALIGN
 * (a needed pointer), PKA_ERR_WORKSPACE (ws missing or too small). */
typedef struct {
  int64_t n_rows;        /* N >= 1: rows of x, dy and dx                      */
  int64_t n_keep;        /* K: entries of keep                                */
  int32_t in_features;   /* columns of x and w, multiple of 128               */
  int32_t out_features;  /* rows of w, columns of dy, multiple of 128         */
} pka_rs_dims;
size_t pka_row_sparse_linear_bwd_workspace_bytes(const pka_rs_dims* dims);
pka_status pka_row_sparse_linear_bwd(const pka_rs_dims* dims, const void* x, const void* w,
                                     const void* dy, const int32_t* keep, float* dw, void* dx,
                                     void* ws, size_t ws_bytes, pka_stream_t stream);

/* Test hook: dequantise rows [row0, row0+rows) of both K and V of a Q8_0 cache of
 * `batch` windows x `n_heads_kv` heads exactly as the attention kernels read them:
 * out_f32 = f32(scale) * code (exact), out_bf16 = bf16(out_f32) (RNE, may be NULL).
 * Outputs are [2][batch][n_heads_kv][rows][D] (K first, then V). */
pka_status pka_kv_dequant_q8_0(const pka_cache* cache, int32_t batch,
                               int32_t n_heads_kv, int64_t row0, int64_t rows,
                               float* out_f32, void* out_bf16, pka_stream_t stream);

/* A static description of a status code. */
const char* pka_status_string(pka_status status);
/* The message of the last failed call on this thread ("" if none). */
const char* pka_last_error(void);

/* Opt-in kernel timing for benchmarks. When enabled, each launch of a selected
 * kernel is bracketed by two HIP events recorded on the call's stream (timing-only
 * events, created without the system-scope memory fence); pka_profile_read synchronises on those events and returns the summed elapsed
 * milliseconds and the number of launches of one kernel since the last reset. At
 * most 65536 launches per kernel are recorded between resets (later ones are
 * counted in `dropped`). pka_profile_select limits the bracketing to the kernels
 * whose bit (1u << pka_kernel_id) is set in kernel_mask (after load: all), so a
 * timed loop can carry the events of one kernel only. Enable and select are
 * process-wide settings; changing them while another thread launches affects
 * that thread's next launches only. */
typedef enum {
  PKA_KERNEL_FWD = 0,        /* forward tiles (one launch per pka_chunk_attn_fwd) */
  PKA_KERNEL_FWD_COMBINE = 1,/* merge of prefix splits                            */
  PKA_KERNEL_BWD_PREP = 2,   /* delta launch, only when the chunk dk, dv run in the
                                dq grid (shapes whose dq grid leaves CUs idle)     */
  PKA_KERNEL_BWD_DQ = 3,     /* dq over prefix and chunk keys (with the chunk dk, dv
                                when those run in the same grid)                   */
  PKA_KERNEL_BWD_DKDV = 4,   /* chunk-only dk, dv                                  */
  PKA_KERNEL_BWD_DQ_REDUCE = 5, /* sums of dq and dk/dv split partials (one launch) */
  PKA_KERNEL_APPEND = 6,     /* kv_append_*                                        */
  PKA_KERNEL_DEQUANT = 7,    /* kv_dequant_q8_0                                    */
  PKA_KERNEL_BWD_DKDV_REDUCE = 8, /* reserved: folded into PKA_KERNEL_BWD_DQ_REDUCE */
  PKA_KERNEL_PREFIX_KV = 9,  /* prefix dk, dv within the horizon                    */
  PKA_KERNEL_PREFIX_KV_REDUCE = 10, /* sums of their row-split partials             */
  PKA_KERNEL_RS_ZERO = 11,   /* row-sparse backward: zeros of the rows not kept   */
  PKA_KERNEL_RS_DX = 12,     /* row-sparse backward: dX of the kept rows          */
  PKA_KERNEL_RS_DW = 13,     /* row-sparse backward: dW                           */
  PKA_KERNEL_RS_DX_REDUCE = 14, /* row-sparse backward: sums of dX split partials */
  PKA_KERNEL_COUNT = 15
} pka_kernel_id;

pka_status pka_profile_enable(int32_t on);
pka_status pka_profile_select(uint32_t kernel_mask);
pka_status pka_profile_reset(void);
pka_status pka_profile_read(int32_t kernel, double* total_ms, int64_t* launches,
                            int64_t* dropped);

#ifdef __cplusplus
}
#endif
#endif /* PKA_H */
