/*
 * st.h -- C ABI of libst.so: factorized sparse causal self-attention on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (nlp-lineage milestone page on the Sparse Transformer,
 * "The notation"; llm-arch-kb "Sparse Transformer", §2 Derivation):
 *
 *   out[b,h,t,:] = sum_{j in S_h(t)} softmax_j( q[b,h,t,:] . k[b,h,j,:] / sqrt(D) ) v[b,h,j,:]
 *
 * where the softmax normalises over S_h(t) only (keys outside the set carry
 * no probability mass) and S_h(t) is one half of a factorized pattern:
 * head h uses sub-pattern (h mod 2), "kind 0" or "kind 1".
 *
 *   ST_STRIDED (llm-arch-kb §2, Pattern A -- strided; nlp-lineage "The idea"):
 *     kind 0: the last l positions, t included:  max(0, t-l+1) <= j <= t
 *     kind 1: every l-th position back from t:   j <= t and (t - j) mod l == 0
 *   ST_FIXED (llm-arch-kb §2, Pattern B -- fixed; nlp-lineage "The idea"):
 *     kind 0: t's own l-block up to t:           l*floor(t/l) <= j <= t
 *     kind 1: the c summary positions at the end of every *earlier* block:
 *             floor(j/l) < floor(t/l) and (j mod l) >= l - c
 *   ST_FIXED_R1: as ST_FIXED, but kind 1 also admits the own block's summary
 *     positions j <= t (the reading of the llm-arch-kb §3 mask sketch).
 *   ST_DENSE: full causal attention, S(t) = {j <= t}, for both kinds (the
 *     dense comparator of nlp-lineage "The notation").
 *   ST_STRIDED_UNION, ST_FIXED_UNION: merged heads -- every head attends the
 *     union of the pattern's two sets (llm-arch-kb §2 states each pattern as
 *     that union; its §3 mask sketch builds one mask from both loops).  The
 *     library computes it as two passes over every head, one per kind: the
 *     first keeps fp32 partial results in the workspace, the second merges
 *     its own into them (the two softmaxes by their log-sum-exps, gradients
 *     by addition).  For that split the strided pass leaves out t itself
 *     (already in the window); the fixed sets are disjoint.  Every entry
 *     point (bf16, fp16, fp32) takes them.
 *
 * Conventions (readings where the pages are silent):
 *   - positions are 0-based; T need not be a multiple of l;
 *   - a row with an empty key set (ST_FIXED kind 1, first block) gets
 *     out = 0 and lse = -inf, and contributes nothing to any gradient;
 *   - lse[b,h,t] = ln sum_{j in S(t)} exp(q_t . k_j / sqrt(D)), fp32;
 *   - keys that no query attends get dk = dv = 0.
 *
 * Layout.  q, k, v, out, dout, dq, dk, dv are dense row-major [B, H, T, D]
 * (D fastest); lse is [B, H, T] fp32.  The unsuffixed entry points take and
 * return bf16 (bfloat16, round-to-nearest-even on output) with fp32
 * arithmetic inside; the _f16 entry points do the same with fp16 (IEEE
 * binary16); the _f32 entry points take and return fp32.
 *
 * Ownership.  All tensor pointers are device pointers owned by the caller;
 * the library never frees them or keeps them past the call.  The library owns
 * a per-device cache of block LUTs and work schedules and a per-device
 * workspace (backward scratch; for merged heads also the fp32 partial results
 * the second pass adds to), both grown on demand and freed by st_release().
 *
 * Asynchrony.  The attention entry points enqueue kernels on `stream` (a
 * hipStream_t; NULL means the default stream) and return without waiting.
 * A call that has to build a LUT or grow the workspace performs blocking
 * host-to-device copies or allocations first.  Calls that use the workspace
 * (every backward call; forward calls with a merged-head pattern) are ordered
 * on it across streams: a call on a stream other than the last user's makes
 * its stream wait (hipStreamWaitEvent) for that user's kernels.  At most 64
 * plans are cached per process; a new one past that drops the least recently
 * used, after synchronising that plan's device.
 *
 * Errors.  Every entry point returns ST_OK (0) or a negative st_status; no
 * C++ exception crosses the ABI.  The message of the last failure on the
 * calling thread is available from st_last_error().
 */
#ifndef ST_H
#define ST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum st_status {
  ST_OK = 0,
  ST_ERR_INVALID = -1,     /* bad argument: null/misaligned pointer, size out of range */
  ST_ERR_UNSUPPORTED = -2, /* well-formed but not implemented (e.g. D not 32, 64 or 128) */
  ST_ERR_HIP = -3,         /* a HIP runtime call or kernel launch failed */
  ST_ERR_NOMEM = -4,       /* host or device allocation failed */
  ST_ERR_BUFFER_TOO_SMALL = -5 /* a caller buffer's capacity is below what the call writes */
} st_status;

/* Element type of the tensors, for the _ex attention entry points. */
typedef enum {
  ST_BF16 = 0, /* bfloat16 (the unsuffixed entry points) */
  ST_F16 = 1,  /* IEEE binary16 (the _f16 entry points)   */
  ST_F32 = 2   /* fp32 (the _f32 entry points)            */
} st_dtype;

typedef enum st_pattern {
  ST_STRIDED = 0,
  ST_FIXED = 1,
  ST_FIXED_R1 = 2,
  ST_DENSE = 3,
  ST_STRIDED_UNION = 4,
  ST_FIXED_UNION = 5
} st_pattern;

/* ---------------------------------------------------------------------------
 * Block layout (host only; no GPU needed).
 *
 * The pages precompute each query's key indices and run the attention as a
 * block-sparse product over non-empty blocks (llm-arch-kb "Sparse
 * Transformer", §2 "Per-layer cost" and §3 Reference implementation).  The
 * library does so in kernel coordinates, per head kind:
 *   kernel row R  holds query position row_pos[R] (-1 = padding),
 *   kernel key K  holds key   position key_pos[K] (-1 = padding),
 * with block size st_block_size() for both.  The maps:
 *   - identity for ST_STRIDED kind 0, ST_FIXED / ST_FIXED_R1 kind 0, ST_DENSE;
 *   - ST_STRIDED kind 1, residue-major: position m*l + r is row and key
 *     r*n_pad + m, n = ceil(T/l), n_pad = n rounded up to a multiple of the
 *     block size; classes r < min(l, T);
 *   - ST_FIXED kind 1, compact summary keys: key b*c + o holds position
 *     b*l + (l-c) + o for blocks b < ceil(T/l) - 1 (ST_FIXED_R1: all blocks,
 *     positions >= T are padding); rows are the identity.
 *   - merged heads: kind p is the p-th pass, with the maps of the base
 *     pattern's kind p; the LUT of the strided pass omits the row's own key.
 * In these coordinates every row attends one contiguous run of kernel keys.
 * A (row block, key block) pair is listed when it holds at least one
 * attended pair; its flag is 1 (FULL) when all block*block pairs are
 * attended, else 0 (PARTIAL).  The CSR lists pairs sorted by (row block,
 * key block); the CSC by (key block, row block).
 * ------------------------------------------------------------------------- */
typedef struct st_layout st_layout; /* opaque, owned by the library */

enum {
  ST_DIM_BLOCK = 0,   /* block size (rows and keys)                    */
  ST_DIM_ROWS = 1,    /* kernel rows, padding included                 */
  ST_DIM_KEYS = 2,    /* kernel keys, padding included                 */
  ST_DIM_QBLOCKS = 3, /* ceil(rows / block): CSR row_ptr has this + 1  */
  ST_DIM_KBLOCKS = 4, /* ceil(keys / block): CSC col_ptr has this + 1  */
  ST_DIM_NNZ = 5,     /* listed block pairs                            */
  ST_DIM_COUNT = 6
};

/* Build the layouts of both head kinds of `pattern` for sequence length T,
 * stride l (>= 1) and summary count c (1 <= c <= l for the fixed patterns,
 * ignored otherwise).  1 <= T <= 2^24.  On success *out owns the result;
 * release it with st_layout_free().  Returns ST_ERR_INVALID on bad
 * arguments, ST_ERR_NOMEM on allocation failure. */
int st_layout_build(int pattern, int T, int l, int c, st_layout** out);

/* Summary sets.  The fixed patterns' summary kind attends, in every l-block,
 * the keys at the offsets of a summary set S (llm-arch-kb §2, Pattern B: a
 * fixed set of offsets within each block; its §3 mask sketch takes it as an
 * argument).  The entry points without `summary` use the last c offsets
 * (nlp-lineage, "The idea": summary positions at the end of each block).
 * `summary`: NULL (the last c offsets), or c offsets in [0, l), strictly
 * ascending, in host memory, read during the call only.  Only the fixed
 * patterns take one (ST_ERR_INVALID otherwise, or for a malformed set).
 * Compact summary key b*c + o then holds position b*l + summary[o]. */
int st_layout_build_ex(int pattern, int T, int l, int c, const int32_t* summary, st_layout** out);

/* dims[ST_DIM_COUNT] of head kind 0 or 1. */
int st_layout_dims(const st_layout* lay, int kind, int32_t* dims);

/* Total attended (query, key) pairs of one head of this kind, sum_t |S(t)|. */
int st_layout_pairs(const st_layout* lay, int kind, int64_t* pairs);

/* Copy-outs into caller buffers (host memory).  Each buffer comes with its
 * capacity in elements; a capacity below the element count the call writes
 * gives ST_ERR_BUFFER_TOO_SMALL and nothing is written.  A buffer may be NULL
 * only when its element count is 0 (else ST_ERR_INVALID).  The counts come
 * from st_layout_dims. */

/* The coordinate maps: row_pos[ROWS], key_pos[KEYS]. */
int st_layout_maps(const st_layout* lay, int kind, int32_t* row_pos, size_t row_pos_cap, int32_t* key_pos,
                   size_t key_pos_cap);

/* The CSR: row_ptr[QBLOCKS+1], col_idx[NNZ], flags[NNZ]. */
int st_layout_csr(const st_layout* lay, int kind, int32_t* row_ptr, size_t row_ptr_cap, int32_t* col_idx,
                  size_t col_idx_cap, uint8_t* flags, size_t flags_cap);

/* The CSC: col_ptr[KBLOCKS+1], row_idx[NNZ], flags[NNZ]. */
int st_layout_csc(const st_layout* lay, int kind, int32_t* col_ptr, size_t col_ptr_cap, int32_t* row_idx,
                  size_t row_idx_cap, uint8_t* flags, size_t flags_cap);

void st_layout_free(st_layout* lay);

/* ---------------------------------------------------------------------------
 * Attention.  Shapes: 1 <= B, 1 <= H, B*H <= 2^20, 1 <= T <= 2^24,
 * D in {32, 64, 128}; pattern, l and c as for st_layout_build.  The bf16 and
 * fp16 entry points also need T*D <= 2^30 (one head within 2^31 bytes; for
 * D = 128, T <= 2^23), else ST_ERR_UNSUPPORTED.  Every pointer must
 * be non-null and 16-byte aligned, and the tensors must not overlap (except
 * that inputs may alias one another).
 * ------------------------------------------------------------------------- */

/* Forward (llm-arch-kb §2 "Sparse attention as an unnormalized form";
 * nlp-lineage "The notation").  Reads q, k, v; writes out [B,H,T,D] and
 * lse [B,H,T].  bf16 in / out, fp32 arithmetic. */
int st_sparse_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                       int B, int H, int T, int D, int pattern, int l, int c, void* stream);

/* Backward of L = <dout, out> with the attention weights recomputed from q,
 * k and lse instead of being stored (nlp-lineage "The idea", recomputation).
 * `out` and `lse` must be what st_sparse_attn_fwd returned for the same
 * q, k, v.  Writes dq, dk, dv [B,H,T,D].  bf16 in / out, fp32 arithmetic. */
int st_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv,
                       int B, int H, int T, int D, int pattern, int l, int c, void* stream);

/* fp16 twins: same arguments, fp16 (IEEE binary16) tensors, fp32 arithmetic
 * (the pages fix only "16-bit" precision; this is the other 16-bit format).
 * Outputs are rounded to nearest even. */
int st_sparse_attn_fwd_f16(const void* q, const void* k, const void* v, void* out, float* lse,
                           int B, int H, int T, int D, int pattern, int l, int c, void* stream);
int st_sparse_attn_bwd_f16(const void* q, const void* k, const void* v, const void* out,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           int B, int H, int T, int D, int pattern, int l, int c, void* stream);

/* Forward and backward with an element type code and a summary set (see
 * st_layout_build_ex); otherwise as the entry points above.  An unknown dtype
 * gives ST_ERR_INVALID. */
int st_sparse_attn_fwd_ex(int dtype, const void* q, const void* k, const void* v, void* out, float* lse,
                          int B, int H, int T, int D, int pattern, int l, int c,
                          const int32_t* summary, void* stream);
int st_sparse_attn_bwd_ex(int dtype, const void* q, const void* k, const void* v, const void* out,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                          int H, int T, int D, int pattern, int l, int c, const int32_t* summary,
                          void* stream);

/* Backward that allocates nothing, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments and results as st_sparse_attn_bwd_ex.
 * Instead of the library's workspace it uses a static device array of 64 MiB
 * (one per device, held until the process ends) and calls no hipMalloc or
 * hipFree.  It needs the plan of its shapes to be cached: one earlier call of
 * any other attention entry point with the same (pattern, B, H, T, l, c,
 * summary set) on this device builds it; otherwise ST_ERR_UNSUPPORTED.  A
 * call whose workspace would exceed 64 MiB (about B*H*T*12 bytes, plus the
 * split partials, plus B*H*T*D*12 bytes for merged heads) gives
 * ST_ERR_UNSUPPORTED.  Nothing in the array needs to start at zero; it keeps
 * the last call's contents.  Every call on one device shares the array:
 * calls that overlap in time on one device (any streams) race -- serialise
 * them. */
int st_sparse_attn_bwd_noalloc(int dtype, const void* q, const void* k, const void* v, const void* out,
                               const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                               int H, int T, int D, int pattern, int l, int c, const int32_t* summary,
                               void* stream);

/* fp32 twins: same arguments, fp32 tensors. */
int st_sparse_attn_fwd_f32(const void* q, const void* k, const void* v, void* out, float* lse,
                           int B, int H, int T, int D, int pattern, int l, int c, void* stream);
int st_sparse_attn_bwd_f32(const void* q, const void* k, const void* v, const void* out,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           int B, int H, int T, int D, int pattern, int l, int c, void* stream);

/* ---------------------------------------------------------------------------
 * Kernel shapes (performance only; not part of the computation).  Two 16-bit
 * kernels at D <= 64 come in two shapes each, which compute every output
 * element with the same operations in the same order, so the results are
 * bitwise identical under either:
 *   - the forward: 32 rows per wave (four waves per pair of 64-row blocks,
 *     each reading its K and V operands once for two 16-row groups) or 16
 *     (eight waves, more of them resident per CU);
 *   - the dK/dV pass: 16 keys per wave (four waves per 64-key block) or 32
 *     (two waves, each reading its Q and dO operands once for two 16-key
 *     tiles).
 * 0 (the default) picks per launch: the forward takes 16 rows per wave for
 * launches of at most 1536 work items (too short to fill the GPU more than
 * about one and a half times), 32 otherwise; dK/dV takes 32 keys per wave
 * where its items far outnumber what the GPU holds at once (full attention,
 * very long sequences), 16 otherwise.  16 or 32 forces that shape for every
 * later call in the process (fp32 inputs and D = 128 always use the four-wave
 * forward and 16 keys per wave).  Other values give ST_ERR_INVALID.  A setting
 * takes effect at the next call; calls already enqueued are unaffected.
 * ------------------------------------------------------------------------- */
int st_set_fwd_rows_per_wave(int rows);
int st_set_dkdv_keys_per_wave(int keys);

/* ---------------------------------------------------------------------------
 * Kernel timing (diagnostics; not part of the computation).  While enabled,
 * every kernel the library launches is bracketed by two HIP events recorded
 * on its launch stream.  st_timing_read() waits for those events and returns,
 * for one kernel, the number of launches and their summed duration in
 * milliseconds since the last st_timing_reset().  Kernel names: "fwd",
 * "bwd_pre", "bwd_dq", "bwd_dkdv", "bwd_reduce", "bwd_delta".  Unknown names give
 * ST_ERR_INVALID; a failing event call gives ST_ERR_HIP.
 * ------------------------------------------------------------------------- */
int st_timing_enable(int on);
int st_timing_read(const char* kernel, int64_t* launches, double* total_ms);
void st_timing_reset(void);

/* ---------------------------------------------------------------------------
 * Utilities.
 * ------------------------------------------------------------------------- */
int st_block_size(void);                 /* block size of the LUTs (64)              */
const char* st_status_string(int status); /* static text for a status code           */
const char* st_last_error(void);         /* last failure message on this thread       */
/* Free the LUT caches and workspaces on every GPU, after waiting for each GPU's
 * queued work (a blocking call).  Later calls rebuild what they need.  It takes
 * the library's lock, so calls from other host threads run before or after it. */
void st_release(void);

#ifdef __cplusplus
}
#endif

#endif /* ST_H */
