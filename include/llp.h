/*
 * llp.h -- C ABI of the fused linear log-prob library for AMD MI355X (gfx950).
 *
 * Operators
 * ---------
 * linear_logp: for hidden states h [N, D], a weight W [V, D] (the layout of a
 * linear layer's weight), an optional bias b [V] and integer targets t [N],
 *     z      = h W^T + b                      (logits, never stored in memory)
 *     lse[n] = log sum_v exp(z[n, v])
 *     logp[n]= z[n, t_n] - lse[n]
 * and, for an upstream gradient g [N] of logp,
 *     dlogits = g (onehot(t) - softmax(z))    (recomputed, never stored whole)
 *     dH = dlogits W,  dW = dlogits^T h (added in place into one table),
 *     db = sum_n dlogits.
 * Sources: RL-Kernel issue #261 "Accumulate portable linear_logp backward dW
 * with FP32 addmm_" (sections "Current production path", "Current
 * accumulation", "Correctness boundary"); Liger-Kernel PR #1324 "Use direct
 * FLCE weight-gradient accumulation for FP16, BF16, and FP32" ("Summary",
 * "Details"); RL-Kernel PR #495 "fused zero-workspace backward for the generic
 * CUDA fused logp" ("Summary", "Behavior changes").
 *
 * logp: the same log-prob and gradient computed from given logits [N, V]
 * (RL-Kernel PR #495, "Summary" and "Results").
 *
 * Conventions (every entry point)
 * -------------------------------
 * - Memory: every pointer argument is DEVICE memory on the current HIP device
 *   unless stated, row-major and contiguous; the caller owns all of it. The
 *   library allocates nothing: scratch space comes from the caller's
 *   `workspace`, sized by the matching *_workspace_size query.
 * - Execution: work is enqueued on `stream` (a hipStream_t; NULL = the null
 *   stream) and the call returns without waiting for it. The library keeps no
 *   mutable global state (except the scratch of linear_logp_fwd_noalloc);
 *   calls on different streams must not share output or workspace buffers.
 *   A call only launches kernels on `stream` (no allocation, copy, memset or
 *   synchronisation), so it may be captured into a HIP graph; a replay
 *   produces the eager call's bits.
 * - dtypes: operands h, W, b, logits, dH and dlogits use `dtype` (LLP_F32,
 *   LLP_BF16 or LLP_F16). logp, lse and g are float32. Targets are int64.
 *   Arithmetic accumulates in float32; 16-bit results are rounded to nearest
 *   even.
 * - Targets outside [0, V) (for example -100) are not errors: that row gets
 *   logp = +0 and an all +0 gradient row (RL-Kernel PR #495, "Behavior
 *   changes"). lse is still reported for it.
 * - Errors: a nonzero llp_status is returned. All argument checks happen
 *   before any HIP call, so on LLP_EINVAL / LLP_EWORKSPACE / LLP_EOVERFLOW
 *   nothing was enqueued and no output was touched. LLP_EHIP reports a failed
 *   kernel launch (hipGetLastError); outputs are then unspecified.
 * - Sizes are int64 everywhere; element offsets are computed in 64 bits
 *   (N * V may exceed 2^31; RL-Kernel PR #495 review of the INT_MAX loop
 *   counters).
 * - Device check (opt-in): with the environment variable LLP_CHECK_DEVICE=1,
 *   every call first asks HIP where each non-NULL pointer argument lives and
 *   returns LLP_EINVAL (enqueuing nothing) unless it is device or managed
 *   memory of the current device (the device-guard lesson of RL-Kernel PR
 *   #495's review). Off by default: it costs a few microseconds per call.
 */
#ifndef LLP_H
#define LLP_H

#include <stddef.h>
#include <stdint.h>

#ifndef LLP_API
#define LLP_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LLP_F32 = 0, LLP_BF16 = 1, LLP_F16 = 2 } llp_dtype;

typedef enum {
  LLP_OK = 0,
  LLP_EINVAL = 1,     /* bad shape, NULL required pointer, bad dtype/flag combination */
  LLP_EWORKSPACE = 2, /* workspace smaller than the query's answer, or NULL when nonzero is needed */
  LLP_EOVERFLOW = 3,  /* an element count or byte size does not fit int64 / size_t */
  LLP_EHIP = 4        /* a HIP launch failed */
} llp_status;

/* Version of this ABI (major * 10000 + minor * 100 + patch). */
LLP_API int llp_version(void);

/* Static message for a status code; never NULL. */
LLP_API const char* llp_strerror(int status);

/*
 * Tokens per backward chunk. chunk > 0 is used as given (clamped to N);
 * chunk <= 0 selects floor(2^24 / V) (RL-Kernel issue #261, "Static traffic
 * model"), clamped to [1, max(N, 1)]. Returns -1 on N < 0 or V < 1.
 */
LLP_API int64_t linear_logp_chunk_rows(int64_t N, int64_t V, int64_t chunk);

/* Number of backward chunks, ceil(N / chunk_rows); 0 for N = 0; -1 on bad input. */
LLP_API int64_t linear_logp_num_chunks(int64_t N, int64_t V, int64_t chunk);

/*
 * Workspace bytes linear_logp_fwd needs for these shapes (0 for N = 0): the
 * per-token partial maxima and exp-sums of each 128-row vocabulary block and
 * the target logits, which replace the [N, V] logits the pages' fused paths
 * never keep (RL-Kernel PR #495, "Summary"; Liger-Kernel PR #1324,
 * "Summary"). Returns a status; *bytes is written on LLP_OK. Errors as
 * linear_logp_fwd's shape errors.
 */
LLP_API int linear_logp_fwd_workspace_size(int64_t N, int64_t D, int64_t V, int dtype, size_t* bytes);

/*
 * Forward (RL-Kernel issue #261, "Current production path": linear_logp over
 * hidden states, weight, optional bias and targets; RL-Kernel PR #495,
 * "Summary": the row's max and sum of exponentials give lse, the target
 * logit minus lse gives logp). h [N, D], W [V, D] (a linear layer's weight),
 * b [V] or NULL, targets [N] int64  ->  logp [N] (required) and lse [N] (NULL
 * to skip), float32. lse is the residual the backward consumes. N = 0
 * enqueues nothing. Errors: LLP_EINVAL for N < 0, D < 1, V < 1, a bad dtype or
 * a NULL h / W / targets / logp (N > 0); LLP_EOVERFLOW when N, V, N D or V D
 * exceed the supported ranges; LLP_EWORKSPACE for a workspace below the
 * query's size. h, W and b are read only; logp and lse are written once.
 */
LLP_API int linear_logp_fwd(int64_t N, int64_t D, int64_t V, int dtype,
                    const void* h, const void* W, const void* b, const int64_t* targets,
                    float* logp, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward without allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): linear_logp_fwd with the same arguments except the workspace,
 * which is replaced by a device-global scratch array of LLP_SCRATCH_BYTES
 * built into the library (one per device, held until the process ends; its
 * device address is looked up on the first call on each device). The call
 * allocates nothing and calls no allocating routine. Results are bitwise
 * those of linear_logp_fwd. Shapes whose forward workspace
 * (linear_logp_fwd_workspace_size) exceeds LLP_SCRATCH_BYTES return
 * LLP_EWORKSPACE, enqueuing nothing: about N * ceil(V / 256) * 16 bytes, so
 * N <= 33487 tokens at V = 32000 and N <= 7058 at V = 151936. Every call on
 * one device shares that device's scratch: calls that may overlap on one
 * device (different streams, or different threads) race and must be
 * serialised by the caller. Nothing in the scratch needs to start at zero.
 * LLP_EHIP if the scratch's address cannot be obtained.
 */
#define LLP_SCRATCH_BYTES (64u << 20)
LLP_API int linear_logp_fwd_noalloc(int64_t N, int64_t D, int64_t V, int dtype,
                            const void* h, const void* W, const void* b, const int64_t* targets,
                            float* logp, float* lse, void* stream);

/*
 * Workspace bytes linear_logp_bwd needs. It depends on which outputs are
 * requested (want_* nonzero) and on whether the caller passes lse
 * (have_lse nonzero); unrequested outputs add nothing (RL-Kernel issue #261,
 * "Correctness boundary": no allocation that the requested outputs do not
 * need). It holds a chunk's softmax part in the operand dtype, vocab-major
 * (the chunk workspace of RL-Kernel issue #261, "Static traffic model"), the
 * chunk's h transposed, and per-token scalars. The schedule, and with it the
 * size, is decided from the shapes alone: the chunks are taken in groups
 * whose dW is one contraction (pairs; small chunks in balanced groups of up
 * to 4096 columns within a 1 GiB buffer), so these buffers hold a group's
 * columns; with 16-bit operands and D % 8 == 0 (V D and V x the group's
 * columns each below 2^30 elements) dH reads W as stored, no transposed copy
 * of W is held, a group runs as one working chunk of its tokens when dW or
 * db is requested (a group of small chunks always), and a second
 * softmax-part buffer lets the next chunk's logits recompute run beside a
 * chunk's dH / dW; with V above one vocabulary part (32768 rows for 16-bit
 * operands, 8192 for fp32) dH's fp32 sums over the parts are held too.
 */
LLP_API int linear_logp_bwd_workspace_size(int64_t N, int64_t D, int64_t V, int dtype, int64_t chunk,
                                   int want_dH, int want_dW, int want_db, int have_lse,
                                   size_t* bytes);

/*
 * Backward, over ceil(N / C) chunks of C = linear_logp_chunk_rows(N, V, chunk)
 * tokens, in increasing chunk order (RL-Kernel issue #261, "Current
 * accumulation"; Liger-Kernel PR #1324, "Details").
 *
 * g [N]: upstream gradient of logp (float32). lse [N]: the forward's lse, or
 * NULL to recompute it here.
 * dH [N, D] (dtype) or NULL: written once per row, no chunk rounding.
 * dW [V, D] or NULL, of dW_dtype (LLP_F32, or the operand dtype): each chunk's
 *   dlogits^T h is added into this table in place, with no [V, D] temporary.
 * db [V] or NULL, same dtype as dW_dtype; requires b != NULL.
 * accumulate = 0: dW and db are first set to +0 (the zero-initialised table
 *   of RL-Kernel issue #261, "Correctness boundary"), so that g = 0 gives +0
 *   with a clear sign bit; accumulate = 1: chunks are added into the caller's
 *   values (gradient accumulation across calls).
 * NULL outputs are never read or written. N = 0 writes only the zero fill of
 * dW/db (when accumulate = 0).
 * Alignment: with 16-bit operands and D % 8 == 0 (the layout without a W
 * transpose, see the workspace query) W and the workspace must be 16-byte
 * aligned, else LLP_EINVAL (nothing is enqueued).
 * Deterministic: the same inputs give bit-identical outputs on every call.
 * Limit: a row of the dlogits^T buffer (the chunk group's columns times the
 * operand size) stays below 2^28 bytes, else LLP_EOVERFLOW.
 */
LLP_API int linear_logp_bwd(int64_t N, int64_t D, int64_t V, int dtype, int64_t chunk,
                    const void* h, const void* W, const void* b, const int64_t* targets,
                    const float* g, const float* lse,
                    void* dH, void* dW, int dW_dtype, void* db, int accumulate,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward and backward in one call, for a caller that knows the upstream
 * gradient g of logp before the forward runs (for example a mean or sum
 * negative log-likelihood, g = -1/N or -1). Same inputs, outputs and
 * conventions as linear_logp_fwd followed by linear_logp_bwd with the
 * forward's lse: logp [N] (required), lse [N] (NULL to skip), dH, dW, db,
 * dW_dtype, accumulate and chunk as in linear_logp_bwd. The difference is the
 * schedule: each chunk's logits tile is computed once, and its softmax
 * numerators exp(z - m) (m: the maximum over the tile's 128-row vocab block)
 * are kept in the chunk workspace in the operand dtype until the chunk's lse
 * is known, instead of recomputing the logits in the backward: three N x V x D
 * contractions instead of four. This follows from g being fixed once the loss
 * reduction is fixed; the fused linear cross-entropy is measured as one
 * complete forward + backward training operation (Liger-Kernel PR #1324,
 * "Benchmark results", "Methodology"). With bf16 operands the numerators are
 * exp(z) itself wherever a block's maximum lies in [-40, 64] (else as above),
 * and each token's gradient factor is applied by the dH, dW and db steps.
 * With two or more chunks, dW is accumulated once per group of consecutive
 * chunks (pairs; small chunks in larger groups), so the table is read and
 * written once per group; with 16-bit operands and D % 8 == 0 the group runs
 * as one working chunk. The workspace then holds the group's columns side by
 * side, twice (with an FP32 table the next chunk's forward runs beside a
 * chunk's dH / dW; an operand-dtype table leaves the second copy unused, as
 * the workspace query does not know the table's dtype).
 * logp and lse are bit-identical to linear_logp_fwd's. The gradients round
 * the softmax part twice (the stored numerator, then the gradient or, for
 * bf16, the h row scaled by the token's factor), so they match
 * linear_logp_bwd's to within that rounding, not bitwise.
 * Alignment: as linear_logp_bwd; with bf16 operands and D % 8 == 0 W and the
 * workspace must be 16-byte aligned even when dH is not requested.
 * With dH, dW and db all NULL this is linear_logp_fwd (and the workspace
 * query returns the forward's size). Deterministic.
 * Limit: a row of the numerator buffer (the group's columns times the operand
 * size) must stay below 2^24 bytes, i.e. fewer than 2^23 tokens per chunk
 * group in 16-bit operands; beyond that LLP_EOVERFLOW (linear_logp_bwd's
 * limit is 2^28 bytes per row of its dlogits^T buffer).
 */
LLP_API int linear_logp_fwd_bwd_workspace_size(int64_t N, int64_t D, int64_t V, int dtype, int64_t chunk,
                                       int want_dH, int want_dW, int want_db, int have_lse,
                                       size_t* bytes);
LLP_API int linear_logp_fwd_bwd(int64_t N, int64_t D, int64_t V, int dtype, int64_t chunk,
                        const void* h, const void* W, const void* b, const int64_t* targets,
                        const float* g, float* logp, float* lse,
                        void* dH, void* dW, int dW_dtype, void* db, int accumulate,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Vocabulary-parallel share. A vocabulary of Vt rows is split into P
 * contiguous shares; a share holds rows [v0, v0 + Vs) of W (W_shard [Vs, D],
 * b_shard [Vs] or NULL) and sees every token. The pages name a tensor-parallel
 * variant of this operator without describing it (RL-Kernel issue #261,
 * "Non-goals and overlap"); these calls are the one-device part of it, built
 * on the associativity of log-sum-exp: lse = log sum_r exp(lse_r) over the
 * shares' lse_r, and the target logit lives in exactly one share. The
 * exchange between devices (an all-gather or all-reduce of 8 bytes per token
 * per share forward, a sum of the dH partials backward) is the caller's.
 * Targets are global rows: a token takes part when 0 <= t < Vt (else it gets
 * logp = +0 and zero gradients, as above); v0 >= 0, Vs >= 1, v0 + Vs <= Vt.
 *
 * linear_logp_shard_fwd: lse_shard [N] = log sum over the share's rows of
 * exp(z), and zt_shard [N] = the target logit z[n, t_n] where the share holds
 * t_n, else -inf (both float32, required). Workspace: the size
 * linear_logp_fwd_workspace_size(N, D, Vs, dtype) reports.
 */
LLP_API int linear_logp_shard_fwd(int64_t N, int64_t D, int64_t Vs, int64_t v0, int64_t Vt, int dtype,
                          const void* h, const void* W_shard, const void* b_shard,
                          const int64_t* targets, float* lse_shard, float* zt_shard,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Merge of P shares' forward results, share-major: lse_shards [P][N] and
 * zt_shards [P][N] (row r from the share r; any order of shares gives the
 * same lse up to rounding, a fixed order gives the same bits). lse [N] =
 * M + log sum_r exp(lse_r - M) with M = max_r lse_r, summed in increasing r;
 * logp [N] = zt - lse for 0 <= t < Vt (zt: the one finite zt_r), else +0.
 * Either output may be NULL, not both. No workspace.
 */
LLP_API int linear_logp_shard_combine(int64_t N, int64_t P, const float* lse_shards,
                              const float* zt_shards, const int64_t* targets, int64_t Vt,
                              float* logp, float* lse, void* stream);

/*
 * Backward of one share, given the global lse [N] (required, from
 * linear_logp_shard_combine) and g [N]. dH [N, D] or NULL receives this
 * share's PARTIAL dH = dlogits[:, v0:v0+Vs] W_shard, of dH_dtype (LLP_F32 or
 * the operand dtype; float32 keeps the sum over shares exact to float32
 * rounding); the caller sums the P partials. dW_shard [Vs, D] and db_shard
 * [Vs] are this share's rows of dW and db, complete (they need no exchange),
 * with dW_dtype, accumulate and chunk as in linear_logp_bwd. Workspace: the
 * size linear_logp_bwd_workspace_size(N, D, Vs, dtype, chunk, want_dH,
 * want_dW, want_db, 1) reports. Deterministic.
 */
LLP_API int linear_logp_shard_bwd(int64_t N, int64_t D, int64_t Vs, int64_t v0, int64_t Vt, int dtype,
                          int64_t chunk, const void* h, const void* W_shard, const void* b_shard,
                          const int64_t* targets, const float* g, const float* lse,
                          void* dH, int dH_dtype, void* dW_shard, int dW_dtype, void* db_shard,
                          int accumulate, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Logits-only forward (RL-Kernel PR #495): logits [N, V] of dtype ->
 * logp [N] (required), lse [N] (NULL to skip). One read of the logits.
 */
LLP_API int logp_fwd(int64_t N, int64_t V, int dtype, const void* logits, const int64_t* targets,
             float* logp, float* lse, void* stream);

/*
 * Logits-only backward: dlogits [N, V] (dtype) = g (onehot - softmax). With
 * lse from logp_fwd the logits are read once; lse = NULL recomputes it per
 * row (two reads). dlogits may alias logits (in-place gradient): each element
 * is read before it is written by the same thread.
 */
LLP_API int logp_bwd(int64_t N, int64_t V, int dtype, const void* logits, const int64_t* targets,
             const float* g, const float* lse, void* dlogits, void* stream);

/*
 * Tracing (opt-in, per calling thread). While enabled, every kernel the
 * library enqueues from this thread is bracketed by a pair of HIP events on
 * its stream, and the elapsed times are summed per kernel kind. Intended for
 * benchmarks that need per-kernel durations on the launch stream; the events
 * are created on first use and reused. Tracing does not change results.
 *
 * llp_trace_enable(1) starts (and clears) a trace; llp_trace_enable(0) stops.
 * llp_trace_read waits for the recorded events, then writes for each kind k
 * in [0, n) the total milliseconds ms[k] and the launch count count[k]
 * (either array may be NULL). Returns a status. At most LLP_TRACE_MAX
 * launches are recorded per trace; later ones are counted in
 * llp_trace_read's return of LLP_EOVERFLOW (the recorded ones stay valid).
 */
#define LLP_TRACE_MAX 65536
typedef enum {
  LLP_K_FWD_LSE = 0,    /* forward logits tile + online max/sum-exp partials (fused: per chunk) */
  LLP_K_COMBINE = 1,    /* per-token merge of partials -> logp, lse */
  LLP_K_DLOGITS = 2,    /* dlogits of a chunk: logits recompute, or (fused) from the numerators */
  LLP_K_DH_DW = 3,      /* dH and/or dW contractions of a chunk (one grid) */
  LLP_K_TRANSPOSE = 4,  /* W^T and per-chunk h^T operand copies */
  LLP_K_SMALL = 5,      /* chunk scales, target lists, db, zero fill */
  LLP_K_ROWS_FWD = 6,   /* logits-only forward */
  LLP_K_ROWS_BWD = 7,   /* logits-only backward */
  LLP_K_DH_DW_FWD = 8,  /* fused path: a chunk's dH / dW with the next chunk's forward tiles (one grid) */
  LLP_K_DH_REDUCE = 9,  /* sum of a dH contraction's vocabulary parts, in fixed order, and its epilogue */
  LLP_K_DH_DW_DL = 10,  /* backward: a chunk's dH / dW with the next chunk's dlogits recompute (one grid) */
  LLP_K_COUNT = 11
} llp_kernel_kind;
LLP_API int llp_trace_enable(int on);
LLP_API int llp_trace_read(double* ms, int64_t* count, int n);

#ifdef __cplusplus
}
#endif

#endif /* LLP_H */
