// Internal launch interface between the C-ABI layer (llp_api.hip) and the
// gfx950 kernels. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tile_config.h"

namespace llp {

// Per-token numerator mode (fused path, bf16): a 128-row block whose max m
// (log2 units) lies in [kQtokLo, kQtokHi] stores 2^(z log2 e) itself. The range
// keeps q and the fp32 sums of q W finite (m <= 64 nats) and keeps the
// probabilities that matter out of bf16's subnormals (m >= -40 nats).
constexpr float kQtokLo = -57.70780f;  // -40 log2 e
constexpr float kQtokHi = 92.33248f;   // 64 log2 e

// Element type codes (same values as llp_dtype).
enum Dt : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

inline int dt_size(int dt) { return dt == DT_F32 ? 4 : 2; }

// Epilogue kinds of the MFMA contraction C[m, n] = sum_k A[m, k] B[n, k].
enum Epi : int {
  EPI_NONE = 0,
  EPI_LSE_PARTIAL = 1,  // logits tile -> per-token (max, sum-exp) partials + target logit
  EPI_DLOGITS = 2,      // logits tile -> dlogits / scale, stored token-major and/or vocab-major
  EPI_STORE = 3,        // out[m, n] = scale * C, rounded to the operand dtype (dH)
  EPI_ACCUM = 4,        // table[m, n] += scale * C (dW, fp32 or operand-dtype table)
  EPI_LSE_Q = 5         // EPI_LSE_PARTIAL, plus the tile's exp2(z log2 e - m) stored vocab-major
};

// dlogits = g (onehot(t) - softmax(z)) is split into its softmax part
// -g p, stored in the operand dtype (divided by the chunk's power-of-two
// scale s) as the contraction operand, and its one-hot part g (1 - p_t), one
// fp32 value per token ("tcoef") that the epilogues add exactly:
//   dH[n, :] += tcoef[n] W[t_n, :],  dW[t_n, :] += tcoef[n] h[n, :],  db[t_n] += tcoef[n].
// A token takes part only if 0 <= t < V and g != 0 ("valid").
struct EpiParams {
  const void* bias;        // [V] operand dtype, or null
  const int64_t* targets;  // [tokens], indexed tok0 + local token
  const float* g;          // [tokens] upstream gradient
  int64_t tok0;            // first token of this problem
  int64_t V;               // vocabulary rows of this problem (a share's rows when sharded)
  // Vocabulary share: this problem's rows are [v0, v0 + V) of a vocabulary of
  // Vt rows (unsharded: v0 = 0, Vt = V). A token takes part when 0 <= t < Vt
  // and g != 0; its one-hot terms belong to the share holding t.
  int64_t v0;
  int64_t Vt;
  // EPI_LSE_PARTIAL (M = vocab, N = tokens)
  float2* partials;        // [kWaveM * tiles_m][ldp]: (max * log2 e, sum exp2) per wave-row block
  int64_t ldp;
  float* zt;               // [tokens] target logit
  // EPI_LSE_Q also stores q = exp2(z log2 e - m) (m: the wave-row block's max, the
  // partial's first member) into dSt [V][ldSt], +0 in columns [N, round8(N)).
  // With qtok (bf16 operands) it stores instead, for a block whose max lies in
  // [kQtokLo, kQtokHi] (log2 units), q = exp2(z log2 e), per-token units; a
  // block of -inf stores +0; any other block stores the block-relative q and
  // sets qflag[token] = 1. The target's entry is +0 in both cases.
  int qtok;
  int32_t* qflag;          // [tokens]
  // EPI_STORE with qtok: out = s rowf[token] C + tcoef W[t] (+0 where rowf is 0)
  const float* rowf;       // [tokens] per-token factor -(g / s) 2^(-lse log2 e), or null
  // EPI_DLOGITS (M = vocab, N = chunk tokens)
  const float* lse;        // [tokens]
  void* dS;                // [N][ldS] token-major softmax part / s, or null
  int64_t ldS;
  void* dSt;               // [V][ldSt] vocab-major softmax part / s, or null
  int64_t ldSt;
  float* tcoef;            // [tokens] one-hot part g (1 - p_t) (written here, read below)
  // EPI_STORE (M = chunk tokens, N = D): out = s C + tcoef W[t]
  const void* W;
  int64_t ldW;
  // EPI_ACCUM (M = V, N = D): table += s C + sum over the chunk's tokens with target m of tcoef h
  const void* h;
  int64_t ldh;
  // head == null: the one-hot rows were added to the table beforehand (FP32
  // table, see ChunkPrep) and the epilogue adds s C only
  const int32_t* head;     // [V] first chunk token with target v (entries for absent v are stale)
  const int32_t* next;     // [C] next chunk token with the same target, -1 at the end
  int64_t ntok;            // tokens in the chunk
  int tab_fast;            // FP32 table without one-hot part, D % 4 == 0, 16-byte aligned, tile span < 2 GiB
  int tab_fast16;          // operand-dtype (16-bit) table: D % 8 == 0, table and h 16-byte aligned, tile span < 2 GiB
  int tab_store;           // the table holds no values yet (first chunk, no accumulate): +0 stands in for
                           // the old values, which are not read (so no zero fill is needed)
  // EPI_STORE and EPI_ACCUM
  void* out;
  int64_t ldo;
  int out_dt;              // dtype of out (EPI_ACCUM table: DT_F32 or the operand dtype)
  // EPI_STORE of a split contraction (GemmProblem::kparts > 1): the tile of
  // part p stores its raw fp32 sums at dhp + p dhp_stride + m ldo + n, and
  // launch_dh_reduce applies the epilogue to their sum
  float* dhp;
  int64_t dhp_stride;
  // backward epilogues: scales[chunk] = (multiplier applied to C, divisor of the stored part)
  const float2* scales;
  int chunk;
};

struct GemmProblem {
  const void* A;  // [M][lda], K contiguous
  const void* B;  // [N][ldb], K contiguous
  int64_t lda, ldb;
  int64_t M, N, K;
  int a_vec, b_vec;  // 1: rows may be read with 16-byte vector loads
  int dma;           // 1: direct-to-LDS pipeline allowed (both operands 16-byte aligned, a 256-row
                     //    tile spans < 2 GiB, and K % (16 / esize) == 0 or the padding columns
                     //    up to the next multiple of 8 are +0)
  int mn;            // 1 (first problem of a STORE launch, 16-bit, DMA): A is stored [K][lda] and B
                     //    [K][ldb] (rows of the tile contiguous within a K row) instead of K-contiguous;
                     //    K * ld * esize < 2 GiB for both, ld % 8 == 0, 16-byte aligned
  int tiles_m, tiles_n;
  // K split into kparts fixed ranges of kpart (a multiple of 8) rows or
  // columns (STORE problems only; 0 or 1: no split); the grid then holds
  // tiles_m * tiles_n * kparts tiles, part-major
  int kparts;
  int64_t kpart;
  int epi;
  EpiParams ep;
};

inline int problem_tiles(const GemmProblem& p) { return p.tiles_m * p.tiles_n * (p.kparts > 1 ? p.kparts : 1); }

// Launch one or two independent problems of the same operand dtype in one
// grid (the second problem's tiles follow the first's). Returns hipError_t.
hipError_t launch_gemm(int dt, const GemmProblem* p0, const GemmProblem* p1, hipStream_t s);
// A chunk's dH (p0: EPI_STORE, K-row-major operands) and dW (p1: EPI_ACCUM,
// fast epilogue, or null) with the next chunk's forward (p2: EPI_LSE_Q) in one
// grid; 16-bit operands, DMA pipeline. Returns hipErrorInvalidValue otherwise.
hipError_t launch_gemm3(int dt, const GemmProblem& p0, const GemmProblem* p1, const GemmProblem& p2, hipStream_t s);

// partials [P][N] + zt -> logp, lse (one thread per token, fixed order over P).
// With cq (per-token mode), also cq[n] = -(g / s) 2^(-lse log2 e) for a valid token
// without qflag, -(g / s) with it, +0 otherwise (s from sc = (s, 1 / s)).
hipError_t launch_lse_combine(const float2* partials, int64_t P, int64_t ldp, const float* zt,
                              const int64_t* targets, int64_t V, int64_t N, float* logp,
                              float* lse, const float* g, float* tcoef, hipStream_t s,
                              const int32_t* qflag = nullptr, const float2* sc = nullptr, float* cq = nullptr);

// Fused forward + backward: softmax part of one chunk's dlogits from the stored
// numerators, in place (vocab-major) and transposed into dS (token-major; dS may
// be null when only the vocab-major copy is needed).
hipError_t launch_softmax_grad(int dt, void* qt, int64_t ldq, const float2* partials, int64_t ldp,
                               const float* lse, const float* g, const int64_t* targets,
                               const float2* scales, int chunk, int64_t V, int64_t C, void* dS,
                               int64_t ldS, hipStream_t s);

// dst[c][r] = src[r][c] for r < rows, c < cols (element size from dt); the
// padding columns r in [rows, round8(rows)) of each dst row are set to +0.
hipError_t launch_transpose(int dt, const void* src, int64_t rows, int64_t cols, int64_t lds,
                            void* dst, int64_t ldd, hipStream_t s);

// scales[k] = (s 2^-headroom, 2^headroom / s), s = smallest power of two >= max |g|
// over chunk k (1 if that is 0); headroom = 15 for fp16 operands, else 0.
hipError_t launch_chunk_scales(const float* g, int64_t N, int64_t C, int64_t K, int headroom,
                               float2* scales, hipStream_t s);

// db[v] += s_k * sum_{c < C} dSt[v][c] + sum of tcoef over the chunk's tokens with target v
// (table dtype tdt; dSt in operand dtype dt).
hipError_t launch_db_accum(int dt, const void* dSt, int64_t ldSt, int64_t V, int64_t C,
                           const float2* scales, int chunk, const int32_t* head, const int32_t* next,
                           const int64_t* targets, const float* g, const float* tcoef, int64_t tok0,
                           int64_t v0, int64_t Vt, void* db, int tdt, hipStream_t s,
                           const float* cq = nullptr);

// Per chunk [tok0, tok0 + C): head[t] = first valid token with target t and
// next[n] = the following one (-1 at the end), local indices, in token order.
// Only head entries of targets present in the chunk are written.
hipError_t launch_target_lists(const int64_t* targets, const float* g, int64_t tok0, int64_t C,
                               int64_t V, int64_t v0, int64_t Vt, int32_t* head, int32_t* next, hipStream_t s);
// Merge of P vocabulary shares' (lse, target logit) per token -> logp, lse.
hipError_t launch_shard_combine(const float* lse_sh, const float* zt_sh, int64_t P, int64_t N,
                                const int64_t* targets, int64_t Vt, float* logp, float* lse, hipStream_t s);

// The per-chunk preparation of the dH / dW contraction in one launch (its
// parts are independent): the one-hot rows of an FP32 dW table (when table !=
// null: table[t, :] += sum over the chunk's valid tokens j with target t, in
// increasing j, of tcoef[j] h[j, :]; the contraction then adds only its dense
// part), the target lists (when head != null, as launch_target_lists), h rows
// [tok0, tok0 + C) transposed into ht [D][ldht] (when ht != null, as
// launch_transpose) and the softmax gradient of the fused path (when qt !=
// null, as launch_softmax_grad, whose per-token arrays lse, gc, tc start at
// the chunk).
struct ChunkPrep {
  int64_t C, V;
  // per-token mode of the fused path (bf16): no softmax-gradient pass; the h
  // transpose multiplies token n's row by cq[n] (chunk-local pointer) and the
  // columns of flagged tokens (qflag) are rescaled to 2^(z log2 e - lse log2 e)
  const float* cq;
  const int32_t* qflag;
  // target lists and one-hot rows (targets, g, tcoef indexed tok0 + local token)
  const int64_t* targets;
  const float* g;
  int64_t tok0, v0, Vt;
  int32_t* head;
  int32_t* next;
  const float* tcoef;
  float* table;  // [V][ldt] FP32 dW table, or null
  int64_t ldt;
  // one-hot rows of tokens [oh_tok0, oh_tok0 + oh_C) (h rows from oh_h); may
  // span the previous chunk too when that chunk's rows were deferred
  int64_t oh_tok0, oh_C;
  const void* oh_h;
  // transpose of the chunk's h rows (also read by the one-hot rows)
  const void* h;  // first row of the chunk
  int64_t D;
  void* ht;
  int64_t ldht;
  // softmax gradient
  void* qt;
  int64_t ldq;
  const float2* partials;
  int64_t ldp;
  const float* lse;
  const float* gc;
  const int64_t* tc;
  const float2* scales;
  int chunk;
  void* dS;
  int64_t ldS;
  // the previous dH contraction's reduction (as launch_dh_reduce), when
  // rd_part != null: it runs in the same launch, beside the parts above
  const float* rd_part;
  int64_t rd_stride;
  int rd_S;
  int64_t rd_M, rd_D;
  EpiParams rd_ep;
};
hipError_t launch_chunk_prep(int dt, const ChunkPrep& c, hipStream_t s);

// dH rows of a split contraction: out[m, n] = the EPI_STORE epilogue (row
// factor s rowf, one-hot term tcoef W[t], rounding to out_dt) applied to
// sum_{p = 0 .. S - 1} part[p][m][n], summed in increasing p; m < M, n < D. `e` carries the STORE epilogue's parameters (tok0 = the
// first token of row 0).
hipError_t launch_dh_reduce(int dt, const float* part, int64_t stride, int S, int64_t M, int64_t D,
                            const EpiParams& e, hipStream_t s);

// Fill n elements of size esize with +0.
hipError_t launch_zero(void* p, int64_t n, int esize, hipStream_t s);
// Fill n 4-byte words (p 4-byte aligned) with the bit pattern `word`.
hipError_t launch_fill32(uint32_t* p, int64_t n, uint32_t word, hipStream_t s);

// Logits-only rows.
hipError_t launch_rows_fwd(int dt, const void* logits, int64_t N, int64_t V,
                           const int64_t* targets, float* logp, float* lse, hipStream_t s);
hipError_t launch_rows_bwd(int dt, const void* logits, int64_t N, int64_t V,
                           const int64_t* targets, const float* g, const float* lse,
                           void* dlogits, hipStream_t s);

}  // namespace llp
