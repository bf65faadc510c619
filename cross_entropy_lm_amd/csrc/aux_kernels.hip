// Small kernels around the MFMA contractions: the log-sum-exp combine, operand
// transposes, per-chunk gradient scales, the db reduction and zero fill.
#include "kernels.h"

#include <math.h>

#include <algorithm>

namespace llp {
namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;

// Per token: merge the per-block (m, s) partials (m in log2 units, s = sum of
// 2^(y - m)), then lse = (M + log2 S) ln 2 and logp = z[t] - lse for a target
// in [0, V), else +0 (RL-Kernel PR #495, "Behavior changes"). A block of 1024
// threads takes 16 tokens; the 64 threads of a token merge the partials
// i = j, j + 64, ... in increasing i (loaded kCombBatch at a time), then the 64
// results are merged by a fixed pairwise tree (j with j + 32, then j + 16,
// ...): an order that depends on neither the batch size nor the chunking.
// Loads are coalesced over the 16 consecutive tokens (one 128-byte line).
// With g and tcoef (fused forward + backward) it also writes the one-hot
// part tcoef[n] = g (1 - p_t), p_t = 2^(z_t log2 e - lse log2 e), for a valid
// token (0 <= t < V, g != 0), else +0.
constexpr int kCombTok = 16, kCombSl = 64, kCombBatch = 4;
__device__ __forceinline__ void lse_merge(float& M, float& S, float m, float s) {
  if (m == -INFINITY) return;
  if (m > M) {
    S = S * __builtin_amdgcn_exp2f(M - m) + s;
    M = m;
  } else {
    S += s * __builtin_amdgcn_exp2f(m - M);
  }
}
__global__ __launch_bounds__(kCombTok * kCombSl) void lse_combine_kernel(
    const float2* __restrict__ partials, int64_t P, int64_t ldp, const float* __restrict__ zt,
    const int64_t* __restrict__ targets, int64_t V, int64_t N, float* __restrict__ logp,
    float* __restrict__ lse, const float* __restrict__ g, float* __restrict__ tcoef,
    const int32_t* __restrict__ qflag, const float2* __restrict__ sc, float* __restrict__ cq) {
  __shared__ float2 part[kCombSl][kCombTok];
  const int tk = threadIdx.x % kCombTok, sl = threadIdx.x / kCombTok;
  const int64_t n = (int64_t)blockIdx.x * kCombTok + tk;
  float M = -INFINITY, S = 0.0f;
  if (n < N)
    for (int64_t i0 = sl; i0 < P; i0 += kCombSl * kCombBatch) {
      float2 q[kCombBatch];
#pragma unroll
      for (int u = 0; u < kCombBatch; ++u) {
        const int64_t i = i0 + u * kCombSl;
        q[u] = i < P ? partials[i * ldp + n] : make_float2(-INFINITY, 0.0f);
      }
#pragma unroll
      for (int u = 0; u < kCombBatch; ++u) lse_merge(M, S, q[u].x, q[u].y);
    }
  part[sl][tk] = make_float2(M, S);
#pragma unroll
  for (int w = kCombSl / 2; w >= 1; w >>= 1) {
    __syncthreads();
    if (sl < w) {
      const float2 o = part[sl + w][tk];
      lse_merge(M, S, o.x, o.y);
      part[sl][tk] = make_float2(M, S);
    }
  }
  if (sl != 0 || n >= N) return;
  const float l = (M + __builtin_amdgcn_logf(S)) * kLn2;
  if (lse != nullptr) lse[n] = l;
  const int64_t t = targets[n];
  if (logp != nullptr) logp[n] = (t >= 0 && t < V) ? zt[n] - l : 0.0f;
  if (tcoef != nullptr) {
    const float gv = g[n];
    const float pt = (t >= 0 && t < V) ? __builtin_amdgcn_exp2f(fmaf(zt[n], kLog2e, -(l * kLog2e))) : 0.0f;
    tcoef[n] = (t >= 0 && t < V && gv != 0.0f) ? fmaf(-gv, pt, gv) : 0.0f;
  }
  if (cq != nullptr) {
    // per-token mode: the factor that turns the stored 2^(z log2 e) into -(g / s) p
    // (a flagged token's column is rescaled to p itself before use)
    const float gv = g[n];
    const float e = qflag[n] ? 1.0f : __builtin_amdgcn_exp2f(-(l * kLog2e));
    cq[n] = (t >= 0 && t < V && gv != 0.0f) ? -(gv * sc[0].y) * e : 0.0f;
  }
}

// Fused forward + backward, one chunk of C tokens: from the stored numerators
// q [v][n] (vocab-major, q = 2^(z log2 e - m_b) with m_b the max of the 128-row
// vocab block b = v / 128 of token n, the first member of partials[b][n]),
// the softmax part of dlogits divided by the chunk's scale,
//     d[v][n] = -(g_n / s) q 2^(m_b - lse_n log2 e)   for a valid token n, v != t_n,
//     d[v][n] = +0                                      otherwise,
// written in place over q and, transposed, into dS [n][v] (token-major, +0 in
// the columns [V, round8(V)); skipped when dS is null). 64 x 64 tiles, 256
// threads, 16-byte accesses along rows where the tile is complete.
template <typename T>
struct SoftmaxGradArgs {
  T* qt;
  int64_t ldq;
  const float2* partials;
  int64_t ldp;
  const float* lse;
  const float* g;
  const int64_t* targets;
  const float2* scales;
  int chunk;
  int64_t V, C;
  T* dS;
  int64_t ldS;
  // per-token mode: only the columns of flagged tokens are rescaled (qfix_tile)
  const int32_t* qflag;
};

template <typename T>
constexpr int softmax_grad_lds() {
  return 64 * (64 + 16 / (int)sizeof(T)) * (int)sizeof(T) + 64 * 4 + 64 * 4;
}

template <typename T>
__device__ __forceinline__ void softmax_grad_tile(int64_t bx, int64_t by, const SoftmaxGradArgs<T>& a, char* smem) {
  T* __restrict__ qt = a.qt;
  const int64_t ldq = a.ldq, ldp = a.ldp, V = a.V, C = a.C, ldS = a.ldS;
  const float2* __restrict__ partials = a.partials;
  const float* __restrict__ lse = a.lse;
  const float* __restrict__ g = a.g;
  const int64_t* __restrict__ targets = a.targets;
  const float2* __restrict__ scales = a.scales;
  const int chunk = a.chunk;
  T* __restrict__ dS = a.dS;
  constexpr int kVec = 16 / (int)sizeof(T);  // elements per 16 bytes
  constexpr int kCpr = 64 / kVec;            // 16-byte chunks per 64-element row
  constexpr int kRpp = 256 / kCpr;           // rows per pass
  typedef __attribute__((__vector_size__(16))) unsigned int u32x4;
  T(*tile)[64 + kVec] = reinterpret_cast<T(*)[64 + kVec]>(smem);  // [64][64 + kVec]
  float* coef_s = reinterpret_cast<float*>(smem + 64 * (64 + kVec) * sizeof(T));
  int32_t* t_s = reinterpret_cast<int32_t*>(coef_s + 64);
  const int64_t v0 = bx * 64, n0 = by * 64;
  const int c = threadIdx.x % kCpr;
  const bool full_n = n0 + (c + 1) * kVec <= C;
  constexpr int kPass = 64 / kRpp;
  // the tile's numerators are loaded first (they do not depend on the
  // coefficients), and the coefficients' loads are unconditional (clamped
  // index), so a tile waits for about one round trip
  u32x4 x[kPass];
#pragma unroll
  for (int ps = 0; ps < kPass; ++ps) {
    const int64_t v = v0 + threadIdx.x / kCpr + ps * kRpp;
    if (v < V && full_n) x[ps] = *reinterpret_cast<const u32x4*>(qt + v * ldq + n0 + c * kVec);
  }
  if (threadIdx.x < 64) {
    // column n: the token's factor -(g / s) 2^(m_b - lse log2 e); 64-row tiles lie in one 128-row block
    const int64_t n = n0 + threadIdx.x;
    const int64_t nc = n < C ? n : C - 1;
    const int64_t tt = targets[nc];
    const float gv = g[nc];
    const float m2 = partials[(v0 >> 7) * ldp + nc].x;
    const float ln = lse[nc];
    float coef = 0.0f;
    int32_t t = -1;
    if (n < C && tt >= 0 && tt < V && gv != 0.0f) {
      const float f = (m2 == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m2 - ln * kLog2e);
      coef = -(gv * scales[chunk].y) * f;
      t = (int32_t)tt;
    }
    coef_s[threadIdx.x] = coef;
    t_s[threadIdx.x] = t;
  }
  __syncthreads();
#pragma unroll
  for (int ps = 0; ps < kPass; ++ps) {
    const int i = threadIdx.x / kCpr + ps * kRpp;
    const int64_t v = v0 + i;
    T val[kVec];
    if (v < V && full_n) {
      T* q = qt + v * ldq + n0 + c * kVec;
      *reinterpret_cast<u32x4*>(val) = x[ps];
#pragma unroll
      for (int j = 0; j < kVec; ++j) {
        const int nl = c * kVec + j;
        const int32_t t = t_s[nl];
        val[j] = (T)((t >= 0 && v != t) ? coef_s[nl] * (float)val[j] : 0.0f);
      }
      *reinterpret_cast<u32x4*>(q) = *reinterpret_cast<const u32x4*>(val);
    } else {
#pragma unroll
      for (int j = 0; j < kVec; ++j) {
        const int nl = c * kVec + j;
        const int64_t n = n0 + nl;
        val[j] = (T)0;
        if (v < V && n < C) {
          T* q = qt + v * ldq + n;
          const int32_t t = t_s[nl];
          val[j] = (T)((t >= 0 && v != t) ? coef_s[nl] * (float)*q : 0.0f);
          *q = val[j];
        }
      }
    }
    if (dS != nullptr) {  // uniform: the token-major copy goes through LDS
#pragma unroll
      for (int j = 0; j < kVec; ++j) tile[i][c * kVec + j] = val[j];
    }
  }
  if (dS == nullptr) return;  // uniform
  __syncthreads();
  const int64_t vpad = (V + 7) & ~int64_t(7);
  const int64_t vs = v0 + c * kVec;  // this thread's kVec vocab columns of dS
  for (int i = threadIdx.x / kCpr; i < 64; i += kRpp) {
    const int64_t n = n0 + i;
    if (n >= C || vs >= vpad) continue;
    T val[kVec];
#pragma unroll
    for (int j = 0; j < kVec; ++j) val[j] = tile[c * kVec + j][i];
    T* o = dS + n * ldS + vs;
    if (vs + kVec <= vpad) {
      *reinterpret_cast<u32x4*>(o) = *reinterpret_cast<const u32x4*>(val);
    } else {
#pragma unroll
      for (int j = 0; j < kVec; ++j)
        if (vs + j < vpad) o[j] = val[j];
    }
  }
}

// Per-token mode: the column of a token whose numerators were stored partly
// block-relative (qflag set) becomes 2^(z log2 e - lse log2 e) = p, in place:
// a block b (128 rows) in range holds 2^(z log2 e) (factor 2^(-lse log2 e)),
// any other block 2^(z log2 e - m_b) (factor 2^(m_b - lse log2 e)), a block of
// -inf holds +0. The same range test as the forward's. A workgroup takes 64
// tokens x 1024 vocab rows and returns at once when none of its tokens is flagged.
template <typename T>
__device__ __forceinline__ void qfix_tile(int64_t bx, int64_t by, const SoftmaxGradArgs<T>& a) {
  const int tn = threadIdx.x & 63, rg = threadIdx.x >> 6;
  const int64_t n = by * 64 + tn;
  const bool fl = n < a.C && a.qflag[n] != 0;
  if (!__syncthreads_or(fl ? 1 : 0)) return;
  if (!fl) return;  // no barrier follows
  const float l2 = a.lse[n] * kLog2e;
  const int64_t v0 = bx * 1024, v1 = (a.V < v0 + 1024) ? a.V : v0 + 1024;
  int64_t bcur = -1;
  float fac = 0.0f;
  for (int64_t v = v0 + rg; v < v1; v += 4) {
    const int64_t b = v >> 7;
    if (b != bcur) {
      bcur = b;
      const float m2 = a.partials[b * a.ldp + n].x;
      const bool inr = m2 >= kQtokLo && m2 <= kQtokHi;
      fac = (m2 == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((inr ? 0.0f : m2) - l2);
    }
    T* q = a.qt + v * a.ldq + n;
    *q = (T)((float)*q * fac);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void softmax_grad_kernel(SoftmaxGradArgs<T> a) {
  __shared__ __attribute__((aligned(16))) char smem[softmax_grad_lds<T>()];
  softmax_grad_tile<T>(blockIdx.x, blockIdx.y, a, smem);
}

// Vocabulary-parallel merge: per token, the P shares' (lse_r, zt_r) (zt_r =
// -inf unless share r holds the target) in increasing r:
// lse = M + log sum_r exp(lse_r - M), M = max_r lse_r; logp = zt_owner - lse
// for a target in [0, Vt), else +0. A share with no finite lse (every logit
// -inf) adds nothing.
__global__ void shard_combine_kernel(const float* __restrict__ lse_sh, const float* __restrict__ zt_sh,
                                     int64_t P, int64_t N, const int64_t* __restrict__ targets, int64_t Vt,
                                     float* __restrict__ logp, float* __restrict__ lse) {
  const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  float M = -INFINITY;
  float zt = -INFINITY;
  for (int64_t r = 0; r < P; ++r) {
    M = fmaxf(M, lse_sh[r * N + n]);
    const float z = zt_sh[r * N + n];
    if (z != -INFINITY) zt = z;
  }
  float S = 0.0f;
  if (M != -INFINITY)
    for (int64_t r = 0; r < P; ++r) {
      const float l = lse_sh[r * N + n];
      if (l != -INFINITY) S += __builtin_amdgcn_exp2f((l - M) * kLog2e);
    }
  const float l = M + __builtin_amdgcn_logf(S) * kLn2;
  if (lse != nullptr) lse[n] = l;
  const int64_t t = targets[n];
  if (logp != nullptr) logp[n] = (t >= 0 && t < Vt) ? zt - l : 0.0f;
}

// dst[c][r] = src[r][c] for r < rows, c < cols, and +0 in the padding columns
// r in [rows, round8(rows)) of dst. 64 x 64 tiles through LDS, 256 threads;
// 16-byte row segments on both sides where the tile is complete and aligned.
template <typename T>
struct TransposeArgs {
  const T* src;
  int64_t rows, cols, lds;
  T* dst;
  int64_t ldd;
  int vec;
  const float* rowscale;  // [rows] or null: dst[c][r] = src[r][c] rowscale[r], rounded once
};

template <typename T>
constexpr int transpose_lds() {
  return 64 * (64 + 2) * (int)sizeof(T);
}

template <typename T>
__device__ __forceinline__ void transpose_tile(int64_t bx, int64_t by, const TransposeArgs<T>& a, char* smem) {
  const T* __restrict__ src = a.src;
  T* __restrict__ dst = a.dst;
  const int64_t rows = a.rows, cols = a.cols, lds = a.lds, ldd = a.ldd;
  const int vec = a.vec;
  constexpr int kVec = 16 / (int)sizeof(T);  // elements per 16 bytes
  constexpr int kCpr = 64 / kVec;            // 16-byte chunks per 64-element row
  constexpr int kRpp = 256 / kCpr;           // rows per pass
  typedef __attribute__((__vector_size__(16))) unsigned int u32x4;
  T(*tile)[64 + 2] = reinterpret_cast<T(*)[64 + 2]>(smem);  // [64][66]
  const int64_t r0 = bx * 64, c0 = by * 64;
  const int ch = threadIdx.x % kCpr;
  for (int i = threadIdx.x / kCpr; i < 64; i += kRpp) {
    const int64_t r = r0 + i, c = c0 + ch * kVec;
    T v[kVec];
    if (vec && r < rows && c + kVec <= cols) {
      *reinterpret_cast<u32x4*>(v) = *reinterpret_cast<const u32x4*>(src + r * lds + c);
    } else {
#pragma unroll
      for (int j = 0; j < kVec; ++j) v[j] = (r < rows && c + j < cols) ? src[r * lds + c + j] : (T)0;
    }
    if (a.rowscale != nullptr && r < rows) {
      const float rs = a.rowscale[r];
#pragma unroll
      for (int j = 0; j < kVec; ++j) v[j] = (T)((float)v[j] * rs);
    }
#pragma unroll
    for (int j = 0; j < kVec; ++j) tile[i][ch * kVec + j] = v[j];
  }
  __syncthreads();
  const int64_t rpad = (rows + 7) & ~int64_t(7);
  for (int i = threadIdx.x / kCpr; i < 64; i += kRpp) {
    const int64_t c = c0 + i, r = r0 + ch * kVec;
    if (c >= cols || r >= rpad) continue;
    T v[kVec];
#pragma unroll
    for (int j = 0; j < kVec; ++j) v[j] = tile[ch * kVec + j][i];  // +0 past rows
    T* o = dst + c * ldd + r;
    if (vec && r + kVec <= rpad) {
      *reinterpret_cast<u32x4*>(o) = *reinterpret_cast<const u32x4*>(v);
    } else {
#pragma unroll
      for (int j = 0; j < kVec; ++j)
        if (r + j < rpad) o[j] = v[j];
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(TransposeArgs<T> a) {
  __shared__ __attribute__((aligned(16))) char smem[transpose_lds<T>()];
  transpose_tile<T>(blockIdx.x, blockIdx.y, a, smem);
}

// s = smallest power of two >= max |g| over the chunk (1 if that maximum is 0
// or not finite), so that the stored softmax part (g / s) p lies in [-1, 1];
// `headroom` further multiplies it by 2^headroom (15 for fp16, whose normal
// range would otherwise lose the typical p ~ 1/V to subnormals; 2^15 * 1 stays
// below fp16's maximum). scales[k] = (s 2^-headroom, 2^headroom / s): the
// first undoes the second exactly in the epilogues.
__global__ void chunk_scales_kernel(const float* __restrict__ g, int64_t N, int64_t C, int headroom,
                                    float2* __restrict__ scales) {
  __shared__ float red[4];
  const int64_t k = blockIdx.x;
  const int64_t c0 = k * C, c1 = min(N, c0 + C);
  float m = 0.0f;
  for (int64_t i = c0 + threadIdx.x; i < c1; i += blockDim.x) m = fmaxf(m, fabsf(g[i]));
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    int e = 0;
    if (m > 0.0f && isfinite(m)) {
      frexpf(m, &e);  // m = f 2^e, f in [0.5, 1)  ->  2^e >= m
      e = max(-100, min(100, e));
    }
    scales[k] = make_float2(ldexpf(1.0f, e - headroom), ldexpf(1.0f, headroom - e));
  }
}

// A token that takes part (0 <= t < Vt, g != 0) and whose target lies in the
// vocabulary share [v0, v0 + V); t is returned as the local row.
__device__ __forceinline__ bool tok_valid(const int64_t* targets, const float* g, int64_t tok,
                                          int64_t V, int64_t v0, int64_t Vt, int64_t& t) {
  const int64_t tg = targets[tok];
  t = tg - v0;
  return tg >= 0 && tg < Vt && t >= 0 && t < V && g[tok] != 0.0f;
}

template <typename T, typename TT>
__global__ void db_accum_kernel(const T* __restrict__ dSt, int64_t ldSt, int64_t V, int64_t C,
                                const float2* __restrict__ scales, int chunk,
                                const int32_t* __restrict__ head, const int32_t* __restrict__ next,
                                const int64_t* __restrict__ targets, const float* __restrict__ g,
                                const float* __restrict__ tcoef, int64_t tok0, int64_t v0, int64_t Vt,
                                TT* __restrict__ db, const float* __restrict__ cq) {
  const int lane = threadIdx.x & 63;
  const int64_t v = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (v >= V) return;  // uniform per wave
  // the row in 16-byte pieces when its start allows (lane l sums pieces l,
  // l + 64, ..., each piece's elements in order), then the remaining
  // elements one per lane; in per-token mode each stored value is multiplied
  // by its token's factor (chunk-local cq) first
  constexpr int kv = 16 / (int)sizeof(T);
  typedef __attribute__((__vector_size__(16))) unsigned int u32x4;
  const T* row = dSt + v * ldSt;
  const int64_t nv = (reinterpret_cast<uintptr_t>(row) % 16 == 0) ? C / kv : 0;  // whole pieces
  float s = 0.0f;
  for (int64_t q = lane; q < nv; q += 64) {
    T x[kv];
    *reinterpret_cast<u32x4*>(x) = *reinterpret_cast<const u32x4*>(row + q * kv);
    if (cq == nullptr) {
#pragma unroll
      for (int i = 0; i < kv; ++i) s += (float)x[i];
    } else {
#pragma unroll
      for (int i = 0; i < kv; ++i) s += (float)x[i] * cq[q * kv + i];
    }
  }
  for (int64_t c = nv * kv + lane; c < C; c += 64) s += cq == nullptr ? (float)row[c] : (float)row[c] * cq[c];
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) {
    float val = s * scales[chunk].x;
    int32_t j = head[v];
    int64_t t;
    if (j >= 0 && j < C && tok_valid(targets, g, tok0 + j, V, v0, Vt, t) && t == v) {
      for (int64_t it = 0; it < C && j >= 0 && j < C; ++it) {
        val += tcoef[tok0 + j];
        j = next[j];
      }
    }
    db[v] = (TT)((float)db[v] + val);
  }
}

// One wave per chunk token n: the 64 lanes split the scan over the chunk, then
// a valid token with no earlier valid token of the same target writes
// head[t], and every valid token writes next[n] (the first later valid token
// with the same target, or -1). No atomics: the lists are in token order.
struct ListArgs {
  const int64_t* targets;
  const float* g;
  int64_t tok0, C, V, v0, Vt;
  int32_t* head;
  int32_t* next;
};

__device__ __forceinline__ void target_lists_block(int64_t bx, const ListArgs& a) {
  const int64_t* __restrict__ targets = a.targets;
  const float* __restrict__ g = a.g;
  const int64_t tok0 = a.tok0, C = a.C, V = a.V, v0 = a.v0, Vt = a.Vt;
  int32_t* __restrict__ head = a.head;
  int32_t* __restrict__ next = a.next;
  const int lane = threadIdx.x & 63;
  const int64_t n = bx * 4 + (threadIdx.x >> 6);  // 256 threads: four tokens
  if (n >= C) return;  // uniform per wave
  int64_t t;
  if (!tok_valid(targets, g, tok0 + n, V, v0, Vt, t)) return;
  bool earlier = false;
  int64_t nxt = INT64_MAX;
  for (int64_t j = lane; j < C; j += 64) {
    int64_t tj;
    if (j != n && tok_valid(targets, g, tok0 + j, V, v0, Vt, tj) && tj == t) {
      if (j < n) earlier = true;
      else if (j < nxt) nxt = j;
    }
  }
  // every lane takes part in every shuffle (no short-circuit around them)
  int any_earlier = earlier ? 1 : 0;
  for (int o = 32; o > 0; o >>= 1) {
    any_earlier |= __shfl_xor(any_earlier, o);
    const int64_t other = __shfl_xor(nxt, o);
    nxt = other < nxt ? other : nxt;
  }
  earlier = any_earlier != 0;
  if (lane == 0) {
    next[n] = nxt == INT64_MAX ? -1 : (int32_t)nxt;
    if (!earlier) head[t] = (int32_t)n;
  }
}

__global__ __launch_bounds__(256) void target_lists_kernel(ListArgs a) { target_lists_block(blockIdx.x, a); }

// One-hot rows of an FP32 dW table for one chunk: for every vocabulary row t
// that is the target of valid tokens of the chunk,
//     table[t, :] += sum over those tokens j, in increasing j, of tcoef[j] h[j, :]
// (fp32, the sum formed from +0 and added to the table once per batch of up to
// kOhCap - 2048 tokens, so once for any realistic chunk). The dense part
// s * (dlogits^T h) is added afterwards by the contraction's epilogue.
// Block n takes the row of token n's target when n is the first valid token
// with that target, so every row has one writer and a fixed order of
// additions; the other blocks return after the scan.
template <typename T>
struct OnehotArgs {
  const int64_t* targets;  // indexed tok0 + local token, as g and tcoef
  const float* g;
  const float* tcoef;
  int64_t tok0, C, V, v0, Vt;
  const T* h;  // the chunk's first row
  int64_t ldh, D;
  float* table;  // [V][ldt]
  int64_t ldt;
  int vec;  // h rows and table rows may be accessed in 16-byte pieces
};
constexpr int kOhPer = 8;    // table columns per thread and pass (2048 per pass of 256 threads)
constexpr int kOhWin = 8;    // 256-token windows whose targets a thread loads at once
constexpr int kOhGroup = kOhWin * 256;
constexpr int kOhCap = 2 * kOhGroup;  // list entries (a flush is due once more than kOhCap - kOhGroup)
constexpr int onehot_lds() { return kOhCap * 4 + kOhWin * 4 * 4; }

template <typename T>
__device__ __forceinline__ void load_piece(const T* p, float (&x)[kOhPer]) {
  typedef __attribute__((__vector_size__(16))) unsigned int u32x4;
  constexpr int kv = 16 / (int)sizeof(T);
#pragma unroll
  for (int q = 0; q < kOhPer / kv; ++q) {
    T v[kv];
    *reinterpret_cast<u32x4*>(v) = *reinterpret_cast<const u32x4*>(p + q * kv);
#pragma unroll
    for (int i = 0; i < kv; ++i) x[q * kv + i] = (float)v[i];
  }
}

template <typename T>
__device__ __forceinline__ void onehot_rows_block(int64_t n, const OnehotArgs<T>& a, char* smem) {
  int32_t* lst = reinterpret_cast<int32_t*>(smem);
  int(*wcnt)[4] = reinterpret_cast<int(*)[4]>(smem + kOhCap * 4);  // [kOhWin][4]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t* __restrict__ targets = a.targets + a.tok0;
  const float* __restrict__ g = a.g + a.tok0;
  const int64_t tn = targets[n];
  const float gn = g[n];
  const int64_t t = tn - a.v0;
  const bool valid = tn >= 0 && tn < a.Vt && t >= 0 && t < a.V && gn != 0.0f;
  float* row = a.table + (valid ? t : 0) * a.ldt;
  // row += sum over the listed tokens of tcoef h, in list order; the row's old
  // values are loaded before the h rows, so a pass waits about one round trip
  auto flush = [&](int count) {
#pragma unroll 1
    for (int64_t d = (int64_t)tid * kOhPer; d < a.D; d += 256 * kOhPer) {
      const bool full = a.vec && d + kOhPer <= a.D;
      float o[kOhPer], acc[kOhPer];
      if (full) {
        load_piece(row + d, o);
      } else {
#pragma unroll
        for (int i = 0; i < kOhPer; ++i) o[i] = (d + i < a.D) ? row[d + i] : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < kOhPer; ++i) acc[i] = 0.0f;
#pragma unroll 1
      for (int e = 0; e < count; ++e) {
        const int64_t j = lst[e];
        const T* hr = a.h + j * a.ldh + d;
        const float c = a.tcoef[a.tok0 + j];
        float x[kOhPer];
        if (full) {
          load_piece(hr, x);
        } else {
#pragma unroll
          for (int i = 0; i < kOhPer; ++i) x[i] = (d + i < a.D) ? (float)hr[i] : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kOhPer; ++i) acc[i] = fmaf(c, x[i], acc[i]);
      }
#pragma unroll
      for (int i = 0; i < kOhPer; ++i) o[i] += acc[i];
      if (full) {
        typedef __attribute__((__vector_size__(16))) unsigned int u32x4;
#pragma unroll
        for (int q = 0; q < kOhPer / 4; ++q)
          *reinterpret_cast<u32x4*>(row + d + q * 4) = *reinterpret_cast<const u32x4*>(o + q * 4);
      } else {
#pragma unroll
        for (int i = 0; i < kOhPer; ++i)
          if (d + i < a.D) row[d + i] = o[i];
      }
    }
  };
  // scan the chunk in groups of kOhWin x 256 tokens, one round trip each (the
  // loads use clamped indices, so they are unconditional): a valid token
  // earlier than n with the same target means another block owns the row; the
  // tokens j >= n with the target are appended to the list in increasing j
  int count = 0;  // uniform over the block
  for (int64_t base = 0; base < a.C; base += kOhGroup) {
    bool m[kOhWin];
#pragma unroll
    for (int w = 0; w < kOhWin; ++w) {
      const int64_t j = base + w * 256 + tid;
      const int64_t jc = j < a.C ? j : a.C - 1;
      const int64_t tj = targets[jc];
      const float gj = g[jc];
      m[w] = (j < a.C) & (tj >= 0) & (tj < a.Vt) & (tj - a.v0 == t) & (gj != 0.0f);
    }
    if (!valid) return;  // uniform over the block
    int earlier = 0;
#pragma unroll
    for (int w = 0; w < kOhWin; ++w) earlier |= (m[w] & (base + w * 256 + tid < n)) ? 1 : 0;
    if (__syncthreads_or(earlier)) return;
    uint64_t bal[kOhWin];
#pragma unroll
    for (int w = 0; w < kOhWin; ++w) {
      m[w] = m[w] & (base + w * 256 + tid >= n);
      bal[w] = __ballot(m[w]);
      if (lane == 0) wcnt[w][wave] = __popcll(bal[w]);
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kOhWin; ++w) {
      int before = count, total = 0;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        before += (v < wave) ? wcnt[w][v] : 0;
        total += wcnt[w][v];
      }
      // count <= kOhCap - kOhGroup before a group, so every position is < kOhCap
      if (m[w]) lst[before + __popcll(bal[w] & ((uint64_t(1) << lane) - 1))] = (int32_t)(base + w * 256 + tid);
      count += total;
    }
    __syncthreads();  // the list is complete; wcnt may be rewritten
    if (count > kOhCap - kOhGroup || base + kOhGroup >= a.C) {
      if (count > 0) flush(count);
      count = 0;
      __syncthreads();  // every thread has read the list before it is rewritten
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void onehot_rows_kernel(OnehotArgs<T> a) {
  __shared__ __attribute__((aligned(16))) char smem[onehot_lds()];
  onehot_rows_block<T>(blockIdx.x, a, smem);
}

// The per-chunk preparation before the dH / dW contraction in one launch, so
// that its independent parts overlap instead of queueing: the one-hot rows of
// an FP32 dW table (blocks [0, no)), the target lists (next nl blocks), the
// chunk's h transposed (next nt blocks) and the softmax gradient tiles (next
// ns blocks). Each part is optional.
// dH rows of a split contraction: the S parts summed in increasing order,
// then the dH tile epilogue's operations (same expressions, same order): the
// row factor s rowf (0 for a token that takes no part), the one-hot term
// tcoef W[t] for a valid token, rounding to the output dtype. v8 (D % 8 ==
// 0): 8 consecutive columns per thread with 16-byte loads, and 16-byte
// stores where vec says the output rows are 16-byte aligned; otherwise one
// column per thread. 256 threads per block.
struct DhReduceArgs {
  const float* part;
  int64_t stride;
  int S;
  int64_t M, D;
  int v8, vec;
  EpiParams e;
};

inline int64_t dh_reduce_blocks(const DhReduceArgs& a) {
  return a.part == nullptr ? 0 : (a.M * (a.v8 ? a.D / 8 : a.D) + 255) / 256;
}

template <typename T, bool kVec>
__device__ __forceinline__ void dh_reduce_elems(int64_t q, const DhReduceArgs& a) {
  constexpr int kCols = kVec ? 8 : 1;
  const EpiParams& e = a.e;
  const int64_t nq = a.D / kCols;
  const int64_t m = q / nq;
  if (m >= a.M) return;
  const int64_t n = (q - m * nq) * kCols;
  const float* pp = a.part + m * a.D + n;
  float sv[kCols];
  if constexpr (kVec) {
    const float4 x = *reinterpret_cast<const float4*>(pp);
    const float4 y = *reinterpret_cast<const float4*>(pp + 4);
    sv[0] = x.x, sv[1] = x.y, sv[2] = x.z, sv[3] = x.w, sv[4] = y.x, sv[5] = y.y, sv[6] = y.z, sv[7] = y.w;
    for (int i = 1; i < a.S; ++i) {
      const float4 u = *reinterpret_cast<const float4*>(pp + (int64_t)i * a.stride);
      const float4 v = *reinterpret_cast<const float4*>(pp + (int64_t)i * a.stride + 4);
      sv[0] += u.x, sv[1] += u.y, sv[2] += u.z, sv[3] += u.w;
      sv[4] += v.x, sv[5] += v.y, sv[6] += v.z, sv[7] += v.w;
    }
  } else {
    sv[0] = pp[0];
    for (int i = 1; i < a.S; ++i) sv[0] += pp[(int64_t)i * a.stride];
  }
  const int64_t tok = e.tok0 + m;
  const int64_t tg = e.targets[tok];
  const int64_t t = tg - e.v0;
  const bool valid = tg >= 0 && tg < e.Vt && t >= 0 && t < e.V && e.g[tok] != 0.0f;
  const float sc = e.scales[e.chunk].x;
  const float fr = e.rowf == nullptr ? sc : sc * e.rowf[tok];
  const float c = valid ? e.tcoef[tok] : 0.0f;
  const T* w = static_cast<const T*>(e.W) + (valid ? t : 0) * e.ldW + n;
  float o[kCols];
#pragma unroll
  for (int j = 0; j < kCols; ++j) {
    // a zero factor (a token that takes no part) gives +0, whatever the sign of the sum
    const float base = fr == 0.0f ? 0.0f : sv[j] * fr;
    o[j] = valid ? fmaf(c, (float)w[j], base) : base;
  }
  if (e.out_dt == DT_F32) {
    float* out = static_cast<float*>(e.out) + m * e.ldo + n;
#pragma unroll
    for (int j = 0; j < kCols; ++j) out[j] = o[j];
  } else {
    T* out = static_cast<T*>(e.out) + m * e.ldo + n;
    if constexpr (kVec && sizeof(T) == 2) {
      if (a.vec) {
        union {
          T h[8];
          uint4 u;
        } pk;
#pragma unroll
        for (int j = 0; j < 8; ++j) pk.h[j] = (T)o[j];
        *reinterpret_cast<uint4*>(out) = pk.u;
        return;
      }
    }
#pragma unroll
    for (int j = 0; j < kCols; ++j) out[j] = (T)o[j];
  }
}

template <typename T>
__device__ __forceinline__ void dh_reduce_block(int64_t b, const DhReduceArgs& a) {
  const int64_t q = b * 256 + threadIdx.x;
  if (a.v8)
    dh_reduce_elems<T, true>(q, a);
  else
    dh_reduce_elems<T, false>(q, a);
}

template <typename T>
__global__ __launch_bounds__(256) void dh_reduce_kernel(DhReduceArgs a) {
  dh_reduce_block<T>(blockIdx.x, a);
}

DhReduceArgs dh_reduce_args(const float* part, int64_t stride, int S, int64_t M, int64_t D, const EpiParams& e) {
  DhReduceArgs a;
  a.part = part;
  a.stride = stride;
  a.S = S;
  a.M = M;
  a.D = D;
  a.v8 = D % 8 == 0;
  a.vec = (reinterpret_cast<uintptr_t>(e.out) % 16 == 0) && (e.ldo % 8 == 0);
  a.e = e;
  return a;
}

template <typename T>
__global__ __launch_bounds__(256) void chunk_prep_kernel(OnehotArgs<T> oa, int64_t no, ListArgs la, int64_t nl,
                                                         TransposeArgs<T> ta, int64_t tgx, int64_t nt,
                                                         SoftmaxGradArgs<T> sa, int64_t sgx, int64_t ns,
                                                         DhReduceArgs ra) {
  // the one-hot blocks come first: they are latency-bound and short, so the
  // memory-bound parts that follow run beside them
  // one LDS buffer for whichever part this block runs
  __shared__ __attribute__((aligned(16))) char smem[std::max(std::max(softmax_grad_lds<T>(), transpose_lds<T>()),
                                                             onehot_lds())];
  int64_t b = blockIdx.x;
  if (b < no) {
    onehot_rows_block<T>(b, oa, smem);
    return;
  }
  b -= no;
  if (b < nl) {
    target_lists_block(b, la);
    return;
  }
  b -= nl;
  if (b < nt) {
    transpose_tile<T>(b % tgx, b / tgx, ta, smem);
    return;
  }
  b -= nt;
  if (b < ns) {
    if (sa.qflag != nullptr)
      qfix_tile<T>(b % sgx, b / sgx, sa);
    else
      softmax_grad_tile<T>(b % sgx, b / sgx, sa, smem);
    return;
  }
  b -= ns;
  // the previous dH contraction's parts (memory-bound, like the rest)
  dh_reduce_block<T>(b, ra);
}

__global__ void fill_kernel(uint32_t* __restrict__ p, int64_t nwords, uint32_t word) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += stride) p[i] = word;
}

__global__ void zero_u16_kernel(uint16_t* __restrict__ p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

template <typename T>
hipError_t transpose_t(const void* src, int64_t rows, int64_t cols, int64_t lds, void* dst,
                       int64_t ldd, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  dim3 grid((unsigned)((rows + 63) / 64), (unsigned)((cols + 63) / 64));  // cols <= 2^22 (validated)
  // 16-byte segments need 16-byte aligned bases and leading dimensions in whole segments
  constexpr int64_t kVec = 16 / (int64_t)sizeof(T);
  const int vec = (reinterpret_cast<uintptr_t>(src) % 16 == 0) && (reinterpret_cast<uintptr_t>(dst) % 16 == 0) &&
                  (lds % kVec == 0) && (ldd % kVec == 0);
  transpose_kernel<T><<<grid, 256, 0, s>>>(
      TransposeArgs<T>{static_cast<const T*>(src), rows, cols, lds, static_cast<T*>(dst), ldd, vec});
  return hipGetLastError();
}

template <typename T>
hipError_t db_t(const void* dSt, int64_t ldSt, int64_t V, int64_t C, const float2* scales, int chunk,
                const int32_t* head, const int32_t* next, const int64_t* targets, const float* g,
                const float* tcoef, int64_t tok0, int64_t v0, int64_t Vt, void* db, int tdt, hipStream_t s,
                const float* cq) {
  dim3 grid((unsigned)((V + 3) / 4));
  if (tdt == DT_F32)
    db_accum_kernel<T, float><<<grid, 256, 0, s>>>(static_cast<const T*>(dSt), ldSt, V, C, scales, chunk,
                                                   head, next, targets, g, tcoef, tok0, v0, Vt,
                                                   static_cast<float*>(db), cq);
  else
    db_accum_kernel<T, T><<<grid, 256, 0, s>>>(static_cast<const T*>(dSt), ldSt, V, C, scales, chunk,
                                               head, next, targets, g, tcoef, tok0, v0, Vt, static_cast<T*>(db), cq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dh_reduce(int dt, const float* part, int64_t stride, int S, int64_t M, int64_t D,
                            const EpiParams& e, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (S < 1) return hipErrorInvalidValue;
  const DhReduceArgs a = dh_reduce_args(part, stride, S, M, D, e);
  const int64_t nb = dh_reduce_blocks(a);
  if (nb > INT32_MAX) return hipErrorInvalidValue;
  switch (dt) {
    case DT_F32: dh_reduce_kernel<float><<<(unsigned)nb, 256, 0, s>>>(a); break;
    case DT_BF16: dh_reduce_kernel<__bf16><<<(unsigned)nb, 256, 0, s>>>(a); break;
    case DT_F16: dh_reduce_kernel<_Float16><<<(unsigned)nb, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_lse_combine(const float2* partials, int64_t P, int64_t ldp, const float* zt,
                              const int64_t* targets, int64_t V, int64_t N, float* logp,
                              float* lse, const float* g, float* tcoef, hipStream_t s,
                              const int32_t* qflag, const float2* sc, float* cq) {
  if (N == 0) return hipSuccess;
  if (cq != nullptr && (qflag == nullptr || sc == nullptr || g == nullptr)) return hipErrorInvalidValue;
  lse_combine_kernel<<<(unsigned)((N + kCombTok - 1) / kCombTok), kCombTok * kCombSl, 0, s>>>(
      partials, P, ldp, zt, targets, V, N, logp, lse, g, tcoef, qflag, sc, cq);
  return hipGetLastError();
}

hipError_t launch_shard_combine(const float* lse_sh, const float* zt_sh, int64_t P, int64_t N,
                                const int64_t* targets, int64_t Vt, float* logp, float* lse, hipStream_t s) {
  if (N == 0) return hipSuccess;
  shard_combine_kernel<<<(unsigned)((N + 255) / 256), 256, 0, s>>>(lse_sh, zt_sh, P, N, targets, Vt, logp, lse);
  return hipGetLastError();
}

template <typename T>
SoftmaxGradArgs<T> sg_args(void* qt, int64_t ldq, const float2* partials, int64_t ldp, const float* lse,
                           const float* g, const int64_t* targets, const float2* scales, int chunk, int64_t V,
                           int64_t C, void* dS, int64_t ldS) {
  return SoftmaxGradArgs<T>{static_cast<T*>(qt), ldq, partials, ldp, lse, g, targets, scales, chunk, V, C,
                            static_cast<T*>(dS), ldS};
}

hipError_t launch_softmax_grad(int dt, void* qt, int64_t ldq, const float2* partials, int64_t ldp,
                               const float* lse, const float* g, const int64_t* targets,
                               const float2* scales, int chunk, int64_t V, int64_t C, void* dS,
                               int64_t ldS, hipStream_t s) {
  if (V == 0 || C == 0) return hipSuccess;
  dim3 grid((unsigned)((V + 63) / 64), (unsigned)((C + 63) / 64));  // C <= 2^31 - 1 (validated)
  switch (dt) {
    case DT_F32:
      softmax_grad_kernel<float><<<grid, 256, 0, s>>>(
          sg_args<float>(qt, ldq, partials, ldp, lse, g, targets, scales, chunk, V, C, dS, ldS));
      break;
    case DT_BF16:
      softmax_grad_kernel<__bf16><<<grid, 256, 0, s>>>(
          sg_args<__bf16>(qt, ldq, partials, ldp, lse, g, targets, scales, chunk, V, C, dS, ldS));
      break;
    case DT_F16:
      softmax_grad_kernel<_Float16><<<grid, 256, 0, s>>>(
          sg_args<_Float16>(qt, ldq, partials, ldp, lse, g, targets, scales, chunk, V, C, dS, ldS));
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_transpose(int dt, const void* src, int64_t rows, int64_t cols, int64_t lds,
                            void* dst, int64_t ldd, hipStream_t s) {
  switch (dt) {
    case DT_F32: return transpose_t<float>(src, rows, cols, lds, dst, ldd, s);
    case DT_BF16:
    case DT_F16: return transpose_t<uint16_t>(src, rows, cols, lds, dst, ldd, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t chunk_prep_t(const ChunkPrep& c, hipStream_t s) {
  const ListArgs la{c.targets, c.g, c.tok0, c.C, c.V, c.v0, c.Vt, c.head, c.next};
  const int64_t nl = c.head != nullptr ? (c.C + 3) / 4 : 0;
  constexpr int64_t kVec = 16 / (int64_t)sizeof(T);
  const int ovec = (reinterpret_cast<uintptr_t>(c.oh_h) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(c.table) % 16 == 0) && (c.D % kVec == 0) && (c.ldt % 4 == 0) &&
                   (c.D % 4 == 0);  // pieces start at multiples of 16
  const OnehotArgs<T> oa{c.targets, c.g, c.tcoef, c.oh_tok0, c.oh_C, c.V, c.v0, c.Vt,
                         static_cast<const T*>(c.oh_h), c.D, c.D, c.table, c.ldt, ovec};
  const int64_t no = c.table != nullptr ? c.oh_C : 0;
  const int vec = (reinterpret_cast<uintptr_t>(c.h) % 16 == 0) && (reinterpret_cast<uintptr_t>(c.ht) % 16 == 0) &&
                  (c.D % kVec == 0) && (c.ldht % kVec == 0);
  const TransposeArgs<T> ta{static_cast<const T*>(c.h), c.C, c.D, c.D, static_cast<T*>(c.ht), c.ldht, vec, c.cq};
  const int64_t tgx = (c.C + 63) / 64;
  const int64_t nt = c.ht != nullptr ? tgx * ((c.D + 63) / 64) : 0;
  SoftmaxGradArgs<T> sa = sg_args<T>(c.qt, c.ldq, c.partials, c.ldp, c.lse, c.gc, c.tc, c.scales, c.chunk, c.V,
                                     c.C, c.dS, c.ldS);
  sa.qflag = c.qflag;  // per-token mode: the fixup of flagged columns instead of the gradient pass
  const int64_t sgx = c.qflag != nullptr ? (c.V + 1023) / 1024 : (c.V + 63) / 64;
  const int64_t ns = c.qt != nullptr ? sgx * ((c.C + 63) / 64) : 0;
  const DhReduceArgs ra = c.rd_part != nullptr ? dh_reduce_args(c.rd_part, c.rd_stride, c.rd_S, c.rd_M, c.rd_D, c.rd_ep)
                                               : DhReduceArgs{};
  const int64_t nr = dh_reduce_blocks(ra);
  const int64_t total = no + nl + nt + ns + nr;
  if (total == 0) return hipSuccess;
  if (total > INT32_MAX) {  // one launch per part
    if (no) onehot_rows_kernel<T><<<(unsigned)no, 256, 0, s>>>(oa);
    if (nl) target_lists_kernel<<<(unsigned)nl, 256, 0, s>>>(la);
    if (nt) transpose_kernel<T><<<dim3((unsigned)tgx, (unsigned)(nt / tgx)), 256, 0, s>>>(ta);
    if (ns && c.qflag != nullptr) return hipErrorInvalidValue;  // the fixup runs in the joint launch only
    if (ns) softmax_grad_kernel<T><<<dim3((unsigned)sgx, (unsigned)(ns / sgx)), 256, 0, s>>>(sa);
    if (nr) {
      if (nr > INT32_MAX) return hipErrorInvalidValue;
      dh_reduce_kernel<T><<<(unsigned)nr, 256, 0, s>>>(ra);
    }
    return hipGetLastError();
  }
  chunk_prep_kernel<T><<<(unsigned)total, 256, 0, s>>>(oa, no, la, nl, ta, tgx, nt, sa, sgx, ns, ra);
  return hipGetLastError();
}

hipError_t launch_chunk_prep(int dt, const ChunkPrep& c, hipStream_t s) {
  if (c.C == 0 && (c.table == nullptr || c.oh_C == 0) && c.rd_part == nullptr) return hipSuccess;
  switch (dt) {
    case DT_F32: return chunk_prep_t<float>(c, s);
    case DT_BF16: return chunk_prep_t<__bf16>(c, s);
    case DT_F16: return chunk_prep_t<_Float16>(c, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_chunk_scales(const float* g, int64_t N, int64_t C, int64_t K, int headroom,
                               float2* scales, hipStream_t s) {
  if (K == 0) return hipSuccess;
  chunk_scales_kernel<<<(unsigned)K, 256, 0, s>>>(g, N, C, headroom, scales);
  return hipGetLastError();
}

hipError_t launch_db_accum(int dt, const void* dSt, int64_t ldSt, int64_t V, int64_t C,
                           const float2* scales, int chunk, const int32_t* head, const int32_t* next,
                           const int64_t* targets, const float* g, const float* tcoef, int64_t tok0,
                           int64_t v0, int64_t Vt, void* db, int tdt, hipStream_t s, const float* cq) {
  switch (dt) {
    case DT_F32:
      return db_t<float>(dSt, ldSt, V, C, scales, chunk, head, next, targets, g, tcoef, tok0, v0, Vt, db, tdt, s, cq);
    case DT_BF16:
      return db_t<__bf16>(dSt, ldSt, V, C, scales, chunk, head, next, targets, g, tcoef, tok0, v0, Vt, db, tdt, s,
                          cq);
    case DT_F16:
      return db_t<_Float16>(dSt, ldSt, V, C, scales, chunk, head, next, targets, g, tcoef, tok0, v0, Vt, db, tdt,
                            s, cq);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_target_lists(const int64_t* targets, const float* g, int64_t tok0, int64_t C,
                               int64_t V, int64_t v0, int64_t Vt, int32_t* head, int32_t* next, hipStream_t s) {
  if (C == 0) return hipSuccess;
  target_lists_kernel<<<(unsigned)((C + 3) / 4), 256, 0, s>>>(ListArgs{targets, g, tok0, C, V, v0, Vt, head, next});
  return hipGetLastError();
}

hipError_t launch_zero(void* p, int64_t n, int esize, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t bytes = n * esize;
  if (bytes % 4 == 0 && (reinterpret_cast<uintptr_t>(p) & 3) == 0) {
    const int64_t words = bytes / 4;
    const unsigned blocks = (unsigned)std::min<int64_t>((words + 255) / 256, 65536);
    fill_kernel<<<blocks, 256, 0, s>>>(static_cast<uint32_t*>(p), words, 0u);
  } else {
    const int64_t halves = bytes / 2;
    const unsigned blocks = (unsigned)std::min<int64_t>((halves + 255) / 256, 65536);
    zero_u16_kernel<<<blocks, 256, 0, s>>>(static_cast<uint16_t*>(p), halves);
  }
  return hipGetLastError();
}

hipError_t launch_fill32(uint32_t* p, int64_t n, uint32_t word, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 65536);
  fill_kernel<<<blocks, 256, 0, s>>>(p, n, word);
  return hipGetLastError();
}

}  // namespace llp
