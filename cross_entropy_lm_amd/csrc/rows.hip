// Logits-only log-prob forward and backward (RL-Kernel PR #495, "Summary" and
// "Results"): one workgroup per row of the [N, V] logits.
//
// Forward: a single pass keeps an online (max, sum-exp) per thread over
// 16-byte vector loads, merges the threads with wave shuffles and LDS, and
// gathers the target logit: logp = z[t] - lse, +0 for a target outside
// [0, V) ("Behavior changes"). One read of the row.
// Backward: dlogits = g [v == t] - g exp(z - lse) in the logits dtype, from
// the forward's lse: one read and one write of the row (the pages' kernel
// re-reduces the row twice before writing, "Results"). Without lse the row is
// reduced first, then written (two reads).
// Rows whose byte address is not 16-byte aligned are handled with an element
// head and tail around the vector body; all offsets are 64-bit.
#include "kernels.h"

#include <math.h>

namespace llp {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kRowThreads = 256;
#ifndef LLP_BWD_UNROLL
#define LLP_BWD_UNROLL 4
#endif
constexpr int kBwdUnroll = LLP_BWD_UNROLL;  // 16-byte pieces per thread in flight (backward)

template <typename T> struct RT;
template <> struct RT<__bf16> { static constexpr int per16 = 8; };
template <> struct RT<_Float16> { static constexpr int per16 = 8; };
template <> struct RT<float> { static constexpr int per16 = 4; };

template <typename T>
__device__ __forceinline__ void unpack(u32x4 u, float (&x)[RT<T>::per16]) {
  union {
    u32x4 u;
    T e[RT<T>::per16];
  } c;
  c.u = u;
#pragma unroll
  for (int i = 0; i < RT<T>::per16; ++i) x[i] = (float)c.e[i];
}

template <typename T>
__device__ __forceinline__ u32x4 pack(const float (&x)[RT<T>::per16]) {
  union {
    u32x4 u;
    T e[RT<T>::per16];
  } c;
#pragma unroll
  for (int i = 0; i < RT<T>::per16; ++i) c.e[i] = (T)x[i];
  return c.u;
}

// Online (m, s): s = sum over seen x of 2^((x - m) log2 e), m = max seen x.
struct Online {
  float m = -INFINITY, s = 0.0f;
  __device__ __forceinline__ void add_max(float cm) {
    if (cm > m) {
      s *= __builtin_amdgcn_exp2f((m - cm) * kLog2e);
      m = cm;
    }
  }
  template <int K>
  __device__ __forceinline__ void add(const float (&x)[K]) {
    float cm = x[0];
#pragma unroll
    for (int i = 1; i < K; ++i) cm = fmaxf(cm, x[i]);
    add_max(cm);
    if (m != -INFINITY) {
      const float mm = m * kLog2e;
#pragma unroll
      for (int i = 0; i < K; ++i) s += __builtin_amdgcn_exp2f(fmaf(x[i], kLog2e, -mm));
    }
  }
  __device__ __forceinline__ void add1(float x) {
    float a[1] = {x};
    add<1>(a);
  }
  __device__ __forceinline__ void merge(float om, float os) {
    const float M = fmaxf(m, om);
    if (M == -INFINITY) return;
    s = s * __builtin_amdgcn_exp2f((m - M) * kLog2e) + os * __builtin_amdgcn_exp2f((om - M) * kLog2e);
    m = M;
  }
};

// Reduces the row's (m, s) over the workgroup; every thread gets lse.
template <typename T>
__device__ float row_lse(const T* __restrict__ x, int64_t V, float* red) {
  constexpr int per16 = RT<T>::per16;
  const int tid = threadIdx.x;
  Online o;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(x);
  int64_t head = (int64_t)(((16 - (addr & 15)) & 15) / sizeof(T));
  if (head > V) head = V;
  for (int64_t i = tid; i < head; i += kRowThreads) o.add1((float)x[i]);
  const u32x4* xv = reinterpret_cast<const u32x4*>(x + head);
  const int64_t nv = (V - head) / per16;
  int64_t j = tid;
  for (; j + 3 * kRowThreads < nv; j += 4 * kRowThreads) {
    const u32x4 a0 = xv[j], a1 = xv[j + kRowThreads], a2 = xv[j + 2 * kRowThreads],
                a3 = xv[j + 3 * kRowThreads];
    float f[per16];
    unpack<T>(a0, f);
    o.add(f);
    unpack<T>(a1, f);
    o.add(f);
    unpack<T>(a2, f);
    o.add(f);
    unpack<T>(a3, f);
    o.add(f);
  }
  for (; j < nv; j += kRowThreads) {
    float f[per16];
    unpack<T>(xv[j], f);
    o.add(f);
  }
  for (int64_t i = head + nv * per16 + tid; i < V; i += kRowThreads) o.add1((float)x[i]);
  for (int off = 32; off > 0; off >>= 1) {
    const float om = __shfl_xor(o.m, off), os = __shfl_xor(o.s, off);
    o.merge(om, os);
  }
  if ((tid & 63) == 0) {
    red[2 * (tid >> 6)] = o.m;
    red[2 * (tid >> 6) + 1] = o.s;
  }
  __syncthreads();
  Online r;
#pragma unroll
  for (int w = 0; w < kRowThreads / 64; ++w) r.merge(red[2 * w], red[2 * w + 1]);
  return r.m + __builtin_amdgcn_logf(r.s) * kLn2;
}

template <typename T>
__global__ __launch_bounds__(kRowThreads) void rows_fwd_kernel(const T* __restrict__ X, int64_t V,
                                                               const int64_t* __restrict__ targets,
                                                               float* __restrict__ logp,
                                                               float* __restrict__ lse) {
  __shared__ float red[2 * kRowThreads / 64];
  const int64_t row = blockIdx.x;
  const T* x = X + row * V;
  const float l = row_lse<T>(x, V, red);
  if (threadIdx.x == 0) {
    const int64_t t = targets[row];
    logp[row] = (t >= 0 && t < V) ? (float)x[t] - l : 0.0f;
    if (lse != nullptr) lse[row] = l;
  }
}

template <typename T>
__device__ __forceinline__ float grad1(float z, int64_t v, int64_t t, float g, float l2, bool valid) {
  return valid ? fmaf(-g, __builtin_amdgcn_exp2f(fmaf(z, kLog2e, -l2)), v == t ? g : 0.0f) : 0.0f;
}

// X and dX may be the same buffer: each element is read and then written by
// the same thread, and the optional lse pass finishes (barrier) before any write.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void rows_bwd_kernel(const T* X, int64_t V,
                                                               const int64_t* __restrict__ targets,
                                                               const float* __restrict__ g,
                                                               const float* __restrict__ lse_in,
                                                               T* dX, int vec_ok) {
  __shared__ float red[2 * kRowThreads / 64];
  constexpr int per16 = RT<T>::per16;
  const int64_t row = blockIdx.x;
  const T* x = X + row * V;
  T* dx = dX + row * V;
  const int tid = threadIdx.x;
  const int64_t t = targets[row];
  const float gv = g[row];
  const bool valid = t >= 0 && t < V && gv != 0.0f;
  float l = 0.0f;
  if (valid) l = (lse_in != nullptr) ? lse_in[row] : row_lse<T>(x, V, red);
  const float l2 = l * kLog2e;
  if (!vec_ok) {
    for (int64_t i = tid; i < V; i += kRowThreads) dx[i] = (T)grad1<T>((float)x[i], i, t, gv, l2, valid);
    return;
  }
  const uintptr_t addr = reinterpret_cast<uintptr_t>(x);
  int64_t head = (int64_t)(((16 - (addr & 15)) & 15) / sizeof(T));
  if (head > V) head = V;
  for (int64_t i = tid; i < head; i += kRowThreads) dx[i] = (T)grad1<T>((float)x[i], i, t, gv, l2, valid);
  const u32x4* xv = reinterpret_cast<const u32x4*>(x + head);
  u32x4* dv = reinterpret_cast<u32x4*>(dx + head);
  const int64_t nv = (V - head) / per16;
  int64_t j = tid;
  // kBwdUnroll 16-byte pieces per thread in flight; the row is streamed once,
  // so loads and stores are non-temporal
  for (; j + (kBwdUnroll - 1) * kRowThreads < nv; j += kBwdUnroll * kRowThreads) {
    u32x4 a[kBwdUnroll];
#pragma unroll
    for (int u = 0; u < kBwdUnroll; ++u) a[u] = __builtin_nontemporal_load(&xv[j + u * kRowThreads]);
#pragma unroll
    for (int u = 0; u < kBwdUnroll; ++u) {
      float f[per16];
      unpack<T>(a[u], f);
      const int64_t v0 = head + (j + u * kRowThreads) * per16;
#pragma unroll
      for (int i = 0; i < per16; ++i) f[i] = grad1<T>(f[i], v0 + i, t, gv, l2, valid);
      __builtin_nontemporal_store(pack<T>(f), &dv[j + u * kRowThreads]);
    }
  }
  for (; j < nv; j += kRowThreads) {
    float f0[per16];
    unpack<T>(xv[j], f0);
    const int64_t v0 = head + j * per16;
#pragma unroll
    for (int i = 0; i < per16; ++i) f0[i] = grad1<T>(f0[i], v0 + i, t, gv, l2, valid);
    dv[j] = pack<T>(f0);
  }
  for (int64_t i = head + nv * per16 + tid; i < V; i += kRowThreads)
    dx[i] = (T)grad1<T>((float)x[i], i, t, gv, l2, valid);
}

template <typename T>
hipError_t fwd_t(const void* logits, int64_t N, int64_t V, const int64_t* targets, float* logp,
                 float* lse, hipStream_t s) {
  rows_fwd_kernel<T><<<(unsigned)N, kRowThreads, 0, s>>>(static_cast<const T*>(logits), V, targets,
                                                         logp, lse);
  return hipGetLastError();
}

template <typename T>
hipError_t bwd_t(const void* logits, int64_t N, int64_t V, const int64_t* targets, const float* g,
                 const float* lse, void* dlogits, hipStream_t s) {
  const int vec_ok = (reinterpret_cast<uintptr_t>(logits) & 15) == (reinterpret_cast<uintptr_t>(dlogits) & 15);
  rows_bwd_kernel<T><<<(unsigned)N, kRowThreads, 0, s>>>(static_cast<const T*>(logits), V, targets, g,
                                                         lse, static_cast<T*>(dlogits), vec_ok);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rows_fwd(int dt, const void* logits, int64_t N, int64_t V, const int64_t* targets,
                           float* logp, float* lse, hipStream_t s) {
  if (N == 0) return hipSuccess;
  switch (dt) {
    case DT_F32: return fwd_t<float>(logits, N, V, targets, logp, lse, s);
    case DT_BF16: return fwd_t<__bf16>(logits, N, V, targets, logp, lse, s);
    case DT_F16: return fwd_t<_Float16>(logits, N, V, targets, logp, lse, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_rows_bwd(int dt, const void* logits, int64_t N, int64_t V, const int64_t* targets,
                           const float* g, const float* lse, void* dlogits, hipStream_t s) {
  if (N == 0) return hipSuccess;
  switch (dt) {
    case DT_F32: return bwd_t<float>(logits, N, V, targets, g, lse, dlogits, s);
    case DT_BF16: return bwd_t<__bf16>(logits, N, V, targets, g, lse, dlogits, s);
    case DT_F16: return bwd_t<_Float16>(logits, N, V, targets, g, lse, dlogits, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace llp
