// Same-box ceilings for the roofline figures: what one MI355X actually
// sustains, measured beside the kernels, rather than the published peaks.
//
//  - llpc_mfma_loop: back-to-back v_mfma_f32_32x32x16_bf16 on register
//    operands (eight independent accumulators per wave, eight distinct
//    pseudo-random operand pairs, no memory traffic in the loop): the MFMA
//    rate the chip holds under full load at the clock that load allows.
//  - llpc_copy: a 16-byte-per-lane copy, one 256 KiB chunk per workgroup
//    (one read and one write of every byte, non-temporal): the read + write
//    streaming rate of HBM.
//  - llpc_read: the same walk reading only: the streaming read rate.
//
// These are measurement tools for the benchmark and play no part in the
// library's operators. C ABI; every pointer is device memory of the current
// device; work is enqueued on `stream` (a hipStream_t) and the call returns a
// hipError_t value (0 = success).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kThreads = 256;

// 32 pseudo-random bits per (lane, index): the MurmurHash3 fmix32 finalizer
__device__ __forceinline__ uint32_t mix(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  h ^= h >> 16;
  return h;
}

// bf16 operand with random sign and mantissa, exponent 2^-1 or 2^-2 (so the
// multipliers toggle as with real data, and the sums stay finite)
__device__ __forceinline__ uint32_t rand_bf16x2(uint32_t h) {
  const uint32_t lo = 0x3E80u | (h & 0x807Fu) | ((h >> 8) & 0x0080u);
  const uint32_t hi = 0x3E80u | ((h >> 16) & 0x807Fu) | ((h >> 24) & 0x0080u);
  return lo | (hi << 16);
}

__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(int64_t iters, float* out) {
  // eight distinct operand pairs, so consecutive MFMAs see different inputs
  u32x4 a[8], b[8];
  const uint32_t seed = (blockIdx.x * kThreads + threadIdx.x) * 64u;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[j][i] = rand_bf16x2(mix(seed + 4 * j + i));
      b[j][i] = rand_bf16x2(mix(seed + 32 + 4 * j + i));
    }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[j]),
                                                       __builtin_bit_cast(bf16x8, b[j]), acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

// Streaming: workgroup w owns the contiguous 256 KiB chunk w (the last one
// possibly shorter), walked in 16 KiB steps, four 16-byte pieces per thread
// in flight, non-temporal (the access pattern of one logits row per workgroup).
constexpr int64_t kChunk16 = (256 << 10) / 16;  // 16-byte pieces per chunk
constexpr int kInFlight = 4;

__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        int64_t n) {
  const int64_t c0 = (int64_t)blockIdx.x * kChunk16;
  const int64_t c1 = c0 + kChunk16 < n ? c0 + kChunk16 : n;
  int64_t i = c0 + threadIdx.x;
  for (; i + (kInFlight - 1) * kThreads < c1; i += kInFlight * kThreads) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = __builtin_nontemporal_load(&src[i + u * kThreads]);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) __builtin_nontemporal_store(v[u], &dst[i + u * kThreads]);
  }
  for (; i < c1; i += kThreads) __builtin_nontemporal_store(__builtin_nontemporal_load(&src[i]), &dst[i]);
}

__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ src, int64_t n,
                                                        uint32_t* __restrict__ out) {
  const int64_t c0 = (int64_t)blockIdx.x * kChunk16;
  const int64_t c1 = c0 + kChunk16 < n ? c0 + kChunk16 : n;
  int64_t i = c0 + threadIdx.x;
  uint32_t x = 0;
  for (; i + (kInFlight - 1) * kThreads < c1; i += kInFlight * kThreads) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = __builtin_nontemporal_load(&src[i + u * kThreads]);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < c1; i += kThreads) {
    const u32x4 v = __builtin_nontemporal_load(&src[i]);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = x;
}

// one workgroup per chunk; the entry points keep n16 below 2^31 chunks' worth
int grid_for(int64_t n16) { return (int)((n16 + kChunk16 - 1) / kChunk16); }

}  // namespace

extern "C" {

// `blocks` workgroups of 256 threads, each wave `iters` rounds of 8 MFMAs
// (32768 flop each); `out` holds blocks x 256 floats. 1 <= blocks <= 65536,
// 1 <= iters <= 2^24, else hipErrorInvalidValue.
__attribute__((visibility("default"))) int llpc_mfma_loop(int blocks, int64_t iters, float* out, void* stream) {
  if (blocks < 1 || blocks > 65536 || iters < 1 || iters > (int64_t(1) << 24) || out == nullptr)
    return (int)hipErrorInvalidValue;
  mfma_loop_kernel<<<blocks, kThreads, 0, static_cast<hipStream_t>(stream)>>>(iters, out);
  return (int)hipGetLastError();
}

// Copies `bytes` (a positive multiple of 16 below 2^46; both pointers 16-byte aligned).
__attribute__((visibility("default"))) int llpc_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (src == nullptr || dst == nullptr || bytes <= 0 || bytes % 16 != 0 || bytes >= (int64_t(1) << 46) ||
      (reinterpret_cast<uintptr_t>(src) & 15) != 0 || (reinterpret_cast<uintptr_t>(dst) & 15) != 0)
    return (int)hipErrorInvalidValue;
  const int64_t n = bytes / 16;
  copy_kernel<<<grid_for(n), kThreads, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const u32x4*>(src),
                                                                             static_cast<u32x4*>(dst), n);
  return (int)hipGetLastError();
}

// Reads `bytes` (a positive multiple of 16 below 2^46, 16-byte aligned); `out` holds
// llpc_read_out_len(bytes) words (an XOR of what each thread read).
__attribute__((visibility("default"))) int64_t llpc_read_out_len(int64_t bytes) {
  return bytes > 0 && bytes < (int64_t(1) << 46) ? (int64_t)grid_for(bytes / 16) * kThreads : 0;
}
__attribute__((visibility("default"))) int llpc_read(const void* src, int64_t bytes, uint32_t* out, void* stream) {
  if (src == nullptr || out == nullptr || bytes <= 0 || bytes % 16 != 0 || bytes >= (int64_t(1) << 46) ||
      (reinterpret_cast<uintptr_t>(src) & 15) != 0)
    return (int)hipErrorInvalidValue;
  const int64_t n = bytes / 16;
  read_kernel<<<grid_for(n), kThreads, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const u32x4*>(src), n,
                                                                             out);
  return (int)hipGetLastError();
}

}  // extern "C"
