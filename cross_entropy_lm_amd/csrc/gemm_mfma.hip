// MFMA contraction kernels for gfx950 (CDNA4) with the fused log-prob epilogues.
//
// Every contraction of the operator is written as C[m, n] = sum_k A[m, k] B[n, k]
// with both operands K-contiguous (row-major [rows][ld]):
//   logits (forward and backward recompute): A = W [V, D], B = h [N, D]
//   dH = dlogits W:                         A = dlogits [C, V], B = W^T [D, V]
//   dW += dlogits^T h:                      A = dlogits^T [V, C], B = h^T [D, C]
// (the transposed operands are produced in the caller's workspace).
//
// Tile: 256 x 256 outputs per workgroup of kWaveM x kWaveN waves (each wave
// owns MI x NI blocks of the 32x32 MFMA). K advances 128 bytes per stage (64
// bf16/fp16 or 32 fp32); the two operand tiles of a stage are staged through
// LDS with a 16-byte row pad, double-buffered (144 KiB). Workgroups are
// remapped so that each XCD (own L2) works on a contiguous range of tiles,
// taken in groups of kGroupM tiles along M.
//
// MFMA operand layout: for the 32x32 instructions lane l supplies row (l % 32)
// of A (and column (l % 32) of B) and a group of K values selected by l / 32;
// A and B use the same lane -> k mapping, so the order of k inside a stage is
// free. Output: lane l, accumulator r holds C[(r/4)*8 + (l/32)*4 + r%4][l % 32].
//
// The epilogues implement, on the fp32 tile of logits z (vocab rows x token
// columns):
//   LSE_PARTIAL: per token, m = max_v z and s = sum_v exp(z - m) over the wave's
//     rows of the tile (the online max / sum-exp of RL-Kernel PR #495, "Summary",
//     done per tile), plus the target logit z[t]. exp/log use the hardware
//     base-2 instructions with z scaled by log2(e).
//   DLOGITS: dlogits = g [v == t] - g exp(z - lse) (RL-Kernel PR #495,
//     "Summary", second commit), divided by the chunk's power-of-two scale s
//     and rounded to the operand dtype; +0 for an out-of-range target or g = 0
//     ("Behavior changes").
//   STORE: dH rows = s * C.   ACCUM: table += s * C, in place (RL-Kernel issue
//     #261, "Current accumulation"; Liger-Kernel PR #1324, "Details").
#include "kernels.h"

#include <math.h>

#include <type_traits>

namespace llp {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr float kLog2e = 1.4426950408889634f;

constexpr int kRowBytes = 128;          // K bytes of one tile row per stage
constexpr int kPitch = kRowBytes + 16;  // LDS row pitch: the pad puts 8 consecutive rows on distinct banks
constexpr int kStageBytes = (kTileM + kTileN) * kPitch;
constexpr int kLdsBytes = 2 * kStageBytes;
constexpr int kLoadsPerThread = kTileM * (kRowBytes / 16) / kThreads;  // 16-byte chunks per operand
constexpr int MI = kTileM / (32 * kWaveM);  // 32x32 blocks per wave along M
constexpr int NI = kTileN / (32 * kWaveN);  // ... along N
constexpr int kWaveRowsM = 32 * MI;
constexpr int kWaveColsN = 32 * NI;
static_assert(kTileM == kTileN, "loader assumes square tiles");
typedef f32x16 Acc[MI][NI];

// Direct-to-LDS pipeline (operands 16-byte aligned, see mainloop_dma): five
// operand slots, each one 128-byte K slice (one cache line per row) of the A or
// the B tile (32 KiB, rows XOR-swizzled in 16-byte units, no padding), filled
// by buffer_load ... lds. The slots are distinct LDS objects so the compiler
// can tell reads of one slot from in-flight DMA into another.
constexpr int kSB = 128;            // K bytes of a slot row
constexpr int kOpB = kTileM * kSB;  // one slot
constexpr int kNS = 5;              // slots
constexpr int kStageArr = kOpB;
static_assert(kNS * kStageArr <= 160 * 1024, "gfx950 LDS per workgroup");
typedef __attribute__((address_space(3))) void lds_void_t;

// Swizzle of the K-contiguous slots: chunk c (16 bytes) of row r sits at
// position c ^ swz_row(r). gfx950's LDS serves a 16-byte read for 16 lanes
// per cycle from 64 four-byte banks (256 bytes): the 16 rows a fragment read
// touches in one cycle (rows r0 .. r0 + 15, 128 bytes apart) must cover the
// 16 distinct 16-byte bank groups, i.e. rows of equal parity need distinct
// positions. (r & 7) alone repeats at r + 8 (a 2-way conflict); the extra
// bit (r / 8) & 1 separates them and keeps any 8 consecutive rows distinct.
__device__ __forceinline__ int swz_row(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// LDS handed to the epilogues: four regions of kOpB bytes, and with the DMA
// pipeline a fifth one (its fifth operand slot; null otherwise).
struct EpiLds {
  char* a[4];
  char* x;
};

template <typename T> struct ET;
template <> struct ET<__bf16> { static constexpr int per16 = 8; };
template <> struct ET<_Float16> { static constexpr int per16 = 8; };
template <> struct ET<float> { static constexpr int per16 = 4; };

__device__ __forceinline__ f32x16 mfma_step(__bf16*, u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_step(_Float16*, u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
// fp32: four K=2 steps per 16-byte fragment. Each element is copied to a
// scalar before the bit cast: a bit cast applied directly to an ext-vector
// element expression is lowered to element 0 by this compiler.
__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ f32x16 mfma_step(float*, u32x4 a, u32x4 b, f32x16 c) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t aj = a[j], bj = b[j];
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(as_f32(aj), as_f32(bj), c, 0, 0, 0);
  }
  return c;
}

// One 16-byte chunk of row `row`, elements [k, k + per16), zero outside [0, rows) x [0, K).
template <typename T>
__device__ __forceinline__ u32x4 load_chunk(const T* base, int64_t ld, int64_t row, int64_t rows, int64_t k,
                                   int64_t K, bool vec) {
  constexpr int per16 = ET<T>::per16;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (row < rows && k < K) {
    const T* p = base + row * ld + k;
    if (vec && k + per16 <= K) {
      v = *reinterpret_cast<const u32x4*>(p);
    } else {
      union {
        T e[per16];
        u32x4 u;
      } tmp;
#pragma unroll
      for (int e = 0; e < per16; ++e) tmp.e[e] = (k + e < K) ? p[e] : (T)0.0f;
      v = tmp.u;
    }
  }
  return v;
}

// Block -> tile. The hardware deals workgroups round-robin to the XCDs
// (block b runs on XCD b % 8); remap so that XCD x takes the contiguous tile
// range [x * T / 8, (x + 1) * T / 8), then walk that range in groups of
// kGroupM tiles along M, N-major inside a group, so the workgroups resident on
// one XCD share A rows and B rows in its L2.
__device__ __forceinline__ int xcd_remap(int b, int T) {
  const int per = T / kXcds, rem = T % kXcds;
  const int x = b % kXcds, local = b / kXcds;
  return x * per + min(x, rem) + local;
}

__device__ __forceinline__ void tile_coords(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int group_size = kGroupM * tiles_n;
  const int group = id / group_size;
  const int first = group * kGroupM;
  const int gm = min(tiles_m - first, kGroupM);
  const int in = id - group * group_size;
  tm = first + in % gm;
  tn = in / gm;
}

template <typename T>
__device__ __forceinline__ float ld_f32(const T* p, int64_t i) {
  return (float)p[i];
}

struct Frag {
  int lane, wm, wn;
  __device__ inline int row(int mi, int r) const {  // row inside the 256-row tile
    return wm * kWaveRowsM + mi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
  }
  __device__ inline int col(int ni) const { return wn * kWaveColsN + ni * 32 + (lane & 31); }
};

// ---------------------------------------------------------------- epilogues
// Forward tile: per token (column) and wave-row block of 128 vocab rows, the
// partial (m log2 e, sum of 2^(z log2 e - m log2 e)) and, for the row holding
// the token's target, the target logit. With kQ (the fused forward + backward)
// each summand q = 2^(z log2 e - m log2 e), in (0, 1], is also stored
// vocab-major in the operand dtype (per-token mode: 2^(z log2 e) itself), so
// that the softmax gradient can be formed once the token's lse is known.
// No per-element branches: tile-local 32-bit row indices; rows past M become
// -inf by a select; the target logit is picked by a select and stored once
// per column; the numerators leave through buffer stores whose offsets fall
// out of range for rows past M and columns at or past round8(N), which the
// hardware drops (the whole offset is in the vector operand, which the range
// check covers), and the per-token mode's +0 at a token's target is one more
// store after the row loop. Each wave's 128-row block has its own buffer
// range, so a row of the vocab-major buffer must stay below 2^24 bytes (the
// plan checks it).
template <typename T, bool kQ>
__device__ __forceinline__ void epi_lse_partial(const GemmProblem& p, Acc& acc, int tm, int64_t m0, int64_t n0,
                                                const Frag& f) {
  const EpiParams& e = p.ep;
  const T* bias = static_cast<const T*>(e.bias);
  const int64_t mleft = p.M - m0;
  const int mr = mleft < kTileM ? (int)mleft : kTileM;  // rows of this tile that exist
  const int rl0 = f.wm * kWaveRowsM + (f.lane >> 5) * 4;  // tile row of (mi = 0, r = 0) in this lane
  int tl[NI];    // tile row of the column's target, or -1 outside [0, mr)
  bool hit[NI];  // this lane holds that row
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    const int64_t n = n0 + f.col(ni);
    const int64_t d = (n < p.N) ? e.targets[e.tok0 + n] - e.v0 - m0 : -1;
    tl[ni] = (d >= 0 && d < mr) ? (int)d : -1;
    const int u = tl[ni] - rl0;
    hit[ni] = tl[ni] >= 0 && u >= 0 && u < kWaveRowsM && (u & 4) == 0;
  }
  float mx[NI], zsel[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    mx[ni] = -INFINITY;
    zsel[ni] = -INFINITY;
  }
  auto pass1 = [&](auto has_bias) {
    constexpr bool kB = decltype(has_bias)::value;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = rl0 + mi * 32 + (r >> 2) * 8 + (r & 3);
        const bool vv = rl < mr;
        const float bv = kB ? ld_f32(bias + m0, vv ? rl : 0) : 0.0f;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const float z = vv ? acc[mi][ni][r] + bv : -INFINITY;
          acc[mi][ni][r] = z;
          mx[ni] = fmaxf(mx[ni], z);
          zsel[ni] = (rl == tl[ni]) ? z : zsel[ni];
        }
      }
      // keeps the bias loads of later row groups from all being hoisted
      // here (their registers would spill)
      if constexpr (kB) __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (bias != nullptr)
    pass1(std::true_type{});
  else
    pass1(std::false_type{});
  float m2[NI], m2e[NI], s[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    mx[ni] = fmaxf(mx[ni], __shfl_xor(mx[ni], 32));
    m2[ni] = mx[ni] * kLog2e;
    // a block whose rows all lie past V or are -inf: its q are +0, not 2^(-inf - (-inf))
    m2e[ni] = (m2[ni] == -INFINITY) ? 0.0f : m2[ni];
    s[ni] = 0.0f;
    if (hit[ni]) e.zt[e.tok0 + n0 + f.col(ni)] = zsel[ni];
  }
  if constexpr (!kQ) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) s[ni] += __builtin_amdgcn_exp2f(fmaf(acc[mi][ni][r], kLog2e, -m2e[ni]));
  } else {
    constexpr int es = (int)sizeof(T);
    constexpr uint32_t kOut = 0x80000000u;  // a column offset that puts every store out of range
    const int64_t npad = (p.N + 7) & ~int64_t(7);
    const int64_t rowb = e.ldSt * es;       // bytes per row, below 2^24
    const int64_t w0 = m0 + f.wm * kWaveRowsM;  // first row of this wave's block
    const int64_t wleft = p.M - w0;             // rows of the block that exist (may be <= 0)
    const int64_t span = wleft > 0 ? wleft * rowb : 0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<char*>(e.dSt) + (wleft > 0 ? w0 * rowb : 0), (short)0,
        span < 0x7FFFFFF0LL ? (int)span : 0x7FFFFFF0, 0x00020000);
    uint32_t coff[NI];  // this lane's row half and column, or kOut at or past round8(N)
    float mul[NI];      // stored value = q mul: 2^m in the per-token mode, +0 past N or for a -inf block
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int64_t n = n0 + f.col(ni);
      coff[ni] = n < npad ? (uint32_t)((f.lane >> 5) * 4 * rowb + f.col(ni) * es) : kOut;
      const bool live = n < p.N && m2[ni] != -INFINITY;
      mul[ni] = live ? 1.0f : 0.0f;
      if (e.qtok) {
        const bool inr = m2[ni] >= kQtokLo && m2[ni] <= kQtokHi;
        if (inr && live) mul[ni] = __builtin_amdgcn_exp2f(m2[ni]);
        // lanes l and l + 32 hold the same column and block: one of them flags it
        if (!inr && m2[ni] != -INFINITY && f.lane < 32 && n < p.N) e.qflag[e.tok0 + n] = 1;
      }
    }
    // the buffer starts at column n0's row w0 entry minus the tile's first column
    const uint32_t cbase = (uint32_t)(n0 * es);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
      if (coff[ni] != kOut) coff[ni] += cbase;
    auto put = [&](uint32_t off, float v) {
      if constexpr (es == 2)
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (T)v), rs, off, 0, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, off, 0, 0);
    };
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t roff = (uint32_t)((mi * 32 + (r >> 2) * 8 + (r & 3)) * rowb);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const float q = __builtin_amdgcn_exp2f(fmaf(acc[mi][ni][r], kLog2e, -m2e[ni]));
          s[ni] += q;
          put(coff[ni] + roff, q * mul[ni]);
        }
      }
    }
    if (e.qtok) {
      // per-token mode: the target's entry is +0 (its one-hot part is exact elsewhere)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        if (hit[ni]) put(coff[ni] + (uint32_t)((tl[ni] - rl0) * rowb), 0.0f);
    }
  }
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    float sv = s[ni] + __shfl_xor(s[ni], 32);
    if (mx[ni] == -INFINITY) sv = 0.0f;  // this wave's rows all lie past V
    const int64_t n = n0 + f.col(ni);
    if (f.lane < 32 && n < p.N)
      e.partials[(int64_t)(tm * kWaveM + f.wm) * e.ldp + n] = make_float2(m2[ni], sv);
  }
}

// The token-major copy of the softmax part is staged through LDS (the
// operand buffers are free once the K loop has ended) so that it leaves as
// 16-byte row segments; the vocab-major copy leaves straight from the
// accumulator layout, where 32 lanes hold 32 consecutive tokens of one row.
template <typename T>
__device__ __forceinline__ void epi_dlogits(const GemmProblem& p, Acc& acc, int64_t m0, int64_t n0,
                                            const Frag& f, const EpiLds& L) {
  const EpiParams& e = p.ep;
  const T* bias = static_cast<const T*>(e.bias);
  T* dS = static_cast<T*>(e.dS);
  T* dSt = static_cast<T*>(e.dSt);
  const float inv = e.scales[e.chunk].y;
  int64_t tgt[NI];
  float gv[NI], gs[NI], l2[NI];
  bool rv[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    const int64_t n = n0 + f.col(ni);
    const bool nv = n < p.N;
    const int64_t tok = e.tok0 + (nv ? n : 0);
    const int64_t tg = nv ? e.targets[tok] : -1;
    tgt[ni] = tg - e.v0;  // local row of the target; matches only in the share holding it
    gv[ni] = nv ? e.g[tok] : 0.0f;
    rv[ni] = nv && tg >= 0 && tg < e.Vt && gv[ni] != 0.0f;
    gs[ni] = gv[ni] * inv;
    l2[ni] = nv ? e.lse[tok] * kLog2e : 0.0f;
  }
  // softmax part in place of the logits (0 past V / past the chunk), with one
  // per-element branch left, the rarely taken store of a target's exact part:
  // tile-local 32-bit rows; the vocab-major copy leaves through buffer
  // stores, one buffer range per 8-row group (its
  // 64-bit base in scalar registers), whose offsets fall out of range for rows
  // past M and columns at or past round8(N) (the hardware drops those; the
  // whole offset is in the range-checked vector operand). Values are formed
  // as before, so the results are the same bits. A row of the vocab-major
  // buffer stays below 2^28 bytes (the plan checks it).
  constexpr int es = (int)sizeof(T);
  constexpr uint32_t kOut = 0x80000000u;  // a column offset that puts every store out of range
  const int64_t mleft = p.M - m0;
  const int mr = mleft < kTileM ? (int)mleft : kTileM;  // rows of this tile that exist
  const int rl0 = f.wm * kWaveRowsM + (f.lane >> 5) * 4;  // tile row of (mi = 0, r = 0) in this lane
  const int64_t rowb = e.ldSt * es;
  const int64_t npad = (p.N + 7) & ~int64_t(7);
  int tl[NI];         // tile row of the column's target, or -1 outside [0, mr)
  uint32_t coff[NI];  // this lane's row half and column inside an 8-row group, or kOut
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    const int64_t n = n0 + f.col(ni);
    const int64_t d = rv[ni] ? tgt[ni] - m0 : -1;
    tl[ni] = (d >= 0 && d < mr) ? (int)d : -1;
    coff[ni] = n < npad ? (uint32_t)((f.lane >> 5) * 4 * rowb + n * es) : kOut;
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int g8 = 0; g8 < 4; ++g8) {
      // rows m0 + wm 128 + mi 32 + g8 8 + [0, 8) of the buffer (this lane: half 4 + [0, 4))
      const int64_t R = m0 + f.wm * kWaveRowsM + mi * 32 + g8 * 8;
      const int64_t left = p.M - R;
      const int64_t span = left > 0 ? left * rowb : 0;
      // (not used without a vocab-major copy: the stores below are skipped then)
      const uintptr_t base = reinterpret_cast<uintptr_t>(dSt) + (uintptr_t)(left > 0 ? R * rowb : 0);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<void*>(base), (short)0, span < 0x7FFFFFF0LL ? (int)span : 0x7FFFFFF0, 0x00020000);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int r = g8 * 4 + r4;
        const int rl = rl0 + mi * 32 + g8 * 8 + r4;
        const bool vv = rl < mr;
        const float bv = (bias != nullptr) ? ld_f32(bias + m0, vv ? rl : 0) : 0.0f;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const float z = acc[mi][ni][r] + bv;
          const float pr = __builtin_amdgcn_exp2f(fmaf(z, kLog2e, -l2[ni]));
          if (rl == tl[ni]) e.tcoef[e.tok0 + n0 + f.col(ni)] = fmaf(-gv[ni], pr, gv[ni]);  // g (1 - p_t)
          // +0 for a row that takes no part, and at the target (its part is exact)
          const bool part = rv[ni] && vv && rl != tl[ni];
          const float d = part ? -gs[ni] * pr : 0.0f;
          acc[mi][ni][r] = d;
          // columns [N, round8(N)) get +0: a 16-byte K chunk that straddles the
          // chunk's end then contributes nothing to the dW contraction
          if (dSt != nullptr) {
            const uint32_t off = coff[ni] + (uint32_t)(r4 * rowb);
            if constexpr (std::is_same<T, _Float16>::value) {
              // fp16: the product p (-g/s) rounded once, straight to fp16
              // (a mixed-precision FMA with fp32 sources and a +0 addend),
              // not rounded to fp32 first
              uint32_t hv = 0;
              const float ng = -gs[ni];
              asm("v_fma_mixlo_f16 %0, %1, %2, 0" : "+v"(hv) : "v"(pr), "v"(ng));
              __builtin_amdgcn_raw_buffer_store_b16(part ? (unsigned short)hv : (unsigned short)0, rs, off, 0, 0);
            } else if constexpr (es == 2) {
              __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (T)d), rs, off, 0, 0);
            } else {
              __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, d), rs, off, 0, 0);
            }
          }
        }
      }
    }
  }
  if (dS == nullptr) return;
  // token-major copy through LDS, in passes of kPassRows tokens x 256 vocab
  // (+ a 16-byte pad per row), each pass in one of the four LDS regions
  constexpr int kPad = 16 / (int)sizeof(T);
  constexpr int kPitchE = kTileM + kPad;  // elements
  constexpr int kRegion = kOpB;  // bytes of each LDS region
  constexpr int kPassRows = (kRegion / (kPitchE * (int)sizeof(T))) >= 64   ? 64
                            : (kRegion / (kPitchE * (int)sizeof(T))) >= 32 ? 32
                                                                          : 16;
  constexpr int kPasses = kTileN / kPassRows;
  constexpr int kChunksPerRow = kTileM * (int)sizeof(T) / 16;
  constexpr int per16 = ET<T>::per16;
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    T* st = reinterpret_cast<T*>(L.a[pass % 4]);
    const int nb = pass * kPassRows;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int nl = f.col(ni) - nb;
          if (nl < 0 || nl >= kPassRows) continue;
          T* q = st + nl * kPitchE + f.row(mi, rg * 4);  // 4 consecutive vocab rows
#pragma unroll
          for (int i = 0; i < 4; ++i) q[i] = (T)acc[mi][ni][rg * 4 + i];
        }
    __syncthreads();
    for (int c = threadIdx.x; c < kPassRows * kChunksPerRow; c += kThreads) {
      const int nl = c / kChunksPerRow, vc = (c % kChunksPerRow) * per16;
      const int64_t n = n0 + nb + nl, v = m0 + vc;
      if (n < p.N && v < p.M)
        *reinterpret_cast<u32x4*>(dS + n * e.ldS + v) = *reinterpret_cast<const u32x4*>(st + nl * kPitchE + vc);
    }
    __syncthreads();
  }
}

// A token that takes part (0 <= t < Vt, g != 0) and whose target row lies in
// this problem's share; t is returned as the local row.
__device__ __forceinline__ bool token_valid(const EpiParams& e, int64_t tok, int64_t& t) {
  const int64_t tg = e.targets[tok];
  t = tg - e.v0;
  return tg >= 0 && tg < e.Vt && t >= 0 && t < e.V && e.g[tok] != 0.0f;
}

// A part of a split dH contraction: the raw fp32 sums of this tile's K range,
// stored for the reduction, which adds the parts in increasing order and
// applies the epilogue below. 32 lanes store 32 consecutive columns of a row.
__device__ __forceinline__ void epi_store_part(const GemmProblem& p, Acc& acc, int part, int64_t m0, int64_t n0,
                                               const Frag& f) {
  const EpiParams& e = p.ep;
  float* P = e.dhp + (int64_t)part * e.dhp_stride;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = m0 + f.row(mi, r);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int64_t n = n0 + f.col(ni);
        if (m < p.M && n < p.N) P[m * e.ldo + n] = acc[mi][ni][r];
      }
    }
}

// dH rows of the chunk: out[m, :] = s C[m, :] + tcoef[m] W[t_m, :]. The
// tile's per-token (target, coefficient) pairs are staged in LDS first.
template <typename T>
__device__ __forceinline__ void epi_store(const GemmProblem& p, Acc& acc, int64_t m0, int64_t n0,
                                          const Frag& f, const EpiLds& L) {
  char* smem = L.a[0];
  const EpiParams& e = p.ep;
  T* out = static_cast<T*>(e.out);
  float* out32 = static_cast<float*>(e.out);  // out_dt == DT_F32: a share's partial dH
  const bool f32 = e.out_dt == DT_F32 && !std::is_same<T, float>::value;
  const T* W = static_cast<const T*>(e.W);
  const float sc = e.scales[e.chunk].x;
  int32_t* ts = reinterpret_cast<int32_t*>(smem);
  float* cs = reinterpret_cast<float*>(smem + kTileM * sizeof(int32_t));
  float* fs = reinterpret_cast<float*>(smem + kTileM * (sizeof(int32_t) + sizeof(float)));
  for (int i = threadIdx.x; i < kTileM; i += kThreads) {
    const int64_t m = m0 + i;
    int64_t t = -1;
    const bool valid = m < p.M && token_valid(e, e.tok0 + m, t);
    ts[i] = valid ? (int32_t)t : -1;
    cs[i] = valid ? e.tcoef[e.tok0 + m] : 0.0f;
    // per-token mode: the row's factor s rowf (s a power of two, so the product is exact)
    fs[i] = e.rowf == nullptr ? sc : (m < p.M ? sc * e.rowf[e.tok0 + m] : 0.0f);
  }
  __syncthreads();
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = f.row(mi, r);
      const int64_t m = m0 + rl;
      const int32_t tr = ts[rl];
      const T* wrow = W + (int64_t)(tr >= 0 ? tr : 0) * e.ldW;  // row 0 stands in; its value is not used
      const float c = cs[rl];
      const float fr = fs[rl];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int64_t n = n0 + f.col(ni);
        // a zero factor (a token that takes no part) gives +0, whatever the sign of C
        const float base = fr == 0.0f ? 0.0f : acc[mi][ni][r] * fr;
        const float withw = fmaf(c, ld_f32(wrow, n < p.N ? n : 0), base);
        if (m < p.M && n < p.N) {
          const float o = tr >= 0 ? withw : base;
          if (f32) out32[m * e.ldo + n] = o;
          else out[m * e.ldo + n] = (T)o;
        }
      }
    }
}

// dW rows: table[v, :] += s C[v, :] + sum, in token order, of tcoef[n] h[n, :]
// (the table is read and written once per chunk: non-temporal accesses keep
// it from displacing the operand panels that other tiles share in L2)
// over the chunk's valid tokens with target v. The tile's 256 list heads are
// loaded and validated once into LDS (entries of targets absent from the
// chunk are stale), so a row without targets costs one LDS read.
template <typename T, typename TT>
__device__ __forceinline__ void epi_accum_t(const GemmProblem& p, Acc& acc, int64_t m0, int64_t n0,
                                            const Frag& f, const EpiLds& L) {
  char* smem = L.a[0];
  const EpiParams& e = p.ep;
  TT* tab = static_cast<TT*>(e.out);
  const T* h = static_cast<const T*>(e.h);
  const float sc = e.scales[e.chunk].x;
  int32_t* hs = reinterpret_cast<int32_t*>(smem);
  for (int i = threadIdx.x; i < kTileM; i += kThreads) {
    const int64_t m = m0 + i;
    int32_t j = (m < p.M && e.head != nullptr) ? e.head[m] : -1;
    int64_t t;
    if (!(j >= 0 && j < e.ntok && token_valid(e, e.tok0 + j, t) && t == m)) j = -1;
    hs[i] = j;
  }
  __syncthreads();
  TT* __restrict__ tb = tab;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    // per block of 16 rows: load every old table value first, then add and store
    float val[16][NI];
    TT old[16][NI];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = m0 + f.row(mi, r);
      const int64_t mc = m < p.M ? m : p.M - 1;  // in-bounds stand-in, not stored
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int64_t n = n0 + f.col(ni);
        old[r][ni] = e.tab_store ? (TT)0.0f : __builtin_nontemporal_load(&tb[mc * e.ldo + (n < p.N ? n : p.N - 1)]);
        val[r][ni] = acc[mi][ni][r] * sc;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = f.row(mi, r);
      int32_t j = hs[rl];
      // at most ntok steps: the walk ends even if the list were malformed
      for (int64_t it = 0; it < e.ntok && j >= 0 && j < e.ntok; ++it) {
        const float c = e.tcoef[e.tok0 + j];
        const T* hrow = h + (e.tok0 + j) * e.ldh;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int64_t n = n0 + f.col(ni);
          if (n < p.N) val[r][ni] = fmaf(c, ld_f32(hrow, n), val[r][ni]);
        }
        j = e.next[j];
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = m0 + f.row(mi, r);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int64_t n = n0 + f.col(ni);
        if (m < p.M && n < p.N) __builtin_nontemporal_store((TT)((float)old[r][ni] + val[r][ni]), &tb[m * e.ldo + n]);
      }
    }
  }
}

// dW rows of an FP32 table whose one-hot rows were added beforehand:
// table[v, :] += s C[v, :]. The tile goes through LDS (free once the K loop
// has ended) in two halves of 128 rows x 256 columns, four 32-row regions
// each; every thread then reads and writes whole 16-byte pieces of table rows
// with buffer instructions. The whole offset (row and column) is in the
// vector operand, which the range check covers (the scalar offset may not
// be), so the rows of a last tile that lie past the table's end read as 0
// instead of reading past the allocation; their stores are skipped. The old values of
// half 1 are in flight while half 0 is added and stored, so a tile waits for
// about one table round trip. Requires D % 4 == 0, a 16-byte aligned table
// and a 256-row tile span below 2 GiB (EpiParams::tab_fast).
// LDS region layout: row rr, column c at float rr * 256 + (c ^ 32 [bit 2 of rr]),
// so the two 32-lane row groups of an accumulator write fall on distinct banks.
__device__ __forceinline__ int tab_swz(int rr) { return ((rr >> 2) & 1) << 5; }

// Half h of the tile (rows of mi = 2 h and 2 h + 1 in both wave rows), times
// s, into the four LDS regions: region 2 wm + mh holds the 32 rows of
// mi = 2 h + mh of wave row wm, row rr and column c at float rr * 256 +
// (c ^ tab_swz(rr)).
__device__ __forceinline__ void tab_stage_half(const Acc& acc, int h, float sc, const Frag& f, const EpiLds& L) {
#pragma unroll
  for (int mh = 0; mh < 2; ++mh) {
    // the region pointer is chosen without a runtime index into L.a (which
    // would place the pointer array in private memory)
    float* reg = reinterpret_cast<float*>(f.wm ? L.a[2 + mh] : L.a[mh]);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = (r >> 2) * 8 + (f.lane >> 5) * 4 + (r & 3);
        const int col = f.wn * kWaveColsN + ni * 32 + (f.lane & 31);
        reg[rr * 256 + (col ^ tab_swz(rr))] = acc[2 * h + mh][ni][r] * sc;
      }
  }
}

// kFresh: the table holds no values yet (first chunk without accumulate): +0
// stands in for the old values, which are not read.
template <bool kFresh>
__device__ __forceinline__ void epi_accum_fast(const GemmProblem& p, Acc& acc, int64_t m0, int64_t n0,
                                               const Frag& f, const EpiLds& L) {
  static_assert(MI == 4 && kWaveM == 2 && kTileN == 256, "two halves of four 32-row regions");
  constexpr int kRpp = kThreads / 64;  // region rows covered by one pass of all threads (one per wave)
  constexpr int kPpr = 32 / kRpp;      // pieces of one region per thread
  static_assert(kPpr * kRpp == 32, "waves divide a region");
  const EpiParams& e = p.ep;
  const float sc = e.scales[e.chunk].x;
  const int tid = threadIdx.x;
  float* tb0 = static_cast<float*>(e.out) + m0 * e.ldo + n0;
  const int64_t span = ((p.M - m0) * e.ldo - n0) * 4;  // bytes from the tile's first element to the table's end
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(tb0, (short)0, span < 0x7FFFFFF0LL ? (int)span : 0x7FFFFFF0, 0x00020000);
  const int wrow = tid >> 6;             // this wave's row inside a kRpp-row group (wave-uniform)
  const int c = (tid & 63) * 4;          // this thread's first column inside the tile
  const bool colok = n0 + c < p.N;       // N % 4 == 0: the whole piece lies in [0, N)
  const int vbase = (wrow * (int)e.ldo + c) * 4;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  // row (inside the tile, less wrow) of piece i of half h: region q = i / kPpr
  // holds rows wm = q / 2, mi = 2h + q % 2; rows of a region advance by kRpp
  auto row_of = [](int h, int i) {
    const int q = i / kPpr;
    return (q >> 1) * 128 + (2 * h + (q & 1)) * 32 + kRpp * (i % kPpr);
  };
  // quarter k of half h: regions 2k and 2k + 1, pieces [2k kPpr, (2k + 2) kPpr)
  auto load_q = [&](int h, int k, f32x4 (&o)[2 * kPpr]) {
#pragma unroll
    for (int j = 0; j < 2 * kPpr; ++j) {
      if constexpr (kFresh)
        o[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      else
        o[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rs, vbase + row_of(h, 2 * kPpr * k + j) * (int)e.ldo * 4, 0, 2 /* nt */));
    }
  };
  auto to_lds = [&](int h) { tab_stage_half(acc, h, sc, f, L); };
  auto store_q = [&](int h, int k, const f32x4 (&o)[2 * kPpr]) {
#pragma unroll
    for (int j = 0; j < 2 * kPpr; ++j) {
      const int i = 2 * kPpr * k + j;
      const int rr = wrow + kRpp * (i % kPpr);
      const bool odd = (i / kPpr) & 1;
      const float* reg = reinterpret_cast<const float*>(k ? (odd ? L.a[3] : L.a[2]) : (odd ? L.a[1] : L.a[0]));
      const f32x4 add = *reinterpret_cast<const f32x4*>(reg + rr * 256 + (c ^ tab_swz(rr)));
      const int row = row_of(h, i) + wrow;
      if (colok && m0 + row < p.M)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o[j] + add), rs,
                                               vbase + row_of(h, i) * (int)e.ldo * 4, 0, 2 /* nt */);
    }
  };
  // the scheduling barriers keep the loads of half 1 where they are issued
  // (the scheduler would otherwise sink them below the barrier, next to
  // their use, and serialise the two round trips)
  f32x4 qa[2 * kPpr], qb[2 * kPpr];
  to_lds(0);
  load_q(0, 0, qa);
  load_q(0, 1, qb);
  __syncthreads();
  store_q(0, 0, qa);
  __builtin_amdgcn_sched_barrier(0);
  load_q(1, 0, qa);
  __builtin_amdgcn_sched_barrier(0);
  store_q(0, 1, qb);
  __builtin_amdgcn_sched_barrier(0);
  load_q(1, 1, qb);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  to_lds(1);
  __syncthreads();
  store_q(1, 0, qa);
  store_q(1, 1, qb);
}

// dW rows of an operand-dtype (16-bit) table: each element becomes
//     round(old + (s C + sum, in list order, of tcoef[n] h[n, col]))
// over the chunk's valid tokens n with that row as target, the same
// operations in the same order as epi_accum_t (so the same bits). The tile
// goes through LDS as in epi_accum_fast (two halves of 128 rows, s C in fp32)
// and every thread reads and writes whole 16-byte pieces (8 elements) of table
// rows with buffer instructions whose whole offset is in the vector operand:
// rows of a last tile past the table's end read as 0 and are not stored. The
// old values of half 1 are in flight while half 0 is finished. The tile's
// validated list heads sit in the fifth LDS region (DMA pipeline only).
// Requires D % 8 == 0, a 16-byte aligned table and h, and a 256-row tile span
// below 2 GiB (EpiParams::tab_fast16).
template <typename T>
__device__ __forceinline__ void epi_accum_fast16(const GemmProblem& p, Acc& acc, int64_t m0, int64_t n0,
                                                 const Frag& f, const EpiLds& L) {
  static_assert(sizeof(T) == 2, "a 16-bit table");
  static_assert(MI == 4 && kWaveM == 2 && kTileN == 256, "two halves of four 32-row regions");
  constexpr int kPpr = kTileN / 8;           // 16-byte pieces per tile row
  constexpr int kRowStep = kThreads / kPpr;  // rows covered by one pass of all threads
  constexpr int kPieces = 128 / kRowStep;    // pieces per thread and half
  static_assert(kPieces * kRowStep == 128 && 32 % kRowStep == 0, "threads divide a half and a region");
  typedef T t8 __attribute__((ext_vector_type(8)));
  const EpiParams& e = p.ep;
  const float sc = e.scales[e.chunk].x;
  const int tid = threadIdx.x;
  const T* h = static_cast<const T*>(e.h);
  T* tb0 = static_cast<T*>(e.out) + m0 * e.ldo + n0;
  const int64_t span = ((p.M - m0) * e.ldo - n0) * 2;  // bytes from the tile's first element to the table's end
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(tb0, (short)0, span < 0x7FFFFFF0LL ? (int)span : 0x7FFFFFF0, 0x00020000);
  const int pc = tid % kPpr;             // this thread's columns [8 pc, 8 pc + 8) of the tile
  const int r0 = tid / kPpr;             // its first local row; piece q adds q kRowStep rows
  const bool colok = n0 + 8 * pc < p.N;  // D % 8 == 0: a piece lies in [0, N) or past it
  int32_t* hs = reinterpret_cast<int32_t*>(L.x);
  for (int i = tid; i < kTileM; i += kThreads) {
    const int64_t m = m0 + i;
    int32_t j = (m < p.M && e.head != nullptr) ? e.head[m] : -1;
    int64_t t;
    if (!(j >= 0 && j < e.ntok && token_valid(e, e.tok0 + j, t) && t == m)) j = -1;
    hs[i] = j;
  }
  // piece q of half hf: local row r0 + q kRowStep, in region (q kRowStep) / 32
  // (r0 < kRowStep, so the region does not depend on the thread and no
  // runtime index into L.a is needed), which holds the 32 tile rows of wave
  // row region / 2 and block mi = 2 hf + region % 2
  auto region = [](int q) { return (q * kRowStep) >> 5; };
  auto tile_row = [&](int hf, int q) {
    const int g = region(q);
    return (g >> 1) * 128 + (2 * hf + (g & 1)) * 32 + ((q * kRowStep) & 31) + r0;
  };
  auto load_old = [&](int hf, u32x4 (&o)[kPieces]) {
#pragma unroll
    for (int q = 0; q < kPieces; ++q) {
      const int row = tile_row(hf, q);
      if (e.tab_store)
        o[q] = u32x4{0u, 0u, 0u, 0u};
      else
        o[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, (row * (int)e.ldo + 8 * pc) * 2, 0, 2 /* nt */);
    }
  };
  auto finish = [&](int hf, const u32x4 (&o)[kPieces]) {
#pragma unroll
    for (int q = 0; q < kPieces; ++q) {
      const int row = tile_row(hf, q);
      const int rr = ((q * kRowStep) & 31) + r0;
      const float* reg = reinterpret_cast<const float*>(L.a[region(q)]);
      const float* src = reg + rr * 256 + ((8 * pc) ^ tab_swz(rr));
      float v[8];
      *reinterpret_cast<float4*>(v) = *reinterpret_cast<const float4*>(src);
      *reinterpret_cast<float4*>(v + 4) = *reinterpret_cast<const float4*>(src + 4);
      // the one-hot part, at most ntok steps: the walk ends even if the list were malformed
      int32_t j = hs[row];
      for (int64_t it = 0; colok && it < e.ntok && j >= 0 && j < e.ntok; ++it) {
        const float c = e.tcoef[e.tok0 + j];
        const t8 x = *reinterpret_cast<const t8*>(h + (e.tok0 + j) * e.ldh + n0 + 8 * pc);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = fmaf(c, (float)x[k], v[k]);
        j = e.next[j];
      }
      const t8 old = __builtin_bit_cast(t8, o[q]);
      t8 out;
#pragma unroll
      for (int k = 0; k < 8; ++k) out[k] = (T)((float)old[k] + v[k]);
      if (colok && m0 + row < p.M)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, out), rs, (row * (int)e.ldo + 8 * pc) * 2, 0,
                                               2 /* nt */);
    }
  };
  u32x4 qa[kPieces], qb[kPieces];
  load_old(0, qa);
  tab_stage_half(acc, 0, sc, f, L);
  __syncthreads();  // the list heads and half 0 are in LDS
  __builtin_amdgcn_sched_barrier(0);
  load_old(1, qb);
  __builtin_amdgcn_sched_barrier(0);
  finish(0, qa);
  __syncthreads();  // half 0 has been read
  tab_stage_half(acc, 1, sc, f, L);
  __syncthreads();
  finish(1, qb);
}

// Which dW epilogue a kernel carries (one per kernel keeps the code small: the
// dH and dW tiles' loops run side by side and share the instruction cache):
// ACC_FAST and ACC_FRESH are epi_accum_fast (an FP32 table whose one-hot rows
// are added beforehand; FRESH for a first chunk without accumulate),
// ACC_FAST16 is epi_accum_fast16 (a 16-bit operand-dtype table), ACC_ANY
// decides at run time among the list-walking epilogues.
enum AccMode : int { ACC_ANY = 0, ACC_FAST = 1, ACC_FRESH = 2, ACC_FAST16 = 3 };

template <typename T, int kAcc>
__device__ __forceinline__ void epi_accum(const GemmProblem& p, Acc& acc, int64_t m0, int64_t n0,
                                          const Frag& f, const EpiLds& L) {
  if constexpr (kAcc == ACC_FAST) {
    epi_accum_fast<false>(p, acc, m0, n0, f, L);
  } else if constexpr (kAcc == ACC_FRESH) {
    epi_accum_fast<true>(p, acc, m0, n0, f, L);
  } else if constexpr (kAcc == ACC_FAST16) {
    if constexpr (sizeof(T) == 2) epi_accum_fast16<T>(p, acc, m0, n0, f, L);
  } else {
    if (p.ep.out_dt == DT_F32)
      epi_accum_t<T, float>(p, acc, m0, n0, f, L);
    else
      epi_accum_t<T, T>(p, acc, m0, n0, f, L);
  }
}

// ---------------------------------------------------------------- main loop
// Operand staging: each thread moves kLoadsPerThread 16-byte chunks of A and
// of B per stage; chunk c covers row c / 8 of the tile, bytes (c % 8) * 16.
//
// Fast path (both operands 16-byte aligned): rows past M / N are clamped to
// the last valid row (finite data; those outputs are never stored, and the
// log-sum-exp epilogue masks them to -inf), and every stage but a partial
// last one is loaded with unconditional vector loads. The partial last stage
// (K % BK != 0) goes through load_chunk, which zero-fills k >= K.
template <typename T, bool kFast>
__device__ __forceinline__ void mainloop(const GemmProblem& p, int64_t m0, int64_t n0, const Frag& f,
                                         char* smem, Acc& acc, int part = 0) {
  constexpr int per16 = ET<T>::per16;
  constexpr int BK = (kRowBytes / 16) * per16;  // K elements per stage
  const int tid = threadIdx.x;
  // a split problem's part covers the columns [k0, k0 + Kp) of both operands
  const int64_t k0 = p.kparts > 1 ? (int64_t)part * p.kpart : 0;
  const int64_t Kp = p.kparts > 1 ? min(p.K - k0, p.kpart) : p.K;
  const T* A = static_cast<const T*>(p.A) + k0;
  const T* B = static_cast<const T*>(p.B) + k0;
  const int64_t nfull = kFast ? Kp / BK : 0;              // stages loaded without masks
  const int64_t nstage = (Kp + BK - 1) / BK;              // >= 1
  const int64_t kc = (tid & 7) * per16;                    // this thread's k offset in a stage

  const T* pa[kLoadsPerThread];
  const T* pb[kLoadsPerThread];
  if constexpr (kFast) {
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
      const int row = (tid >> 3) + i * (kThreads / 8);
      const int64_t ra = min(m0 + row, p.M - 1), rb = min(n0 + row, p.N - 1);
      pa[i] = A + ra * p.lda + kc;
      pb[i] = B + rb * p.ldb + kc;
    }
  }
  u32x4 ra[kLoadsPerThread], rb[kLoadsPerThread];
  auto gload = [&](int64_t kt) {
    if (kFast && kt < nfull) {
#pragma unroll
      for (int i = 0; i < kLoadsPerThread; ++i) {
        ra[i] = *reinterpret_cast<const u32x4*>(pa[i] + kt * BK);
        rb[i] = *reinterpret_cast<const u32x4*>(pb[i] + kt * BK);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kLoadsPerThread; ++i) {
        const int row = (tid >> 3) + i * (kThreads / 8);
        const int64_t k = kt * BK + kc;
        ra[i] = load_chunk<T>(A, p.lda, m0 + row, p.M, k, Kp, p.a_vec != 0);
        rb[i] = load_chunk<T>(B, p.ldb, n0 + row, p.N, k, Kp, p.b_vec != 0);
      }
    }
  };
  auto sstore = [&](int buf) {
    char* sa = smem + buf * kStageBytes;
    char* sb = sa + kTileM * kPitch;
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
      const int c = tid + i * kThreads;
      const int off = (c >> 3) * kPitch + (c & 7) * 16;
      *reinterpret_cast<u32x4*>(sa + off) = ra[i];
      *reinterpret_cast<u32x4*>(sb + off) = rb[i];
    }
  };
  const int lrow = f.lane & 31;
  const int lk = (f.lane >> 5) * 16;
  auto compute = [&](int buf) {
    const char* sa = smem + buf * kStageBytes + (f.wm * kWaveRowsM + lrow) * kPitch + lk;
    const char* sb = smem + buf * kStageBytes + kTileM * kPitch + (f.wn * kWaveColsN + lrow) * kPitch + lk;
    u32x4 af[2][MI], bf[2][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) af[0][mi] = *reinterpret_cast<const u32x4*>(sa + mi * 32 * kPitch);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) bf[0][ni] = *reinterpret_cast<const u32x4*>(sb + ni * 32 * kPitch);
#pragma unroll
    for (int s = 0; s < kRowBytes / 32; ++s) {
      const int cur = s & 1;
      if (s + 1 < kRowBytes / 32) {  // fragments of the next slab while this one multiplies
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
          af[cur ^ 1][mi] = *reinterpret_cast<const u32x4*>(sa + mi * 32 * kPitch + (s + 1) * 32);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          bf[cur ^ 1][ni] = *reinterpret_cast<const u32x4*>(sb + ni * 32 * kPitch + (s + 1) * 32);
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = mfma_step((T*)nullptr, af[cur][mi], bf[cur][ni], acc[mi][ni]);
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int64_t kt = 0; kt < nstage; ++kt) {
    const int buf = (int)(kt & 1);
    if (kt + 1 < nstage) gload(kt + 1);
    compute(buf);
    if (kt + 1 < nstage) sstore(buf ^ 1);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- direct-to-LDS main loop
// Raw workgroup barrier: the memory clobber keeps the compiler from moving
// LDS accesses across it, and no vmcnt(0) is implied (the DMA of later
// stages stays in flight); each wave waits for exactly the loads it needs.
#define LLP_BARRIER()                       \
  do {                                      \
    __builtin_amdgcn_sched_barrier(0);      \
    asm volatile("s_barrier" ::: "memory"); \
    __builtin_amdgcn_sched_barrier(0);      \
  } while (0)
// s_waitcnt vmcnt(N) through the builtin, so the compiler's own wait
// insertion knows which DMA has landed (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14; expcnt 7 and lgkmcnt 15 mean no wait on those counters)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt lgkmcnt(0): this wave's LDS reads have completed (vmcnt 63 and
// expcnt 7 mean no wait on those counters)
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// Scheduling of one MFMA step: the next step's kR fragment reads (into the
// other fragment registers) spread among this step's kM MFMAs, ceil(kR / kM)
// reads after each MFMA, so that each read has a whole step to land and the two
// fragment sets stay distinct registers (the scheduler would otherwise sink
// the reads behind most of the MFMAs and reuse their source registers).
template <int kPer, int kLeft>
__device__ __forceinline__ void sched_pairs() {
  if constexpr (kLeft > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, kPer, 0);  // then kPer DS reads
    sched_pairs<kPer, kLeft - 1>();
  }
}
template <int kR, int kM>
__device__ __forceinline__ void interleave_reads_mfma() {
  constexpr int kPer = (kR + kM - 1) / kM;  // reads after each of the first MFMAs
  static_assert(kR % kPer == 0 && kR / kPer <= kM, "reads divide evenly");
  constexpr int kPairs = kR / kPer;
  sched_pairs<kPer, kPairs>();
  if constexpr (kM > kPairs) __builtin_amdgcn_sched_group_barrier(0x008, kM - kPairs, 0);
}

// Stage k covers 128 bytes of K (four MFMA steps). Its A tile is unit 2k and
// its B tile unit 2k + 1; unit u lives in slot u % 5. Every wave moves a
// quarter-column of 8-row pieces of every unit from global memory to LDS by
// DMA (buffer_load ... lds): no wave stages operands through registers or
// writes them to LDS itself, and each row piece is one whole 128-byte line, so
// every L1 miss fetches a full line. While stage k multiplies, stage k + 1 is
// landing and the A tile of stage k + 2 is in flight; the barrier that ends
// stage k makes stage k + 1 visible and frees stage k's two slots. The B tile
// of stage k + 2 is issued right after that barrier into the first of them;
// the A tile of stage k + 3 goes into the second during the first two steps
// of stage k + 1. Fragments of step j + 1 are read from LDS while step j
// multiplies.
// K chunks at or past K read as 0 (offset past the buffer's end); a chunk that
// straddles K relies on the operand's padding columns being +0, which the
// host guarantees when it enables this path.
//
// kMn: both operands are stored K-row-major instead ([K][ld], the tile's 256
// rows contiguous within each K row: A = dlogits^T [V][C], B = W [V][D] for
// dH). A stage is then 64 K rows of 512 bytes per operand (the same 32 KiB
// slot); one DMA instruction moves two K rows, chunk p of K row k lands at
// chunk p ^ 4 (k % 4). A fragment is two ds_read_b64_tr_b16: in each group
// of 16 lanes, lane s points at 4 consecutive rows of K row s / 4, and the
// transposed read hands lane r the row r of 4 consecutive K rows, so a lane
// gets the same 8 K values in the same order as a 16-byte read of the
// K-contiguous layout. K rows at or past K read as 0 (past the buffer end).
template <typename T, bool kMn = false>
__device__ __forceinline__ void mainloop_dma(const GemmProblem& p, int64_t m0, int64_t n0, const Frag& f,
                                             char* const (&buf)[kNS], Acc& acc, int part = 0) {
  static_assert(kTileM == kTileN, "A and B slots have one shape");
  static_assert(!kMn || sizeof(T) == 2, "K-row-major operands are 16-bit");
  constexpr int per16 = ET<T>::per16;
  constexpr int BKE = kSB / (int)sizeof(T);                    // K elements per stage
  constexpr int kRowsPerLoad = 64 * 16 / kSB;                  // rows one wave instruction covers
  constexpr int kLoads = kTileM / kRowsPerLoad / (kThreads / 64);  // instructions per wave per unit
  static_assert(kLoads * kRowsPerLoad * (kThreads / 64) == kTileM, "the waves cover a slot");
  constexpr int kSteps = kSB / 32;  // MFMA steps per stage: a step takes 32 bytes of K per row
  const int lane = f.lane;
  const int wave = f.wm * kWaveN + f.wn;
  auto rsrc_of = [](const void* base, int64_t rows, int64_t ld) {
    const int64_t bytes = rows * ld * (int64_t)sizeof(T);
    const int nrec = bytes < 0x7FFFFFF0LL ? (int)bytes : 0x7FFFFFF0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nrec, 0x00020000);
  };
  auto rsrc_mn = [](const void* base, int64_t off, int64_t K, int64_t ld, int64_t cols) {
    // from column `off` of K row 0 to column round8(cols) of K row K - 1 (the
    // operand may be the column range of a wider buffer that ends there)
    const int64_t bytes = ((K - 1) * ld + ((cols + 7) & ~int64_t(7)) - off) * (int64_t)sizeof(T);
    const int nrec = bytes < 0x7FFFFFF0LL ? (int)bytes : 0x7FFFFFF0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(static_cast<const T*>(base) + off), (short)0, nrec,
                                             0x00020000);
  };
  // K-row-major problems may be split into fixed K ranges (parts): this
  // tile's rows [k0, k0 + Kp) of both operands
  // (K-contiguous operands: the columns [k0, k0 + Kp) of every row; the part
  // size is a multiple of 8, so no 16-byte piece straddles two parts)
  int64_t k0 = 0, Kp = p.K;
  if (p.kparts > 1) {
    k0 = (int64_t)part * p.kpart;
    Kp = min(p.K - k0, p.kpart);
  }
  const T* const Ak = static_cast<const T*>(p.A) + (kMn ? k0 * p.lda : k0);
  const T* const Bk = static_cast<const T*>(p.B) + (kMn ? k0 * p.ldb : k0);
  const __amdgpu_buffer_rsrc_t rsA = kMn ? rsrc_mn(Ak, m0, Kp, p.lda, p.M) : rsrc_of(Ak + m0 * p.lda, p.M - m0, p.lda);
  const __amdgpu_buffer_rsrc_t rsB = kMn ? rsrc_mn(Bk, n0, Kp, p.ldb, p.N) : rsrc_of(Bk + n0 * p.ldb, p.N - n0, p.ldb);
  // Per-lane offsets of the wave's first DMA instruction of a unit; the
  // others follow at a wave-uniform stride (the swizzle term depends on the
  // lane only), so one register per operand covers all of them.
  uint32_t voA, voB, strA, strB;
  int kel;            // K-contiguous: first K element of this lane's chunk (even instructions)
  uint32_t dodd = 0;  // K-contiguous: byte offset of odd instructions' chunk relative to even ones
  int kel_odd = 0;
  if constexpr (kMn) {
    constexpr int nw = kThreads / 64;
    static_assert(nw % 2 == 0 && kLoads * 2 * nw == 64, "K-row-major placement: two K rows per instruction");
    // instruction j of wave w moves K rows 2w + 2 nw j + {0, 1} (lanes 0-31,
    // 32-63); 2 nw is a multiple of 4, so a lane's K row modulo 4, and with it
    // the swizzle, is the same for every j
    const int krow = 2 * wave + (lane >> 5);        // K row of the stage this lane moves first
    const int c = (lane & 31) ^ (4 * (krow & 3));   // LDS chunk lane & 31 holds global chunk c
    voA = (uint32_t)(krow * p.lda * (int64_t)sizeof(T)) + (uint32_t)(c * 16);
    voB = (uint32_t)(krow * p.ldb * (int64_t)sizeof(T)) + (uint32_t)(c * 16);
    strA = (uint32_t)(2 * nw * p.lda * (int64_t)sizeof(T));
    strB = (uint32_t)(2 * nw * p.ldb * (int64_t)sizeof(T));
    kel = 0;
  } else {
    // LDS chunk position q of row r holds global chunk q ^ swz(r) (see
    // swz_row). The first instruction's rows r = 32 w + lane / 8 have r / 8
    // even; instruction j adds 8 j rows, so odd instructions flip bit 0 of
    // the chunk: one more per-lane constant, the byte delta to that chunk.
    static_assert(kRowsPerLoad == 8 && (kLoads * kRowsPerLoad) % 16 == 0, "row blocks of 8, wave blocks of 16");
    const int row = (wave * kLoads) * kRowsPerLoad + (lane >> 3);
    const int c = (lane & 7) ^ swz_row(row);  // LDS chunk lane & 7 holds global chunk c
    const int c1 = c ^ 1;                     // the same lane's chunk in odd instructions
    voA = (uint32_t)(row * p.lda * (int64_t)sizeof(T)) + (uint32_t)(c * 16);
    voB = (uint32_t)(row * p.ldb * (int64_t)sizeof(T)) + (uint32_t)(c * 16);
    strA = (uint32_t)(kRowsPerLoad * p.lda * (int64_t)sizeof(T));
    strB = (uint32_t)(kRowsPerLoad * p.ldb * (int64_t)sizeof(T));
    kel = c * per16;
    kel_odd = c1 * per16;
    dodd = (uint32_t)((c1 - c) * 16);  // +16 or -16 bytes (modulo 2^32)
  }
  const int lds_off = wave * kLoads * kRowsPerLoad * kSB;
  const int64_t nst = (Kp + BKE - 1) / BKE;

  // pieces [j0, j1) of unit (stage s, operand O) into `slot`
  // per-stage byte step of each operand (K-row-major: BKE K rows; else kSB
  // bytes of every row) and the part's K, all below 2^31 (checked by the host)
  const uint32_t kstA = kMn ? (uint32_t)(BKE * p.lda * (int64_t)sizeof(T)) : (uint32_t)kSB;
  const uint32_t kstB = kMn ? (uint32_t)(BKE * p.ldb * (int64_t)sizeof(T)) : (uint32_t)kSB;
  const int Kp32 = (int)Kp;
  auto issue = [&](char* slot, int64_t s64, auto Ov, int j0 = 0, int j1 = kLoads) {
    constexpr int O = decltype(Ov)::value;
    const int s = (int)s64;
    const uint32_t sofs = (uint32_t)s * (O ? kstB : kstA);
    const int klim = Kp32 - s * BKE;  // K elements of this stage that exist (uniform)
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      if (j < j0 || j >= j1) continue;
      uint32_t vo = (O ? voB : voA) + (uint32_t)j * (O ? strB : strA);
      uint32_t off;
      if constexpr (kMn) {  // K rows past K lie past the buffer's end and read as 0
        off = vo + sofs;
      } else {
        if (j & 1) vo += dodd;
        off = (((j & 1) ? kel_odd : kel) < klim) ? vo + sofs : 0xFFFFFFF0u;
      }
      // K-row-major: the 1 KiB block of instruction j holds K rows 2w + 2 nw j, +1
      char* const dst = kMn ? slot + wave * 1024 + j * (kThreads / 64) * 1024 : slot + lds_off + j * kRowsPerLoad * kSB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(O ? rsB : rsA, (lds_void_t*)dst, 16, off, 0, 0, 0);
    }
  };
  // fragments of step j of the stage held in slots (sa, sb)
  // K-row-major fragments: per-lane byte offset inside a slot of the fragment
  // rows [r0, r0 + 32) for step 0 and the first half of K (steps and the second
  // half add 16 and 4 K rows: immediate offsets)
  auto mn_off = [&](int r0) {
    const int s4 = (lane & 15) >> 2;                                // K row inside the group of 4
    const int m = r0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);     // first of this lane's 4 rows
    const int krow = 8 * (lane >> 5) + s4;
    return krow * 512 + (((m >> 3) ^ (4 * s4)) << 4) + ((m & 7) << 1);
  };
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  auto read_mn = [&](const char* slot, int off, int j) {
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(slot + off + j * 16 * 512));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(slot + off + j * 16 * 512 + 4 * 512));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
    u32x4 r;
    r[0] = a[0];
    r[1] = a[1];
    r[2] = b[0];
    r[3] = b[1];
    return r;
  };
  int mnA[MI], mnB[NI];
  if constexpr (kMn) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) mnA[mi] = mn_off(f.wm * kWaveRowsM + mi * 32);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) mnB[ni] = mn_off(f.wn * kWaveColsN + ni * 32);
  }
  auto read_step = [&](const char* sa, const char* sb, int j, u32x4 (&fa)[MI], u32x4 (&fb)[NI]) {
    if constexpr (kMn) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) fa[mi] = read_mn(sa, mnA[mi], j);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) fb[ni] = read_mn(sb, mnB[ni], j);
      return;
    }
    const int c = 2 * j + (lane >> 5);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int row = f.wm * kWaveRowsM + mi * 32 + (lane & 31);
      fa[mi] = *reinterpret_cast<const u32x4*>(sa + row * kSB + ((c ^ swz_row(row)) * 16));
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int row = f.wn * kWaveColsN + ni * 32 + (lane & 31);
      fb[ni] = *reinterpret_cast<const u32x4*>(sb + row * kSB + ((c ^ swz_row(row)) * 16));
    }
  };
  auto mma = [&](const u32x4 (&fa)[MI], const u32x4 (&fb)[NI]) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = mfma_step((T*)nullptr, fa[mi], fb[ni], acc[mi][ni]);
  };
  // LDS read instructions of one step's fragments: one 16-byte read per
  // block, or two transposed 8-byte reads per block (K-row-major)
  constexpr int kReadsPerStep = (kMn ? 2 : 1) * (MI + NI);
  using O_A = std::integral_constant<int, 0>;
  using O_B = std::integral_constant<int, 1>;
  u32x4 fa[2][MI], fb[2][NI];  // by step parity

  auto stage = [&](int64_t k, auto Iv) {
    constexpr int I = decltype(Iv)::value;  // k % kNS
    char* const sa = buf[(2 * I) % kNS];
    char* const sb = buf[(2 * I + 1) % kNS];
    if (k >= nst) return;  // uniform over the workgroup
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      if (j + 1 < kSteps) read_step(sa, sb, j + 1, fa[(j + 1) & 1], fb[(j + 1) & 1]);
      if (j + 1 < kSteps) mma(fa[j & 1], fb[j & 1]);
      // the A tile of stage k + 2 goes, half after each of the first two
      // steps, into the slot that held stage k - 1's B tile: spreading the
      // DMA keeps the address queues from filling at the barrier
      constexpr int kHalf = kLoads / 2;
      if (j < 2 && k >= 1 && k + 2 < nst) issue(buf[(2 * I + 4) % kNS], k + 2, O_A{}, j * kHalf, (j + 1) * kHalf);
      if (j + 1 < kSteps) interleave_reads_mfma<kReadsPerStep, MI * NI>();
    }
    // this wave's pieces of stage k + 1 have landed (only the A tile of stage
    // k + 2 may remain in flight) and its reads of stage k have completed
    // (the last step's fragments are in registers), so stage k's slots may
    // be refilled once every wave has passed the barrier
    if (k + 2 < nst) wait_vm<kLoads>();
    else wait_vm<0>();
    wait_lgkm0();
    LLP_BARRIER();
    if (k + 1 < nst) read_step(buf[(2 * I + 2) % kNS], buf[(2 * I + 3) % kNS], 0, fa[0], fb[0]);
    if (k + 2 < nst) issue(sa, k + 2, O_B{});  // unit 2k + 5 goes to slot (2k) % 5
    // the last step of stage k multiplies while the next stage's first
    // fragments come from LDS (after the barrier every wave reads at once)
    mma(fa[(kSteps - 1) & 1], fb[(kSteps - 1) & 1]);
    if (k + 1 < nst) interleave_reads_mfma<kReadsPerStep, MI * NI>();
  };

  // units 0 .. 4: stages 0 and 1 and the A tile of stage 2
  issue(buf[0], 0, O_A{});
  issue(buf[1], 0, O_B{});
  if (nst > 1) {
    issue(buf[2], 1, O_A{});
    issue(buf[3], 1, O_B{});
  }
  if (nst > 2) issue(buf[4], 2, O_A{});
  if (nst > 2) wait_vm<3 * kLoads>();  // stage 0 landed
  else if (nst > 1) wait_vm<2 * kLoads>();
  else wait_vm<0>();
  LLP_BARRIER();
  read_step(buf[0], buf[1], 0, fa[0], fb[0]);
  static_assert(kSteps % 2 == 0, "step parity restarts with every stage");
  for (int64_t kb = 0; kb < nst; kb += kNS) {
    stage(kb + 0, std::integral_constant<int, 0>{});
    stage(kb + 1, std::integral_constant<int, 1>{});
    stage(kb + 2, std::integral_constant<int, 2>{});
    stage(kb + 3, std::integral_constant<int, 3>{});
    stage(kb + 4, std::integral_constant<int, 4>{});
  }
}

template <typename T, int E, bool kDma, bool kMn = false, int kAcc = ACC_ANY>
__device__ __forceinline__ void tile_run(const GemmProblem& p, int id, char* const (&buf)[kNS]) {
  int tm, tn;
  int part = 0;  // K range of a split problem (part-major tile order)
  if constexpr (E == EPI_STORE) {
    if (p.kparts > 1) {
      const int per = p.tiles_m * p.tiles_n;
      part = id / per;
      id -= part * per;
    }
  }
  tile_coords(id, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * kTileM;
  const int64_t n0 = (int64_t)tn * kTileN;
  const int tid = threadIdx.x;
  // the wave index is uniform per wave; readfirstlane tells the compiler so,
  // which keeps per-wave addresses and buffer descriptors in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  Frag f;
  f.lane = tid & 63;
  f.wm = wave / kWaveN;
  f.wn = wave % kWaveN;

  Acc acc;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  if constexpr (kDma) {
    mainloop_dma<T, kMn>(p, m0, n0, f, buf, acc, part);
  } else {
    if (p.a_vec && p.b_vec)
      mainloop<T, true>(p, m0, n0, f, buf[0], acc, part);
    else
      mainloop<T, false>(p, m0, n0, f, buf[0], acc, part);
  }
  const EpiLds L = {{buf[0], buf[1], buf[2], buf[3]}, kDma ? buf[4] : nullptr};

  if constexpr (E == EPI_LSE_PARTIAL) epi_lse_partial<T, false>(p, acc, tm, m0, n0, f);
  if constexpr (E == EPI_LSE_Q) epi_lse_partial<T, true>(p, acc, tm, m0, n0, f);
  if constexpr (E == EPI_DLOGITS) epi_dlogits<T>(p, acc, m0, n0, f, L);
  if constexpr (E == EPI_STORE) {
    if (p.kparts > 1)
      epi_store_part(p, acc, part, m0, n0, f);
    else
      epi_store<T>(p, acc, m0, n0, f, L);
  }
  if constexpr (E == EPI_ACCUM) epi_accum<T, kAcc>(p, acc, m0, n0, f, L);
}

template <typename T, int E0, int E1, bool kDma, bool kMn0, int kAcc>
__device__ __forceinline__ void gemm_dispatch(const GemmProblem& p0, const GemmProblem& p1, int ntiles0,
                                              char* const (&buf)[kNS]) {
  const int bid = blockIdx.x;
  if (bid < ntiles0) {
    tile_run<T, E0, kDma, kMn0>(p0, xcd_remap(bid, ntiles0), buf);
  } else {
    const int b1 = bid - ntiles0;
    if constexpr (E1 != EPI_NONE) tile_run<T, E1, kDma, false, kAcc>(p1, xcd_remap(b1, (int)gridDim.x - ntiles0), buf);
  }
}

// The body of a one- or two-problem launch. kMn0: the first problem's
// operands are K-row-major (DMA pipeline only).
template <typename T, int E0, int E1, bool kDma, bool kMn0 = false, int kAcc = ACC_ANY>
__device__ __forceinline__ void gemm_entry(const GemmProblem& p0, const GemmProblem& p1, int ntiles0) {
  if constexpr (kDma) {
    // distinct LDS objects per slot (see kNS)
    __shared__ __attribute__((aligned(16))) char st0[kStageArr];
    __shared__ __attribute__((aligned(16))) char st1[kStageArr];
    __shared__ __attribute__((aligned(16))) char st2[kStageArr];
    __shared__ __attribute__((aligned(16))) char st3[kStageArr];
    __shared__ __attribute__((aligned(16))) char st4[kStageArr];
    char* const buf[kNS] = {st0, st1, st2, st3, st4};
    gemm_dispatch<T, E0, E1, true, kMn0, kAcc>(p0, p1, ntiles0, buf);
  } else {
    static_assert(kLdsBytes >= 4 * kOpB, "epilogue regions fit in the staged buffer");
    __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
    // the epilogues use the first four regions; the fifth is never touched
    char* const buf[kNS] = {smem, smem + kOpB, smem + 2 * kOpB, smem + 3 * kOpB, smem};
    static_assert(!kMn0, "K-row-major operands need the DMA pipeline");
    gemm_dispatch<T, E0, E1, false, false, ACC_ANY>(p0, p1, ntiles0, buf);
  }
}

// One kernel name per role, so that traces and counter runs tell them apart
// by name alone: the forward's logits tiles with lse partials (over a batch)
// or with the single call's numerators, the backward's dlogits recompute,
// and a chunk's dH (first problem) and dW (second) contractions.
template <typename T, bool kDma>
__global__ __launch_bounds__(kThreads, 1) void lse_partial_kernel(GemmProblem p0, int ntiles0) {
  gemm_entry<T, EPI_LSE_PARTIAL, EPI_NONE, kDma>(p0, p0, ntiles0);
}
template <typename T, bool kDma>
__global__ __launch_bounds__(kThreads, 1) void lse_q_kernel(GemmProblem p0, int ntiles0) {
  gemm_entry<T, EPI_LSE_Q, EPI_NONE, kDma>(p0, p0, ntiles0);
}
template <typename T, bool kDma>
__global__ __launch_bounds__(kThreads, 1) void dlogits_kernel(GemmProblem p0, int ntiles0) {
  gemm_entry<T, EPI_DLOGITS, EPI_NONE, kDma>(p0, p0, ntiles0);
}
template <typename T, bool kDma, bool kMn0 = false, int kAcc = ACC_ANY>
__global__ __launch_bounds__(kThreads, 1) void dh_dw_kernel(GemmProblem p0, GemmProblem p1, int ntiles0) {
  gemm_entry<T, EPI_STORE, EPI_ACCUM, kDma, kMn0, kAcc>(p0, p1, ntiles0);
}

// One chunk's dH (K-row-major operands) and dW tiles together with the next
// chunk's logits tiles, which write their own buffers: the single call's
// forward (EPI_LSE_Q: numerators and partials) or the backward's dlogits
// recompute (EPI_DLOGITS: dlogits^T). The launch tails overlap. The dW tiles,
// the shortest, come last.
template <typename T, int kAcc, int E2>
__device__ __forceinline__ void gemm3_entry(const GemmProblem& p0, const GemmProblem& p1, const GemmProblem& p2,
                                            int nt0, int nt2) {
  __shared__ __attribute__((aligned(16))) char st0[kStageArr];
  __shared__ __attribute__((aligned(16))) char st1[kStageArr];
  __shared__ __attribute__((aligned(16))) char st2[kStageArr];
  __shared__ __attribute__((aligned(16))) char st3[kStageArr];
  __shared__ __attribute__((aligned(16))) char st4[kStageArr];
  char* const buf[kNS] = {st0, st1, st2, st3, st4};
  const int bid = blockIdx.x;
  if (bid < nt0) {
    tile_run<T, EPI_STORE, true, true, kAcc>(p0, xcd_remap(bid, nt0), buf);
  } else if (bid < nt0 + nt2) {
    tile_run<T, E2, true, false, kAcc>(p2, xcd_remap(bid - nt0, nt2), buf);
  } else {
    tile_run<T, EPI_ACCUM, true, false, kAcc>(p1, xcd_remap(bid - nt0 - nt2, (int)gridDim.x - nt0 - nt2), buf);
  }
}
template <typename T, int kAcc>
__global__ __launch_bounds__(kThreads, 1) void dh_dw_fwd_kernel(GemmProblem p0, GemmProblem p1, GemmProblem p2,
                                                                 int nt0, int nt2) {
  gemm3_entry<T, kAcc, EPI_LSE_Q>(p0, p1, p2, nt0, nt2);
}
template <typename T, int kAcc>
__global__ __launch_bounds__(kThreads, 1) void dh_dw_dlogits_kernel(GemmProblem p0, GemmProblem p1,
                                                                     GemmProblem p2, int nt0, int nt2) {
  gemm3_entry<T, kAcc, EPI_DLOGITS>(p0, p1, p2, nt0, nt2);
}

template <typename T>
hipError_t launch3_t(const GemmProblem& p0, const GemmProblem* p1, const GemmProblem& p2, hipStream_t s) {
  if constexpr (sizeof(T) != 2) {
    return hipErrorInvalidValue;
  } else {
    const int nt0 = problem_tiles(p0), nt2 = problem_tiles(p2);
    const int nt1 = p1 ? problem_tiles(*p1) : 0;
    GemmProblem empty = {};
    const GemmProblem& b = p1 ? *p1 : empty;
    const int acc = p1 == nullptr ? ACC_FAST : !p1->ep.tab_fast ? ACC_ANY : p1->ep.tab_store ? ACC_FRESH : ACC_FAST;
    if (!p0.mn || !p0.dma || !p2.dma || (p1 && !p1->dma) || acc == ACC_ANY || p0.epi != EPI_STORE ||
        (p2.epi != EPI_LSE_Q && p2.epi != EPI_DLOGITS) || p2.kparts > 1 || (p1 && p1->kparts > 1))
      return hipErrorInvalidValue;
    dim3 grid(nt0 + nt1 + nt2), block(kThreads);
    if (p2.epi == EPI_LSE_Q) {
      if (acc == ACC_FAST) dh_dw_fwd_kernel<T, ACC_FAST><<<grid, block, 0, s>>>(p0, b, p2, nt0, nt2);
      else dh_dw_fwd_kernel<T, ACC_FRESH><<<grid, block, 0, s>>>(p0, b, p2, nt0, nt2);
    } else {
      if (acc == ACC_FAST) dh_dw_dlogits_kernel<T, ACC_FAST><<<grid, block, 0, s>>>(p0, b, p2, nt0, nt2);
      else dh_dw_dlogits_kernel<T, ACC_FRESH><<<grid, block, 0, s>>>(p0, b, p2, nt0, nt2);
    }
    return hipGetLastError();
  }
}

template <typename T>
hipError_t launch_t(const GemmProblem* p0, const GemmProblem* p1, hipStream_t s) {
  const int nt0 = p0 ? problem_tiles(*p0) : 0;
  const int nt1 = p1 ? problem_tiles(*p1) : 0;
  if (nt0 + nt1 == 0) return hipSuccess;
  // a split problem (dH, EPI_STORE) comes first; every other problem is unsplit
  if ((p1 && p1->kparts > 1) || (p0 && p0->kparts > 1 && p0->epi != EPI_STORE)) return hipErrorInvalidValue;
  GemmProblem empty = {};
  const GemmProblem& a = p0 ? *p0 : empty;
  const GemmProblem& b = p1 ? *p1 : empty;
  const int e0 = p0 ? p0->epi : EPI_NONE;
  const int e1 = p1 ? p1->epi : EPI_NONE;
  dim3 grid(nt0 + nt1), block(kThreads);
  const bool dma = (p0 == nullptr || p0->dma) && (p1 == nullptr || p1->dma);
  if (e0 == EPI_LSE_PARTIAL && e1 == EPI_NONE) {
    if (dma) lse_partial_kernel<T, true><<<grid, block, 0, s>>>(a, nt0);
    else lse_partial_kernel<T, false><<<grid, block, 0, s>>>(a, nt0);
  } else if (e0 == EPI_LSE_Q && e1 == EPI_NONE) {
    if (dma) lse_q_kernel<T, true><<<grid, block, 0, s>>>(a, nt0);
    else lse_q_kernel<T, false><<<grid, block, 0, s>>>(a, nt0);
  } else if (e0 == EPI_DLOGITS && e1 == EPI_NONE) {
    if (dma) dlogits_kernel<T, true><<<grid, block, 0, s>>>(a, nt0);
    else dlogits_kernel<T, false><<<grid, block, 0, s>>>(a, nt0);
  } else if ((e0 == EPI_STORE || e0 == EPI_NONE) && (e1 == EPI_ACCUM || e1 == EPI_NONE)) {
    const bool mn = p0 != nullptr && p0->mn;
    // the dW epilogue of this launch (any mode serves when there are no dW tiles)
    const int acc = p1 == nullptr ? ACC_FAST
                    : p1->ep.tab_fast16 && sizeof(T) == 2 && p1->ep.out_dt != DT_F32 ? ACC_FAST16
                    : !p1->ep.tab_fast ? ACC_ANY
                    : p1->ep.tab_store ? ACC_FRESH
                                       : ACC_FAST;
    if (mn && !(sizeof(T) == 2 && dma)) return hipErrorInvalidValue;  // K-row-major: 16-bit, DMA pipeline
    if (!dma) {
      dh_dw_kernel<T, false><<<grid, block, 0, s>>>(a, b, nt0);
    } else if (mn) {
      if constexpr (sizeof(T) == 2) {
        if (acc == ACC_FAST) dh_dw_kernel<T, true, true, ACC_FAST><<<grid, block, 0, s>>>(a, b, nt0);
        else if (acc == ACC_FRESH)
          dh_dw_kernel<T, true, true, ACC_FRESH><<<grid, block, 0, s>>>(a, b, nt0);
        else if (acc == ACC_FAST16)
          dh_dw_kernel<T, true, true, ACC_FAST16><<<grid, block, 0, s>>>(a, b, nt0);
        else dh_dw_kernel<T, true, true, ACC_ANY><<<grid, block, 0, s>>>(a, b, nt0);
      }
    } else {
      if (acc == ACC_FAST) dh_dw_kernel<T, true, false, ACC_FAST><<<grid, block, 0, s>>>(a, b, nt0);
      else if (acc == ACC_FRESH)
        dh_dw_kernel<T, true, false, ACC_FRESH><<<grid, block, 0, s>>>(a, b, nt0);
      else if (acc == ACC_FAST16) {
        if constexpr (sizeof(T) == 2) dh_dw_kernel<T, true, false, ACC_FAST16><<<grid, block, 0, s>>>(a, b, nt0);
      } else dh_dw_kernel<T, true, false, ACC_ANY><<<grid, block, 0, s>>>(a, b, nt0);
    }
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm3(int dt, const GemmProblem& p0, const GemmProblem* p1, const GemmProblem& p2, hipStream_t s) {
  switch (dt) {
    case DT_BF16: return launch3_t<__bf16>(p0, p1, p2, s);
    case DT_F16: return launch3_t<_Float16>(p0, p1, p2, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(int dt, const GemmProblem* p0, const GemmProblem* p1, hipStream_t s) {
  switch (dt) {
    case DT_BF16: return launch_t<__bf16>(p0, p1, s);
    case DT_F16: return launch_t<_Float16>(p0, p1, s);
    case DT_F32: return launch_t<float>(p0, p1, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace llp
