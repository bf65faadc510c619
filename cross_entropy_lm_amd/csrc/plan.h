// Host-side argument checks, chunk policy and workspace layout of the C ABI.
// Pure C++: no HIP call, so every error path can be exercised without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/llp.h"
#include "tile_config.h"

namespace llp {

constexpr int64_t kMaxD = int64_t(1) << 22;     // transpose grid.y and tile count limits
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;  // one workgroup per row / grid.x
constexpr int64_t kTile = kTileM;               // contraction tile edge (M and N)
static_assert(kTileM == kTileN, "square tiles");
constexpr int64_t kAlign = 256;                 // workspace region alignment (bytes)
constexpr int64_t kGroupCols = 4096;            // small chunks: columns of a dW group at most
constexpr int64_t kGroupBytes = int64_t(1) << 30;  // ... and bytes of one group buffer at most

inline bool dtype_ok(int dt) { return dt == LLP_F32 || dt == LLP_BF16 || dt == LLP_F16; }
inline int64_t esize(int dt) { return dt == LLP_F32 ? 4 : 2; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// a * b with overflow detection (a, b >= 0).
inline bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}
inline bool add_ok(int64_t a, int64_t b, int64_t* out) {
  if (a > INT64_MAX - b) return false;
  *out = a + b;
  return true;
}

inline int64_t chunk_rows(int64_t N, int64_t V, int64_t chunk) {
  if (N < 0 || V < 1) return -1;
  int64_t c = chunk > 0 ? chunk : (int64_t(1) << 24) / V;
  if (c < 1) c = 1;
  const int64_t cap = N > 0 ? N : 1;
  return c < cap ? c : cap;
}

// Byte layout of a workspace: regions appended at kAlign boundaries.
struct Layout {
  int64_t bytes = 0;
  bool ok = true;
  int64_t add(int64_t n) {  // returns the region's offset, or -1 (sets ok = false)
    if (!ok) return -1;
    int64_t off = round_up(bytes, kAlign);
    int64_t end;
    if (n < 0 || !add_ok(off, n, &end)) {
      ok = false;
      return -1;
    }
    bytes = end;
    return off;
  }
};

// Shapes common to both linear entry points; returns an llp_status.
inline int check_linear_shapes(int64_t N, int64_t D, int64_t V, int dtype) {
  if (!dtype_ok(dtype)) return LLP_EINVAL;
  if (N < 0 || D < 1 || V < 1) return LLP_EINVAL;
  if (N > kMaxRows || V > kMaxRows || D > kMaxD) return LLP_EOVERFLOW;
  int64_t t;
  if (!mul_ok(N, D, &t) || !mul_ok(t, esize(dtype), &t)) return LLP_EOVERFLOW;
  if (!mul_ok(V, D, &t) || !mul_ok(t, 4, &t)) return LLP_EOVERFLOW;
  // one workgroup per 256 x 256 output tile: the tile count must fit grid.x
  if (ceil_div(V, kTile) * ceil_div(N > 0 ? N : 1, kTile) > kMaxRows) return LLP_EOVERFLOW;
  if (ceil_div(V, kTile) * ceil_div(D, kTile) > kMaxRows) return LLP_EOVERFLOW;
  return LLP_OK;
}

struct FwdPlan {
  int64_t P = 0;             // partial rows: kWaveM per vocab tile
  int64_t off_partials = 0;  // float2 [P][N]
  int64_t off_zt = 0;        // float [N]
  int64_t bytes = 0;
};

inline int plan_fwd(int64_t N, int64_t D, int64_t V, int dtype, FwdPlan* p) {
  int st = check_linear_shapes(N, D, V, dtype);
  if (st != LLP_OK) return st;
  *p = FwdPlan();
  if (N == 0) return LLP_OK;
  p->P = kWaveM * ceil_div(V, kTile);
  Layout L;
  int64_t n;
  if (!mul_ok(p->P, N, &n) || !mul_ok(n, 8, &n)) return LLP_EOVERFLOW;
  p->off_partials = L.add(n);
  p->off_zt = L.add(N * 4);
  if (!L.ok) return LLP_EOVERFLOW;
  p->bytes = L.bytes;
  return LLP_OK;
}

struct BwdPlan {
  int64_t C = 0, K = 0;                  // tokens per chunk, number of chunks
  int64_t ldWt = 0, ldS = 0, ldSt = 0;   // leading dimensions (elements), multiples of 8
  // dW is accumulated once per group of G consecutive chunks (G = 1: per
  // chunk): the single call with dW and K >= 2, and the two-call path for
  // small chunks (fewer than 128 dH tiles) or 16-bit operands with
  // D % 8 == 0. G = 2, or for small chunks up to 4096 group columns while one
  // group buffer stays within 1 GiB.
  int64_t G = 1;
  // Working chunk. With more than two small chunks per group, or a pair of
  // chunks when dW or db is requested, and the layout without W^T, a group
  // is processed as one chunk of Cw = min(G C, N) tokens when the table is
  // FP32: its logits, dH and dW in one pass each, which fills the 256-token
  // tiles that a 110-token chunk would leave half empty and, for a pair of
  // large chunks, halves the launches in the same group buffer. Otherwise
  // Cw = C. Buffers are sized for Cw.
  int64_t Cw = 0;
  // leading dimension of the vocab-major and h^T buffers: G ldSt (chunk j of
  // a group in the columns [j ldSt, j ldSt + C)), which also holds round8(Cw)
  int64_t ldP = 0;
  int64_t off_scales = -1;               // float2 [K]
  int64_t off_lse = -1;                  // float [N] when the caller gives no lse
  FwdPlan fwd;                           // and the forward's workspace, placed after it
  int64_t off_fwd = -1;
  // dH reads its operands as stored (vocabulary rows: dlogits^T [V][ldq] and
  // W [V][D]) when the shapes allow it: 16-bit operands, D % 8 == 0, and both
  // operands spanning < 2 GiB. The layout then holds no W^T and no token-major
  // dlogits; W and the workspace must be 16-byte aligned (else LLP_EINVAL).
  bool kmajor = false;
  // bf16 single call: per-token numerators (same shape conditions, whether or
  // not dH is asked for, so that every subset of outputs computes alike)
  bool qtok = false;
  // dH: the vocabulary is cut into dh_parts = ceil(V / dh_part) fixed parts
  // of dh_part rows (kDhPart, or kDhPartF32 for fp32 operands); with more
  // than one, each part's fp32 sums go to [dh_parts][dh_rows][D]
  // (dh_rows: the most rows one dH contraction covers, G C where small chunks group)
  int64_t dh_part = kDhPart;
  int64_t dh_parts = 1;
  int64_t dh_rows = 0;
  int64_t off_dhp = -1;
  int64_t off_Wt = -1;                   // W^T [D][ldWt]            (dH, not kmajor)
  int64_t off_dS = -1;                   // dlogits [C][ldS]         (dH, not kmajor)
  int64_t off_dSt = -1;                  // dlogits^T [V][ldP]       (dW or db)
  int64_t off_ht = -1;                   // h^T of one chunk (or pair) [D][ldP] (dW)
  int64_t off_tcoef = -1;                // float [N]: one-hot part g (1 - p_t) per token
  int64_t off_head = -1;                 // int32 [V]: first chunk token per target   (dW or db)
  int64_t off_next = -1;                 // int32 [C]: next chunk token, same target (dW or db)
  // fused forward + backward only
  int64_t P = 0;                         // partial rows per token: kWaveM per vocab tile
  int64_t off_part = -1;                 // float2 [P][C]: one chunk's forward partials
  int64_t off_zt = -1;                   // float [N]: target logits
  int64_t off_qflag = -1;                // int32 [N]: per-token mode, tokens with block-relative numerators
  int64_t off_cq = -1;                   // float [N]: per-token mode, the tokens' gradient factors
  // second numerator and partial buffers (16-bit operands, dH, K >= 2): the
  // next chunk's forward then runs in the same launch as this chunk's dH / dW
  // (the groups alternate between the two numerator buffers)
  int64_t off_dSt2 = -1;
  int64_t off_part2 = -1;
  int64_t bytes = 0;
};

// fused = 1: the layout of linear_logp_fwd_bwd, where each chunk's forward
// runs first: the chunk's partials, the target logits and (when the caller
// passes no lse) an lse buffer are added; the vocab-major buffer always exists
// (it first holds the chunk's softmax numerators); no separate forward.
inline int plan_bwd(int64_t N, int64_t D, int64_t V, int dtype, int64_t chunk, int want_dH,
                    int want_dW, int want_db, int have_lse, BwdPlan* p, int fused = 0) {
  int st = check_linear_shapes(N, D, V, dtype);
  if (st != LLP_OK) return st;
  *p = BwdPlan();
  p->C = chunk_rows(N, V, chunk);
  p->K = N > 0 ? ceil_div(N, p->C) : 0;
  if (N == 0 || !(want_dH || want_dW || want_db)) return LLP_OK;
  const int64_t e = esize(dtype);
  p->ldWt = round_up(V, 8);
  p->ldS = round_up(V, 8);
  p->ldSt = round_up(p->C, 8);
  // small chunks: 16-bit operands and fewer than 128 tiles of 256 x 256 in a
  // chunk's dH
  const bool few = esize(dtype) == 2 && ceil_div(p->C, kTile) * ceil_div(D, kTile) < 128;
  // with C % 8 == 0 a group's token rows are contiguous columns, and dH runs once per group
  const bool small = few && p->C % 8 == 0;
  // Group size from the shapes alone (which outputs are requested does not
  // change the schedule): 2 chunks, or for small chunks up to kGroupCols
  // columns and kGroupBytes of group buffer, balanced over the groups.
  // 16-bit operands with D % 8 == 0 whose W and pair of chunk columns each
  // span < 2 GiB (the layout the overlapped backward reads as stored): the
  // two-call path pairs chunks too, its next chunk's dlogits recompute filling
  // the launches that carry no dW
  bool pairable;
  {
    const int64_t lim = 0x7FFFFFF0LL;
    int64_t vd, vq;
    pairable = e == 2 && D % 8 == 0 && mul_ok(V, D, &vd) && mul_ok(vd, e, &vd) && vd < lim &&
               mul_ok(V, 2 * p->ldSt, &vq) && mul_ok(vq, e, &vq) && vq < lim;
  }
  int64_t gc = 1;
  if (p->K >= 2 && (fused || few || pairable)) {
    int64_t g = 2;
    if (few) {
      int64_t vb;
      const int64_t by_cols = kGroupCols / p->ldSt;
      const int64_t by_bytes = (mul_ok(V, p->ldSt, &vb) && mul_ok(vb, e, &vb) && vb > 0) ? kGroupBytes / vb : 0;
      const int64_t m = by_cols < by_bytes ? by_cols : by_bytes;
      if (m > g) g = m;
    }
    gc = g < p->K ? g : p->K;
    // as many groups as that size needs, of balanced sizes (a last group of a
    // few chunks would leave its launches' token tiles part empty)
    gc = ceil_div(p->K, ceil_div(p->K, gc));
  }
  p->G = want_dW ? gc : 1;
  // 16-bit operands with D % 8 == 0 whose operands (W, and a group's
  // dlogits^T) each span < 2 GiB: dH reads them as stored (kmajor), the bf16
  // single call stores per-token numerators (qtok), and a group runs as one
  // working chunk (Cw)
  bool shape;
  {
    const int64_t lim = 0x7FFFFFF0LL;
    int64_t vd, vq;
    const int64_t cols = gc > 2 ? gc * p->ldSt : 2 * p->ldSt;
    shape = e == 2 && D % 8 == 0 && mul_ok(V, D, &vd) && mul_ok(vd, e, &vd) && vd < lim && mul_ok(V, cols, &vq) &&
            mul_ok(vq, e, &vq) && vq < lim;
    p->kmajor = want_dH && shape;
    p->qtok = fused && dtype == LLP_BF16 && shape;
  }
  // (a pair of chunks only when dW or db is requested: their group buffer is
  // then there anyway, and logp, lse and dH do not depend on the chunking)
  p->Cw = (shape && (gc > 2 || (gc == 2 && (want_dW || want_db)))) ? (gc * p->C < N ? gc * p->C : N) : p->C;
  {
    const int64_t wcols = round_up(p->Cw, 8);
    if (!mul_ok(p->G, p->ldSt, &p->ldP)) return LLP_EOVERFLOW;
    if (wcols > p->ldP) p->ldP = wcols;
    // the single call's forward tiles store numerators with 32-bit offsets
    // inside 128-row blocks: a row of that buffer stays below 2^24 bytes
    if (fused && p->ldP * e >= (int64_t(1) << 24)) return LLP_EOVERFLOW;
  }
  Layout L;
  int64_t n;
  p->off_scales = L.add(p->K * 8);
  if (!have_lse) {
    p->off_lse = L.add(N * 4);
    if (!fused) {
      st = plan_fwd(N, D, V, dtype, &p->fwd);
      if (st != LLP_OK) return st;
      p->off_fwd = L.add(p->fwd.bytes);
    }
  }
  if (fused) {
    p->P = kWaveM * ceil_div(V, kTile);
    if (!mul_ok(p->P, p->Cw, &n) || !mul_ok(n, 8, &n)) return LLP_EOVERFLOW;
    p->off_part = L.add(n);
    p->off_zt = L.add(N * 4);
    p->off_qflag = L.add(N * 4);
    p->off_cq = L.add(N * 4);
  }
  if (want_dH) {
    p->dh_part = e == 4 ? kDhPartF32 : kDhPart;
    p->dh_parts = ceil_div(V, p->dh_part);
    // small chunks take dH per group (C % 8 == 0) or per working chunk
    p->dh_rows = p->Cw > p->C ? p->Cw : (p->kmajor && p->G > 1 && small) ? p->G * p->C : p->C;
    if (p->dh_parts > 1) {
      int64_t rd;
      if (!mul_ok(p->dh_rows, D, &rd) || !mul_ok(rd, p->dh_parts, &n) || !mul_ok(n, 4, &n)) return LLP_EOVERFLOW;
      if (rd / 4 / 256 + 1 > kMaxRows) return LLP_EOVERFLOW;  // the reduction's grid
      // the dH tiles of every part, with a chunk's forward and dW tiles, in one grid
      if ((ceil_div(p->dh_rows, kTile) * ceil_div(D, kTile) * p->dh_parts + 3 * ceil_div(V, kTile) *
           (ceil_div(D, kTile) + ceil_div(p->Cw, kTile))) > kMaxRows)
        return LLP_EOVERFLOW;
      p->off_dhp = L.add(n);
    }
  }
  if (want_dH && !p->kmajor) {
    if (!mul_ok(D, p->ldWt, &n) || !mul_ok(n, e, &n)) return LLP_EOVERFLOW;
    p->off_Wt = L.add(n);
    if (!mul_ok(p->C, p->ldS, &n) || !mul_ok(n, e, &n)) return LLP_EOVERFLOW;
    p->off_dS = L.add(n);
  }
  if (want_dW || want_db || fused || p->kmajor) {
    if (!mul_ok(V, p->ldP, &n) || !mul_ok(n, e, &n)) return LLP_EOVERFLOW;
    // the backward's dlogits tiles store into this buffer with 32-bit offsets
    // inside 8-row groups: a row stays below 2^28 bytes
    if (p->ldP * e >= (int64_t(1) << 28)) return LLP_EOVERFLOW;
    p->off_dSt = L.add(n);
    // a second one, so that chunk k + 1's logits tiles (the single call's
    // forward, the backward's dlogits recompute) run in the launch of chunk
    // k's dH / dW (only when the working schedule has two chunks or more)
    if (p->kmajor && ceil_div(N, p->Cw) >= 2) {
      p->off_dSt2 = L.add(n);
      if (fused) {
        if (!mul_ok(p->P, p->Cw, &n) || !mul_ok(n, 8, &n)) return LLP_EOVERFLOW;
        p->off_part2 = L.add(n);
      }
    }
  }
  if (want_dW) {
    if (!mul_ok(D, p->ldP, &n) || !mul_ok(n, e, &n)) return LLP_EOVERFLOW;
    p->off_ht = L.add(n);
  }
  p->off_tcoef = L.add(N * 4);
  if (want_dW || want_db) {
    p->off_head = L.add(V * 4);
    p->off_next = L.add(p->Cw * 4);
  }
  if (!L.ok) return LLP_EOVERFLOW;
  // the working chunk's contraction tiles must fit grid.x too
  if (ceil_div(p->Cw, kTile) * ceil_div(V, kTile) > kMaxRows) return LLP_EOVERFLOW;
  p->bytes = L.bytes;
  return LLP_OK;
}

inline int check_rows(int64_t N, int64_t V, int dtype) {
  if (!dtype_ok(dtype)) return LLP_EINVAL;
  if (N < 0 || V < 1) return LLP_EINVAL;
  if (N > kMaxRows) return LLP_EOVERFLOW;
  int64_t t;
  if (!mul_ok(N, V, &t) || !mul_ok(t, esize(dtype), &t)) return LLP_EOVERFLOW;
  return LLP_OK;
}

}  // namespace llp
