// CPU-only check of the library's host plan (argument validation, chunk
// policy, workspace layout), built with the address and undefined-behaviour
// sanitizers by tests/test_plan_sanitize.py. It exercises the overflow shapes
// of the INT_MAX loop-counter review of RL-Kernel PR #495 (for example
// V = 2147482624, and N V beyond 2^31) and checks every status code and the
// layout invariants over a deterministic sweep of shapes. No GPU, no HIP.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <utility>
#include <vector>

#include "../../cross_entropy_lm_amd/csrc/plan.h"

using namespace llp;

static int g_fail = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

// Regions of a backward plan: (offset, bytes) of every region that exists.
static std::vector<std::pair<int64_t, int64_t>> regions(const BwdPlan& p, int64_t N, int64_t D, int64_t V,
                                                        int dt, bool fused) {
  const int64_t e = esize(dt);
  std::vector<std::pair<int64_t, int64_t>> r;
  auto add = [&](int64_t off, int64_t n) {
    if (off >= 0) r.push_back({off, n});
  };
  add(p.off_scales, p.K * 8);
  add(p.off_lse, N * 4);
  if (p.off_fwd >= 0) add(p.off_fwd, p.fwd.bytes);
  add(p.off_Wt, D * p.ldWt * e);
  add(p.off_dS, p.C * p.ldS * e);
  add(p.off_dSt, V * p.ldP * e);
  add(p.off_dSt2, V * p.ldP * e);
  add(p.off_ht, D * p.ldP * e);
  add(p.off_dhp, p.dh_parts * p.dh_rows * D * 4);
  add(p.off_tcoef, N * 4);
  add(p.off_head, V * 4);
  add(p.off_next, p.Cw * 4);
  if (fused) {
    add(p.off_part, p.P * p.Cw * 8);
    add(p.off_part2, p.P * p.Cw * 8);
    add(p.off_zt, N * 4);
    add(p.off_qflag, N * 4);
    add(p.off_cq, N * 4);
  }
  return r;
}

static void check_layout(int64_t N, int64_t D, int64_t V, int dt, int64_t chunk, int dh, int dw, int db, int lse,
                         bool fused) {
  BwdPlan p;
  const int st = plan_bwd(N, D, V, dt, chunk, dh, dw, db, lse, &p, fused ? 1 : 0);
  EXPECT(st == LLP_OK || st == LLP_EOVERFLOW);
  if (st != LLP_OK) return;
  EXPECT(p.C >= 1 && (N == 0 || p.C <= N));
  EXPECT(p.K == (N > 0 ? (N + p.C - 1) / p.C : 0));
  if (N == 0 || !(dh || dw || db)) {
    EXPECT(p.bytes == 0);
    return;
  }
  EXPECT(p.ldSt % 8 == 0 && p.ldSt >= p.C);
  // dW groups of G chunks: G = 1 or 2, or more for small chunks within the
  // 4096-column and 1 GiB caps, never more than the chunks
  EXPECT(p.G >= 1 && p.G <= (p.K > 1 ? p.K : 1) && p.ldP >= p.G * p.ldSt);
  EXPECT(p.ldP == (p.G * p.ldSt > round_up(p.Cw, 8) ? p.G * p.ldSt : round_up(p.Cw, 8)));
  if (p.G > 2) EXPECT(p.G * p.ldSt <= 4096 && V * p.ldP * esize(dt) <= (int64_t(1) << 30));
  // balanced groups: G is the smallest size that gives its number of groups
  if (p.G >= 2) EXPECT(p.G == (p.K + (p.K + p.G - 1) / p.G - 1) / ((p.K + p.G - 1) / p.G));
  if (!dw) EXPECT(p.G == 1);
  // the layout holds only what the requested outputs need
  EXPECT(p.kmajor == (dh && esize(dt) == 2 && D % 8 == 0 && (p.off_Wt < 0)));
  if (p.kmajor) EXPECT(p.off_Wt < 0 && p.off_dS < 0 && p.off_dSt >= 0);
  if (dh) EXPECT(p.dh_part == (esize(dt) == 4 ? 8192 : 32768) && p.dh_parts == (V + p.dh_part - 1) / p.dh_part);
  if (dh) EXPECT(p.dh_rows == p.C || p.dh_rows == p.G * p.C || p.dh_rows == p.Cw);
  // the working chunk: the chunk, or a whole group of two or more chunks (at most N tokens)
  // (Cw does not depend on which outputs are requested: G is the group of the dW schedule)
  EXPECT(p.Cw >= p.C && p.Cw <= (N > p.C ? N : p.C) && (p.Cw - p.C) % p.C == 0 || p.Cw == N);
  if (dw && p.Cw > p.C) EXPECT(p.G >= 2 && p.Cw == (p.G * p.C < N ? p.G * p.C : N));
  // a dH-only call on chunks of 128 or more dH tiles keeps the caller's chunk
  // (no group buffer to reuse, and dH does not depend on the chunking)
  if (dh && !dw && !db && (p.C + kTile - 1) / kTile * ((D + kTile - 1) / kTile) >= 128) EXPECT(p.Cw == p.C);
  // a group of two or more chunks on the layout without W^T runs as one working chunk
  if (dw && p.G >= 2 && esize(dt) == 2 && D % 8 == 0 && V * D * 2 < 0x7FFFFFF0LL &&
      V * p.ldP * 2 < 0x7FFFFFF0LL)
    EXPECT(p.Cw == (p.G * p.C < N ? p.G * p.C : N));
  EXPECT(round_up(p.Cw, 8) <= p.ldP);
  EXPECT((p.off_dhp >= 0) == (dh && p.dh_parts > 1));
  if (dh && !p.kmajor) EXPECT(p.off_Wt >= 0 && p.off_dS >= 0);
  if (!dh) EXPECT(p.off_Wt < 0 && p.off_dS < 0 && p.off_dSt2 < 0);
  if (!dw) EXPECT(p.off_ht < 0);
  if (!(dw || db)) EXPECT(p.off_head < 0 && p.off_next < 0);
  if (p.qtok) EXPECT(fused && dt == LLP_BF16);
  auto r = regions(p, N, D, V, dt, fused);
  std::sort(r.begin(), r.end());
  int64_t end = 0;
  for (auto& x : r) {
    EXPECT(x.first % kAlign == 0);  // every region starts on a 256-byte boundary
    EXPECT(x.first >= end);         // regions do not overlap
    end = x.first + x.second;
  }
  EXPECT(end <= p.bytes);
}

int main() {
  const int dts[3] = {LLP_F32, LLP_BF16, LLP_F16};
  // --- status codes of the shape checks
  FwdPlan f;
  EXPECT(plan_fwd(-1, 128, 1024, LLP_F32, &f) == LLP_EINVAL);
  EXPECT(plan_fwd(4, 0, 1024, LLP_F32, &f) == LLP_EINVAL);
  EXPECT(plan_fwd(4, 128, 0, LLP_F32, &f) == LLP_EINVAL);
  EXPECT(plan_fwd(4, 128, 1024, 7, &f) == LLP_EINVAL);
  EXPECT(plan_fwd(int64_t(1) << 31, 128, 1024, LLP_F32, &f) == LLP_EOVERFLOW);
  EXPECT(plan_fwd(4, int64_t(1) << 23, 1024, LLP_F32, &f) == LLP_EOVERFLOW);
  EXPECT(plan_fwd(INT64_MAX, INT64_MAX, INT64_MAX, LLP_BF16, &f) == LLP_EOVERFLOW);
  // V just below 2^31 (the review's boundary case): the shapes are accepted
  // with 64-bit sizes; the forward's partials N x 2 ceil(V / 256) x 8 bytes fit
  const int64_t Vbig = 2147482624;
  EXPECT(plan_fwd(64, 8, Vbig, LLP_BF16, &f) == LLP_OK);
  EXPECT(f.P == 2 * ((Vbig + 255) / 256) && f.bytes >= f.P * 64 * 8);
  EXPECT(plan_fwd(1, 1, Vbig + 1024, LLP_BF16, &f) == LLP_EOVERFLOW);  // V > 2^31 - 1
  EXPECT(plan_fwd(1 << 20, 1 << 22, Vbig, LLP_BF16, &f) == LLP_EOVERFLOW);  // tile count exceeds grid.x
  // N V beyond 2^31 is an ordinary logits-only shape
  EXPECT(check_rows(32768, 151936, LLP_BF16) == LLP_OK);
  EXPECT(check_rows(1, Vbig, LLP_BF16) == LLP_OK);
  EXPECT(check_rows(int64_t(1) << 31, 2, LLP_BF16) == LLP_EOVERFLOW);
  EXPECT(check_rows(int64_t(1) << 30, INT64_MAX / 4, LLP_F32) == LLP_EOVERFLOW);
  EXPECT(check_rows(-1, 2, LLP_F32) == LLP_EINVAL && check_rows(1, 0, LLP_F32) == LLP_EINVAL);
  EXPECT(check_rows(1, 2, 9) == LLP_EINVAL);
  // --- chunk policy
  EXPECT(chunk_rows(32768, 151936, 0) == 110);
  EXPECT(chunk_rows(4096, 32768, 0) == 512);
  EXPECT(chunk_rows(8, 1, 0) == 8);                    // 2^24 clamped to N
  EXPECT(chunk_rows(100, Vbig, 0) == 1);               // V > 2^24: one row per chunk
  EXPECT(chunk_rows(100, 10, INT64_MAX) == 100);
  EXPECT(chunk_rows(0, 10, 0) == 1 && chunk_rows(-1, 10, 0) == -1 && chunk_rows(5, 0, 0) == -1);
  // --- backward plans at the boundary shapes
  BwdPlan b;
  EXPECT(plan_bwd(8, 8, Vbig, LLP_BF16, 0, 1, 1, 1, 1, &b) == LLP_OK);
  EXPECT(b.C == 1 && b.K == 8 && !b.kmajor);  // V D 2 bytes > 2 GiB: dH keeps the transposed copy
  EXPECT(plan_bwd(8, 8, Vbig, LLP_BF16, 0, 1, 1, 1, 1, &b, 1) == LLP_OK);
  EXPECT(plan_bwd(int64_t(1) << 30, 1 << 22, 1 << 30, LLP_BF16, 0, 1, 1, 1, 1, &b) == LLP_EOVERFLOW);
  EXPECT(plan_bwd(1 << 20, 4096, 1 << 20, LLP_F32, 1 << 20, 1, 1, 1, 0, &b) == LLP_OK);
  EXPECT(plan_bwd(16384, 4096, 32000, LLP_BF16, 2048, 1, 1, 0, 1, &b) == LLP_OK && b.kmajor && b.off_Wt < 0);
  EXPECT(plan_bwd(16384, 4096, 32000, LLP_BF16, 2048, 1, 1, 0, 1, &b, 1) == LLP_OK && b.qtok);
  EXPECT(plan_bwd(16384, 4096, 32000, LLP_F32, 2048, 1, 1, 0, 1, &b) == LLP_OK && !b.kmajor && b.off_Wt >= 0);
  EXPECT(plan_bwd(16384, 4092, 32000, LLP_F16, 2048, 1, 0, 0, 1, &b) == LLP_OK && !b.kmajor && b.off_Wt >= 0);
  // --- layout invariants over a deterministic sweep (including chunk
  // extremes and shapes whose byte sizes approach the 2 GiB operand limit)
  uint64_t x = 0x9E3779B97F4A7C15ull;
  auto rnd = [&](int64_t lo, int64_t hi) {
    x ^= x << 13;
    x ^= x >> 7;
    x ^= x << 17;
    return lo + (int64_t)(x % (uint64_t)(hi - lo + 1));
  };
  const int64_t Ns[] = {0, 1, 7, 255, 256, 257, 4096, 16384, 32768, 1 << 20};
  const int64_t Ds[] = {1, 8, 99, 136, 2048, 4096, 8192, 1 << 22};
  const int64_t Vs[] = {1, 255, 1031, 32000, 151936, 1 << 24, 1 << 25, Vbig};
  const int64_t chunks[] = {0, 1, 7, 64, 110, 512, 2048, 1 << 30, INT64_MAX};
  int cases = 0;
  for (int64_t N : Ns)
    for (int64_t D : Ds)
      for (int64_t V : Vs) {
        for (int k = 0; k < 3; ++k) {
          const int dt = dts[rnd(0, 2)];
          const int64_t ch = chunks[rnd(0, 8)];
          const int fl = (int)rnd(0, 15);
          check_layout(N, D, V, dt, ch, fl & 1, (fl >> 1) & 1, (fl >> 2) & 1, (fl >> 3) & 1, rnd(0, 1) == 1);
          ++cases;
        }
      }
  for (int i = 0; i < 20000; ++i) {
    const int64_t N = rnd(0, 1 << 16), D = rnd(1, 1 << 14), V = rnd(1, 1 << 18);
    check_layout(N, D, V, dts[rnd(0, 2)], rnd(-4, N + 3), (int)rnd(0, 1), (int)rnd(0, 1), (int)rnd(0, 1),
                 (int)rnd(0, 1), rnd(0, 1) == 1);
    ++cases;
  }
  printf("plan_check: %d layout cases, %d failures\n", cases, g_fail);
  return g_fail == 0 ? 0 : 1;
}
