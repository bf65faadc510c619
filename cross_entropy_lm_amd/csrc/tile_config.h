// Contraction tile geometry, shared by the host plan (grid sizes, workspace
// layout) and the gfx950 kernels. No HIP dependency.
#pragma once

#ifndef LLP_WAVES_M
#define LLP_WAVES_M 2  // waves along M (the rows of a 256 x 256 output tile)
#endif
#ifndef LLP_WAVES_N
#define LLP_WAVES_N 4  // waves along N
#endif
#ifndef LLP_GROUP_M
#define LLP_GROUP_M 4  // tiles along M per scheduling group (operand reuse in L2)
#endif

namespace llp {
constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kWaveM = LLP_WAVES_M;
constexpr int kWaveN = LLP_WAVES_N;
constexpr int kThreads = 64 * kWaveM * kWaveN;
constexpr int kGroupM = LLP_GROUP_M;
constexpr int kXcds = 8;  // MI355X: workgroups are dealt round-robin to 8 XCDs
// dH = dlogits W sums over the vocabulary in fixed parts of kDhPart rows
// (ceil(V / kDhPart) parts, a function of V and the operand width alone),
// each part a tile of its own whose fp32 partial is added in increasing part
// order: a chunk's few dH tiles then spread over many CUs, and a token's dH
// does not depend on the chunking or the batch. fp32 operands take shorter
// parts: their contraction runs 16 times slower per flop, so a 32768-row dH
// tile would outlast every dW tile of its launch.
constexpr long long kDhPart = 32768;     // 16-bit operands
constexpr long long kDhPartF32 = 8192;   // fp32 operands
static_assert(kTileM % (32 * kWaveM) == 0 && kTileN % (32 * kWaveN) == 0, "wave tile must be 32-aligned");
}  // namespace llp
