// C ABI entry points (declared in include/llp.h): validate, lay out the
// caller's workspace, and enqueue the kernels on the caller's stream.
#include <stdlib.h>
#include <string.h>

#include <initializer_list>
#include <mutex>
#include <vector>

#include "../../include/llp.h"
#include "kernels.h"
#include "plan.h"

namespace llp {
namespace {

inline char* at(void* base, int64_t off) { return static_cast<char*>(base) + off; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Direct-to-LDS pipeline eligibility (see GemmProblem::dma): both operands
// aligned for vector loads and a 256-row tile of each spanning < 2 GiB.
// `kpad_zero`: the operands' padding columns up to round8(K) hold +0.
inline int dma_ok(const GemmProblem& p, int64_t e, bool kpad_zero) {
  const int64_t lim = 0x7FFFFFF0LL;
  const bool span = kTile * p.lda * e < lim && kTile * p.ldb * e < lim;
  const bool ktail = (p.K % (16 / e)) == 0 || kpad_zero;
  return (p.a_vec && p.b_vec && span && ktail) ? 1 : 0;
}

#define LLP_TRY(expr)                      \
  do {                                     \
    const hipError_t e_ = (expr);          \
    if (e_ != hipSuccess) return LLP_EHIP; \
  } while (0)

// Opt-in per-thread launch tracing (llp_trace_enable / llp_trace_read).
struct TraceRec {
  int kind;
  hipEvent_t start, stop;
};
struct Trace {
  bool on = false;
  std::vector<hipEvent_t> pool;  // created on demand, reused across traces
  size_t used = 0;
  std::vector<TraceRec> recs;
  int64_t dropped = 0;
};
thread_local Trace g_trace;

hipEvent_t trace_event() {
  Trace& t = g_trace;
  if (t.used == t.pool.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    t.pool.push_back(e);
  }
  return t.pool[t.used++];
}

template <class F>
hipError_t traced(int kind, hipStream_t s, F&& launch) {
  Trace& t = g_trace;
  if (!t.on) return launch();
  if (t.recs.size() >= (size_t)LLP_TRACE_MAX) {
    ++t.dropped;
    return launch();
  }
  hipEvent_t a = trace_event(), b = trace_event();
  if (a == nullptr || b == nullptr) return hipErrorOutOfMemory;
  hipError_t e = hipEventRecord(a, s);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, s);
  if (e == hipSuccess) t.recs.push_back({kind, a, b});
  return e;
}
#define LLP_LAUNCH(kind, expr) LLP_TRY(traced((kind), s, [&]() { return (expr); }))

// Opt-in device check (LLP_CHECK_DEVICE=1 in the environment, read on every
// call): each non-null pointer must be device or managed memory of the
// current device. Runs after the other argument checks and before any launch.
int check_device(std::initializer_list<const void*> ptrs) {
  const char* v = getenv("LLP_CHECK_DEVICE");
  if (v == nullptr || v[0] != '1') return LLP_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return LLP_EHIP;
  for (const void* p : ptrs) {
    if (p == nullptr) continue;
    hipPointerAttribute_t a = {};
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
      (void)hipGetLastError();  // an unknown (host) pointer: clear the error it leaves
      return LLP_EINVAL;
    }
    if (!(a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) || a.device != dev) return LLP_EINVAL;
  }
  return LLP_OK;
}
#define LLP_CHECK_DEVICE(...)                        \
  do {                                               \
    const int st_ = check_device({__VA_ARGS__});     \
    if (st_ != LLP_OK) return st_;                   \
  } while (0)

// Logits tile problem over tokens [tok0, tok0 + n) of h: A = W [V][D], B = h rows.
GemmProblem logits_problem(int64_t tok0, int64_t n, int64_t D, int64_t V, int dtype,
                           const void* h, const void* W) {
  GemmProblem p = {};
  const int64_t e = esize(dtype);
  const int per16 = (int)(16 / e);
  p.A = W;
  p.B = static_cast<const char*>(h) + tok0 * D * e;
  p.lda = D;
  p.ldb = D;
  p.M = V;
  p.N = n;
  p.K = D;
  p.a_vec = (D % per16 == 0) && aligned16(W);
  p.b_vec = (D % per16 == 0) && aligned16(p.B);
  p.tiles_m = (int)ceil_div(V, kTile);
  p.tiles_n = (int)ceil_div(n, kTile);
  p.dma = dma_ok(p, e, false);
  p.ep.V = V;
  p.ep.v0 = 0;  // the whole vocabulary unless the caller names a share
  p.ep.Vt = V;
  return p;
}

// Forward into (partials, zt) then the combine; shared by linear_logp_fwd and
// by the backward when no lse is given.
int run_forward(int64_t N, int64_t D, int64_t V, int dtype, const void* h, const void* W,
                const void* b, const int64_t* targets, float* logp, float* lse, void* ws,
                const FwdPlan& fp, hipStream_t s) {
  float2* partials = reinterpret_cast<float2*>(at(ws, fp.off_partials));
  float* zt = reinterpret_cast<float*>(at(ws, fp.off_zt));
  GemmProblem p = logits_problem(0, N, D, V, dtype, h, W);
  p.epi = EPI_LSE_PARTIAL;
  p.ep.bias = b;
  p.ep.targets = targets;
  p.ep.tok0 = 0;
  p.ep.partials = partials;
  p.ep.ldp = N;
  p.ep.zt = zt;
  LLP_LAUNCH(LLP_K_FWD_LSE, launch_gemm(dtype, &p, nullptr, s));
  LLP_LAUNCH(LLP_K_COMBINE, launch_lse_combine(partials, fp.P, N, zt, targets, V, N, logp, lse, nullptr, nullptr, s));
  return LLP_OK;
}

}  // namespace

// ---------------------------------------------------------------- forward without allocation
// Scratch of linear_logp_fwd_noalloc: the forward's per-block partials and
// target logits, in a device-global array instead of a caller's workspace
// (every device the library runs on holds its own copy until the process
// ends). Host code never uses the array's name as an address: the device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __attribute__((aligned(256))) unsigned char scratch[LLP_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on the first call on
// that device, with that device current).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LLP_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return LLP_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LLP_OK;
}
}  // namespace
}  // namespace llp

using namespace llp;

extern "C" {

int llp_version(void) { return 100; }

const char* llp_strerror(int status) {
  switch (status) {
    case LLP_OK: return "ok";
    case LLP_EINVAL: return "invalid argument";
    case LLP_EWORKSPACE: return "workspace too small";
    case LLP_EOVERFLOW: return "size overflow";
    case LLP_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int64_t linear_logp_chunk_rows(int64_t N, int64_t V, int64_t chunk) { return chunk_rows(N, V, chunk); }

int64_t linear_logp_num_chunks(int64_t N, int64_t V, int64_t chunk) {
  const int64_t c = chunk_rows(N, V, chunk);
  if (c < 0) return -1;
  return N > 0 ? ceil_div(N, c) : 0;
}

int linear_logp_fwd_workspace_size(int64_t N, int64_t D, int64_t V, int dtype, size_t* bytes) {
  if (bytes == nullptr) return LLP_EINVAL;
  FwdPlan fp;
  const int st = plan_fwd(N, D, V, dtype, &fp);
  if (st != LLP_OK) return st;
  *bytes = (size_t)fp.bytes;
  return LLP_OK;
}

int linear_logp_fwd(int64_t N, int64_t D, int64_t V, int dtype, const void* h, const void* W,
                    const void* b, const int64_t* targets, float* logp, float* lse, void* workspace,
                    size_t workspace_bytes, void* stream) {
  FwdPlan fp;
  int st = plan_fwd(N, D, V, dtype, &fp);
  if (st != LLP_OK) return st;
  if (N == 0) return LLP_OK;
  if (h == nullptr || W == nullptr || targets == nullptr || logp == nullptr) return LLP_EINVAL;
  if ((size_t)fp.bytes > workspace_bytes || (fp.bytes > 0 && workspace == nullptr)) return LLP_EWORKSPACE;
  LLP_CHECK_DEVICE(h, W, b, targets, logp, lse, workspace);
  return run_forward(N, D, V, dtype, h, W, b, targets, logp, lse, workspace, fp,
                     static_cast<hipStream_t>(stream));
}

int linear_logp_fwd_noalloc(int64_t N, int64_t D, int64_t V, int dtype, const void* h, const void* W,
                            const void* b, const int64_t* targets, float* logp, float* lse, void* stream) {
  FwdPlan fp;
  int st = plan_fwd(N, D, V, dtype, &fp);
  if (st != LLP_OK) return st;
  if (N == 0) return LLP_OK;
  if (h == nullptr || W == nullptr || targets == nullptr || logp == nullptr) return LLP_EINVAL;
  if ((size_t)fp.bytes > (size_t)LLP_SCRATCH_BYTES) return LLP_EWORKSPACE;
  LLP_CHECK_DEVICE(h, W, b, targets, logp, lse);
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != LLP_OK) return st;
  // every partial and every valid target's logit is written before it is
  // read, so nothing left by an earlier call needs clearing
  return run_forward(N, D, V, dtype, h, W, b, targets, logp, lse, ws, fp, static_cast<hipStream_t>(stream));
}

int linear_logp_bwd_workspace_size(int64_t N, int64_t D, int64_t V, int dtype, int64_t chunk,
                                   int want_dH, int want_dW, int want_db, int have_lse,
                                   size_t* bytes) {
  if (bytes == nullptr) return LLP_EINVAL;
  BwdPlan bp;
  const int st = plan_bwd(N, D, V, dtype, chunk, want_dH, want_dW, want_db, have_lse, &bp);
  if (st != LLP_OK) return st;
  *bytes = (size_t)bp.bytes;
  return LLP_OK;
}

}  // extern "C"
namespace llp {
namespace {
// The backward, and with `fused` the forward + backward of linear_logp_fwd_bwd:
// there each chunk's logits tile yields the chunk's lse partials and softmax
// numerators, the combine gives logp / lse / the one-hot part, and the
// softmax gradient is formed from the numerators; the logits are not
// recomputed. Everything after that is shared.
int backward_impl(int64_t N, int64_t D, int64_t V, int dtype, int64_t chunk, const void* h,
                  const void* W, const void* b, const int64_t* targets, const float* g,
                  const float* lse, float* logp_out, float* lse_out, void* dH, void* dW, int dW_dtype,
                  void* db, int accumulate, void* workspace, size_t workspace_bytes, void* stream,
                  bool fused, int64_t v0 = 0, int64_t Vt = -1, int dH_dtype = -1) {
  if (Vt < 0) Vt = V;
  if (dH_dtype < 0) dH_dtype = dtype;
  const bool want_dH = dH != nullptr, want_dW = dW != nullptr, want_db = db != nullptr;
  BwdPlan bp;
  const bool have_lse = fused ? lse_out != nullptr : lse != nullptr;
  int st = plan_bwd(N, D, V, dtype, chunk, want_dH, want_dW, want_db, have_lse, &bp, fused ? 1 : 0);
  if (st != LLP_OK) return st;
  if (accumulate != 0 && accumulate != 1) return LLP_EINVAL;
  if ((want_dW || want_db) && !(dW_dtype == LLP_F32 || dW_dtype == dtype)) return LLP_EINVAL;
  if (want_dH && !(dH_dtype == LLP_F32 || dH_dtype == dtype)) return LLP_EINVAL;
  if (want_db && b == nullptr) return LLP_EINVAL;
  if (N > 0 && (want_dH || want_dW || want_db) &&
      (h == nullptr || W == nullptr || targets == nullptr || g == nullptr))
    return LLP_EINVAL;
  if (fused && N > 0 && logp_out == nullptr) return LLP_EINVAL;
  if ((size_t)bp.bytes > workspace_bytes || (bp.bytes > 0 && workspace == nullptr)) return LLP_EWORKSPACE;
  // the layouts without W^T read W and the workspace with 16-byte accesses
  if (N > 0 && (bp.kmajor || bp.qtok) && !(aligned16(W) && aligned16(workspace))) return LLP_EINVAL;
  LLP_CHECK_DEVICE(h, W, b, targets, g, lse, logp_out, lse_out, dH, dW, db, workspace);

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t e = esize(dtype);
  const int64_t te = (dW_dtype == LLP_F32) ? 4 : e;
  // Without accumulate the first chunk's dW contraction stores into the
  // table instead of adding (+0 standing in for the old values), so the table
  // is zero-filled only when there is no chunk. An FP32 table's one-hot rows
  // of that first chunk are added after it, by the next chunk's preparation
  // (or by a launch of their own when there is one chunk).
  const bool store_first = want_dW && !accumulate && N > 0;
  if (!accumulate) {
    if (want_dW && !store_first) LLP_LAUNCH(LLP_K_SMALL, launch_zero(dW, V * D, (int)te, s));
    if (want_db) LLP_LAUNCH(LLP_K_SMALL, launch_zero(db, V, (int)te, s));
  }
  if (N == 0 || !(want_dH || want_dW || want_db)) return LLP_OK;

  const int64_t lim = 0x7FFFFFF0LL;
  const bool tab_fast = dW_dtype == LLP_F32 && D % 4 == 0 && aligned16(dW) && kTile * D * 4 < lim;
  // With an FP32 table (both paths): one dW contraction per group of G
  // consecutive chunks (the plan's G, from the shapes alone) over the columns
  // of all of them, which sit side by side in the vocab-major buffer
  // [V][G ldSt] and the h^T buffer [D][G ldSt]: the table is read and written
  // once per group. The group shares one power-of-two scale (scale index =
  // group index), so every part of the contraction is in the same units.
  // The two-call path groups small chunks (16-bit operands, a dH grid of
  // fewer than 128 tiles) and pairs the chunks of 16-bit operands with
  // D % 8 == 0, whose launches without dW carry the next chunk's dlogits
  // recompute; with C % 8 == 0 small chunks' dH runs once per group too (see
  // group_dh). Shapes alone decide, so every subset of outputs accumulates dW
  // alike.
  // The working schedule: with a plan whose working chunk covers a whole
  // group of chunks (Cw > C; the buffers are sized for it whatever the
  // table's dtype), chunks of Cw tokens and no further grouping; otherwise
  // the caller's chunks, grouped by the plan's G. (logp, lse and dH do not
  // depend on the chunking; dW and db come in another order of additions,
  // and an operand-dtype table is rounded once per working chunk.)
  const bool work = bp.Cw > bp.C;
  const int64_t C = work ? bp.Cw : bp.C;
  const int64_t K = work ? ceil_div(N, C) : bp.K;
  const int64_t ldSt = work ? round_up(C, 8) : bp.ldSt;
  const bool small_dh = e == 2 && C % 8 == 0 && ceil_div(C, kTile) * ceil_div(D, kTile) < 128;
  const int64_t G = (want_dW && tab_fast && bp.G > 1 && !work) ? bp.G : 1;
  const bool grouping = G > 1;
  const int64_t ldq = grouping ? bp.ldP : ldSt;  // leading dimension of those buffers
  auto gj = [&](int64_t k) { return k % G; };       // position of chunk k in its group
  auto sidx = [&](int64_t k) { return (int)(k / G); };
  // the chunk whose launch carries the first dW contraction
  const int64_t fdw = (G < K ? G : K) - 1;

  float2* scales = reinterpret_cast<float2*>(at(workspace, bp.off_scales));
  const float* lse_use = lse;
  float* lse_fused = nullptr;  // where the fused path writes lse
  if (fused) {
    lse_fused = lse_out != nullptr ? lse_out : reinterpret_cast<float*>(at(workspace, bp.off_lse));
    lse_use = lse_fused;
  } else if (lse == nullptr) {
    float* lse_ws = reinterpret_cast<float*>(at(workspace, bp.off_lse));
    void* fws = at(workspace, bp.off_fwd);
    st = run_forward(N, D, V, dtype, h, W, b, targets, nullptr, lse_ws, fws, bp.fwd, s);
    if (st != LLP_OK) return st;
    lse_use = lse_ws;
  }
  // dH = dlogits W takes both operands as stored when the plan says so
  // (kmajor): K (vocabulary) rows with the tile's rows contiguous, dlogits^T
  // [V][ldq] and W [V][D] itself; then neither W^T nor the token-major
  // dlogits copy exists. 16-bit operands on the DMA pipeline only.
  const bool mn = bp.kmajor;
  void* Wt = (want_dH && !mn) ? at(workspace, bp.off_Wt) : nullptr;
  void* dS = (want_dH && !mn) ? at(workspace, bp.off_dS) : nullptr;
  void* dSt = bp.off_dSt >= 0 ? at(workspace, bp.off_dSt) : nullptr;
  float2* part = fused ? reinterpret_cast<float2*>(at(workspace, bp.off_part)) : nullptr;
  float* zt = fused ? reinterpret_cast<float*>(at(workspace, bp.off_zt)) : nullptr;
  void* ht = want_dW ? at(workspace, bp.off_ht) : nullptr;
  float* tcoef = reinterpret_cast<float*>(at(workspace, bp.off_tcoef));
  int32_t* head = (want_dW || want_db) ? reinterpret_cast<int32_t*>(at(workspace, bp.off_head)) : nullptr;
  int32_t* next = (want_dW || want_db) ? reinterpret_cast<int32_t*>(at(workspace, bp.off_next)) : nullptr;
  // Per-token mode of the single call (bf16 operands, decided by the plan from
  // the shapes alone, whether or not dH is asked for, so that every subset of
  // outputs computes alike): the forward stores 2^(z log2 e) for blocks in
  // range, the combine forms each token's factor -(g / s) 2^(-lse log2 e), and
  // the consumers apply it: the dH epilogue per row, the dW contraction through
  // the h transpose scaled per token, db per token. No softmax-gradient pass;
  // the preparation only rescales the columns of flagged tokens.
  const bool qtok = bp.qtok;
  int32_t* const qflag = qtok ? reinterpret_cast<int32_t*>(at(workspace, bp.off_qflag)) : nullptr;
  float* const cq = qtok ? reinterpret_cast<float*>(at(workspace, bp.off_cq)) : nullptr;
  LLP_LAUNCH(LLP_K_SMALL, launch_chunk_scales(g, N, G * C, ceil_div(K, G), dtype == LLP_F16 ? 15 : 0, scales,
                                              s));
  if (want_dH && !mn) LLP_LAUNCH(LLP_K_TRANSPOSE, launch_transpose(dtype, W, V, D, D, Wt, bp.ldWt, s));
  // With two numerator / dlogits^T buffers (and, single call, two partial
  // buffers), chunk k + 1's logits tiles run in the launch of chunk k's dH /
  // dW (its fast epilogue only): the single call's forward, the backward's
  // dlogits recompute. The launch tails overlap.
  const bool overlap = mn && aligned16(h) && bp.off_dSt2 >= 0 && (!want_dW || tab_fast);
  void* const dSt_buf[2] = {dSt, overlap ? at(workspace, bp.off_dSt2) : dSt};
  float2* const part_buf[2] = {part, (overlap && fused) ? reinterpret_cast<float2*>(at(workspace, bp.off_part2))
                                                        : part};
  // chunk k's numerator / dlogits^T columns: with grouping, column block
  // k % G of the buffer of group k / G (the groups alternate between the two
  // buffers with overlap); the h^T columns likewise, in the one h^T buffer
  auto qbuf = [&](int64_t k) -> void* {
    if (!grouping) return dSt_buf[k & 1];
    return static_cast<char*>(dSt_buf[(k / G) & 1]) + gj(k) * ldSt * e;
  };
  auto hbuf = [&](int64_t k) -> void* {
    return grouping ? static_cast<char*>(ht) + gj(k) * ldSt * e : ht;
  };
  if (qtok) LLP_LAUNCH(LLP_K_SMALL, launch_zero(qflag, N, 4, s));
  // With grouping and the K-row-major dH, a chunk whose dH grid is small
  // (fewer than 128 tiles: small chunks) takes dH once per group as well,
  // over all its chunks' columns (contiguous when C % 8 == 0): G times the
  // tiles for the same contraction over the vocabulary. Every dH element
  // still accumulates over V in the same order, so dH is bitwise the same
  // either way.
  const bool group_dh = grouping && mn && small_dh;
  // the forward tile problem and the combine of chunk kk (fused path)
  auto fwd_problem = [&](int64_t kk) {
    const int64_t c0 = kk * C;
    const int64_t Ck = (N - c0 < C) ? (N - c0) : C;
    GemmProblem p = logits_problem(c0, Ck, D, V, dtype, h, W);
    p.ep.bias = b;
    p.ep.targets = targets;
    p.ep.tok0 = c0;
    p.ep.v0 = v0;
    p.ep.Vt = Vt;
    p.epi = EPI_LSE_Q;
    p.ep.partials = part_buf[kk & 1];
    p.ep.ldp = C;
    p.ep.zt = zt;
    p.ep.dSt = qbuf(kk);
    p.ep.ldSt = ldq;
    p.ep.qtok = qtok ? 1 : 0;
    p.ep.qflag = qflag;
    return p;
  };
  // the dlogits recompute of chunk kk from its logits tile and the saved lse
  // (backward)
  auto dl_problem = [&](int64_t kk) {
    const int64_t c0 = kk * C;
    const int64_t Ck = (N - c0 < C) ? (N - c0) : C;
    GemmProblem p = logits_problem(c0, Ck, D, V, dtype, h, W);
    p.ep.bias = b;
    p.ep.targets = targets;
    p.ep.tok0 = c0;
    p.ep.v0 = v0;
    p.ep.Vt = Vt;
    p.epi = EPI_DLOGITS;
    p.ep.g = g;
    p.ep.lse = lse_use;
    p.ep.tcoef = tcoef;
    p.ep.dS = dS;
    p.ep.ldS = bp.ldS;
    p.ep.dSt = (want_dW || want_db || mn) ? qbuf(kk) : nullptr;
    p.ep.ldSt = ldq;
    p.ep.scales = scales;
    p.ep.chunk = sidx(kk);
    return p;
  };
  auto combine = [&](int64_t kk) {
    const int64_t c0 = kk * C;
    const int64_t Ck = (N - c0 < C) ? (N - c0) : C;
    return launch_lse_combine(part_buf[kk & 1], bp.P, C, zt + c0, targets + c0, V, Ck, logp_out + c0,
                              lse_fused + c0, g + c0, tcoef + c0, s, qtok ? qflag + c0 : nullptr,
                              scales + sidx(kk), qtok ? cq + c0 : nullptr);
  };
  // per-chunk target lists: walked by db and by an operand-dtype dW table's
  // epilogue (an FP32 table takes its one-hot rows in the chunk preparation)
  const bool lists = want_db || (want_dW && dW_dtype != LLP_F32);

  // A split dH contraction's reduction runs in the next chunk's preparation
  // launch when there is one (memory-bound work beside memory-bound work, one
  // launch fewer), else on its own before the partial buffer is reused.
  struct Pending {
    bool on = false;
    const float* part = nullptr;
    int64_t stride = 0, M = 0;
    int S = 1;
    EpiParams ep = {};
  } pend;
  auto flush = [&]() -> int {
    if (pend.on) {
      pend.on = false;
      LLP_LAUNCH(LLP_K_DH_REDUCE, launch_dh_reduce(dtype, pend.part, pend.stride, pend.S, pend.M, D, pend.ep, s));
    }
    return LLP_OK;
  };
  for (int64_t k = 0; k < K; ++k) {
    const int64_t c0 = k * C;
    const int64_t Ck = (N - c0 < C) ? (N - c0) : C;
    void* const dSt = qbuf(k);             // this chunk's numerator / dlogits^T columns
    float2* const part = part_buf[k & 1];  // and its forward partials
    // the chunk's logits tile (with overlap, chunks after the first were
    // launched with the previous chunk's dH / dW)
    if (!overlap || k == 0) {
      if (fused) {  // lse partials, target logits, softmax numerators
        const GemmProblem pf = fwd_problem(k);
        LLP_LAUNCH(LLP_K_FWD_LSE, launch_gemm(dtype, &pf, nullptr, s));
        LLP_LAUNCH(LLP_K_COMBINE, combine(k));
      } else {  // dlogits, recomputed from the logits and the saved lse
        const GemmProblem pd = dl_problem(k);
        LLP_LAUNCH(LLP_K_DLOGITS, launch_gemm(dtype, &pd, nullptr, s));
      }
    }
    // one launch: target lists, the chunk's h transposed, and (fused) the softmax gradient
    ChunkPrep cp = {};
    cp.C = Ck;
    cp.V = V;
    if (want_dW || want_db) {
      cp.targets = targets;
      cp.g = g;
      cp.tok0 = c0;
      cp.v0 = v0;
      cp.Vt = Vt;
      if (lists) {
        cp.head = head;
        cp.next = next;
      }
    }
    if (want_dW) {
      cp.h = static_cast<const char*>(h) + c0 * D * e;
      cp.D = D;
      cp.ht = hbuf(k);
      cp.ldht = ldq;
      if (dW_dtype == LLP_F32 && !(store_first && k <= fdw)) {  // the one-hot rows go into the table here
        cp.tcoef = tcoef;
        cp.table = static_cast<float*>(dW);
        cp.ldt = D;
        // after the contraction that stored the table, the next chunk adds the
        // rows of every chunk so far, in token order
        cp.oh_tok0 = (store_first && k == fdw + 1) ? 0 : c0;
        cp.oh_C = c0 + Ck - cp.oh_tok0;
        cp.oh_h = static_cast<const char*>(h) + cp.oh_tok0 * D * e;
      }
    }
    if (fused) {
      cp.qt = dSt;
      cp.ldq = ldq;
      cp.partials = part;
      cp.ldp = C;
      cp.lse = lse_fused + c0;
      cp.gc = g + c0;
      cp.tc = targets + c0;
      cp.scales = scales;
      cp.chunk = sidx(k);
      cp.dS = dS;
      cp.ldS = bp.ldS;
      if (qtok) {
        cp.cq = cq + c0;  // scales the chunk's h rows in the transpose
        cp.qflag = qflag + c0;
      }
    }
    if (cp.head != nullptr || cp.ht != nullptr || cp.qt != nullptr || cp.table != nullptr) {
      if (pend.on) {  // the previous dH's reduction rides in this launch
        cp.rd_part = pend.part;
        cp.rd_stride = pend.stride;
        cp.rd_S = pend.S;
        cp.rd_M = pend.M;
        cp.rd_D = D;
        cp.rd_ep = pend.ep;
        pend.on = false;
      }
      LLP_LAUNCH(fused ? LLP_K_DLOGITS : LLP_K_TRANSPOSE, launch_chunk_prep(dtype, cp, s));
    }
    if (want_db)
      LLP_LAUNCH(LLP_K_SMALL, launch_db_accum(dtype, dSt, ldq, V, Ck, scales, sidx(k), head, next, targets, g, tcoef,
                              c0, v0, Vt, db, dW_dtype, s, qtok ? cq + c0 : nullptr));
    GemmProblem ph = {}, pw = {};
    // the group of chunk k: first chunk kg, k is its last chunk (so far)
    const int64_t kg = k - gj(k);
    const bool group_end = gj(k) == G - 1 || k == K - 1;
    // this launch's dH: chunk k, or with group_dh the whole group at its last
    // chunk (none at the group's other chunks)
    const bool do_dh = want_dH && (!group_dh || group_end);
    const int64_t h0 = group_dh ? kg * C : c0;           // first token of this dH
    const int64_t hM = group_dh ? (k - kg) * C + Ck : Ck;  // its tokens
    if (do_dh && mn) {
      ph.A = group_dh ? qbuf(kg) : dSt;
      ph.B = W;
      ph.lda = ldq;
      ph.ldb = D;
      ph.M = hM;
      ph.N = D;
      ph.K = V;
      ph.a_vec = ph.b_vec = 1;
      ph.mn = 1;
      ph.dma = 1;
    } else if (do_dh) {
      ph.A = dS;
      ph.B = Wt;
      ph.lda = bp.ldS;
      ph.ldb = bp.ldWt;
      ph.M = Ck;
      ph.N = D;
      ph.K = V;
      ph.a_vec = ph.b_vec = 1;
      ph.dma = dma_ok(ph, e, true);  // dS and W^T padding columns are written +0
    }
    if (do_dh) {
      ph.tiles_m = (int)ceil_div(hM, kTile);
      ph.tiles_n = (int)ceil_div(D, kTile);
      ph.epi = EPI_STORE;
      ph.ep.out = static_cast<char*>(dH) + h0 * D * (dH_dtype == LLP_F32 ? 4 : e);
      ph.ep.ldo = D;
      ph.ep.out_dt = dH_dtype;
      ph.ep.targets = targets;
      ph.ep.g = g;
      ph.ep.tok0 = h0;
      ph.ep.V = V;
      ph.ep.v0 = v0;
      ph.ep.Vt = Vt;
      ph.ep.tcoef = tcoef;
      ph.ep.W = W;
      ph.ep.ldW = D;
      ph.ep.scales = scales;
      ph.ep.chunk = sidx(k);
      ph.ep.rowf = cq;  // per-token mode: indexed tok0 + row
      if (bp.dh_parts > 1) {
        // the vocabulary in fixed parts: one tile per part, fp32 partials,
        // then the reduction below applies this epilogue to their sum
        ph.kparts = (int)bp.dh_parts;
        ph.kpart = bp.dh_part;
        ph.ep.dhp = reinterpret_cast<float*>(at(workspace, bp.off_dhp));
        ph.ep.dhp_stride = bp.dh_rows * D;
      }
    }
    // with grouping, the dW contraction of a group runs in the launch of its
    // last chunk, over K = (k - kg) ldSt + Ck columns (the earlier chunks'
    // padding columns are +0 in both operands)
    const bool do_dw = want_dW && group_end;
    if (do_dw) {
      pw.A = qbuf(kg);
      pw.B = hbuf(kg);
      pw.lda = ldq;
      pw.ldb = ldq;
      pw.M = V;
      pw.N = D;
      pw.K = (k - kg) * ldSt + Ck;
      pw.a_vec = pw.b_vec = 1;
      pw.dma = dma_ok(pw, e, true);  // dlogits^T and h^T padding columns are written +0
      pw.tiles_m = (int)ceil_div(V, kTile);
      pw.tiles_n = (int)ceil_div(D, kTile);
      pw.epi = EPI_ACCUM;
      pw.ep.out = dW;
      pw.ep.ldo = D;
      pw.ep.out_dt = dW_dtype;
      pw.ep.targets = targets;
      pw.ep.g = g;
      pw.ep.tok0 = kg * C;
      pw.ep.V = V;
      pw.ep.v0 = v0;
      pw.ep.Vt = Vt;
      pw.ep.tcoef = tcoef;
      pw.ep.h = h;
      pw.ep.ldh = D;
      pw.ep.head = dW_dtype == LLP_F32 ? nullptr : head;  // null: one-hot rows already added
      pw.ep.next = next;
      pw.ep.tab_fast = dW_dtype == LLP_F32 && D % 4 == 0 && aligned16(dW) && kTile * D * 4 < 0x7FFFFFF0LL;
      // an operand-dtype table in 16-byte pieces (the list heads and next links are built for it)
      pw.ep.tab_fast16 = dW_dtype == dtype && e == 2 && D % 8 == 0 && aligned16(dW) && aligned16(h) &&
                         kTile * D * 2 < 0x7FFFFFF0LL;
      pw.ep.tab_store = (store_first && k == fdw) ? 1 : 0;
      pw.ep.ntok = Ck;
      pw.ep.scales = scales;
      pw.ep.chunk = sidx(k);
    }
    // the partial buffer is about to be rewritten: its previous sums must be reduced
    if (do_dh && ph.kparts > 1) {
      st = flush();
      if (st != LLP_OK) return st;
    }
    if (overlap && k + 1 < K) {
      // with the next chunk's logits tiles (single call: then that chunk's combine)
      const GemmProblem pn = fused ? fwd_problem(k + 1) : dl_problem(k + 1);
      if (do_dh)
        LLP_LAUNCH(fused ? LLP_K_DH_DW_FWD : LLP_K_DH_DW_DL, launch_gemm3(dtype, ph, do_dw ? &pw : nullptr, pn, s));
      else  // group_dh before the group's last chunk: no dH and (grouping) no dW in this launch
        LLP_LAUNCH(fused ? LLP_K_FWD_LSE : LLP_K_DLOGITS, launch_gemm(dtype, &pn, nullptr, s));
      if (fused) LLP_LAUNCH(LLP_K_COMBINE, combine(k + 1));
    } else if (do_dh || do_dw) {
      LLP_LAUNCH(LLP_K_DH_DW, launch_gemm(dtype, do_dh ? &ph : nullptr, do_dw ? &pw : nullptr, s));
    }
    if (do_dh && ph.kparts > 1) {
      pend.on = true;
      pend.part = ph.ep.dhp;
      pend.stride = ph.ep.dhp_stride;
      pend.S = ph.kparts;
      pend.M = hM;
      pend.ep = ph.ep;
    }
  }
  st = flush();
  if (st != LLP_OK) return st;
  if (store_first && K == fdw + 1 && dW_dtype == LLP_F32) {
    // the contraction that stored the table was the last one: the one-hot
    // rows of every chunk follow it
    ChunkPrep cp = {};
    cp.V = V;
    cp.D = D;
    cp.targets = targets;
    cp.g = g;
    cp.v0 = v0;
    cp.Vt = Vt;
    cp.tcoef = tcoef;
    cp.table = static_cast<float*>(dW);
    cp.ldt = D;
    cp.oh_tok0 = 0;
    cp.oh_C = N;
    cp.oh_h = h;
    LLP_LAUNCH(LLP_K_TRANSPOSE, launch_chunk_prep(dtype, cp, s));
  }
  return LLP_OK;
}

}  // namespace
}  // namespace llp

extern "C" {

int linear_logp_bwd(int64_t N, int64_t D, int64_t V, int dtype, int64_t chunk, const void* h,
                    const void* W, const void* b, const int64_t* targets, const float* g,
                    const float* lse, void* dH, void* dW, int dW_dtype, void* db, int accumulate,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(N, D, V, dtype, chunk, h, W, b, targets, g, lse, nullptr, nullptr, dH, dW, dW_dtype, db,
                       accumulate, workspace, workspace_bytes, stream, false);
}

int linear_logp_fwd_bwd_workspace_size(int64_t N, int64_t D, int64_t V, int dtype, int64_t chunk,
                                       int want_dH, int want_dW, int want_db, int have_lse,
                                       size_t* bytes) {
  if (bytes == nullptr) return LLP_EINVAL;
  if (!(want_dH || want_dW || want_db)) return linear_logp_fwd_workspace_size(N, D, V, dtype, bytes);
  BwdPlan bp;
  const int st = plan_bwd(N, D, V, dtype, chunk, want_dH, want_dW, want_db, have_lse, &bp, 1);
  if (st != LLP_OK) return st;
  *bytes = (size_t)bp.bytes;
  return LLP_OK;
}

int linear_logp_fwd_bwd(int64_t N, int64_t D, int64_t V, int dtype, int64_t chunk, const void* h,
                        const void* W, const void* b, const int64_t* targets, const float* g,
                        float* logp, float* lse, void* dH, void* dW, int dW_dtype, void* db,
                        int accumulate, void* workspace, size_t workspace_bytes, void* stream) {
  if (dH == nullptr && dW == nullptr && db == nullptr) {
    // nothing to differentiate: the forward alone
    const int st = linear_logp_fwd(N, D, V, dtype, h, W, b, targets, logp, lse, workspace, workspace_bytes, stream);
    if (st != LLP_OK) return st;
    return (accumulate == 0 || accumulate == 1) ? LLP_OK : LLP_EINVAL;
  }
  return backward_impl(N, D, V, dtype, chunk, h, W, b, targets, g, nullptr, logp, lse, dH, dW, dW_dtype, db,
                       accumulate, workspace, workspace_bytes, stream, true);
}

int linear_logp_shard_fwd(int64_t N, int64_t D, int64_t Vs, int64_t v0, int64_t Vt, int dtype, const void* h,
                          const void* W, const void* b, const int64_t* targets, float* lse_shard, float* zt_shard,
                          void* workspace, size_t workspace_bytes, void* stream) {
  FwdPlan fp;
  int st = plan_fwd(N, D, Vs, dtype, &fp);
  if (st != LLP_OK) return st;
  if (v0 < 0 || Vt < 1 || v0 > Vt - Vs) return LLP_EINVAL;
  if (N == 0) return LLP_OK;
  if (h == nullptr || W == nullptr || targets == nullptr || lse_shard == nullptr || zt_shard == nullptr)
    return LLP_EINVAL;
  if ((reinterpret_cast<uintptr_t>(zt_shard) & 3) != 0) return LLP_EINVAL;
  if ((size_t)fp.bytes > workspace_bytes || (fp.bytes > 0 && workspace == nullptr)) return LLP_EWORKSPACE;
  LLP_CHECK_DEVICE(h, W, b, targets, lse_shard, zt_shard, workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float2* partials = reinterpret_cast<float2*>(at(workspace, fp.off_partials));
  // -inf marks "target not in this share"; the tile holding the target overwrites it
  LLP_LAUNCH(LLP_K_SMALL, launch_fill32(reinterpret_cast<uint32_t*>(zt_shard), N, 0xFF800000u, s));
  GemmProblem p = logits_problem(0, N, D, Vs, dtype, h, W);
  p.epi = EPI_LSE_PARTIAL;
  p.ep.bias = b;
  p.ep.targets = targets;
  p.ep.tok0 = 0;
  p.ep.v0 = v0;
  p.ep.Vt = Vt;
  p.ep.partials = partials;
  p.ep.ldp = N;
  p.ep.zt = zt_shard;
  LLP_LAUNCH(LLP_K_FWD_LSE, launch_gemm(dtype, &p, nullptr, s));
  LLP_LAUNCH(LLP_K_COMBINE,
             launch_lse_combine(partials, fp.P, N, zt_shard, targets, Vs, N, nullptr, lse_shard, nullptr, nullptr, s));
  return LLP_OK;
}

int linear_logp_shard_combine(int64_t N, int64_t P, const float* lse_shards, const float* zt_shards,
                              const int64_t* targets, int64_t Vt, float* logp, float* lse, void* stream) {
  if (N < 0 || P < 1 || Vt < 1) return LLP_EINVAL;
  if (N > (INT64_MAX / 4) / P) return LLP_EOVERFLOW;
  if (N == 0) return LLP_OK;
  if (lse_shards == nullptr || zt_shards == nullptr || targets == nullptr || (logp == nullptr && lse == nullptr))
    return LLP_EINVAL;
  LLP_CHECK_DEVICE(lse_shards, zt_shards, targets, logp, lse);
  hipStream_t s = static_cast<hipStream_t>(stream);
  LLP_LAUNCH(LLP_K_COMBINE, launch_shard_combine(lse_shards, zt_shards, P, N, targets, Vt, logp, lse, s));
  return LLP_OK;
}

int linear_logp_shard_bwd(int64_t N, int64_t D, int64_t Vs, int64_t v0, int64_t Vt, int dtype, int64_t chunk,
                          const void* h, const void* W, const void* b, const int64_t* targets, const float* g,
                          const float* lse, void* dH, int dH_dtype, void* dW, int dW_dtype, void* db,
                          int accumulate, void* workspace, size_t workspace_bytes, void* stream) {
  if (v0 < 0 || Vs < 1 || Vt < 1 || v0 > Vt - Vs) return LLP_EINVAL;
  if (N > 0 && lse == nullptr && (dH != nullptr || dW != nullptr || db != nullptr)) return LLP_EINVAL;
  return backward_impl(N, D, Vs, dtype, chunk, h, W, b, targets, g, lse, nullptr, nullptr, dH, dW, dW_dtype, db,
                       accumulate, workspace, workspace_bytes, stream, false, v0, Vt,
                       dH != nullptr ? dH_dtype : dtype);
}

int logp_fwd(int64_t N, int64_t V, int dtype, const void* logits, const int64_t* targets, float* logp,
             float* lse, void* stream) {
  const int st = check_rows(N, V, dtype);
  if (st != LLP_OK) return st;
  if (N == 0) return LLP_OK;
  if (logits == nullptr || targets == nullptr || logp == nullptr) return LLP_EINVAL;
  LLP_CHECK_DEVICE(logits, targets, logp, lse);
  hipStream_t s = static_cast<hipStream_t>(stream);
  LLP_LAUNCH(LLP_K_ROWS_FWD, launch_rows_fwd(dtype, logits, N, V, targets, logp, lse, s));
  return LLP_OK;
}

int logp_bwd(int64_t N, int64_t V, int dtype, const void* logits, const int64_t* targets, const float* g,
             const float* lse, void* dlogits, void* stream) {
  const int st = check_rows(N, V, dtype);
  if (st != LLP_OK) return st;
  if (N == 0) return LLP_OK;
  if (logits == nullptr || targets == nullptr || g == nullptr || dlogits == nullptr) return LLP_EINVAL;
  LLP_CHECK_DEVICE(logits, targets, g, lse, dlogits);
  hipStream_t s = static_cast<hipStream_t>(stream);
  LLP_LAUNCH(LLP_K_ROWS_BWD, launch_rows_bwd(dtype, logits, N, V, targets, g, lse, dlogits, s));
  return LLP_OK;
}

int llp_trace_enable(int on) {
  Trace& t = g_trace;
  if (on) {
    t.recs.clear();
    t.used = 0;
    t.dropped = 0;
  }
  t.on = on != 0;
  return LLP_OK;
}

int llp_trace_read(double* ms, int64_t* count, int n) {
  if (n < 0) return LLP_EINVAL;
  for (int k = 0; k < n; ++k) {
    if (ms) ms[k] = 0.0;
    if (count) count[k] = 0;
  }
  for (const TraceRec& r : g_trace.recs) {
    if (hipEventSynchronize(r.stop) != hipSuccess) return LLP_EHIP;
    float e = 0.0f;
    if (hipEventElapsedTime(&e, r.start, r.stop) != hipSuccess) return LLP_EHIP;
    if (r.kind >= 0 && r.kind < n) {
      if (ms) ms[r.kind] += e;
      if (count) count[r.kind] += 1;
    }
  }
  return g_trace.dropped ? LLP_EOVERFLOW : LLP_OK;
}

}  // extern "C"
