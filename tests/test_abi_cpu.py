"""The C ABI on a machine without a GPU: the library loads, exports every
symbol include/llp.h declares, and every argument check returns its status
before any HIP call (nothing here launches a kernel)."""

import ctypes
import json
import os
import re

import pytest

from cross_entropy_lm_amd import llp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "page_figures.json")))

F32, BF16, F16 = llp.LLP_F32, llp.LLP_BF16, llp.LLP_F16
FAKE = 0x10000  # a non-null pointer value that is never dereferenced: every call below fails validation first


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "llp.h")).read()
    return re.findall(r"LLP_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_library_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) == 18
    L = llp.lib()
    for n in names:
        assert hasattr(L, n), n
        assert n in llp.SIGNATURES, n
    assert llp.llp_version() == 100
    assert llp.llp_strerror(llp.LLP_EWORKSPACE) == "workspace too small"
    assert llp.llp_strerror(99) == "unknown status"


def test_default_chunk_policy_matches_the_pages():
    tm = GOLD["traffic_model"]
    assert llp.linear_logp_chunk_rows(tm["N"], tm["V"], 0) == tm["chunk_rows"]
    assert llp.linear_logp_num_chunks(tm["N"], tm["V"], 0) == tm["chunks"]
    # floor(2^24 / 151936) = 110 rows, the 2^24-element row of RL-Kernel PR #495's sweep
    sweep = GOLD["chunk_sweep_rows"]
    assert llp.linear_logp_chunk_rows(32768, sweep["V"], 0) == sweep["elems_to_rows"][str(1 << 24)]
    assert llp.linear_logp_chunk_rows(100, 1 << 25, 0) == 1  # V > 2^24 -> one row per chunk
    assert llp.linear_logp_chunk_rows(10, 1024, 0) == 10  # clamped to N
    assert llp.linear_logp_chunk_rows(0, 1024, 0) == 1
    assert llp.linear_logp_num_chunks(0, 1024, 0) == 0
    assert llp.linear_logp_num_chunks(256, 1024, 64) == 4
    assert llp.linear_logp_num_chunks(8192, 151936, 0) == 75
    assert llp.linear_logp_chunk_rows(-1, 10, 0) == -1
    assert llp.linear_logp_chunk_rows(5, 0, 0) == -1


def test_workspace_queries():
    f = llp.linear_logp_fwd_workspace_size
    assert f(0, 128, 1024, F32) == 0
    assert f(256, 128, 1024, F32) >= 2 * 4 * 256 * 8 + 256 * 4
    b = llp.linear_logp_bwd_workspace_size
    assert b(256, 128, 1024, F32, 64, False, False, False, True) == 0
    full = b(16384, 4096, 32000, BF16, 2048, True, True, False, True)
    only_dh = b(16384, 4096, 32000, BF16, 2048, True, False, False, True)
    only_dw = b(16384, 4096, 32000, BF16, 2048, False, True, False, True)
    no_lse = b(16384, 4096, 32000, BF16, 2048, True, True, False, False)
    assert only_dh < full and only_dw <= full and no_lse > full
    # 16-bit operands with D % 8 == 0: dH reads dlogits^T and W as stored (no
    # W^T, no token-major dlogits); dW pairs chunks, and the next chunk's
    # dlogits recompute runs beside a chunk's dH / dW, so the workspace is two
    # pair buffers of dlogits^T [V][2 x 2048] plus h^T of a pair; with more
    # than one vocabulary part of 32768 rows, the parts' fp32 sums too
    parts = lambda V: -(-V // 32768)  # noqa: E731
    dhp = lambda V, rows, D: parts(V) * rows * D * 4 if parts(V) > 1 else 0  # noqa: E731
    expect = 2 * 32000 * 4096 * 2 + 4096 * 4096 * 2 + dhp(32000, 2048, 4096)
    assert expect <= full < expect + (1 << 20)
    # dW alone: no dH, so no second buffer (nothing overlaps); still pairs
    expect_dw = 32000 * 4096 * 2 + 4096 * 4096 * 2
    assert expect_dw <= only_dw < expect_dw + (1 << 20)
    # small chunks (fewer than 128 dH tiles) group dW: at 512-token chunks,
    # V = 32768, D = 2048, groups of 8 chunks (4096 columns), which run as one
    # 4096-token working chunk: dlogits^T and h^T of the working chunk
    small = b(4096, 2048, 32768, BF16, 512, True, True, False, True)
    expect_small = 4096 * 32768 * 2 + 2048 * 4096 * 2 + dhp(32768, 4096, 2048)
    assert expect_small <= small < expect_small + (1 << 20)
    # dH alone: the vocab-major dlogits of one chunk, twice (no pairs without dW)
    expect_dh = 2 * 2048 * 32000 * 2 + dhp(32000, 2048, 4096)
    assert expect_dh <= only_dh < expect_dh + (1 << 20)
    # the schedule depends on the shapes only, so a dH-only call holds the
    # 4096-token working chunk (8 small chunks) that a call with dW runs
    one = b(4096, 1024, 8192, BF16, 512, True, False, False, True)
    assert 4096 * 8192 * 2 <= one < 4096 * 8192 * 2 + (1 << 20)
    # 151936 rows: 5 parts of dH sums
    bigdh = b(2048, 1024, 151936, BF16, 2048, True, False, False, True)
    expect_bigdh = 2048 * 151936 * 2 + 5 * 2048 * 1024 * 4
    assert expect_bigdh <= bigdh < expect_bigdh + (1 << 20)
    # fp32 operands (and D % 8 != 0) keep the transposed path: W^T, both
    # dlogits layouts and h^T
    f32 = b(4096, 1024, 8192, F32, 512, True, True, False, True)
    expect_f32 = 1024 * 8192 * 4 + 512 * 8192 * 4 * 2 + 1024 * 512 * 4
    assert expect_f32 <= f32 < expect_f32 + (1 << 20)
    odd = b(4096, 1020, 8192, BF16, 512, True, False, False, True)
    expect_odd = 1020 * 8192 * 2 + 512 * 8192 * 2
    assert expect_odd <= odd < expect_odd + (1 << 20)
    # the single call at 16384 x 4096 x 32000, bf16, chunk 2048, FP32 table:
    # each pair of chunks runs as one 4096-token working chunk, so two pair
    # buffers of numerators [V][2 x 2048], h^T of a pair, two working chunks'
    # forward partials and per-token arrays (about 548 MiB)
    fq = llp.linear_logp_fwd_bwd_workspace_size
    single = fq(16384, 4096, 32000, BF16, 2048, True, True, False, True)
    expect_single = 2 * 32000 * 4096 * 2 + 4096 * 4096 * 2 + 2 * 250 * 4096 * 8
    assert expect_single <= single < expect_single + (1 << 20)
    # 110-token chunks at V = 151936: a 1 GiB group buffer holds 31 x 112
    # columns, so the 75 chunks need three groups, balanced to 25 chunks each,
    # which run as 2750-token working chunks: two group buffers, h^T of a
    # group, two working chunks' forward partials, 5 dH parts of a working
    # chunk
    big = fq(8192, 4096, 151936, BF16, 0, True, True, True, True)
    expect_big = (2 * 151936 * 25 * 112 * 2 + 4096 * 25 * 112 * 2 + 2 * 1188 * 2750 * 8 + 5 * 2750 * 4096 * 4 +
                  151936 * 4)
    assert expect_big <= big < expect_big + (1 << 20)


def test_bench_group_rule_matches_the_library():
    """The benchmark's copy of the dW group rule (for its per-launch flop
    accounting) agrees with the library's plan, seen through the workspace
    sizes of shapes that differ only in it."""
    import sys
    sys.path.insert(0, ROOT)
    import bench

    fq = llp.linear_logp_fwd_bwd_workspace_size
    bq = llp.linear_logp_bwd_workspace_size
    for N, D, V, C in ((8192, 4096, 151936, 110), (4096, 2048, 32768, 512), (16384, 4096, 32000, 2048),
                       (3000, 512, 50000, 64), (2000, 1024, 4096, 100), (700, 256, 1031, 300),
                       (4096, 1020, 8192, 2048), (1000, 512, 2000, 1000)):
        K = -(-N // C)
        ld = -(-C // 8) * 8
        P = 2 * (-(-V // 256))
        for fused, q in ((True, fq), (False, bq)):
            G = bench.dw_group(N, D, V, C, K, 2, fused)
            with_dw = q(N, D, V, BF16, C, False, True, False, True)
            # dW alone: the group buffer [V][G ld] and h^T [D][G ld], (single
            # call) the forward's partials of one working chunk (a whole group
            # when G >= 2 on the layout without W^T), and per-token arrays
            Cw = min(G * C, N) if G >= 2 and D % 8 == 0 else C
            core = V * G * ld * 2 + D * G * ld * 2 + (P * Cw * 8 if fused else 0)
            assert core <= with_dw < core + (1 << 20) + 4 * V + 16 * N + 4 * Cw, (N, D, V, C, G, fused)


@pytest.mark.parametrize("args,status", [
    ((-1, 128, 1024, F32), llp.LLP_EINVAL),
    ((4, 0, 1024, F32), llp.LLP_EINVAL),
    ((4, 128, 0, F32), llp.LLP_EINVAL),
    ((4, 128, 1024, 7), llp.LLP_EINVAL),
    ((1 << 31, 128, 1024, F32), llp.LLP_EOVERFLOW),
    ((4, 1 << 23, 1024, F32), llp.LLP_EOVERFLOW),
    ((1 << 30, 1 << 22, 1 << 30, BF16), llp.LLP_EOVERFLOW),
])
def test_fwd_shape_errors(args, status):
    out = ctypes.c_size_t(0)
    assert llp.lib().linear_logp_fwd_workspace_size(*args, ctypes.byref(out)) == status
    N, D, V, dt = args
    st = llp.lib().linear_logp_fwd(N, D, V, dt, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == status


def test_fwd_pointer_and_workspace_errors():
    L = llp.lib()
    N, D, V = 256, 128, 1024
    need = llp.linear_logp_fwd_workspace_size(N, D, V, F32)
    for null in range(4):  # h, W, targets, logp are required
        p = [FAKE] * 4
        p[null] = None
        st = L.linear_logp_fwd(N, D, V, F32, p[0], p[1], None, p[2], p[3], None, FAKE, need, None)
        assert st == llp.LLP_EINVAL
    assert L.linear_logp_fwd(N, D, V, F32, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, need - 1, None) \
        == llp.LLP_EWORKSPACE
    assert L.linear_logp_fwd(N, D, V, F32, FAKE, FAKE, None, FAKE, FAKE, None, None, need, None) \
        == llp.LLP_EWORKSPACE
    # N = 0 is a no-op that touches nothing, even with null pointers
    assert L.linear_logp_fwd(0, D, V, F32, None, None, None, None, None, None, None, 0, None) == llp.LLP_OK


def test_noalloc_forward_argument_errors():
    """The forward on the library's scratch checks its arguments and the
    scratch's size before any HIP call."""
    L = llp.lib()
    f = L.linear_logp_fwd_noalloc
    assert f(-1, 128, 1024, F32, FAKE, FAKE, None, FAKE, FAKE, None, None) == llp.LLP_EINVAL
    assert f(4, 128, 1024, 7, FAKE, FAKE, None, FAKE, FAKE, None, None) == llp.LLP_EINVAL
    for null in range(4):  # h, W, targets, logp are required
        p = [FAKE] * 4
        p[null] = None
        assert f(256, 128, 1024, F32, p[0], p[1], None, p[2], p[3], None, None) == llp.LLP_EINVAL
    # 33487 tokens at V = 32000 fit in the 64 MiB scratch, 33488 do not
    assert llp.linear_logp_fwd_workspace_size(33487, 4096, 32000, BF16) <= llp.LLP_SCRATCH_BYTES
    assert llp.linear_logp_fwd_workspace_size(33488, 4096, 32000, BF16) > llp.LLP_SCRATCH_BYTES
    assert f(33488, 4096, 32000, BF16, FAKE, FAKE, None, FAKE, FAKE, None, None) == llp.LLP_EWORKSPACE
    assert f(7059, 4096, 151936, BF16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == llp.LLP_EWORKSPACE
    assert f(0, 128, 1024, F32, None, None, None, None, None, None, None) == llp.LLP_OK
    assert f(1 << 31, 128, 1024, F32, FAKE, FAKE, None, FAKE, FAKE, None, None) == llp.LLP_EOVERFLOW


def _bwd(N=256, D=128, V=1024, dt=F32, chunk=64, h=FAKE, W=FAKE, b=FAKE, t=FAKE, g=FAKE, lse=FAKE,
         dH=FAKE, dW=FAKE, tdt=F32, db=FAKE, acc=0, ws=FAKE, nbytes=1 << 40):
    return llp.lib().linear_logp_bwd(N, D, V, dt, chunk, h, W, b, t, g, lse, dH, dW, tdt, db, acc, ws,
                                     nbytes, None)


def test_bwd_argument_errors():
    E = llp.LLP_EINVAL
    assert _bwd(N=-1) == E
    assert _bwd(D=0) == E
    assert _bwd(V=0) == E
    assert _bwd(dt=3) == E
    assert _bwd(acc=2) == E
    assert _bwd(tdt=F16) == E          # table dtype must be fp32 or the operand dtype
    assert _bwd(dt=BF16, tdt=F16) == E
    assert _bwd(b=None) == E           # db requested without a bias
    assert _bwd(h=None) == E
    assert _bwd(W=None) == E
    assert _bwd(t=None) == E
    assert _bwd(g=None) == E
    need = llp.linear_logp_bwd_workspace_size(256, 128, 1024, F32, 64, True, True, True, True)
    assert _bwd(nbytes=need - 1) == llp.LLP_EWORKSPACE
    assert _bwd(ws=None, nbytes=need) == llp.LLP_EWORKSPACE
    assert _bwd(N=1 << 31) == llp.LLP_EOVERFLOW
    # 16-bit operands with D % 8 == 0 read W and the workspace with 16-byte
    # accesses: a misaligned pointer is rejected before any launch
    assert _bwd(dt=BF16, W=FAKE + 2) == E
    assert _bwd(dt=F16, ws=FAKE + 8) == E
    assert _bwd(dt=BF16, W=FAKE + 2, dH=None, dW=None, db=None) == llp.LLP_OK  # nothing requested


def _fused(N=256, D=128, V=1024, dt=F32, chunk=64, h=FAKE, W=FAKE, b=FAKE, t=FAKE, g=FAKE, logp=FAKE,
           lse=FAKE, dH=FAKE, dW=FAKE, tdt=F32, db=FAKE, acc=0, ws=FAKE, nbytes=1 << 40):
    return llp.lib().linear_logp_fwd_bwd(N, D, V, dt, chunk, h, W, b, t, g, logp, lse, dH, dW, tdt, db, acc,
                                         ws, nbytes, None)


def test_fused_argument_errors_and_workspace():
    E = llp.LLP_EINVAL
    assert _fused(N=-1) == E
    assert _fused(D=0) == E
    assert _fused(dt=3) == E
    assert _fused(acc=2) == E
    assert _fused(tdt=F16) == E
    assert _fused(b=None) == E         # db requested without a bias
    assert _fused(h=None) == E
    assert _fused(g=None) == E
    assert _fused(logp=None) == E      # logp is required, as in linear_logp_fwd
    fq = llp.linear_logp_fwd_bwd_workspace_size
    need = fq(256, 128, 1024, F32, 64, True, True, True, True)
    assert _fused(nbytes=need - 1) == llp.LLP_EWORKSPACE
    assert _fused(ws=None, nbytes=need) == llp.LLP_EWORKSPACE
    assert _fused(N=1 << 31) == llp.LLP_EOVERFLOW
    assert _fused(dt=BF16, W=FAKE + 2) == E
    assert _fused(dt=BF16, W=FAKE + 2, dH=None) == E   # bf16 per-token numerators read W as stored too
    assert _fused(dt=F16, ws=FAKE + 4) == E
    # the fused layout adds the chunk's forward partials and target logits, and
    # always holds the vocab-major buffer; without lse it also holds one
    bq = llp.linear_logp_bwd_workspace_size
    assert need > bq(256, 128, 1024, F32, 64, True, True, True, True)
    assert fq(256, 128, 1024, F32, 64, True, True, True, False) >= need + 256 * 4
    # no gradient requested: the forward's workspace
    assert fq(256, 128, 1024, F32, 64, False, False, False, True) == llp.linear_logp_fwd_workspace_size(
        256, 128, 1024, F32)
    # N = 0 with accumulate: nothing to do, null pointers allowed
    assert llp.lib().linear_logp_fwd_bwd(0, 128, 1024, F32, 0, None, None, None, None, None, None, None, None,
                                         None, F32, None, 1, None, 0, None) == llp.LLP_OK
    # the single call keeps a row of its numerator buffer below 2^24 bytes (its
    # stores use 32-bit offsets inside 128-row blocks): a 2^23-token chunk in
    # bf16 (2^24 bytes per row) is refused, the two-call path takes it
    out = ctypes.c_size_t(0)
    assert llp.lib().linear_logp_fwd_bwd_workspace_size(1 << 23, 8, 2, BF16, 1 << 23, 1, 0, 0, 1,
                                                        ctypes.byref(out)) == llp.LLP_EOVERFLOW
    assert llp.lib().linear_logp_fwd_bwd_workspace_size((1 << 23) - 8, 8, 2, BF16, (1 << 23) - 8, 1, 0, 0, 1,
                                                        ctypes.byref(out)) == llp.LLP_OK
    assert llp.lib().linear_logp_bwd_workspace_size(1 << 23, 8, 2, BF16, 1 << 23, 1, 0, 0, 1,
                                                    ctypes.byref(out)) == llp.LLP_OK
    # the two-call backward's dlogits^T rows stay below 2^28 bytes (32-bit
    # offsets inside 8-row groups): 2^27 bf16 columns are refused
    assert llp.lib().linear_logp_bwd_workspace_size(1 << 27, 8, 1, BF16, 1 << 27, 1, 0, 0, 1,
                                                    ctypes.byref(out)) == llp.LLP_EOVERFLOW
    assert llp.lib().linear_logp_bwd_workspace_size((1 << 27) - 8, 8, 1, BF16, (1 << 27) - 8, 1, 0, 0, 1,
                                                    ctypes.byref(out)) == llp.LLP_OK


def _sfwd(N=256, D=128, Vs=400, v0=400, Vt=1031, dt=F32, h=FAKE, W=FAKE, b=FAKE, t=FAKE, lse=FAKE, zt=FAKE,
          ws=FAKE, nbytes=1 << 40):
    return llp.lib().linear_logp_shard_fwd(N, D, Vs, v0, Vt, dt, h, W, b, t, lse, zt, ws, nbytes, None)


def _sbwd(N=256, D=128, Vs=400, v0=400, Vt=1031, dt=F32, chunk=64, h=FAKE, W=FAKE, b=FAKE, t=FAKE, g=FAKE,
          lse=FAKE, dH=FAKE, hdt=F32, dW=FAKE, tdt=F32, db=FAKE, acc=0, ws=FAKE, nbytes=1 << 40):
    return llp.lib().linear_logp_shard_bwd(N, D, Vs, v0, Vt, dt, chunk, h, W, b, t, g, lse, dH, hdt, dW, tdt, db,
                                           acc, ws, nbytes, None)


def test_shard_argument_errors():
    E = llp.LLP_EINVAL
    # the share must lie inside the vocabulary
    for kw in (dict(v0=-1), dict(v0=632), dict(Vt=0), dict(Vs=0), dict(Vs=1032, v0=0)):
        assert _sfwd(**kw) == E, kw
        assert _sbwd(**kw) == E, kw
    assert _sfwd(lse=None) == E and _sfwd(zt=None) == E and _sfwd(h=None) == E
    assert _sfwd(zt=FAKE + 2) == E  # zt_shard must be 4-byte aligned
    need = llp.linear_logp_fwd_workspace_size(256, 128, 400, F32)
    assert _sfwd(nbytes=need - 1) == llp.LLP_EWORKSPACE
    assert _sfwd(N=1 << 31) == llp.LLP_EOVERFLOW
    assert _sbwd(lse=None) == E        # the global lse is required
    assert _sbwd(hdt=F16) == E         # dH partial: float32 or the operand dtype
    assert _sbwd(tdt=BF16) == E
    assert _sbwd(b=None) == E
    assert _sbwd(acc=2) == E
    bneed = llp.linear_logp_bwd_workspace_size(256, 128, 400, F32, 64, True, True, True, True)
    assert _sbwd(nbytes=bneed - 1) == llp.LLP_EWORKSPACE
    comb = llp.lib().linear_logp_shard_combine
    assert comb(-1, 2, FAKE, FAKE, FAKE, 1031, FAKE, FAKE, None) == E
    assert comb(256, 0, FAKE, FAKE, FAKE, 1031, FAKE, FAKE, None) == E
    assert comb(256, 2, FAKE, FAKE, FAKE, 0, FAKE, FAKE, None) == E
    assert comb(256, 2, None, FAKE, FAKE, 1031, FAKE, FAKE, None) == E
    assert comb(256, 2, FAKE, FAKE, FAKE, 1031, None, None, None) == E
    assert comb(1 << 60, 8, FAKE, FAKE, FAKE, 1031, FAKE, FAKE, None) == llp.LLP_EOVERFLOW
    assert comb(0, 3, None, None, None, 1031, None, None, None) == llp.LLP_OK


def test_header_documents_each_entry_point():
    text = open(os.path.join(ROOT, "include", "llp.h")).read()
    assert "RL-Kernel issue #261" in text and "Liger-Kernel PR #1324" in text and "RL-Kernel PR #495" in text
    for n in declared_symbols():
        i = text.index(n + "(")
        assert "*/" in text[max(0, i - 1500):i], n  # a comment precedes every declaration


def test_ceilings_library_checks_its_arguments():
    """The benchmark's same-box ceilings library (MFMA loop, stream copy and
    read) exports its entry points and rejects bad arguments before any launch
    (hipErrorInvalidValue = 1), so these calls need no GPU."""
    path = os.path.join(ROOT, "cross_entropy_lm_amd", "libllp_ceilings.so")
    if not os.path.exists(path):
        pytest.skip("libllp_ceilings.so is not built")
    lib = ctypes.CDLL(path)
    lib.llpc_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.llpc_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.llpc_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.llpc_read_out_len.argtypes = [ctypes.c_int64]
    lib.llpc_read_out_len.restype = ctypes.c_int64
    fake = ctypes.c_void_p(1 << 40)
    assert lib.llpc_mfma_loop(0, 10, fake, None) == 1
    assert lib.llpc_mfma_loop(8, 0, fake, None) == 1
    assert lib.llpc_mfma_loop(8, 10, None, None) == 1
    assert lib.llpc_copy(fake, fake, 15, None) == 1
    assert lib.llpc_copy(ctypes.c_void_p((1 << 40) + 8), fake, 16, None) == 1
    assert lib.llpc_read(fake, 0, fake, None) == 1
    # one workgroup of 256 threads per 256 KiB chunk
    assert lib.llpc_read_out_len(1 << 31) == 8192 * 256
    assert lib.llpc_read_out_len(16 * 100) == 256
    assert lib.llpc_read_out_len(0) == 0
