"""GPU parity of linear_logp (forward + backward) against the FP64 oracle,
through the C ABI, on shapes that span several 256 x 256 tiles with ragged
tails, plus the edge cases and the bitwise properties of the contract."""

import numpy as np
import pytest

import synth
from oracle import linear_logp as O

from gpu_common import TOL, assert_close, bits_equal, chunk_rounding_budget, say, torch_dtype

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def llp():
    from cross_entropy_lm_amd import llp as m

    return m


def run_case(w, want=(True, True, True), tdt=None, lse_given=True, chunk=None, g_override=None):
    say(f"linear {w.name} N={w.N} D={w.D} V={w.V} {w.dtype} bias={w.bias} chunk={w.chunk} want={want}")
    d = synth.make_linear_t(w, DEV)
    if g_override is not None:
        d["g"] = g_override.to(DEV)
    L = llp()
    logp, lse = L.linear_logp_fwd(d["h"], d["W"], d["b"], d["t"])
    dH, dW, db = L.linear_logp_bwd(d["h"], d["W"], d["b"], d["t"], d["g"], lse if lse_given else None,
                                   want[0], want[1], want[2] and w.bias, dW_dtype=tdt,
                                   chunk=w.chunk if chunk is None else chunk)
    torch.cuda.synchronize()
    return d, logp, lse, dH, dW, db


def oracle_case(w, g=None):
    host = synth.make_linear_np(w)
    gg = host["g64"] if g is None else g
    logp, lse = O.linear_logp_fwd(host["h64"], host["W64"], host["b64"], host["t"])
    dH, dW, db = O.linear_logp_bwd(host["h64"], host["W64"], host["b64"], host["t"], gg, True, True,
                                   w.bias)
    return host, logp, lse, dH, dW, db


SMALL = [
    # several tiles along V and N, ragged everywhere, K tail in D (136 = 2 x 64 + 8)
    synth.LinearWorkload("ragged_bf16", 300, 136, 1031, "bf16", True, 128, "normal"),
    synth.LinearWorkload("ragged_f16", 300, 136, 1031, "f16", True, 128, "normal"),
    synth.LinearWorkload("ragged_f32", 300, 136, 1031, "f32", True, 128, "normal"),
    # D not a multiple of 8: element-wise operand loads
    synth.LinearWorkload("oddD_bf16", 130, 99, 515, "bf16", True, 64, "normal"),
    synth.LinearWorkload("oddD_f32", 130, 99, 515, "f32", False, 50, "normal"),
    # V = 255 and V = 1, no bias; chunk 7 leaves a K tail in dW
    synth.LinearWorkload("v255_bf16", 77, 64, 255, "bf16", False, 7, "normal"),
    synth.LinearWorkload("v1_f32", 33, 32, 1, "f32", True, 16, "normal"),
    # tiny fp32 workload: 4 chunks of 64
    synth.TINY,
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_linear_matches_oracle(w):
    _, logp, lse, dH, dW, db = run_case(w)
    _, rlogp, rlse, rdH, rdW, rdb = oracle_case(w)
    tl, tg = TOL[w.dtype]["logp"], TOL[w.dtype]["grad"]
    assert_close(logp, rlogp, *tl, "logp")
    assert_close(lse, rlse, *tl, "lse")
    assert_close(dH, rdH, *tg, "dH")
    assert_close(dW, rdW, *tg, "dW")
    if w.bias:
        assert_close(db, rdb, *tg, "db")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_operand_dtype_table(dt):
    # The stated gradient tolerance plus the table's own re-rounding after
    # every chunk (an operand-dtype table is rounded K times).
    w = synth.LinearWorkload(f"optable_{dt}", 300, 136, 1031, dt, True, 128, "normal")
    _, _, _, dH, dW, db = run_case(w, tdt=torch_dtype(dt))
    assert dW.dtype == torch_dtype(dt) and db.dtype == torch_dtype(dt)
    host, _, _, rdH, rdW, rdb = oracle_case(w)
    bw, bb = chunk_rounding_budget(w, host, 8 if dt == "bf16" else 11)
    atol, rtol = TOL[dt]["grad"]
    assert_close(dH, rdH, atol, rtol, "dH")
    gw = dW.double().cpu().numpy()
    gb = db.double().cpu().numpy()
    assert np.all(np.abs(gw - rdW) <= atol + rtol * np.abs(rdW) + bw), "dW (operand-dtype table)"
    assert np.all(np.abs(gb - rdb) <= atol + rtol * np.abs(rdb) + bb), "db (operand-dtype table)"
    # and the FP32 table of the same run meets the stated tolerance without the budget
    _, _, _, _, dW32, db32 = run_case(w)
    assert_close(dW32, rdW, atol, rtol, "dW (fp32 table)")


def test_recomputed_lse_is_bitwise_the_forward_lse():
    w = SMALL[0]
    _, _, _, dH, dW, db = run_case(w, lse_given=True)
    _, _, _, dH2, dW2, db2 = run_case(w, lse_given=False)
    assert bits_equal(dH, dH2) and bits_equal(dW, dW2) and bits_equal(db, db2)


def test_repeat_is_bit_identical():
    w = SMALL[0]
    a = run_case(w)
    b = run_case(w)
    for x, y in zip(a[1:], b[1:]):
        assert bits_equal(x, y)


def test_requested_subsets_match_the_full_run():
    w = synth.LinearWorkload("subsets_bf16", 300, 136, 1031, "bf16", True, 128, "normal")
    full = run_case(w, want=(True, True, True))
    only_dh = run_case(w, want=(True, False, False))
    only_dw = run_case(w, want=(False, True, False))
    only_db = run_case(w, want=(False, False, True))
    assert only_dh[4] is None and only_dh[5] is None
    assert bits_equal(full[3], only_dh[3])
    assert only_dw[3] is None and bits_equal(full[4], only_dw[4])
    assert only_db[3] is None and only_db[4] is None and bits_equal(full[5], only_db[5])


def test_logp_and_dH_do_not_depend_on_the_chunk():
    w = synth.LinearWorkload("chunks_bf16", 300, 136, 1031, "bf16", True, 128, "normal")
    ref = run_case(w, chunk=300)
    for c in (1, 7, 64, 128, 0):
        r = run_case(w, chunk=c)
        assert bits_equal(ref[1], r[1]), c
        assert bits_equal(ref[3], r[3]), c


def test_power_of_two_upstream_scales_results_exactly():
    w = synth.LinearWorkload("pow2_bf16", 300, 136, 1031, "bf16", True, 128, "normal")
    a = run_case(w)
    g2 = a[0]["g"] * 2.0 ** -14
    b = run_case(w, g_override=g2)
    for x, y in zip(a[3:], b[3:]):
        assert bits_equal(x.float() * 2.0 ** -14, y.float()) if x.dtype == torch.float32 else \
            bits_equal((x.float() * 2.0 ** -14).to(x.dtype), y)


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_zero_upstream_gives_positive_zeros(dt):
    w = synth.LinearWorkload(f"g0_{dt}", 300, 136, 1031, dt, True, 128, "normal")
    for g0 in (0.0, -0.0):
        g = torch.full((w.N,), g0, dtype=torch.float32)
        _, _, _, dH, dW, db = run_case(w, g_override=g)
        for x in (dH, dW, db):
            xf = x.float()
            assert bool((xf == 0).all()), "nonzero gradient for g = 0"
            assert not bool(torch.signbit(xf).any()), "negative zero for g = 0"


def test_out_of_range_targets():
    w = synth.LinearWorkload("oor_bf16", 300, 136, 1031, "bf16", True, 128, "normal")
    d = synth.make_linear_t(w, DEV)
    t = d["t"].clone()
    bad = torch.tensor([1, 150, 299])
    t[bad] = torch.tensor([-100, w.V, w.V + 5], device=DEV)
    L = llp()
    say("out-of-range targets")
    logp, lse = L.linear_logp_fwd(d["h"], d["W"], d["b"], t)
    dH, dW, db = L.linear_logp_bwd(d["h"], d["W"], d["b"], t, d["g"], lse, True, True, True, chunk=w.chunk)
    torch.cuda.synchronize()
    lp = logp.cpu()
    assert bool((lp[bad] == 0).all()) and not bool(torch.signbit(lp[bad]).any())
    dHf = dH.float().cpu()
    assert bool((dHf[bad] == 0).all()) and not bool(torch.signbit(dHf[bad]).any())
    host = synth.make_linear_np(w)
    tt = host["t"].copy()
    tt[bad.numpy()] = [-100, w.V, w.V + 5]
    rlogp, rlse = O.linear_logp_fwd(host["h64"], host["W64"], host["b64"], tt)
    rdH, rdW, rdb = O.linear_logp_bwd(host["h64"], host["W64"], host["b64"], tt, host["g64"], True, True, True)
    tl, tg = TOL["bf16"]["logp"], TOL["bf16"]["grad"]
    assert_close(logp, rlogp, *tl, "logp")
    assert_close(lse, rlse, *tl, "lse")
    assert_close(dH, rdH, *tg, "dH")
    assert_close(dW, rdW, *tg, "dW")
    assert_close(db, rdb, *tg, "db")


def test_empty_batch():
    L = llp()
    say("N = 0")
    D, V = 64, 300
    h = torch.empty((0, D), dtype=torch.bfloat16, device=DEV)
    W = torch.randn((V, D), device=DEV).to(torch.bfloat16)
    b = torch.randn(V, device=DEV).to(torch.bfloat16)
    t = torch.empty(0, dtype=torch.int64, device=DEV)
    g = torch.empty(0, dtype=torch.float32, device=DEV)
    logp, lse = L.linear_logp_fwd(h, W, b, t)
    assert logp.shape == (0,) and lse.shape == (0,)
    dW0 = torch.full((V, D), float("nan"), device=DEV)
    db0 = torch.full((V,), float("nan"), device=DEV)
    dH, dW, db = L.linear_logp_bwd(h, W, b, t, g, lse, True, True, True, dW=dW0, db=db0)
    torch.cuda.synchronize()
    assert dH.shape == (0, D)
    for x in (dW, db):
        assert bool((x == 0).all()) and not bool(torch.signbit(x).any())


def test_accumulate_adds_into_the_callers_table():
    w = synth.LinearWorkload("acc_f32", 200, 72, 600, "f32", True, 64, "normal")
    d = synth.make_linear_t(w, DEV)
    L = llp()
    say("accumulate")
    gen = torch.Generator().manual_seed(5)
    dW0 = torch.randn((w.V, w.D), generator=gen).to(DEV)
    db0 = torch.randn((w.V,), generator=gen).to(DEV)
    logp, lse = L.linear_logp_fwd(d["h"], d["W"], d["b"], d["t"])
    _, dW, db = L.linear_logp_bwd(d["h"], d["W"], d["b"], d["t"], d["g"], lse, False, True, True,
                                  accumulate=True, dW=dW0.clone(), db=db0.clone(), chunk=w.chunk)
    torch.cuda.synchronize()
    host = synth.make_linear_np(w)
    _, rdW, rdb = O.linear_logp_bwd(host["h64"], host["W64"], host["b64"], host["t"], host["g64"], False,
                                    True, True, dW0=dW0.cpu().double().numpy(), db0=db0.cpu().double().numpy())
    assert_close(dW, rdW, 1e-5, 5e-4, "dW accumulate")
    assert_close(db, rdb, 1e-5, 5e-4, "db accumulate")


def test_gradient_tables_sum_to_zero_over_vocab():
    w = synth.LinearWorkload("sum0_f32", 300, 136, 1031, "f32", True, 128, "normal")
    _, _, _, _, dW, db = run_case(w)
    host = synth.make_linear_np(w)
    # sum_v dW[v, d] = 0 exactly in exact arithmetic; allow fp32 rounding of the column sums
    col = dW.double().sum(0).abs().max().item()
    assert col < 1e-4 * dW.double().abs().sum(0).max().item() + 1e-6
    assert abs(db.double().sum().item()) < 1e-5 * db.double().abs().sum().item() + 1e-6
    del host


@pytest.mark.parametrize("fused", [False, True], ids=["split", "fused"])
def test_many_tokens_share_a_target(fused):
    # Half of a 1200-token chunk has one target (several batches of the
    # one-hot row sum), a seventh has the last vocabulary row (ragged tile),
    # and some of them have g = 0 (they take no part); FP32 table.
    w = synth.LinearWorkload("shared_bf16", 1500, 136, 1031, "bf16", True, 1200, "normal")
    d = synth.make_linear_t(w, DEV)
    host = synth.make_linear_np(w)
    i = np.arange(w.N)
    tt = host["t"].copy()
    tt[i % 2 == 0] = 5
    tt[i % 7 == 1] = w.V - 1
    g64 = host["g64"].copy()
    g64[i % 11 == 0] = 0.0
    t = torch.from_numpy(tt).to(DEV)
    g = torch.from_numpy(g64.astype(np.float32)).to(DEV)
    L = llp()
    say(f"shared targets fused={fused}")
    if fused:
        logp, lse, dH, dW, db = L.linear_logp_fwd_bwd(d["h"], d["W"], d["b"], t, g, True, True, True,
                                                      chunk=w.chunk)
    else:
        logp, lse = L.linear_logp_fwd(d["h"], d["W"], d["b"], t)
        dH, dW, db = L.linear_logp_bwd(d["h"], d["W"], d["b"], t, g, lse, True, True, True, chunk=w.chunk)
    torch.cuda.synchronize()
    rlogp, _ = O.linear_logp_fwd(host["h64"], host["W64"], host["b64"], tt)
    rdH, rdW, rdb = O.linear_logp_bwd(host["h64"], host["W64"], host["b64"], tt, g64, True, True, True)
    tl, tg = TOL["bf16"]["logp"], TOL["bf16"]["grad"]
    assert_close(logp, rlogp, *tl, "logp")
    assert_close(dH, rdH, *tg, "dH")
    assert_close(dW, rdW, *tg, "dW")
    assert_close(db, rdb, *tg, "db")
    # the rows of the shared targets carry most of the one-hot mass: check them tighter
    # than the stated tolerance, relative to their own scale
    for v in (5, w.V - 1):
        x = dW[v].double().cpu().numpy()
        assert np.abs(x - rdW[v]).max() <= 1e-3 * np.abs(rdW[v]).max() + 1e-6, v
