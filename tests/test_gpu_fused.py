"""GPU parity of the single-call forward + backward (linear_logp_fwd_bwd)
against the FP64 oracle through the C ABI: the small ragged shapes of the
split path, the edge cases, the bitwise properties (logp / lse equal to the
forward's, repeats, requested subsets, lse given or not, exact power-of-two
scaling), closeness to the split path's gradients, and the headline workloads
at full size on sampled outputs."""

import numpy as np
import pytest

import synth
from oracle import linear_logp as O

from gpu_common import (TOL, HostCase, assert_close, assert_within, bits_equal, chunk_rounding_budget, norm_err,
                        propagated_bound, sample_tokens, sample_vocab, say, to64, torch_dtype)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# the fused gradients round the softmax part twice (stored numerator, then the
# gradient); their distance to the split path's, relative to its largest entry
SPLIT_CLOSE = {"bf16": 2.0 ** -6, "f16": 2.0 ** -9, "f32": 1e-5}


def llp():
    from cross_entropy_lm_amd import llp as m

    return m


def fused(w, d, want=(True, True, True), tdt=None, chunk=None, g=None, want_lse=True, t=None, **kw):
    say(f"fused {w.name} N={w.N} D={w.D} V={w.V} {w.dtype} chunk={w.chunk if chunk is None else chunk} want={want}")
    out = llp().linear_logp_fwd_bwd(d["h"], d["W"], d["b"], d["t"] if t is None else t,
                                    d["g"] if g is None else g, want[0], want[1], want[2] and w.bias,
                                    dW_dtype=tdt, chunk=w.chunk if chunk is None else chunk,
                                    want_lse=want_lse, **kw)
    torch.cuda.synchronize()
    return out


def split(w, d, tdt=None, chunk=None):
    L = llp()
    logp, lse = L.linear_logp_fwd(d["h"], d["W"], d["b"], d["t"])
    dH, dW, db = L.linear_logp_bwd(d["h"], d["W"], d["b"], d["t"], d["g"], lse, True, True, w.bias,
                                   dW_dtype=tdt, chunk=w.chunk if chunk is None else chunk)
    torch.cuda.synchronize()
    return logp, lse, dH, dW, db


SMALL = [
    synth.LinearWorkload("ragged_bf16", 300, 136, 1031, "bf16", True, 128, "normal"),
    synth.LinearWorkload("ragged_f16", 300, 136, 1031, "f16", True, 128, "normal"),
    synth.LinearWorkload("ragged_f32", 300, 136, 1031, "f32", True, 128, "normal"),
    synth.LinearWorkload("oddD_bf16", 130, 99, 515, "bf16", True, 64, "normal"),
    synth.LinearWorkload("oddD_f32", 130, 99, 515, "f32", False, 50, "normal"),
    synth.LinearWorkload("v255_bf16", 77, 64, 255, "bf16", False, 7, "normal"),
    synth.LinearWorkload("v1_f32", 33, 32, 1, "f32", True, 16, "normal"),
    synth.TINY,
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_fused_matches_oracle_and_the_split_path(w):
    d = synth.make_linear_t(w, DEV)
    logp, lse, dH, dW, db = fused(w, d)
    host = synth.make_linear_np(w)
    rlogp, rlse = O.linear_logp_fwd(host["h64"], host["W64"], host["b64"], host["t"])
    rdH, rdW, rdb = O.linear_logp_bwd(host["h64"], host["W64"], host["b64"], host["t"], host["g64"], True, True,
                                      w.bias)
    tl, tg = TOL[w.dtype]["logp"], TOL[w.dtype]["grad"]
    assert_close(logp, rlogp, *tl, "logp")
    assert_close(lse, rlse, *tl, "lse")
    assert_close(dH, rdH, *tg, "dH")
    assert_close(dW, rdW, *tg, "dW")
    if w.bias:
        assert_close(db, rdb, *tg, "db")
    s_logp, s_lse, s_dH, s_dW, s_db = split(w, d)
    # the forward is the same arithmetic: bitwise
    assert bits_equal(logp, s_logp) and bits_equal(lse, s_lse)
    for x, y, n in ((dH, s_dH, "dH"), (dW, s_dW, "dW"), (db, s_db, "db")):
        if x is None:
            continue
        e = norm_err(x, y.double().cpu().numpy())
        assert e <= SPLIT_CLOSE[w.dtype], f"{n}: fused vs split {e:.2e}"


def test_fused_repeat_subsets_and_lse_are_bitwise():
    w = SMALL[0]
    d = synth.make_linear_t(w, DEV)
    full = fused(w, d)
    again = fused(w, d)
    for x, y in zip(full, again):
        assert bits_equal(x, y)
    no_lse = fused(w, d, want_lse=False)
    assert no_lse[1] is None
    for i in (0, 2, 3, 4):
        assert bits_equal(full[i], no_lse[i])
    only_dh = fused(w, d, want=(True, False, False))
    only_dw = fused(w, d, want=(False, True, False))
    only_db = fused(w, d, want=(False, False, True))
    assert bits_equal(full[2], only_dh[2]) and only_dh[3] is None and only_dh[4] is None
    assert bits_equal(full[3], only_dw[3]) and only_dw[2] is None and only_dw[4] is None
    assert bits_equal(full[4], only_db[4]) and only_db[2] is None and only_db[3] is None
    for o in (only_dh, only_dw, only_db):
        assert bits_equal(full[0], o[0]) and bits_equal(full[1], o[1])
    # nothing to differentiate: the forward alone
    fwd_only = fused(w, d, want=(False, False, False))
    assert bits_equal(full[0], fwd_only[0]) and bits_equal(full[1], fwd_only[1])
    assert fwd_only[2] is None and fwd_only[3] is None and fwd_only[4] is None


def test_fused_logp_and_dH_do_not_depend_on_the_chunk():
    w = SMALL[0]
    d = synth.make_linear_t(w, DEV)
    ref = fused(w, d, chunk=300)
    for c in (1, 7, 64, 128, 0):
        r = fused(w, d, chunk=c)
        assert bits_equal(ref[0], r[0]) and bits_equal(ref[1], r[1]), c
        assert bits_equal(ref[2], r[2]), c


def test_fused_power_of_two_upstream_scales_exactly():
    w = SMALL[0]
    d = synth.make_linear_t(w, DEV)
    a = fused(w, d)
    b = fused(w, d, g=d["g"] * 2.0 ** -14)
    assert bits_equal(a[0], b[0]) and bits_equal(a[1], b[1])
    for x, y in zip(a[2:], b[2:]):
        assert bits_equal(x.float() * 2.0 ** -14, y.float()) if x.dtype == torch.float32 else \
            bits_equal((x.float() * 2.0 ** -14).to(x.dtype), y)


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_fused_zero_upstream_gives_positive_zeros(dt):
    w = synth.LinearWorkload(f"g0_{dt}", 300, 136, 1031, dt, True, 128, "normal")
    d = synth.make_linear_t(w, DEV)
    for g0 in (0.0, -0.0):
        g = torch.full((w.N,), g0, dtype=torch.float32, device=DEV)
        _, _, dH, dW, db = fused(w, d, g=g)
        for x in (dH, dW, db):
            xf = x.float()
            assert bool((xf == 0).all()), "nonzero gradient for g = 0"
            assert not bool(torch.signbit(xf).any()), "negative zero for g = 0"


def test_fused_out_of_range_targets():
    w = synth.LinearWorkload("oor_bf16", 300, 136, 1031, "bf16", True, 128, "normal")
    d = synth.make_linear_t(w, DEV)
    t = d["t"].clone()
    bad = torch.tensor([1, 150, 299])
    t[bad] = torch.tensor([-100, w.V, w.V + 5], device=DEV)
    logp, lse, dH, dW, db = fused(w, d, t=t)
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


def test_fused_empty_batch_and_accumulate():
    L = llp()
    say("fused N = 0")
    D, V = 64, 300
    h = torch.empty((0, D), dtype=torch.bfloat16, device=DEV)
    W = torch.randn((V, D), device=DEV).to(torch.bfloat16)
    b = torch.randn(V, device=DEV).to(torch.bfloat16)
    t = torch.empty(0, dtype=torch.int64, device=DEV)
    g = torch.empty(0, dtype=torch.float32, device=DEV)
    dW0 = torch.full((V, D), float("nan"), device=DEV)
    db0 = torch.full((V,), float("nan"), device=DEV)
    logp, lse, dH, dW, db = L.linear_logp_fwd_bwd(h, W, b, t, g, True, True, True, dW=dW0, db=db0)
    torch.cuda.synchronize()
    assert logp.shape == (0,) and dH.shape == (0, D)
    for x in (dW, db):
        assert bool((x == 0).all()) and not bool(torch.signbit(x).any())
    # accumulate into the caller's tables
    w = synth.LinearWorkload("acc_f32", 200, 72, 600, "f32", True, 64, "normal")
    d = synth.make_linear_t(w, DEV)
    gen = torch.Generator().manual_seed(5)
    a0 = torch.randn((w.V, w.D), generator=gen).to(DEV)
    b0 = torch.randn((w.V,), generator=gen).to(DEV)
    _, _, _, dW, db = fused(w, d, want=(False, True, True), accumulate=True, dW=a0.clone(), db=b0.clone())
    host = synth.make_linear_np(w)
    _, rdW, rdb = O.linear_logp_bwd(host["h64"], host["W64"], host["b64"], host["t"], host["g64"], False,
                                    True, True, dW0=a0.cpu().double().numpy(), db0=b0.cpu().double().numpy())
    assert_close(dW, rdW, 1e-5, 5e-4, "dW accumulate")
    assert_close(db, rdb, 1e-5, 5e-4, "db accumulate")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_fused_operand_dtype_table(dt):
    """The single call's operand-dtype dW / db tables against the oracle: the
    stated gradient tolerance plus the table's own re-rounding (an
    operand-dtype table is rounded once per working chunk, as a same-dtype
    addmm_ would be per chunk), bounded from the oracle's per-chunk partial
    sums. D = 136 takes
    the table epilogue in 16-byte pieces, D = 100 (D % 8 != 0) the one that
    walks the lists per element."""
    for D in (136, 100):
        w = synth.LinearWorkload(f"optable_{dt}_{D}", 300, D, 1031, dt, True, 128, "normal")
        d = synth.make_linear_t(w, DEV)
        logp, lse, dH, dW, db = fused(w, d, tdt=torch_dtype(dt))
        assert dW.dtype == torch_dtype(dt) and db.dtype == torch_dtype(dt)
        host = synth.make_linear_np(w)
        rdH, rdW, rdb = O.linear_logp_bwd(host["h64"], host["W64"], host["b64"], host["t"], host["g64"], True,
                                          True, True)
        bw, bb = chunk_rounding_budget(w, host, 8 if dt == "bf16" else 11)
        atol, rtol = TOL[dt]["grad"]
        assert_close(dH, rdH, atol, rtol, f"dH D={D}")
        assert_within(dW, rdW, atol, rtol, bw, f"dW (operand-dtype table) D={D}")
        assert_within(db, rdb, atol, rtol, bb, f"db (operand-dtype table) D={D}")
        say(f"fused {dt} table D={D}: dW normalised error {norm_err(dW, rdW):.2e}, db {norm_err(db, rdb):.2e}")


# ----------------------------------------------------------------------------- full size
FLCE_W = {"bf16": synth.FLCE, "f16": synth.FLCE_F16, "f32": synth.FLCE_F32}


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_fused_flce_full_size(dt):
    """16384 x 4096 x 32000 in each operand dtype, FP32 table, chunk 2048: the
    single call's logp / lse bitwise the forward's, and sampled tokens and
    vocabulary rows against the oracle at g = -1 (exactly 2^14 x the
    mean-loss upstream, so that the gradient tolerance bites)."""
    w = FLCE_W[dt]
    d = synth.make_linear_t(w, DEV)
    logp, lse, dH, dW, _ = fused(w, d, want=(True, True, False))
    g1 = torch.full((w.N,), -1.0, device=DEV)
    _, _, dH1, dW1, _ = fused(w, d, want=(True, True, False), g=g1)
    # g = -1 is exactly 2^14 x the mean-loss upstream; the results scale exactly
    # unless the small one falls into fp16's subnormal range (dH at g = -2^-14)
    assert bits_equal(dW1, dW * 16384.0)
    if dt != "f16":
        assert bits_equal(dH1, (dH.float() * 16384.0).to(dH1.dtype))
    L = llp()
    flogp, flse = L.linear_logp_fwd(d["h"], d["W"], d["b"], d["t"])
    torch.cuda.synchronize()
    assert bits_equal(logp, flogp) and bits_equal(lse, flse)
    host = HostCase(w)
    tok = sample_tokens(w.N, w.chunk)
    vr = sample_vocab(w.V, host.full["t"])
    tl, tg = TOL[dt]["logp"], TOL[dt]["grad"]
    g64 = -np.ones(w.N)
    rl, rs, rh = host.tokens(tok, g64)
    assert_close(logp[tok], rl, *tl, "logp")
    assert_close(lse[tok], rs, *tl, "lse")
    assert_close(dH1[tok], rh, *tg, "dH (g = -1)")
    acc = synth.accuracy(dH1[tok].double().cpu().numpy(), rh, dt)
    say(f"fused {dt} dH max err / max {acc['max_err_over_max']:.2e}, "
        f"{acc['pct_correctly_rounded']:.4f}% correctly rounded ({acc['elements']} elements)")
    rw, _ = host.vocab(vr, g64)
    assert_close(dW1[vr], rw, *tg, "dW (g = -1)")
    say(f"fused {dt} dW normalised error {norm_err(dW1[vr], rw):.2e}")


def test_fused_flce_bf16_operand_dtype_table_full_size():
    """16384 x 4096 x 32000, bf16 operands, bf16 dW table (one rounding of the
    table per 4096-token working chunk), g = -1: sampled vocabulary rows
    against the oracle within the stated tolerance plus the rounding budget of
    the running table summed over the 2048-token chunks (a superset of the
    points where it is rounded), and sampled dH rows at the stated tolerance."""
    w = synth.FLCE
    d = synth.make_linear_t(w, DEV)
    g1 = torch.full((w.N,), -1.0, device=DEV)
    _, _, dH, dW, _ = fused(w, d, want=(True, True, False), tdt=torch.bfloat16, g=g1)
    assert dW.dtype == torch.bfloat16
    host = HostCase(w)
    vr = sample_vocab(w.V, host.full["t"])
    tok = sample_tokens(w.N, w.chunk)
    g64 = -np.ones(w.N)
    atol, rtol = TOL["bf16"]["grad"]
    _, _, rh = host.tokens(tok, g64)
    assert_close(dH[tok], rh, atol, rtol, "dH (bf16 table run)")
    run = np.zeros((vr.size, w.D))
    budget = np.zeros((vr.size, w.D))
    for c0 in range(0, w.N, w.chunk):
        pw, _ = host.vocab(vr, g64, tok=slice(c0, c0 + w.chunk))
        run += pw
        budget += np.abs(run) * 2.0 ** -8
    needed = assert_within(dW[vr], run, atol, rtol, budget, "dW (bf16 table)")
    say(f"fused bf16 table: dW normalised error {norm_err(dW[vr], run):.2e}; "
        f"{needed} of {run.size} elements used the table's rounding budget")


def test_fused_bias_big_vocab_default_chunk():
    w = synth.BIAS_BIGV
    d = synth.make_linear_t(w, DEV)
    logp, lse, dH, dW, db = fused(w, d, chunk=0)
    L = llp()
    flogp, flse = L.linear_logp_fwd(d["h"], d["W"], d["b"], d["t"])
    torch.cuda.synchronize()
    assert bits_equal(logp, flogp) and bits_equal(lse, flse)
    host = HostCase(w)
    tok = sample_tokens(w.N, 110)
    vr = sample_vocab(w.V, host.full["t"])
    tg = TOL["bf16"]["grad"]
    _, _, rh = host.tokens(tok)
    assert_close(dH[tok], rh, *tg, "dH")
    rw, rb = host.vocab(vr)
    assert_close(dW[vr], rw, *tg, "dW")
    assert_close(db[vr], rb, *tg, "db")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_fused_dw_chunk_pairs(dt):
    """The FP32 table takes one dW contraction per group of chunks. fp32
    operands keep pairs of chunks: K = 2 (the pair's store is the last
    contraction and the one-hot rows of both chunks follow it), K = 3 (a last
    chunk without a partner), K = 4 with a ragged last chunk, and K = 5 with
    accumulate; bf16 operands (D % 8 == 0) run each group as one working
    chunk. dW and db against the oracle, dH bitwise equal to the unchunked
    run's."""
    w = synth.LinearWorkload(f"pairs_{dt}", 300, 136, 1031, dt, True, 128, "normal")
    d = synth.make_linear_t(w, DEV)
    host = synth.make_linear_np(w)
    _, rdW, rdb = O.linear_logp_bwd(host["h64"], host["W64"], host["b64"], host["t"], host["g64"], False, True,
                                    True)
    tg = TOL[dt]["grad"]
    ref = fused(w, d, chunk=300)
    for chunk in (150, 100, 80):  # K = 2, 3, 4 (last chunk 60 tokens)
        _, _, dH, dW, db = fused(w, d, chunk=chunk)
        assert bits_equal(dH, ref[2]), chunk
        assert_close(dW, rdW, *tg, f"dW chunk {chunk}")
        assert_close(db, rdb, *tg, f"db chunk {chunk}")
    gen = torch.Generator().manual_seed(11)
    a0 = torch.randn((w.V, w.D), generator=gen).to(DEV)
    b0 = torch.randn((w.V,), generator=gen).to(DEV)
    _, _, _, dW, db = fused(w, d, want=(True, True, True), chunk=64, accumulate=True, dW=a0.clone(),
                            db=b0.clone())  # K = 5
    _, adW, adb = O.linear_logp_bwd(host["h64"], host["W64"], host["b64"], host["t"], host["g64"], False, True,
                                    True, dW0=a0.cpu().double().numpy(), db0=b0.cpu().double().numpy())
    assert_close(dW, adW, *tg, "dW accumulate, chunk 64")
    assert_close(db, adb, *tg, "db accumulate, chunk 64")


def _oracle_all(h, W, b, t, g):
    h64, W64 = h.double().cpu().numpy(), W.double().cpu().numpy()
    b64 = b.double().cpu().numpy() if b is not None else None
    t64, g64 = t.cpu().numpy(), g.double().cpu().numpy()
    rlogp, rlse = O.linear_logp_fwd(h64, W64, b64, t64)
    rdH, rdW, rdb = O.linear_logp_bwd(h64, W64, b64, t64, g64, True, True, b is not None)
    return rlogp, rlse, rdH, rdW, rdb, h64 @ W64.T + (b64 if b64 is not None else 0.0)


def _block_max_range(z):
    """(smallest, largest) over tokens and 128-row vocab blocks of the block's max logit."""
    V = z.shape[1]
    m = np.stack([z[:, i:i + 128].max(axis=1) for i in range(0, V, 128)], axis=1)
    return float(m.min()), float(m.max())


def test_fused_bf16_logits_out_of_the_stored_range():
    """bf16 numerators are stored per token (2^(z log2 e)) for 128-row blocks whose
    max lies in [-40, 64] nats; other blocks are stored relative to their max and
    their token's column is rescaled before use. Mixed batch: 64 tokens with h
    scaled by 256 (block maxima far above 64 nats) beside ordinary tokens; then
    every logit near -100 (every block below -40).

    The scaled tokens' softmax rows are nearly one-hot and their dW terms
    (|h| ~ 256) cancel between tokens, so the fp32 rounding of their logits and
    lse, which the oracle does not have, shows in dW beyond the stated
    tolerance for ANY fp32-logit implementation: the two-call path on the same
    inputs is checked the same way. Both are compared element by element with
    the stated tolerance plus propagated_bound (the first-order effect of fp32
    logits / lse and of the operand-dtype storage of the softmax part)."""
    w = synth.LinearWorkload("range_bf16", 300, 136, 1031, "bf16", True, 128, "normal")
    d = synth.make_linear_t(w, DEV)
    h = d["h"].clone()
    h[:64] = h[:64] * 256.0  # a power of two: exact in bf16
    rlogp, rlse, rdH, rdW, rdb, z = _oracle_all(h, d["W"], d["b"], d["t"], d["g"])
    assert _block_max_range(z[:64])[1] > 64.0  # the scaled tokens' blocks leave the range
    lo2, hi2 = _block_max_range(z[64:])
    assert -40.0 < lo2 and hi2 < 64.0, (lo2, hi2)  # the others stay inside it
    h64 = h.double().cpu().numpy()
    W64 = d["W"].double().cpu().numpy()
    b64 = d["b"].double().cpu().numpy()
    t64 = d["t"].cpu().numpy()
    g64 = d["g"].double().cpu().numpy()
    tl, tg = TOL["bf16"]["logp"], TOL["bf16"]["grad"]
    L = llp()
    # split path: the softmax part is stored once in bf16
    slogp, slse = L.linear_logp_fwd(h, d["W"], d["b"], d["t"])
    sdH, sdW, sdb = L.linear_logp_bwd(h, d["W"], d["b"], d["t"], d["g"], slse, True, True, True, chunk=128)
    torch.cuda.synchronize()
    bH, bW, bb = propagated_bound(h64, W64, b64, t64, g64, "bf16", 1)
    split_needed = [assert_within(x, r, *tg, e, f"split {n}")
                    for x, r, e, n in ((sdH, rdH, bH, "dH"), (sdW, rdW, bW, "dW"), (sdb, rdb, bb, "db"))]
    say(f"split path: elements beyond the stated tolerance (dH, dW, db) = {split_needed}")
    # the two-call path needs the extra term too: the loss comes from fp32
    # logits and lse, not from the single call's rescaling of flagged columns
    assert split_needed[1] > 0
    # single call: stored numerator, the rescale of flagged tokens' columns and the
    # scaled h^T are three roundings of the softmax part's factors
    bH3, bW3, bb3 = propagated_bound(h64, W64, b64, t64, g64, "bf16", 3)
    for chunk in (128, 300):
        logp, lse, dH, dW, db = L.linear_logp_fwd_bwd(h, d["W"], d["b"], d["t"], d["g"], True, True, True,
                                                      chunk=chunk)
        torch.cuda.synchronize()
        assert_close(logp, rlogp, *tl, f"logp chunk {chunk}")
        assert_close(lse, rlse, *tl, f"lse chunk {chunk}")
        assert bits_equal(logp, slogp) and bits_equal(lse, slse)
        needed = [assert_within(x, r, *tg, e, f"fused {n} chunk {chunk}")
                  for x, r, e, n in ((dH, rdH, bH3, "dH"), (dW, rdW, bW3, "dW"), (db, rdb, bb3, "db"))]
        say(f"fused chunk {chunk}: elements beyond the stated tolerance (dH, dW, db) = {needed}")
        # the ordinary tokens' dH rows need no extra term
        assert_close(dH[64:], rdH[64:], *tg, f"dH (unscaled tokens) chunk {chunk}")
    # every logit near -100: every block lies below the range
    b2 = (d["b"].float() - 100.0).to(torch.bfloat16)
    rlogp, rlse, rdH, rdW, rdb, z = _oracle_all(d["h"], d["W"], b2, d["t"], d["g"])
    assert _block_max_range(z)[1] < -40.0
    logp, lse, dH, dW, db = fused(w, dict(d, b=b2))
    assert_close(logp, rlogp, *tl, "logp (logits near -100)")
    for x, r, n in ((dH, rdH, "dH"), (dW, rdW, "dW"), (db, rdb, "db")):
        assert_close(x, r, *tg, f"{n} (logits near -100)")


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_fused_masked_vocab_blocks(dt):
    """A bias of -inf on vocabulary rows [512, V) masks whole 128-row blocks:
    their probabilities are 0 (stored numerators +0) and every output stays
    finite and matches the oracle; targets lie in the unmasked rows."""
    w = synth.LinearWorkload(f"masked_{dt}", 300, 136, 1031, dt, True, 128, "normal")
    d = synth.make_linear_t(w, DEV)
    b = d["b"].clone()
    b[512:] = float("-inf")
    t = d["t"] % 512
    rlogp, rlse, rdH, rdW, rdb, _ = _oracle_all(d["h"], d["W"], b, t, d["g"])
    logp, lse, dH, dW, db = fused(w, dict(d, b=b, t=t))
    for x in (logp, lse, dH, dW, db):
        assert bool(torch.isfinite(x.float()).all())
    tl, tg = TOL[dt]["logp"], TOL[dt]["grad"]
    assert_close(logp, rlogp, *tl, "logp (masked)")
    assert_close(dH, rdH, *tg, "dH (masked)")
    assert_close(dW, rdW, *tg, "dW (masked)")
    assert_close(db, rdb, *tg, "db (masked)")
    assert bool((dW[512:] == 0).all()) and bool((db[512:] == 0).all())


@pytest.mark.parametrize("chunk", [64, 60])
def test_dw_groups_of_many_chunks(chunk):
    """Small chunks accumulate dW once per group of G chunks, and with an FP32
    table a group runs as one working chunk. At V = 65536 the 4096-column cap
    holds G to 64 chunks of 64 columns, so 5000 tokens need two groups,
    balanced: working chunks of 2560 + 2440 tokens at chunk 64, 2520 + 2480
    at chunk 60 (and dH sums two vocabulary parts). Both paths (single call and two-call), FP32
    table with bias, against the oracle; each path's dH bitwise equal to its
    own unchunked run (the two paths round the softmax part differently)."""
    w = synth.LinearWorkload(f"groups_{chunk}", 5000, 136, 65536, "bf16", True, chunk, "normal")
    d = synth.make_linear_t(w, DEV)
    host = synth.make_linear_np(w)
    rdH, rdW, rdb = O.linear_logp_bwd(host["h64"], host["W64"], host["b64"], host["t"], host["g64"], True, True,
                                      True)
    tg = TOL["bf16"]["grad"]
    ref = fused(w, d, chunk=w.N)
    got = fused(w, d)
    assert bits_equal(ref[2], got[2]) and bits_equal(ref[0], got[0])
    assert_close(got[2], rdH, *tg, "dH")
    assert_close(got[3], rdW, *tg, "dW (single call)")
    assert_close(got[4], rdb, *tg, "db (single call)")
    _, _, sdH, sdW, sdb = split(w, d)
    _, _, sref, _, _ = split(w, d, chunk=w.N)
    assert bits_equal(sref, sdH)  # the two-call path's own dH, unchunked
    assert_close(sdH, rdH, *tg, "dH (two-call)")
    assert_close(sdW, rdW, *tg, "dW (two-call)")
    assert_close(sdb, rdb, *tg, "db (two-call)")


@pytest.mark.parametrize("tab", ["f32", "bf16"])
def test_pairs_run_as_working_chunks(tab):
    """Chunks whose dH has 128 or more tiles pair for dW, and with dW or db
    requested a pair runs as one working chunk: 1024-token chunks at D = 8192
    (4 x 32 dH tiles each) give working chunks of 2048 tokens and a ragged
    452. Both paths, with bias, an FP32 or a bf16 table. The stored softmax
    parts do not depend on the chunking (per-token values, power-of-two chunk
    scales), so dW and db equal those of one unchunked call up to the order
    of the fp32 additions: a token dropped or added twice by the schedule
    would move them by about 1e-3 of their largest element. Against the
    oracle: at D = 8192 the logits spread enough (std 1.8) that some
    vocabulary rows collect large softmax terms that cancel, so the stated
    tolerance takes the first-order bound of their bf16 storage (three
    roundings on the single call, one on the two-call path), plus a bf16
    table's rounding budget over the 1024-token chunks. logp, lse and dH are
    bitwise those of a dH-only call, which keeps the caller's chunks; a
    dW-only and a db-only call give the full call's dW and db bit for bit."""
    w = synth.LinearWorkload(f"pairs_{tab}", 2500, 8192, 1031, "bf16", True, 1024, "normal")
    d = synth.make_linear_t(w, DEV)
    host = synth.make_linear_np(w)
    h64, W64, b64, t64, g64 = host["h64"], host["W64"], host["b64"], host["t"], host["g64"]
    rdH, rdW, rdb = O.linear_logp_bwd(h64, W64, b64, t64, g64, True, True, True)
    atol, rtol = TOL["bf16"]["grad"]
    tdt = None if tab == "f32" else torch.bfloat16
    got = fused(w, d, tdt=tdt)
    one = fused(w, d, tdt=tdt, chunk=w.N)
    only_dh = fused(w, d, want=(True, False, False))
    assert bits_equal(only_dh[0], got[0]) and bits_equal(only_dh[1], got[1]) and bits_equal(only_dh[2], got[2])
    # dW alone and db alone run the same working chunks as the full call
    only_dw = fused(w, d, tdt=tdt, want=(False, True, False))
    only_db = fused(w, d, tdt=tdt, want=(False, False, True))
    assert bits_equal(only_dw[3], got[3]) and only_dw[2] is None and only_dw[4] is None
    assert bits_equal(only_db[4], got[4]) and only_db[2] is None and only_db[3] is None
    assert_close(got[2], rdH, atol, rtol, "dH")
    _, _, sdH, sdW, sdb = split(w, d, tdt=tdt)
    _, _, _, sdW1, sdb1 = split(w, d, tdt=tdt, chunk=w.N)
    assert_close(sdH, rdH, atol, rtol, "dH (two-call)")
    _, bW1, bb1 = propagated_bound(h64, W64, b64, t64, g64, "bf16", 1)
    _, bW3, bb3 = propagated_bound(h64, W64, b64, t64, g64, "bf16", 3)
    if tab == "f32":
        for name, x, y in (("dW", got[3], one[3]), ("db", got[4], one[4]), ("dW (two-call)", sdW, sdW1),
                           ("db (two-call)", sdb, sdb1)):
            e = norm_err(x, to64(y))
            assert e < 1e-5, f"{name}: paired schedule vs one chunk {e:.2e}"
        bw = bb = 0.0
    else:
        bw, bb = chunk_rounding_budget(w, host, 8)
    needed = [assert_within(x, r, atol, rtol, b + e, f"{name} ({tab} table)")
              for name, x, r, b, e in (("dW", got[3], rdW, bw, bW3), ("db", got[4], rdb, bb, bb3),
                                       ("dW (two-call)", sdW, rdW, bw, bW1), ("db (two-call)", sdb, rdb, bb, bb1))]
    assert all(x.dtype == (torch.float32 if tab == "f32" else torch.bfloat16) for x in (got[3], got[4], sdW, sdb))
    say(f"pairs {tab} table: elements beyond the stated tolerance (dW, db, two-call dW, db) = {needed}")


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_dh_vocabulary_parts(dt):
    """dH sums the vocabulary in fixed parts whose fp32 sums are added in
    increasing order (V = 70000: parts of 32768, 32768 and 4464 rows for
    16-bit operands; eight of 8192 and one of 4464 for fp32).
    Both paths against the oracle (dH, dW, db, logp); each path's dH bitwise
    the same at every chunking (the parts depend on V alone); bf16 also with
    D % 8 != 0 (the layout with a transposed W, split the same way)."""
    for D in ((136, 100) if dt == "bf16" else (136,)):
        w = synth.LinearWorkload(f"parts_{dt}_{D}", 300, D, 70000, dt, True, 128, "normal")
        d = synth.make_linear_t(w, DEV)
        host = synth.make_linear_np(w)
        rlogp, _ = O.linear_logp_fwd(host["h64"], host["W64"], host["b64"], host["t"])
        rdH, rdW, rdb = O.linear_logp_bwd(host["h64"], host["W64"], host["b64"], host["t"], host["g64"], True,
                                          True, True)
        tl, tg = TOL[dt]["logp"], TOL[dt]["grad"]
        ref_f = fused(w, d, chunk=w.N)
        ref_s = split(w, d, chunk=w.N)
        for chunk in (128, 64, 0):
            f_out = fused(w, d, chunk=chunk)
            s_out = split(w, d, chunk=chunk)
            assert bits_equal(f_out[2], ref_f[2]) and bits_equal(s_out[2], ref_s[2]), (D, chunk)
            for (logp, _, dH, dW, db), n in ((f_out, "single call"), (s_out, "two-call")):
                assert_close(logp, rlogp, *tl, f"logp {n} D={D} chunk {chunk}")
                assert_close(dH, rdH, *tg, f"dH {n} D={D} chunk {chunk}")
                assert_close(dW, rdW, *tg, f"dW {n} D={D} chunk {chunk}")
                assert_close(db, rdb, *tg, f"db {n} D={D} chunk {chunk}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_fast_table_tails_in_both_dimensions(dt):
    """The FP32 table's read-modify-write epilogue on ragged tiles in both
    dimensions: V = 1031 leaves a last row tile of 7 rows, and D = 520 spreads
    each row tile over three column tiles, the last holding 8 columns. Every
    table access of such a tile must stay inside a buffer range that ends at
    the table's last element. Both paths are checked against the oracle,
    storing the table and accumulating into a given one (which makes every
    contraction read the old values)."""
    w = synth.LinearWorkload(f"tails_{dt}", 300, 520, 1031, dt, True, 64, "normal")
    d = synth.make_linear_t(w, DEV)
    host = synth.make_linear_np(w)
    rlogp, _ = O.linear_logp_fwd(host["h64"], host["W64"], host["b64"], host["t"])
    rdH, rdW, rdb = O.linear_logp_bwd(host["h64"], host["W64"], host["b64"], host["t"], host["g64"], True,
                                      True, True)
    tl, tg = TOL[dt]["logp"], TOL[dt]["grad"]
    for (logp, _, dH, dW, db), n in ((fused(w, d), "single call"), (split(w, d), "two-call")):
        assert dW.dtype == torch.float32 and db.dtype == torch.float32
        assert_close(logp, rlogp, *tl, f"logp {n}")
        assert_close(dH, rdH, *tg, f"dH {n}")
        assert_close(dW, rdW, *tg, f"dW {n}")
        assert_close(db, rdb, *tg, f"db {n}")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(11)
    t0 = torch.randn(w.V, w.D, generator=gen, device=DEV)
    b0 = torch.randn(w.V, generator=gen, device=DEV)
    base_w, base_b = t0.double().cpu().numpy(), b0.double().cpu().numpy()
    dW, db = t0.clone(), b0.clone()
    fused(w, d, accumulate=True, dW=dW, db=db)
    assert_close(dW, base_w + rdW, *tg, "dW single call, accumulate")
    assert_close(db, base_b + rdb, *tg, "db single call, accumulate")
    dW, db = t0.clone(), b0.clone()
    L = llp()
    _, lse = L.linear_logp_fwd(d["h"], d["W"], d["b"], d["t"])
    L.linear_logp_bwd(d["h"], d["W"], d["b"], d["t"], d["g"], lse, True, True, True, chunk=w.chunk,
                      accumulate=True, dW=dW, db=db)
    torch.cuda.synchronize()
    assert_close(dW, base_w + rdW, *tg, "dW two-call, accumulate")
    assert_close(db, base_b + rdb, *tg, "db two-call, accumulate")
