"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times, on outputs the FP64 oracle computes one by one: sampled
tokens (at least 64, both sides of every chunk boundary: logp, lse, dH) and
sampled vocabulary rows (at least 64: dW, db, which need every token's lse),
plus properties that hold at any size (bitwise chunk
invariance of logp / dH, exact power-of-two upstream scaling, requested-output
subsets equal to the full run, zero workspace beyond the outputs for the
logits-only op)."""

import numpy as np
import pytest

import synth
from oracle import linear_logp as O

from gpu_common import TOL, HostCase, assert_close, bits_equal, norm_err, sample_tokens, sample_vocab, say, torch_dtype

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def llp():
    from cross_entropy_lm_amd import llp as m

    return m


def run_linear(w, tdt=None, chunk=None, want=(True, True, True), g=None):
    chunk = w.chunk if chunk is None else chunk
    say(f"full-size {w.name} N={w.N} D={w.D} V={w.V} {w.dtype} chunk={chunk} want={want}")
    d = synth.make_linear_t(w, DEV)
    if g is not None:
        d["g"] = g
    L = llp()
    logp, lse = L.linear_logp_fwd(d["h"], d["W"], d["b"], d["t"])
    dH, dW, db = L.linear_logp_bwd(d["h"], d["W"], d["b"], d["t"], d["g"], lse, want[0], want[1],
                                   want[2] and w.bias, dW_dtype=tdt, chunk=chunk)
    torch.cuda.synchronize()
    return d, logp, lse, dH, dW, db


def check_linear(w, host, logp, lse, dH, dW, db, tok, vr, g64=None, tdt_budget=None, label=""):
    dt = w.dtype
    tl, tg = TOL[dt]["logp"], TOL[dt]["grad"]
    rl, rs, rh = host.tokens(tok, g64)
    assert_close(logp[tok], rl, *tl, f"{label} logp")
    assert_close(lse[tok], rs, *tl, f"{label} lse")
    if dH is not None:
        assert_close(dH[tok], rh, *tg, f"{label} dH")
        acc = synth.accuracy(dH[tok].double().cpu().numpy(), rh, dt)
        say(f"{label} dH max err / max {acc['max_err_over_max']:.2e}, "
            f"{acc['pct_correctly_rounded']:.4f}% correctly rounded ({acc['elements']} elements)")
    if dW is not None or db is not None:
        rw, rb = host.vocab(vr, g64)
        if dW is not None:
            if tdt_budget is None:
                assert_close(dW[vr], rw, *tg, f"{label} dW")
            else:
                got = dW[vr].double().cpu().numpy()
                assert np.all(np.abs(got - rw) <= tg[0] + tg[1] * np.abs(rw) + tdt_budget[0]), f"{label} dW"
            say(f"{label} dW normalised error {norm_err(dW[vr], rw):.2e}")
        if db is not None:
            if tdt_budget is None:
                assert_close(db[vr], rb, *tg, f"{label} db")
            else:
                got = db[vr].double().cpu().numpy()
                assert np.all(np.abs(got - rb) <= tg[0] + tg[1] * np.abs(rb) + tdt_budget[1]), f"{label} db"


# ----------------------------------------------------------------------------- tiny fp32 workload
def test_tiny_fp32_edges():
    w = synth.TINY
    d, logp, lse, dH, dW, db = run_linear(w)
    host = HostCase(w)
    rlogp, rlse = O.linear_logp_fwd(host.full["h64"], host.full["W64"], host.full["b64"], host.full["t"])
    rdH, rdW, rdb = O.linear_logp_bwd(host.full["h64"], host.full["W64"], host.full["b64"], host.full["t"],
                                      host.full["g64"], True, True, True)
    for x, r, n in ((logp, rlogp, "logp"), (lse, rlse, "lse"), (dH, rdH, "dH"), (dW, rdW, "dW"), (db, rdb, "db")):
        assert_close(x, r, 1e-5, 5e-4, n)
    # g = 0: +0 everywhere; N = 0: empty logp / dH, +0 tables
    L = llp()
    z = torch.zeros(w.N, device=DEV)
    dH0, dW0, db0 = L.linear_logp_bwd(d["h"], d["W"], d["b"], d["t"], z, lse, True, True, True, chunk=w.chunk)
    e = torch.empty((0, w.D), device=DEV)
    lp, ls = L.linear_logp_fwd(e, d["W"], d["b"], d["t"][:0])
    dHe, dWe, dbe = L.linear_logp_bwd(e, d["W"], d["b"], d["t"][:0], z[:0], ls, True, True, True,
                                      chunk=w.chunk)
    torch.cuda.synchronize()
    for x in (dH0, dW0, db0, dWe, dbe):
        assert bool((x == 0).all()) and not bool(torch.signbit(x).any())
    assert lp.shape == (0,) and dHe.shape == (0, w.D)


# ----------------------------------------------------------------------------- 4096 x 2048 x 32768
def test_rl_default_chunking_and_sweep():
    w = synth.RL_DEFAULT
    L = llp()
    assert L.linear_logp_chunk_rows(w.N, w.V, 0) == 512 and L.linear_logp_num_chunks(w.N, w.V, 0) == 8
    runs = {}
    for k in (1, 2, 4, 8):
        c = w.N // k
        runs[k] = run_linear(w, chunk=c, want=(True, True, False))
    host = HostCase(w)
    tok = sample_tokens(w.N, w.chunk)
    vr = sample_vocab(w.V, host.full["t"])
    for k, (_, logp, lse, dH, dW, _) in runs.items():
        check_linear(w, host, logp, lse, dH, dW, None, tok, vr, label=f"K={k}")
        assert bits_equal(runs[1][1], logp) and bits_equal(runs[1][3], dH), f"chunking changed logp/dH at K={k}"
    # the mean-loss upstream makes the gradients tiny; rerun at g = -1 (exact 2^12 scaling)
    g1 = torch.full((w.N,), -1.0, device=DEV)
    _, _, _, dH1, dW1, _ = run_linear(w, chunk=512, want=(True, True, False), g=g1)
    assert bits_equal(dH1, (runs[8][3].float() * 4096.0).to(dH1.dtype))
    assert bits_equal(dW1, runs[8][4] * 4096.0)
    check_linear(w, host, runs[8][1], runs[8][2], dH1, dW1, None, tok, vr, g64=-np.ones(w.N), label="g=-1")


# ----------------------------------------------------------------------------- 16384 x 4096 x 32000
@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_flce_full_size(dt):
    w = {"bf16": synth.FLCE, "f16": synth.FLCE_F16, "f32": synth.FLCE_F32}[dt]
    d, logp, lse, dH, dW, _ = run_linear(w, want=(True, True, False))
    host = HostCase(w)
    tok = sample_tokens(w.N, w.chunk)
    vr = sample_vocab(w.V, host.full["t"])
    check_linear(w, host, logp, lse, dH, dW, None, tok, vr, label=f"{dt} fp32 table")
    if dt == "bf16":
        # meaningful gradient magnitudes: g = -1 is 2^14 x the mean-loss upstream, exactly
        g1 = torch.full((w.N,), -1.0, device=DEV)
        _, _, _, dH1, dW1, _ = run_linear(w, want=(True, True, False), g=g1)
        assert bits_equal(dH1, (dH.float() * 16384.0).to(dH1.dtype))
        assert bits_equal(dW1, dW * 16384.0)
        check_linear(w, host, logp, lse, dH1, dW1, None, tok, vr, g64=-np.ones(w.N), label="bf16 g=-1")


def test_flce_bf16_operand_dtype_table():
    w = synth.FLCE
    g1 = torch.full((w.N,), -1.0, device=DEV)
    d, logp, lse, dH, dW, _ = run_linear(w, tdt=torch.bfloat16, want=(False, True, False), g=g1)
    assert dW.dtype == torch.bfloat16
    host = HostCase(w)
    vr = sample_vocab(w.V, host.full["t"])
    g64 = -np.ones(w.N)
    # rounding budget of the bf16 table: 2^-8 |running value| after every chunk (the
    # table is rounded once per working chunk of consecutive chunks, a subset of these)
    run = np.zeros((vr.size, w.D))
    budget = np.zeros((vr.size, w.D))
    for c0 in range(0, w.N, w.chunk):
        pw, _ = host.vocab(vr, g64, tok=slice(c0, c0 + w.chunk))
        run += pw
        budget += np.abs(run) * 2.0 ** -8
    atol, rtol = TOL["bf16"]["grad"]
    got = dW[vr].double().cpu().numpy()
    assert np.all(np.abs(got - run) <= atol + rtol * np.abs(run) + budget)
    say(f"bf16 table normalised error {norm_err(got, run):.2e}")


# ----------------------------------------------------------------------------- 8192 x 4096 x 151936, bias
def test_bias_big_vocab_variants():
    w = synth.BIAS_BIGV
    L = llp()
    assert L.linear_logp_chunk_rows(w.N, w.V, 0) == 110 and L.linear_logp_num_chunks(w.N, w.V, 0) == 75
    full = run_linear(w, want=(True, True, True))
    only_dh = run_linear(w, want=(True, False, False))
    only_dw = run_linear(w, want=(False, True, False))
    only_db = run_linear(w, want=(False, False, True))
    assert bits_equal(full[3], only_dh[3]) and only_dh[4] is None and only_dh[5] is None
    assert bits_equal(full[4], only_dw[4]) and only_dw[3] is None and only_dw[5] is None
    assert bits_equal(full[5], only_db[5]) and only_db[3] is None and only_db[4] is None
    perf = run_linear(w, chunk=2048, want=(True, True, True))
    assert bits_equal(full[1], perf[1]) and bits_equal(full[3], perf[3])
    host = HostCase(w)
    tok = sample_tokens(w.N, 110)
    vr = sample_vocab(w.V, host.full["t"])
    _, logp, lse, dH, dW, db = full
    check_linear(w, host, logp, lse, dH, dW, db, tok, vr, label="chunk 110")
    assert_close(perf[4][vr], host.vocab(vr)[0], *TOL["bf16"]["grad"], "chunk 2048 dW")


# ----------------------------------------------------------------------------- logits only, 32768 x 151936
def test_logits_only_full_size():
    w = synth.LOGITS
    L = llp()
    say(f"full-size logits-only {w.N} x {w.V}")
    d = synth.make_logits_t(w, DEV)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    logp, lse = L.logp_fwd(d["logits"], d["t"])
    dl = L.logp_bwd(d["logits"], d["t"], d["g"], lse)
    torch.cuda.synchronize()
    extra = torch.cuda.max_memory_allocated() - base
    need = dl.numel() * dl.element_size() + 2 * w.N * 4
    assert extra <= need + (8 << 20), f"peak extra {extra} vs outputs {need}"  # nothing beyond the outputs
    dl2 = L.logp_bwd(d["logits"], d["t"], d["g"], None)
    torch.cuda.synchronize()
    assert bits_equal(dl, dl2)
    rows = sample_tokens(w.N, 4096, 64)
    host = synth.make_logits_rows_np(w, rows)
    rlogp, rlse = O.logp_fwd(host["logits64"], host["t"])
    rd = O.logp_bwd(host["logits64"], host["t"], host["g64"])
    assert_close(logp[rows], rlogp, *TOL["bf16"]["logp"], "logp")
    assert_close(lse[rows], rlse, *TOL["bf16"]["logp"], "lse")
    assert_close(dl[rows], rd, *TOL["bf16"]["grad"], "dlogits")
    acc = synth.accuracy(dl[rows].double().cpu().numpy(), rd, "bf16")
    say(f"logits-only dlogits max err / max {acc['max_err_over_max']:.2e}, "
        f"{acc['pct_correctly_rounded']:.4f}% correctly rounded ({acc['elements']} elements)")
