"""GPU parity of the logits-only log-prob (logp_fwd / logp_bwd) against the
FP64 oracle through the C ABI: dtypes, ragged and misaligned rows, V = 1,
out-of-range targets, a -inf masked tail, the lse-free backward, in-place
gradients and bitwise repeats."""

import numpy as np
import pytest

import synth
from oracle import linear_logp as O

from gpu_common import TOL, assert_close, bits_equal, say, torch_dtype

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def llp():
    from cross_entropy_lm_amd import llp as m

    return m


def make(N, V, dt, seed=0, scale=2.0):
    w = synth.LogitsWorkload(f"logits_{dt}", N, V, dt, seed, scale)
    d = synth.make_logits_t(w, DEV)
    host = synth.make_logits_rows_np(w, np.arange(N))
    return w, d, host


# V = 1, 255 and 1031 are the vocabulary sizes of RL-Kernel PR #495's FP64
# agreement tests ("Tests"); 4099 and 151936 add long rows, odd V misaligns rows.
@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("N,V", [(5, 1), (37, 255), (64, 1031), (9, 4099), (6, 151936)])
def test_logits_only_matches_oracle(dt, N, V):
    say(f"logits-only N={N} V={V} {dt}")
    w, d, host = make(N, V, dt, seed=V)
    L = llp()
    logp, lse = L.logp_fwd(d["logits"], d["t"])
    dl = L.logp_bwd(d["logits"], d["t"], d["g"], lse)
    dl2 = L.logp_bwd(d["logits"], d["t"], d["g"], None)
    torch.cuda.synchronize()
    rlogp, rlse = O.logp_fwd(host["logits64"], host["t"])
    rd = O.logp_bwd(host["logits64"], host["t"], host["g64"])
    tl, tg = TOL[dt]["logp"], TOL[dt]["grad"]
    assert_close(logp, rlogp, *tl, "logp")
    assert_close(lse, rlse, *tl, "lse")
    assert_close(dl, rd, *tg, "dlogits")
    assert_close(dl2, rd, *tg, "dlogits (lse recomputed)")
    # the backward that keeps no residual reduces the row exactly as the forward does
    assert bits_equal(dl, dl2)


def test_out_of_range_targets_and_masked_tail():
    say("logits-only: out-of-range targets, -inf tail")
    N, V = 8, 1031
    w, d, host = make(N, V, "bf16", seed=3)
    x = d["logits"].clone()
    x[:, 1000:] = float("-inf")
    t = d["t"].clone() % 1000
    t[2], t[5] = -100, V + 5
    L = llp()
    logp, lse = L.logp_fwd(x, t)
    dl = L.logp_bwd(x, t, d["g"], lse)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(logp).all()) and bool(torch.isfinite(dl.float()).all())
    assert logp[2].item() == 0 and logp[5].item() == 0
    dlf = dl.float()
    assert bool((dlf[[2, 5]] == 0).all()) and not bool(torch.signbit(dlf[[2, 5]]).any())
    assert bool((dlf[:, 1000:] == 0).all()) and not bool(torch.signbit(dlf[:, 1000:]).any())
    x64 = host["logits64"].copy()
    x64[:, 1000:] = -np.inf
    tt = t.cpu().numpy()
    rlogp, _ = O.logp_fwd(x64, tt)
    rd = O.logp_bwd(x64, tt, host["g64"])
    assert_close(logp, rlogp, *TOL["bf16"]["logp"], "logp")
    assert_close(dl, rd, *TOL["bf16"]["grad"], "dlogits")


def test_in_place_gradient_and_repeats():
    say("logits-only: in place, repeats")
    N, V = 16, 4099
    w, d, host = make(N, V, "bf16", seed=9)
    L = llp()
    logp, lse = L.logp_fwd(d["logits"], d["t"])
    a = L.logp_bwd(d["logits"], d["t"], d["g"], lse)
    b = L.logp_bwd(d["logits"], d["t"], d["g"], lse)
    x = d["logits"].clone()
    c = L.logp_bwd(x, d["t"], d["g"], lse, dlogits=x)
    y = d["logits"].clone()
    e = L.logp_bwd(y, d["t"], d["g"], None, dlogits=y)
    torch.cuda.synchronize()
    assert bits_equal(a, b) and bits_equal(a, c) and bits_equal(a, e)


def test_zero_upstream():
    say("logits-only: g = 0")
    w, d, host = make(12, 1031, "f16", seed=4)
    L = llp()
    for g0 in (0.0, -0.0):
        g = torch.full((12,), g0, device=DEV)
        dl = L.logp_bwd(d["logits"], d["t"], g, None).float()
        torch.cuda.synchronize()
        assert bool((dl == 0).all()) and not bool(torch.signbit(dl).any())


def test_empty():
    L = llp()
    x = torch.empty((0, 77), dtype=torch.bfloat16, device=DEV)
    t = torch.empty(0, dtype=torch.int64, device=DEV)
    logp, lse = L.logp_fwd(x, t)
    dl = L.logp_bwd(x, t, torch.empty(0, device=DEV), lse)
    assert logp.shape == (0,) and dl.shape == (0, 77)
