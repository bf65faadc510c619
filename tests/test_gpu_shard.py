"""GPU parity of the vocabulary-parallel share calls (linear_logp_shard_fwd,
linear_logp_shard_combine, linear_logp_shard_bwd) against the FP64 oracle.

A vocabulary of Vt rows is cut into contiguous shares; each share's lse and
target logit are checked against the oracle's log-sum-exp over those rows
alone, the merged logp / lse against the oracle over the whole vocabulary, the
summed dH partials against the oracle's dH, and each share's dW / db rows
against the oracle's rows. The pages only name the tensor-parallel operator
(RL-Kernel issue #261, "Non-goals and overlap"); what a share computes follows
from log-sum-exp being associative over any partition of the rows."""

import numpy as np
import pytest

import synth
from oracle import linear_logp as O

from gpu_common import TOL, assert_close, bits_equal, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def llp():
    from cross_entropy_lm_amd import llp as m

    return m


def special_tokens(t, g, Vt):
    """Ignored (-100) and out-of-range (>= Vt) targets and g = 0 on a few tokens."""
    t = t.copy()
    g = g.copy()
    n = len(t)
    t[5] = -100
    t[77] = Vt + 3
    t[n // 2:n // 2 + 10] = -100
    g[9] = 0.0
    g[n - 2] = 0.0
    return t, g


def case(w, bounds):
    host = synth.make_linear_np(w)
    t, g = special_tokens(host["t"], host["g"], w.V)
    d = synth.make_linear_t(w, DEV)
    d["t"] = torch.from_numpy(t).to(DEV)
    d["g"] = torch.from_numpy(g).to(DEV)
    host["t"], host["g64"] = t, g.astype(np.float64)
    shares = list(zip(bounds[:-1], bounds[1:]))
    return host, d, shares


SPLITS = [
    # ragged shares, none aligned to a 256-row tile; K tail in D
    (synth.LinearWorkload("shard_bf16", 300, 136, 1031, "bf16", True, 128, "normal"), [0, 400, 800, 1031]),
    (synth.LinearWorkload("shard_f16", 300, 136, 1031, "f16", True, 128, "normal"), [0, 400, 800, 1031]),
    (synth.LinearWorkload("shard_f32", 300, 136, 1031, "f32", True, 128, "normal"), [0, 400, 800, 1031]),
    # a one-row share at the end and a share that starts past the first tile
    (synth.LinearWorkload("shard_edge_f32", 130, 99, 515, "f32", True, 50, "normal"), [0, 300, 514, 515]),
]


@pytest.mark.parametrize("w,bounds", SPLITS, ids=[s[0].name for s in SPLITS])
def test_shares_match_the_oracle(w, bounds):
    say(f"shard {w.name} N={w.N} D={w.D} Vt={w.V} shares={bounds}")
    host, d, shares = case(w, bounds)
    L = llp()
    P, N, Vt = len(shares), w.N, w.V
    lse_sh = torch.empty((P, N), dtype=torch.float32, device=DEV)
    zt_sh = torch.empty((P, N), dtype=torch.float32, device=DEV)
    for r, (a, z) in enumerate(shares):
        b = d["b"][a:z].contiguous() if w.bias else None
        L.linear_logp_shard_fwd(d["h"], d["W"][a:z].contiguous(), b, d["t"], a, Vt, lse_sh[r], zt_sh[r])
    logp, lse = L.linear_logp_shard_combine(lse_sh, zt_sh, d["t"], Vt)
    torch.cuda.synchronize()

    tl = TOL[w.dtype]["logp"]
    z64 = O.logits(host["h64"], host["W64"], host["b64"])
    t = host["t"]
    for r, (a, z) in enumerate(shares):
        lse_r = O.row_logsumexp(z64[:, a:z])
        assert_close(lse_sh[r], lse_r, *tl, f"lse share {r}")
        own = (t >= a) & (t < z)
        zt = to_np(zt_sh[r])
        assert np.all(np.isneginf(zt[~own])), f"share {r}: zt not -inf off the share"
        assert_close(zt[own], z64[np.nonzero(own)[0], t[own]], *tl, f"zt share {r}")
    ologp, olse = O.linear_logp_fwd(host["h64"], host["W64"], host["b64"], t)
    assert_close(lse, olse, *tl, "lse")
    assert_close(logp, ologp, *tl, "logp")
    bad = (t < 0) | (t >= Vt)
    assert np.all(to_np(logp)[bad] == 0.0) and not np.any(np.signbit(to_np(logp)[bad]))

    # backward of each share with the merged lse; the dH partials summed in fp32
    dH = torch.zeros((N, w.D), dtype=torch.float32, device=DEV)
    dWs, dbs = [], []
    for a, z in shares:
        b = d["b"][a:z].contiguous() if w.bias else None
        ph, pw, pb = L.linear_logp_shard_bwd(d["h"], d["W"][a:z].contiguous(), b, d["t"], d["g"], lse, a, Vt,
                                             True, True, w.bias, chunk=w.chunk)
        assert ph.dtype == torch.float32
        dH += ph
        dWs.append(pw)
        dbs.append(pb)
    torch.cuda.synchronize()
    oH, oW, ob = O.linear_logp_bwd(host["h64"], host["W64"], host["b64"], t, host["g64"], True, True, w.bias)
    tg = TOL[w.dtype]["grad"]
    assert_close(dH, oH, *tg, "dH (sum of partials)")
    assert_close(torch.cat(dWs), oW, *tg, "dW")
    if w.bias:
        assert_close(torch.cat(dbs), ob, *tg, "db")
    # tokens that take no part have exactly +0 gradient rows
    dead = bad | (host["g64"] == 0.0)
    dh = to_np(dH)
    assert np.all(dh[dead] == 0.0)


def to_np(x):
    return x.detach().float().cpu().double().numpy()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_share_rows_equal_the_unsharded_call(dt):
    """With the same lse and chunk, a share's dW / db rows are the unsharded
    call's rows bit for bit (each logit, and each row's contraction over the
    chunk's tokens, has the same operands in the same order); a single share
    covering the whole vocabulary gives linear_logp_fwd's logp and lse."""
    w = synth.LinearWorkload(f"shard_rows_{dt}", 300, 136, 1031, dt, True, 128, "normal")
    say(f"shard rows vs unsharded {dt}")
    host, d, shares = case(w, [0, 400, 800, 1031])
    L = llp()
    logp, lse = L.linear_logp_fwd(d["h"], d["W"], d["b"], d["t"])
    dH, dW, db = L.linear_logp_bwd(d["h"], d["W"], d["b"], d["t"], d["g"], lse, True, True, True, chunk=128)
    for a, z in shares:
        _, pw, pb = L.linear_logp_shard_bwd(d["h"], d["W"][a:z].contiguous(), d["b"][a:z].contiguous(), d["t"],
                                            d["g"], lse, a, w.V, False, True, True, chunk=128)
        torch.cuda.synchronize()
        assert bits_equal(pw, dW[a:z].contiguous()), f"dW rows [{a}, {z})"
        assert bits_equal(pb, db[a:z].contiguous()), f"db rows [{a}, {z})"
    # one share = the whole vocabulary
    lse1, zt1 = L.linear_logp_shard_fwd(d["h"], d["W"], d["b"], d["t"], 0, w.V)
    logp1, lse1m = L.linear_logp_shard_combine(lse1.view(1, -1), zt1.view(1, -1), d["t"], w.V)
    torch.cuda.synchronize()
    assert bits_equal(lse1, lse) and bits_equal(lse1m, lse) and bits_equal(logp1, logp)
    # a dH partial in the operand dtype is the unsharded dH when the share is everything
    ph, _, _ = L.linear_logp_shard_bwd(d["h"], d["W"], d["b"], d["t"], d["g"], lse, 0, w.V, True, False, False,
                                       dH_dtype=d["h"].dtype, chunk=128)
    torch.cuda.synchronize()
    assert bits_equal(ph, dH)


def test_shard_combine_order_and_empty_batch():
    """Merging the shares in another order changes lse only by rounding; N = 0 is a no-op."""
    w = synth.LinearWorkload("shard_order_f32", 256, 64, 700, "f32", False, 64, "normal")
    say("shard combine order")
    host, d, shares = case(w, [0, 100, 350, 700])
    L = llp()
    lse_sh = torch.empty((3, w.N), dtype=torch.float32, device=DEV)
    zt_sh = torch.empty((3, w.N), dtype=torch.float32, device=DEV)
    for r, (a, z) in enumerate(shares):
        L.linear_logp_shard_fwd(d["h"], d["W"][a:z].contiguous(), None, d["t"], a, w.V, lse_sh[r], zt_sh[r])
    logp, lse = L.linear_logp_shard_combine(lse_sh, zt_sh, d["t"], w.V)
    perm = torch.tensor([2, 0, 1], device=DEV)
    logp2, lse2 = L.linear_logp_shard_combine(lse_sh[perm].contiguous(), zt_sh[perm].contiguous(), d["t"], w.V)
    torch.cuda.synchronize()
    assert_close(lse2, to_np(lse), 0.0, 4e-7, "lse, other order")
    assert_close(logp2, to_np(logp), 1e-6, 4e-7, "logp, other order")
    e = torch.empty((3, 0), dtype=torch.float32, device=DEV)
    lp, ls = L.linear_logp_shard_combine(e, e, d["t"][:0], w.V)
    assert lp.numel() == 0 and ls.numel() == 0
