"""Batch invariance: a token's logp, lse and dH, and a row's logp / lse /
dlogits in the logits-only op, are bitwise the same whatever batch the token
or row is computed in (its size, its position in it, its neighbours) and
whatever the chunking. The vocabulary split (256-row tiles, 128-row partial
blocks), the partials' merge order and the K order of every contraction are
fixed independently of the batch; the per-chunk gradient scale is a power of
two, which rescales the stored softmax part exactly (bf16 and fp32; fp16's
subnormal range is excepted). The pages check batch invariance by computing
rows alone and at the front, middle and end of a batch (RL-Kernel PR #495,
"Summary" and "Prior art & reuse decision")."""

import pytest

import synth

from gpu_common import bits_equal, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def llp():
    from cross_entropy_lm_amd import llp as m

    return m


def run(L, fused, h, W, b, t, g, chunk):
    if fused:
        logp, lse, dH, _, _ = L.linear_logp_fwd_bwd(h, W, b, t, g, True, False, False, chunk=chunk)
    else:
        logp, lse = L.linear_logp_fwd(h, W, b, t)
        dH, _, _ = L.linear_logp_bwd(h, W, b, t, g, lse, True, False, False, chunk=chunk)
    torch.cuda.synchronize()
    return logp, lse, dH


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("fused", [False, True], ids=["split", "fused"])
def test_linear_rows_do_not_depend_on_the_batch(dt, fused):
    w = synth.LinearWorkload(f"inv_{dt}", 1000, 136, 1031, dt, True, 128, "normal")
    d = synth.make_linear_t(w, DEV)
    L = llp()
    lo, hi = 200, 500  # the tokens under test
    say(f"batch invariance {dt} fused={fused}")
    ref = run(L, fused, d["h"][lo:hi].contiguous(), d["W"], d["b"], d["t"][lo:hi].contiguous(),
              d["g"][lo:hi].contiguous(), 64)
    # the same tokens inside larger batches, at other positions, with other chunkings
    cases = [(0, 1000, 0), (0, 777, 128), (150, 1000, 300)]
    for a, z, chunk in cases:
        got = run(L, fused, d["h"][a:z].contiguous(), d["W"], d["b"], d["t"][a:z].contiguous(),
                  d["g"][a:z].contiguous(), chunk)
        for x, y, n in zip(ref, got, ("logp", "lse", "dH")):
            assert bits_equal(x, y[lo - a:hi - a].contiguous()), f"{n} changed in batch [{a}, {z}) chunk {chunk}"
    # and shuffled neighbours: the tokens at position 17 of a batch made of other rows
    idx = torch.cat([torch.arange(600, 617), torch.arange(lo, hi), torch.arange(700, 1000)]).to(DEV)
    got = run(L, fused, d["h"][idx].contiguous(), d["W"], d["b"], d["t"][idx].contiguous(),
              d["g"][idx].contiguous(), 0)
    for x, y, n in zip(ref, got, ("logp", "lse", "dH")):
        assert bits_equal(x, y[17:17 + hi - lo].contiguous()), f"{n} changed among other neighbours"


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_logits_only_rows_do_not_depend_on_the_batch(dt):
    w = synth.LogitsWorkload(f"inv_logits_{dt}", 96, 4099, dt, 5, 2.0)
    d = synth.make_logits_t(w, DEV)
    L = llp()
    say(f"logits-only batch invariance {dt}")
    lo, hi = 30, 50
    sub = d["logits"][lo:hi].contiguous()
    logp, lse = L.logp_fwd(sub, d["t"][lo:hi].contiguous())
    dl = L.logp_bwd(sub, d["t"][lo:hi].contiguous(), d["g"][lo:hi].contiguous(), lse)
    blogp, blse = L.logp_fwd(d["logits"], d["t"])
    bdl = L.logp_bwd(d["logits"], d["t"], d["g"], blse)
    torch.cuda.synchronize()
    assert bits_equal(logp, blogp[lo:hi].contiguous()) and bits_equal(lse, blse[lo:hi].contiguous())
    assert bits_equal(dl, bdl[lo:hi].contiguous())
