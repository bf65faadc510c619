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


# ----------------------------------------------------------------------------- the pages' batch-size sweep
# Eight probe rows, each computed alone and at the front, middle and back of
# batches of every size 1..9 and 2^k - 1 / 2^k / 2^k + 1 up to 2048, over three
# seeds (RL-Kernel PR #495, "Prior art & reuse decision"): 32 sizes, 93 distinct
# placements (sizes 1 and 2 have one and two), so 8 x 93 x 3 = 2232 probe
# placements per quantity, the count the page reports. The other rows of a
# batch are drawn from a pool of different rows, per seed.
SWEEP_SIZES = list(range(1, 10)) + sorted({2 ** k + d for k in range(4, 12) for d in (-1, 0, 1)
                                           if 2 ** k + d <= 2048})
N_PROBES = 8
SEEDS = (0, 1, 2)


def placements():
    for S in SWEEP_SIZES:
        for pos in sorted({0, S // 2, S - 1}):
            yield S, pos


def test_sweep_has_the_pages_count():
    n = sum(1 for _ in placements())
    assert len(SWEEP_SIZES) == 32 and n == 93 and n * N_PROBES * len(SEEDS) == 2232


def batch_index(pool_rows, probe_row, S, pos, filler):
    """Row indices of a batch of size S with `probe_row` at `pos` and the
    first S - 1 rows of `filler` elsewhere."""
    idx = filler[:S - 1].tolist()
    idx.insert(pos, probe_row)
    return torch.tensor(idx, dtype=torch.int64, device=DEV)


def differ(a, b):
    """1 if the two tensors differ in any bit (on the device, no sync)."""
    view = torch.int16 if a.element_size() == 2 else torch.int32
    return (a.contiguous().view(view) != b.contiguous().view(view)).any().int()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("fused", [False, True], ids=["split", "fused"])
def test_linear_batch_size_sweep(dt, fused):
    """logp, lse and dH of each probe token are bitwise the same alone and at
    every placement (default chunk floor(2^24 / V) = 512 tokens at V = 32768,
    so the larger batches span several chunks)."""
    L = llp()
    pool = 2048 + N_PROBES
    counts = {"logp": 0, "lse": 0, "dH": 0}
    total = 0
    for seed in SEEDS:
        w = synth.LinearWorkload(f"sweep_{dt}_{seed}", pool, 136, 32768, dt, True, 0, "normal", seed=seed)
        d = synth.make_linear_t(w, DEV)
        say(f"batch-size sweep {dt} fused={fused} seed {seed}")
        probes = list(range(N_PROBES))
        filler = torch.randperm(pool - N_PROBES, generator=torch.Generator().manual_seed(100 + seed)) + N_PROBES
        def batch(idx):  # (h, t, g) rows of a batch; default chunk
            return run(L, fused, d["h"][idx].contiguous(), d["W"], d["b"], d["t"][idx].contiguous(),
                       d["g"][idx].contiguous(), 0)

        ref = [batch(torch.tensor([p], device=DEV)) for p in probes]
        bad = {k: torch.zeros((), dtype=torch.int32, device=DEV) for k in counts}
        for S, pos in placements():
            for p in probes:
                got = batch(batch_index(pool, p, S, pos, filler))
                for k, x, r in zip(("logp", "lse", "dH"), got, ref[p]):
                    bad[k] += differ(x[pos:pos + 1], r)
                total += 1
        for k in counts:
            counts[k] += int(bad[k].item())
    say(f"batch-size sweep {dt} {'fused' if fused else 'split'}: logp / lse / dH differing "
        f"{counts['logp']} / {counts['lse']} / {counts['dH']} of {total}")
    assert total == 2232
    assert counts == {"logp": 0, "lse": 0, "dH": 0}


def test_logits_only_batch_size_sweep():
    """Logits-only logp and dlogits of each probe row, 32768 x 151936-shaped
    rows (V = 151936, bf16, logits ~ N(0, 2^2)), bitwise the same alone and at
    every placement."""
    L = llp()
    pool = 2048 + N_PROBES
    counts = {"logp": 0, "dlogits": 0}
    total = 0
    for seed in SEEDS:
        w = synth.LogitsWorkload(f"sweep_logits_{seed}", pool, 151936, "bf16", seed, 2.0)
        d = synth.make_logits_t(w, DEV)
        say(f"logits-only batch-size sweep seed {seed}")
        filler = torch.randperm(pool - N_PROBES, generator=torch.Generator().manual_seed(200 + seed)) + N_PROBES
        ref = []
        for p in range(N_PROBES):
            z = d["logits"][p:p + 1].contiguous()
            lp, ls = L.logp_fwd(z, d["t"][p:p + 1].contiguous())
            ref.append((lp, L.logp_bwd(z, d["t"][p:p + 1].contiguous(), d["g"][p:p + 1].contiguous(), ls)))
        bad = {k: torch.zeros((), dtype=torch.int32, device=DEV) for k in counts}
        for S, pos in placements():
            for p in range(N_PROBES):
                idx = batch_index(pool, p, S, pos, filler)
                z = d["logits"][idx].contiguous()
                t = d["t"][idx].contiguous()
                lp, ls = L.logp_fwd(z, t)
                dl = L.logp_bwd(z, t, d["g"][idx].contiguous(), ls)
                bad["logp"] += differ(lp[pos:pos + 1], ref[p][0])
                bad["dlogits"] += differ(dl[pos:pos + 1], ref[p][1])
                total += 1
        torch.cuda.synchronize()
        for k in counts:
            counts[k] += int(bad[k].item())
    say(f"logits-only batch-size sweep: logp / dlogits differing {counts['logp']} / {counts['dlogits']} of {total}")
    assert total == 2232
    assert counts == {"logp": 0, "dlogits": 0}
