"""linear_logp_fwd_noalloc (the forward with the library's device-global
scratch, for callers that cannot allocate) against linear_logp_fwd through
the C ABI: two calls in a row on the same scratch, the second with a smaller
input, bitwise equal to the workspace forward; no device memory allocated by
the call; a shape whose forward workspace exceeds the scratch is rejected
before anything is enqueued."""

import pytest

import synth

from gpu_common import bits_equal, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def llp():
    from cross_entropy_lm_amd import llp as m

    return m


CASES = [
    # near the scratch's limit first (33000 tokens x 125 vocab tiles x 2 blocks x 8 bytes = 66 MB)
    synth.LinearWorkload("noalloc_big_bf16", 33000, 256, 32000, "bf16", True, 0, "normal"),
    # then a smaller, ragged one on the same scratch
    synth.LinearWorkload("noalloc_small_bf16", 700, 136, 1031, "bf16", False, 0, "normal", seed=3),
    synth.LinearWorkload("noalloc_small_f32", 300, 136, 1031, "f32", True, 0, "normal", seed=4),
]


def test_noalloc_forward_equals_the_workspace_forward():
    L = llp()
    for w in CASES:
        say(f"noalloc forward {w.name} N={w.N} D={w.D} V={w.V} {w.dtype}")
        need = L.linear_logp_fwd_workspace_size(w.N, w.D, w.V, L.dtype_code(synth_dtype(w)))
        assert need <= L.LLP_SCRATCH_BYTES
        d = synth.make_linear_t(w, DEV)
        ref_logp, ref_lse = L.linear_logp_fwd(d["h"], d["W"], d["b"], d["t"])
        logp = torch.full((w.N,), float("nan"), device=DEV)
        lse = torch.full((w.N,), float("nan"), device=DEV)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        L.linear_logp_fwd_noalloc(d["h"], d["W"], d["b"], d["t"], logp, lse)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        assert bits_equal(logp, ref_logp) and bits_equal(lse, ref_lse)
        # and without lse
        logp2 = torch.empty(w.N, device=DEV)
        L.linear_logp_fwd_noalloc(d["h"], d["W"], d["b"], d["t"], logp2, None)
        torch.cuda.synchronize()
        assert bits_equal(logp2, ref_logp)


def synth_dtype(w):
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.dtype]


def test_noalloc_rejects_shapes_beyond_the_scratch():
    L = llp()
    w = synth.LinearWorkload("noalloc_over_bf16", 34000, 64, 32000, "bf16", False, 0, "normal")
    assert L.linear_logp_fwd_workspace_size(w.N, w.D, w.V, L.LLP_BF16) > L.LLP_SCRATCH_BYTES
    d = synth.make_linear_t(w, DEV)
    logp = torch.full((w.N,), 7.0, device=DEV)
    with pytest.raises(L.LlpError) as e:
        L.linear_logp_fwd_noalloc(d["h"], d["W"], d["b"], d["t"], logp)
    assert e.value.status == L.LLP_EWORKSPACE
    torch.cuda.synchronize()
    assert bool((logp == 7.0).all())  # nothing was enqueued
    # N = 0 enqueues nothing and succeeds
    e0 = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    out = torch.empty(0, device=DEV)
    L.linear_logp_fwd_noalloc(e0, d["W"], None, d["t"][:0], out)
