"""Graph capture of the library's calls. Every kernel of linear_logp_fwd_bwd,
of linear_logp_fwd + linear_logp_bwd and of logp_fwd + logp_bwd goes onto the
caller's stream, and the library allocates, copies and clears nothing itself
(zeroing is done by its own kernels), so a call can be captured into a HIP
graph. Each replay must reproduce the eager call bit for bit, also after the
outputs were overwritten in between by eager work."""

import pytest

import synth

from gpu_common import bits_equal, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
W_GRAPH = synth.LinearWorkload("graph_bf16", 300, 136, 1031, "bf16", True, 128, "normal")


def llp():
    from cross_entropy_lm_amd import llp as m

    return m


def capture(step):
    """Warm the step up on a side stream, then capture it; returns the graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def replay_matches(g, outs, ref, name, replays=3):
    for r in range(replays):
        # eager work between replays: the outputs are scribbled over first
        for x in outs:
            x.fill_(float("nan") if x.is_floating_point() else 0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(outs, ref)):
            assert bits_equal(x, y), f"{name}: replay {r}, output {i} differs from the eager call"


def linear_setup(w):
    L = llp()
    d = synth.make_linear_t(w, DEV)
    N, D, V = w.N, w.D, w.V
    op = L.dtype_code(d["h"].dtype)
    o = {
        "logp": torch.empty(N, dtype=torch.float32, device=DEV),
        "lse": torch.empty(N, dtype=torch.float32, device=DEV),
        "dH": torch.empty((N, D), dtype=d["h"].dtype, device=DEV),
        "dW": torch.empty((V, D), dtype=torch.float32, device=DEV),
        "db": torch.empty((V,), dtype=torch.float32, device=DEV),
    }
    return L, d, op, o


def test_graph_single_call_replays_bitwise():
    w = W_GRAPH
    say(f"graph single call {w.name} N={w.N} D={w.D} V={w.V} chunk={w.chunk}")
    L, d, op, o = linear_setup(w)
    ws = torch.empty(L.linear_logp_fwd_bwd_workspace_size(w.N, w.D, w.V, op, w.chunk, True, True, True, True),
                     dtype=torch.uint8, device=DEV)

    def step():
        L.linear_logp_fwd_bwd(d["h"], d["W"], d["b"], d["t"], d["g"], True, True, True, chunk=w.chunk,
                              logp=o["logp"], lse=o["lse"], dH=o["dH"], dW=o["dW"], db=o["db"], workspace=ws)

    step()
    torch.cuda.synchronize()
    outs = [o["logp"], o["lse"], o["dH"], o["dW"], o["db"]]
    ref = [x.clone() for x in outs]
    replay_matches(capture(step), outs, ref, "linear_logp_fwd_bwd")


def test_graph_two_calls_replay_bitwise():
    w = W_GRAPH
    say(f"graph two calls {w.name} N={w.N} D={w.D} V={w.V} chunk={w.chunk}")
    L, d, op, o = linear_setup(w)
    ws_f = torch.empty(L.linear_logp_fwd_workspace_size(w.N, w.D, w.V, op), dtype=torch.uint8, device=DEV)
    ws_b = torch.empty(L.linear_logp_bwd_workspace_size(w.N, w.D, w.V, op, w.chunk, True, True, True, True),
                       dtype=torch.uint8, device=DEV)

    def step():
        L.linear_logp_fwd(d["h"], d["W"], d["b"], d["t"], logp=o["logp"], lse=o["lse"], workspace=ws_f)
        L.linear_logp_bwd(d["h"], d["W"], d["b"], d["t"], d["g"], o["lse"], True, True, True, chunk=w.chunk,
                          dH=o["dH"], dW=o["dW"], db=o["db"], workspace=ws_b)

    step()
    torch.cuda.synchronize()
    outs = [o["logp"], o["lse"], o["dH"], o["dW"], o["db"]]
    ref = [x.clone() for x in outs]
    replay_matches(capture(step), outs, ref, "linear_logp_fwd + linear_logp_bwd")


def test_graph_logits_only_replays_bitwise():
    N, V = 257, 5000
    say(f"graph logits-only N={N} V={V} bf16")
    L = llp()
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7)
    logits = (2.0 * torch.randn(N, V, generator=gen, device=DEV)).to(torch.bfloat16)
    t = torch.randint(0, V, (N,), generator=gen, device=DEV)
    g = torch.randn(N, generator=gen, device=DEV)
    logp = torch.empty(N, dtype=torch.float32, device=DEV)
    lse = torch.empty(N, dtype=torch.float32, device=DEV)
    dl = torch.empty_like(logits)

    def step():
        L.logp_fwd(logits, t, logp=logp, lse=lse)
        L.logp_bwd(logits, t, g, lse=lse, dlogits=dl)

    step()
    torch.cuda.synchronize()
    outs = [logp, lse, dl]
    ref = [x.clone() for x in outs]
    replay_matches(capture(step), outs, ref, "logp_fwd + logp_bwd")
