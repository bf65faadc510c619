"""The binding and the C ABI on the GPU: calls on a caller's stream (with the
workspace allocated on that stream) give the same bits as on the current
stream, and the opt-in device check rejects a pointer that is not device
memory before anything is enqueued."""

import os

import pytest

import synth

from gpu_common import bits_equal, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def llp():
    from cross_entropy_lm_amd import llp as m

    return m


W_SMALL = synth.LinearWorkload("stream_bf16", 300, 136, 1031, "bf16", True, 128, "normal")


def test_calls_on_a_side_stream_match_the_current_stream():
    L = llp()
    w = W_SMALL
    d = synth.make_linear_t(w, DEV)
    say("binding: current stream vs a side stream (raw handle and Stream object)")
    ref = L.linear_logp_fwd_bwd(d["h"], d["W"], d["b"], d["t"], d["g"], True, True, True, chunk=w.chunk)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got_raw = L.linear_logp_fwd_bwd(d["h"], d["W"], d["b"], d["t"], d["g"], True, True, True, chunk=w.chunk,
                                    stream=side.cuda_stream)
    got_obj = L.linear_logp_fwd_bwd(d["h"], d["W"], d["b"], d["t"], d["g"], True, True, True, chunk=w.chunk,
                                    stream=side)
    lp_s, ls_s = L.linear_logp_fwd(d["h"], d["W"], d["b"], d["t"], stream=side)
    dl_in = torch.randn((64, 1031), device=DEV).to(torch.bfloat16)
    t_in = d["t"][:64].contiguous()
    zl, zs = L.logp_fwd(dl_in, t_in, stream=side)
    zd = L.logp_bwd(dl_in, t_in, d["g"][:64].contiguous(), zs, stream=side)
    side.synchronize()
    for a, b in zip(ref, got_raw):
        assert bits_equal(a, b)
    for a, b in zip(ref, got_obj):
        assert bits_equal(a, b)
    assert bits_equal(ref[0], lp_s) and bits_equal(ref[1], ls_s)
    rl, rs = L.logp_fwd(dl_in, t_in)
    rd = L.logp_bwd(dl_in, t_in, d["g"][:64].contiguous(), rs)
    torch.cuda.synchronize()
    assert bits_equal(rl, zl) and bits_equal(rd, zd)


def test_device_check_rejects_host_memory(monkeypatch):
    L = llp()
    w = W_SMALL
    d = synth.make_linear_t(w, DEV)
    lib = L.lib()
    ws = torch.empty(L.linear_logp_fwd_workspace_size(w.N, w.D, w.V, L.LLP_BF16), dtype=torch.uint8, device=DEV)
    logp_dev = torch.empty(w.N, device=DEV)
    # pinned host memory: reachable by a kernel (so a missed check could not
    # fault), but not device memory of the current device
    logp_host = torch.empty(w.N, pin_memory=True)
    stream = torch.cuda.current_stream().cuda_stream

    def call(logp_ptr):
        return lib.linear_logp_fwd(w.N, w.D, w.V, L.LLP_BF16, d["h"].data_ptr(), d["W"].data_ptr(),
                                   d["b"].data_ptr(), d["t"].data_ptr(), logp_ptr, None, ws.data_ptr(),
                                   ws.numel(), stream)

    say("device check: off by default, on with LLP_CHECK_DEVICE=1")
    monkeypatch.setenv("LLP_CHECK_DEVICE", "1")
    assert call(logp_dev.data_ptr()) == L.LLP_OK
    logp_host.fill_(7.0)
    assert call(logp_host.data_ptr()) == L.LLP_EINVAL
    torch.cuda.synchronize()
    assert bool((logp_host == 7.0).all())  # nothing was enqueued
    assert lib.logp_fwd(4, 1031, L.LLP_BF16, d["W"].data_ptr(), d["t"].data_ptr(), logp_host.data_ptr(), None,
                        stream) == L.LLP_EINVAL
    monkeypatch.delenv("LLP_CHECK_DEVICE")
    assert os.environ.get("LLP_CHECK_DEVICE") is None
    ref, _ = L.linear_logp_fwd(d["h"], d["W"], d["b"], d["t"])
    torch.cuda.synchronize()
    assert bits_equal(ref, logp_dev)
