"""The Python binding rejects every dtype, shape and device mismatch before it
calls the C library (CPU only: the tensors here are host tensors, so each
call must fail in the binding's checks, never reach a kernel)."""

import pytest

torch = pytest.importorskip("torch")

from cross_entropy_lm_amd import llp  # noqa: E402

N, D, V = 6, 8, 10


def ok_inputs(dt=torch.bfloat16):
    return dict(h=torch.zeros((N, D), dtype=dt), W=torch.zeros((V, D), dtype=dt), b=torch.zeros(V, dtype=dt),
                targets=torch.zeros(N, dtype=torch.int64), g=torch.zeros(N, dtype=torch.float32))


def call_bwd(**over):
    a = ok_inputs()
    a.update(over)
    return llp.linear_logp_bwd(a["h"], a["W"], a["b"], a["targets"], a["g"], a.get("lse"), True, True, True,
                               dH=a.get("dH"), dW=a.get("dW"), db=a.get("db"), dW_dtype=a.get("dW_dtype"))


def call_fused(**over):
    a = ok_inputs()
    a.update(over)
    return llp.linear_logp_fwd_bwd(a["h"], a["W"], a["b"], a["targets"], a["g"], True, True, True,
                                   logp=a.get("logp"), dH=a.get("dH"), dW=a.get("dW"), db=a.get("db"))


@pytest.mark.parametrize("call", [call_bwd, call_fused], ids=["bwd", "fwd_bwd"])
@pytest.mark.parametrize("over,exc", [
    (dict(targets=torch.zeros(N, dtype=torch.int32)), TypeError),          # int32 targets
    (dict(targets=torch.zeros(N + 1, dtype=torch.int64)), ValueError),     # wrong length
    (dict(g=torch.zeros(N, dtype=torch.float64)), TypeError),              # g must be float32
    (dict(g=torch.zeros(N - 1)), ValueError),
    (dict(W=torch.zeros((V, D + 1), dtype=torch.bfloat16)), ValueError),    # W.shape[1] != D
    (dict(W=torch.zeros((V, D), dtype=torch.float16)), TypeError),         # W dtype != h dtype
    (dict(b=torch.zeros(V + 1, dtype=torch.bfloat16)), ValueError),        # bias length != V
    (dict(b=torch.zeros(V, dtype=torch.float32)), TypeError),              # bias dtype != h dtype
    (dict(dH=torch.zeros((N, D), dtype=torch.float32)), TypeError),        # dH in the operand dtype
    (dict(dH=torch.zeros((N, D + 1), dtype=torch.bfloat16)), ValueError),
    (dict(dW=torch.zeros((V, D), dtype=torch.float16)), TypeError),        # table: fp32 or operand dtype
    (dict(dW=torch.zeros((V + 1, D))), ValueError),
    (dict(db=torch.zeros(V - 1)), ValueError),
    (dict(dW=torch.zeros((V, D)), db=torch.zeros(V, dtype=torch.bfloat16)), TypeError),  # one table dtype
    (dict(h=torch.zeros((N, D), dtype=torch.float64), W=torch.zeros((V, D), dtype=torch.float64),
          b=None), TypeError),                                               # unsupported operand dtype
    (dict(h=torch.zeros((N, 2 * D), dtype=torch.bfloat16)[:, ::2]), ValueError),  # not contiguous
    (dict(), ValueError),                                                    # host tensors: not on a GPU
])
def test_linear_wrappers_reject_bad_arguments(call, over, exc):
    with pytest.raises(exc):
        call(**over)


def test_bwd_specific_checks():
    with pytest.raises(TypeError):
        call_bwd(lse=torch.zeros(N, dtype=torch.float16))
    with pytest.raises(ValueError):
        call_bwd(lse=torch.zeros(N + 2))
    with pytest.raises(TypeError):
        call_bwd(dW_dtype=torch.float16)
    with pytest.raises(ValueError):  # db without a bias
        call_bwd(b=None)


def test_fused_output_checks():
    with pytest.raises(TypeError):
        call_fused(logp=torch.zeros(N, dtype=torch.float64))
    with pytest.raises(ValueError):
        call_fused(logp=torch.zeros(N + 1))


def test_fwd_and_shard_checks():
    a = ok_inputs()
    with pytest.raises(TypeError):
        llp.linear_logp_fwd(a["h"], a["W"], a["b"], a["targets"].int())
    with pytest.raises(ValueError):
        llp.linear_logp_fwd(a["h"], a["W"], a["b"], a["targets"], lse=torch.zeros(N + 1))
    with pytest.raises(ValueError):
        llp.linear_logp_fwd(a["h"], a["W"], a["b"], a["targets"])  # host tensors
    with pytest.raises(ValueError):
        llp.linear_logp_shard_fwd(a["h"], a["W"], torch.zeros(V + 1, dtype=torch.bfloat16), a["targets"], 0, V)
    with pytest.raises(ValueError):
        llp.linear_logp_shard_bwd(a["h"], a["W"], a["b"], a["targets"], a["g"], None, 0, V)  # lse required
    with pytest.raises(TypeError):
        llp.linear_logp_shard_bwd(a["h"], a["W"], a["b"], a["targets"], a["g"], torch.zeros(N), 0, V,
                                  dH_dtype=torch.float16)
    with pytest.raises(TypeError):
        llp.linear_logp_shard_combine(torch.zeros((2, N)), torch.zeros((2, N), dtype=torch.float16),
                                      a["targets"], V)
    with pytest.raises(ValueError):
        llp.linear_logp_shard_combine(torch.zeros((2, N)), torch.zeros((3, N)), a["targets"], V)


def test_logits_wrappers():
    z = torch.zeros((N, V), dtype=torch.bfloat16)
    t = torch.zeros(N, dtype=torch.int64)
    with pytest.raises(TypeError):
        llp.logp_fwd(z, t.int())
    with pytest.raises(ValueError):
        llp.logp_fwd(z[:, ::2], t)
    with pytest.raises(TypeError):
        llp.logp_bwd(z, t, torch.zeros(N, dtype=torch.float64))
    with pytest.raises(TypeError):
        llp.logp_bwd(z, t, torch.zeros(N), dlogits=torch.zeros((N, V)))  # dlogits in the logits' dtype
    with pytest.raises(ValueError):
        llp.logp_bwd(z, t, torch.zeros(N))  # host tensors
