"""Helpers shared by the GPU tests: device inputs, oracle comparisons."""

from __future__ import annotations

import sys

import numpy as np

import synth

# Tolerances: fp32 operands atol 1e-5 / rtol 5e-4 (Liger-Kernel PR #1324,
# "Correctness"); 16-bit operands atol 5e-3 / rtol 5e-2 on logp (same table)
# and the tighter atol 5e-4 / rtol 2e-2 on gradients.
TOL = {
    "f32": {"logp": (1e-5, 5e-4), "grad": (1e-5, 5e-4)},
    "bf16": {"logp": (5e-3, 5e-2), "grad": (5e-4, 2e-2)},
    "f16": {"logp": (5e-3, 5e-2), "grad": (5e-4, 2e-2)},
}


def say(msg: str):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def torch_dtype(dt: str):
    import torch

    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dt]


def to64(x) -> np.ndarray:
    """Device tensor -> float64 numpy (bf16/fp16 widen exactly)."""
    return x.detach().float().cpu().double().numpy()


def assert_close(x, ref, atol, rtol, name):
    x = to64(x) if not isinstance(x, np.ndarray) else x
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (name, x.shape, ref.shape)
    err = np.abs(x - ref)
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        i = np.unravel_index(np.argmax(err - (atol + rtol * np.abs(ref))), err.shape)
        raise AssertionError(
            f"{name}: {int(bad.sum())}/{bad.size} outside atol={atol} rtol={rtol}; worst at {i}: "
            f"got {x[i]!r} want {ref[i]!r}; max abs err {err.max():.3e}, max |ref| {np.abs(ref).max():.3e}")


def norm_err(x, ref) -> float:
    x = to64(x) if not isinstance(x, np.ndarray) else x
    m = np.abs(ref).max()
    return float(np.abs(x - ref).max() / m) if m > 0 else float(np.abs(x).max())


def bits_equal(a, b) -> bool:
    import torch

    if a is None or b is None:
        return a is None and b is None
    if a.dtype != b.dtype or a.shape != b.shape:
        return False
    view = torch.int16 if a.element_size() == 2 else torch.int32
    return bool(torch.equal(a.contiguous().view(view), b.contiguous().view(view)))


def device_case(w: synth.LinearWorkload, dev):
    return synth.make_linear_t(w, dev)
