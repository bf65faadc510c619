"""Seeded synthetic inputs for the fused linear log-prob workloads.

This module only draws numbers and rounds them to an operand dtype; it holds
none of the log-prob arithmetic. Both the FP64 oracle and the GPU path receive
the arrays it makes.

Generator (counter-based, so any element can be regenerated on its own):

* 32 random bits per element come from two rounds of the MurmurHash3 32-bit
  finalizer ("fmix32", A. Appleby, public domain) applied to the element's flat
  index, keyed by (seed, tensor id).
* A standard normal is read from those bits by piecewise-linear interpolation
  in a 65537-knot table of normal quantiles at probabilities (j + 1/2) / 65537
  (high 16 bits pick the segment, low 16 bits the position in it). The tails
  are therefore cut at about +-4.32 sigma; the shape is otherwise Gaussian.
* A scale is applied with one fp32 multiply, then the value is rounded to the
  operand dtype with round-to-nearest-even.
* Integer targets are floor(u * V / 2^32) for the element's 32 bits u.

Every step is an integer operation or a single IEEE fp32 operation, so the
numpy implementation (host) and the torch implementation (any device) give
bit-identical arrays; ``tests/test_synth.py`` checks this. Large tensors (such
as 32768 x 151936 bf16 logits) are made on the device with the torch path and
the oracle regenerates just the rows it needs with the numpy path.
"""

from __future__ import annotations

import dataclasses
import math
import os

import numpy as np

_M32 = 0xFFFFFFFF
_C1 = 0x85EBCA6B
_C2 = 0xC2B2AE35

# tensor ids: part of the key, so each tensor of a workload is an independent stream
TID_H, TID_W, TID_B, TID_T, TID_G, TID_LOGITS = 1, 2, 3, 4, 5, 6

_TABLE = None


def normal_quantile_table() -> np.ndarray:
    """65537 fp32 knots of the standard-normal inverse CDF at (j + 1/2) / 65537."""
    global _TABLE
    if _TABLE is None:
        from scipy.special import ndtri

        p = (np.arange(65537, dtype=np.float64) + 0.5) / 65537.0
        _TABLE = ndtri(p).astype(np.float32)
    return _TABLE


def _keys(seed: int, tid: int):
    k1 = (seed * 0x9E3779B1 + tid * 0x7F4A7C15 + 0x632BE5AB) & _M32
    k2 = _fmix32_int((k1 ^ 0x5BD1E995) & _M32)
    return k1, k2


def _fmix32_int(h: int) -> int:
    h ^= h >> 16
    h = (h * _C1) & _M32
    h ^= h >> 13
    h = (h * _C2) & _M32
    h ^= h >> 16
    return h


# ----------------------------------------------------------------------------- numpy path
def _fmix32_np(h: np.ndarray) -> np.ndarray:
    # uint32 arithmetic wraps mod 2^32, which is the finalizer's definition
    h = h ^ (h >> np.uint32(16))
    h = h * np.uint32(_C1)
    h = h ^ (h >> np.uint32(13))
    h = h * np.uint32(_C2)
    h = h ^ (h >> np.uint32(16))
    return h


def bits_np(seed: int, tid: int, idx: np.ndarray) -> np.ndarray:
    """32 random bits (uint32) for flat indices ``idx`` (any integer array)."""
    k1, k2 = _keys(seed, tid)
    idx = np.asarray(idx).astype(np.uint64, copy=False)
    lo = (idx & np.uint64(_M32)).astype(np.uint32)
    hi = (idx >> np.uint64(32)).astype(np.uint32)
    a = _fmix32_np(lo ^ np.uint32(k1))
    return _fmix32_np((a ^ np.uint32(k2)) + hi)


def _normal_from_bits_np(u: np.ndarray) -> np.ndarray:
    tab = normal_quantile_table()
    j = (u >> np.uint32(16)).astype(np.int64)
    f = (u & np.uint32(0xFFFF)).astype(np.float32)
    frac = (f + np.float32(0.5)) / np.float32(65536.0)
    t0 = tab[j]
    d = tab[j + 1] - t0
    e = d * frac
    return t0 + e


def normal_rows_np(seed: int, tid: int, cols: int, rows_idx, scale: float = 1.0,
                   threads: int | None = None) -> np.ndarray:
    """fp32 N(0, scale^2) values of the given rows of a [*, cols] tensor.

    Cache-sized row blocks, spread over a thread pool for large requests
    (numpy releases the GIL inside its array operations).
    """
    r = np.asarray(rows_idx, dtype=np.uint64).reshape(-1)
    out = np.empty((r.size, cols), dtype=np.float32)
    step = max(1, (1 << 16) // max(cols, 1))
    cidx = np.arange(cols, dtype=np.uint64)[None, :]

    def fill(i):
        idx = r[i:i + step, None] * np.uint64(cols) + cidx
        x = _normal_from_bits_np(bits_np(seed, tid, idx))
        if scale != 1.0:
            x = x * np.float32(scale)
        out[i:i + step] = x

    starts = range(0, r.size, step)
    if threads is None:
        threads = min(16, os.cpu_count() or 1) if r.size * cols >= (1 << 22) else 1
    if threads > 1:
        from concurrent.futures import ThreadPoolExecutor

        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, starts))
    else:
        for i in starts:
            fill(i)
    return out


def normal_np(seed: int, tid: int, rows: int, cols: int, scale: float = 1.0,
              row0: int = 0, row1: int | None = None) -> np.ndarray:
    """fp32 N(0, scale^2) values of rows [row0, row1) of a [rows, cols] tensor."""
    row1 = rows if row1 is None else row1
    return normal_rows_np(seed, tid, cols, np.arange(row0, row1, dtype=np.uint64), scale)


def targets_np(seed: int, tid: int, n: int, V: int) -> np.ndarray:
    u = bits_np(seed, tid, np.arange(n, dtype=np.uint64)).astype(np.uint64)
    return ((u * np.uint64(V)) >> np.uint64(32)).astype(np.int64)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    r = np.where(nan, np.uint64(0x7FC0), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize_np(x32: np.ndarray, dtype: str):
    """Round fp32 values to an operand dtype.

    Returns (storage, exact) where ``storage`` holds the dtype's bits in the
    numpy type torch can view (uint16 for bf16, float16, float32) and ``exact``
    is the same values as float64 (every bf16/fp16/fp32 value is exact in fp64).
    """
    if dtype == "f32":
        s = np.ascontiguousarray(x32, dtype=np.float32)
        return s, s.astype(np.float64)
    if dtype == "f16":
        s = np.ascontiguousarray(x32, dtype=np.float32).astype(np.float16)
        return s, s.astype(np.float64)
    if dtype == "bf16":
        s = f32_to_bf16_bits(x32)
        return s, bf16_bits_to_f32(s).astype(np.float64)
    raise ValueError(dtype)


# significant bits and smallest quantum (subnormal spacing) of each dtype
_PREC = {"bf16": (8, -133), "f16": (11, -24), "f32": (24, -149)}


def round_f64_np(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the nearest value of ``dtype`` (ties to even),
    returned as float64: the "correctly rounded" reference of a result stored
    in that dtype. One rounding, straight from float64 (no double rounding via
    fp32). Values beyond the dtype's finite range are not handled (the
    gradients compared here are far inside it)."""
    x = np.asarray(x, dtype=np.float64)
    bits, qmin = _PREC[dtype]
    _, e = np.frexp(x)  # |x| = m 2^e with m in [0.5, 1)
    q = np.ldexp(1.0, np.maximum(e - bits, qmin))
    return np.round(x / q) * q  # x / q is exact (a power-of-two scaling); np.round ties to even


def accuracy(got: np.ndarray, ref: np.ndarray, dtype: str) -> dict:
    """Diagnostics of a low-precision result against a float64 reference:
    max |err| / max |ref| and the fraction of elements equal to the correctly
    rounded reference (the two figures RL-Kernel PR #495 prints per
    implementation, "Prior art & reuse decision")."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = float(np.abs(ref).max()) if ref.size else 0.0
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    cr = float(np.mean(got == round_f64_np(ref, dtype))) if ref.size else 1.0
    return {"max_err": err, "max_ref": m, "max_err_over_max": err / m if m > 0 else err,
            "pct_correctly_rounded": 100.0 * cr, "elements": int(ref.size), "dtype": dtype}


# ----------------------------------------------------------------------------- torch path
def _torch():
    import torch

    return torch


def _fmix32_t(h):
    h = h ^ (h >> 16)
    h = (h * _C1) & _M32
    h = h ^ (h >> 13)
    h = (h * _C2) & _M32
    h = h ^ (h >> 16)
    return h


def bits_t(seed: int, tid: int, idx):
    """Same bits as :func:`bits_np` for an int64 torch tensor of flat indices.

    All intermediate values stay in [0, 2^32) before each multiply, so the int64
    products wrap the same way on every device and the masked low 32 bits equal
    the uint64 numpy result.
    """
    k1, k2 = _keys(seed, tid)
    lo = idx & _M32
    hi = idx >> 32
    a = _fmix32_t(lo ^ k1)
    return _fmix32_t(((a ^ k2) + hi) & _M32)


_TAB_T = {}


def _table_t(device):
    torch = _torch()
    key = str(device)
    if key not in _TAB_T:
        _TAB_T[key] = torch.from_numpy(normal_quantile_table()).to(device)
    return _TAB_T[key]


def normal_t(seed: int, tid: int, rows: int, cols: int, scale: float = 1.0, device="cpu",
             out_dtype: str = "f32", row_block: int | None = None):
    """Tensor [rows, cols] of the operand dtype, bit-identical to numpy's path.

    Works in row blocks so the int64 intermediates stay small.
    """
    torch = _torch()
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[out_dtype]
    out = torch.empty((rows, cols), dtype=tdt, device=device)
    tab = _table_t(device)
    if row_block is None:
        row_block = max(1, (1 << 25) // max(cols, 1))
    colidx = torch.arange(cols, dtype=torch.int64, device=device)
    sc = torch.tensor(scale, dtype=torch.float32, device=device)
    for r0 in range(0, rows, row_block):
        r1 = min(rows, r0 + row_block)
        idx = torch.arange(r0, r1, dtype=torch.int64, device=device)[:, None] * cols + colidx[None, :]
        u = bits_t(seed, tid, idx)
        del idx
        j = u >> 16
        frac = ((u & 0xFFFF).to(torch.float32) + 0.5) / 65536.0
        t0 = tab[j]
        d = tab[j + 1] - t0
        x = t0 + d * frac
        if scale != 1.0:
            x = x * sc
        out[r0:r1] = x.to(tdt)
    return out


def targets_t(seed: int, tid: int, n: int, V: int, device="cpu"):
    torch = _torch()
    u = bits_t(seed, tid, torch.arange(n, dtype=torch.int64, device=device))
    return (u * V) >> 32


# ----------------------------------------------------------------------------- workloads
@dataclasses.dataclass(frozen=True)
class LinearWorkload:
    """Shapes and value recipe of one linear log-prob workload."""

    name: str
    N: int
    D: int
    V: int
    dtype: str  # operand dtype of h, W, b: "f32" | "bf16" | "f16"
    bias: bool
    chunk: int  # tokens per backward chunk (0: floor(2^24 / V))
    g: str  # "normal" or "mean" (g = -1/N for every token)
    seed: int = 0
    h_scale: float = 1.0
    w_scale: float = 0.02
    b_scale: float = 0.01


@dataclasses.dataclass(frozen=True)
class LogitsWorkload:
    name: str
    N: int
    V: int
    dtype: str
    seed: int = 0
    scale: float = 2.0


# Workloads of the pages: tiny fp32 (4 chunks of 64); the 4096 x 2048 x 32768 bf16
# default-chunking shape of RL-Kernel issue #261 ("Static traffic model"); the
# 16384 x 4096 x 32000 FLCE shape of Liger-Kernel PR #1324 ("Benchmark results");
# the 32768 x 151936 bf16 logits of RL-Kernel PR #495 ("Results"); and a biased
# large-vocabulary bf16 case at V = 151936.
TINY = LinearWorkload("tiny_f32", 256, 128, 1024, "f32", True, 64, "normal")
RL_DEFAULT = LinearWorkload("rl_default_bf16", 4096, 2048, 32768, "bf16", False, 512, "mean")
FLCE = LinearWorkload("flce_bf16", 16384, 4096, 32000, "bf16", False, 2048, "mean")
FLCE_F16 = dataclasses.replace(FLCE, name="flce_f16", dtype="f16")
FLCE_F32 = dataclasses.replace(FLCE, name="flce_f32", dtype="f32")
BIAS_BIGV = LinearWorkload("bias_bigvocab_bf16", 8192, 4096, 151936, "bf16", True, 0, "normal")
LOGITS = LogitsWorkload("logits_only_bf16", 32768, 151936, "bf16")


def mean_g(N: int) -> float:
    return -1.0 / N if N else 0.0


def make_linear_np(w: LinearWorkload, rows=None):
    """Host arrays of a linear workload.

    Returns a dict with storage arrays ("h", "W", "b", "t", "g") and their exact
    float64 values ("h64", "W64", "b64", "g64"). ``rows`` restricts h, t and g to
    the given token rows (W and b are always whole).
    """
    out = {}
    if rows is None:
        h32 = normal_np(w.seed, TID_H, w.N, w.D, w.h_scale)
        tok = np.arange(w.N)
    else:
        tok = np.asarray(rows, dtype=np.int64)
        h32 = normal_rows_np(w.seed, TID_H, w.D, tok, w.h_scale)
    out["h"], out["h64"] = quantize_np(h32, w.dtype)
    out["W"], out["W64"] = quantize_np(normal_np(w.seed, TID_W, w.V, w.D, w.w_scale), w.dtype)
    if w.bias:
        out["b"], out["b64"] = quantize_np(normal_np(w.seed, TID_B, 1, w.V, w.b_scale)[0], w.dtype)
    else:
        out["b"], out["b64"] = None, None
    t_all = targets_np(w.seed, TID_T, w.N, w.V) if rows is None else \
        _targets_rows_np(w.seed, TID_T, tok, w.V)
    out["t"] = t_all
    if w.g == "mean":
        g = np.full(len(tok), np.float32(mean_g(w.N)), dtype=np.float32)
    else:
        g = (normal_np(w.seed, TID_G, 1, w.N)[0] if rows is None else
             normal_rows_np(w.seed, TID_G, w.N, [0])[0][tok])
    out["g"] = g.astype(np.float32)
    out["g64"] = out["g"].astype(np.float64)
    return out


def _targets_rows_np(seed, tid, rows, V):
    u = bits_np(seed, tid, np.asarray(rows, dtype=np.uint64)).astype(np.uint64)
    return ((u * np.uint64(V)) >> np.uint64(32)).astype(np.int64)


def make_linear_t(w: LinearWorkload, device):
    """Device tensors of a linear workload (bit-identical to :func:`make_linear_np`)."""
    torch = _torch()
    d = {}
    d["h"] = normal_t(w.seed, TID_H, w.N, w.D, w.h_scale, device, w.dtype)
    d["W"] = normal_t(w.seed, TID_W, w.V, w.D, w.w_scale, device, w.dtype)
    d["b"] = normal_t(w.seed, TID_B, 1, w.V, w.b_scale, device, w.dtype)[0].contiguous() if w.bias else None
    d["t"] = targets_t(w.seed, TID_T, w.N, w.V, device)
    if w.g == "mean":
        d["g"] = torch.full((w.N,), mean_g(w.N), dtype=torch.float32, device=device)
    else:
        d["g"] = normal_t(w.seed, TID_G, 1, w.N, 1.0, device, "f32")[0].contiguous()
    return d


def make_logits_t(w: LogitsWorkload, device):
    torch = _torch()
    return {
        "logits": normal_t(w.seed, TID_LOGITS, w.N, w.V, w.scale, device, w.dtype),
        "t": targets_t(w.seed, TID_T, w.N, w.V, device),
        "g": normal_t(w.seed, TID_G, 1, w.N, 1.0, device, "f32")[0].contiguous(),
    }


def make_logits_rows_np(w: LogitsWorkload, rows):
    rows = np.asarray(rows, dtype=np.int64)
    x, x64 = quantize_np(normal_rows_np(w.seed, TID_LOGITS, w.V, rows, w.scale), w.dtype)
    t = _targets_rows_np(w.seed, TID_T, rows, w.V)
    g = normal_rows_np(w.seed, TID_G, w.N, [0])[0][rows].astype(np.float32)
    return {"logits": x, "logits64": x64, "t": t, "g": g, "g64": g.astype(np.float64)}
