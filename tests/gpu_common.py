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


# ----------------------------------------------------------------------------- full-size oracle samples
def sample_tokens(N: int, C: int, n: int = 64) -> np.ndarray:
    """At least n token rows: both sides of every chunk boundary, the ends,
    the middle, and seeded random rows."""
    s = {0, 1, N // 2, N - 2, N - 1}
    for c0 in range(C, N, C):
        s |= {c0 - 1, c0}
    rng = np.random.default_rng(N * 7 + C)
    while len([x for x in s if 0 <= x < N]) < min(n, N):
        s.add(int(rng.integers(0, N)))
    return np.array(sorted(x for x in s if 0 <= x < N))


def sample_vocab(V: int, t_host: np.ndarray, n: int = 64) -> np.ndarray:
    """At least n vocabulary rows: the ends, tile edges, targets of the first
    tokens (rows with one-hot terms), the most frequent target, and seeded
    random rows."""
    s = {0, V - 1, V // 2}
    s |= {x for x in (255, 256, 511, 512, V - 256, V - 257) if 0 <= x < V}
    s |= set(int(x) for x in t_host[:8] if 0 <= x < V)
    vals, cnt = np.unique(t_host[(t_host >= 0) & (t_host < V)], return_counts=True)
    if cnt.size and (cnt > 1).any():
        s.add(int(vals[np.argmax(cnt)]))
    rng = np.random.default_rng(V)
    while len(s) < min(n, V):
        s.add(int(rng.integers(0, V)))
    return np.array(sorted(s))


_LSE_CACHE = {}


class HostCase:
    """Host copies of a workload for the oracle. Every token's lse is
    evaluated once per workload (oracle.linear_lse) and reused by the sampled
    vocabulary rows."""

    def __init__(self, w):
        from oracle import linear_logp as O

        say(f"host inputs for {w.name}")
        self.O = O
        self.w = w
        self.full = synth.make_linear_np(w)

    def lse(self):
        key = (self.w.name, self.w.N, self.w.D, self.w.V, self.w.dtype, self.w.bias)
        if key not in _LSE_CACHE:
            say(f"oracle lse of every token of {self.w.name}")
            f = self.full
            _LSE_CACHE.clear()  # one workload at a time keeps host memory bounded
            _LSE_CACHE[key] = self.O.linear_lse(f["h64"], f["W64"], f["b64"], token_block=2048)
        return _LSE_CACHE[key]

    def tokens(self, rows, g64=None):
        f = self.full
        g = f["g64"][rows] if g64 is None else g64[rows]
        return self.O.linear_logp_token_rows(f["h64"][rows], f["W64"], f["b64"], f["t"][rows], g)

    def vocab(self, vrows, g64=None, tok=slice(None)):
        f = self.full
        g = f["g64"] if g64 is None else g64
        return self.O.linear_logp_vocab_rows(f["h64"][tok], f["W64"], f["b64"], f["t"][tok], g[tok], vrows,
                                             token_block=4096, lse=self.lse()[tok])


# ----------------------------------------------------------------------------- rounding bound
U32 = 2.0 ** -24  # unit roundoff of fp32
U_OP = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -24}


def gamma(n):
    return n * U32 / (1 - n * U32)


def propagated_bound(h64, W64, b64, t, g64, dtype, stored_roundings):
    """First-order bound on the extra error of dH, dW and db that fp32 logits
    and lse (and the operand-dtype storage of the softmax part) cause,
    against the exact float64 definition (elementwise, added to the stated
    tolerance where the softmax rows are nearly one-hot and the gradient
    terms cancel):

    * z = h W^T + b accumulated in fp32 over D products (exact products of
      16-bit values): |dz| <= gamma_{D+1} (|h| |W|^T + |b|).
    * lse = m + ln sum exp(z - m) in fp32 with the hardware exp2 / log2 (a
      few ulp each) and the log2(e) scalings: |dlse| <= max_v |dz| +
      gamma_V + 8u + 4u (|lse| + max_v |z|).
    * p = exp(z - lse): |dp| <= p (|dz| + |dlse| + 2u).
    * the softmax part -g p is stored `stored_roundings` times in the operand
      dtype (relative U_OP each); the one-hot part g (1 - p_t) is fp32.
    * dH = dS W and dW = dS^T h, db = sum dS accumulated in fp32: gamma of
      the contraction length times the sum of the magnitudes.
    Returns (bound_dH [N, D], bound_dW [V, D], bound_db [V]).
    """
    from oracle import linear_logp as O

    N, D = h64.shape
    V = W64.shape[0]
    z = O.logits(h64, W64, b64)
    lse = O.row_logsumexp(z)
    p = np.exp(z - lse[:, None])
    mag = np.abs(h64) @ np.abs(W64).T + (np.abs(b64)[None, :] if b64 is not None else 0.0)
    dz = gamma(D + 1) * mag
    dlse = dz.max(axis=1) + gamma(V) + 8 * U32 + 4 * U32 * (np.abs(lse) + np.abs(z).max(axis=1))
    ok = (t >= 0) & (t < V) & (g64 != 0)
    ag = np.where(ok, np.abs(g64), 0.0)
    dp = p * (dz + dlse[:, None] + 2 * U32)
    e_soft = ag[:, None] * (dp + stored_roundings * U_OP[dtype] * p)   # error of each dS element
    dS = O.softmax_grad(z, lse, t, g64)
    bdH = e_soft @ np.abs(W64) + gamma(V + 1) * (np.abs(dS) @ np.abs(W64)) + U_OP[dtype] * np.abs(dS @ W64)
    bdW = e_soft.T @ np.abs(h64) + gamma(N + 1) * (np.abs(dS).T @ np.abs(h64))
    bdb = e_soft.sum(axis=0) + gamma(N + 1) * np.abs(dS).sum(axis=0)
    return bdH, bdW, bdb


def assert_within(x, ref, atol, rtol, extra, name):
    """Elementwise |x - ref| <= atol + rtol |ref| + extra."""
    x = to64(x) if not isinstance(x, np.ndarray) else x
    err = np.abs(x - ref)
    lim = atol + rtol * np.abs(ref) + extra
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError(f"{name}: {int(bad.sum())}/{bad.size} outside the bound; worst at {i}: got {x[i]!r} "
                             f"want {ref[i]!r} (bound {lim[i]:.3e})")
    return int((err > atol + rtol * np.abs(ref)).sum())  # elements that needed the extra term


def chunk_rounding_budget(w, host, esize_bits):
    """Bound on the extra error of an operand-dtype table: after each chunk the
    running table is rounded to the operand dtype, which moves it by at most
    2^-p |running value| (p = 8 for bf16, 11 for fp16). The running values are
    the oracle's partial sums over the chunks' tokens. The library rounds once
    per working chunk (a run of consecutive chunks), at a subset of these
    points, so the sum over every chunk bounds it too."""
    from oracle import linear_logp as O

    run_w = np.zeros((w.V, w.D))
    run_b = np.zeros(w.V)
    bw = np.zeros((w.V, w.D))
    bb = np.zeros(w.V)
    for c0 in range(0, w.N, w.chunk):
        c1 = min(w.N, c0 + w.chunk)
        _, dw, db = O.linear_logp_bwd(host["h64"][c0:c1], host["W64"], host["b64"], host["t"][c0:c1],
                                      host["g64"][c0:c1], False, True, w.bias)
        run_w += dw
        bw += np.abs(run_w) * 2.0 ** -esize_bits
        if w.bias:
            run_b += db
            bb += np.abs(run_b) * 2.0 ** -esize_bits
    return bw, bb
