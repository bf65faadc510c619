"""FP64 CPU oracle of the fused linear log-prob, forward and backward.

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg import this module. The GPU library never calls
it, and it shares no code with the GPU library.

It is the plain definition of what the operator computes, written out in
float64 with numpy (a matrix product is the only library step). It does no
chunking, blocking, fusion or reduced-precision rounding: the chunked, fused
GPU path has to reach these numbers up to rounding.

Definitions and where they come from:

* logits ``z = h W^T + b`` over the vocabulary, hidden states ``h [N, D]``,
  weight ``W [V, D]`` in the layout of a linear layer's weight, optional bias
  ``b [V]`` ("linear_logp", RL-Kernel issue #261, "Current production path";
  fused linear cross-entropy, Liger-Kernel PR #1324, "Summary").
* ``lse = m + ln(sum_v exp(z_v - m))`` with ``m = max_v z_v`` and
  ``logp = z[t] - lse``: the log-softmax taken at the target token
  (RL-Kernel PR #495, "Summary": the fused logp forward's max and sum-exp
  passes).
* Targets outside ``[0, V)`` (for example the ignore index -100) give
  ``logp = 0`` and an exactly zero gradient row (RL-Kernel PR #495,
  "Behavior changes", out-of-range targets).
* ``dlogits = g * (onehot(t) - softmax(z))`` for an upstream gradient ``g``
  of logp (RL-Kernel PR #495, "Summary", second commit). It is evaluated as
  the two products ``g*[v==t] - g*p`` so that ``g = +-0`` gives +0.
* ``dH = dlogits W``, ``dW = dlogits^T h`` added into one table that starts
  at +0 (RL-Kernel issue #261, "Current accumulation" and "Correctness
  boundary": the zero-initialised table is kept), ``db = sum_n dlogits``.
  With ``accumulate`` the caller's table is added as the last term (in-place
  accumulation into an existing gradient, Liger-Kernel PR #1324, "Details").
* N = 0 gives empty logp/dH and +0 dW/db (RL-Kernel issue #261, "Correctness
  boundary": preserved N=0 behaviour).

All pins of this module (closed forms, invariants, finite differences, a
hand-derived worked example and an independent library routine) are in
``tests/test_oracle_pins.py``.
"""

from __future__ import annotations

import numpy as np

F64 = np.float64


def _as64(x):
    return None if x is None else np.asarray(x, dtype=F64)


def logits(h, W, b=None):
    """z[n, v] = sum_d h[n, d] W[v, d] (+ b[v]), in float64."""
    z = _as64(h) @ _as64(W).T
    if b is not None:
        z = z + _as64(b)[None, :]
    return z


def row_logsumexp(z):
    """Per row: m = max_v z, S = sum_v exp(z - m), lse = m + ln S."""
    z = _as64(z)
    m = z.max(axis=1)
    S = np.exp(z - m[:, None]).sum(axis=1)
    return m + np.log(S)


def valid_targets(t, V):
    t = np.asarray(t, dtype=np.int64)
    return (t >= 0) & (t < V)


def target_logp(z, lse, t):
    """logp[n] = z[n, t_n] - lse[n] for a valid target, else +0."""
    z = _as64(z)
    t = np.asarray(t, dtype=np.int64)
    V = z.shape[1]
    ok = valid_targets(t, V)
    out = np.zeros(z.shape[0], dtype=F64)
    rows = np.nonzero(ok)[0]
    out[rows] = z[rows, t[rows]] - lse[rows]
    return out


def softmax_grad(z, lse, t, g):
    """dlogits[n, v] = g_n [v == t_n] - g_n p[n, v], p = exp(z - lse).

    Rows with an out-of-range target or with g_n == 0 are +0.
    """
    z = _as64(z)
    g = _as64(g)
    t = np.asarray(t, dtype=np.int64)
    N, V = z.shape
    ok = valid_targets(t, V) & (g != 0)
    p = np.exp(z - lse[:, None])
    onehot = np.zeros((N, V), dtype=F64)
    rows = np.nonzero(ok)[0]
    onehot[rows, t[rows]] = 1.0
    d = g[:, None] * onehot - g[:, None] * p
    d[~ok] = 0.0
    return d + 0.0  # x + (+0) turns any -0 produced above into +0


# ----------------------------------------------------------------------------- linear op
def linear_logp_fwd(h, W, b, t):
    """Returns (logp [N], lse [N]) in float64."""
    h = _as64(h)
    if h.shape[0] == 0:
        return np.zeros(0, F64), np.zeros(0, F64)
    z = logits(h, W, b)
    lse = row_logsumexp(z)
    return target_logp(z, lse, t), lse


def linear_logp_bwd(h, W, b, t, g, want_dH=True, want_dW=True, want_db=False,
                    dW0=None, db0=None):
    """Returns (dH [N, D] | None, dW [V, D] | None, db [V] | None) in float64.

    ``dW0``/``db0`` are the caller's tables for accumulate mode (added last).
    """
    h = _as64(h)
    W = _as64(W)
    N, D = h.shape
    V = W.shape[0]
    if N:
        z = logits(h, W, b)
        lse = row_logsumexp(z)
        dS = softmax_grad(z, lse, t, g)
    else:
        dS = np.zeros((0, V), F64)
    dH = (dS @ W + 0.0) if want_dH else None
    dW = None
    if want_dW:
        dW = np.zeros((V, D), F64) + dS.T @ h
        if dW0 is not None:
            dW = dW + _as64(dW0)
        dW = dW + 0.0
    db = None
    if want_db:
        db = np.zeros(V, F64) + dS.sum(axis=0)
        if db0 is not None:
            db = db + _as64(db0)
        db = db + 0.0
    return dH, dW, db


def linear_logp_token_rows(h_rows, W, b, t_rows, g_rows):
    """logp, lse and dH for a subset of tokens (each token is independent).

    ``h_rows``, ``t_rows`` and ``g_rows`` hold only the sampled tokens.
    """
    z = logits(h_rows, W, b)
    lse = row_logsumexp(z)
    logp = target_logp(z, lse, t_rows)
    dS = softmax_grad(z, lse, t_rows, g_rows)
    return logp, lse, dS @ _as64(W) + 0.0


def linear_lse(h, W, b, token_block=1024):
    """lse [N] of every token (``row_logsumexp`` of its logits), evaluated
    token block by token block so that the [N, V] logits are never held."""
    h = _as64(h)
    W = _as64(W)
    bb = None if b is None else _as64(b)
    out = np.zeros(h.shape[0], F64)
    for n0 in range(0, h.shape[0], token_block):
        n1 = min(h.shape[0], n0 + token_block)
        out[n0:n1] = row_logsumexp(logits(h[n0:n1], W, bb))
    return out


def linear_logp_vocab_rows(h, W, b, t, g, vrows, token_block=1024, lse=None):
    """dW[v, :] and db[v] for a subset of vocabulary rows ``vrows``.

    These need every token's lse, which is evaluated token block by token
    block (each token's lse is independent of the others), or taken from
    ``lse`` (the ``linear_lse`` of the same h, W, b) when given; the sum over
    tokens then runs over all N in increasing token order per block and
    block order, as a plain sum.
    """
    h = _as64(h)
    W = _as64(W)
    vrows = np.asarray(vrows, dtype=np.int64)
    N, D = h.shape
    V = W.shape[0]
    t = np.asarray(t, dtype=np.int64)
    g = _as64(g)
    dW = np.zeros((vrows.size, D), F64)
    db = np.zeros(vrows.size, F64)
    bb = None if b is None else _as64(b)
    # the sampled rows' logits and, when lse is given, only those: the
    # softmax gradient of a column needs its token's lse and its own logit
    Wv = W[vrows]
    bv = None if bb is None else bb[vrows]
    for n0 in range(0, N, token_block):
        n1 = min(N, n0 + token_block)
        if lse is None:
            z = logits(h[n0:n1], W, bb)
            lse_b = row_logsumexp(z)
            dS = softmax_grad(z, lse_b, t[n0:n1], g[n0:n1])[:, vrows]
        else:
            dS = _softmax_grad_columns(logits(h[n0:n1], Wv, bv), _as64(lse)[n0:n1], t[n0:n1], g[n0:n1], vrows, V)
        dW += dS.T @ h[n0:n1]
        db += dS.sum(axis=0)
    return dW + 0.0, db + 0.0


def _softmax_grad_columns(zc, lse, t, g, vrows, V):
    """Columns ``vrows`` of ``softmax_grad``: the same two products
    g [v == t] - g exp(z - lse), with +0 rows for an out-of-range target or
    g == 0, evaluated on the sampled columns' logits ``zc`` only."""
    g = _as64(g)
    t = np.asarray(t, dtype=np.int64)
    ok = valid_targets(t, V) & (g != 0)
    p = np.exp(_as64(zc) - lse[:, None])
    onehot = (t[:, None] == vrows[None, :]).astype(F64) * ok[:, None]
    d = g[:, None] * onehot - g[:, None] * p
    d[~ok] = 0.0
    return d + 0.0


# ----------------------------------------------------------------------------- logits-only op
def logp_fwd(z, t):
    """Logits-only forward: (logp [N], lse [N]) from given logits [N, V]."""
    z = _as64(z)
    if z.shape[0] == 0:
        return np.zeros(0, F64), np.zeros(0, F64)
    lse = row_logsumexp(z)
    return target_logp(z, lse, t), lse


def logp_bwd(z, t, g):
    """Logits-only backward: dlogits [N, V] = g (onehot - softmax)."""
    z = _as64(z)
    if z.shape[0] == 0:
        return np.zeros(z.shape, F64)
    lse = row_logsumexp(z)
    return softmax_grad(z, lse, t, g)
