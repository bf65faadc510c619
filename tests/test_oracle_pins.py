"""Pins of the FP64 oracle to facts other than itself.

Each test checks the oracle against something the pages or the mathematics
fix: closed forms, invariants, central finite differences, special cases, a
hand-derived example and an independent library routine (torch's float64
log_softmax with autograd). Together they are chosen so that a plausible
mistake in the oracle (a dropped term, a wrong sign or index, a transposed
operand, a missing max shift, a bias left out, an out-of-range target not
zeroed) fails at least one of them. CPU only.
"""

import math

import numpy as np
import pytest

from oracle import linear_logp as O

RNG = np.random.default_rng(1234)


def _rand_case(N, D, V, bias=True, scale_w=0.5, seed=0):
    r = np.random.default_rng(seed)
    h = r.standard_normal((N, D))
    W = r.standard_normal((V, D)) * scale_w
    b = r.standard_normal(V) * 0.3 if bias else None
    t = r.integers(0, V, N)
    g = r.standard_normal(N)
    return h, W, b, t, g


# ----------------------------------------------------------------------------- closed forms
@pytest.mark.parametrize("V", [1, 7, 1000])
def test_zero_weight_gives_uniform_softmax(V):
    # W = 0, b = 0: every logit is 0, so lse = ln V and logp = -ln V exactly.
    h = RNG.standard_normal((5, 3))
    W = np.zeros((V, 3))
    t = RNG.integers(0, V, 5)
    logp, lse = O.linear_logp_fwd(h, W, None, t)
    np.testing.assert_allclose(lse, math.log(V), rtol=0, atol=1e-13)
    np.testing.assert_allclose(logp, -math.log(V), rtol=0, atol=1e-13)


def test_zero_hidden_reduces_to_bias_softmax():
    # h = 0, b = (0, 0, ln 2, ln 4): exp(b) sums to 8, so lse = ln 8 and
    # logp(t) = b_t - ln 8: t = 3 -> -ln 2, t = 0 -> -ln 8, t = 2 -> -ln 4.
    b = np.array([0.0, 0.0, math.log(2), math.log(4)])
    h = np.zeros((3, 2))
    W = RNG.standard_normal((4, 2))
    t = np.array([3, 0, 2])
    logp, lse = O.linear_logp_fwd(h, W, b, t)
    np.testing.assert_allclose(lse, math.log(8), atol=1e-14)
    np.testing.assert_allclose(logp, [-math.log(2), -math.log(8), -math.log(4)], atol=1e-14)


def test_single_token_vocab():
    # V = 1: softmax is 1, so logp = 0 and every gradient is 0.
    h, W, b, _, g = _rand_case(4, 3, 1)
    t = np.zeros(4, dtype=np.int64)
    logp, lse = O.linear_logp_fwd(h, W, b, t)
    np.testing.assert_allclose(logp, 0.0, atol=1e-15)
    dH, dW, db = O.linear_logp_bwd(h, W, b, t, g, True, True, True)
    assert np.all(np.abs(dH) < 1e-15) and np.all(np.abs(dW) < 1e-15) and np.all(np.abs(db) < 1e-15)


def test_large_logits_need_the_max_shift():
    # z = (1000, 1000 + ln 3): exp overflows without the max shift, but
    # lse = 1000 + ln 4 and logp(1) = ln 3 - ln 4 in closed form.
    z = np.array([[1000.0, 1000.0 + math.log(3)]])
    logp, lse = O.logp_fwd(z, np.array([1]))
    assert np.isfinite(lse).all()
    np.testing.assert_allclose(lse, 1000.0 + math.log(4), rtol=1e-15)
    np.testing.assert_allclose(logp, math.log(3) - math.log(4), atol=1e-12)
    d = O.logp_bwd(z, np.array([1]), np.array([2.0]))
    np.testing.assert_allclose(d, [[-2 * 0.25, 2 * 0.25]], atol=1e-12)


def test_hand_derived_example():
    # Worked by hand from the definitions (N = 2, D = 2, V = 3, with bias):
    #   W rows (1, 0), (0, 1), (0, 0); b = (0, 0, ln 2)
    #   token 0: h = (ln 2, 0), t = 1, g = 1  -> z = (ln 2, 0, ln 2), exp sums to 5
    #   token 1: h = (0, ln 3), t = 2, g = -2 -> z = (0, ln 3, ln 2), exp sums to 6
    # so lse = (ln 5, ln 6), logp = (-ln 5, -ln 3),
    # p0 = (2, 1, 2)/5, p1 = (1, 3, 2)/6,
    # dlogits0 = 1 * ((0,1,0) - p0) = (-2/5, 4/5, -2/5),
    # dlogits1 = -2 * ((0,0,1) - p1) = (1/3, 1, -4/3),
    # dH = dlogits W, dW = dlogits^T h, db = column sums.
    l2, l3 = math.log(2), math.log(3)
    W = np.array([[1.0, 0.0], [0.0, 1.0], [0.0, 0.0]])
    b = np.array([0.0, 0.0, l2])
    h = np.array([[l2, 0.0], [0.0, l3]])
    t = np.array([1, 2])
    g = np.array([1.0, -2.0])
    logp, lse = O.linear_logp_fwd(h, W, b, t)
    np.testing.assert_allclose(lse, [math.log(5), math.log(6)], atol=1e-14)
    np.testing.assert_allclose(logp, [-math.log(5), -l3], atol=1e-14)
    dH, dW, db = O.linear_logp_bwd(h, W, b, t, g, True, True, True)
    np.testing.assert_allclose(dH, [[-2 / 5, 4 / 5], [1 / 3, 1.0]], atol=1e-14)
    np.testing.assert_allclose(
        dW, [[-(2 / 5) * l2, l3 / 3], [(4 / 5) * l2, l3], [-(2 / 5) * l2, -(4 / 3) * l3]], atol=1e-14)
    np.testing.assert_allclose(db, [-1 / 15, 9 / 5, -26 / 15], atol=1e-14)


# ----------------------------------------------------------------------------- invariants
def test_softmax_rows_sum_to_one_and_dlogits_rows_to_zero():
    z = RNG.standard_normal((6, 151936)) * 2.0
    lse = O.row_logsumexp(z)
    p = np.exp(z - lse[:, None])
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-10
    t = RNG.integers(0, z.shape[1], 6)
    d = O.softmax_grad(z, lse, t, np.ones(6))
    assert np.max(np.abs(d.sum(axis=1))) < 1e-10


def test_bias_shift_invariance():
    h, W, b, t, g = _rand_case(5, 4, 9)
    logp0, _ = O.linear_logp_fwd(h, W, b, t)
    logp1, _ = O.linear_logp_fwd(h, W, b + 3.25, t)
    np.testing.assert_allclose(logp0, logp1, atol=1e-13)
    r0 = O.linear_logp_bwd(h, W, b, t, g, True, True, True)
    r1 = O.linear_logp_bwd(h, W, b + 3.25, t, g, True, True, True)
    for a, c in zip(r0, r1):
        np.testing.assert_allclose(a, c, atol=1e-13)


def test_gradient_tables_sum_to_zero_over_vocab():
    # sum_v dlogits = 0 per row, hence sum_v dW[v, d] = 0 and sum_v db = 0.
    h, W, b, t, g = _rand_case(16, 6, 33)
    _, dW, db = O.linear_logp_bwd(h, W, b, t, g, False, True, True)
    assert np.max(np.abs(dW.sum(axis=0))) < 1e-12
    assert abs(db.sum()) < 1e-12


def test_equal_weight_rows_give_zero_dH():
    # All W rows equal: dH = (sum_v dlogits) w = 0.
    h, _, b, t, g = _rand_case(4, 5, 7)
    W = np.tile(RNG.standard_normal(5), (7, 1))
    dH, _, _ = O.linear_logp_bwd(h, W, b, t, g, True, False, False)
    assert np.max(np.abs(dH)) < 1e-13


def test_power_of_two_upstream_scaling_is_exact():
    h, W, b, t, g = _rand_case(5, 4, 11)
    r0 = O.linear_logp_bwd(h, W, b, t, g, True, True, True)
    r1 = O.linear_logp_bwd(h, W, b, t, g * 2.0 ** -14, True, True, True)
    for a, c in zip(r0, r1):
        np.testing.assert_array_equal(a * 2.0 ** -14, c)


# ----------------------------------------------------------------------------- finite differences
def _objective(h, W, b, t, g):
    logp, _ = O.linear_logp_fwd(h, W, b, t)
    return float(np.dot(g, logp))


def _central_diff(f, x):
    out = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        eps = 1e-6 * max(1.0, abs(x[i]))
        old = x[i]
        x[i] = old + eps
        fp = f()
        x[i] = old - eps
        fm = f()
        x[i] = old
        out[i] = (fp - fm) / (2 * eps)
    return out


@pytest.mark.parametrize("N,D,V,bias", [(3, 4, 5, True), (3, 4, 1, True), (4, 3, 6, False)])
def test_gradients_match_central_differences(N, D, V, bias):
    h, W, b, t, g = _rand_case(N, D, V, bias, seed=N * 100 + V)
    dH, dW, db = O.linear_logp_bwd(h, W, b, t, g, True, True, bias)
    f = lambda: _objective(h, W, b, t, g)  # noqa: E731
    np.testing.assert_allclose(dH, _central_diff(f, h), atol=2e-8, rtol=1e-6)
    np.testing.assert_allclose(dW, _central_diff(f, W), atol=2e-8, rtol=1e-6)
    if bias:
        np.testing.assert_allclose(db, _central_diff(f, b), atol=2e-8, rtol=1e-6)


def test_logits_only_gradient_matches_central_differences():
    r = np.random.default_rng(7)
    z = r.standard_normal((3, 6)) * 2
    t = np.array([0, 5, 2])
    g = r.standard_normal(3)
    d = O.logp_bwd(z, t, g)
    f = lambda: float(np.dot(g, O.logp_fwd(z, t)[0]))  # noqa: E731
    np.testing.assert_allclose(d, _central_diff(f, z), atol=2e-8, rtol=1e-6)


# ----------------------------------------------------------------------------- special cases
@pytest.mark.parametrize("g0", [0.0, -0.0])
def test_zero_upstream_gives_positive_zero_gradients(g0):
    h, W, b, t, _ = _rand_case(6, 5, 8)
    g = np.full(6, g0)
    dH, dW, db = O.linear_logp_bwd(h, W, b, t, g, True, True, True)
    for x in (dH, dW, db):
        assert np.all(x == 0) and not np.any(np.signbit(x))


def test_out_of_range_targets_give_zero_logp_and_zero_rows():
    h, W, b, t, g = _rand_case(6, 4, 10)
    t_bad = t.copy()
    t_bad[[1, 3, 4]] = [-100, 10, 15]
    logp, lse = O.linear_logp_fwd(h, W, b, t_bad)
    logp_ok, lse_ok = O.linear_logp_fwd(h, W, b, t)
    assert np.all(logp[[1, 3, 4]] == 0) and not np.any(np.signbit(logp[[1, 3, 4]]))
    np.testing.assert_array_equal(logp[[0, 2, 5]], logp_ok[[0, 2, 5]])
    np.testing.assert_array_equal(lse, lse_ok)  # lse is reported for every row
    z = O.logits(h, W, b)
    d = O.softmax_grad(z, lse, t_bad, g)
    assert np.all(d[[1, 3, 4]] == 0) and not np.any(np.signbit(d[[1, 3, 4]]))
    d_ok = O.softmax_grad(z, lse, t, g)
    np.testing.assert_array_equal(d[[0, 2, 5]], d_ok[[0, 2, 5]])


def test_empty_batch():
    _, W, b, _, _ = _rand_case(1, 4, 9)
    h = np.zeros((0, 4))
    t = np.zeros(0, dtype=np.int64)
    logp, lse = O.linear_logp_fwd(h, W, b, t)
    assert logp.shape == (0,) and lse.shape == (0,)
    dH, dW, db = O.linear_logp_bwd(h, W, b, t, np.zeros(0), True, True, True)
    assert dH.shape == (0, 4)
    assert dW.shape == (9, 4) and np.all(dW == 0) and not np.any(np.signbit(dW))
    assert db.shape == (9,) and np.all(db == 0) and not np.any(np.signbit(db))


def test_masked_negative_infinity_tail_stays_finite():
    r = np.random.default_rng(3)
    z = r.standard_normal((4, 12))
    z[:, 8:] = -np.inf
    t = np.array([0, 3, 7, 2])
    g = r.standard_normal(4)
    logp, lse = O.logp_fwd(z, t)
    assert np.isfinite(logp).all() and np.isfinite(lse).all()
    ref_logp, ref_lse = O.logp_fwd(z[:, :8], t)
    np.testing.assert_allclose(logp, ref_logp, atol=1e-14)
    d = O.logp_bwd(z, t, g)
    assert np.isfinite(d).all() and np.all(d[:, 8:] == 0) and not np.any(np.signbit(d[:, 8:]))


def test_accumulate_adds_the_callers_table_last():
    h, W, b, t, g = _rand_case(5, 3, 7)
    dW0 = RNG.standard_normal((7, 3))
    db0 = RNG.standard_normal(7)
    _, dW, db = O.linear_logp_bwd(h, W, b, t, g, False, True, True)
    _, dWa, dba = O.linear_logp_bwd(h, W, b, t, g, False, True, True, dW0=dW0, db0=db0)
    np.testing.assert_array_equal(dWa, dW + dW0)
    np.testing.assert_array_equal(dba, db + db0)


def test_sampled_helpers_equal_the_full_definition():
    h, W, b, t, g = _rand_case(37, 6, 29, seed=11)
    logp, lse = O.linear_logp_fwd(h, W, b, t)
    dH, dW, db = O.linear_logp_bwd(h, W, b, t, g, True, True, True)
    rows = np.array([0, 5, 36])
    lp, ls, dh = O.linear_logp_token_rows(h[rows], W, b, t[rows], g[rows])
    np.testing.assert_allclose(lp, logp[rows], atol=1e-14)
    np.testing.assert_allclose(ls, lse[rows], atol=1e-14)
    np.testing.assert_allclose(dh, dH[rows], atol=1e-14)
    vr = np.array([0, 13, 28])
    dw, dbb = O.linear_logp_vocab_rows(h, W, b, t, g, vr, token_block=8)
    np.testing.assert_allclose(dw, dW[vr], atol=1e-13)
    np.testing.assert_allclose(dbb, db[vr], atol=1e-13)
    # with every token's lse passed in (blocked evaluation), the same rows;
    # out-of-range targets and g = 0 rows keep their +0 columns there too
    ls_all = O.linear_lse(h, W, b, token_block=5)
    np.testing.assert_allclose(ls_all, lse, atol=1e-14)
    t2 = t.copy()
    t2[[1, 4]] = [-100, 29]
    g2 = g.copy()
    g2[7] = 0.0
    vr2 = np.array([0, int(t[3]), 13, 28])
    _, dW2, db2 = O.linear_logp_bwd(h, W, b, t2, g2, False, True, True)
    dw, dbb = O.linear_logp_vocab_rows(h, W, b, t2, g2, vr2, token_block=8, lse=ls_all)
    np.testing.assert_allclose(dw, dW2[vr2], atol=1e-13)
    np.testing.assert_allclose(dbb, db2[vr2], atol=1e-13)
    dw0, _ = O.linear_logp_vocab_rows(h, W, b, t2, np.zeros_like(g2), vr2, lse=ls_all)
    assert np.all(dw0 == 0) and not np.signbit(dw0).any()


def test_logits_only_equals_linear_on_the_same_logits():
    h, W, b, t, g = _rand_case(7, 5, 13)
    z = O.logits(h, W, b)
    np.testing.assert_allclose(O.logp_fwd(z, t)[0], O.linear_logp_fwd(h, W, b, t)[0], atol=1e-14)
    dH, _, db = O.linear_logp_bwd(h, W, b, t, g, True, False, True)
    d = O.logp_bwd(z, t, g)
    np.testing.assert_allclose(d @ W, dH, atol=1e-14)
    np.testing.assert_allclose(d.sum(axis=0), db, atol=1e-14)


# ----------------------------------------------------------------------------- library routine
def test_agrees_with_torch_float64_log_softmax_and_autograd():
    torch = pytest.importorskip("torch")
    for (N, D, V, bias) in [(9, 7, 31, True), (4, 16, 255, False), (1, 3, 2, True)]:
        h, W, b, t, g = _rand_case(N, D, V, bias, seed=N + V)
        th = torch.tensor(h, requires_grad=True)
        tW = torch.tensor(W, requires_grad=True)
        tb = torch.tensor(b, requires_grad=True) if bias else None
        z = torch.nn.functional.linear(th, tW, tb)
        lp = torch.log_softmax(z, dim=-1).gather(1, torch.tensor(t)[:, None])[:, 0]
        (lp * torch.tensor(g)).sum().backward()
        logp, _ = O.linear_logp_fwd(h, W, b, t)
        dH, dW, db = O.linear_logp_bwd(h, W, b, t, g, True, True, bias)
        np.testing.assert_allclose(logp, lp.detach().numpy(), atol=1e-12)
        np.testing.assert_allclose(dH, th.grad.numpy(), atol=1e-12)
        np.testing.assert_allclose(dW, tW.grad.numpy(), atol=1e-12)
        if bias:
            np.testing.assert_allclose(db, tb.grad.numpy(), atol=1e-12)


# ----------------------------------------------------------------------------- planted mistakes
def test_pins_catch_planted_mistakes(monkeypatch):
    """Each plausible oracle mistake, planted on the CPU, fails a pin above."""
    h, W, b, t, g = _rand_case(3, 4, 5, True, seed=305)

    def fd_ok():
        dH, dW, db = O.linear_logp_bwd(h, W, b, t, g, True, True, True)
        f = lambda: _objective(h, W, b, t, g)  # noqa: E731
        return (np.allclose(dH, _central_diff(f, h), atol=2e-8, rtol=1e-6)
                and np.allclose(dW, _central_diff(f, W), atol=2e-8, rtol=1e-6)
                and np.allclose(db, _central_diff(f, b), atol=2e-8, rtol=1e-6))

    assert fd_ok()
    good = O.softmax_grad
    # dropped one-hot term
    monkeypatch.setattr(O, "softmax_grad", lambda z, lse, t_, g_: good(z, lse, np.full_like(t_, -1), g_) * 0
                        - g_[:, None] * np.exp(z - lse[:, None]))
    assert not fd_ok()
    # wrong sign
    monkeypatch.setattr(O, "softmax_grad", lambda z, lse, t_, g_: -good(z, lse, t_, g_))
    assert not fd_ok()
    monkeypatch.setattr(O, "softmax_grad", good)
    # target index off by one
    good_tl = O.target_logp
    monkeypatch.setattr(O, "target_logp", lambda z, lse, t_: good_tl(z, lse, (t_ + 1) % z.shape[1]))
    assert not fd_ok()
    monkeypatch.setattr(O, "target_logp", good_tl)
    # logsumexp without the max shift overflows on large logits
    monkeypatch.setattr(O, "row_logsumexp", lambda z: np.log(np.exp(np.asarray(z, float)).sum(axis=1)))
    with np.errstate(over="ignore"):
        _, lse = O.logp_fwd(np.array([[1000.0, 1000.0 + math.log(3)]]), np.array([1]))
    assert not np.isfinite(lse).all()
