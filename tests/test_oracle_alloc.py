"""Pins for the oracle's offline inputs (Method 1 and Method 2): the lifetime weight against its
geometric closed form, the multiple-choice DP against brute force, the Lagrangian allocation
against the DP optimum, pivot choice, and row impact against closed forms."""
import itertools

import numpy as np
import pytest


def test_lifetime_weight_closed_form(orc):
    l = np.array([-0.2, -0.05, -0.001, -1e-6, -3.0])
    H = 512
    got = orc.lifetime_weight(l, H)
    ref = (1 - np.exp(2 * H * l)) / (1 - np.exp(2 * l))
    assert np.allclose(got, ref, rtol=1e-12)
    assert abs(orc.lifetime_weight(np.array([0.0]), H)[0] - H) < 1e-9   # no decay: H steps
    assert orc.lifetime_weight(np.array([-50.0]), H)[0] == pytest.approx(1.0)


def _brute(cost, choices, cap_bits):
    best, arg = None, None
    for combo in itertools.product(range(len(choices)), repeat=cost.shape[0]):
        bits = sum(choices[c] for c in combo)
        if bits > cap_bits:
            continue
        val = sum(cost[u, c] for u, c in enumerate(combo))
        if best is None or val < best - 1e-12 * abs(best):
            best, arg = val, combo
    return best, arg


@pytest.mark.parametrize("seed", range(40))
def test_mcdp_equals_brute_force(orc, seed):
    g = np.random.default_rng(seed)
    N = int(g.integers(1, 7))
    choices = [2, 4, 6, 8] if seed % 2 else [4, 6, 8]
    L = orc.lifetime_weight(g.uniform(-0.2, -0.001, N), 512)
    s = g.lognormal(0, 1, N)
    cost = L[:, None] * s[:, None] * np.exp2(-2.0 * np.array(choices))[None, :]
    if seed % 5 == 0:   # adversarial: equal costs everywhere
        cost[:] = 1.0
    nominal = 4 if seed % 2 else 6
    cap = nominal * N + int(g.integers(-2, 3)) * 2
    cap = max(cap, min(choices) * N)
    bits, obj = orc.mcdp_allocate(cost, choices, cap)
    best, arg = _brute(cost, choices, cap)
    assert sum(bits) <= cap
    assert obj == pytest.approx(best, rel=1e-12)
    assert orc.objective(np.ones(N), cost, choices, bits) == pytest.approx(best, rel=1e-12)
    if seed % 5 == 0:   # ties go to fewer bits
        assert sum(bits) == min(choices) * N


@pytest.mark.parametrize("seed", range(10))
def test_lagrangian_feasible_and_not_better_than_dp(orc, seed):
    g = np.random.default_rng(1000 + seed)
    N = 40
    choices = [4, 6, 8]
    L = orc.lifetime_weight(g.uniform(-0.2, -0.001, N), 512)
    s = g.lognormal(0, 1, N)
    d = s[:, None] * np.exp2(-2.0 * np.array(choices))[None, :]
    n = np.full(N, 128.0)
    budget = 6 * float(n.sum())
    b, obj = orc.lagrangian_allocate(L, d, n, choices, budget)
    assert float(np.sum(n * b)) <= budget
    b_dp, obj_dp = orc.mcdp_allocate(L[:, None] * d, choices, 6 * N)
    assert obj >= obj_dp * (1 - 1e-12)
    assert obj <= obj_dp * 1.5          # close to optimal on these instances
    # repaired: no single upgrade fits any more with a positive gain
    left = budget - float(np.sum(n * b))
    assert all(bb == 8 or n[u] * 2 > left for u, bb in enumerate(b))


def test_pivot_selection(orc):
    risk = np.array([3.0, 7.0, 7.0, 1.0, 9.0])
    assert list(orc.select_pivots(risk, 2)) == [1, 4]      # tie at 7: lower index wins
    assert list(orc.select_pivots(risk, 0)) == []


def test_row_impact_closed_forms(orc):
    g = np.random.default_rng(3)
    n, d = 500, 16
    q = g.standard_normal((n, d))
    k = g.standard_normal((n, d))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    a = g.uniform(0.8, 1.0, (n, d))
    beta = g.uniform(0, 1, n)
    # beta = 0: g = a*q
    assert np.allclose(orc.row_impact(q, k, a, np.zeros(n)), np.mean((a * q) ** 2, 0))
    # against the explicit matrix A_t^T q_t
    om = orc.row_impact(q, k, a, beta)
    ref = np.zeros(d)
    for t in range(n):
        A = np.diag(a[t]) @ (np.eye(d) - beta[t] * np.outer(k[t], k[t]))
        ref += (A.T @ q[t]) ** 2
    assert np.allclose(om, ref / n, rtol=1e-12)
    # the other gate order, A = (I - beta k k^T) Diag(a)
    om2 = orc.row_impact(q, k, a, beta, order=orc.DECAY_FIRST)
    ref2 = np.zeros(d)
    for t in range(n):
        A = (np.eye(d) - beta[t] * np.outer(k[t], k[t])) @ np.diag(a[t])
        ref2 += (A.T @ q[t]) ** 2
    assert np.allclose(om2, ref2 / n, rtol=1e-12)
    assert not np.allclose(om2, om, rtol=1e-3)
    # a scalar gate commutes with the delta update: both orders give the same impact
    a1 = np.repeat(a[:, :1], d, axis=1)
    assert np.allclose(orc.row_impact(q, k, a1, beta, order=orc.DECAY_FIRST),
                       orc.row_impact(q, k, a1, beta), rtol=1e-12)
