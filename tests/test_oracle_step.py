"""Pins for the oracle's decode step against the mathematics of the delta rule:
identity step (alpha = 1, beta = 0), exact retrieval with orthonormal keys in FP32-state mode,
the update against the binary64 formula S <- Diag(a)(I - beta k k^T) S + beta k v^T, and the
error-propagation identity of the readout (Background, "why plain INT8 is still not stable":
output error = E_{t-1}^T A_t^T q_t)."""
import numpy as np
import pytest


def _unit(g, n):
    x = g.standard_normal(n)
    return (x / np.linalg.norm(x)).astype(np.float32)


def _make(orc, g, d, kda):
    bits = (g.choice([4, 6, 8], size=d) if kda else np.full(d, 6)).astype(np.int8)
    piv = np.zeros(d, np.uint8)
    if kda:
        piv[g.choice(d, 2, replace=False)] = 1
    head = orc.Head(bits, piv, g.exponential(1.0, d).astype(np.float32))
    S0 = (g.standard_normal((d, d)) * 0.3).astype(np.float32)
    return head, head.encode(S0)


@pytest.mark.parametrize("kda", [False, True])
def test_identity_step(orc, kda):
    g = np.random.default_rng(21)
    d = 128
    head, seg = _make(orc, g, d, kda)
    S_hat, _, _, _ = head.unpack(seg)
    q, k, v = _unit(g, d), _unit(g, d), g.standard_normal(d).astype(np.float32)
    out, S_upd, _, _ = head.step(seg.copy(), q, k, v, np.ones(d, np.float32), 0.0,
                                 want_state=True)
    assert np.array_equal(S_upd, S_hat)                 # bit for bit
    ref = S_hat.astype(np.float64).T @ q.astype(np.float64)
    bound = 12 * 2.0 ** -24 * (np.abs(S_hat.astype(np.float64)).T @ np.abs(q))
    assert np.all(np.abs(out - ref) <= bound)


def test_orthonormal_retrieval_fp32_state(orc):
    g = np.random.default_rng(22)
    d = 128
    Q, _ = np.linalg.qr(g.standard_normal((d, d)))
    keys = Q.T.astype(np.float32)        # rows: orthonormal keys (rounded to binary32)
    vals = g.standard_normal((d, d)).astype(np.float32)
    for m in (1, 17, 64, 128):
        S = np.zeros((d, d), np.float32)
        for i in range(m):
            orc.fp32_step(S, keys[i], keys[i], vals[i], np.ones(d, np.float32), 1.0)
        for i in range(m):
            got = S.T.astype(np.float64) @ keys[i].astype(np.float64)
            rel = np.linalg.norm(got - vals[i]) / np.linalg.norm(vals[i])
            assert rel <= 1e-5, (m, i, rel)


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("kda", [False, True])
def test_update_matches_binary64_formula(orc, kda, order):
    """Both gate orders against the matrix formula in binary64: order 0 (delta update first,
    A = Diag(a)(I - beta k k^T)) and order 1 (rows decay first, A = (I - beta k k^T) Diag(a))."""
    g = np.random.default_rng(23)
    d = 128
    head, seg = _make(orc, g, d, kda)
    head.order = order
    S_hat, _, _, _ = head.unpack(seg)
    q, k, v = _unit(g, d), _unit(g, d), g.standard_normal(d).astype(np.float32)
    a = (g.uniform(0.8, 1.0, d) if kda else np.full(d, 0.97)).astype(np.float32)
    beta = np.float32(0.6)
    out, S_upd, _, _ = head.step(seg.copy(), q, k, v, a, beta, want_state=True)
    S64, k64, q64 = S_hat.astype(np.float64), k.astype(np.float64), q.astype(np.float64)
    Da = np.diag(a.astype(np.float64))
    P_ = np.eye(d) - float(beta) * np.outer(k64, k64)
    A, A_other = (Da @ P_, P_ @ Da) if order == 0 else (P_ @ Da, Da @ P_)
    ref = A @ S64 + float(beta) * np.outer(k64, v.astype(np.float64))
    scale = np.abs(S64).max() + 1
    assert np.max(np.abs(S_upd - ref)) <= 1e-5 * scale
    # the other gate order is measurably different for a per-row gate (KDA)
    if kda:
        alt = A_other @ S64 + float(beta) * np.outer(k64, v)
        assert np.max(np.abs(S_upd - alt)) > 1e-3 * np.max(np.abs(ref - S64))
    assert np.max(np.abs(out - ref.T @ q64)) <= 1e-5 * scale


def test_gate_orders_agree_for_a_scalar_gate(orc):
    """With one gate for all rows (GDN) the two orders are the same map: their binary32 results
    differ only by rounding, and FP32-state runs stay together."""
    g = np.random.default_rng(29)
    d = 64
    S1 = (g.standard_normal((d, d)) * 0.3).astype(np.float32)
    S2 = S1.copy()
    for t in range(20):
        q, k, v = _unit(g, d), _unit(g, d), g.standard_normal(d).astype(np.float32)
        a = np.full(d, g.uniform(0.9, 1.0), np.float32)
        beta = np.float32(g.uniform(0.2, 0.9))
        o1 = orc.fp32_step(S1, q, k, v, a, beta, order=0)
        o2 = orc.fp32_step(S2, q, k, v, a, beta, order=1)
        assert np.max(np.abs(o1 - o2)) <= 1e-5 * (np.abs(o1).max() + 1)
    assert np.max(np.abs(S1 - S2)) <= 1e-5 * (np.abs(S1).max() + 1)
    assert not np.array_equal(S1, S2)  # the rounding does differ


@pytest.mark.parametrize("kda", [False, True])
def test_readout_error_propagation_identity(orc, kda):
    """Quantized run vs exact (binary64, unquantized) run from the same decoded start:
    o_t - o*_t = E_{t-1}^T A_t^T q_t with E = S_hat - S*, to binary32 rounding."""
    g = np.random.default_rng(24)
    d = 128
    head, seg = _make(orc, g, d, kda)
    S_hat, _, _, _ = head.unpack(seg)
    S_star = S_hat.astype(np.float64)
    for t in range(12):
        q, k, v = _unit(g, d), _unit(g, d), g.standard_normal(d).astype(np.float32)
        a = (g.uniform(0.8, 1.0, d) if kda else np.full(d, g.uniform(0.9, 1.0))).astype(
            np.float32)
        beta = np.float32(g.uniform(0.2, 0.9))
        k64, q64, a64 = k.astype(np.float64), q.astype(np.float64), a.astype(np.float64)
        A = np.diag(a64) @ (np.eye(d) - float(beta) * np.outer(k64, k64))
        E_prev = S_hat.astype(np.float64) - S_star
        out = head.step(seg, q, k, v, a, beta)
        S_star = A @ S_star + float(beta) * np.outer(k64, v.astype(np.float64))
        o_star = S_star.T @ q64
        pred = o_star + E_prev.T @ (A.T @ q64)
        assert np.max(np.abs(out - pred)) <= 2e-5 * (1 + np.abs(pred).max())
        S_hat, _, _, _ = head.unpack(seg)
    # the requantization error is genuinely present (the identity is not vacuous)
    assert np.max(np.abs(S_hat - S_star)) > 1e-4


def test_alpha_one_beta_zero_decoded_state_is_stable(orc):
    """alpha = 1, beta = 0 leaves the dequantized state invariant through the step; the refit
    then moves entries by at most about one quantization step."""
    g = np.random.default_rng(25)
    d = 64
    head, seg = _make(orc, g, d, False)
    S_hat, r16, c16, _ = head.unpack(seg)
    out, S_upd, pre, _ = head.step(seg, _unit(g, d), _unit(g, d), np.zeros(d, np.float32),
                                   np.ones(d, np.float32), 0.0, want_state=True)
    assert np.array_equal(S_upd, S_hat)
    S2, r2, c2, _ = head.unpack(seg)
    step_new = r2.view(np.float16).astype(np.float64)[:, None] * \
        c2.view(np.float16).astype(np.float64)[None, :]
    assert np.all(np.abs(S2 - S_hat) <= 0.5 * step_new * (1 + 1e-5) + 1e-30)
