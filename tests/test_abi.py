"""C-ABI checks that need no GPU: the library loads, exports every function stepq.h declares,
rejects invalid plans before touching a device, and its host-side planners agree with the
oracle's."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sq():
    from quantized_delta_rule_amd import stepq
    stepq.lib()
    return stepq


def declared():
    src = open(os.path.join(ROOT, "include", "stepq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(stepq_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(sq):
    names = declared()
    assert len(names) >= 15
    L = ctypes.CDLL(sq.LIB_PATH)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def _desc(sq, **kw):
    H, d = kw.pop("H", 2), kw.pop("d", 128)
    bits = kw.pop("bits", np.full((H, d), 6, np.int8))
    piv = kw.pop("pivot", np.zeros((H, d), np.uint8))
    om = kw.pop("omega", np.ones((H, d), np.float32))
    kind = kw.pop("kind", sq.GDN)
    return bits, piv, om, kind


@pytest.mark.parametrize("case", ["bits", "omega_nan", "omega_neg", "gdn_mixed", "gdn_partial_pivot",
                                  "d96", "pivot2", "order", "heads"])
def test_invalid_plans_are_rejected(sq, case):
    H, d = 2, 128
    bits = np.full((H, d), 6, np.int8)
    piv = np.zeros((H, d), np.uint8)
    om = np.ones((H, d), np.float32)
    kind = sq.GDN
    if case == "bits":
        bits[1, 3] = 5
    elif case == "omega_nan":
        om[0, 0] = np.nan
    elif case == "omega_neg":
        om[0, 0] = -1
    elif case == "gdn_mixed":
        bits[0, 7] = 4
    elif case == "gdn_partial_pivot":
        piv[0, :3] = 1
    elif case == "d96":
        bits, piv, om = bits[:, :96], piv[:, :96], om[:, :96]
    elif case == "pivot2":
        piv[0, 0] = 2
    elif case == "heads":  # the launch grid's second dimension holds the heads
        H, d = 65536, 64
        bits = np.full((H, d), 6, np.int8)
        piv = np.zeros((H, d), np.uint8)
        om = np.ones((H, d), np.float32)
    order = 2 if case == "order" else 0
    with pytest.raises(sq.StepqError) as ei:
        sq.Plan(kind, bits, piv, om, order=order)
    msg = str(ei.value)
    assert "(-1)" in msg or "(-2)" in msg, msg
    if case == "heads":
        assert "n_heads must be <= 65535" in msg, msg


def test_kda_allows_mixed_rows_until_the_device_check(sq):
    # a valid KDA description fails only at the device lookup on a machine without a GPU
    import torch
    if torch.cuda.is_available():
        pytest.skip("has a GPU")
    bits = np.tile(np.array([4, 6, 8, 2], np.int8), (2, 32))
    with pytest.raises(sq.StepqError, match="device 0 not available"):
        sq.Plan(sq.KDA, bits, np.zeros_like(bits, np.uint8), np.ones(bits.shape, np.float32))


def test_c_client_is_built_and_needs_a_device():
    # the plain-C client links the library and the HIP runtime; without a GPU it exits with 2
    import subprocess
    import torch
    if torch.cuda.is_available():
        pytest.skip("has a GPU (the client runs in tests/test_gpu_c_abi.py)")
    client = os.path.join(ROOT, "tests", "c", "abi_client")
    assert os.path.exists(client), "run __graft_entry__.build() first"
    res = subprocess.run([client], capture_output=True, text=True, timeout=60)
    assert res.returncode == 2 and "no GPU" in res.stderr, (res.returncode, res.stderr)


def test_lifetime_weights_match_oracle(sq, orc):
    l = np.random.default_rng(0).uniform(-0.2, -0.001, 200)
    l[0] = 0.0
    assert np.allclose(sq.lifetime_weights(l, 512), orc.lifetime_weight(l, 512), rtol=1e-12)


@pytest.mark.parametrize("order", [0, 1])
def test_row_impact_matches_oracle(sq, orc, order):
    g = np.random.default_rng(1)
    n, d = 64, 128
    q = g.standard_normal((n, d)).astype(np.float32)
    k = g.standard_normal((n, d)).astype(np.float32)
    a = g.uniform(0.8, 1, (n, d)).astype(np.float32)
    b = g.uniform(0, 1, n).astype(np.float32)
    acc = np.zeros(d)
    sq.row_impact_accumulate(q, k, a, b, acc, order=order)
    assert np.allclose(acc / n, orc.row_impact(q, k, a, b, order=order), rtol=1e-10)


def test_pivots_match_oracle(sq, orc):
    g = np.random.default_rng(2)
    risk = g.lognormal(0, 1, 500)
    risk[[10, 20, 30]] = risk.max() + 1      # a three-way tie at the top
    for n in (0, 1, 2, 8, 26):
        assert list(sq.select_pivots(risk, n)) == list(orc.select_pivots(risk, n))


@pytest.mark.parametrize("seed", range(12))
def test_mcdp_matches_oracle(sq, orc, seed):
    g = np.random.default_rng(seed)
    N = int(g.integers(1, 60))
    choices = [2, 4, 6, 8] if seed % 2 else [4, 6, 8]
    L = orc.lifetime_weight(g.uniform(-0.2, -0.001, N), 512)
    cost = L[:, None] * g.lognormal(0, 1, N)[:, None] * np.exp2(-2.0 * np.array(choices))
    cap = (4 if seed % 2 else 6) * N
    b1, o1 = sq.alloc_mcdp(cost, choices, cap)
    b2, o2 = orc.mcdp_allocate(cost, choices, cap)
    assert o1 == pytest.approx(o2, rel=1e-12)
    assert np.array_equal(b1, b2)


@pytest.mark.parametrize("seed", range(6))
def test_lagrangian_matches_oracle(sq, orc, seed):
    g = np.random.default_rng(100 + seed)
    N = 300
    choices = [4, 6, 8]
    L = orc.lifetime_weight(g.uniform(-0.2, -0.001, N), 512)
    d = g.lognormal(0, 1, N)[:, None] * np.exp2(-2.0 * np.array(choices))
    n = np.full(N, 128.0)
    b1, o1 = sq.alloc_lagrangian(L, d, n, choices, 6 * n.sum())
    b2, o2 = orc.lagrangian_allocate(L, d, n, choices, 6 * n.sum())
    assert o1 == pytest.approx(o2, rel=1e-12)
    assert np.array_equal(b1, b2)


def test_refused_planner_calls_report_their_own_message(sq):
    """A refused host planner call leaves its message in stepq_last_error (the one error slot
    of the library), and a successful call clears it."""
    L = sq.lib()
    cost = np.ones((3, 2))
    ch = np.array([4, 6], np.int32)
    out = np.zeros(3, np.int32)
    obj = ctypes.c_double()
    rc = L.stepq_alloc_mcdp(cost.ctypes.data, 3, ch.ctypes.data, 2, 2, out.ctypes.data,
                            ctypes.byref(obj))
    assert rc == -1 and "alloc_mcdp: budget below the narrowest width" in \
        L.stepq_last_error().decode()
    bad_ch = np.array([6, 4], np.int32)
    rc = L.stepq_alloc_mcdp(cost.ctypes.data, 3, bad_ch.ctypes.data, 2, 30, out.ctypes.data,
                            ctypes.byref(obj))
    assert rc == -1 and "ascending" in L.stepq_last_error().decode()
    l_u = np.array([0.5])
    Lw = np.zeros(1)
    assert L.stepq_lifetime_weights(l_u.ctypes.data, 1, 8, Lw.ctypes.data) == -1
    assert "l_u must be finite and <= 0" in L.stepq_last_error().decode()
    l_u[0] = -0.1
    assert L.stepq_lifetime_weights(l_u.ctypes.data, 1, 8, Lw.ctypes.data) == 0
    assert L.stepq_last_error().decode() == ""
    with pytest.raises(sq.StepqError, match="budget below"):
        sq.alloc_mcdp(cost, [4, 6], 2)
