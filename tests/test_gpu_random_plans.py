"""Seeded random plans against the oracle: kind, d, heads, batch, gate order, fused or split
mode, per-head (GDN) or per-row (KDA) widths from {2, 4, 6, 8}, FP16 pivot heads or rows (none,
a few, many, or a whole head), contrast geometry.  Each plan encodes an oracle warm-up state and
runs two decode steps; every tile of every step must match the oracle (codes bit-exact up to the
documented .5-boundary exemption, readouts within rel L2 1e-4).  STEPQ_RANDOM_PLANS sets the
number of plans (default 48) for a longer sweep."""
import os

import numpy as np
import pytest

import paritylib as P
from quantized_delta_rule_amd import synth

pytestmark = pytest.mark.gpu

N_PLANS = int(os.environ.get("STEPQ_RANDOM_PLANS", "48"))


@pytest.fixture(scope="module")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from quantized_delta_rule_amd import stepq
    stepq.lib()
    return torch


def _random_case(seed):
    g = np.random.default_rng(9000 + seed)
    kind = "gdn" if seed % 2 == 0 else "kda"
    d = int(g.choice([64, 128]))
    H = int(g.integers(1, 5))
    B = int(g.integers(1, 7))
    order = int(g.integers(0, 2))
    mode = int(g.integers(0, 2))
    contrast = bool(g.integers(0, 2))
    if kind == "gdn":
        fixed = tuple(int(x) for x in g.choice([2, 4, 6, 8, 0], size=H))
        w = synth.Workload(800 + seed, f"rand-{seed}", kind, B=B, layers=1, H=H, d=d, steps=2,
                           warmup=6, choices=(2, 4, 6, 8), nominal=6, n_pivots=0, alloc="fixed",
                           fixed_bits=fixed, contrast=contrast, order=order)
        bits, piv, om = [a[0] for a in P.oracle_plan(w)]
        return w, bits, piv, om, mode
    w = synth.Workload(800 + seed, f"rand-{seed}", kind, B=B, layers=1, H=H, d=d, steps=2,
                       warmup=6, choices=(2, 4, 6, 8), nominal=6, n_pivots=0, alloc="fixed",
                       contrast=contrast, order=order)
    bits = g.choice([2, 4, 6, 8], size=(H, d)).astype(np.int8)
    piv = np.zeros((H, d), np.uint8)
    for h in range(H):
        style = g.integers(0, 5)
        if style == 1:        # a few pivot rows
            piv[h, g.choice(d, size=3, replace=False)] = 1
        elif style == 2:      # many
            piv[h, g.random(d) < 0.3] = 1
        elif style == 3:      # one width for the whole head
            bits[h] = g.choice([2, 4, 6, 8])
        elif style == 4 and H > 1 and h == H - 1:  # every row a pivot
            piv[h] = 1
    om = P.omega_from_steps(w, 0, "warmup", w.warmup)
    return w, bits, piv, om, mode


@pytest.mark.parametrize("seed", range(N_PLANS))
def test_random_plan_matches_oracle(gpu, seed):
    w, bits, piv, om, mode = _random_case(seed)
    P.log(f"[random] seed {seed}: {w.kind} d={w.d} H={w.H} B={w.B} order={w.order} "
          f"mode={'split' if mode else 'fused'} contrast={w.contrast} "
          f"pivots={int(piv.sum())} widths={sorted(set(bits[piv == 0].tolist()))}")
    tr, plan, _ = P.run_layer(w, 0, bits, piv, om, w.steps, mode=mode)
    assert tr.worst_readout <= P.READOUT_TOL
    assert plan.status() == 0
