"""Parity at the full sizes of the five synthetic workloads, in the launch configuration the
benchmark uses (one launch per layer and step over every tile).  The GPU runs every tile through
every step; the oracle follows a sample of tiles (every head at least once) through every step,
bit for bit, and a few of them also against the plain binary64 reference.

Workload 5 (12 layers x 256 requests x 48 heads, split mode, 128 steps): the oracle follows four
heads per layer (head h in layer h mod 12, so every head index in some layer) plus two random
tiles per layer, one of each layer's tiles against the plain reference each step, and layer 0
also runs a fused plan on the same inputs that must equal the split result bit for bit."""
import numpy as np
import pytest

import paritylib as P
from quantized_delta_rule_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from quantized_delta_rule_amd import stepq
    stepq.lib()
    return torch


@pytest.mark.parametrize("wid", [2, 3, 4])
def test_full_size_workload(gpu, wid):
    w = synth.WORKLOADS[wid]
    P.log(f"[parity] workload {wid} {w.name}: B={w.B} H={w.H} d={w.d} steps={w.steps}: plan")
    bits, piv, om = P.oracle_plan(w)
    tiles = P.sample_tiles(w, per_head=1, extra=8, seed=wid)
    P.log(f"[parity] workload {wid}: {len(tiles)} sampled tiles, running")
    tr, plan, _ = P.run_layer(w, 0, bits[0], piv[0], om[0], w.steps, tiles=tiles)
    P.log(f"[parity] workload {wid} ok: {tr.summary()}")
    assert tr.steps == w.steps and tr.plain.steps > 0
    assert plan.status() == 0


def _stress_tiles(w, layer):
    """Head h (h = layer mod 12) with request (5 h + 3 layer) mod B, plus two random tiles."""
    g = np.random.default_rng(100 + layer)
    tl = [((5 * h + 3 * layer) % w.B) * w.H + h for h in range(layer % w.layers, w.H, w.layers)]
    tl += [int(t) for t in g.choice(w.B * w.H, 2, replace=False)]
    return sorted(set(tl))


def test_full_size_workload_5_split(gpu):
    w = synth.WORKLOADS[5]
    P.log(f"[parity] workload 5 {w.name}: {w.layers} layers x B={w.B} x H={w.H}: plan")
    plans_np, S0s = P.split_setup(w)
    covered = {t % w.H for l in range(w.layers) for t in _stress_tiles(w, l)}
    assert covered == set(range(w.H))
    tr, plans = P.run_layers_split(w, plans_np, w.steps, lambda l: _stress_tiles(w, l), S0s=S0s)
    P.log(f"[parity] workload 5 ok: {tr.summary()}")
    assert tr.steps == w.steps and tr.plain.steps == w.steps * w.layers
    assert all(p.status() == 0 for p in plans)


def test_split_waits_for_a_delayed_writeback(gpu):
    """Split mode with a bounded spin before every side-stream writeback: the next step's
    readout must still see the written-back state (results equal the fused plan's)."""
    import torch
    from quantized_delta_rule_amd import stepq
    w = synth.Workload(501, "race", "gdn", B=8, layers=1, H=6, d=128, steps=5, warmup=8,
                       choices=(4, 6, 8), nominal=6, n_pivots=0, alloc="fixed",
                       fixed_bits=(4, 6, 8, 0, 2, 6))
    bits, piv, om = P.oracle_plan(w)
    dev = torch.device("cuda:0")
    S0 = torch.from_numpy(P.warm_state(w, 0)).to(dev)
    fused = stepq.Plan(stepq.GDN, bits[0], piv[0], om[0])
    split = stepq.Plan(stepq.GDN, bits[0], piv[0], om[0], mode=stepq.SPLIT, max_batch=w.B)
    split.debug_side_delay(5_000_000)  # ~2 ms per writeback
    pf, ps = fused.alloc_pool(w.B), split.alloc_pool(w.B)
    fused.encode(S0, pf, w.B)
    split.encode(S0, ps, w.B)
    for s in range(w.steps):
        g = {k: torch.from_numpy(v).to(dev) for k, v in synth.step_inputs(w, 0, s).items()}
        of = torch.empty((w.B, w.H, w.d), device=dev)
        os_ = torch.empty_like(of)
        fused.step(pf, w.B, g["q"], g["k"], g["v"], g["alpha"], g["beta"], of)
        split.step(ps, w.B, g["q"], g["k"], g["v"], g["alpha"], g["beta"], os_)
        torch.cuda.synchronize()
        assert torch.equal(of, os_), f"step {s}: readouts differ"
    split.sync()
    assert torch.equal(pf, ps)


def test_unpack_debug_matches_oracle(gpu):
    import torch
    from quantized_delta_rule_amd import stepq
    w = synth.Workload(502, "unpack", "kda", B=3, layers=1, H=3, d=128, steps=1, warmup=8,
                       choices=(4, 6, 8), nominal=6, n_pivots=0, alloc="fixed")
    g = np.random.default_rng(7)
    bits = g.choice([2, 4, 6, 8], size=(w.H, w.d)).astype(np.int8)
    piv = np.zeros((w.H, w.d), np.uint8)
    piv[1, [3, 60, 99]] = 1
    om = P.omega_from_steps(w, 0, "warmup", w.warmup)
    plan = stepq.Plan(stepq.KDA, bits, piv, om)
    S0 = P.warm_state(w, 0)
    pool = plan.alloc_pool(w.B)
    plan.encode(torch.from_numpy(S0).to("cuda:0"), pool, w.B)
    Sg, rg, cg, zg = (x.cpu().numpy() for x in plan.unpack(pool, w.B))
    host = pool.cpu().numpy()
    import oracle
    for t in range(w.B * w.H):
        b, h = divmod(t, w.H)
        off, n = plan.head_segment(h)
        So, ro, co, zo = oracle.Head(bits[h], piv[h], om[h]).unpack(
            host[b * plan.bytes_per_request + off:][:n])
        assert np.array_equal(Sg[b, h].view(np.uint32), So.view(np.uint32))
        assert np.array_equal(rg[b, h].view(np.uint16), ro)
        assert np.array_equal(cg[b, h].view(np.uint16), co)
        assert np.array_equal(zg[b, h], zo)
