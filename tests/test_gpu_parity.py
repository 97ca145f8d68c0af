"""GPU <-> oracle parity through the C ABI (needs an MI355X and the built library)."""
import dataclasses

import numpy as np
import pytest

import paritylib as P
from quantized_delta_rule_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from quantized_delta_rule_amd import stepq
    stepq.lib()
    return torch


def _small(wid, kind="gdn", d=128, B=3, H=4, steps=6, **kw):
    return synth.Workload(wid, f"case{wid}", kind, B=B, layers=1, H=H, d=d, steps=steps,
                          warmup=8, choices=(4, 6, 8), nominal=6, n_pivots=0,
                          alloc="fixed", **kw)


def test_workload1_every_tile_every_step(torch_gpu):
    w = synth.WORKLOADS[1]
    P.log(f"[parity] workload 1 {w.name}: B={w.B} H={w.H} d={w.d} steps={w.steps}")
    bits, piv, om = P.oracle_plan(w)
    tr, plan, _ = P.run_layer(w, 0, bits[0], piv[0], om[0], w.steps)
    P.log(f"[parity] workload 1 ok: boundary={tr.boundary} worst readout={tr.worst_readout:.2e}")
    assert plan.status() == 0


@pytest.mark.parametrize("b", [2, 4, 6, 8])
@pytest.mark.parametrize("d", [64, 128])
def test_gdn_each_width(torch_gpu, b, d):
    w = _small(200 + b + d, d=d, H=2, fixed_bits=(b, 0))
    P.log(f"[parity] GDN width {b} d={d}")
    bits, piv, om = P.oracle_plan(w)
    tr, plan, _ = P.run_layer(w, 0, bits[0], piv[0], om[0], w.steps)
    assert plan.status() == 0


@pytest.mark.parametrize("d", [64, 128])
def test_kda_mixed_rows_and_pivots(torch_gpu, d):
    w = _small(300 + d, kind="kda", d=d, H=3)
    P.log(f"[parity] KDA mixed d={d}")
    g = np.random.default_rng(d)
    bits = g.choice([2, 4, 6, 8], size=(w.H, d)).astype(np.int8)
    piv = np.zeros((w.H, d), np.uint8)
    piv[0, [0, 5, d - 1]] = 1
    piv[1, g.choice(d, 9, replace=False)] = 1
    om = P.omega_from_steps(w, 0, "warmup", w.warmup)
    tr, plan, _ = P.run_layer(w, 0, bits, piv, om, w.steps)
    assert plan.status() == 0


def test_dead_rows_columns_and_identity_step(torch_gpu):
    w = _small(401, d=128, B=2, H=2, fixed_bits=(6, 4))
    bits, piv, om = P.oracle_plan(w)
    S0 = P.warm_state(w, 0)
    S0[0, 3, :] = 0.0      # dead row
    S0[1, :, 7] = 0.0      # dead column
    S0[2] = 0.0            # all-zero tile
    d = w.d

    def inputs(s):  # alpha = 1, beta = 0: the decoded state passes through unchanged
        x = synth.step_inputs(w, 0, s)
        x["alpha"][:] = 1.0
        x["beta"][:] = 0.0
        return x
    P.log("[parity] dead rows/columns, identity steps")
    tr, plan, _ = P.run_layer(w, 0, bits[0], piv[0], om[0], 3, S0=S0, inputs=inputs)
    assert plan.status() == 0


def test_empty_batch_is_a_no_op(torch_gpu):
    import torch
    from quantized_delta_rule_amd import stepq
    w = _small(402, B=1, H=2, fixed_bits=(6, 0))
    bits, piv, om = P.oracle_plan(w)
    plan = stepq.Plan(stepq.GDN, bits[0], piv[0], om[0])
    pool = plan.alloc_pool(1)
    z = torch.empty(0, device="cuda:0")
    plan.step(pool, 0, z, z, z, z, z, z)
    torch.cuda.synchronize()
    assert int(pool.sum()) == 0

@pytest.mark.parametrize("kind,d,mode", [("kda", 128, 0), ("kda", 64, 0), ("kda", 128, 1),
                                         ("gdn", 128, 0), ("gdn", 64, 1)])
def test_decay_first_gate_order(torch_gpu, kind, d, mode):
    """Plan order 1, A = (I - beta k k^T) Diag(a): every tile and step against the oracle's
    decay-first step, fused and split, KDA with mixed rows and pivots and GDN with each width."""
    if kind == "kda":
        w = dataclasses.replace(_small(700 + d + mode, kind="kda", d=d, H=3), order=1)
        g = np.random.default_rng(d + mode)
        bits = g.choice([2, 4, 6, 8], size=(w.H, d)).astype(np.int8)
        piv = np.zeros((w.H, d), np.uint8)
        piv[1, g.choice(d, 5, replace=False)] = 1
        om = P.omega_from_steps(w, 0, "warmup", w.warmup)
    else:
        w = dataclasses.replace(_small(710 + d + mode, d=d, H=5, fixed_bits=(2, 4, 6, 8, 0)),
                                order=1)
        bits, piv, om = (a[0] for a in P.oracle_plan(w))
    P.log(f"[parity] decay-first {kind} d={d} mode={mode}")
    tr, plan, _ = P.run_layer(w, 0, bits, piv, om, w.steps, mode=mode)
    assert plan.status() == 0


@pytest.mark.parametrize("d,mode", [(128, 0), (64, 1)])
def test_kda_head_with_every_row_a_pivot(torch_gpu, d, mode):
    """A KDA head whose rows are all FP16 pivots stores no factor blocks; its neighbours must be
    untouched and every tile must match the oracle (fused and split), and the debug decode
    must return the stored binary16 values."""
    torch = torch_gpu
    from quantized_delta_rule_amd import stepq
    w = _small(800 + d + mode, kind="kda", d=d, H=3)
    g = np.random.default_rng(d)
    bits = g.choice([2, 4, 6, 8], size=(w.H, d)).astype(np.int8)
    piv = np.zeros((w.H, d), np.uint8)
    piv[1, :] = 1                      # head 1: every row a pivot
    piv[2, [0, d - 1]] = 1
    om = P.omega_from_steps(w, 0, "warmup", w.warmup)
    P.log(f"[parity] KDA all-pivot head d={d} mode={mode}")
    tr, plan, pool = P.run_layer(w, 0, bits, piv, om, w.steps, mode=mode)
    assert plan.status() == 0
    off, n = plan.head_segment(1)
    assert n == 2 * d * d              # the raw binary16 tile only
    Sg, rg, cg, zg = (x.cpu().numpy() for x in plan.unpack(pool, w.B))
    host = pool.cpu().numpy()
    import oracle
    for b in range(w.B):
        seg = host[b * plan.bytes_per_request + off:][:n]
        So, _, _, _ = oracle.Head(bits[1], piv[1], om[1]).unpack(seg)
        assert np.array_equal(Sg[b, 1].view(np.uint32), So.view(np.uint32))
        assert not rg[b, 1].any() and not cg[b, 1].any() and not zg[b, 1].any()


def test_status_flags_match_oracle(torch_gpu):
    """Binary16 overflow of a row/column factor, of an FP16 pivot entry, and a non-finite
    updated state raise the same status bits on the GPU as in the oracle."""
    torch = torch_gpu
    import oracle
    from quantized_delta_rule_amd import stepq
    dev = torch.device("cuda:0")
    w = _small(901, d=128, B=2, H=2, fixed_bits=(6, 0))
    bits, piv, om = (a[0] for a in P.oracle_plan(w))
    heads = [oracle.Head(bits[h], piv[h], om[h]) for h in range(w.H)]
    plan = stepq.Plan(stepq.GDN, bits, piv, om)
    S0 = P.warm_state(w, 0)
    S0[0] *= 1e7                       # quantized head 0 of request 0: its factors overflow
    S0[3] *= 1e7                       # pivot head 1 of request 1: its entries overflow
    pool = plan.alloc_pool(w.B)
    plan.encode(torch.from_numpy(S0).to(dev), pool, w.B)
    want = 0
    for t in range(w.B * w.H):
        _, _, fl = heads[t % w.H].encode(S0[t], want_pre=True)
        want |= fl
    got = plan.status(reset=True)
    P.log(f"[parity] encode flags gpu {got} oracle {want}")
    assert want == stepq.FLAG_SCALE_OVF | stepq.FLAG_PIVOT_OVF
    assert got == want
    # a NaN in v makes the updated state non-finite
    S1 = P.warm_state(w, 0)
    plan.encode(torch.from_numpy(S1).to(dev), pool, w.B)
    torch.cuda.synchronize()
    segs = [pool.cpu().numpy()[b * plan.bytes_per_request:][:plan.bytes_per_request].copy()
            for b in range(w.B)]
    assert plan.status(reset=True) == 0
    x = synth.step_inputs(w, 0, 0)
    x["v"][1, 0, 5] = np.nan
    gx = {k: torch.from_numpy(v).to(dev) for k, v in x.items()}
    out = torch.empty((w.B, w.H, w.d), device=dev)
    plan.step(pool, w.B, gx["q"], gx["k"], gx["v"], gx["alpha"], gx["beta"], out)
    want = 0
    a_rows = synth.alpha_rows(w, x["alpha"])
    for t in range(w.B * w.H):
        b, h = divmod(t, w.H)
        off, n = plan.head_segment(h)
        seg = segs[b][off:off + n].copy()
        _, _, _, fl = heads[h].step(seg, x["q"][b, h], x["k"][b, h], x["v"][b, h],
                                    a_rows[b, h], x["beta"][b, h], want_state=True)
        want |= fl
    got = plan.status(reset=True)
    P.log(f"[parity] step flags gpu {got} oracle {want}")
    assert want & stepq.FLAG_NONFINITE
    assert got == want


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_uniform_width_unit_impact_plan(torch_gpu, kind):
    """The baseline plan of the ablation (every unit at one width, no pivots, omega = 1, so every
    row's denominator is 1 + 1 = 2 and the refit weights rows evenly) through the same kernels,
    checked against the oracle and the plain reference like the STEPQuant plans."""
    w = dataclasses.replace(synth.WORKLOADS[2], wid=420 + (kind == "kda"), kind=kind, B=6,
                            steps=12, alloc="fixed", n_pivots=0)
    P.log(f"[parity] uniform-6, omega = 1, {kind}: B={w.B} H={w.H}")
    bits = np.full((w.H, w.d), 6, np.int8)
    piv = np.zeros((w.H, w.d), np.uint8)
    om = np.ones((w.H, w.d), np.float32)
    tr, plan, _ = P.run_layer(w, 0, bits, piv, om, w.steps,
                              tiles=P.sample_tiles(w, per_head=1, extra=4, seed=42))
    P.log(f"[parity] uniform-6 {kind} ok: {tr.summary()}")
    assert plan.status() == 0 and tr.plain.steps > 0
