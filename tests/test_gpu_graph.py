"""Decode steps captured into a HIP graph (torch.cuda.CUDAGraph) through the C ABI.  A fused
plan's step only enqueues kernels, so a captured step replayed n times must leave the pool and
the readout bit-identical to n eager steps on the same inputs.  Every replay is checked, with
eager work of the program (another plan's step on another pool, host syncs) between replays.
A split-mode plan must refuse a capturing stream with STEPQ_ERR_UNSUPPORTED."""
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


def _workload(kind, d, B):
    fixed = (6, 4, 8, 0) if kind == "gdn" else None
    return synth.Workload(730 + d + (kind == "kda"), f"graph-{kind}", kind, B=B, layers=1, H=4,
                          d=d, steps=2, warmup=6, choices=(4, 6, 8), nominal=6, n_pivots=0,
                          alloc="fixed", fixed_bits=fixed)


def _plan(w, mode):
    from quantized_delta_rule_amd import stepq
    if w.kind == "gdn":
        bits, piv, om = [a[0] for a in P.oracle_plan(w)]
    else:
        g = np.random.default_rng(w.d)
        bits = g.choice([2, 4, 6, 8], size=(w.H, w.d)).astype(np.int8)
        piv = np.zeros((w.H, w.d), np.uint8)
        piv[1, [0, 9, w.d - 1]] = 1
        om = P.omega_from_steps(w, 0, "warmup", w.warmup)
    kind = stepq.GDN if w.kind == "gdn" else stepq.KDA
    m = stepq.SPLIT if mode == "split" else stepq.FUSED
    return stepq.Plan(kind, bits, piv, om, mode=m, max_batch=w.B)


def _setup(torch, kind, d, B, mode="fused"):
    dev = torch.device("cuda:0")
    w = _workload(kind, d, B)
    plan = _plan(w, mode)
    S0 = torch.from_numpy(P.warm_state(w, 0)).to(dev)
    x = {k: torch.from_numpy(v).to(dev) for k, v in synth.step_inputs(w, 0, 0, "decode").items()}
    return w, plan, S0, x


@pytest.mark.parametrize("kind,d,B", [("gdn", 128, 5), ("kda", 128, 3), ("gdn", 64, 7),
                                      ("kda", 64, 2)])
def test_captured_step_replays_match_eager_steps(gpu, kind, d, B):
    torch = gpu
    P.log(f"[graph] captured step {kind} d={d} B={B}")
    w, plan, S0, x = _setup(torch, kind, d, B)
    dev = S0.device
    args = (x["q"], x["k"], x["v"], x["alpha"], x["beta"])
    # eager reference: three steps from the encoded state
    ref_pool = plan.alloc_pool(B)
    plan.encode(S0, ref_pool, B)
    ref_out = torch.empty((B, w.H, d), device=dev)
    refs = []
    for _ in range(3):
        plan.step(ref_pool, B, *args, ref_out)
        torch.cuda.synchronize()
        refs.append((ref_pool.clone(), ref_out.clone()))
    # unrelated eager work between replays: another plan stepping another pool
    _, other, oS0, ox = _setup(torch, kind, d, B)
    opool = other.alloc_pool(B)
    other.encode(oS0, opool, B)
    oout = torch.empty((B, w.H, d), device=dev)
    # captured step
    pool = plan.alloc_pool(B)
    plan.encode(S0, pool, B)
    out = torch.full((B, w.H, d), float("nan"), device=dev)
    torch.cuda.synchronize()
    initial = pool.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.step(pool, B, *args, out)
    torch.cuda.synchronize()
    assert torch.equal(pool, initial), "capturing must not run the step"
    for i, (rp, ro) in enumerate(refs):
        g.replay()
        other.step(opool, B, ox["q"], ox["k"], ox["v"], ox["alpha"], ox["beta"], oout)
        torch.cuda.synchronize()
        assert torch.equal(pool, rp), f"replay {i}: pool differs from eager step {i}"
        assert torch.equal(out, ro), f"replay {i}: readout differs from eager step {i}"
    assert plan.status() == 0 and other.status() == 0


def test_captured_slot_step_replays(gpu):
    import dataclasses
    torch = gpu
    P.log("[graph] captured slot step gdn d=128")
    B, n_slots = 3, 6
    wp = _workload("gdn", 128, n_slots)          # states of every slot
    wb = dataclasses.replace(wp, B=B)            # inputs of the batch rows
    plan = _plan(wp, "fused")
    dev = torch.device("cuda:0")
    S0 = torch.from_numpy(P.warm_state(wp, 0)).to(dev)
    x = {k: torch.from_numpy(v).to(dev) for k, v in synth.step_inputs(wb, 0, 0, "decode").items()}
    args = (x["q"], x["k"], x["v"], x["alpha"], x["beta"])
    slots = torch.tensor([4, -1, 1], dtype=torch.int32, device=dev)
    ref_pool = plan.alloc_pool(n_slots)
    plan.encode(S0, ref_pool, n_slots)
    ref_out = torch.zeros((B, wp.H, 128), device=dev)
    refs = []
    for _ in range(2):
        plan.step_slots(ref_pool, n_slots, slots, B, *args, ref_out)
        torch.cuda.synchronize()
        refs.append((ref_pool.clone(), ref_out.clone()))
    pool = plan.alloc_pool(n_slots)
    plan.encode(S0, pool, n_slots)
    out = torch.zeros((B, wp.H, 128), device=dev)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.step_slots(pool, n_slots, slots, B, *args, out)
    for i, (rp, ro) in enumerate(refs):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(pool, rp), f"replay {i}: pool differs"
        assert torch.equal(out, ro), f"replay {i}: readout differs"
    assert plan.status() == 0


def test_split_plan_refuses_capture(gpu):
    torch = gpu
    from quantized_delta_rule_amd import stepq
    P.log("[graph] split plan under capture")
    B = 2
    w, plan, S0, x = _setup(torch, "gdn", 128, B, mode="split")
    pool = plan.alloc_pool(B)
    plan.encode(S0, pool, B)
    out = torch.empty((B, w.H, 128), device=S0.device)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    err = None
    with torch.cuda.graph(g):   # the refused call enqueues nothing: the capture ends empty
        try:
            plan.step(pool, B, x["q"], x["k"], x["v"], x["alpha"], x["beta"], out)
        except stepq.StepqError as e:
            err = e
    assert err is not None and "capturing stream" in str(err) and "(-2)" in str(err), err
    # the plan still works eagerly afterwards
    plan.step(pool, B, x["q"], x["k"], x["v"], x["alpha"], x["beta"], out)
    plan.sync()
    torch.cuda.synchronize()
    assert plan.status() == 0
