"""Slot-indexed pools through the C ABI: batch rows address pool slots through an int32 index
array (padding rows = -1).  Every stepped slot must equal the oracle's step of that slot's
segment with that row's inputs; every other slot must keep its bytes; padding and bad rows must
leave their out rows alone, and a bad index must raise the bad-slot flag."""
import dataclasses

import numpy as np
import pytest

import oracle
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
    fixed = (6, 4, 0) if kind == "gdn" else None
    return synth.Workload(610 + d + (kind == "kda"), f"slots-{kind}", kind, B=B, layers=1, H=3,
                          d=d, steps=2, warmup=8, choices=(4, 6, 8), nominal=6, n_pivots=0,
                          alloc="fixed", fixed_bits=fixed)


def _plan_arrays(w):
    if w.kind == "gdn":
        return [a[0] for a in P.oracle_plan(w)]
    g = np.random.default_rng(w.d)
    bits = g.choice([2, 4, 6, 8], size=(w.H, w.d)).astype(np.int8)
    piv = np.zeros((w.H, w.d), np.uint8)
    piv[2, [1, 17, w.d - 2]] = 1
    return bits, piv, P.omega_from_steps(w, 0, "warmup", w.warmup)


def _seg(host, plan, slot, h):
    off, n = plan.head_segment(h)
    base = slot * plan.bytes_per_request + off
    return host[base: base + n]


def _run(torch, kind, d, mode, slots_list, n_slots):
    from quantized_delta_rule_amd import stepq
    dev = torch.device("cuda:0")
    B = len(slots_list)
    wpool = _workload(kind, d, n_slots)        # states of every slot
    wbatch = dataclasses.replace(wpool, B=B)   # inputs of the batch rows
    bits, piv, om = _plan_arrays(wpool)
    H = wpool.H
    plan = stepq.Plan(stepq.GDN if kind == "gdn" else stepq.KDA, bits, piv, om, mode=mode,
                      max_batch=max(B, n_slots))
    heads = [oracle.Head(bits[h], piv[h], om[h]) for h in range(H)]
    S0 = P.warm_state(wpool, 0)
    pool = plan.alloc_pool(n_slots)
    plan.encode(torch.from_numpy(S0).to(dev), pool, n_slots)
    torch.cuda.synchronize()
    before = pool.cpu().numpy().copy()
    x = synth.step_inputs(wbatch, 0, 0, "decode")
    a_rows = synth.alpha_rows(wbatch, x["alpha"])
    g = {k: torch.from_numpy(v).to(dev) for k, v in x.items()}
    out = torch.full((B, H, d), float("nan"), device=dev)
    slots = torch.tensor(slots_list, dtype=torch.int32, device=dev)
    plan.step_slots(pool, n_slots, slots, B, g["q"], g["k"], g["v"], g["alpha"], g["beta"], out)
    # the caller may reuse its slot array once the stream has run: scribble over it at once
    slots.fill_(0)
    plan.sync()
    torch.cuda.synchronize()
    after = pool.cpu().numpy()
    outh = out.cpu().numpy()
    stepped = set()
    for b, s in enumerate(slots_list):
        if not 0 <= s < n_slots:
            assert np.isnan(outh[b]).all(), f"row {b} (slot {s}) wrote its out row"
            continue
        stepped.add(s)
        for h in range(H):
            so = _seg(before, plan, s, h).copy()   # stepped in place by the oracle
            o, _, pre, _ = heads[h].step(so, x["q"][b, h], x["k"][b, h], x["v"][b, h],
                                         a_rows[b, h], x["beta"][b, h], want_state=True)
            assert P.rel_l2(outh[b, h], o) <= P.READOUT_TOL
            P.compare_segment(heads[h], _seg(after, plan, s, h), so, pre,
                              f"slot {s} row {b} head {h}")
    bpr = plan.bytes_per_request
    for s in range(n_slots):
        if s not in stepped:
            assert np.array_equal(after[s * bpr:(s + 1) * bpr], before[s * bpr:(s + 1) * bpr]), \
                f"slot {s} changed without being addressed"
    return plan


@pytest.mark.parametrize("kind,d,mode", [("gdn", 128, 0), ("kda", 64, 0), ("gdn", 64, 1),
                                         ("kda", 128, 1)])
def test_slot_indexed_step_matches_oracle(gpu, kind, d, mode):
    P.log(f"[parity] slots {kind} d={d} mode={mode}")
    plan = _run(gpu, kind, d, mode, [5, -1, 2, 7, 0], 9)
    assert plan.status() == 0


def test_bad_slot_raises_flag_and_skips_row(gpu):
    from quantized_delta_rule_amd import stepq
    P.log("[parity] slots: out-of-range index")
    plan = _run(gpu, "gdn", 128, 0, [1, 99, -7, 3], 4)
    assert plan.status(reset=True) == stepq.FLAG_BAD_SLOT
    assert plan.status() == 0


def test_identity_slots_equal_plain_step(gpu):
    """slots[b] = b on an n_slots = B pool gives the plain call's bytes and readouts."""
    torch = gpu
    from quantized_delta_rule_amd import stepq
    dev = torch.device("cuda:0")
    w = _workload("gdn", 128, 6)
    bits, piv, om = _plan_arrays(w)
    plan = stepq.Plan(stepq.GDN, bits, piv, om)
    S0 = torch.from_numpy(P.warm_state(w, 0)).to(dev)
    pa, pb = plan.alloc_pool(w.B), plan.alloc_pool(w.B)
    slots = torch.arange(w.B, dtype=torch.int32, device=dev)
    plan.encode(S0, pa, w.B)
    plan.encode_slots(S0, pb, w.B, slots, w.B)
    torch.cuda.synchronize()
    assert torch.equal(pa, pb)
    for s in range(2):
        g = {k: torch.from_numpy(v).to(dev) for k, v in synth.step_inputs(w, 0, s).items()}
        oa = torch.empty((w.B, w.H, w.d), device=dev)
        ob = torch.empty_like(oa)
        plan.step(pa, w.B, g["q"], g["k"], g["v"], g["alpha"], g["beta"], oa)
        plan.step_slots(pb, w.B, slots, w.B, g["q"], g["k"], g["v"], g["alpha"], g["beta"], ob)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob) and torch.equal(pa, pb)
    assert plan.status() == 0


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_encode_into_slots(gpu, kind):
    """encode_state_slots writes exactly the addressed slots, each equal to the oracle's
    encoding of that batch row's state; padding rows and other slots are left alone."""
    torch = gpu
    from quantized_delta_rule_amd import stepq
    dev = torch.device("cuda:0")
    slots_list, n_slots = [3, -1, 0], 5
    w = _workload(kind, 128, len(slots_list))
    bits, piv, om = _plan_arrays(w)
    plan = stepq.Plan(stepq.GDN if kind == "gdn" else stepq.KDA, bits, piv, om)
    S = P.warm_state(w, 0)
    pool = plan.alloc_pool(n_slots)
    pool.fill_(0xAB)
    torch.cuda.synchronize()
    before = pool.cpu().numpy().copy()
    slots = torch.tensor(slots_list, dtype=torch.int32, device=dev)
    plan.encode_slots(torch.from_numpy(S).to(dev), pool, n_slots, slots, len(slots_list))
    torch.cuda.synchronize()
    after = pool.cpu().numpy()
    bpr = plan.bytes_per_request
    for b, s in enumerate(slots_list):
        if s < 0:
            continue
        for h in range(w.H):
            head = oracle.Head(bits[h], piv[h], om[h])
            so, pre, _ = head.encode(S[b * w.H + h], want_pre=True)
            P.compare_segment(head, _seg(after, plan, s, h), so, pre, f"slot {s} head {h}")
    for s in (1, 2, 4):
        assert np.array_equal(after[s * bpr:(s + 1) * bpr], before[s * bpr:(s + 1) * bpr])
    assert plan.status() == 0


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_slot_array_rewritten_by_a_kernel_between_steps(gpu, kind):
    """The kernels read the slot array through the scalar cache.  A slot array rewritten on the
    device (a copy kernel on the same stream) between two steps must be seen by the second step:
    the pool and readouts equal those of steps given freshly uploaded arrays."""
    torch = gpu
    from quantized_delta_rule_amd import stepq
    dev = torch.device("cuda:0")
    n_slots, first, second = 6, [0, 1, 2], [5, 3, 1]
    wpool = _workload(kind, 128, n_slots)
    wb = dataclasses.replace(wpool, B=len(first))
    bits, piv, om = _plan_arrays(wpool)
    plan = stepq.Plan(stepq.GDN if kind == "gdn" else stepq.KDA, bits, piv, om)
    S0 = torch.from_numpy(P.warm_state(wpool, 0)).to(dev)
    pa, pb = plan.alloc_pool(n_slots), plan.alloc_pool(n_slots)
    plan.encode(S0, pa, n_slots)
    plan.encode(S0, pb, n_slots)
    g = {k: torch.from_numpy(v).to(dev) for k, v in synth.step_inputs(wb, 0, 0).items()}
    args = (g["q"], g["k"], g["v"], g["alpha"], g["beta"])
    B = len(first)
    oa, ob = torch.empty((B, wb.H, wb.d), device=dev), torch.empty((B, wb.H, wb.d), device=dev)
    reused = torch.tensor(first, dtype=torch.int32, device=dev)
    src = torch.tensor(second, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    plan.step_slots(pa, n_slots, reused, B, *args, oa)
    reused.copy_(src)                     # device-side rewrite between the two steps
    plan.step_slots(pa, n_slots, reused, B, *args, oa)
    plan.step_slots(pb, n_slots, torch.tensor(first, dtype=torch.int32, device=dev), B, *args, ob)
    plan.step_slots(pb, n_slots, torch.tensor(second, dtype=torch.int32, device=dev), B, *args, ob)
    torch.cuda.synchronize()
    assert torch.equal(pa, pb) and torch.equal(oa, ob)
    assert plan.status() == 0
