"""stepq_decode_step_noalloc, through the C ABI, against stepq_decode_step: bit-identical
readouts and packed states on two calls in a row (the second with a smaller batch), for split
plans (the hand-over through the library's static device scratch) and a fused plan, with several
split plans interleaved on one GPU, and a refused oversized batch that leaves the pool alone."""
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


def _case(kind):
    if kind == "gdn":
        w = synth.Workload(601, "noalloc-gdn", "gdn", B=9, layers=1, H=6, d=128, steps=2,
                           warmup=8, choices=(4, 6, 8), nominal=6, n_pivots=0, alloc="fixed",
                           fixed_bits=(4, 6, 8, 0, 2, 6))
        bits, piv, om = (a[0] for a in P.oracle_plan(w))
    else:
        w = synth.Workload(602, "noalloc-kda", "kda", B=7, layers=1, H=3, d=64, steps=2,
                           warmup=8, choices=(4, 6, 8), nominal=6, n_pivots=0, alloc="fixed")
        g = np.random.default_rng(5)
        bits = g.choice([2, 4, 6, 8], size=(w.H, w.d)).astype(np.int8)
        piv = np.zeros((w.H, w.d), np.uint8)
        piv[1, [2, 40]] = 1
        om = P.omega_from_steps(w, 0, "warmup", w.warmup)
    return w, bits, piv, om


def _inputs(torch, w, s, Bs):
    x = synth.step_inputs(w, 0, s)
    return {k: torch.from_numpy(np.ascontiguousarray(v[:Bs])).to("cuda:0") for k, v in x.items()}


@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("mode", ["split", "fused"])
def test_noalloc_matches_decode_step(gpu, kind, mode):
    torch = gpu
    from quantized_delta_rule_amd import stepq
    w, bits, piv, om = _case(kind)
    K = stepq.GDN if kind == "gdn" else stepq.KDA
    M = stepq.SPLIT if mode == "split" else stepq.FUSED
    P.log(f"[noalloc] {kind} {mode}: B={w.B} H={w.H} d={w.d}")
    ref = stepq.Plan(K, bits, piv, om, mode=M, max_batch=w.B)
    # the no-allocation call does not use the plan's own hand-over (sized for one request)
    na = stepq.Plan(K, bits, piv, om, mode=M, max_batch=1)
    S0 = torch.from_numpy(P.warm_state(w, 0)).to("cuda:0")
    pr, pn = ref.alloc_pool(w.B), na.alloc_pool(w.B)
    ref.encode(S0, pr, w.B)
    pn.copy_(pr)                                      # both start from the same packed state
    for s, Bs in enumerate((w.B, w.B - 3)):           # two calls, the second with fewer rows
        x = _inputs(torch, w, s, Bs)
        o_r = torch.full((Bs, w.H, w.d), float("nan"), device="cuda:0")
        o_n = torch.full_like(o_r, float("nan"))
        ref.step(pr, Bs, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o_r)
        na.step_noalloc(pn, Bs, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o_n)
        ref.sync()
        na.sync()
        torch.cuda.synchronize()
        assert torch.equal(o_r, o_n), f"step {s}: readouts differ"
        assert torch.equal(pr, pn), f"step {s}: packed states differ"
    assert ref.status() == 0 and na.status() == 0


def test_noalloc_plans_interleaved(gpu):
    """Three split plans (three layers) stepped back to back through the no-allocation call
    share the one scratch array: each readout waits for the previous plan's writeback, so the
    results equal three plans stepped with their own buffers."""
    torch = gpu
    from quantized_delta_rule_amd import stepq
    w, bits, piv, om = _case("gdn")
    S0 = torch.from_numpy(P.warm_state(w, 0)).to("cuda:0")
    refs = [stepq.Plan(stepq.GDN, bits, piv, om, mode=stepq.SPLIT, max_batch=w.B)
            for _ in range(3)]
    nas = [stepq.Plan(stepq.GDN, bits, piv, om, mode=stepq.SPLIT, max_batch=1) for _ in range(3)]
    prs = [p.alloc_pool(w.B) for p in refs]
    for p, pool in zip(refs, prs):
        p.encode(S0, pool, w.B)
    torch.cuda.synchronize()
    pns = [pool.clone() for pool in prs]
    for s in range(3):
        x = [_inputs(torch, w, s * 3 + l, w.B) for l in range(3)]
        o_r = [torch.empty((w.B, w.H, w.d), device="cuda:0") for _ in range(3)]
        o_n = [torch.empty_like(o) for o in o_r]
        for l in range(3):
            a = x[l]
            refs[l].step(prs[l], w.B, a["q"], a["k"], a["v"], a["alpha"], a["beta"], o_r[l])
            nas[l].step_noalloc(pns[l], w.B, a["q"], a["k"], a["v"], a["alpha"], a["beta"],
                                o_n[l])
        for p in refs + nas:
            p.sync()
        torch.cuda.synchronize()
        for l in range(3):
            assert torch.equal(o_r[l], o_n[l]) and torch.equal(prs[l], pns[l]), (s, l)


def test_noalloc_refuses_a_batch_beyond_the_scratch(gpu):
    torch = gpu
    from quantized_delta_rule_amd import stepq
    H, d = 64, 128                      # 16384 tiles fit 32 MiB at d = 128; 16385 do not
    bits = np.full((H, d), 6, np.int8)
    plan = stepq.Plan(stepq.GDN, bits, np.zeros((H, d), np.uint8), np.ones((H, d), np.float32),
                      mode=stepq.SPLIT, max_batch=1)
    B = 257
    pool = plan.alloc_pool(B)
    pool.fill_(7)
    q = torch.zeros((B, H, d), device="cuda:0")
    a = torch.ones((B, H), device="cuda:0")
    out = torch.zeros((B, H, d), device="cuda:0")
    with pytest.raises(stepq.StepqError, match="scratch"):
        plan.step_noalloc(pool, B, q, q, q, a, a, out)
    torch.cuda.synchronize()
    assert bool((pool == 7).all()) and bool((out == 0).all())
