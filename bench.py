"""Decode-step benchmark: head-steps/s and achieved HBM bandwidth of the fused packed-state
decode step on one MI355X.

Default workload: 70 concurrent requests x 48 GDN heads, d_k = d_v = 128, nominal 6-bit per-head
map from the multiple-choice DP (widths {4,6,8}, one FP16 pivot head), initial states from 16
unquantized warm-up steps.  A step is one decode step of the whole batch (one kernel launch over
3,360 tiles).  The timed loop rotates over pool replicas (independent request batches) whose
total size exceeds twice the 256 MB Infinity Cache, so the packed state streams from HBM.

Prints one JSON line.  Inputs are synthetic (seeded); nothing is read from disk except the
optional committed counter summary under profiles/.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, vendor figure
# Vector ALU issue peak without packed FP32: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
# (= 78.6 TFLOP/s counting an FMA as two; the 157.3 TFLOP/s figure needs packed FP32, which this
# build does not use).
PEAK_ALU_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
METRIC = "decode head-steps/s + achieved HBM GB/s vs peak, nominal-6-bit GDN state pool"
# counter summary of a workload (HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE)
COUNTERS = os.path.join(ROOT, "profiles", "{name}_counters.json")
KERNEL_SOURCES = ["quantized_delta_rule_amd/csrc/stepq_device.h",
                  "quantized_delta_rule_amd/csrc/stepq_k128_gdn.hip",
                  "quantized_delta_rule_amd/csrc/stepq_k128_kda.hip",
                  "quantized_delta_rule_amd/csrc/stepq_internal.h"]


def kernel_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def warm_state(w, layer, dev):
    """Initial states [B*H, d, d]: w.warmup unquantized delta-rule steps from zero (workload
    synthesis with plain torch ops; not the decode path)."""
    import torch
    from quantized_delta_rule_amd import synth
    d = w.d
    S = torch.zeros((w.B * w.H, d, d), dtype=torch.float32, device=dev)
    for s in range(w.warmup):
        x = synth.step_inputs(w, layer, s, "warmup")
        k = torch.from_numpy(x["k"].reshape(-1, d)).to(dev)
        v = torch.from_numpy(x["v"].reshape(-1, d)).to(dev)
        a = torch.from_numpy(synth.alpha_rows(w, x["alpha"]).reshape(-1, d)).to(dev)
        b = torch.from_numpy(x["beta"].reshape(-1)).to(dev)
        u = (S * k[:, :, None]).sum(1)                                   # S^T k
        e = v[:, None, :] - a[:, :, None] * u[:, None, :]                # v - a_i u
        S = a[:, :, None] * S + (b[:, None] * k)[:, :, None] * e
    return S


def cpu_baseline(w, plan_arrays, S_tiles, budget_s, threads):
    """The oracle (as it stands) on a bounded sample of tiles of the same workload."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    from quantized_delta_rule_amd import synth
    bits, piv, om = plan_arrays
    tiles = list(S_tiles.keys())
    heads = {h: oracle.Head(bits[0, h], piv[0, h], om[0, h]) for h in {t % w.H for t in tiles}}
    segs = {t: heads[t % w.H].encode(S_tiles[t]) for t in tiles}
    x = synth.step_inputs(w, 0, 0, "decode")
    a_rows = synth.alpha_rows(w, x["alpha"])
    # calibrate: one step per tile on one thread, then size the run to the budget
    t0 = time.perf_counter()
    for t in tiles[:4]:
        b, h = divmod(t, w.H)
        heads[h].step(segs[t].copy(), x["q"][b, h], x["k"][b, h], x["v"][b, h], a_rows[b, h],
                      x["beta"][b, h])
    per = (time.perf_counter() - t0) / 4
    steps = max(1, int(budget_s * threads / (per * len(tiles))))

    def work(chunk):
        for s in range(steps):  # the same inputs every step: this only times the oracle
            for t in chunk:
                b, h = divmod(t, w.H)
                heads[h].step(segs[t], x["q"][b, h], x["k"][b, h], x["v"][b, h],
                              a_rows[b, h], x["beta"][b, h])
        return len(chunk) * steps

    chunks = [tiles[i::threads] for i in range(threads)]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        done = sum(ex.map(work, chunks))
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "head-steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(tiles)} tiles of replica 0 (every head), {steps} steps each, "
                      f"{done} tile-steps in {dt:.1f} s"}


# Pool replicas rotated per timed step (one-layer workloads): enough that the replicas together
# exceed twice the 256 MB Infinity Cache, so the packed state streams from HBM.
REPLICAS = {1: 12, 2: 12, 3: 10, 4: 20, 6: 12}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=600)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--replicas", type=int, default=None,
                    help="pool replicas rotated per step (one-layer workloads)")
    ap.add_argument("--inputs", type=int, default=4, help="distinct input sets per replica")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the decode step "
              "shards by request or head with no cross-GPU traffic, so N GPUs run N copies.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from quantized_delta_rule_amd import planning, stepq, synth

    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[args.workload]
    print(f"[bench] workload {w.wid} {w.name}: planning", file=sys.stderr, flush=True)
    bits, piv, om = planning.plan_arrays(w)
    kind = stepq.GDN if w.kind == "gdn" else stepq.KDA
    mode = stepq.SPLIT if w.split else stepq.FUSED
    multi = w.layers > 1
    # one plan per layer; a one-layer workload steps R independent replicas of its pool in turn
    plans = [stepq.Plan(kind, bits[l], piv[l], om[l], mode=mode, max_batch=w.B, order=w.order)
             for l in range(w.layers)]
    R = 1 if multi else (args.replicas or REPLICAS.get(w.wid, 12))
    units = [(plans[l], l) for l in range(w.layers)] if multi else [(plans[0], r) for r in range(R)]
    alg_bytes = sum(planning.algorithmic_bytes(w, p) for p in plans)
    alg_ops = sum(planning.algorithmic_ops(w, p) for p in plans)
    pools, inputs, S_sample = [], [], {}
    enc_ms = []
    for i, (plan, seed) in enumerate(units):
        S0 = warm_state(w, seed, dev)
        pool = plan.alloc_pool(w.B)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        plan.encode(S0, pool, w.B)
        e1.record()
        e1.synchronize()
        enc_ms.append(e0.elapsed_time(e1))
        if i == 0 and not args.no_cpu:
            pick = [b * w.H + h for b, h in zip(range(0, w.B, max(1, w.B // w.H)), range(w.H))]
            S_sample = {t: S0[t].cpu().numpy() for t in pick}
        del S0
        pools.append(pool)
        sets = []
        for j in range(args.inputs):
            x = synth.step_inputs(w, seed, j, "decode")
            sets.append({k: torch.from_numpy(v).to(dev) for k, v in x.items()})
        inputs.append(sets)
    torch.cuda.synchronize()
    pool_mib = sum(p.bytes_per_request for p in plans) * w.B / 2 ** 20
    print(f"[bench] {len(units)} {'layers' if multi else 'replicas'} x "
          f"{plans[0].bytes_per_request * w.B / 2**20:.1f} MiB pool "
          f"({plans[0].bits_per_value:.3f} bits/value), timing", file=sys.stderr, flush=True)

    out = torch.empty((w.B, w.H, w.d), dtype=torch.float32, device=dev)
    L = stepq.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = ctypes.c_void_p

    def call(u, j):
        plan, x = units[u][0], inputs[u][j]
        return (plan._h, P(pools[u].data_ptr()), w.B, P(x["q"].data_ptr()),
                P(x["k"].data_ptr()), P(x["v"].data_ptr()), P(x["alpha"].data_ptr()),
                P(x["beta"].data_ptr()), P(out.data_ptr()), stream)

    # a step: every layer once (multi-layer workloads), or one replica in turn, replica-major
    # rotation so consecutive steps touch different pools
    if multi:
        steps = [[call(u, j) for u in range(len(units))] for j in range(args.inputs)]
    else:
        flat = [call(u, j) for u in range(R) for j in range(args.inputs)]
        steps = [[flat[(i % R) * args.inputs + (i // R) % args.inputs]] for i in range(len(flat))]
    launches = len(steps[0])
    step_fn = L.stepq_decode_step

    def run(i):
        for c in steps[i % len(steps)]:
            step_fn(*c)

    def drain():
        torch.cuda.synchronize()
        for p in plans:
            p.sync()

    for i in range(args.warmup):
        for c in steps[i % len(steps)]:
            if step_fn(*c):
                raise RuntimeError(L.stepq_last_error().decode())
    drain()
    # timed region: K steps back to back on the launch stream, one event pair around them (an
    # event pair per launch would add its own overhead to every step); split-mode refits run on
    # the plans' side streams and are included by the host clock
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        run(i)
    ev1.record()
    drain()
    wall = time.perf_counter() - t0
    avg_k = ev0.elapsed_time(ev1) / (args.steps * launches)
    if any(p.status() != 0 for p in plans):
        raise RuntimeError("status flags raised during the benchmark")
    ms_per_step = wall * 1e3 / args.steps
    # the kernel time a step takes: the launch stream's events (fused), or the host clock when
    # a side stream carries part of the work (split)
    step_ms = ms_per_step if w.split else avg_k * launches

    k_ms, hot_ms, graph_ms = None, None, None
    if not multi:
        # spread over launches (outside the timed region): each launch between its own event
        # pair, so these figures include that pair's overhead
        nspread = min(100, args.steps)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(nspread)]
        for i in range(nspread):
            ev[i][0].record()
            run(i)
            ev[i][1].record()
        drain()
        k_ms = np.array([a.elapsed_time(b) for a, b in ev])
        # cache-hot reference: one pool stepped repeatedly (labelled, not the headline)
        h0, h1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        h0.record()
        for _ in range(50):
            step_fn(*steps[0][0])
        h1.record()
        drain()
        hot_ms = h0.elapsed_time(h1) / 50
        if not w.split:
            # graph replay (labelled, not the headline): one captured step per replica, the
            # graph replayed back to back, so no step pays a host-side launch
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
                for r in range(R):
                    if step_fn(*(steps[r][0][:-1] + (cs,))):
                        raise RuntimeError(L.stepq_last_error().decode())
            g.replay()
            drain()
            reps = max(1, args.steps // R)
            g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            g0.record()
            for _ in range(reps):
                g.replay()
            g1.record()
            drain()
            graph_ms = g0.elapsed_time(g1) / (reps * R)
            del g
        if any(p.status() != 0 for p in plans):
            raise RuntimeError("status flags raised during the benchmark")

    if args.copy_calib:
        src = torch.empty(2 ** 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    heads = w.B * w.H * w.layers
    achieved = alg_bytes / (step_ms * 1e-3) / 1e9
    achieved_ops = alg_ops / (step_ms * 1e-3) / 1e12
    kname = ("k_gdn" if w.kind == "gdn" else "k_kda") + f"<{w.d}, " + \
        ("READ> + WRITE (side stream)" if w.split else "FUSED>")
    traffic = None
    cpath = COUNTERS.format(name=w.name)
    if os.path.exists(cpath):
        c = json.load(open(cpath))
        if c.get("kernel_sha") == kernel_sha() and c.get("workload") == w.name:
            traffic = c["hbm_bytes_per_launch"]
    unit_desc = (f"MC-DP map {w.choices}" if w.alloc == "mcdp" else
                 f"Lagrangian row map {w.choices}" if w.alloc == "lagrangian" else
                 f"fixed head widths {w.fixed_bits}")
    config = {
        "workload": f"{w.name}: {w.B} requests x {w.layers} layer(s) x {w.H} "
                    f"{w.kind.upper()} heads, d_k=d_v={w.d}, nominal {w.nominal}-bit {unit_desc}"
                    f", {w.n_pivots} FP16 pivot unit(s), "
                    + (f"{w.layers} layers back to back per step, refit and writeback on a side "
                       f"stream" if multi else f"{R} rotating pool replicas"),
        "bits_per_value": round(plans[0].bits_per_value, 4),
        "pool_mib_per_replica": round(pool_mib, 2),
        "algorithmic_bytes_per_step": alg_bytes,
        "kernel_ms_mean": avg_k,
        "launches_per_step": launches,
        "hbm": {"achieved_GBps": achieved, "peak_GBps": PEAK_HBM_GBS,
                "frac": achieved / PEAK_HBM_GBS},
        "algorithmic_ops_per_step": alg_ops,
    }
    if k_ms is not None:
        config["event_bracketed_launch_ms_p10_p50_p90"] = [float(np.percentile(k_ms, p))
                                                           for p in (10, 50, 90)]
        config["cache_hot_single_pool_kernel_ms"] = hot_ms
        config["cache_hot_single_pool_GBps"] = alg_bytes / (hot_ms * 1e-3) / 1e9
    if graph_ms is not None:
        config["graph_replay_ms_per_step"] = graph_ms
        config["graph_replay_head_steps_per_s"] = heads / (graph_ms * 1e-3)
    # encoding an fp32 state into the pool (the hand-off from prefill): the median over the
    # setup encodes, each between its own event pair; bytes = fp32 state read + packed write
    enc = float(np.median(enc_ms[1:] if len(enc_ms) > 1 else enc_ms))
    enc_bytes = w.B * w.H * w.d * w.d * 4 + w.B * float(np.mean([p.bytes_per_request for p in plans]))
    config["encode"] = {"kernel": kname.split("<")[0] + f"<{w.d}, ENCODE>", "ms_per_batch": enc,
                        "bytes_per_batch": enc_bytes, "GBps": enc_bytes / (enc * 1e-3) / 1e9,
                        "hbm_frac": enc_bytes / (enc * 1e-3) / 1e9 / PEAK_HBM_GBS}
    if w.split:
        config["split_code_reread_bytes_per_step"] = sum(
            planning.code_bytes(w, p) for p in plans)
    res = {
        "metric": METRIC,
        "value": heads / (ms_per_step * 1e-3),
        "unit": "head-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": config,
        # the kernel is bound by vector-ALU issue (the cache-hot pool is only ~15% faster than
        # the HBM-streaming one); traffic is the counter-measured HBM bytes per launch
        "roofline": {"bound": "alu", "achieved": achieved_ops, "peak": PEAK_ALU_TOPS,
                     "unit": "TOP/s", "frac": achieved_ops / PEAK_ALU_TOPS, "traffic": traffic,
                     "kernel": kname, "kernel_sha": kernel_sha()},
    }
    if not args.no_cpu and S_sample:
        threads = max(1, min(16, os.cpu_count() or 1))
        print(f"[bench] CPU oracle baseline ({threads} threads, ~{args.cpu_seconds:.0f} s)",
              file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, (bits, piv, om), S_sample, args.cpu_seconds,
                                           threads)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
