"""Decode-step benchmark: head-steps/s and achieved HBM bandwidth of the packed-state decode step
on one MI355X.

Headline workload: 70 concurrent requests x 48 GDN heads, d_k = d_v = 128, nominal 6-bit per-head
map from the multiple-choice DP (widths {4,6,8}, one FP16 pivot head), initial states from 16
unquantized warm-up steps.  A step is one decode step of the whole batch (one kernel launch over
3,360 tiles).  The timed loop rotates over pool replicas (independent request batches) whose
total size exceeds twice the 256 MB Infinity Cache, so the packed state streams from HBM.  The
other synthetic workloads (tiny GDN, 4-bit contrast GDN, KDA, 12-layer split-mode stress) are
timed the same way after it and reported as flat fields of the config.

Prints one JSON line.  Inputs are synthetic (seeded); nothing is read from disk except the
committed counter summaries under profiles/ (used only while the kernel sources match them).
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
# Vector ALU issue peak without packed FP32: 256 CUs x 4 SIMDs, one wave64 instruction per SIMD
# every 4 clocks (16 lanes) at 2.4 GHz = 614.4 G wave-instructions/s = 39.3 T lane-ops/s.
PEAK_VALU_WAVE_INSTS = 256 * 4 * 2.4e9 / 4
METRIC = "decode head-steps/s + achieved HBM GB/s vs peak, nominal-6-bit GDN state pool"
COUNTERS = os.path.join(ROOT, "profiles", "{name}_counters.json")
SQ_COUNTERS = os.path.join(ROOT, "profiles", "{name}_sq.json")
KERNEL_SOURCES = ["quantized_delta_rule_amd/csrc/stepq_device.h",
                  "quantized_delta_rule_amd/csrc/stepq_k128_gdn.hip",
                  "quantized_delta_rule_amd/csrc/stepq_k128_kda.hip",
                  "quantized_delta_rule_amd/csrc/stepq_internal.h"]
# Pool replicas rotated per timed step (one-layer workloads): enough that the replicas together
# exceed twice the 256 MB Infinity Cache, so the packed state streams from HBM.
REPLICAS = {1: 12, 2: 12, 3: 10, 4: 20, 6: 12}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def committed(path_fmt, w):
    """A committed counter summary of workload w, if it was taken on the current kernels."""
    p = path_fmt.format(name=w.name)
    if not os.path.exists(p):
        return None
    c = json.load(open(p))
    return c if c.get("kernel_sha") == kernel_sha() and c.get("workload") == w.name else None


def host_cpu():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count() or 1
    return model, os.cpu_count() or 1, aff


# ----------------------------------------------------------------------------------------------
# one workload: setup and timed steps
# ----------------------------------------------------------------------------------------------

class Run:
    """Plans, pools (replicas or layers) and device inputs of one workload."""

    def __init__(self, w, dev, n_inputs, replicas=None, keep_state=False):
        import torch
        from quantized_delta_rule_amd import planning, reference, stepq, synth
        self.w = w
        t0 = time.time()
        bits, piv, om = planning.plan_arrays(w)
        self.plan_arrays = (bits, piv, om)
        kind = stepq.GDN if w.kind == "gdn" else stepq.KDA
        mode = stepq.SPLIT if w.split else stepq.FUSED
        self.multi = w.layers > 1
        self.plans = [stepq.Plan(kind, bits[l], piv[l], om[l], mode=mode, max_batch=w.B,
                                 order=w.order) for l in range(w.layers)]
        self.R = 1 if self.multi else (replicas or REPLICAS.get(w.wid, 12))
        self.units = ([(self.plans[l], l) for l in range(w.layers)] if self.multi
                      else [(self.plans[0], r) for r in range(self.R)])
        self.alg_bytes = sum(planning.algorithmic_bytes(w, p) for p in self.plans)
        self.pools, self.inputs, self.enc_ms = [], [], []
        self.S0_first = None
        for i, (plan, seed) in enumerate(self.units):
            S0 = reference.warm_state(w, seed, dev)
            pool = plan.alloc_pool(w.B)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            plan.encode(S0, pool, w.B)
            e1.record()
            e1.synchronize()
            self.enc_ms.append(e0.elapsed_time(e1))
            if i == 0:
                if keep_state:
                    self.S0_first = S0.cpu().numpy()
                self.S0_dev = S0
            del S0
            self.pools.append(pool)
            xs = synth.step_inputs_many(w, seed, range(n_inputs), "decode")
            self.inputs.append([{k: torch.from_numpy(v).to(dev) for k, v in x.items()}
                                for x in xs])
        torch.cuda.synchronize()
        self.setup_s = time.time() - t0
        self.out = torch.empty((w.B, w.H, w.d), dtype=torch.float32, device=dev)
        self.L = stepq.lib()
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        P = ctypes.c_void_p

        def call(u, j, stream=self.stream):
            plan, x = self.units[u][0], self.inputs[u][j]
            return (plan._h, P(self.pools[u].data_ptr()), w.B, P(x["q"].data_ptr()),
                    P(x["k"].data_ptr()), P(x["v"].data_ptr()), P(x["alpha"].data_ptr()),
                    P(x["beta"].data_ptr()), P(self.out.data_ptr()), stream)
        self.call = call
        # a step: every layer once (multi-layer workloads), or one replica in turn, replica-
        # major rotation so consecutive steps touch different pools
        if self.multi:
            self.steps = [[call(u, j) for u in range(len(self.units))] for j in range(n_inputs)]
        else:
            flat = [call(u, j) for u in range(self.R) for j in range(n_inputs)]
            self.steps = [[flat[(i % self.R) * n_inputs + (i // self.R) % n_inputs]]
                          for i in range(len(flat))]
        self.launches = len(self.steps[0])

    def run(self, i):
        for c in self.steps[i % len(self.steps)]:
            if self.L.stepq_decode_step(*c):
                raise RuntimeError(self.L.stepq_last_error().decode())

    def drain(self):
        import torch
        torch.cuda.synchronize()
        for p in self.plans:
            p.sync()

    def check_status(self):
        if any(p.status() != 0 for p in self.plans):
            raise RuntimeError(f"{self.w.name}: status flags raised during the benchmark")

    def timed(self, steps, warmup):
        """warmup untimed steps, then `steps` steps back to back on the launch stream between
        one pair of HIP events (the kernel time per launch includes the dependency gap between
        back-to-back launches); split-mode writebacks run on the plans' side streams, covered by
        the host clock that brackets the same region."""
        import torch
        for i in range(warmup):
            self.run(i)
        self.drain()
        if not self.multi:
            flush_infinity_cache()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record()
        # the rotation continues from the warm-up: a short timed run does not start on the
        # replicas the warm-up has just left in the Infinity Cache
        for i in range(warmup, warmup + steps):
            self.run(i)
        ev1.record()
        self.drain()
        wall = time.perf_counter() - t0
        self.check_status()
        avg_k = ev0.elapsed_time(ev1) / (steps * self.launches)
        ms_per_step = wall * 1e3 / steps
        step_ms = ms_per_step if self.w.split else avg_k * self.launches
        return dict(ms_per_step=ms_per_step, kernel_ms=avg_k, step_ms=step_ms)

    def summary(self, t):
        w = self.w
        heads = w.B * w.H * w.layers
        return dict(head_steps_per_s=heads / (t["ms_per_step"] * 1e-3),
                    us_per_step=t["ms_per_step"] * 1e3,
                    hbm_GBps=self.alg_bytes / (t["step_ms"] * 1e-3) / 1e9,
                    hbm_frac=self.alg_bytes / (t["step_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS)


_FLUSH = []


def flush_infinity_cache(nbytes=1 << 29):
    """Writes 512 MB (twice the 256 MB Infinity Cache) of zeros and waits, so that a timed run
    that follows finds none of its pools cache-resident from the set-up or the warm-up."""
    import torch
    if not _FLUSH:
        _FLUSH.append(torch.empty(nbytes, dtype=torch.uint8, device="cuda"))
    _FLUSH[0].zero_()
    torch.cuda.synchronize()


def copy_ceiling(dev, nbytes=1 << 30, reps=5):
    """Device-to-device copy of nbytes, event-timed: (read + write bytes) / time."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    e1.synchronize()
    gbps = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbps


def cpu_baseline(run, budget_s, threads):
    """The oracle (as it stands) on a bounded sample of the same workload: every tile of replica
    0 from its initial state, through the workload's first n decode steps (n sized so the run
    takes about budget_s on `threads` threads)."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    from quantized_delta_rule_amd import synth
    w = run.w
    bits, piv, om = run.plan_arrays
    S0 = run.S0_first
    tiles = list(range(w.B * w.H))
    heads = [oracle.Head(bits[0, h], piv[0, h], om[0, h], order=w.order) for h in range(w.H)]
    with ThreadPoolExecutor(threads) as ex:
        segs = list(ex.map(lambda t: heads[t % w.H].encode(S0[t]), tiles))
    x0 = synth.step_inputs(w, 0, 0, "decode")
    a0 = synth.alpha_rows(w, x0["alpha"])
    t0 = time.perf_counter()
    for t in tiles[:8]:
        b, h = divmod(t, w.H)
        heads[h].step(segs[t].copy(), x0["q"][b, h], x0["k"][b, h], x0["v"][b, h], a0[b, h],
                      x0["beta"][b, h])
    per = (time.perf_counter() - t0) / 8
    n = int(max(1, min(w.steps, budget_s * threads / (per * len(tiles)))))
    xs = synth.step_inputs_many(w, 0, range(n), "decode")
    ar = [synth.alpha_rows(w, x["alpha"]) for x in xs]

    def work(chunk):
        for s in range(n):
            x, a = xs[s], ar[s]
            for t in chunk:
                b, h = divmod(t, w.H)
                heads[h].step(segs[t], x["q"][b, h], x["k"][b, h], x["v"][b, h], a[b, h],
                              x["beta"][b, h])
        return len(chunk) * n

    chunks = [tiles[i::threads] for i in range(threads)]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        done = sum(ex.map(work, chunks))
    dt = time.perf_counter() - t0
    model, nproc, aff = host_cpu()
    return {"value": done / dt, "unit": "head-steps/s", "cores": threads, "kind": "oracle",
            "sample": f"all {len(tiles)} tiles of replica 0, decode steps 0..{n - 1} of the "
                      f"workload ({done} tile-steps in {dt:.1f} s) on {threads} threads; host "
                      f"{model}, nproc {nproc}, {aff} CPUs in this process's affinity"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=600)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--also", default="1,3,4,5",
                    help="other workloads timed after the headline one (flat config fields); "
                         "empty for none")
    ap.add_argument("--replicas", type=int, default=None,
                    help="pool replicas rotated per step (one-layer workloads)")
    ap.add_argument("--inputs", type=int, default=4, help="distinct input sets per replica")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the labelled extras (spread, cache-hot, graph replay, copy)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run only the 1 GiB device copy (counter scale calibration) after the "
                         "headline workload")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the decode step "
              "shards by request or head with no cross-GPU traffic, so N GPUs run N copies.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from quantized_delta_rule_amd import synth

    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[args.workload]
    log(f"workload {w.wid} {w.name}: planning and initial states")
    run = Run(w, dev, args.inputs, args.replicas, keep_state=not args.no_cpu)
    plans = run.plans
    log(f"{len(run.units)} {'layers' if run.multi else 'replicas'} x "
        f"{plans[0].bytes_per_request * w.B / 2**20:.1f} MiB pool "
        f"({plans[0].bits_per_value:.3f} bits/value), setup {run.setup_s:.1f} s, timing")
    t = run.timed(args.steps, args.warmup)
    ms_per_step, avg_k, step_ms = t["ms_per_step"], t["kernel_ms"], t["step_ms"]
    heads = w.B * w.H * w.layers
    kname = ("k_gdn" if w.kind == "gdn" else "k_kda") + f"<{w.d}, " + \
        ("READ> + WRITE (side stream)" if w.split else "FUSED>")

    config = {
        "workload": f"{w.name}: {w.B} requests x {w.layers} layer(s) x {w.H} "
                    f"{w.kind.upper()} heads, d_k=d_v={w.d}, nominal {w.nominal}-bit "
                    + (f"MC-DP map {w.choices}" if w.alloc == "mcdp" else
                       f"Lagrangian row map {w.choices}" if w.alloc == "lagrangian" else
                       f"fixed head widths {w.fixed_bits}")
                    + f", {w.n_pivots} FP16 pivot unit(s), "
                    + (f"{w.layers} layers back to back per step, refit and writeback on a side "
                       f"stream" if run.multi else f"{run.R} rotating pool replicas"),
        "bits_per_value": round(plans[0].bits_per_value, 4),
        "pool_mib_per_replica": round(sum(p.bytes_per_request for p in plans) * w.B / 2**20, 2),
        "algorithmic_bytes_per_step": run.alg_bytes,
        "kernel_ms_mean": avg_k,
        "launches_per_step": run.launches,
    }

    # ---- labelled extras (not the headline): a sustained run, per-launch spread, cache-hot
    # pool, graph replay
    if not run.multi and not args.no_extras and not args.copy_calib:
        # 600 back-to-back steps: on the 6-bit GDN workload a 20-step run reads several percent
        # faster than 100 or 600 steps do, with the Infinity Cache flushed before each
        ts = run.timed(600, args.warmup)
        config["sustained_600_kernel_ms"] = ts["kernel_ms"]
        config["sustained_600_hbm_frac"] = (run.alg_bytes / run.launches / (ts["kernel_ms"] * 1e-3)
                                             / 1e9 / PEAK_HBM_GBS)
        nspread = min(100, args.steps)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(nspread)]
        for i in range(nspread):
            ev[i][0].record()
            run.run(i)
            ev[i][1].record()
        run.drain()
        k_ms = np.array([a.elapsed_time(b) for a, b in ev])
        config["event_bracketed_launch_ms_p10_p50_p90"] = [float(np.percentile(k_ms, p))
                                                           for p in (10, 50, 90)]
        h0, h1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        h0.record()
        for _ in range(50):
            run.L.stepq_decode_step(*run.steps[0][0])
        h1.record()
        run.drain()
        hot_ms = h0.elapsed_time(h1) / 50
        config["cache_hot_single_pool_kernel_ms"] = hot_ms
        config["cache_hot_single_pool_GBps"] = run.alg_bytes / (hot_ms * 1e-3) / 1e9
        if not w.split:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
                for r in range(run.R):
                    if run.L.stepq_decode_step(*(run.steps[r][0][:-1] + (cs,))):
                        raise RuntimeError(run.L.stepq_last_error().decode())
            g.replay()
            run.drain()
            reps = max(1, args.steps // run.R)
            g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            g0.record()
            for _ in range(reps):
                g.replay()
            g1.record()
            run.drain()
            graph_ms = g0.elapsed_time(g1) / (reps * run.R)
            config["graph_replay_ms_per_step"] = graph_ms
            config["graph_replay_head_steps_per_s"] = heads / (graph_ms * 1e-3)
            del g
        run.check_status()
    # encoding an fp32 state into the pool (the hand-off from prefill): 20 back-to-back encodes
    # of the first unit's initial state into one spare pool between one event pair; bytes =
    # fp32 state read + packed write.  (The setup's first encodes into freshly allocated pools
    # run slower and are not this figure.)
    plan0 = run.units[0][0]
    spare = plan0.alloc_pool(w.B)
    plan0.encode(run.S0_dev, spare, w.B)
    torch.cuda.synchronize()  # the spare pool's first touch stays outside the timed encodes
    x0, x1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    x0.record()
    for _ in range(20):
        plan0.encode(run.S0_dev, spare, w.B)
    x1.record()
    x1.synchronize()
    enc = x0.elapsed_time(x1) / 20
    config["encode_first_touch_ms_median"] = float(np.median(run.enc_ms))
    del spare
    enc_bytes = w.B * w.H * w.d * w.d * 4 + w.B * float(np.mean([p.bytes_per_request
                                                                   for p in plans]))
    config["encode_ms_per_batch"] = enc
    config["encode_hbm_frac"] = enc_bytes / (enc * 1e-3) / 1e9 / PEAK_HBM_GBS
    if w.split:
        from quantized_delta_rule_amd import planning
        config["split_code_reread_bytes_per_step"] = sum(planning.code_bytes(w, p) for p in plans)

    # ---- copy ceiling (also the counter calibration run under rocprofv3 --pmc)
    if args.copy_calib or not args.no_extras:
        config["copy_ceiling_GBps"] = copy_ceiling(dev)

    # ---- the roofline of the dominant kernel: algorithmic HBM bytes per launch over its
    # event-timed average launch duration, against the 8 TB/s peak
    per_launch = run.alg_bytes / run.launches
    achieved = per_launch / (avg_k * 1e-3) / 1e9
    traffic = None
    c = committed(COUNTERS, w)
    if c is not None:
        traffic = c["hbm_bytes_per_launch"]
    roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS, "traffic": traffic, "kernel": kname,
            "kernel_sha": kernel_sha(), "algorithmic_bytes_per_launch": per_launch}
    if run.multi:
        # split mode: the step (readout + side-stream writeback of every layer) by the host
        # clock; the launch-stream figure covers the readout kernels only
        roof["achieved"] = run.alg_bytes / (step_ms * 1e-3) / 1e9
        roof["frac"] = roof["achieved"] / PEAK_HBM_GBS
    if traffic is not None:
        # HBM bytes by the committed counters (FETCH_SIZE + WRITE_SIZE, scaled by the copy
        # calibration) over this run's time of the same launches
        span_ms = step_ms / run.launches if run.multi else avg_k
        roof["traffic_GBps"] = traffic / (span_ms * 1e-3) / 1e9
        roof["traffic_frac"] = roof["traffic_GBps"] / PEAK_HBM_GBS
    if "copy_ceiling_GBps" in config:
        roof["frac_of_copy_ceiling"] = roof["achieved"] / config["copy_ceiling_GBps"]
    sq = committed(SQ_COUNTERS, w)
    if sq is not None and run.multi:
        # split mode: the readout and writeback kernels' VALU wave-instructions of one step
        # over the issue capacity of the step's host-clock time
        roof["valu_insts_per_step"] = sq["sq_insts_valu_per_step"]
        roof["valu_issue_frac"] = sq["sq_insts_valu_per_step"] / (step_ms * 1e-3 *
                                                                  PEAK_VALU_WAVE_INSTS)
        roof["valu_lane_ops_per_entry"] = sq["sq_insts_valu_per_step"] * 64 / sq["entries"]
        roof["valu_lane_ops_per_entry_by_kernel"] = sq["lane_ops_per_entry_by_kernel"]
    elif sq is not None:
        # vector-ALU issue: measured VALU wave-instructions per launch (SQ_INSTS_VALU) over the
        # issue capacity of the launch's duration
        roof["valu_insts_per_launch"] = sq["sq_insts_valu_per_launch"]
        roof["valu_issue_frac"] = sq["sq_insts_valu_per_launch"] / (avg_k * 1e-3 *
                                                                     PEAK_VALU_WAVE_INSTS)
        roof["valu_lane_ops_per_entry"] = sq["sq_insts_valu_per_launch"] * 64 / sq["entries"]

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
        "roofline": roof,
    }

    if not args.no_cpu:
        model, nproc, aff = host_cpu()
        # the machine's CPU share: OMP_NUM_THREADS where set (16 per GPU), else every CPU we may use
        share = int(os.environ.get("OMP_NUM_THREADS", aff))
        threads = max(1, min(aff, share))
        log(f"CPU oracle baseline ({threads} threads of nproc {nproc}, ~{args.cpu_seconds:.0f} s)")
        res["cpu_baseline"] = cpu_baseline(run, args.cpu_seconds, threads)

    # ---- the other workloads: flat fields (head-steps/s, us/step, HBM fraction)
    also = [] if (args.copy_calib or not args.also) else [int(x) for x in args.also.split(",")]
    del run
    torch.cuda.empty_cache()
    for wid in also:
        if wid == w.wid:
            continue
        wx = synth.WORKLOADS[wid]
        log(f"workload {wid} {wx.name}: setup")
        rx = Run(wx, dev, args.inputs)
        # at least 200 timed steps: a short run of a small launch measures the host clock's
        # bracketing more than the steps
        nx = max(args.steps, 200)
        tx = rx.timed(nx, max(args.warmup, 20))
        sx = rx.summary(tx)
        sx["steps"] = nx
        cx = committed(COUNTERS, wx)
        if cx is not None:
            sx["traffic_frac"] = (cx["hbm_bytes_per_launch"] * rx.launches /
                                  (tx["step_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS)
        log(f"workload {wid}: {sx['head_steps_per_s'] / 1e6:.1f} M head-steps/s, "
            f"{sx['us_per_step']:.1f} us/step, HBM frac {sx['hbm_frac']:.3f} "
            f"(setup {rx.setup_s:.0f} s)")
        for k, v in sx.items():
            config[f"w{wid}_{k}"] = v
        del rx
        torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
