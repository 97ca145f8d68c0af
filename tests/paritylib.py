"""Helpers of the GPU parity tests: the oracle builds every plan, initial state and expected
value; the GPU library runs the same seeded inputs through its C ABI; results are compared per
step with the acceptance rule of the decode path:

* readout: relative L2 error <= 1e-4 per tile and step;
* row/column factors and FP16 pivots: bit-exact;
* codes: bit-exact, except entries whose oracle pre-rounding value lies within 1e-5 of a
  rounding boundary (x.5); after such a mismatch the oracle continues from the GPU's segment.

Beside that, a subset of tiles is checked against the plain binary64 reference of the step
(oracle/plain.py) with the decision-aware rule of tests/plainparity.py: readouts within their
binary32 error bound (and relative L2 <= 1e-6), every binary16 factor, pivot value and code equal
to the binary64 rounding or adjacent to it with the binary64 value inside the binary32 error
window of the boundary.
"""
from __future__ import annotations

import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import plainparity as PP
from quantized_delta_rule_amd import synth

BOUNDARY_TOL = 1e-5
READOUT_TOL = 1e-4


def log(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------------------------------
# plans (oracle side)
# ------------------------------------------------------------------------------------------

def omega_from_steps(w, layer, phase, steps, xs=None):
    """omega [H, d] = mean over requests and steps of g_i^2 (oracle row impact).  xs: the
    steps' inputs if already drawn."""
    acc = np.zeros((w.H, w.d))
    for s in range(steps):
        x = synth.step_inputs(w, layer, s, phase) if xs is None else xs[s]
        a = synth.alpha_rows(w, x["alpha"])
        for h in range(w.H):
            acc[h] += oracle.row_impact(x["q"][:, h], x["k"][:, h], a[:, h], x["beta"][:, h],
                                        order=w.order)
    return (acc / steps).astype(np.float32)


def measured_distortion(w, omegas, n_req=8, samples=(32, 64)):
    """KDA d_u(b): per key row, the squared reconstruction error summed over the row, of the
    uniform-b quantizer without pivots, averaged over calibration states (fp32 runs from zero on
    the calibration stream, n_req requests, states at the sample steps)."""
    d, H = w.d, w.H
    choices = list(w.choices)
    du = np.zeros((w.layers, H, d, len(choices)))
    for layer in range(w.layers):
        S = np.zeros((n_req * H, d, d), np.float32)
        cnt = 0
        prev = 0
        for smp in samples:
            xs = [synth.step_inputs(w, layer, s, "calib") for s in range(prev, smp)]
            prev = smp
            q = np.stack([x["q"][:n_req].reshape(-1, d) for x in xs])
            k = np.stack([x["k"][:n_req].reshape(-1, d) for x in xs])
            v = np.stack([x["v"][:n_req].reshape(-1, d) for x in xs])
            a = np.stack([synth.alpha_rows(w, x["alpha"])[:n_req].reshape(-1, d) for x in xs])
            be = np.stack([x["beta"][:n_req].reshape(-1) for x in xs])
            oracle.fp32_run(S, q, k, v, a, be, order=w.order)
            for t in range(n_req * H):
                h = t % H
                for ci, b in enumerate(choices):
                    head = oracle.Head(np.full(d, b, np.int8), np.zeros(d, np.uint8),
                                       omegas[layer, h])
                    Sh, _, _, _ = head.unpack(head.encode(S[t]))
                    err = (S[t].astype(np.float64) - Sh) ** 2
                    du[layer, h, :, ci] += err.sum(axis=1)
            cnt += 1
        du[layer] /= cnt * n_req
    return du


def oracle_plan(w, omegas=None):
    """(bits, pivot, omega) each [layers, H, d] for workload w, computed by the oracle (omegas
    [layers, H, d] if already computed)."""
    L_, H, d = w.layers, w.H, w.d
    phase, nsteps = ("calib", w.calib_steps) if w.calib_steps else ("warmup", w.warmup)
    if omegas is None:
        omegas = np.stack([omega_from_steps(w, l, phase, nsteps) for l in range(L_)])
    bits = np.zeros((L_, H, d), np.int8)
    piv = np.zeros((L_, H, d), np.uint8)
    if w.alloc == "fixed":
        for h, b in enumerate(w.fixed_bits):
            if b == 0:
                piv[:, h] = 1
                bits[:, h] = max(w.choices)
            else:
                bits[:, h] = b
        return bits, piv, omegas
    l_u, s_u = synth.plan_tables(w)
    Lw = oracle.lifetime_weight(l_u, w.horizon)
    choices = list(w.choices)
    if w.du == "synthetic":
        du = synth.synthetic_distortion(s_u, choices)
    else:
        du = measured_distortion(w, omegas).reshape(-1, len(choices))
    risk = Lw * du[:, -1]
    pv = oracle.select_pivots(risk, w.n_pivots)
    keep = np.setdiff1d(np.arange(Lw.size), pv)
    if w.alloc == "mcdp":
        cost = Lw[keep, None] * du[keep]
        b_keep, _ = oracle.mcdp_allocate(cost, choices, w.nominal * keep.size)
    else:
        n = np.full(keep.size, float(d))
        b_keep, _ = oracle.lagrangian_allocate(Lw[keep], du[keep], n, choices,
                                               w.nominal * float(n.sum()))
    unit_bits = np.full(Lw.size, max(choices), np.int64)
    unit_bits[keep] = b_keep
    unit_piv = np.zeros(Lw.size, np.uint8)
    unit_piv[pv] = 1
    if w.kind == "gdn":
        bits[:] = unit_bits.reshape(L_, H)[:, :, None]
        piv[:] = unit_piv.reshape(L_, H)[:, :, None]
    else:
        bits[:] = unit_bits.reshape(L_, H, d)
        piv[:] = unit_piv.reshape(L_, H, d)
    return bits, piv, omegas


def warm_state(w, layer, threads=16, xs=None):
    """Initial fp32 states [B*H, d, d]: w.warmup unquantized steps from zero (oracle).  xs: the
    warm-up steps' inputs if already drawn."""
    d = w.d
    S = np.zeros((w.B * w.H, d, d), np.float32)
    if xs is None:
        xs = [synth.step_inputs(w, layer, s, "warmup") for s in range(w.warmup)]
    q = np.stack([x["q"].reshape(-1, d) for x in xs])
    k = np.stack([x["k"].reshape(-1, d) for x in xs])
    v = np.stack([x["v"].reshape(-1, d) for x in xs])
    a = np.stack([synth.alpha_rows(w, x["alpha"]).reshape(-1, d) for x in xs])
    be = np.stack([x["beta"].reshape(-1) for x in xs])
    oracle.fp32_run(S, q, k, v, a, be, threads=threads, order=w.order)
    return S


# ------------------------------------------------------------------------------------------
# comparison
# ------------------------------------------------------------------------------------------

class Mismatch(AssertionError):
    pass


def compare_segment(head, seg_gpu, seg_orc, pre, where):
    """Returns the number of allowed boundary mismatches; raises on anything else."""
    if np.array_equal(seg_gpu, seg_orc):
        return 0
    Sg, rg, cg, zg = head.unpack(seg_gpu)
    So, ro, co, zo = head.unpack(seg_orc)
    if not np.array_equal(rg, ro):
        i = np.nonzero(rg != ro)[0]
        raise Mismatch(f"{where}: row factors differ at rows {i[:8]} gpu {rg[i[:4]]} orc {ro[i[:4]]}")
    if not np.array_equal(cg, co):
        j = np.nonzero(cg != co)[0]
        raise Mismatch(f"{where}: column factors differ at cols {j[:8]} gpu {cg[j[:4]]} orc {co[j[:4]]}")
    piv = head.pivot.astype(bool)
    if piv.any() and not np.array_equal(Sg[piv].view(np.uint32), So[piv].view(np.uint32)):
        raise Mismatch(f"{where}: FP16 pivot rows differ")
    bad = zg != zo
    if bad.any():
        frac = np.abs(np.abs(pre[bad]) - np.floor(np.abs(pre[bad])) - 0.5)
        if np.any(frac > BOUNDARY_TOL) or np.any(np.abs(zg[bad].astype(int) - zo[bad]) > 1):
            ii = np.argwhere(bad)[:6]
            raise Mismatch(f"{where}: codes differ away from a rounding boundary at {ii.tolist()}"
                           f" gpu {zg[bad][:6]} orc {zo[bad][:6]} pre {pre[bad][:6]}")
        return int(bad.sum())
    # codes equal but bytes differ: padding or stray bits
    raise Mismatch(f"{where}: segments differ outside codes/factors")


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (n if n > 0 else 1.0))


class Tracker:
    def __init__(self):
        self.boundary = 0
        self.worst_readout = 0.0
        self.steps = 0
        self.plain = PP.PlainStats()
        self.t0 = time.time()

    def summary(self):
        return (f"{self.steps} steps, boundary mismatches {self.boundary}, worst readout "
                f"{self.worst_readout:.2e}; {self.plain.summary()}")


def check_tile(tr, head, seg_o, t, gs, out_gpu, q, k, v, a, beta, where, plain_check=False):
    """One tile of one step: the oracle steps its copy seg_o[t] and the GPU's readout out_gpu and
    segment gs must match it (readout rel L2 <= READOUT_TOL; segment by compare_segment).  After
    an allowed boundary mismatch the oracle's copy becomes the GPU's segment (teacher forcing).
    With plain_check the GPU's step is also checked against the plain binary64 reference."""
    before = seg_o[t].copy() if plain_check else None
    dbg = head.step_dbg(seg_o[t], q, k, v, a, beta)
    err = rel_l2(out_gpu, dbg["out"])
    tr.worst_readout = max(tr.worst_readout, err)
    if err > READOUT_TOL:
        raise Mismatch(f"{where}: readout rel L2 {err:.3e}")
    nb = compare_segment(head, gs, seg_o[t], dbg["pre"], where)
    if nb:
        tr.boundary += nb
        seg_o[t] = np.array(gs, np.uint8, copy=True)
    if plain_check:
        PP.check_step(head.bits, head.pivot, head.omega, head.order, before, gs, out_gpu,
                      dbg["z0"], q, k, v, a, beta, where + " vs plain", tr.plain)
    return nb


def _plain_subset(tiles, n):
    """n tiles spread evenly over the checked tiles (all of them if there are at most n)."""
    tiles = list(tiles)
    if len(tiles) <= n:
        return set(tiles)
    return set(tiles[int(i)] for i in np.linspace(0, len(tiles) - 1, n))


# ------------------------------------------------------------------------------------------
# one-layer run: GPU through the C ABI, oracle on the chosen tiles
# ------------------------------------------------------------------------------------------

def run_layer(w, layer, bits, piv, om, steps, tiles=None, mode=0, S0=None, check_encode=True,
              plan=None, pool=None, inputs=None, plain_tiles=8):
    """Encodes S0 (oracle warm-up unless given) on the GPU, checks the encode against the
    oracle, then runs `steps` decode steps and checks every step on `tiles` (default: all),
    bit for bit against the oracle and, on `plain_tiles` of them, against the plain binary64
    reference.  Returns (Tracker, plan, pool)."""
    import torch
    from quantized_delta_rule_amd import stepq

    d, H, B = w.d, w.H, w.B
    kind = stepq.GDN if w.kind == "gdn" else stepq.KDA
    if plan is None:
        plan = stepq.Plan(kind, bits, piv, om, mode=mode, max_batch=B, order=w.order)
    heads = [oracle.Head(bits[h], piv[h], om[h], order=w.order) for h in range(H)]
    bpr = plan.bytes_per_request
    segs = [plan.head_segment(h) for h in range(H)]
    tiles = list(range(B * H)) if tiles is None else list(tiles)
    pset = _plain_subset(tiles, plain_tiles)
    dev = torch.device("cuda:0")
    if S0 is None:
        S0 = warm_state(w, layer)
    if pool is None:
        pool = plan.alloc_pool(B)
        plan.encode(torch.from_numpy(S0).to(dev), pool, B)
        torch.cuda.synchronize()
    tr = Tracker()

    def gpu_seg(host_pool, t):
        b, h = divmod(t, H)
        off, n = segs[h]
        return host_pool[b * bpr + off: b * bpr + off + n]

    seg_o = {}
    host = pool.cpu().numpy()
    for t in tiles:
        h = t % H
        so, dbg = heads[h].encode_dbg(S0[t])
        if check_encode:
            tr.boundary += compare_segment(heads[h], gpu_seg(host, t), so, dbg["pre"],
                                           f"encode tile {t} (head {h})")
            if t in pset:
                PP.check_encode(bits[h], piv[h], om[h], S0[t], gpu_seg(host, t), dbg["z0"],
                                f"encode tile {t} (head {h}) vs plain", tr.plain)
        seg_o[t] = gpu_seg(host, t).copy() if not check_encode else so
    for s in range(steps):
        x = synth.step_inputs(w, layer, s, "decode") if inputs is None else inputs(s)
        a_rows = synth.alpha_rows(w, x["alpha"])
        g = {k_: torch.from_numpy(v_).to(dev) for k_, v_ in x.items()}
        out = torch.empty((B, H, d), dtype=torch.float32, device=dev)
        plan.step(pool, B, g["q"], g["k"], g["v"], g["alpha"], g["beta"], out)
        if mode == 1:
            plan.sync()
        torch.cuda.synchronize()
        host = pool.cpu().numpy()
        outh = out.cpu().numpy()
        for t in tiles:
            b, h = divmod(t, H)
            check_tile(tr, heads[h], seg_o, t, gpu_seg(host, t), outh[b, h], x["q"][b, h],
                       x["k"][b, h], x["v"][b, h], a_rows[b, h], x["beta"][b, h],
                       f"step {s} tile {t} (head {h})", plain_check=t in pset)
        tr.steps += 1
    return tr, plan, pool


def sample_tiles(w, per_head=1, extra=0, seed=0):
    """Tiles to check: per_head requests for every head (request index spread over the batch),
    plus `extra` random tiles."""
    g = np.random.default_rng(seed)
    tiles = []
    for h in range(w.H):
        for j in range(per_head):
            b = (h * 7 + j * 13) % w.B
            tiles.append(b * w.H + h)
    tiles += list(g.choice(w.B * w.H, extra, replace=False))
    return sorted(set(int(t) for t in tiles))


def layer_inputs(w, layers, step, phase="decode", workers=12):
    """One step's inputs of every layer, drawn in parallel (each layer has its own stream)."""
    with ThreadPoolExecutor(min(workers, len(layers))) as ex:
        return list(ex.map(lambda l: synth.step_inputs(w, l, step, phase), layers))


def split_setup(w, workers=12):
    """Per layer: omega from the warm-up inputs and the oracle's warm-up state, both from one
    draw of those inputs; then the oracle plan.  Returns (plans_np, S0 per layer)."""
    phase, nsteps = ("calib", w.calib_steps) if w.calib_steps else ("warmup", w.warmup)
    assert phase == "warmup"
    omegas, S0s = [], []
    for l in range(w.layers):
        with ThreadPoolExecutor(workers) as ex:
            xs = list(ex.map(lambda s: synth.step_inputs(w, l, s, "warmup"), range(w.warmup)))
        omegas.append(omega_from_steps(w, l, phase, nsteps, xs=xs))
        S0s.append(warm_state(w, l, xs=xs))
        del xs
        log(f"[parity] layer {l}: omega and warm-up state")
    return oracle_plan(w, np.stack(omegas)), S0s


def run_layers_split(w, plans_np, steps, tiles_per_layer, S0s=None, fused_check_layer=0,
                     plain_per_layer=1):
    """Multi-layer workload, layers stepped back to back each decode step with the refit and
    writeback on the library's side stream (split mode).  Every step: the oracle checks the
    sampled tiles of every layer bit for bit, `plain_per_layer` of each layer's sampled tiles
    (rotating) are checked against the plain binary64 reference, and one layer also runs a
    fused plan side by side on the same inputs, which must match the split result bit for bit.
    The next step's inputs are drawn while the current step is checked."""
    import torch
    from quantized_delta_rule_amd import stepq

    d, H, B = w.d, w.H, w.B
    dev = torch.device("cuda:0")
    bits, piv, om = plans_np
    plans, pools, heads, segs_o, tiles, segmap = [], [], [], [], [], []
    for l in range(w.layers):
        plan = stepq.Plan(stepq.GDN, bits[l], piv[l], om[l], mode=stepq.SPLIT, max_batch=B)
        S0 = warm_state(w, l) if S0s is None else S0s[l]
        pool = plan.alloc_pool(B)
        plan.encode(torch.from_numpy(S0).to(dev), pool, B)
        hl = [oracle.Head(bits[l, h], piv[l, h], om[l, h]) for h in range(H)]
        tl = list(tiles_per_layer(l))
        so = {t: hl[t % H].encode(S0[t]) for t in tl}
        if l == fused_check_layer:
            fplan = stepq.Plan(stepq.GDN, bits[l], piv[l], om[l])
            fpool = fplan.alloc_pool(B)
            fplan.encode(torch.from_numpy(S0).to(dev), fpool, B)
        if S0s is not None:
            S0s[l] = None
        del S0
        bpr = plan.bytes_per_request
        segmap.append({t: (t // H) * bpr + plan.head_segment(t % H)[0] for t in tl})
        plans.append(plan)
        pools.append(pool)
        heads.append(hl)
        segs_o.append(so)
        tiles.append(tl)
        log(f"[parity] layer {l}: encoded, {len(tl)} sampled tiles")
    torch.cuda.synchronize()
    tr = Tracker()
    pool_ex = ThreadPoolExecutor(1)
    nxt = pool_ex.submit(layer_inputs, w, range(w.layers), 0)
    for s in range(steps):
        xs = nxt.result()
        if s + 1 < steps:
            nxt = pool_ex.submit(layer_inputs, w, range(w.layers), s + 1)
        outs = []
        for l in range(w.layers):
            g = {k_: torch.from_numpy(v_).to(dev) for k_, v_ in xs[l].items()}
            out = torch.empty((B, H, d), dtype=torch.float32, device=dev)
            plans[l].step(pools[l], B, g["q"], g["k"], g["v"], g["alpha"], g["beta"], out)
            outs.append(out)
            if l == fused_check_layer:
                fout = torch.empty_like(out)
                fplan.step(fpool, B, g["q"], g["k"], g["v"], g["alpha"], g["beta"], fout)
        for p in plans:
            p.sync()
        torch.cuda.synchronize()
        fl = fused_check_layer
        if not torch.equal(pools[fl], fpool) or not torch.equal(outs[fl], fout):
            raise Mismatch(f"step {s}: split and fused results differ on layer {fl}")
        for l in range(w.layers):
            # only the sampled tiles' segments and readouts leave the device
            gsegs = {t: pools[l][segmap[l][t]: segmap[l][t] + plans[l].head_segment(t % H)[1]]
                     .cpu().numpy() for t in tiles[l]}
            outh = {t: outs[l][t // H, t % H].cpu().numpy() for t in tiles[l]}
            a_rows = synth.alpha_rows(w, xs[l]["alpha"])
            x = xs[l]
            pl = tiles[l][s % len(tiles[l])] if plain_per_layer else None
            for t in tiles[l]:
                b, h = divmod(t, H)
                check_tile(tr, heads[l][h], segs_o[l], t, gsegs[t], outh[t], x["q"][b, h],
                           x["k"][b, h], x["v"][b, h], a_rows[b, h], x["beta"][b, h],
                           f"step {s} layer {l} tile {t}", plain_check=t == pl)
        tr.steps += 1
        if s % 8 == 7 or s == steps - 1:
            log(f"[parity] step {s} ok ({tr.summary()}, {time.time() - tr.t0:.0f} s)")
    pool_ex.shutdown()
    return tr, plans
