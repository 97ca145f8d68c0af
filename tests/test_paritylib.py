"""CPU tests of the GPU parity checker (tests/paritylib.py): its acceptance rule is exercised
with a simulated GPU result -- the oracle's own step, with a planted difference -- so that every
branch (allowed boundary mismatch and teacher forcing, mismatch away from a boundary, factor
mismatch, readout tolerance) runs without a GPU."""
import numpy as np
import pytest

import oracle
import paritylib as P
from oracle import codec


def _tile(seed=3, d=64, bits=6):
    g = np.random.default_rng(seed)
    head = oracle.Head(np.full(d, bits, np.int8), np.zeros(d, np.uint8),
                       g.exponential(1.0, d).astype(np.float32))
    S = (g.standard_normal((d, d)) * 0.3).astype(np.float32)
    seg = head.encode(S)
    x = dict(q=g.standard_normal(d).astype(np.float32), k=g.standard_normal(d).astype(np.float32),
             v=g.standard_normal(d).astype(np.float32), a=np.full(d, 0.97, np.float32), beta=0.6)
    x["q"] /= np.linalg.norm(x["q"])
    x["k"] /= np.linalg.norm(x["k"])
    return head, seg, x


def _gpu_like(head, seg, x):
    """The step as the GPU computes it (bit-identical to the oracle): (segment, readout, pre)."""
    s = seg.copy()
    out, _, pre, _ = head.step(s, x["q"], x["k"], x["v"], x["a"], x["beta"], want_state=True)
    return s, out, pre


def _flip_code(head, seg, i, j, delta):
    b, p = head.bits, head.pivot
    z, r16, c16, h16 = codec.unpack(seg, b, p, head.dv)
    z[i, j] += delta
    return codec.pack(b, p, head.dv, z, r16, c16, h16)


def test_equal_segments_pass():
    head, seg, x = _tile()
    gs, out, pre = _gpu_like(head, seg, x)
    assert P.compare_segment(head, gs, gs.copy(), pre, "same") == 0


def test_boundary_mismatch_is_counted_and_teacher_forced():
    head, seg, x = _tile()
    gs, out, pre = _gpu_like(head, seg, x)
    z = codec.unpack(gs, head.bits, head.pivot, head.dv)[0]
    i, j = np.argwhere((np.abs(z) < 31) & (np.abs(z) > 0))[0]
    # the simulated GPU rounded this entry the other way; make its pre-rounding value sit
    # 1e-6 from the .5 boundary between the two codes
    gpu = _flip_code(head, gs, i, j, 1)
    pre = pre.copy()
    pre[i, j] = z[i, j] + 0.5 - 1e-6
    assert P.compare_segment(head, gpu, gs, pre, "boundary") == 1
    # the one-step driver counts it and continues from the GPU's segment
    tr = P.Tracker()
    seg_o = {0: seg.copy()}
    orig = head.step_dbg

    def step_dbg_near_tie(s, *a):
        r = orig(s, *a)
        r["pre"] = pre
        return r

    head.step_dbg = step_dbg_near_tie
    assert P.check_tile(tr, head, seg_o, 0, gpu, out, x["q"], x["k"], x["v"], x["a"],
                        x["beta"], "drive") == 1
    assert tr.boundary == 1 and np.array_equal(seg_o[0], gpu)


def test_mismatch_away_from_boundary_raises():
    head, seg, x = _tile()
    gs, out, pre = _gpu_like(head, seg, x)
    z = codec.unpack(gs, head.bits, head.pivot, head.dv)[0]
    i, j = np.argwhere(np.abs(z) < 31)[0]
    gpu = _flip_code(head, gs, i, j, 1)
    pre = pre.copy()
    pre[i, j] = z[i, j] + 0.25
    with pytest.raises(P.Mismatch, match="away from a rounding boundary"):
        P.compare_segment(head, gpu, gs, pre, "far")
    # a code two steps away is never a boundary case
    gpu2 = _flip_code(head, gs, i, j, 2 if z[i, j] < 29 else -2)
    pre[i, j] = z[i, j] + 0.5
    with pytest.raises(P.Mismatch):
        P.compare_segment(head, gpu2, gs, pre, "two")


@pytest.mark.parametrize("which", ["r", "c"])
def test_factor_mismatch_raises(which):
    head, seg, x = _tile()
    gs, out, pre = _gpu_like(head, seg, x)
    z, r16, c16, h16 = codec.unpack(gs, head.bits, head.pivot, head.dv)
    if which == "r":
        r16 = r16.copy()
        r16[5] += 1
    else:
        c16 = c16.copy()
        c16[7] += 1
    gpu = codec.pack(head.bits, head.pivot, head.dv, z, r16, c16, h16)
    with pytest.raises(P.Mismatch, match="row factors" if which == "r" else "column factors"):
        P.compare_segment(head, gpu, gs, pre, "factor")


def test_stray_bits_raise():
    head, seg, x = _tile()
    head = oracle.Head(head.bits, np.r_[1, np.zeros(head.dk - 1)].astype(np.uint8), head.omega)
    seg = head.encode(codec.unpack(seg, head.bits, np.zeros(head.dk), head.dv)[0] * 0.01)
    gs, out, pre = _gpu_like(head, seg, x)
    L = codec.layout(head.bits, head.pivot, head.dv)
    lane_bits = int(L.G * head.bits[1:].astype(int).sum())
    assert lane_bits % 32 != 0                       # the last word of each stream is padded
    gpu = gs.copy()
    gpu[4 * (64 * (L.words - 1) + 0) + 3] ^= 0x80    # bit 31 of lane 0's last word
    with pytest.raises(P.Mismatch, match="outside codes"):
        P.compare_segment(head, gpu, gs, pre, "padding")


def test_readout_tolerance():
    head, seg, x = _tile()
    gs, out, pre = _gpu_like(head, seg, x)
    tr = P.Tracker()
    seg_o = {0: seg.copy()}
    out_bad = out * (1 + 2e-4)
    with pytest.raises(P.Mismatch, match="readout"):
        P.check_tile(tr, head, seg_o, 0, gs, out_bad, x["q"], x["k"], x["v"], x["a"], x["beta"],
                     "readout")
    seg_o = {0: seg.copy()}
    assert P.check_tile(tr, head, seg_o, 0, gs, out, x["q"], x["k"], x["v"], x["a"], x["beta"],
                        "ok", plain_check=True) == 0
    assert tr.plain.steps == 1
