"""Test-side description of the packed segment layout, written from the layout's definition
(lane-interleaved 32-bit words of per-lane code streams, then FP16 pivot rows, FP16 row factors,
FP16 column factors, 256-byte padding).  Used to build segments with chosen codes and to read
fields back, independently of both the oracle and the GPU library."""
import numpy as np

LANES = 64


def seg_fields(bits, pivot, dv):
    bits = np.asarray(bits)
    pivot = np.asarray(pivot).astype(bool)
    dk = bits.size
    G = dv // LANES
    lane_bits = int(sum(G * int(b) for b, p in zip(bits, pivot) if not p))
    words = (lane_bits + 31) // 32
    npiv = int(pivot.sum())
    allpiv = npiv == dk
    off_piv = 256 * words
    off_r = off_piv + 2 * dv * npiv
    off_c = off_r + (0 if allpiv else 2 * dk)
    end = off_c + (0 if allpiv else 2 * dv)
    return dict(G=G, words=words, off_piv=off_piv, off_r=off_r, off_c=off_c,
                bytes=(end + 255) // 256 * 256, allpiv=allpiv, npiv=npiv)


def code_positions(bits, pivot, dv):
    """(lane, stream bit) of every code (i, j) of a non-pivot row."""
    bits = np.asarray(bits)
    G = dv // LANES
    pos = {}
    p = 0
    for i, b in enumerate(bits):
        if pivot[i]:
            continue
        for j in range(dv):
            pos[(i, j)] = (j // G, p + (j % G) * int(b))
        p += G * int(b)
    return pos


def build_segment(bits, pivot, dv, z, r16, c16, piv16=None):
    """Segment bytes holding codes z [dk, dv], row factors r16 [dk], column factors c16 [dv]
    (binary16 bit patterns) and pivot rows piv16 [npiv, dv]."""
    f = seg_fields(bits, pivot, dv)
    words = np.zeros((max(f["words"], 1), LANES), np.uint64)
    for (i, j), (lane, p) in code_positions(bits, pivot, dv).items():
        b = int(bits[i])
        v = int(z[i, j]) & ((1 << b) - 1)
        for t in range(b):
            q = p + t
            words[q // 32, lane] |= np.uint64(((v >> t) & 1) << (q % 32))
    seg = np.zeros(f["bytes"], np.uint8)
    seg[: 256 * f["words"]] = words[: f["words"]].astype(np.uint32).view(np.uint8).ravel()
    if f["npiv"]:
        seg[f["off_piv"]: f["off_piv"] + 2 * dv * f["npiv"]] = \
            np.asarray(piv16, np.uint16).view(np.uint8).ravel()
    if not f["allpiv"]:
        seg[f["off_r"]: f["off_r"] + 2 * len(bits)] = np.asarray(r16, np.uint16).view(np.uint8)
        seg[f["off_c"]: f["off_c"] + 2 * dv] = np.asarray(c16, np.uint16).view(np.uint8)
    return seg


def read_codes(seg, bits, pivot, dv):
    """Codes [dk, dv] read from a segment (0 on pivot rows)."""
    dk = len(bits)
    f = seg_fields(bits, pivot, dv)
    w = np.frombuffer(bytes(seg[: 256 * f["words"]]), np.uint32).reshape(-1, LANES) \
        if f["words"] else np.zeros((0, LANES), np.uint32)
    z = np.zeros((dk, dv), np.int64)
    for (i, j), (lane, p) in code_positions(bits, pivot, dv).items():
        b = int(bits[i])
        v = 0
        for t in range(b):
            q = p + t
            v |= ((int(w[q // 32, lane]) >> (q % 32)) & 1) << t
        if v >= 1 << (b - 1):
            v -= 1 << b
        z[i, j] = v
    return z


def read_f16(seg, off, n):
    return np.frombuffer(bytes(seg[off: off + 2 * n]), np.uint16).copy()
