"""Byte codec of one head's packed segment, in NumPy (no arithmetic of the method).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``.  The plain binary64 reference
(``oracle/plain.py``) works on fields -- integer codes z, binary16 row and column factors, binary16
pivot rows -- and this module moves those fields in and out of the segment bytes.  It is written
from the layout's definition and shares no code with ``stepq_oracle.c``'s layout functions or with
the GPU library.

Layout of one head (d_k rows, d_v columns, per-row width b_i and pivot flag):

  code block   G = d_v / 64 columns per lane: lane L owns columns G*L .. G*L+G-1.  Lane L's bit
               stream holds, for each non-pivot row in ascending order, that row's G codes in
               column order, b_i bits each, two's complement, least significant bit first, padded
               with zero bits to D whole 32-bit words.  Word w of lane L is the little-endian
               uint32 at byte 4*(64 w + L).
  pivot block  every pivot row in ascending order, d_v binary16 values.
  r block      d_k binary16 row factors (0 on pivot rows)     -- absent if every row is a pivot
  c block      d_v binary16 column factors                    -- absent if every row is a pivot
  padding      zero bytes up to a multiple of 256.

The pages fix none of this: it is the layout the library stores (the digest, Method 4, only says
that codes, scale metadata and FP16 pivots are packed back in place).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

LANES = 64


@dataclass(frozen=True)
class Layout:
    dk: int
    dv: int
    G: int
    words: int          # D, 32-bit words per lane
    npiv: int
    allpiv: bool
    off_piv: int
    off_r: int
    off_c: int
    bytes: int
    rowpos: np.ndarray  # [dk] first stream bit of each non-pivot row (-1 on pivots)


def layout(bits, pivot, dv: int) -> Layout:
    bits = np.asarray(bits, np.int64)
    piv = np.asarray(pivot).astype(bool)
    dk = bits.size
    G = dv // LANES
    per_row = np.where(piv, 0, G * bits)
    start = np.concatenate([[0], np.cumsum(per_row)[:-1]])
    rowpos = np.where(piv, -1, start)
    lane_bits = int(per_row.sum())
    words = (lane_bits + 31) // 32
    npiv = int(piv.sum())
    allpiv = npiv == dk
    off_piv = 256 * words
    off_r = off_piv + 2 * dv * npiv
    off_c = off_r + (0 if allpiv else 2 * dk)
    end = off_c + (0 if allpiv else 2 * dv)
    return Layout(dk, dv, G, words, npiv, allpiv, off_piv, off_r, off_c,
                  (end + 255) // 256 * 256, rowpos)


def _bit_index(L: Layout, bits, pivot):
    """(rows, cols, lane, stream bit of the code's bit 0) of every code of a non-pivot row."""
    bits = np.asarray(bits, np.int64)
    piv = np.asarray(pivot).astype(bool)
    rows = np.nonzero(~piv)[0]
    j = np.arange(L.dv)
    ii, jj = np.meshgrid(rows, j, indexing="ij")
    lane = jj // L.G
    p0 = L.rowpos[ii] + (jj % L.G) * bits[ii]
    return ii, jj, lane, p0


def unpack(seg, bits, pivot, dv: int):
    """Fields of a segment: (z [dk, dv] int64 with 0 on pivot rows, r16 [dk] uint16,
    c16 [dv] uint16, h16 [dk, dv] uint16 pivot values with 0 on other rows).  Raises ValueError
    on the code -2^(b-1), which the packer never writes."""
    bits = np.asarray(bits, np.int64)
    piv = np.asarray(pivot).astype(bool)
    L = layout(bits, piv, dv)
    seg = np.asarray(seg, np.uint8)
    dk = L.dk
    z = np.zeros((dk, dv), np.int64)
    if L.words:
        # a code spans at most two consecutive words of its lane: read both as one 64-bit window
        w = seg[: 256 * L.words].view(np.uint32).reshape(L.words, LANES).astype(np.uint64)
        w = np.concatenate([w, np.zeros((1, LANES), np.uint64)])
        ii, jj, lane, p0 = _bit_index(L, bits, piv)
        b = bits[ii]
        wi = p0 >> 5
        win = w[wi, lane] | (w[wi + 1, lane] << np.uint64(32))
        val = ((win >> (p0 & 31).astype(np.uint64)).astype(np.int64)) & ((np.int64(1) << b) - 1)
        neg = val >= (np.int64(1) << (b - 1))
        val = np.where(neg, val - (np.int64(1) << b), val)
        if np.any(val == -(np.int64(1) << (b - 1))):
            raise ValueError("corrupt code (-2^(b-1)) in segment")
        z[ii, jj] = val
    h16 = np.zeros((dk, dv), np.uint16)
    if L.npiv:
        h16[piv] = seg[L.off_piv: L.off_piv + 2 * dv * L.npiv].view(np.uint16).reshape(L.npiv, dv)
    if L.allpiv:
        r16 = np.zeros(dk, np.uint16)
        c16 = np.zeros(dv, np.uint16)
    else:
        r16 = seg[L.off_r: L.off_r + 2 * dk].view(np.uint16).copy()
        c16 = seg[L.off_c: L.off_c + 2 * dv].view(np.uint16).copy()
    return z, r16, c16, h16


def pack(bits, pivot, dv: int, z, r16, c16, h16=None) -> np.ndarray:
    """Segment bytes holding codes z [dk, dv] (|z| <= 2^(b-1) - 1), row factors r16 [dk], column
    factors c16 [dv] and pivot values h16 [dk, dv] (read on pivot rows only)."""
    bits = np.asarray(bits, np.int64)
    piv = np.asarray(pivot).astype(bool)
    L = layout(bits, piv, dv)
    seg = np.zeros(L.bytes, np.uint8)
    if L.words:
        streams = np.zeros((LANES, 32 * L.words), np.uint8)
        ii, jj, lane, p0 = _bit_index(L, bits, piv)
        b = bits[ii]
        v = np.asarray(z, np.int64)[ii, jj] & ((np.int64(1) << b) - 1)
        t = np.arange(int(bits.max()))
        m = t < b[..., None]
        pos = p0[..., None] + t
        streams[np.broadcast_to(lane[..., None], pos.shape)[m], pos[m]] = \
            ((v[..., None] >> t) & 1)[m]
        words = np.packbits(streams, axis=1, bitorder="little").view(np.uint32)  # [64, D]
        seg[: 256 * L.words] = words.T.copy().view(np.uint8).ravel()
    if L.npiv:
        seg[L.off_piv: L.off_piv + 2 * dv * L.npiv] = \
            np.asarray(h16, np.uint16)[piv].view(np.uint8).ravel()
    if not L.allpiv:
        seg[L.off_r: L.off_r + 2 * L.dk] = np.asarray(r16, np.uint16).view(np.uint8)
        seg[L.off_c: L.off_c + 2 * dv] = np.asarray(c16, np.uint16).view(np.uint8)
    return seg
