"""Pins for the oracle's packed layout: known-answer words, code round trips over every code of
every width, and segment sizes."""
import os

import numpy as np
import pytest

from layout_ref import build_segment, read_codes, seg_fields

GOLD = os.path.join(os.path.dirname(__file__), "golden", "pack_kat.txt")
ONE16 = 0x3C00  # binary16 1.0


def _kat():
    rows = []
    for line in open(GOLD):
        if line.startswith("#") or not line.strip():
            continue
        b, codes, by = (s.strip() for s in line.split("|"))
        rows.append((int(b), [int(c) for c in codes.split()], bytes.fromhex(by.replace(" ", ""))))
    return rows


@pytest.mark.parametrize("b,codes,want", _kat())
def test_known_answer_words(orc, b, codes, want):
    # G = 1 (d_v = 64): lane 0's stream walks down column 0; put the codes there, encode nothing
    dk = dv = 64
    bits = np.full(dk, b, np.int8)
    piv = np.zeros(dk, np.uint8)
    z = np.zeros((dk, dv), np.int64)
    z[: len(codes), 0] = codes
    seg = build_segment(bits, piv, dv, z, np.full(dk, ONE16), np.full(dv, ONE16))
    assert bytes(seg[:4]) == want          # test-side layout matches the hand-written word
    S, r, c, zz = orc.Head(bits, piv, np.ones(dk)).unpack(seg)
    assert np.array_equal(zz[: len(codes), 0], codes)   # the oracle reads the same codes
    assert np.array_equal(S[: len(codes), 0], np.array(codes, np.float32))


@pytest.mark.parametrize("dv", [64, 128])
@pytest.mark.parametrize("b", [2, 4, 6, 8])
def test_every_code_round_trips(orc, b, dv):
    dk = dv
    q = (1 << (b - 1)) - 1
    bits = np.full(dk, b, np.int8)
    piv = np.zeros(dk, np.uint8)
    vals = np.arange(-q, q + 1)
    z = np.resize(vals, dk * dv).reshape(dk, dv)
    np.random.default_rng(b).shuffle(z.ravel())
    seg = build_segment(bits, piv, dv, z, np.full(dk, ONE16), np.full(dv, ONE16))
    S, r, c, zz = orc.Head(bits, piv, np.ones(dk), dv).unpack(seg)
    assert np.array_equal(zz, z)
    assert np.array_equal(S, z.astype(np.float32))
    assert np.array_equal(read_codes(seg, bits, piv, dv), z)


def test_mixed_rows_and_pivots(orc):
    g = np.random.default_rng(5)
    dk = dv = 128
    bits = g.choice([4, 6, 8], size=dk).astype(np.int8)
    piv = np.zeros(dk, np.uint8)
    piv[[3, 77, 127]] = 1
    z = np.zeros((dk, dv), np.int64)
    for i in range(dk):
        q = (1 << (int(bits[i]) - 1)) - 1
        z[i] = 0 if piv[i] else g.integers(-q, q + 1, size=dv)
    r16 = np.where(piv, 0, 0x3800).astype(np.uint16)          # 0.5
    c16 = np.full(dv, 0x4000, np.uint16)                       # 2.0
    p16 = np.asarray(g.standard_normal((3, dv)), np.float16).view(np.uint16)
    seg = build_segment(bits, piv, dv, z, r16, c16, p16)
    h = orc.Head(bits, piv, np.ones(dk), dv)
    assert h.seg_bytes == seg.size == seg_fields(bits, piv, dv)["bytes"]
    S, r, c, zz = h.unpack(seg)
    assert np.array_equal(zz, z)
    assert np.array_equal(S[piv == 0], z[piv == 0].astype(np.float32))  # 0.5 * 2 * z
    assert np.array_equal(S[piv == 1], p16.view(np.float16).astype(np.float32))


def test_corrupt_code_is_rejected(orc):
    dk = dv = 64
    bits = np.full(dk, 4, np.int8)
    piv = np.zeros(dk, np.uint8)
    z = np.zeros((dk, dv), np.int64)
    z[5, 7] = -8  # -2^(b-1) is never written
    seg = build_segment(bits, piv, dv, z, np.full(dk, ONE16), np.full(dv, ONE16))
    with pytest.raises(ValueError):
        orc.Head(bits, piv, np.ones(dk)).unpack(seg)


def test_segment_sizes(orc):
    # GDN 6-bit head, d = 128: 12288 code bytes + 256 + 256 scale bytes
    h = orc.Head(np.full(128, 6, np.int8), np.zeros(128, np.uint8), np.ones(128))
    assert h.seg_bytes == 12800
    # FP16 pivot head: the raw binary16 tile only
    h = orc.Head(np.full(128, 6, np.int8), np.ones(128, np.uint8), np.ones(128))
    assert h.seg_bytes == 32768
