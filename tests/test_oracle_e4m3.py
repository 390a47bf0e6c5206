"""Pins for the oracle's E4M3 decode/encode (CPU only).

The decode is checked against the special points the OCP OFP8 specification prints
(tests/golden/ofp8_e4m3_points.txt; the page "Fine-Grained FP8/FP4 Quantization", table
"UE8M0 vs E4M3 Scale Formats", puts the top of the E4M3 range at 448).  The encode is
checked exhaustively over every binary32 bit pattern against an independent integer
bit-manipulation encoder (tests/helpers/e4m3_bitenc.c).
"""
import ctypes
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ofp8_e4m3_points.txt")


def _golden_points():
    pts = []
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        code, value, *_ = line.split()
        pts.append((int(code, 16), float(value)))
    return pts


def test_decode_matches_spec_points():
    pts = _golden_points()
    assert len(pts) == 10
    dec = oracle.e4m3_decode([c for c, _ in pts])
    for (code, value), got in zip(pts, dec):
        if math.isnan(value):
            assert math.isnan(got), hex(code)
        else:
            assert got == value and math.copysign(1, got) == math.copysign(1, value), hex(code)


def test_decode_structure():
    vals = oracle.e4m3_decode(np.arange(256))
    finite = vals[~np.isnan(vals)]
    assert np.isnan(vals).sum() == 2                      # 0x7F, 0xFF
    assert len(np.unique(finite)) == 253                  # +0 and -0 are one value
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0)                       # codes 0..0x7E increase
    assert np.array_equal(vals[0x80:0xFF], -pos)          # sign bit mirrors
    assert pos.max() == 448.0
    # every finite value is an integer multiple of 2^-9
    assert np.all(np.floor(finite * 512) == finite * 512)


def test_encode_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    y = oracle.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(y), codes)


def test_encode_ties_and_saturation():
    cases = {
        1.0625: 0x38,            # midpoint 1 / 1.125 -> even (1.0)
        1.1875: 0x3A,            # midpoint 1.125 / 1.25 -> even (1.25)
        2.0 ** -10: 0x00,        # midpoint 0 / 2^-9 -> even (0)
        3 * 2.0 ** -10: 0x02,    # midpoint 2^-9 / 2^-8 -> even (2^-8)
        272.0: 0x78,             # midpoint 256 / 288 -> even (256)
        464.0: 0x7E, 465.0: 0x7E, 1e30: 0x7E, float("inf"): 0x7E,  # saturate
        -449.0: 0xFE, -0.0: 0x80, -1e-30: 0x80, 1e-40: 0x00,
    }
    ys = np.array(list(cases), dtype=np.float32)
    got = oracle.e4m3_encode(ys)
    for y, want, g in zip(cases, cases.values(), got):
        assert g == want, (y, hex(want), hex(g))


def test_encode_exhaustive_vs_bit_encoder(helper_lib):
    lib = oracle._load()
    fn = ctypes.cast(lib.oracle_e4m3_encode, ctypes.c_void_p).value
    total = 1 << 32
    parts = 64
    step = total // parts

    def run(i):
        first = ctypes.c_uint64()
        bad = helper_lib.helper_sweep(fn, i * step, (i + 1) * step, ctypes.byref(first))
        return bad, first.value

    with ThreadPoolExecutor(max_workers=oracle.threads()) as ex:
        res = list(ex.map(run, range(parts)))
    bad = sum(r[0] for r in res)
    firsts = [hex(r[1]) for r in res if r[0]]
    assert bad == 0, f"{bad} mismatches, first at {firsts[:3]}"
