"""Pins for the oracle's UE8M0 (power-of-two scale) quantizers (CPU only).

Page "Fine-Grained FP8/FP4 Quantization": section "Blackwell: Native Block Scaling" (a UE8M0
byte e stands for 2^(e-127)), table "UE8M0 vs E4M3 Scale Formats" (powers of two only; E4M3
reaches 448), section "Scaling Granularities" (1x128 / 128x128 groups).  The reading pinned
here: e is the smallest exponent with 448 * 2^(e-127) >= amax (e = 0 for groups that even
2^-127 covers), and code = E4M3(fl32(x / 2^(e-127))) with the same rounding as the fp32-scale
path.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.domain import bf16_to_f32, domain_tiles, sampled_amax_bits
from tests.exact import bf16_fraction, rn_f32


def f32_to_bf16_bits(v):
    return (np.array([v], np.float32).view(np.uint32)[0] >> 16).astype(np.uint16)


# hand-derived cases of the rule: amax -> e
#   448 = 448*2^0                      -> e = 127
#   450 (first bf16 above 448)         -> 2^0 too small, 2^1 covers  -> 128
#   224 = 448*2^-1                     -> 126;   225 -> 127
#   1.0: 448*2^-8 = 1.75 >= 1 > 448*2^-9 = 0.875 -> e = 119
#   3.3895e38 (largest bf16): 448*2^120 = 5.96e38 >= it > 448*2^119 -> e = 247
#   0 and the smallest subnormal bf16 2^-133 (448*2^-127 already covers) -> e = 0
GOLDEN = [(448.0, 127), (450.0, 128), (224.0, 126), (225.0, 127), (1.0, 119),
          (float(np.uint32(0x7F7F0000).view(np.float32)), 247), (0.0, 0), (2.0 ** -133, 0)]


@pytest.mark.parametrize("amax,e", GOLDEN)
def test_exponent_golden(amax, e):
    X = np.zeros((1, 128), np.uint16)
    X[0, 17] = f32_to_bf16_bits(amax) if amax != 2.0 ** -133 else np.uint16(1)
    Xq, sX = oracle.quantize_act_ue8m0(X)
    assert sX[0, 0] == e
    assert float(oracle.ue8m0_decode([e])[0]) == 2.0 ** (e - 127)


def test_decode_table():
    d = oracle.ue8m0_decode(np.arange(255))
    assert np.all(d[1:] / d[:-1] == 2.0) and d[127] == 1.0 and d[0] == np.float32(2.0 ** -127)
    assert np.isnan(oracle.ue8m0_decode([255])[0])


def test_agrees_with_fp32_scales_when_amax_is_448_times_a_power_of_two():
    """Where amax/448 is itself a power of two the two scale formats are the same number:
    UE8M0 codes must equal the (separately pinned) fp32-scale codes, scale for scale."""
    rng = np.random.default_rng(11)
    M, K = 64, 256
    X = (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    for m in range(M):
        for kb in range(K // 128):
            k = int(rng.integers(-100, 100))
            amax = 448.0 * 2.0 ** k
            g = X[m, kb * 128:(kb + 1) * 128]
            vals = bf16_to_f32(g).astype(np.float64)
            vals = vals / np.max(np.abs(vals)) * amax * 0.999
            g[:] = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
            g[int(rng.integers(0, 128))] = f32_to_bf16_bits(amax if rng.random() < 0.5 else -amax)
    q8, e8 = oracle.quantize_act_ue8m0(X)
    q32, s32 = oracle.quantize_act(X)
    assert np.array_equal(oracle.ue8m0_decode(e8), s32)
    assert np.array_equal(q8, q32)


def test_minimal_covering_power_over_all_bf16_amax():
    """every positive finite bf16 amax: 448*s >= amax, and half of s would not cover it
    (unless e = 0); e is monotone in amax"""
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    X = np.zeros((bits.size, 128), np.uint16)
    X[:, 5] = bits
    _, e = oracle.quantize_act_ue8m0(X)
    e = e[:, 0].astype(np.int64)
    amax = bf16_to_f32(bits).astype(np.float64)
    s = np.ldexp(1.0, e - 127)
    assert np.all(448.0 * s >= amax)
    assert np.all((e == 0) | (448.0 * s / 2 < amax))
    assert np.all(np.diff(e) >= 0)


def test_act_brute_force_tiny(helper_lib):
    """exact rationals: s = 2^(e-127), y = RN32(x/s), code by the independent bit encoder"""
    rng = np.random.default_rng(12)
    M, K = 3, 384
    X = (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    X[1, 128:256] = 0
    X[1, 140] = 0x8000
    X[2, 7] = f32_to_bf16_bits(-987.5)
    X[0, 300] = f32_to_bf16_bits(3e-30)
    Xq, e8 = oracle.quantize_act_ue8m0(X)
    for m in range(M):
        for kb in range(K // 128):
            tile = X[m, kb * 128:(kb + 1) * 128]
            xs = [bf16_fraction(b) for b in tile]
            amax = max(abs(x) for x in xs)
            e = 0
            while e < 254 and 448 * Fraction(2) ** (e - 127) < amax:
                e += 1
            assert e8[m, kb] == e
            s = Fraction(2) ** (e - 127)
            for j, (b, x) in enumerate(zip(tile, xs)):
                want = helper_lib.helper_bitenc(rn_f32(x / s))
                if want == 0 and (int(b) & 0x8000):
                    want = 0x80
                assert Xq[m, kb * 128 + j] == want, (m, kb, j)
    assert e8[1, 1] == 0 and Xq[1, 140] == 0x80


def test_weight_block_geometry_and_locality():
    """128x128 blocks: a block scaled by 2^j gets e + j and the same codes; one outlier
    changes only its own block's exponent and codes"""
    rng = np.random.default_rng(13)
    base = (rng.standard_normal((128, 128)).astype(np.float32) * 0.02)
    KB, NB = 2, 3
    W = np.empty((KB * 128, NB * 128), np.float32)
    for kb in range(KB):
        for nb in range(NB):
            W[kb * 128:(kb + 1) * 128, nb * 128:(nb + 1) * 128] = base * 2.0 ** (kb * NB + nb)
    Wb = (W.view(np.uint32) >> 16).astype(np.uint16)
    Wq, e8 = oracle.quantize_weight_ue8m0(Wb)
    for kb in range(KB):
        for nb in range(NB):
            j = kb * NB + nb
            assert int(e8[kb, nb]) == int(e8[0, 0]) + j
            assert np.array_equal(Wq[kb * 128:(kb + 1) * 128, nb * 128:(nb + 1) * 128],
                                  Wq[:128, :128])
    W2 = Wb.copy()
    W2[200, 140] = f32_to_bf16_bits(1000.0)
    Wq2, e82 = oracle.quantize_weight_ue8m0(W2)
    assert [tuple(d) for d in np.argwhere(e8 != e82)] == [(1, 1)]
    r, c = np.nonzero(Wq != Wq2)
    assert len(r) > 0 and np.all(r // 128 == 1) and np.all(c // 128 == 1)


def test_domain_sweep_properties():
    """every bf16 x with |x| <= amax over a stride of amax values: no NaN or saturated-past
    code, sign symmetry, |dec(q)*s - x| within half an E4M3 step of the exact quotient"""
    X, amax_bits, counts = domain_tiles(sampled_amax_bits(61))
    Xq, e8 = oracle.quantize_act_ue8m0(X.reshape(1, -1))
    Xq = Xq.reshape(X.shape)
    s = oracle.ue8m0_decode(e8.reshape(-1)).astype(np.float64)
    assert not np.any((Xq & 0x7F) == 0x7F)
    x = bf16_to_f32(X).astype(np.float64)
    y = x / s[:, None]
    ay = np.abs(y)
    assert np.all(ay <= 448.0)
    step = np.where(ay >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(ay, 2.0 ** -6))) - 3), 2.0 ** -9)
    dec = oracle.e4m3_decode(Xq)
    err = np.abs(dec * s[:, None] - x)
    # the quotient by a power of two is exact unless it falls below binary32's subnormal step
    bound = s[:, None] * (0.5 * step + np.maximum(ay * 2.0 ** -23, 2.0 ** -150))
    assert np.all(err <= bound)
