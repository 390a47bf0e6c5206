"""Pins for the oracle's NVFP4 (two-level scaled E2M1) quantizer and GEMM (CPU only).

Page "Fine-Grained FP8/FP4 Quantization", section "NVFP4 Two-Level Scaling": E2M1 values
0, 0.5, 1, 1.5, 2, 3, 4, 6; one E4M3 scale per 16 elements along K; one FP32 global scale;
value = global * block * e2m1.  Readings pinned here (the page gives only the format):
g = amax/2688, block scale = E4M3(amax_block / (6g)), code = E2M1(x / (block*g)), nearest
with ties to the even code, saturating at 6."""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.exact import rn_f32

HERE = os.path.dirname(os.path.abspath(__file__))


def golden_e2m1():
    rows = []
    for line in open(os.path.join(HERE, "golden", "e2m1_values.txt")):
        line = line.split("#")[0].strip()
        if line:
            c, v = line.split()
            rows.append((int(c), float(v)))
    return rows


def test_e2m1_values_match_the_page():
    for c, v in golden_e2m1():
        assert oracle.e2m1_decode([c])[0] == v
        assert oracle.e2m1_decode([c | 8])[0] == -v
        if v:
            assert oracle.e2m1_encode([v])[0] == c and oracle.e2m1_encode([-v])[0] == (c | 8)


def _nearest_brute(y):
    """nearest E2M1 code by exhaustive search in exact rationals, ties to even code,
    saturating at 6 (values from the golden table)"""
    vals = [(c, Fraction(v)) for c, v in golden_e2m1()]
    a = abs(Fraction(y))
    if a >= 6:
        best = 7
    else:
        dmin = min(abs(a - v) for _, v in vals)
        cands = [c for c, v in vals if abs(a - v) == dmin]
        best = min(cands, key=lambda c: (c % 2, c))
    return best | (8 if np.signbit(np.float32(y)) else 0)


def test_e2m1_encode_against_brute_force():
    rng = np.random.default_rng(21)
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]
    ys = []
    for m in mids:
        f = np.float32(m)
        ys += [f, np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(10))]
    ys += list(rng.uniform(-8, 8, 3000).astype(np.float32))
    ys += list((rng.standard_normal(1000) * 0.3).astype(np.float32))
    ys += [np.float32(0.0), np.float32(-0.0), np.float32(1e-30), np.float32(-1e30)]
    got = oracle.e2m1_encode(np.array(ys, np.float32))
    want = [_nearest_brute(float(y)) for y in ys]
    assert list(got) == want


def _bf16(v):
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _dequant(Xq, sX, g):
    R, C2 = Xq.shape
    codes = np.empty((R, C2 * 2), np.uint8)
    codes[:, 0::2] = Xq & 15
    codes[:, 1::2] = Xq >> 4
    blk = np.repeat(oracle.e4m3_decode(sX), 16, axis=1)
    return float(g) * blk * oracle.e2m1_decode(codes), codes


def test_tensor_amax_block_and_error_bound():
    rng = np.random.default_rng(22)
    X = _bf16(rng.standard_normal((8, 256)).astype(np.float32))
    X[3, 77] = _bf16(np.float32(-9.5))              # the tensor amax
    Xq, sX, g = oracle.quantize_nvfp4(X)
    x = ((X.astype(np.uint32) << 16).view(np.float32)).astype(np.float64)
    assert g == np.float32(np.float32(9.5) / np.float32(2688))
    assert sX[3, 77 // 16] == 0x7E                     # scale 448
    xh, codes = _dequant(Xq, sX, g)
    assert codes[3, 77] == 0xF                          # -6
    D = np.repeat(oracle.e4m3_decode(sX), 16, axis=1) * float(g)
    y = np.abs(x) / D
    step = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    # half an E2M1 step of the quotient, plus the fp32 roundings of D and of x/D (a quotient
    # a hair below a midpoint can round onto it and take the even code)
    slack = 2.0 ** -22 * np.abs(x)
    assert np.all(np.abs(x - xh) <= np.maximum(0.5 * step * D, np.abs(x) - 6 * D) + slack)


def test_power_of_two_scaling_moves_only_the_global_scale():
    rng = np.random.default_rng(23)
    base = rng.standard_normal((4, 128)).astype(np.float32)
    q0, s0, g0 = oracle.quantize_nvfp4(_bf16(base))
    for j in (-20, -3, 5, 40):
        q1, s1, g1 = oracle.quantize_nvfp4(_bf16(base * np.float32(2.0 ** j)))
        assert g1 == np.float32(g0 * np.float32(2.0 ** j))
        assert np.array_equal(q0, q1) and np.array_equal(s0, s1)


def test_block_locality():
    rng = np.random.default_rng(24)
    X = _bf16(rng.standard_normal((4, 128)).astype(np.float32))
    X[0, 0] = _bf16(np.float32(20.0))          # keeps the tensor amax (and g) fixed
    q0, s0, g0 = oracle.quantize_nvfp4(X)
    X2 = X.copy()
    X2[2, 40] = _bf16(np.float32(7.0))         # block (2, 2) only
    q1, s1, g1 = oracle.quantize_nvfp4(X2)
    assert g1 == g0
    assert [tuple(d) for d in np.argwhere(s0 != s1)] == [(2, 2)]
    r, c = np.nonzero(q0 != q1)
    assert np.all(r == 2) and np.all(c // 8 == 2)


def test_zero_tensor_and_signed_zeros():
    X = np.zeros((2, 32), np.uint16)
    X[1, 5] = 0x8000
    q, s, g = oracle.quantize_nvfp4(X)
    assert g == 0 and np.all(s == 0)
    # element 5 of row 1 is the high nibble of byte 2: sign only
    assert q[1, 2] == 0x80
    assert np.all(np.delete(q.reshape(-1), 16 + 2) == 0)


def test_brute_force_chain_tiny():
    """exact rationals for one small tensor: g, block scales (E4M3 by the pinned encoder),
    codes (E2M1 by exhaustive search)"""
    rng = np.random.default_rng(25)
    X = _bf16((rng.standard_normal((2, 48)) * 3).astype(np.float32))
    Xq, sX, g = oracle.quantize_nvfp4(X)
    xs = [[Fraction(float(v)) for v in row] for row in ((X.astype(np.uint32) << 16).view(np.float32))]
    amax = max(abs(v) for row in xs for v in row)
    gg = rn_f32(amax / 2688)
    assert np.float32(g) == np.float32(gg)
    six_g = rn_f32(6 * Fraction(gg))
    for r in range(2):
        for b in range(3):
            blk = xs[r][16 * b:16 * b + 16]
            ab = max(abs(v) for v in blk)
            sb = int(oracle.e4m3_encode(np.array([rn_f32(ab / Fraction(six_g))], np.float32))[0])
            assert sX[r, b] == sb
            D = rn_f32(Fraction(float(oracle.e4m3_decode(np.array([sb], np.uint8))[0])) * Fraction(gg))
            for j, v in enumerate(blk):
                want = _nearest_brute(rn_f32(v / Fraction(D)))
                k = 16 * b + j
                got = (Xq[r, k // 2] >> (4 * (k % 2))) & 15
                assert got == want, (r, k)


def test_gemm_small_integers_exact():
    """unit block scales (E4M3 0x38 = 1.0) and g = 1: the GEMM is a plain matmul of E2M1
    values, exact in binary64"""
    rng = np.random.default_rng(26)
    M, N, K = 5, 7, 64
    a = rng.integers(0, 16, (M, K)).astype(np.uint8)
    b = rng.integers(0, 16, (N, K)).astype(np.uint8)
    pack = lambda c: (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    sA = np.full((M, K // 16), 0x38, np.uint8)
    sB = np.full((N, K // 16), 0x38, np.uint8)
    C, S = oracle.gemm_nvfp4_f64(pack(a), sA, 1.0, pack(b), sB, 1.0)
    va, vb = oracle.e2m1_decode(a), oracle.e2m1_decode(b)
    assert np.array_equal(C, va @ vb.T)
    assert np.array_equal(S, np.abs(va) @ np.abs(vb).T)


def test_gemm_block_scale_linearity():
    """doubling one block scale of A (E4M3 code +8 = one exponent step) doubles exactly that
    block's contribution"""
    rng = np.random.default_rng(27)
    M, N, K = 3, 4, 64
    Aq = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    Bq = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sA = np.full((M, K // 16), 0x30, np.uint8)
    sB = rng.integers(0x28, 0x40, (N, K // 16)).astype(np.uint8)
    C0, _ = oracle.gemm_nvfp4_f64(Aq, sA, 0.5, Bq, sB, 2.0)
    sA2 = sA.copy()
    sA2[1, 2] += 8
    C1, _ = oracle.gemm_nvfp4_f64(Aq, sA2, 0.5, Bq, sB, 2.0)
    Aonly = np.zeros_like(Aq)
    Aonly[1, 16:24] = Aq[1, 16:24]                     # block 2 of row 1 (k 32..47)
    Cb, _ = oracle.gemm_nvfp4_f64(Aonly, sA, 0.5, Bq, sB, 2.0)
    assert np.array_equal(C1 - C0, Cb)


def test_coder_division_is_correctly_rounded(markstein_lib):
    """The NVFP4 coder replaces the per-element IEEE divide x/D by one correctly rounded
    reciprocal per block and Markstein's correction.  On every bf16 x against 3000 random D
    in [2^-100, 2^100]: the quotient is the correctly rounded one wherever |x/D| reaches the
    E2M1 boundaries (1/8 .. 16), the E2M1 code equals that of the correctly rounded quotient
    for every x (where tiny x make the remainder underflow, the quotient is far below the
    first boundary), and the sign of x (signed zeros included) is kept; |x/D| <= 16 covers
    everything the coder sees, since its block scale keeps |x| < 9*D."""
    import ctypes
    code_err, sign_err, checked = ctypes.c_uint64(0), ctypes.c_uint64(0), ctypes.c_uint64(0)
    bad = markstein_lib.markstein_sweep(3000, 12345, ctypes.byref(code_err),
                                        ctypes.byref(sign_err), ctypes.byref(checked))
    assert checked.value > 5_000_000
    assert bad == 0 and code_err.value == 0 and sign_err.value == 0


def test_block_and_tensor_amax_at_every_position():
    """A block's E4M3 scale follows its largest magnitude at each of the block's 16 positions,
    and the global scale follows the tensor's largest magnitude when it is the very last
    element: g = fl32(6/2688), every block whose maximum is 3 gets ENC(fl32(3/fl32(6g)))."""
    rng = np.random.default_rng(5)
    R = 16
    small = rng.integers(0x3A00, 0x3EFF, (R, 32)).astype(np.uint16)   # |x| < 0.5
    small |= (rng.integers(0, 2, (R, 32)) << 15).astype(np.uint16)
    X = small
    for r in range(R):
        X[r, r] = 0x4040                   # 3.0 at position r of block 0
        X[r, 16 + (15 - r)] = 0xC040       # -3.0 at position 15 - r of block 1
    X[R - 1, 31] = 0x40C0                  # 6.0, the tensor's maximum, last element
    Xq, sX, g = oracle.quantize_nvfp4(X)
    g_want = np.float32(6.0) / np.float32(2688.0)
    assert g == g_want
    six_g = np.float32(6.0) * g_want
    s3 = oracle.e4m3_encode(np.array([np.float32(3.0) / six_g], dtype=np.float32))[0]
    s6 = oracle.e4m3_encode(np.array([np.float32(6.0) / six_g], dtype=np.float32))[0]
    assert np.all(sX[:, 0] == s3)
    assert np.all(sX[:R - 1, 1] == s3) and sX[R - 1, 1] == s6
