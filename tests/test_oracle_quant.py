"""Pins for the oracle's 1x128 activation and 128x128 weight quantizers (CPU only).

Page "Fine-Grained FP8/FP4 Quantization": section "Scaling Granularities" (one scale per
1x128 tile / per 128x128 block, so an outlier only affects its own group), section
"DeepGEMM: Tile-wise and Block-wise Scaling" (scale_A [M,K/128], scale_B [K/128,N/128]),
table "UE8M0 vs E4M3 Scale Formats" (E4M3 tops out at 448).
"""
import numpy as np
import pytest

import oracle
from tests.domain import bf16_to_f32, domain_tiles, sampled_amax_bits
from tests.exact import bf16_fraction, rn_f32


def _rand_bf16(shape, rng, scale=1.0):
    v = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)   # truncation is fine for test data


def _expected_codes_exact(x_bits_row, helper_lib):
    """Brute force for one group: amax by max over |x|, s = RN32(amax/448) and
    y = RN32(x/s) in exact rationals, code by the independent bit encoder."""
    xs = [bf16_fraction(b) for b in x_bits_row]
    amax = max(abs(x) for x in xs)
    s = rn_f32(amax / 448)
    if s == 0:
        codes = [0x80 if (int(b) & 0x8000) else 0x00 for b in x_bits_row]
        return codes, 0.0
    codes = [helper_lib.helper_bitenc(rn_f32(x / __import__("fractions").Fraction(s)))
             for x in xs]
    # the bit encoder sees a Python float; -0.0 results keep their sign via rn_f32
    return codes, s


def test_act_brute_force_tiny(helper_lib):
    rng = np.random.default_rng(1)
    M, K = 3, 384
    X = _rand_bf16((M, K), rng)
    X[1, 128:256] = 0                       # all-zero tile
    X[1, 130] = 0x8000                      # with a negative zero
    X[2, 5] = _rand_bf16((1,), rng, 300.0)[0]
    Xq, sX = oracle.quantize_act(X)
    assert Xq.shape == (M, K) and sX.shape == (M, K // 128)
    for m in range(M):
        for kb in range(K // 128):
            tile = X[m, kb * 128:(kb + 1) * 128]
            codes, s = _expected_codes_exact(tile, helper_lib)
            assert np.float32(sX[m, kb]) == np.float32(s)
            got = Xq[m, kb * 128:(kb + 1) * 128]
            # -0.0 from rn_f32 loses its sign only for x == -0: handle via x's sign bit
            want = np.array(codes, dtype=np.uint8)
            neg_zero = (want == 0) & ((tile & 0x8000) != 0)
            want[neg_zero] = 0x80
            assert np.array_equal(got, want), (m, kb)
    assert sX[1, 1] == 0 and Xq[1, 130] == 0x80 and np.all(Xq[1, 128:256][tile_zero_mask(X[1, 128:256])] == 0)


def tile_zero_mask(tile):
    return (tile & 0x8000) == 0


def test_weight_brute_force_tiny(helper_lib):
    rng = np.random.default_rng(2)
    K, N = 256, 256
    W = _rand_bf16((K, N), rng, 0.02)
    W[200, 3] = _rand_bf16((1,), rng, 5.0)[0]
    Wq, sW = oracle.quantize_weight(W)
    assert Wq.shape == (K, N) and sW.shape == (2, 2)
    for kb in range(2):
        for nb in range(2):
            blk = W[kb * 128:(kb + 1) * 128, nb * 128:(nb + 1) * 128]
            amax = max(abs(bf16_fraction(b)) for b in blk.reshape(-1))
            s = rn_f32(amax / 448)
            assert np.float32(sW[kb, nb]) == np.float32(s)
            # spot-check 300 elements of the block by exact rationals
            idx = rng.choice(blk.size, 300, replace=False)
            from fractions import Fraction
            for i in idx:
                b = blk.reshape(-1)[i]
                y = rn_f32(bf16_fraction(b) / Fraction(s))
                want = helper_lib.helper_bitenc(y)
                if want == 0 and (b & 0x8000):
                    want = 0x80
                assert Wq[kb * 128 + i // 128, nb * 128 + i % 128] == want


def test_group_geometry_by_power_of_two_blocks():
    """Each group is a scaled copy 2^j of one base tile/block, j distinct per group: every
    scale must be base*2^j exactly and every group's codes identical -- a swapped index,
    stride or group shape breaks this."""
    rng = np.random.default_rng(3)
    # activations: M=3 rows x KB=4 tiles
    base = _rand_bf16((128,), rng)
    M, KB = 3, 4
    X = np.empty((M, KB * 128), dtype=np.uint16)
    for m in range(M):
        for kb in range(KB):
            j = m * KB + kb
            X[m, kb * 128:(kb + 1) * 128] = (base.astype(np.int32) + ((j - 6) << 7) * (base & 0x7FFF != 0)).astype(np.uint16)
    Xq, sX = oracle.quantize_act(X)
    for m in range(M):
        for kb in range(KB):
            j = m * KB + kb
            assert sX[m, kb] == np.float32(sX[0, 0] * 2.0 ** j)
            assert np.array_equal(Xq[m, kb * 128:(kb + 1) * 128], Xq[0, :128])
    # weights: KB=2 x NB=3 blocks
    bblk = _rand_bf16((128, 128), rng, 0.02)
    KB, NB = 2, 3
    W = np.empty((KB * 128, NB * 128), dtype=np.uint16)
    for kb in range(KB):
        for nb in range(NB):
            j = kb * NB + nb
            W[kb * 128:(kb + 1) * 128, nb * 128:(nb + 1) * 128] = (
                bblk.astype(np.int32) + (j << 7) * (bblk & 0x7FFF != 0)).astype(np.uint16)
    Wq, sW = oracle.quantize_weight(W)
    for kb in range(KB):
        for nb in range(NB):
            j = kb * NB + nb
            assert sW[kb, nb] == np.float32(sW[0, 0] * 2.0 ** j)
            assert np.array_equal(Wq[kb * 128:(kb + 1) * 128, nb * 128:(nb + 1) * 128], Wq[:128, :128])


@pytest.mark.parametrize("kind", ["act", "weight"])
def test_outlier_locality(kind):
    rng = np.random.default_rng(4)
    if kind == "act":
        X = _rand_bf16((4, 512), rng)
        q0, s0 = oracle.quantize_act(X)
        pos = (2, 300)
        grp = lambda r, c: (r, c // 128)
    else:
        X = _rand_bf16((384, 256), rng, 0.02)
        q0, s0 = oracle.quantize_weight(X)
        pos = (200, 140)
        grp = lambda r, c: (r // 128, c // 128)
    g = grp(*pos)
    big = np.float32(float(s0[g]) * 448 * 10)
    X2 = X.copy()
    X2[pos] = (np.array([big], np.float32).view(np.uint32)[0] >> 16)
    q1, s1 = (oracle.quantize_act if kind == "act" else oracle.quantize_weight)(X2)
    diff_s = np.argwhere(s0 != s1)
    assert [tuple(d) for d in diff_s] == [g]
    rows, cols = np.nonzero(q0 != q1)
    assert len(rows) > 0
    assert all(grp(r, c) == g for r, c in zip(rows, cols))
    assert q1[pos] == 0x7E


def test_domain_sweep_properties():
    """Over every bf16 x with |x| <= amax for a broad set of amax (all subnormal amax, a
    stride through the rest, the edges): amax -> 0x7E, no NaN code, sign symmetry,
    monotone in x, and |dec(q)*s - x| within half an E4M3 step (plus the fp32 quotient's
    rounding)."""
    X, amax_bits, counts = domain_tiles(sampled_amax_bits(61))
    Xq, sX = oracle.quantize_act(X.reshape(1, -1))
    Xq = Xq.reshape(X.shape)
    s = sX.reshape(-1).astype(np.float64)
    amax = bf16_to_f32(amax_bits).astype(np.float64)
    assert np.array_equal(s, (bf16_to_f32(amax_bits) / np.float32(448)).astype(np.float64))
    assert np.all(Xq[:, 0] == 0x7E)
    assert not np.any((Xq & 0x7F) == 0x7F)
    x = bf16_to_f32(X).astype(np.float64)
    j = np.arange(128)[None, :]
    valid = (j >= 1) & (j <= counts[:, None])
    dec = oracle.e4m3_decode(Xq)
    y = x / s[:, None]
    ay = np.abs(y)
    step = np.where(ay >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(ay, 2.0 ** -6))) - 3), 2.0 ** -9)
    err = np.abs(dec * s[:, None] - x)
    bound = s[:, None] * (0.5 * step + ay * 2.0 ** -23) + 1e-300
    assert np.all(err <= bound)
    # sign symmetry and monotonicity, per amax: gather (x, code) pairs
    flat_x = X[valid]
    flat_q = Xq[valid]
    flat_a = np.repeat(amax_bits, counts)
    order = np.lexsort((flat_x, flat_a))
    fx, fq, fa = flat_x[order], flat_q[order], flat_a[order]
    pos = fx < 0x8000
    neg = ~pos
    # positive and negative halves line up by magnitude within each amax
    assert np.array_equal(fq[neg], fq[pos] | 0x80)
    vpos = oracle.e4m3_decode(fq[pos])
    same = np.diff(fa[pos]) == 0
    assert np.all(np.diff(vpos)[same] >= 0)


# (amax, x) bf16 pairs where a reciprocal multiply x * fl32(1/s) and the correctly rounded
# divide fl32(x / s) give different E4M3 codes (found by search over bf16 pairs)
DIVIDE_CASES = [(16810, 14762), (16978, 14870), (16978, 15043), (16376, 14522),
                (16376, 14650), (17094, 15046)]


def test_divide_not_reciprocal_cases(helper_lib):
    """Codes come from the correctly rounded quotient x/s: on the pairs where x*(1/s) rounds to
    another code, the oracle agrees with the exact-rational brute force."""
    X = np.zeros((len(DIVIDE_CASES), 128), dtype=np.uint16)
    for r, (a, x) in enumerate(DIVIDE_CASES):
        X[r, 0], X[r, 77] = a, x
    Xq, sX = oracle.quantize_act(X)
    for r in range(len(DIVIDE_CASES)):
        codes, s = _expected_codes_exact(X[r], helper_lib)
        assert np.float32(sX[r, 0]) == np.float32(s)
        assert Xq[r, 77] == codes[77], r


def _one_max_rows(n, rng):
    """n rows of 128 small bf16 values (|x| < 1) whose unique largest magnitude, 3.5 with
    alternating sign, sits at column r of row r"""
    X = (np.abs(_rand_bf16((n, 128), rng, 0.2)) & 0x7FFF) | (rng.integers(0, 2, (n, 128)) << 15)
    X = X.astype(np.uint16)
    X[(X & 0x7FFF) >= 0x3F80] &= 0x803F          # keep |x| < 1
    for r in range(n):
        X[r, r % 128] = 0x4060 | ((r & 1) << 15)  # +-3.5
    return X


def test_amax_at_every_position():
    """The scale follows a group's largest magnitude wherever it sits: a 1x128 tile with it at
    each of the 128 positions, a 128x128 block with it at corners, edges and inside, for the
    fp32 and UE8M0 scales -- s = fl32(3.5/448), e = 120 (448 * 2^-7 is the first power-of-two
    multiple of 448 that covers 3.5) -- and its own code is the saturating +-448."""
    rng = np.random.default_rng(3)
    X = _one_max_rows(128, rng)
    s_want = np.float32(3.5) / np.float32(448.0)
    Xq, sX = oracle.quantize_act(X)
    assert np.all(sX[:, 0] == s_want)
    for r in range(128):
        assert Xq[r, r] == (0x7E | ((r & 1) << 7)), r
    Xq, eX = oracle.quantize_act_ue8m0(X)
    assert np.all(eX[:, 0] == 120)
    for (i, j) in [(0, 0), (0, 127), (127, 0), (127, 127), (64, 63), (1, 126)]:
        W = _one_max_rows(128, rng)
        W[np.arange(128), np.arange(128)] = 0x3E00    # 0.125: no longer the maximum
        W[i, j] = 0xC060                              # -3.5
        Wq, sW = oracle.quantize_weight(W)
        assert sW[0, 0] == s_want and Wq[i, j] == 0xFE, (i, j)
        _, eW = oracle.quantize_weight_ue8m0(W)
        assert eW[0, 0] == 120, (i, j)


def test_fine_grained_beats_per_tensor_scaling_on_outlier_data():
    """The method's motivation (page "Fine-Grained FP8/FP4 Quantization", section "Overview":
    one scale for a whole tensor lets a few outliers set it, and the other values lose
    precision).  E4M3 is a floating-point code, so a larger scale only hurts once it pushes
    ordinary values below its normal range (2^-6); with a few x1e5 outliers in N(0,1)
    activations, one per-tensor scale amax/448 sends them there, while the 1x128 scales of
    the tiles without an outlier keep them at the code's 3-bit relative precision.
    Documents the design; not a parity check."""
    rng = np.random.default_rng(11)
    M, K = 64, 1024
    x = rng.standard_normal((M, K)).astype(np.float32)
    out = [(3, 5), (17, 700), (40, 260)]
    for r, c in out:
        x[r, c] = 1.0e5 * np.sign(x[r, c])
    X = (x.view(np.uint32) >> 16).astype(np.uint16)
    xf = bf16_to_f32(X).astype(np.float64)
    Xq, sX = oracle.quantize_act(X)
    fine = oracle.e4m3_decode(Xq).reshape(M, K) * np.repeat(sX.astype(np.float64), 128, axis=1)
    s_t = np.float32(np.abs(xf).max()) / np.float32(448.0)
    q_t = oracle.e4m3_encode((xf / np.float64(s_t)).astype(np.float32).ravel())
    tensor = oracle.e4m3_decode(q_t).reshape(M, K) * np.float64(s_t)
    clean = np.ones((M, K // 128), dtype=bool)
    for r, c in out:
        clean[r, c // 128] = False
    mask = np.repeat(clean, 128, axis=1) & (np.abs(xf) > 0.1)
    rel = lambda d: np.sqrt(np.mean(((d[mask] - xf[mask]) / xf[mask]) ** 2))
    assert rel(fine) < 0.04                     # about the 3-bit mantissa's half step
    assert rel(tensor) > 10 * rel(fine)
