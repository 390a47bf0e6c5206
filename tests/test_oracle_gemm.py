"""Pins for the oracle's block-scaled GEMM (CPU only).

Page "Fine-Grained FP8/FP4 Quantization", section "DeepGEMM: Tile-wise and Block-wise
Scaling": for each 128-wide K chunk the FP8 partial A_q*B_q is multiplied by
scale_A[m, kb] * scale_B[kb, n/128] and accumulated into C.  Pins: special cases that
reduce to a library integer matmul, exact power-of-two linearity per row / column block /
K block, and an exact int64 per-block formulation.
"""
import numpy as np
import pytest

import oracle


def _codes_for_ints(vals):
    """E4M3 codes whose values are the given small integers (found via the oracle's
    decode table, which is pinned to the OFP8 spec points separately)."""
    table = oracle.e4m3_decode(np.arange(256))
    lut = {}
    for c in range(256):
        v = table[c]
        if not np.isnan(v) and v == int(v) and int(v) not in lut and not (v == 0 and c == 0x80):
            lut[int(v)] = c
    return np.vectorize(lambda v: lut[int(v)])(vals).astype(np.uint8)


def _rand_codes(shape, rng):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3F      # no NaN codes
    return c


@pytest.mark.parametrize("M,N,K", [(5, 128, 128), (17, 256, 384)])
def test_integer_codes_unit_scales_equal_integer_matmul(M, N, K):
    rng = np.random.default_rng(10)
    ia = rng.integers(-8, 9, (M, K))
    ib = rng.integers(-8, 9, (K, N))
    Aq, Bq = _codes_for_ints(ia), _codes_for_ints(ib)
    sA = np.ones((M, K // 128), np.float32)
    sB = np.ones((K // 128, N // 128), np.float32)
    C, S = oracle.gemm_f64(Aq, sA, Bq, sB)
    assert np.array_equal(C, (ia @ ib).astype(np.float64))
    assert np.array_equal(S, (np.abs(ia) @ np.abs(ib)).astype(np.float64))


def test_int64_block_formulation():
    """C = sum_kb sA[m,kb] sB[kb,nb] 2^-18 P_kb with P_kb an exact int64 block product of
    the codes scaled to integers (value * 2^9)."""
    rng = np.random.default_rng(11)
    M, N, K = 9, 256, 512
    Aq, Bq = _rand_codes((M, K), rng), _rand_codes((K, N), rng)
    sA = rng.uniform(0.001, 2.0, (M, K // 128)).astype(np.float32)
    sB = rng.uniform(0.001, 2.0, (K // 128, N // 128)).astype(np.float32)
    C, S = oracle.gemm_f64(Aq, sA, Bq, sB)
    table = oracle.e4m3_decode(np.arange(256))
    ia = np.rint(table[Aq] * 512).astype(np.int64)
    ib = np.rint(table[Bq] * 512).astype(np.int64)
    assert np.array_equal(ia.astype(np.float64), table[Aq] * 512)
    ref = np.zeros((M, N))
    for kb in range(K // 128):
        P = ia[:, kb * 128:(kb + 1) * 128] @ ib[kb * 128:(kb + 1) * 128, :]   # exact int64
        sc = sA[:, kb:kb + 1].astype(np.float64) * np.repeat(sB[kb].astype(np.float64), 128)[None, :]
        ref += sc * (P.astype(np.float64) * 2.0 ** -18)
    assert np.all(np.abs(C - ref) <= 1e-12 * S + 1e-300)
    absref = np.abs(table[Aq] * np.repeat(sA.astype(np.float64), 128, axis=1)) @ \
        np.abs(table[Bq] * np.repeat(np.repeat(sB.astype(np.float64), 128, axis=0), 128, axis=1))
    assert np.allclose(S, absref, rtol=1e-12, atol=0)


def test_power_of_two_linearity_rows_columns_kblocks():
    rng = np.random.default_rng(12)
    M, N, K = 6, 384, 384
    Aq, Bq = _rand_codes((M, K), rng), _rand_codes((K, N), rng)
    sA = rng.uniform(0.01, 1.0, (M, K // 128)).astype(np.float32)
    sB = rng.uniform(0.01, 1.0, (K // 128, N // 128)).astype(np.float32)
    C, _ = oracle.gemm_f64(Aq, sA, Bq, sB)
    # doubling every scale of row m doubles exactly row m of C
    sA2 = sA.copy(); sA2[3, :] *= 2
    C2, _ = oracle.gemm_f64(Aq, sA2, Bq, sB)
    assert np.array_equal(C2[3], 2 * C[3]) and np.array_equal(np.delete(C2, 3, 0), np.delete(C, 3, 0))
    # doubling scale_B[:, nb] doubles exactly columns 128nb..128nb+127
    sB2 = sB.copy(); sB2[:, 1] *= 4
    C3, _ = oracle.gemm_f64(Aq, sA, Bq, sB2)
    assert np.array_equal(C3[:, 128:256], 4 * C[:, 128:256])
    assert np.array_equal(C3[:, :128], C[:, :128]) and np.array_equal(C3[:, 256:], C[:, 256:])
    # zeroing all K blocks but one leaves exactly that block's term
    for kb in range(K // 128):
        sBk = np.zeros_like(sB); sBk[kb] = sB[kb]
        Ck, _ = oracle.gemm_f64(Aq, sA, Bq, sBk)
        table = oracle.e4m3_decode(np.arange(256))
        a = table[Aq[:, kb * 128:(kb + 1) * 128]] * sA[:, kb:kb + 1].astype(np.float64)
        b = table[Bq[kb * 128:(kb + 1) * 128]] * np.repeat(sB[kb].astype(np.float64), 128)[None, :]
        assert np.all(np.abs(Ck - a @ b) <= 1e-13 * (np.abs(a) @ np.abs(b)))


def test_uniform_scales_reduce_to_per_tensor():
    rng = np.random.default_rng(13)
    M, N, K = 8, 128, 256
    Aq, Bq = _rand_codes((M, K), rng), _rand_codes((K, N), rng)
    sa, sb = np.float32(0.37), np.float32(0.0123)
    C, S = oracle.gemm_f64(Aq, np.full((M, 2), sa, np.float32), Bq, np.full((2, 1), sb, np.float32))
    table = oracle.e4m3_decode(np.arange(256))
    ref = float(sa) * float(sb) * (table[Aq] @ table[Bq])
    assert np.all(np.abs(C - ref) <= 1e-13 * S)


def test_pointwise_matches_full():
    rng = np.random.default_rng(14)
    M, N, K = 7, 256, 384
    Aq, Bq = _rand_codes((M, K), rng), _rand_codes((K, N), rng)
    sA = rng.uniform(0.01, 1.0, (M, 3)).astype(np.float32)
    sB = rng.uniform(0.01, 1.0, (3, 2)).astype(np.float32)
    C, S = oracle.gemm_f64(Aq, sA, Bq, sB)
    rows = rng.integers(0, M, 200); cols = rng.integers(0, N, 200)
    c, s = oracle.gemm_f64_at(Aq, sA, Bq, sB, rows, cols)
    assert np.array_equal(c, C[rows, cols]) and np.array_equal(s, S[rows, cols])


def test_rejects_bad_shapes():
    Aq = np.zeros((4, 200), np.uint8)
    with pytest.raises(ValueError):
        oracle.gemm_f64(Aq, np.ones((4, 1), np.float32), np.zeros((200, 128), np.uint8),
                        np.ones((1, 1), np.float32))
