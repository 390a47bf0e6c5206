"""Operands past 2^31 elements: every offset the kernels form must be 64-bit.  Each test
uses a tensor of 2^31 + 2^24 or more elements (random finite inputs from numpy's seeded
generator), runs the library on it, and checks a sample spread over the whole tensor,
including its last rows and columns, against the oracle: quantizer codes and scales bit for
bit, GEMM outputs within the tolerance.  A 32-bit offset would wrap and either fault
(refused by the host-side checks long before) or read and write the wrong elements, which
the sampled comparison at the far end of the tensor catches."""
import numpy as np
import pytest
import torch

import fine_grained_block_fgq_amd as fgq
import oracle
from tests.gpu_util import dev_u8, free, gemm_error_ratio, log

pytestmark = pytest.mark.gpu

BIG = 131072            # a dimension of 2^17
ROWS = 16512            # 2^17 * 16512 = 2^31 + 2^24 elements


def finite_bf16(rng, shape):
    """Random bf16 bit patterns that are finite (no exponent 0xFF), any sign."""
    h = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    h[(h & 0x7F80) == 0x7F80] &= np.uint16(0xFF7F)
    return h


def to_dev_bits(h):
    return torch.from_numpy(h.view(np.int16)).cuda().view(torch.bfloat16)


def test_act_quantizer_past_2g_elements():
    rng = np.random.default_rng(31)
    M, K = ROWS, BIG
    log(f"act quantizer [{M},{K}] ({M * K} elements)")
    X = finite_bf16(rng, (M, K))
    Xd = to_dev_bits(X)
    Xq, sX = fgq.fgq_quantize_act_1x128(Xd)
    torch.cuda.synchronize()
    del Xd
    rows = np.array([0, 1, 4097, 8191, 8192, M // 2 + 3, M - 2, M - 1])
    got_q = Xq[torch.from_numpy(rows).cuda()].cpu().numpy()
    got_s = sX[torch.from_numpy(rows).cuda()].cpu().numpy()
    del Xq, sX
    free()
    want_q, want_s = oracle.quantize_act(np.ascontiguousarray(X[rows]))
    assert np.array_equal(got_q, want_q)
    assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32))


def test_weight_quantizer_past_2g_elements():
    rng = np.random.default_rng(32)
    K, N = BIG, ROWS                                # ROWS = 129 * 128
    log(f"weight quantizer [{K},{N}] ({K * N} elements)")
    W = finite_bf16(rng, (K, N))
    Wd = to_dev_bits(W)
    Wq, sW = fgq.fgq_quantize_weight_128x128(Wd)
    torch.cuda.synchronize()
    del Wd
    for kb in (0, 511, K // 128 - 1):               # block rows, all N blocks of each
        ks = slice(128 * kb, 128 * kb + 128)
        got_q = Wq[ks].cpu().numpy()
        got_s = sW[kb].cpu().numpy()
        want_q, want_s = oracle.quantize_weight(np.ascontiguousarray(W[ks]))
        assert np.array_equal(got_q, want_q), kb
        assert np.array_equal(got_s.view(np.uint32), want_s[0].view(np.uint32)), kb
    del Wq, sW
    free()


def random_codes(rng, shape):
    q = rng.integers(0, 256, size=shape, dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x3E                    # no NaN codes
    return q


@pytest.mark.parametrize("big", ["A", "B"])
def test_gemm_past_2g_operand_elements(big):
    rng = np.random.default_rng(33 if big == "A" else 34)
    K = BIG
    M, N = (ROWS, 128) if big == "A" else (128, ROWS)
    Aq = random_codes(rng, (M, K))
    Bq = random_codes(rng, (K, N))
    sA = (10.0 ** rng.uniform(-2, 1, (M, K // 128))).astype(np.float32)
    sB = (10.0 ** rng.uniform(-2, 1, (K // 128, N // 128))).astype(np.float32)
    rows = np.concatenate([rng.integers(0, M, 120), [0, M - 1, M - 1, 0]])
    cols = np.concatenate([rng.integers(0, N, 120), [0, N - 1, 0, N - 1]])
    cr, s = oracle.gemm_f64_at(Aq, sA, Bq, sB, rows, cols)
    dA, dB = dev_u8(Aq), dev_u8(Bq)
    dsA, dsB = torch.from_numpy(sA).cuda(), torch.from_numpy(sB).cuda()
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    # the automatic choice, then every family (0 = automatic)
    for variant in (0, 1, 2, 3, 4, 5):
        log(f"gemm {M}x{N}x{K}, {big} past 2^31 elements, variant {variant}")
        C.fill_(float("nan"))
        fgq.fgq_gemm_fp8_blockscaled_variant(dA, dsA, dB, dsB, C, variant=variant)
        torch.cuda.synchronize()
        assert not torch.isnan(C).any()
        got = C[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].cpu().numpy()
        ratio = gemm_error_ratio(got.astype(np.float64), cr, s, False)
        log(f"  max error ratio {ratio:.3e}")
        assert ratio <= 1.0
    del dA, dB, C
    free()
