"""Parity over seeded random shapes: M in 1..700, N and K multiples of 128 up to 2048, random
E4M3 codes (every finite code can occur) and scales over four decades.  Each shape runs the
automatic choice and one other GEMM family picked at random, with fp32 or bf16 output, and
the UE8M0 and NVFP4 GEMMs on their own random operands; every output element is checked
against the fp64 oracle (|C - C_ref| <= 1e-5 * sum|ab| + 1e-6, plus one bf16 ulp for bf16)."""
import numpy as np
import pytest
import torch

import fine_grained_block_fgq_amd as fgq
import oracle
from tests.gpu_util import dev_f32, dev_u8, gemm_error_ratio, gpu_gemm, log

pytestmark = pytest.mark.gpu

SHAPES = 40


def shapes():
    rng = np.random.default_rng(2024)
    out = []
    for i in range(SHAPES):
        M = int(rng.integers(1, 701))
        N = 128 * int(rng.integers(1, 17))
        K = 128 * int(rng.integers(1, 17))
        variant = int(rng.integers(1, 6))
        out.append((i, M, N, K, variant, bool(rng.integers(0, 2))))
    return out


def codes(rng, shape):
    q = rng.integers(0, 256, shape).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x3E
    return q


@pytest.mark.parametrize("i,M,N,K,variant,bf16", shapes())
def test_random_shape(i, M, N, K, variant, bf16):
    rng = np.random.default_rng(100 + i)
    Aq, Bq = codes(rng, (M, K)), codes(rng, (K, N))
    sA = (10.0 ** rng.uniform(-3, 1, (M, K // 128))).astype(np.float32)
    sB = (10.0 ** rng.uniform(-3, 1, (K // 128, N // 128))).astype(np.float32)
    Cr, S = oracle.gemm_f64(Aq, sA, Bq, sB)
    out = torch.bfloat16 if bf16 else torch.float32
    for v in (None, variant):
        log(f"random shape {i}: {M}x{N}x{K} variant {v} {'bf16' if bf16 else 'f32'}")
        C = gpu_gemm(Aq, sA, Bq, sB, out, v)
        assert gemm_error_ratio(C, Cr, S, bf16) <= 1.0

    # UE8M0 scales: exponent bytes over a range that keeps products inside fp32
    eA = rng.integers(100, 140, (M, K // 128)).astype(np.uint8)
    eB = rng.integers(100, 140, (K // 128, N // 128)).astype(np.uint8)
    Ce = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    fgq.fgq_gemm_fp8_blockscaled_ue8m0(dev_u8(Aq), dev_u8(eA), dev_u8(Bq), dev_u8(eB), Ce)
    torch.cuda.synchronize()
    Cr_e, S_e = oracle.gemm_f64(Aq, oracle.ue8m0_decode(eA).astype(np.float32), Bq,
                                oracle.ue8m0_decode(eB).astype(np.float32))
    assert gemm_error_ratio(Ce.cpu().numpy().astype(np.float64), Cr_e, S_e, False) <= 1.0

    # NVFP4: packed E2M1 codes, E4M3 block scales, fp32 global scales; B stored [N, K]
    a4 = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    b4 = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sa4 = rng.integers(0x08, 0x7E, (M, K // 16)).astype(np.uint8)
    sb4 = rng.integers(0x08, 0x7E, (N, K // 16)).astype(np.uint8)
    gA, gB = np.float32(0.031), np.float32(2.5)
    C4 = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    fgq.fgq_gemm_nvfp4(dev_u8(a4), dev_u8(sa4), dev_f32(np.array([gA])), dev_u8(b4),
                       dev_u8(sb4), dev_f32(np.array([gB])), C4)
    torch.cuda.synchronize()
    Cr4, S4 = oracle.gemm_nvfp4_f64(a4, sa4, gA, b4, sb4, gB)
    assert gemm_error_ratio(C4.cpu().numpy().astype(np.float64), Cr4, S4, False) <= 1.0


def quant_shapes():
    rng = np.random.default_rng(77)
    return [(i, int(rng.integers(1, 301)), 128 * int(rng.integers(1, 33)),
             16 * int(rng.integers(1, 257))) for i in range(30)]


def bf16_data(rng, shape):
    """bf16 bits: normals over a wide magnitude range, a few outliers, an all-zero row part"""
    x = rng.standard_normal(shape) * 10.0 ** rng.uniform(-6, 4, shape[0])[:, None]
    x[rng.random(shape) < 0.001] *= 300.0
    h = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    if shape[1] >= 256:
        h[0, 128:256] = 0
    return h


@pytest.mark.parametrize("i,M,K,C", quant_shapes())
def test_random_shape_quantizers(i, M, K, C):
    from tests.gpu_util import dev_bf16, gpu_quant_act, gpu_quant_weight
    rng = np.random.default_rng(500 + i)
    log(f"random quantizer shapes {i}: act/ue8m0 [{M},{K}], weight [{K},{min(K, 1024)}], nvfp4 [{M},{C}]")
    X = bf16_data(rng, (M, K))
    q, s = gpu_quant_act(X)
    rq, rs = oracle.quantize_act(X)
    assert np.array_equal(q, rq) and np.array_equal(s.view(np.uint32), rs.view(np.uint32))
    q, e = fgq.fgq_quantize_act_1x128_ue8m0(dev_bf16(X))
    rq, re = oracle.quantize_act_ue8m0(X)
    assert np.array_equal(q.cpu().numpy(), rq) and np.array_equal(e.cpu().numpy(), re)
    W = bf16_data(rng, (K, min(K, 1024)))
    q, s = gpu_quant_weight(W)
    rq, rs = oracle.quantize_weight(W)
    assert np.array_equal(q, rq) and np.array_equal(s.view(np.uint32), rs.view(np.uint32))
    Y = bf16_data(rng, (M, C))
    q, s, g = fgq.fgq_quantize_nvfp4(dev_bf16(Y))
    rq, rs, rg = oracle.quantize_nvfp4(Y)
    assert np.array_equal(q.cpu().numpy(), rq) and np.array_equal(s.cpu().numpy(), rs)
    assert np.float32(g.cpu().numpy()[0]).view(np.uint32) == np.float32(rg).view(np.uint32)
