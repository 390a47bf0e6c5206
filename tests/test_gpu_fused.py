"""GPU parity of the GEMM with the fused 1x128 epilogue quantization.

Page "Kernel Fusion" (overview) applied to page "Fine-Grained FP8/FP4 Quantization",
section "Scaling Granularities": the fused call must return the bf16 GEMM result C and,
bit for bit, the oracle's 1x128 activation quantization of that very C.  C itself is checked
against the oracle's fp64 GEMM with the bf16 tolerance of the plain GEMM, and against the
plain GEMM of the same kernel family bit for bit."""
import numpy as np
import pytest
import torch

import fine_grained_block_fgq_amd as fgq
import oracle
from tests.gpu_util import dev_f32, dev_u8, free, gemm_error_ratio, gpu_gemm, log
from tests.test_gpu_gemm import random_operands, workload_operands, _sample

pytestmark = pytest.mark.gpu


def gpu_fused(Aq, sA, Bq, sB):
    M, N = Aq.shape[0], Bq.shape[1]
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    Cq = torch.full((M, N), 0xFF, dtype=torch.uint8, device="cuda")
    sC = torch.full((M, N // 128), float("nan"), dtype=torch.float32, device="cuda")
    fgq.fgq_gemm_fp8_blockscaled_quant(dev_u8(Aq), dev_f32(sA), dev_u8(Bq), dev_f32(sB), C, Cq,
                                       sC)
    torch.cuda.synchronize()
    bits = C.view(torch.int16).cpu().numpy().view(np.uint16)
    return bits, Cq.cpu().numpy(), sC.cpu().numpy()


def family(M, N):
    """the GEMM the fused call runs for this shape: the fused wide kernel (1: 256x128,
    2: 128x128) when its 128x128 tiles cover the 256 CUs, else the automatic choice (0) of
    the plain GEMM followed by the quantizer"""
    if ((M + 127) // 128) * (N // 128) < 256:
        return 0
    return 1 if M >= 256 and ((M + 255) // 256) * (N // 128) >= 256 else 2


def check_quant_of_c(bits, Cq, sC):
    q_ref, s_ref = oracle.quantize_act(bits)
    assert np.array_equal(sC.view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(Cq, q_ref)


@pytest.mark.parametrize("M,N,K", [
    # few output tiles: the GEMM family of the shape, then the quantizer
    (1, 128, 128), (7, 128, 384), (129, 256, 256), (255, 384, 128), (300, 512, 640),
    (512, 512, 384), (64, 1024, 1152), (33, 128, 0),
    # the fused kernel (256x128 and 128x128 tiles), ragged M
    (300, 16384, 256), (129, 32768, 128),
])
def test_fused_edge_shapes(M, N, K):
    log(f"fused edge M={M} N={N} K={K}")
    Aq, sA, Bq, sB = random_operands(M, N, K, seed=3 * M + 5 * N + 11 * K)
    bits, Cq, sC = gpu_fused(Aq, sA, Bq, sB)
    C = bits.astype(np.uint32) << 16
    C = C.view(np.float32).astype(np.float64)
    Cr, S = oracle.gemm_f64(Aq, sA, Bq, sB)
    assert gemm_error_ratio(C, Cr, S, True) <= 1.0
    check_quant_of_c(bits, Cq, sC)
    # the same bits as the plain bf16 GEMM of the same kernel family
    Cp = gpu_gemm(Aq, sA, Bq, sB, torch.bfloat16, family(M, N))
    assert np.array_equal(C, Cp)


@pytest.mark.parametrize("name", ["tiny", "skinny", "sq4096"])
def test_fused_workloads(name):
    Aq, sA, Bq, sB = workload_operands(name)
    M, N = Aq.shape[0], Bq.shape[1]
    log(f"fused {name} {M}x{N}x{Aq.shape[1]}")
    bits, Cq, sC = gpu_fused(Aq, sA, Bq, sB)
    check_quant_of_c(bits, Cq, sC)
    C = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rows, cols = _sample(M, N, np.random.default_rng(9), n=5000)
    cr, s = oracle.gemm_f64_at(Aq, sA, Bq, sB, rows, cols)
    r = gemm_error_ratio(C[rows, cols], cr, s, True)
    log(f"  max error ratio {r:.3e}")
    assert r <= 1.0
    free()
