"""Repeatability and full coverage of every output: each kernel family runs 20 times on the
same device inputs, its outputs refilled with sentinels (NaN for floats, 0xFF for codes and
scale bytes) before every run, and every run must equal the first bit for bit with no
sentinel left.  The kernels use no atomics on results (the NVFP4 global amax is an integer
max, order-independent), so nothing may vary between runs."""
import numpy as np
import pytest
import torch

import fine_grained_block_fgq_amd as fgq
import synth
from tests.gpu_util import dev_bf16, log

pytestmark = pytest.mark.gpu

RUNS = 20


def repeat(fn, outs):
    """Run fn() RUNS times with `outs` refilled with sentinels first; return the first run's
    outputs after checking the rest against them."""
    first = None
    for r in range(RUNS):
        for t in outs:
            if t.dtype in (torch.float32, torch.bfloat16):
                t.fill_(float("nan"))
            else:
                t.fill_(0xFF)
        fn()
        torch.cuda.synchronize()
        if first is None:
            first = [t.clone() for t in outs]
            for t in first:
                if t.dtype in (torch.float32, torch.bfloat16):
                    assert not torch.isnan(t).any(), "an output element was not written"
        else:
            for a, b in zip(first, outs):
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"run {r} differs"
    return first


@pytest.fixture(scope="module")
def operands():
    A, B, _ = synth.workload_inputs("tiny")
    Ad, Bd = dev_bf16(A), dev_bf16(B)
    # a wider weight so every family has columns to tile: B [512, 1024]
    Bw = dev_bf16(np.tile(B, (1, 4)))
    return Ad, Bd, Bw


def test_quantizers_repeat(operands):
    A, B, _ = operands
    M, K = A.shape
    N = B.shape[1]
    log("determinism: quantizers x20")
    Aq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sA = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
    repeat(lambda: fgq.fgq_quantize_act_1x128(A, Aq, sA), [Aq, sA])
    Bq = torch.empty((K, N), dtype=torch.uint8, device="cuda")
    sB = torch.empty((K // 128, N // 128), dtype=torch.float32, device="cuda")
    repeat(lambda: fgq.fgq_quantize_weight_128x128(B, Bq, sB), [Bq, sB])
    eA = torch.empty((M, K // 128), dtype=torch.uint8, device="cuda")
    repeat(lambda: fgq.fgq_quantize_act_1x128_ue8m0(A, Aq, eA), [Aq, eA])
    eB = torch.empty((K // 128, N // 128), dtype=torch.uint8, device="cuda")
    repeat(lambda: fgq.fgq_quantize_weight_128x128_ue8m0(B, Bq, eB), [Bq, eB])
    q4 = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    s4 = torch.empty((M, K // 16), dtype=torch.uint8, device="cuda")
    g4 = torch.empty((fgq.FGQ_NVFP4_GLOBAL_FLOATS,), dtype=torch.float32, device="cuda")
    # element 0 of the global-scale array is the output; the rest is the call's scratch
    repeat(lambda: fgq.fgq_quantize_nvfp4(A, q4, s4, g4), [q4, s4, g4[:1]])


@pytest.mark.parametrize("variant", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_gemm_families_repeat(operands, variant, out):
    A, _, Bw = operands
    log(f"determinism: gemm variant {variant} {out} x20")
    Aq, sA = fgq.fgq_quantize_act_1x128(A)
    Bq, sB = fgq.fgq_quantize_weight_128x128(Bw)
    M, N = Aq.shape[0], Bq.shape[1]
    C = torch.empty((M, N), dtype=out, device="cuda")
    repeat(lambda: fgq.fgq_gemm_fp8_blockscaled_variant(Aq, sA, Bq, sB, C, variant=variant), [C])


def test_fused_ue8m0_nvfp4_gemms_repeat(operands):
    A, _, Bw = operands
    log("determinism: fused, ue8m0 and nvfp4 gemms x20")
    Aq, sA = fgq.fgq_quantize_act_1x128(A)
    Bq, sB = fgq.fgq_quantize_weight_128x128(Bw)
    M, N = Aq.shape[0], Bq.shape[1]
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    Cq = torch.empty((M, N), dtype=torch.uint8, device="cuda")
    sC = torch.empty((M, N // 128), dtype=torch.float32, device="cuda")
    repeat(lambda: fgq.fgq_gemm_fp8_blockscaled_quant(Aq, sA, Bq, sB, C, Cq, sC), [C, Cq, sC])
    Ae, eA = fgq.fgq_quantize_act_1x128_ue8m0(A)
    Be, eB = fgq.fgq_quantize_weight_128x128_ue8m0(Bw)
    Cf = torch.empty((M, N), dtype=torch.float32, device="cuda")
    repeat(lambda: fgq.fgq_gemm_fp8_blockscaled_ue8m0(Ae, eA, Be, eB, Cf), [Cf])
    a4, sa4, ga4 = fgq.fgq_quantize_nvfp4(A)
    b4, sb4, gb4 = fgq.fgq_quantize_nvfp4(Bw.t().contiguous())
    repeat(lambda: fgq.fgq_gemm_nvfp4(a4, sa4, ga4, b4, sb4, gb4, Cf), [Cf])
