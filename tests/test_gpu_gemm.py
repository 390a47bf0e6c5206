"""GPU parity of the block-scaled FP8 GEMM against the oracle's fp64 dequantize-then-matmul.

Page "Fine-Grained FP8/FP4 Quantization", section "DeepGEMM: Tile-wise and Block-wise
Scaling".  Pass rule per element: |C - C_ref| <= 1e-5 * sum_k |a_k b_k| + 1e-6, plus one
bf16 ulp of the reference magnitude when C is bf16.  Operand codes and scales come from
the oracle's quantizers (never from the device), on the seeded workloads."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import free, gemm_error_ratio, gpu_gemm, log

pytestmark = pytest.mark.gpu

# every kernel family on every edge shape (0 = the automatic choice)
VARIANTS = [0, 1, 2, 3, 4, 5]


def random_operands(M, N, K, seed):
    rng = np.random.default_rng(seed)
    Aq = rng.integers(0, 256, (M, K)).astype(np.uint8)
    Bq = rng.integers(0, 256, (K, N)).astype(np.uint8)
    Aq[(Aq & 0x7F) == 0x7F] = 0x3E
    Bq[(Bq & 0x7F) == 0x7F] = 0xBE
    sA = (10.0 ** rng.uniform(-3, 1, (M, K // 128))).astype(np.float32)
    sB = (10.0 ** rng.uniform(-3, 1, (K // 128, N // 128))).astype(np.float32)
    if M > 2 and K >= 256:
        sA[1, 1] = 0.0                    # an all-zero activation tile
    return Aq, sA, Bq, sB


def workload_operands(name):
    A, B, _ = synth.workload_inputs(name)
    Aq, sA = oracle.quantize_act(A)
    Bq, sB = oracle.quantize_weight(B)
    return Aq, sA, Bq, sB


@pytest.mark.parametrize("M,N,K", [
    (1, 128, 128), (7, 128, 384), (129, 256, 256), (255, 384, 128), (300, 512, 640),
    (256, 256, 128), (512, 512, 384), (300, 512, 256), (64, 1024, 1152), (33, 128, 0),
])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("variant", VARIANTS)
def test_edge_shapes(M, N, K, out, variant):
    log(f"gemm edge M={M} N={N} K={K} {out} variant={variant}")
    Aq, sA, Bq, sB = random_operands(M, N, K, seed=M + 7 * N + 13 * K)
    C = gpu_gemm(Aq, sA, Bq, sB, torch.float32 if out == "f32" else torch.bfloat16, variant)
    Cr, S = oracle.gemm_f64(Aq, sA, Bq, sB)
    if K == 0:
        assert np.all(C == 0)
    assert gemm_error_ratio(C, Cr, S, out == "bf16") <= 1.0


def test_tiny_workload_full():
    Aq, sA, Bq, sB = workload_operands("tiny")
    log("gemm tiny 128x256x512 f32")
    C = gpu_gemm(Aq, sA, Bq, sB, torch.float32)
    Cr, S = oracle.gemm_f64(Aq, sA, Bq, sB)
    r = gemm_error_ratio(C, Cr, S, False)
    log(f"  max error ratio {r:.3e}")
    assert r <= 1.0


@pytest.mark.parametrize("variant", [None, 2, 3, 4, 5])
def test_skinny_workload_full(variant):
    Aq, sA, Bq, sB = workload_operands("skinny")
    log(f"gemm skinny 128x7168x2048 f32 variant={variant}")
    C = gpu_gemm(Aq, sA, Bq, sB, torch.float32, variant)
    Cr, S = oracle.gemm_f64(Aq, sA, Bq, sB)
    r = gemm_error_ratio(C, Cr, S, False)
    log(f"  max error ratio {r:.3e}")
    assert r <= 1.0
    # repeatable bit for bit (the split-K partials are summed in a fixed order)
    assert np.array_equal(C, gpu_gemm(Aq, sA, Bq, sB, torch.float32, variant))
    free()


def _sample(M, N, rng, n=20000):
    """random output elements plus the first and last rows and columns"""
    rows = np.concatenate([rng.integers(0, M, n), np.full(N, 0), np.full(N, M - 1),
                           np.arange(M), np.arange(M)])
    cols = np.concatenate([rng.integers(0, N, n), np.arange(N), np.arange(N),
                           np.full(M, 0), np.full(M, N - 1)])
    return rows, cols


@pytest.mark.parametrize("name", ["sq4096", "prefill"])
def test_large_workload_full(name):
    """The 4096^3 and the prefill (4096x7168x16384) workloads: every element of C, fp32 and
    bf16 output, against the full fp64 oracle GEMM (the method defines every C[m,n])."""
    Aq, sA, Bq, sB = workload_operands(name)
    M, N = Aq.shape[0], Bq.shape[1]
    log(f"gemm {name} {M}x{N}x{Aq.shape[1]} bf16 + f32, every element")
    Cb = gpu_gemm(Aq, sA, Bq, sB, torch.bfloat16)
    Cf = gpu_gemm(Aq, sA, Bq, sB, torch.float32)
    Cf2 = gpu_gemm(Aq, sA, Bq, sB, torch.float32)
    free()
    Cr, S = oracle.gemm_f64(Aq, sA, Bq, sB)
    rb = gemm_error_ratio(Cb, Cr, S, True)
    rf = gemm_error_ratio(Cf, Cr, S, False)
    log(f"  max error ratio over all {M * N} elements: bf16 {rb:.3e} f32 {rf:.3e}")
    assert rb <= 1.0 and rf <= 1.0
    # bf16 output is the nearest-even rounding of the same fp32 accumulation
    ref_bf16 = torch.from_numpy(Cf.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(Cb, ref_bf16.astype(np.float64))
    # repeatable bit for bit
    assert np.array_equal(Cf, Cf2)


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_wave_tail_split(out):
    """256 x 38400: 300 tiles of 256x128 on 256 CUs leave a last round of 44; those columns
    run as 128x128 tiles in a second launch.  Every element against the oracle."""
    M, N, K = 256, 38400, 256
    log(f"gemm tail split M={M} N={N} K={K} {out}")
    Aq, sA, Bq, sB = random_operands(M, N, K, seed=99)
    C = gpu_gemm(Aq, sA, Bq, sB, torch.float32 if out == "f32" else torch.bfloat16)
    Cr, S = oracle.gemm_f64(Aq, sA, Bq, sB)
    assert gemm_error_ratio(C, Cr, S, out == "bf16") <= 1.0
    free()


@pytest.mark.parametrize("variant", VARIANTS)
def test_long_k(variant):
    """K = 33,280 (260 chunks): more than 64 chunks per wave (or per K group) in every family,
    so scale_B is taken well past the first 64 chunks; scales within a factor 10 of each other
    keep every chunk's share of C above the tolerance"""
    M, N, K = 70, 256, 128 * 260
    rng = np.random.default_rng(260 + variant)
    Aq, _, Bq, _ = random_operands(M, N, K, seed=260)
    sA = (10.0 ** rng.uniform(-1, 0, (M, K // 128))).astype(np.float32)
    sB = (10.0 ** rng.uniform(-1, 0, (K // 128, N // 128))).astype(np.float32)
    log(f"long K {M}x{N}x{K} variant {variant}")
    C = gpu_gemm(Aq, sA, Bq, sB, torch.float32, variant)
    Cr, S = oracle.gemm_f64(Aq, sA, Bq, sB)
    assert gemm_error_ratio(C, Cr, S, False) <= 1.0
