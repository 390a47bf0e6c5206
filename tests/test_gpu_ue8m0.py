"""GPU parity of the UE8M0 (power-of-two scale) quantizers and GEMM against the oracle.

Page "Fine-Grained FP8/FP4 Quantization", section "Blackwell: Native Block Scaling" and
table "UE8M0 vs E4M3 Scale Formats".  Quantization: codes and exponent bytes bit-exact.
With a power-of-two scale a code depends on x and the exponent byte only, so the domain is
covered by (a) every positive finite bf16 amax -> its exponent, and (b) for every exponent
the rule can produce, every x up to the largest amax that maps to it.  GEMM: the fp32
tolerance |C - C_ref| <= 1e-5 * sum|a*b| + 1e-6 (+ one bf16 ulp for bf16 C) against the
oracle's fp64 GEMM on the decoded scales, on every kernel family."""
import numpy as np
import pytest
import torch

import fine_grained_block_fgq_amd as fgq
import oracle
import synth
from tests.domain import all_amax_bits, domain_tiles
from tests.gpu_util import dev_bf16, dev_u8, free, gemm_error_ratio, log
from tests.test_gpu_quant import special_matrix

pytestmark = pytest.mark.gpu


def gpu_act_e8(bits):
    M, K = bits.shape
    Xq = torch.full((M, K), 0xFF, dtype=torch.uint8, device="cuda")
    e = torch.full((M, K // 128), 0xFF, dtype=torch.uint8, device="cuda")
    fgq.fgq_quantize_act_1x128_ue8m0(dev_bf16(bits), Xq, e)
    torch.cuda.synchronize()
    return Xq.cpu().numpy(), e.cpu().numpy()


def gpu_weight_e8(bits):
    K, N = bits.shape
    Wq = torch.full((K, N), 0xFF, dtype=torch.uint8, device="cuda")
    e = torch.full((K // 128, N // 128), 0xFF, dtype=torch.uint8, device="cuda")
    fgq.fgq_quantize_weight_128x128_ue8m0(dev_bf16(bits), Wq, e)
    torch.cuda.synchronize()
    return Wq.cpu().numpy(), e.cpu().numpy()


def test_every_amax_exponent():
    amax = all_amax_bits().astype(np.uint16)
    X = np.zeros((amax.size, 128), np.uint16)
    X[:, 37] = amax
    X[1::2, 37] |= 0x8000                         # the sign of amax must not matter
    q, e = gpu_act_e8(X)
    rq, re = oracle.quantize_act_ue8m0(X)
    assert np.array_equal(e, re) and np.array_equal(q, rq)


def test_every_x_for_every_exponent():
    amax = all_amax_bits().astype(np.uint16)
    X = np.zeros((amax.size, 128), np.uint16)
    X[:, 0] = amax
    _, e = oracle.quantize_act_ue8m0(X)
    e = e[:, 0]
    # the largest amax of each exponent the rule produces
    last = np.nonzero(np.diff(e.astype(np.int64), append=1000))[0]
    reps = amax[last]
    log(f"{reps.size} exponents")
    for ci, ch in enumerate(np.array_split(reps, 4)):
        T, _, _ = domain_tiles(ch)
        q, ge = gpu_act_e8(T)
        rq, rge = oracle.quantize_act_ue8m0(T)
        assert np.array_equal(ge, rge)
        bad = q != rq
        assert not bad.any(), (ci, int(bad.sum()))
        log(f"chunk {ci}: {T.size} elements ok")
    free()


@pytest.mark.parametrize("M,K", [(1, 128), (7, 384), (129, 1024), (64, 7168)])
def test_act_edge_shapes(M, K):
    X = special_matrix(M, K, seed=7 * M + K)
    q, e = gpu_act_e8(X)
    rq, re = oracle.quantize_act_ue8m0(X)
    assert np.array_equal(e, re) and np.array_equal(q, rq)


@pytest.mark.parametrize("K,N", [(128, 128), (384, 256), (1024, 640)])
def test_weight_edge_shapes(K, N):
    W = special_matrix(K, N, seed=11 * K + N)
    q, e = gpu_weight_e8(W)
    rq, re = oracle.quantize_weight_ue8m0(W)
    assert np.array_equal(e, re) and np.array_equal(q, rq)


@pytest.mark.parametrize("name", ["tiny", "skinny", "actq"])
def test_workload_quantizers(name):
    A, B, _ = synth.workload_inputs(name)
    log(f"ue8m0 quantizers on {name}")
    q, e = gpu_act_e8(A)
    rq, re = oracle.quantize_act_ue8m0(A)
    assert np.array_equal(e, re) and np.array_equal(q, rq)
    if B is not None:
        q, e = gpu_weight_e8(B)
        rq, re = oracle.quantize_weight_ue8m0(B)
        assert np.array_equal(e, re) and np.array_equal(q, rq)
    free()


def gpu_gemm_e8(Aq, eA, Bq, eB, out_dtype, variant=0):
    M, N = Aq.shape[0], Bq.shape[1]
    C = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
    fgq.fgq_gemm_fp8_blockscaled_ue8m0(dev_u8(Aq), dev_u8(eA), dev_u8(Bq), dev_u8(eB), C,
                                       variant=variant)
    torch.cuda.synchronize()
    return C.float().cpu().numpy().astype(np.float64)


def random_e8_operands(M, N, K, seed):
    rng = np.random.default_rng(seed)
    Aq = rng.integers(0, 256, (M, K)).astype(np.uint8)
    Bq = rng.integers(0, 256, (K, N)).astype(np.uint8)
    Aq[(Aq & 0x7F) == 0x7F] = 0x3E
    Bq[(Bq & 0x7F) == 0x7F] = 0xBE
    eA = rng.integers(100, 140, (M, K // 128)).astype(np.uint8)
    eB = rng.integers(100, 140, (K // 128, N // 128)).astype(np.uint8)
    if M > 2 and K >= 256:
        eA[1, 1] = 0                     # 2^-127: the combined scale leaves the fp32 range
    return Aq, eA, Bq, eB


@pytest.mark.parametrize("M,N,K", [
    (1, 128, 128), (7, 128, 384), (129, 256, 256), (300, 512, 640), (512, 512, 384),
    (64, 1024, 1152), (33, 128, 0),
])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("variant", [0, 1, 2, 3, 4, 5])
def test_gemm_edge_shapes(M, N, K, out, variant):
    Aq, eA, Bq, eB = random_e8_operands(M, N, K, seed=M + 3 * N + 5 * K)
    C = gpu_gemm_e8(Aq, eA, Bq, eB, torch.float32 if out == "f32" else torch.bfloat16, variant)
    Cr, S = oracle.gemm_f64(Aq, oracle.ue8m0_decode(eA), Bq, oracle.ue8m0_decode(eB))
    if K == 0:
        assert np.all(C == 0)
    assert gemm_error_ratio(C, Cr, S, out == "bf16") <= 1.0


@pytest.mark.parametrize("name,variant", [("tiny", 0), ("skinny", 0), ("skinny", 2),
                                          ("sq4096", 0)])
def test_gemm_workloads(name, variant):
    A, B, _ = synth.workload_inputs(name)
    Aq, eA = oracle.quantize_act_ue8m0(A)
    Bq, eB = oracle.quantize_weight_ue8m0(B)
    M, N = Aq.shape[0], Bq.shape[1]
    log(f"ue8m0 gemm {name} variant {variant}")
    C = gpu_gemm_e8(Aq, eA, Bq, eB, torch.float32, variant)
    sA, sB = oracle.ue8m0_decode(eA), oracle.ue8m0_decode(eB)
    if M * N <= 128 * 7168:
        Cr, S = oracle.gemm_f64(Aq, sA, Bq, sB)
        r = gemm_error_ratio(C, Cr, S, False)
    else:
        rng = np.random.default_rng(3)
        rows, cols = rng.integers(0, M, 20000), rng.integers(0, N, 20000)
        cr, s = oracle.gemm_f64_at(Aq, sA, Bq, sB, rows, cols)
        r = gemm_error_ratio(C[rows, cols], cr, s, False)
    log(f"  max error ratio {r:.3e}")
    assert r <= 1.0
    free()


@pytest.mark.parametrize("variant", [0, 1, 2, 3, 4, 5])
def test_gemm_long_k(variant):
    """K = 33,280 (260 chunks): more than 64 chunks per wave (or per K group) in every family,
    so each wave reloads its scale_B exponent bytes past the first 64 chunks; exponents within
    2^6 of each other keep every chunk's share of C above the tolerance"""
    M, N, K = 70, 256, 128 * 260
    Aq, _, Bq, _ = random_e8_operands(M, N, K, seed=260)
    rng = np.random.default_rng(261 + variant)
    eA = rng.integers(124, 131, (M, K // 128)).astype(np.uint8)
    eB = rng.integers(124, 131, (K // 128, N // 128)).astype(np.uint8)
    log(f"ue8m0 long K {M}x{N}x{K} variant {variant}")
    C = gpu_gemm_e8(Aq, eA, Bq, eB, torch.float32, variant)
    Cr, S = oracle.gemm_f64(Aq, oracle.ue8m0_decode(eA), Bq, oracle.ue8m0_decode(eB))
    assert gemm_error_ratio(C, Cr, S, False) <= 1.0
