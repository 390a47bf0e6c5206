"""GPU parity of the 1x128 activation and 128x128 weight quantizers against the oracle:
codes and scales must be bit-exact (page "Fine-Grained FP8/FP4 Quantization", sections
"Scaling Granularities" and "DeepGEMM: Tile-wise and Block-wise Scaling")."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import bits_equal, free, gpu_quant_act, gpu_quant_weight, log

pytestmark = pytest.mark.gpu


def special_matrix(rows, cols, seed):
    """N(0,1) bf16 with groups of special values: an all-zero group, negative zeros,
    bf16 subnormals, values near the bf16 maximum, and single large outliers."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((rows, cols)).astype(np.float32)
    bits = (v.view(np.uint32) >> 16).astype(np.uint16)
    if cols >= 256 and rows >= 1:
        bits[0, 128:256] = 0
        bits[0, 130] = 0x8000
    if rows >= 2 and cols >= 128:
        bits[1, :128] = rng.integers(0, 0x80, 128).astype(np.uint16) | \
            (rng.integers(0, 2, 128).astype(np.uint16) << 15)          # subnormals only
    if rows >= 3 and cols >= 128:
        bits[2, :128] = (0x7F00 + rng.integers(0, 0x7F, 128)).astype(np.uint16)  # huge
    if rows >= 4:
        bits[rows - 1, cols - 1] = 0x4700                              # 32768
    return bits


@pytest.mark.parametrize("M,K", [(1, 128), (7, 384), (129, 1024), (255, 256), (64, 7168)])
def test_act_edge_shapes(M, K):
    log(f"act edge M={M} K={K}")
    X = special_matrix(M, K, seed=M * 1000 + K)
    q, s = gpu_quant_act(X)
    rq, rs = oracle.quantize_act(X)
    assert bits_equal(s, rs) and bits_equal(q, rq)


def test_act_tiny_workload():
    A, _, _ = synth.workload_inputs("tiny")
    log(f"act tiny {A.shape}")
    q, s = gpu_quant_act(A)
    rq, rs = oracle.quantize_act(A)
    assert bits_equal(s, rs) and bits_equal(q, rq)


def test_act_full_workload_16384x7168():
    A, _, n = synth.workload_inputs("actq")
    log(f"act [16384,7168] outliers={n}")
    q, s = gpu_quant_act(A)
    rq, rs = oracle.quantize_act(A)
    assert bits_equal(s, rs), int(np.sum(s.view(np.uint32) != rs.view(np.uint32)))
    assert bits_equal(q, rq), int(np.sum(q != rq))
    # run again without sentinels: identical bits (no races, nothing left unwritten)
    q2, s2 = gpu_quant_act(A, sentinel=False)
    assert bits_equal(q2, q) and bits_equal(s2, s)
    del A, q, s, rq, rs, q2, s2
    free()


@pytest.mark.parametrize("name", ["tiny", "sq4096", "skinny"])
def test_act_gemm_workloads(name):
    A, _, _ = synth.workload_inputs(name)
    log(f"act {name} {A.shape}")
    q, s = gpu_quant_act(A)
    rq, rs = oracle.quantize_act(A)
    assert bits_equal(s, rs) and bits_equal(q, rq)


@pytest.mark.parametrize("K,N", [(128, 128), (256, 384), (512, 256), (640, 1280)])
def test_weight_edge_shapes(K, N):
    log(f"weight edge K={K} N={N}")
    W = special_matrix(K, N, seed=K * 7 + N)
    q, s = gpu_quant_weight(W)
    rq, rs = oracle.quantize_weight(W)
    assert bits_equal(s, rs) and bits_equal(q, rq)


def test_weight_zero_and_subnormal_blocks():
    W = np.zeros((256, 256), np.uint16)
    W[0, 0] = 0x8000                      # block (0,0): all zeros with a -0
    W[128:, :128] = 0x0001                # block (1,0): smallest subnormal everywhere
    W[200, 5] = 0x8003
    W[:128, 128:] = 0x7F7F                # block (0,1): bf16 max
    q, s = gpu_quant_weight(W)
    rq, rs = oracle.quantize_weight(W)
    assert bits_equal(s, rs) and bits_equal(q, rq)
    assert s[0, 0] == 0 and q[0, 0] == 0x80 and q[0, 1] == 0x00


@pytest.mark.parametrize("name", ["tiny", "sq4096", "skinny", "prefill"])
def test_weight_workloads(name):
    _, B, _ = synth.workload_inputs(name)
    log(f"weight {name} {B.shape}")
    q, s = gpu_quant_weight(B)
    rq, rs = oracle.quantize_weight(B)
    assert bits_equal(s, rs), int(np.sum(s.view(np.uint32) != rs.view(np.uint32)))
    assert bits_equal(q, rq), int(np.sum(q != rq))
    del B, q, s, rq, rs
    free()


def test_act_prefill_workload():
    A, _, n = synth.workload_inputs("prefill")
    log(f"act prefill {A.shape} outliers={n}")
    q, s = gpu_quant_act(A)
    rq, rs = oracle.quantize_act(A)
    assert bits_equal(s, rs) and bits_equal(q, rq)
    del A, q, s, rq, rs
    free()
