"""GPU parity of the K split across workgroups (fgq_gemm_fp8_blockscaled_ws / _splitk): fp32
partial tiles in a caller-owned workspace, summed in slice order by a second pass (page
"Persistent kernel (grid = SM count, internal tile loop)", section "Variants": one tile's K
loop spread over several workgroups).  Every element against the oracle's fp64 GEMM (page
"Fine-Grained FP8/FP4 Quantization", section "DeepGEMM: Tile-wise and Block-wise Scaling"),
repeatability bit for bit, and the fallback without a workspace."""
import numpy as np
import pytest
import torch

import fine_grained_block_fgq_amd as fgq
import oracle
from tests.gpu_util import dev_f32, dev_u8, free, gemm_error_ratio, gpu_gemm, log
from tests.test_gpu_gemm import random_operands, workload_operands

pytestmark = pytest.mark.gpu


def splitk(Aq, sA, Bq, sB, splits, out_dtype, ws_bytes=None):
    M, N, K = Aq.shape[0], Bq.shape[1], Aq.shape[1]
    need = splits * M * N * 4 if splits > 1 else 0
    nbytes = ws_bytes if ws_bytes is not None else need
    ws = torch.full(((nbytes + 15) // 4 + 4,), float("nan"), dtype=torch.float32, device="cuda")
    C = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
    fgq.fgq_gemm_fp8_blockscaled_splitk(dev_u8(Aq), dev_f32(sA), dev_u8(Bq), dev_f32(sB), splits,
                                        ws, C)
    torch.cuda.synchronize()
    return C.float().cpu().numpy().astype(np.float64)


def ws_gemm(Aq, sA, Bq, sB, out_dtype, ws_bytes):
    M, N = Aq.shape[0], Bq.shape[1]
    ws = None if ws_bytes is None else torch.full(((max(ws_bytes, 4) + 3) // 4,), float("nan"),
                                                  dtype=torch.float32, device="cuda")
    C = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
    fgq.fgq_gemm_fp8_blockscaled_ws(dev_u8(Aq), dev_f32(sA), dev_u8(Bq), dev_f32(sB), ws, C)
    torch.cuda.synchronize()
    return C.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("M,N,K,splits", [
    (1, 128, 256, 2), (7, 256, 384, 3), (128, 384, 1024, 4), (129, 256, 1152, 5),
    (300, 512, 2048, 7), (64, 1024, 4096, 16), (128, 128, 128, 1), (33, 256, 512, 4),
])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_explicit_splits(M, N, K, splits, out):
    log(f"splitk M={M} N={N} K={K} splits={splits} {out}")
    Aq, sA, Bq, sB = random_operands(M, N, K, seed=M + 3 * N + 5 * K + splits)
    C = splitk(Aq, sA, Bq, sB, splits, torch.float32 if out == "f32" else torch.bfloat16)
    Cr, S = oracle.gemm_f64(Aq, sA, Bq, sB)
    assert gemm_error_ratio(C, Cr, S, out == "bf16") <= 1.0


@pytest.mark.parametrize("splits", [2, 4, 8])
def test_skinny_workload_full_and_repeatable(splits):
    """the skinny workload 128x7168x2048 (fp32 C) split over workgroups: every element, 20 runs
    bit-identical"""
    Aq, sA, Bq, sB = workload_operands("skinny")
    log(f"splitk skinny splits={splits}")
    C = splitk(Aq, sA, Bq, sB, splits, torch.float32)
    Cr, S = oracle.gemm_f64(Aq, sA, Bq, sB)
    r = gemm_error_ratio(C, Cr, S, False)
    log(f"  max error ratio {r:.3e}")
    assert r <= 1.0
    for _ in range(19):
        assert np.array_equal(C, splitk(Aq, sA, Bq, sB, splits, torch.float32))
    free()


def test_planned_split_long_k():
    """128x1024x16384: the shape class the workspace path splits (16 splits planned on 256
    CUs); every element, 20 runs bit-identical"""
    M, N, K = 128, 1024, 16384
    Aq, sA, Bq, sB = random_operands(M, N, K, seed=1616)
    need = fgq.fgq_gemm_workspace_size(M, N, K)
    log(f"splitk planned {M}x{N}x{K}: workspace {need} bytes")
    assert need > 0 and need % (M * N * 4) == 0
    C = ws_gemm(Aq, sA, Bq, sB, torch.float32, need)
    Cr, S = oracle.gemm_f64(Aq, sA, Bq, sB)
    r = gemm_error_ratio(C, Cr, S, False)
    log(f"  max error ratio {r:.3e}, splits {need // (M * N * 4)}")
    assert r <= 1.0
    for _ in range(19):
        assert np.array_equal(C, ws_gemm(Aq, sA, Bq, sB, torch.float32, need))
    free()


def test_fallback_without_workspace():
    """too small a workspace (or none): the call computes C as fgq_gemm_fp8_blockscaled does,
    bit for bit"""
    Aq, sA, Bq, sB = random_operands(128, 512, 16384, seed=77)
    need = fgq.fgq_gemm_workspace_size(128, 512, 16384)
    assert need > 0
    plain = gpu_gemm(Aq, sA, Bq, sB, torch.float32)
    assert np.array_equal(ws_gemm(Aq, sA, Bq, sB, torch.float32, None), plain)
    assert np.array_equal(ws_gemm(Aq, sA, Bq, sB, torch.float32, need - 4), plain)
    split = ws_gemm(Aq, sA, Bq, sB, torch.float32, need)
    Cr, S = oracle.gemm_f64(Aq, sA, Bq, sB)
    assert gemm_error_ratio(split, Cr, S, False) <= 1.0


def test_plan():
    """many tiles or short K: no split; few tiles and long K: a split"""
    assert fgq.fgq_gemm_workspace_size(4096, 4096, 4096) == 0
    assert fgq.fgq_gemm_workspace_size(4096, 7168, 16384) == 0
    assert fgq.fgq_gemm_workspace_size(128, 7168, 2048) == 0
    assert fgq.fgq_gemm_workspace_size(128, 1024, 16384) > 0
    assert fgq.fgq_gemm_workspace_size(128, 512, 32768) > 0
