"""fgq_gemm_fp8_blockscaled_noalloc (the K-split GEMM whose partials live in the library's own
per-GPU array, for callers that cannot allocate) against fgq_gemm_fp8_blockscaled_ws on the
same inputs, through the C ABI: two calls in a row, the second on a smaller problem, each
equal to the workspace call bit for bit (same kernels, same split) and within the tolerance of
the oracle's fp64 GEMM (page "Fine-Grained FP8/FP4 Quantization", section "DeepGEMM: Tile-wise
and Block-wise Scaling")."""
import numpy as np
import pytest
import torch

import fine_grained_block_fgq_amd as fgq
import oracle
from tests.gpu_util import dev_f32, dev_u8, gemm_error_ratio, log
from tests.test_gpu_gemm import random_operands

pytestmark = pytest.mark.gpu


def _c_abi_noalloc(Aq, sA, Bq, sB, C):
    lib = fgq.load()
    M, K = Aq.shape
    N = Bq.shape[1]
    st = lib.fgq_gemm_fp8_blockscaled_noalloc(Aq.data_ptr(), sA.data_ptr(), Bq.data_ptr(),
                                              sB.data_ptr(), C.data_ptr(), M, N, K,
                                              fgq.FGQ_OUT_F32,
                                              torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.fgq_status_string(st)


def _c_abi_ws(Aq, sA, Bq, sB, C, ws):
    lib = fgq.load()
    M, K = Aq.shape
    N = Bq.shape[1]
    st = lib.fgq_gemm_fp8_blockscaled_ws(Aq.data_ptr(), sA.data_ptr(), Bq.data_ptr(),
                                         sB.data_ptr(), C.data_ptr(), M, N, K, fgq.FGQ_OUT_F32,
                                         ws.data_ptr(), ws.numel() * ws.element_size(),
                                         torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.fgq_status_string(st)


def test_noalloc_matches_workspace_call_twice():
    for (M, N, K, seed) in [(128, 1024, 16384, 5), (96, 512, 16384, 6)]:
        need = fgq.fgq_gemm_workspace_size(M, N, K)
        log(f"noalloc {M}x{N}x{K}: planned workspace {need} bytes")
        assert need > 0   # the call splits K, so it uses the array
        Aq, sA, Bq, sB = random_operands(M, N, K, seed=seed)
        d = [dev_u8(Aq), dev_f32(sA), dev_u8(Bq), dev_f32(sB)]
        C_no = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        C_ws = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
        _c_abi_noalloc(*d, C_no)
        _c_abi_ws(*d, C_ws, ws)
        torch.cuda.synchronize()
        a = C_no.cpu().numpy()
        b = C_ws.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        Cr, S = oracle.gemm_f64(Aq, sA, Bq, sB)
        assert gemm_error_ratio(a.astype(np.float64), Cr, S, False) <= 1.0
