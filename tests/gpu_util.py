"""Helpers for the GPU parity tests: move bf16 bit arrays to the device, run the library
through its binding, and compare with the oracle."""
import os
import sys

import numpy as np
import torch

import fine_grained_block_fgq_amd as fgq


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev_u8(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes)).cuda()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def gpu_quant_act(bits: np.ndarray, sentinel=True):
    X = dev_bf16(bits)
    M, K = bits.shape
    Xq = torch.full((M, K), 0xFF, dtype=torch.uint8, device="cuda") if sentinel else None
    sX = torch.full((M, K // 128), float("nan"), dtype=torch.float32, device="cuda") \
        if sentinel else None
    Xq, sX = fgq.fgq_quantize_act_1x128(X, Xq, sX)
    torch.cuda.synchronize()
    return Xq.cpu().numpy(), sX.cpu().numpy()


def gpu_quant_weight(bits: np.ndarray, sentinel=True):
    W = dev_bf16(bits)
    K, N = bits.shape
    Wq = torch.full((K, N), 0xFF, dtype=torch.uint8, device="cuda") if sentinel else None
    sW = torch.full((K // 128, N // 128), float("nan"), dtype=torch.float32, device="cuda") \
        if sentinel else None
    Wq, sW = fgq.fgq_quantize_weight_128x128(W, Wq, sW)
    torch.cuda.synchronize()
    return Wq.cpu().numpy(), sW.cpu().numpy()


def gpu_gemm(Aq, sA, Bq, sB, out_dtype, variant=None):
    M, N = Aq.shape[0], Bq.shape[1]
    C = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
    if variant is None:
        fgq.fgq_gemm_fp8_blockscaled(dev_u8(Aq), dev_f32(sA), dev_u8(Bq), dev_f32(sB), C)
    else:
        fgq.fgq_gemm_fp8_blockscaled_variant(dev_u8(Aq), dev_f32(sA), dev_u8(Bq), dev_f32(sB),
                                             C, variant=variant)
    torch.cuda.synchronize()
    return C.float().cpu().numpy().astype(np.float64)


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


def ulp_bf16(x):
    """Spacing of bf16 values at magnitude x (x >= 0)."""
    x = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(x)) - 7)


def gemm_error_ratio(C, C_ref, S, bf16: bool):
    """max over elements of |C - C_ref| / allowed, allowed = 1e-5*S + 1e-6 (+ one bf16
    ulp of the reference magnitude for bf16 output); <= 1 passes."""
    tol = 1e-5 * S + 1e-6
    if bf16:
        tol = tol + ulp_bf16(np.abs(C_ref) + tol)
    err = np.abs(C - C_ref)
    if not np.all(np.isfinite(C)):
        return float("inf")
    return float(np.max(err / tol)) if err.size else 0.0


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
