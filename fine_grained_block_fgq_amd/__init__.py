"""Python binding of libfgq, the gfx950 library for fine-grained FP8 quantization and the
block-scaled FP8 GEMM (page "Fine-Grained FP8/FP4 Quantization").

Argument marshalling only: every step runs in the HIP kernels behind the C ABI declared in
``include/fgq.h``.  The functions take torch CUDA (ROCm) tensors for device memory and run
on the current torch stream.  There is no fallback: if ``libfgq.so`` is missing or fails
to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "FgqError", "library_path", "load", "fgq_quantize_act_1x128",
    "fgq_quantize_weight_128x128", "fgq_gemm_fp8_blockscaled",
    "fgq_gemm_fp8_blockscaled_variant", "fgq_gemm_fp8_blockscaled_quant",
    "fgq_quantize_act_1x128_ue8m0", "fgq_quantize_weight_128x128_ue8m0",
    "fgq_gemm_fp8_blockscaled_ue8m0", "fgq_quantize_nvfp4", "fgq_gemm_nvfp4", "FGQ_OUT_F32", "FGQ_OUT_BF16", "FGQ_GEMM_AUTO",
    "FGQ_GEMM_WIDE_256x128", "FGQ_GEMM_WIDE_128x128", "FGQ_GEMM_NARROW_64x32",
    "FGQ_GEMM_SKINNY_128x32", "FGQ_GEMM_NARROW_64x64"
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfgq.so")
FGQ_OUT_F32, FGQ_OUT_BF16 = 0, 1
FGQ_GEMM_AUTO, FGQ_GEMM_WIDE_256x128, FGQ_GEMM_WIDE_128x128, FGQ_GEMM_NARROW_64x32 = 0, 1, 2, 3
FGQ_GEMM_SKINNY_128x32, FGQ_GEMM_NARROW_64x64 = 4, 5
# floats of the NVFP4 quantizer's global-scale argument (element 0 = the global scale)
FGQ_NVFP4_GLOBAL_FLOATS = 512
_lib = None


class FgqError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed: {message} (status {status})")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libfgq.so (built in-tree by ``__graft_entry__.build()``); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise FgqError("load", -100, f"{_LIB_PATH} is not built")
    lib = ctypes.CDLL(_LIB_PATH)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.fgq_quantize_act_1x128.restype = i32
    lib.fgq_quantize_act_1x128.argtypes = [p, p, p, i64, i64, p]
    lib.fgq_quantize_weight_128x128.restype = i32
    lib.fgq_quantize_weight_128x128.argtypes = [p, p, p, i64, i64, p]
    lib.fgq_gemm_fp8_blockscaled.restype = i32
    lib.fgq_gemm_fp8_blockscaled.argtypes = [p, p, p, p, p, i64, i64, i64, i32, p]
    lib.fgq_gemm_fp8_blockscaled_variant.restype = i32
    lib.fgq_gemm_fp8_blockscaled_variant.argtypes = [p, p, p, p, p, i64, i64, i64, i32, i32, p]
    lib.fgq_gemm_workspace_size.restype = i64
    lib.fgq_gemm_workspace_size.argtypes = [i64, i64, i64]
    lib.fgq_gemm_fp8_blockscaled_ws.restype = i32
    lib.fgq_gemm_fp8_blockscaled_ws.argtypes = [p, p, p, p, p, i64, i64, i64, i32, p, i64, p]
    lib.fgq_gemm_fp8_blockscaled_splitk.restype = i32
    lib.fgq_gemm_fp8_blockscaled_splitk.argtypes = [p, p, p, p, p, i64, i64, i64, i32, i32, p,
                                                    i64, p]
    lib.fgq_gemm_fp8_blockscaled_noalloc.restype = i32
    lib.fgq_gemm_fp8_blockscaled_noalloc.argtypes = [p, p, p, p, p, i64, i64, i64, i32, p]
    lib.fgq_quantize_act_1x128_ue8m0.restype = i32
    lib.fgq_quantize_act_1x128_ue8m0.argtypes = [p, p, p, i64, i64, p]
    lib.fgq_quantize_weight_128x128_ue8m0.restype = i32
    lib.fgq_quantize_weight_128x128_ue8m0.argtypes = [p, p, p, i64, i64, p]
    lib.fgq_gemm_fp8_blockscaled_ue8m0.restype = i32
    lib.fgq_gemm_fp8_blockscaled_ue8m0.argtypes = [p, p, p, p, p, i64, i64, i64, i32, i32, p]
    lib.fgq_quantize_nvfp4.restype = i32
    lib.fgq_quantize_nvfp4.argtypes = [p, p, p, p, i64, i64, p]
    lib.fgq_gemm_nvfp4.restype = i32
    lib.fgq_gemm_nvfp4.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, i32, p]
    lib.fgq_gemm_fp8_blockscaled_quant.restype = i32
    lib.fgq_gemm_fp8_blockscaled_quant.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, p]
    lib.fgq_status_string.restype = ctypes.c_char_p
    lib.fgq_status_string.argtypes = [i32]
    lib.fgq_version.restype = i32
    lib.fgq_version.argtypes = []
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        raise FgqError(fn, status, load().fgq_status_string(status).decode())


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev(t: torch.Tensor, name: str, dtype, shape):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (ROCm) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _first(t: torch.Tensor, name: str):
    """pointer to element 0 of a contiguous fp32 device tensor (a global scale, alone or as
    element 0 of the quantizer's global-scale array)"""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (ROCm) tensor")
    if t.dtype != torch.float32 or t.numel() < 1 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor with at least 1 element")
    return t.data_ptr()


def _codes_dtype(t: torch.Tensor):
    return t.dtype if t.dtype in (torch.uint8, torch.float8_e4m3fn) else torch.uint8


def fgq_quantize_act_1x128(X: torch.Tensor, Xq: torch.Tensor | None = None,
                           scale_X: torch.Tensor | None = None, stream=None):
    """X bf16 [M,K] -> (Xq uint8 E4M3FN codes [M,K], scale_X fp32 [M,K/128])."""
    lib = load()
    M, K = X.shape
    if Xq is None:
        Xq = torch.empty((M, K), dtype=torch.uint8, device=X.device)
    if scale_X is None:
        scale_X = torch.empty((M, K // 128), dtype=torch.float32, device=X.device)
    _check("fgq_quantize_act_1x128", lib.fgq_quantize_act_1x128(
        _dev(X, "X", torch.bfloat16, (M, K)), _dev(Xq, "Xq", _codes_dtype(Xq), (M, K)),
        _dev(scale_X, "scale_X", torch.float32, (M, K // 128)), M, K, _stream(stream)))
    return Xq, scale_X


def fgq_quantize_weight_128x128(W: torch.Tensor, Wq: torch.Tensor | None = None,
                                scale_W: torch.Tensor | None = None, stream=None):
    """W bf16 [K,N] -> (Wq uint8 E4M3FN codes [K,N], scale_W fp32 [K/128,N/128])."""
    lib = load()
    K, N = W.shape
    if Wq is None:
        Wq = torch.empty((K, N), dtype=torch.uint8, device=W.device)
    if scale_W is None:
        scale_W = torch.empty((K // 128, N // 128), dtype=torch.float32, device=W.device)
    _check("fgq_quantize_weight_128x128", lib.fgq_quantize_weight_128x128(
        _dev(W, "W", torch.bfloat16, (K, N)), _dev(Wq, "Wq", _codes_dtype(Wq), (K, N)),
        _dev(scale_W, "scale_W", torch.float32, (K // 128, N // 128)), K, N, _stream(stream)))
    return Wq, scale_W


def fgq_gemm_fp8_blockscaled(A_q: torch.Tensor, scale_A: torch.Tensor, B_q: torch.Tensor,
                             scale_B: torch.Tensor, C: torch.Tensor | None = None,
                             out_dtype: torch.dtype = torch.bfloat16, stream=None):
    """C[M,N] = block-scaled A_q[M,K] @ B_q[K,N] (scales [M,K/128] and [K/128,N/128])."""
    return _gemm("fgq_gemm_fp8_blockscaled", A_q, scale_A, B_q, scale_B, C, out_dtype, None,
                 stream)


def fgq_gemm_fp8_blockscaled_variant(A_q: torch.Tensor, scale_A: torch.Tensor,
                                     B_q: torch.Tensor, scale_B: torch.Tensor,
                                     C: torch.Tensor | None = None,
                                     out_dtype: torch.dtype = torch.bfloat16,
                                     variant: int = FGQ_GEMM_AUTO, stream=None):
    """fgq_gemm_fp8_blockscaled with an explicit kernel family (FGQ_GEMM_*)."""
    return _gemm("fgq_gemm_fp8_blockscaled_variant", A_q, scale_A, B_q, scale_B, C, out_dtype,
                 variant, stream)


def fgq_gemm_workspace_size(M: int, N: int, K: int) -> int:
    """Bytes of workspace fgq_gemm_fp8_blockscaled_ws splits K with for this shape on the
    current device (0: none needed)."""
    n = load().fgq_gemm_workspace_size(M, N, K)
    if n < 0:
        _check("fgq_gemm_workspace_size", int(n))
    return int(n)


def _workspace(ws):
    if ws is None:
        return None, 0
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
        raise TypeError("workspace must be a contiguous CUDA (ROCm) tensor")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def fgq_gemm_fp8_blockscaled_ws(A_q: torch.Tensor, scale_A: torch.Tensor, B_q: torch.Tensor,
                                scale_B: torch.Tensor, workspace: torch.Tensor | None,
                                C: torch.Tensor | None = None,
                                out_dtype: torch.dtype = torch.bfloat16, stream=None):
    """fgq_gemm_fp8_blockscaled with a caller-owned workspace (any dtype, contiguous device
    tensor of at least fgq_gemm_workspace_size bytes) for the K split of few-tile shapes."""
    return _gemm("fgq_gemm_fp8_blockscaled_ws", A_q, scale_A, B_q, scale_B, C, out_dtype, None,
                 stream, tail=list(_workspace(workspace)))


def fgq_gemm_fp8_blockscaled_splitk(A_q: torch.Tensor, scale_A: torch.Tensor,
                                    B_q: torch.Tensor, scale_B: torch.Tensor, splits: int,
                                    workspace: torch.Tensor | None, C: torch.Tensor | None = None,
                                    out_dtype: torch.dtype = torch.bfloat16, stream=None):
    """The K-split GEMM with an explicit split count (workspace >= splits*M*N*4 bytes)."""
    return _gemm("fgq_gemm_fp8_blockscaled_splitk", A_q, scale_A, B_q, scale_B, C, out_dtype,
                 int(splits), stream, tail=list(_workspace(workspace)))


def fgq_gemm_fp8_blockscaled_noalloc(A_q: torch.Tensor, scale_A: torch.Tensor,
                                     B_q: torch.Tensor, scale_B: torch.Tensor,
                                     C: torch.Tensor | None = None,
                                     out_dtype: torch.dtype = torch.bfloat16, stream=None):
    """fgq_gemm_fp8_blockscaled_ws with the library's own per-GPU array as its workspace (the C
    entry point allocates nothing; pass C to keep the binding from allocating it)."""
    return _gemm("fgq_gemm_fp8_blockscaled_noalloc", A_q, scale_A, B_q, scale_B, C, out_dtype,
                 None, stream)


def _gemm(fn, A_q, scale_A, B_q, scale_B, C, out_dtype, variant, stream, tail=()):
    lib = load()
    M, K = A_q.shape
    K2, N = B_q.shape
    if K2 != K:
        raise ValueError(f"A_q is [{M},{K}] but B_q is [{K2},{N}]")
    if C is None:
        C = torch.empty((M, N), dtype=out_dtype, device=A_q.device)
    code = {torch.float32: FGQ_OUT_F32, torch.bfloat16: FGQ_OUT_BF16}.get(C.dtype)
    if code is None:
        raise TypeError(f"C must be float32 or bfloat16, got {C.dtype}")
    args = [_dev(A_q, "A_q", _codes_dtype(A_q), (M, K)),
            _dev(scale_A, "scale_A", torch.float32, (M, K // 128)),
            _dev(B_q, "B_q", _codes_dtype(B_q), (K, N)),
            _dev(scale_B, "scale_B", torch.float32, (K // 128, N // 128)),
            _dev(C, "C", C.dtype, (M, N)), M, N, K, code]
    if variant is not None:
        args.append(int(variant))
    _check(fn, getattr(lib, fn)(*args, *tail, _stream(stream)))
    return C


def fgq_gemm_fp8_blockscaled_quant(A_q: torch.Tensor, scale_A: torch.Tensor, B_q: torch.Tensor,
                                   scale_B: torch.Tensor, C: torch.Tensor | None = None,
                                   C_q: torch.Tensor | None = None,
                                   scale_C: torch.Tensor | None = None, stream=None):
    """(C bf16, C_q, scale_C): the bf16 GEMM and the 1x128 quantization of that C, fused."""
    lib = load()
    M, K = A_q.shape
    K2, N = B_q.shape
    if K2 != K:
        raise ValueError(f"A_q is [{M},{K}] but B_q is [{K2},{N}]")
    dev = A_q.device
    if C is None:
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if C_q is None:
        C_q = torch.empty((M, N), dtype=torch.uint8, device=dev)
    if scale_C is None:
        scale_C = torch.empty((M, N // 128), dtype=torch.float32, device=dev)
    _check("fgq_gemm_fp8_blockscaled_quant", lib.fgq_gemm_fp8_blockscaled_quant(
        _dev(A_q, "A_q", _codes_dtype(A_q), (M, K)),
        _dev(scale_A, "scale_A", torch.float32, (M, K // 128)),
        _dev(B_q, "B_q", _codes_dtype(B_q), (K, N)),
        _dev(scale_B, "scale_B", torch.float32, (K // 128, N // 128)),
        _dev(C, "C", torch.bfloat16, (M, N)), _dev(C_q, "C_q", _codes_dtype(C_q), (M, N)),
        _dev(scale_C, "scale_C", torch.float32, (M, N // 128)), M, N, K, _stream(stream)))
    return C, C_q, scale_C


def fgq_quantize_act_1x128_ue8m0(X: torch.Tensor, Xq: torch.Tensor | None = None,
                                 scale_X: torch.Tensor | None = None, stream=None):
    """1x128 activation quantization with UE8M0 exponent-byte scales (uint8 [M, K/128])."""
    lib = load()
    M, K = X.shape
    if Xq is None:
        Xq = torch.empty((M, K), dtype=torch.uint8, device=X.device)
    if scale_X is None:
        scale_X = torch.empty((M, K // 128), dtype=torch.uint8, device=X.device)
    _check("fgq_quantize_act_1x128_ue8m0", lib.fgq_quantize_act_1x128_ue8m0(
        _dev(X, "X", torch.bfloat16, (M, K)), _dev(Xq, "Xq", _codes_dtype(Xq), (M, K)),
        _dev(scale_X, "scale_X", torch.uint8, (M, K // 128)), M, K, _stream(stream)))
    return Xq, scale_X


def fgq_quantize_weight_128x128_ue8m0(W: torch.Tensor, Wq: torch.Tensor | None = None,
                                      scale_W: torch.Tensor | None = None, stream=None):
    """128x128 weight quantization with UE8M0 exponent-byte scales (uint8 [K/128, N/128])."""
    lib = load()
    K, N = W.shape
    if Wq is None:
        Wq = torch.empty((K, N), dtype=torch.uint8, device=W.device)
    if scale_W is None:
        scale_W = torch.empty((K // 128, N // 128), dtype=torch.uint8, device=W.device)
    _check("fgq_quantize_weight_128x128_ue8m0", lib.fgq_quantize_weight_128x128_ue8m0(
        _dev(W, "W", torch.bfloat16, (K, N)), _dev(Wq, "Wq", _codes_dtype(Wq), (K, N)),
        _dev(scale_W, "scale_W", torch.uint8, (K // 128, N // 128)), K, N, _stream(stream)))
    return Wq, scale_W


def fgq_gemm_fp8_blockscaled_ue8m0(A_q: torch.Tensor, scale_A: torch.Tensor,
                                   B_q: torch.Tensor, scale_B: torch.Tensor,
                                   C: torch.Tensor | None = None,
                                   out_dtype: torch.dtype = torch.bfloat16,
                                   variant: int = FGQ_GEMM_AUTO, stream=None):
    """Block-scaled FP8 GEMM on UE8M0 exponent-byte scales."""
    lib = load()
    M, K = A_q.shape
    K2, N = B_q.shape
    if K2 != K:
        raise ValueError(f"A_q is [{M},{K}] but B_q is [{K2},{N}]")
    if C is None:
        C = torch.empty((M, N), dtype=out_dtype, device=A_q.device)
    code = {torch.float32: FGQ_OUT_F32, torch.bfloat16: FGQ_OUT_BF16}.get(C.dtype)
    if code is None:
        raise TypeError(f"C must be float32 or bfloat16, got {C.dtype}")
    _check("fgq_gemm_fp8_blockscaled_ue8m0", lib.fgq_gemm_fp8_blockscaled_ue8m0(
        _dev(A_q, "A_q", _codes_dtype(A_q), (M, K)),
        _dev(scale_A, "scale_A", torch.uint8, (M, K // 128)),
        _dev(B_q, "B_q", _codes_dtype(B_q), (K, N)),
        _dev(scale_B, "scale_B", torch.uint8, (K // 128, N // 128)),
        _dev(C, "C", C.dtype, (M, N)), M, N, K, code, int(variant), _stream(stream)))
    return C


def fgq_quantize_nvfp4(X: torch.Tensor, Xq: torch.Tensor | None = None,
                       scale_X: torch.Tensor | None = None,
                       global_scale: torch.Tensor | None = None, stream=None):
    """NVFP4 of bf16 X [R, C] (blocks of 16 along C): (packed codes uint8 [R, C/2], E4M3
    block scales uint8 [R, C/16], fp32 [FGQ_NVFP4_GLOBAL_FLOATS] whose element 0 is the global
    scale and the rest scratch of the call)."""
    lib = load()
    R, C = X.shape
    dev = X.device
    if Xq is None:
        Xq = torch.empty((R, C // 2), dtype=torch.uint8, device=dev)
    if scale_X is None:
        scale_X = torch.empty((R, C // 16), dtype=torch.uint8, device=dev)
    if global_scale is None:
        global_scale = torch.empty((FGQ_NVFP4_GLOBAL_FLOATS,), dtype=torch.float32, device=dev)
    _check("fgq_quantize_nvfp4", lib.fgq_quantize_nvfp4(
        _dev(X, "X", torch.bfloat16, (R, C)), _dev(Xq, "Xq", torch.uint8, (R, C // 2)),
        _dev(scale_X, "scale_X", torch.uint8, (R, C // 16)),
        _dev(global_scale, "global_scale", torch.float32, (FGQ_NVFP4_GLOBAL_FLOATS,)), R, C,
        _stream(stream)))
    return Xq, scale_X, global_scale


def fgq_gemm_nvfp4(A_q: torch.Tensor, scale_A: torch.Tensor, global_A: torch.Tensor,
                   B_q: torch.Tensor, scale_B: torch.Tensor, global_B: torch.Tensor,
                   C: torch.Tensor | None = None, out_dtype: torch.dtype = torch.bfloat16,
                   stream=None):
    """NVFP4 GEMM: A [M, K] and the weight stored as its transpose [N, K] (both packed)."""
    lib = load()
    M, K2 = A_q.shape
    N, K2b = B_q.shape
    if K2 != K2b:
        raise ValueError(f"A_q is [{M},{K2}] bytes but B_q is [{N},{K2b}]")
    K = 2 * K2
    if C is None:
        C = torch.empty((M, N), dtype=out_dtype, device=A_q.device)
    code = {torch.float32: FGQ_OUT_F32, torch.bfloat16: FGQ_OUT_BF16}.get(C.dtype)
    if code is None:
        raise TypeError(f"C must be float32 or bfloat16, got {C.dtype}")
    _check("fgq_gemm_nvfp4", lib.fgq_gemm_nvfp4(
        _dev(A_q, "A_q", torch.uint8, (M, K // 2)),
        _dev(scale_A, "scale_A", torch.uint8, (M, K // 16)),
        _first(global_A, "global_A"),
        _dev(B_q, "B_q", torch.uint8, (N, K // 2)),
        _dev(scale_B, "scale_B", torch.uint8, (N, K // 16)),
        _first(global_B, "global_B"),
        _dev(C, "C", C.dtype, (M, N)), M, N, K, code, _stream(stream)))
    return C
