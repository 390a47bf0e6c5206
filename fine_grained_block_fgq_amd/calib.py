"""Python binding of libfgq_calib, the measurement library beside libfgq (include/fgq_calib.h):
the ceiling kernels the benchmark compares against and the probe of the FP8 matrix cores' own
accuracy.  None of these is a step of the method.  Argument marshalling only; raises if the
library is missing."""
from __future__ import annotations

import ctypes
import os

import torch

from . import FgqError, _HERE, _check, _dev, _stream

__all__ = ["library_path", "load", "fgq_calib_stream", "fgq_calib_mfma_f16",
           "fgq_calib_mfma_fp8", "fgq_probe_fp8_mfma_partials"]

_LIB_PATH = os.path.join(_HERE, "libfgq_calib.so")
_lib = None


def library_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libfgq_calib.so (built in-tree by ``__graft_entry__.build()``); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise FgqError("load", -100, f"{_LIB_PATH} is not built")
    lib = ctypes.CDLL(_LIB_PATH)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.fgq_calib_stream.restype = i32
    lib.fgq_calib_stream.argtypes = [p, p, i64, p]
    lib.fgq_calib_mfma_f16.restype = i32
    lib.fgq_calib_mfma_f16.argtypes = [p, i64, i64, p]
    lib.fgq_calib_mfma_fp8.restype = i32
    lib.fgq_calib_mfma_fp8.argtypes = [p, i64, i64, p]
    lib.fgq_probe_fp8_mfma_partials.restype = i32
    lib.fgq_probe_fp8_mfma_partials.argtypes = [p, p, p, i64, i64, i64, p]
    _lib = lib
    return lib


def fgq_calib_stream(src: torch.Tensor, dst: torch.Tensor, stream=None) -> int:
    """Measured-ceiling kernel with the activation quantizer's traffic: reads all of `src`
    (16 bytes per lane) and writes half as many bytes to `dst`.  Returns the bytes moved."""
    lib = load()
    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous device tensors")
    nbytes = src.numel() * src.element_size()
    if nbytes % 16 or dst.numel() * dst.element_size() < nbytes // 2:
        raise ValueError("src must be a multiple of 16 bytes and dst at least half its size")
    n16 = nbytes // 16
    _check("fgq_calib_stream", lib.fgq_calib_stream(src.data_ptr(), dst.data_ptr(), n16,
                                                    _stream(stream)))
    return 24 * n16


def fgq_calib_mfma_f16(out: torch.Tensor, blocks: int, iters: int, stream=None) -> float:
    """Measured-ceiling kernel of f16 MFMAs only; `out` float32 with blocks*512 elements.
    Returns the flops it performs."""
    lib = load()
    _dev(out, "out", torch.float32, (blocks * 512,))
    _check("fgq_calib_mfma_f16", lib.fgq_calib_mfma_f16(out.data_ptr(), blocks, iters,
                                                        _stream(stream)))
    return float(blocks) * 8 * iters * 16 * 16384


def fgq_calib_mfma_fp8(out: torch.Tensor, blocks: int, iters: int, stream=None) -> float:
    """Measured-ceiling kernel of FP8 (E4M3) MFMAs only; `out` float32 with blocks*512
    elements.  Returns the flops it performs."""
    lib = load()
    _dev(out, "out", torch.float32, (blocks * 512,))
    _check("fgq_calib_mfma_fp8", lib.fgq_calib_mfma_fp8(out.data_ptr(), blocks, iters,
                                                        _stream(stream)))
    return float(blocks) * 8 * iters * 16 * 65536


def fgq_probe_fp8_mfma_partials(A_q: torch.Tensor, B_q: torch.Tensor, P: torch.Tensor = None,
                                stream=None) -> torch.Tensor:
    """The unscaled 128-K chunk partials of A_q [M,K] and B_q [K,N] (uint8 E4M3 codes) as
    the FP8 matrix cores form them, one v_mfma_f32_16x16x128_f8f6f4 per 16x16 tile and chunk:
    P [K/128, M, N] float32.  For measuring that instruction's accuracy; the GEMM entry points
    do not use it."""
    lib = load()
    M, K = A_q.shape
    N = B_q.shape[1]
    if P is None:
        P = torch.empty((K // 128, M, N), dtype=torch.float32, device=A_q.device)
    _check("fgq_probe_fp8_mfma_partials", lib.fgq_probe_fp8_mfma_partials(
        _dev(A_q, "A_q", torch.uint8, (M, K)), _dev(B_q, "B_q", torch.uint8, (K, N)),
        _dev(P, "P", torch.float32, (K // 128, M, N)), M, N, K, _stream(stream)))
    return P
