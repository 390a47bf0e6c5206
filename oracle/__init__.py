"""CPU oracle for fine-grained FP8 quantization and the block-scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg
may use this package; the product path never does.  It shares no code with the HIP
library.  The arithmetic lives in ``fgq_oracle.c`` (scalar C, fp64 for the GEMM); this
module only builds it, loads it, and splits independent rows across host threads (each
thread runs the same scalar code on its own rows, so the results do not depend on the
thread count).

Method source: the page "Fine-Grained FP8/FP4 Quantization", sections "Scaling
Granularities" (1x128 activation tiles, 128x128 weight blocks) and "DeepGEMM: Tile-wise
and Block-wise Scaling" (scale shapes [M, K/128] and [K/128, N/128]; per-128-K partial
times scale_A[m,kb]*scale_B[kb,nb], accumulated), and its table "UE8M0 vs E4M3 Scale
Formats" (E4M3 reaches 448).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fgq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
CFLAGS = _CFLAGS = ["-O2", "-std=gnu99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-fno-math-errno"]

_lib = None


def build() -> str:
    """Compile fgq_oracle.c into liboracle.so next to it (gcc)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # FGQ_ORACLE_LIB: a separately built copy (the pin-strength test runs the pins against
    # deliberately broken builds of fgq_oracle.c)
    path = os.environ.get("FGQ_ORACLE_LIB")
    if not path:
        path = _LIB
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
    lib = ctypes.CDLL(path)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_e4m3_encode_array.restype = None
    lib.oracle_e4m3_encode_array.argtypes = [p, p, i64]
    lib.oracle_quantize_act_1x128.restype = ctypes.c_int
    lib.oracle_quantize_act_1x128.argtypes = [p, p, p, i64, i64, i64, i64]
    lib.oracle_quantize_weight_128x128.restype = ctypes.c_int
    lib.oracle_quantize_weight_128x128.argtypes = [p, p, p, i64, i64, i64, i64]
    lib.oracle_ue8m0_decode.restype = ctypes.c_double
    lib.oracle_ue8m0_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_quantize_act_1x128_ue8m0.restype = ctypes.c_int
    lib.oracle_quantize_act_1x128_ue8m0.argtypes = [p, p, p, i64, i64, i64, i64]
    lib.oracle_quantize_weight_128x128_ue8m0.restype = ctypes.c_int
    lib.oracle_quantize_weight_128x128_ue8m0.argtypes = [p, p, p, i64, i64, i64, i64]
    lib.oracle_e2m1_decode.restype = ctypes.c_double
    lib.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e2m1_encode.restype = ctypes.c_uint8
    lib.oracle_e2m1_encode.argtypes = [ctypes.c_float]
    lib.oracle_quantize_nvfp4.restype = ctypes.c_int
    lib.oracle_quantize_nvfp4.argtypes = [p, p, p, p, i64, i64]
    lib.oracle_gemm_nvfp4_f64.restype = ctypes.c_int
    lib.oracle_gemm_nvfp4_f64.argtypes = [p, p, ctypes.c_float, p, p, ctypes.c_float, i64, i64,
                                          i64, p, p, i64, i64]
    lib.oracle_gemm_f64.restype = ctypes.c_int
    lib.oracle_gemm_f64.argtypes = [p, p, p, p, i64, i64, i64, p, p, i64, i64]
    lib.oracle_gemm_f64_at.restype = ctypes.c_int
    lib.oracle_gemm_f64_at.argtypes = [p, p, p, p, i64, i64, i64, p, p, i64, p, p]
    _lib = lib
    return lib


def threads() -> int:
    """Host threads used to split independent rows (capped at 16)."""
    return max(1, min(16, os.cpu_count() or 1))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _split(n: int, parts: int):
    parts = max(1, min(parts, n)) if n > 0 else 1
    step = (n + parts - 1) // parts if n > 0 else 0
    return [(i, min(n, i + step)) for i in range(0, n, step)] if n > 0 else []


def _run(fn, ranges, nthreads):
    if not ranges:
        return
    with ThreadPoolExecutor(max_workers=nthreads) as ex:
        codes = list(ex.map(lambda r: fn(*r), ranges))
    if any(c != 0 for c in codes):
        raise ValueError("oracle rejected the arguments")


def e4m3_decode(codes) -> np.ndarray:
    """fp64 value of each E4M3FN code (NaN for 0x7F/0xFF)."""
    lib = _load()
    table = np.array([lib.oracle_e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(y, nthreads: int | None = None) -> np.ndarray:
    """Round fp32 values to E4M3FN codes (nearest, ties to even, saturating at 448)."""
    lib = _load()
    y = np.ascontiguousarray(y, dtype=np.float32).reshape(-1)
    q = np.empty(y.shape, dtype=np.uint8)
    nt = nthreads or threads()

    def part(a, b):
        lib.oracle_e4m3_encode_array(_ptr(y) + 4 * a, _ptr(q) + a, b - a)
        return 0

    _run(part, _split(y.size, nt * 4), nt)
    return q


def quantize_act(X_bits: np.ndarray, nthreads: int | None = None):
    """1x128 activation quantization of bf16 bits X [M,K] -> (codes [M,K], scales [M,K/128])."""
    lib = _load()
    X = np.ascontiguousarray(X_bits, dtype=np.uint16)
    M, K = X.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    Xq = np.empty((M, K), dtype=np.uint8)
    sX = np.empty((M, K // 128), dtype=np.float32)
    nt = nthreads or threads()
    _run(lambda a, b: lib.oracle_quantize_act_1x128(_ptr(X), _ptr(Xq), _ptr(sX), M, K, a, b),
         _split(M, nt * 4), nt)
    return Xq, sX


def quantize_weight(W_bits: np.ndarray, nthreads: int | None = None):
    """128x128 weight quantization of bf16 bits W [K,N] -> (codes [K,N], scales [K/128,N/128])."""
    lib = _load()
    W = np.ascontiguousarray(W_bits, dtype=np.uint16)
    K, N = W.shape
    if K % 128 or N % 128:
        raise ValueError("K and N must be multiples of 128")
    Wq = np.empty((K, N), dtype=np.uint8)
    sW = np.empty((K // 128, N // 128), dtype=np.float32)
    nt = nthreads or threads()
    _run(lambda a, b: lib.oracle_quantize_weight_128x128(_ptr(W), _ptr(Wq), _ptr(sW), K, N, a, b),
         _split(K // 128, nt * 2), nt)
    return Wq, sW


def ue8m0_decode(e) -> np.ndarray:
    """fp32 value 2^(e-127) of each UE8M0 byte (exact; NaN for 255), by the oracle."""
    lib = _load()
    e = np.asarray(e, dtype=np.uint8)
    table = np.array([lib.oracle_ue8m0_decode(c) for c in range(256)], dtype=np.float64)
    return table[e].astype(np.float32)


def quantize_act_ue8m0(X_bits: np.ndarray, nthreads: int | None = None):
    """1x128 activation quantization with UE8M0 scales -> (codes [M,K], exponents [M,K/128])."""
    lib = _load()
    X = np.ascontiguousarray(X_bits, dtype=np.uint16)
    M, K = X.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    Xq = np.empty((M, K), dtype=np.uint8)
    sX = np.empty((M, K // 128), dtype=np.uint8)
    nt = nthreads or threads()
    _run(lambda a, b: lib.oracle_quantize_act_1x128_ue8m0(_ptr(X), _ptr(Xq), _ptr(sX), M, K, a,
                                                         b),
         _split(M, nt * 4), nt)
    return Xq, sX


def quantize_weight_ue8m0(W_bits: np.ndarray, nthreads: int | None = None):
    """128x128 weight quantization with UE8M0 scales -> (codes [K,N], exponents [K/128,N/128])."""
    lib = _load()
    W = np.ascontiguousarray(W_bits, dtype=np.uint16)
    K, N = W.shape
    if K % 128 or N % 128:
        raise ValueError("K and N must be multiples of 128")
    Wq = np.empty((K, N), dtype=np.uint8)
    sW = np.empty((K // 128, N // 128), dtype=np.uint8)
    nt = nthreads or threads()
    _run(lambda a, b: lib.oracle_quantize_weight_128x128_ue8m0(_ptr(W), _ptr(Wq), _ptr(sW), K, N,
                                                              a, b),
         _split(K // 128, nt * 2), nt)
    return Wq, sW


def e2m1_decode(codes) -> np.ndarray:
    """Value of each E2M1 code (low 4 bits), by the oracle."""
    lib = _load()
    table = np.array([lib.oracle_e2m1_decode(c) for c in range(16)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8) & 15]


def e2m1_encode(y) -> np.ndarray:
    """Nearest E2M1 code (ties to even, saturating at 6) of each fp32 value."""
    lib = _load()
    y = np.asarray(y, dtype=np.float32)
    return np.array([lib.oracle_e2m1_encode(float(v)) for v in y.reshape(-1)],
                    dtype=np.uint8).reshape(y.shape)


def quantize_nvfp4(X_bits: np.ndarray):
    """NVFP4 of bf16 bits X [R, C] -> (packed codes [R, C/2], E4M3 block scales [R, C/16],
    fp32 global scale)."""
    lib = _load()
    X = np.ascontiguousarray(X_bits, dtype=np.uint16)
    R, C = X.shape
    if C % 16:
        raise ValueError("C must be a multiple of 16")
    Xq = np.empty((R, C // 2), dtype=np.uint8)
    sX = np.empty((R, C // 16), dtype=np.uint8)
    g = np.zeros(1, dtype=np.float32)
    if lib.oracle_quantize_nvfp4(_ptr(X), _ptr(Xq), _ptr(sX), _ptr(g), R, C) != 0:
        raise ValueError("bad shape")
    return Xq, sX, np.float32(g[0])


def gemm_nvfp4_f64(Aq, sA, gA, Bq, sB, gB, nthreads: int | None = None, rows=None):
    """fp64 NVFP4 GEMM reference: (C [M,N], S [M,N]) for A [M,K] and B stored [N,K];
    rows=(m0, m1) computes only those rows (the others are left as NaN)."""
    lib = _load()
    Aq = np.ascontiguousarray(Aq, dtype=np.uint8)
    Bq = np.ascontiguousarray(Bq, dtype=np.uint8)
    sA = np.ascontiguousarray(sA, dtype=np.uint8)
    sB = np.ascontiguousarray(sB, dtype=np.uint8)
    M, N, K = Aq.shape[0], Bq.shape[0], Aq.shape[1] * 2
    if Bq.shape[1] * 2 != K or sA.shape != (M, K // 16) or sB.shape != (N, K // 16):
        raise ValueError("shape mismatch")
    C = np.full((M, N), np.nan, dtype=np.float64)
    S = np.full((M, N), np.nan, dtype=np.float64)
    r0, r1 = rows if rows is not None else (0, M)
    nt = nthreads or threads()
    _run(lambda a, b: lib.oracle_gemm_nvfp4_f64(_ptr(Aq), _ptr(sA), float(gA), _ptr(Bq), _ptr(sB),
                                                float(gB), M, N, K, _ptr(C), _ptr(S), r0 + a,
                                                r0 + b),
         _split(r1 - r0, nt * 4), nt)
    return C, S


def _gemm_args(Aq, sA, Bq, sB):
    Aq = np.ascontiguousarray(Aq, dtype=np.uint8)
    Bq = np.ascontiguousarray(Bq, dtype=np.uint8)
    sA = np.ascontiguousarray(sA, dtype=np.float32)
    sB = np.ascontiguousarray(sB, dtype=np.float32)
    M, K = Aq.shape
    K2, N = Bq.shape
    if K2 != K or sA.shape != (M, K // 128) or sB.shape != (K // 128, N // 128):
        raise ValueError("inconsistent GEMM operand shapes")
    return Aq, sA, Bq, sB, M, N, K


def gemm_f64(Aq, sA, Bq, sB, nthreads: int | None = None):
    """fp64 dequantize-then-matmul: returns (C [M,N], S [M,N] = sum_k |a b|)."""
    lib = _load()
    Aq, sA, Bq, sB, M, N, K = _gemm_args(Aq, sA, Bq, sB)
    C = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64)
    nt = nthreads or threads()
    _run(lambda a, b: lib.oracle_gemm_f64(_ptr(Aq), _ptr(sA), _ptr(Bq), _ptr(sB), M, N, K,
                                          _ptr(C), _ptr(S), a, b),
         _split(M, nt * 2), nt)
    return C, S


def gemm_f64_at(Aq, sA, Bq, sB, rows, cols, nthreads: int | None = None):
    """The same reference at the listed output elements only: returns (C[i], S[i])."""
    lib = _load()
    Aq, sA, Bq, sB, M, N, K = _gemm_args(Aq, sA, Bq, sB)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in shape")
    C = np.empty(rows.shape, dtype=np.float64)
    S = np.empty(rows.shape, dtype=np.float64)
    nt = nthreads or threads()

    def part(a, b):
        return lib.oracle_gemm_f64_at(_ptr(Aq), _ptr(sA), _ptr(Bq), _ptr(sB), M, N, K,
                                      _ptr(rows) + 8 * a, _ptr(cols) + 8 * a, b - a,
                                      _ptr(C) + 8 * a, _ptr(S) + 8 * a)

    _run(part, _split(rows.size, nt * 4), nt)
    return C, S
