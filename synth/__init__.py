"""Seeded synthetic bf16 inputs (Philox4x32-10 + Box-Muller), shared by the HIP library's
tests/benchmark and the CPU oracle.

Input generation only -- no quantization, scaling or matrix arithmetic lives here.  The
arithmetic is in ``synth_gen.c``; this module builds/loads it and splits rows across host
threads (the output of every element depends only on (seed, stream, index)).

Workloads (all seed 0, bf16 row-major):
  tiny     A [128,512]  N(0,1), 0.1% outliers x100;  B [512,256] N(0,0.02)
  actq     X [16384,7168] N(0,1), 0.01% outliers x200
  sq4096   A [4096,4096] N(0,1);  B [4096,4096] N(0,0.02)
  skinny   A [128,2048] N(0,1) x per-row 10^U(-2,2);  B [2048,7168] N(0,0.02)
  prefill  A [4096,16384] N(0,1), 0.1% outliers x100;  B [16384,7168] N(0,0.02)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth_gen.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None

STREAM_A, STREAM_B, STREAM_OUTLIER, STREAM_ROWMAG = 0, 1, 2, 3


def build() -> str:
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=gnu99", "-fPIC", "-shared", "-ffp-contract=off",
                           "-fno-fast-math", _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    u64, u32, i64, d, p = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_double,
                           ctypes.c_void_p)
    lib.synth_matrix_bf16.restype = i64
    lib.synth_matrix_bf16.argtypes = [p, i64, i64, u64, u32, d, d, d, u32, ctypes.c_int, d, d,
                                      i64, i64]
    lib.synth_uniform_at.restype = d
    lib.synth_uniform_at.argtypes = [u64, u32, u64]
    lib.synth_philox_block.restype = None
    lib.synth_philox_block.argtypes = [u64, u32, u64, p]
    lib.synth_f64_to_bf16.restype = ctypes.c_uint16
    lib.synth_f64_to_bf16.argtypes = [d]
    _lib = lib
    return lib


def philox4x32_10(seed: int, stream: int, index: int) -> tuple:
    """The four 32-bit words for (key=(seed, stream), counter=(index lo, index hi, 0, 0))."""
    out = (ctypes.c_uint32 * 4)()
    _load().synth_philox_block(seed, stream, index, ctypes.addressof(out))
    return tuple(out)


def f64_to_bf16(v: float) -> int:
    return int(_load().synth_f64_to_bf16(float(v)))


@dataclass(frozen=True)
class MatrixSpec:
    rows: int
    cols: int
    stream: int
    sigma: float
    outlier_p: float = 0.0
    outlier_factor: float = 1.0
    row_log_range: tuple | None = None  # (lo, hi): rows scaled by 10^U(lo, hi)


def matrix(spec: MatrixSpec, seed: int = 0, nthreads: int | None = None):
    """Generate a bf16 matrix (returned as uint16 bits) and the number of outliers placed."""
    lib = _load()
    out = np.empty((spec.rows, spec.cols), dtype=np.uint16)
    nt = nthreads or max(1, min(16, os.cpu_count() or 1))
    rows = spec.rows
    parts = max(1, min(rows, nt * 4))
    step = (rows + parts - 1) // parts
    lo_hi = spec.row_log_range or (0.0, 0.0)
    use_rows = 1 if spec.row_log_range else 0

    def part(r0):
        r1 = min(rows, r0 + step)
        return lib.synth_matrix_bf16(out.ctypes.data, spec.rows, spec.cols, seed, spec.stream,
                                     spec.sigma, spec.outlier_p, spec.outlier_factor,
                                     STREAM_OUTLIER, use_rows, lo_hi[0], lo_hi[1], r0, r1)

    with ThreadPoolExecutor(max_workers=nt) as ex:
        counts = list(ex.map(part, range(0, rows, step)))
    if any(c < 0 for c in counts):
        raise ValueError("bad generator arguments")
    return out, int(sum(counts))


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    a: MatrixSpec | None
    b: MatrixSpec | None
    out_dtype: str  # "f32" | "bf16" | "" (quantize only)
    description: str


def _a(M, K, **kw):
    return MatrixSpec(M, K, STREAM_A, 1.0, **kw)


def _b(K, N):
    return MatrixSpec(K, N, STREAM_B, 0.02)


WORKLOADS = {
    "tiny": Workload("tiny", 128, 256, 512, _a(128, 512, outlier_p=1e-3, outlier_factor=100.0),
                     _b(512, 256), "f32",
                     "GEMM 128x256x512: A N(0,1) with 0.1% outliers x100 (1x128), "
                     "B N(0,0.02) (128x128), fp32 C"),
    "actq": Workload("actq", 16384, 0, 7168,
                     _a(16384, 7168, outlier_p=1e-4, outlier_factor=200.0), None, "",
                     "activation quantize X [16384,7168] N(0,1) with 0.01% outliers x200"),
    "sq4096": Workload("sq4096", 4096, 4096, 4096, _a(4096, 4096), _b(4096, 4096), "bf16",
                       "GEMM 4096^3: A N(0,1) (1x128), B N(0,0.02) (128x128), bf16 C"),
    "skinny": Workload("skinny", 128, 7168, 2048, _a(128, 2048, row_log_range=(-2.0, 2.0)),
                       _b(2048, 7168), "f32",
                       "GEMM 128x7168x2048: A N(0,1) x per-row 10^U(-2,2), B N(0,0.02), fp32 C"),
    "prefill": Workload("prefill", 4096, 7168, 16384,
                        _a(4096, 16384, outlier_p=1e-3, outlier_factor=100.0),
                        _b(16384, 7168), "bf16",
                        "GEMM 4096x7168x16384: A N(0,1) with 0.1% outliers x100, "
                        "B N(0,0.02), bf16 C"),
}


def workload_inputs(name: str, seed: int = 0):
    """(A bits or None, B bits or None, outlier count) for a named workload."""
    w = WORKLOADS[name]
    A, nA = matrix(w.a, seed) if w.a else (None, 0)
    B, _ = matrix(w.b, seed) if w.b else (None, 0)
    return A, B, nA
