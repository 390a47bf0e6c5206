"""The C ABI library loads and exports every entry point include/fgq.h declares; host-side
argument validation rejects bad calls before any launch (no GPU needed: every call here
fails validation, so nothing reaches the device)."""
import ctypes
import os
import re

import pytest

import fine_grained_block_fgq_amd as fgq
from fine_grained_block_fgq_amd import calib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fgq.h")
CALIB_HEADER = os.path.join(ROOT, "include", "fgq_calib.h")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fgq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_declared_symbols():
    lib = fgq.load()
    names = declared_functions()
    assert {"fgq_quantize_act_1x128", "fgq_quantize_weight_128x128",
            "fgq_gemm_fp8_blockscaled"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.fgq_version() >= 100


def test_measurement_library_is_separate():
    """The measurement-only kernels live in libfgq_calib (include/fgq_calib.h), not in the
    method's library"""
    lib = calib.load()
    names = declared_functions(CALIB_HEADER)
    assert set(names) == {"fgq_calib_stream", "fgq_calib_mfma_f16", "fgq_calib_mfma_fp8",
                          "fgq_probe_fp8_mfma_partials"}
    for n in names:
        assert hasattr(lib, n), n
    main = set(declared_functions())
    assert not (main & set(names))
    for n in names:
        assert not hasattr(fgq.load(), n), n


def test_status_strings():
    lib = fgq.load()
    for s in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        assert lib.fgq_status_string(s)
    assert lib.fgq_status_string(-99) == b"unknown status"


P = 0x10000  # aligned fake addresses: validation fails before they could be used
Q = 0x20000
R = 0x30000
T = 0x1000000


@pytest.mark.parametrize("args,want", [
    ((P, Q, R, 4, 100), -2),          # K % 128
    ((P, Q, R, -1, 128), -2),         # negative M
    ((P, Q, R, 1 << 31, 128), -2),    # too large
    ((None, Q, R, 4, 128), -1),       # null
    ((P + 2, Q, R, 4, 128), -3),      # misaligned
    ((P, P + 64, R, 4, 128), -6),     # codes overlap X
    ((P, Q, P + 256, 4, 128), -6),    # scales overlap X
    ((None, None, None, 0, 128), 0),  # empty: no-op
    ((None, None, None, 4, 0), 0),
])
def test_act_validation(args, want):
    assert fgq.load().fgq_quantize_act_1x128(*args, None) == want


@pytest.mark.parametrize("args,want", [
    ((P, Q, R, 128, 100), -2),
    ((P, Q, R, 100, 128), -2),
    ((P, Q, R, 128 * 65536, 128), -2),
    ((P, None, R, 128, 128), -1),
    ((P, Q, R + 4, 128, 128), -3),
    ((P, P + 16, R, 128, 128), -6),
    ((None, None, None, 0, 128), 0),
])
def test_weight_validation(args, want):
    assert fgq.load().fgq_quantize_weight_128x128(*args, None) == want


S1, S2 = 0x40000, 0x50000


@pytest.mark.parametrize("args,want", [
    ((P, S1, Q, S2, R, 4, 128, 128, 2), -4),      # dtype
    ((P, S1, Q, S2, R, 4, 100, 128, 0), -2),      # N % 128
    ((P, S1, Q, S2, R, 4, 128, 100, 0), -2),      # K % 128
    ((P, S1, Q, S2, R, -4, 128, 128, 0), -2),
    ((P, None, Q, S2, R, 4, 128, 128, 0), -1),
    ((P, S1, Q, S2, None, 4, 128, 128, 0), -1),
    ((P, S1, Q + 8, S2, R, 4, 128, 128, 0), -3),
    ((P, S1, Q, S2, P, 4, 128, 128, 0), -6),      # C overlaps A_q
    ((P, S1, Q, S2, S2 - 16, 4, 128, 128, 1), -6),  # C overlaps scale_B
    ((None, None, None, None, None, 0, 128, 128, 0), 0),
    ((None, None, None, None, None, 4, 0, 128, 0), 0),
])
def test_gemm_validation(args, want):
    assert fgq.load().fgq_gemm_fp8_blockscaled(*args, None) == want


@pytest.mark.parametrize("args,want", [
    ((P, S1, Q, S2, R, 4, 128, 128, 0, 6), -7),     # unknown variant
    ((P, S1, Q, S2, R, 4, 128, 128, 0, -1), -7),
    ((P, S1, Q, S2, R, 4, 128, 128, 2, 3), -4),     # dtype checked first
    ((P, S1, Q, S2, R, 4, 100, 128, 0, 3), -2),
    ((P, S1, Q + 8, S2, R, 4, 128, 128, 0, 1), -3),
    ((P, S1, Q, S2, P, 4, 128, 128, 0, 2), -6),
    ((None, None, None, None, None, 0, 128, 128, 0, 3), 0),
])
def test_gemm_variant_validation(args, want):
    assert fgq.load().fgq_gemm_fp8_blockscaled_variant(*args, None) == want


T1 = 0x60000


@pytest.mark.parametrize("args,want", [
    ((P, S1, Q, S2, R, T1, 0x70000, 4, 100, 128), -2),
    ((P, S1, Q, S2, R, None, 0x70000, 4, 128, 128), -1),
    ((P, S1, Q, S2, R, T1 + 8, 0x70000, 4, 128, 128), -3),
    ((P, S1, Q, S2, R, R + 64, 0x70000, 4, 128, 128), -6),   # codes overlap C
    ((P, S1, Q, S2, R, T1, P + 16, 4, 128, 128), -6),        # scales overlap A_q
    ((None,) * 7 + (0, 128, 128), 0),
])
def test_gemm_quant_validation(args, want):
    assert fgq.load().fgq_gemm_fp8_blockscaled_quant(*args, None) == want


@pytest.mark.parametrize("fn,args,want", [
    ("fgq_quantize_act_1x128_ue8m0", (P, Q, R, 4, 100), -2),
    ("fgq_quantize_act_1x128_ue8m0", (P, Q, R + 1, 4, 128), -3),
    ("fgq_quantize_act_1x128_ue8m0", (P, Q, P + 32, 4, 128), -6),
    ("fgq_quantize_act_1x128_ue8m0", (None, None, None, 0, 128), 0),
    ("fgq_quantize_weight_128x128_ue8m0", (P, Q, R, 100, 128), -2),
    ("fgq_quantize_weight_128x128_ue8m0", (P, None, R, 128, 128), -1),
    ("fgq_quantize_weight_128x128_ue8m0", (None, None, None, 0, 128), 0),
    ("fgq_gemm_fp8_blockscaled_ue8m0", (P, S1, Q, S2, R, 4, 128, 128, 0, 9), -7),
    ("fgq_gemm_fp8_blockscaled_ue8m0", (P, S1, Q, S2, R, 4, 128, 128, 5, 0), -4),
    ("fgq_gemm_fp8_blockscaled_ue8m0", (P, S1, Q, S2, R, 4, 128, 100, 0, 0), -2),
    ("fgq_gemm_fp8_blockscaled_ue8m0", (P, S1, Q, S2, S1 - 16, 4, 128, 128, 0, 0), -6),
    ("fgq_gemm_fp8_blockscaled_ue8m0", (None,) * 5 + (0, 128, 128, 0, 0), 0),
])
def test_ue8m0_validation(fn, args, want):
    assert getattr(fgq.load(), fn)(*args, None) == want


G1, G2 = 0x80000, 0x90000


@pytest.mark.parametrize("fn,args,want", [
    ("fgq_quantize_nvfp4", (P, Q, R, G1, 4, 24), -2),          # C % 16
    ("fgq_quantize_nvfp4", (P, Q, R, None, 4, 32), -1),
    ("fgq_quantize_nvfp4", (P, Q, R, G1 + 4, 4, 32), -3),
    ("fgq_quantize_nvfp4", (P, Q, R, P + 16, 4, 32), -6),      # global scale inside X
    ("fgq_quantize_nvfp4", (None, None, None, None, 0, 32), 0),
    ("fgq_gemm_nvfp4", (P, S1, G1, Q, S2, G2, R, 4, 128, 100, 0), -2),   # K % 128
    ("fgq_gemm_nvfp4", (P, S1, G1, Q, S2, G2, R, 4, 128, 128, 3), -4),
    ("fgq_gemm_nvfp4", (P, S1, None, Q, S2, G2, R, 4, 128, 128, 0), -1),
    ("fgq_gemm_nvfp4", (P, S1, G1, Q, S2, G2, G1 - 16, 4, 128, 128, 0), -6),
    ("fgq_gemm_nvfp4", (None,) * 7 + (0, 128, 128, 0), 0),
])
def test_nvfp4_validation(fn, args, want):
    assert getattr(fgq.load(), fn)(*args, None) == want


@pytest.mark.parametrize("fn,args,want", [
    ("fgq_calib_stream", (P, Q, -1), -2),
    ("fgq_calib_stream", (None, Q, 4), -1),
    ("fgq_calib_stream", (P + 8, Q, 4), -3),
    ("fgq_calib_stream", (P, P + 32, 4), -6),      # dst inside src
    ("fgq_calib_stream", (None, None, 0), 0),     # empty: no-op
    ("fgq_calib_mfma_f16", (P, 0, 10), -2),
    ("fgq_calib_mfma_f16", (P, 4, -1), -2),
    ("fgq_calib_mfma_f16", (None, 4, 10), -1),
    ("fgq_calib_mfma_f16", (P + 4, 4, 10), -3),
    ("fgq_calib_mfma_fp8", (P, 0, 10), -2),
    ("fgq_calib_mfma_fp8", (None, 4, 10), -1),
    ("fgq_calib_mfma_fp8", (P + 4, 4, 10), -3),
    ("fgq_probe_fp8_mfma_partials", (P, Q, R, 8, 16, 128), -2),      # M % 16
    ("fgq_probe_fp8_mfma_partials", (P, Q, R, 16, 16, 64), -2),      # K % 128
    ("fgq_probe_fp8_mfma_partials", (P, Q, R, 16, 16, 1 << 17), -2),  # too large
    ("fgq_probe_fp8_mfma_partials", (P, None, R, 16, 16, 128), -1),
    ("fgq_probe_fp8_mfma_partials", (P + 8, Q, R, 16, 16, 128), -3),
    ("fgq_probe_fp8_mfma_partials", (P, Q, P + 64, 16, 16, 128), -6),  # P inside A_q
    ("fgq_probe_fp8_mfma_partials", (None, None, None, 0, 16, 128), 0),
])
def test_calib_validation(fn, args, want):
    assert getattr(calib.load(), fn)(*args, None) == want


def test_workspace_size_validation():
    lib = fgq.load()
    assert lib.fgq_gemm_workspace_size(4, 100, 128) == -2      # N % 128
    assert lib.fgq_gemm_workspace_size(4, 128, 100) == -2      # K % 128
    assert lib.fgq_gemm_workspace_size(-1, 128, 128) == -2
    assert lib.fgq_gemm_workspace_size(0, 128, 128) == 0       # empty: nothing to split
    assert lib.fgq_gemm_workspace_size(4, 128, 0) == 0


@pytest.mark.parametrize("args,want", [
    ((P, S1, Q, S2, R, 4, 128, 256, 0, 0, T, 1 << 20), -2),    # splits < 1
    ((P, S1, Q, S2, R, 4, 128, 256, 0, 3, T, 1 << 20), -2),    # splits > K/128
    ((1 << 30, 2 << 30, 3 << 30, 4 << 30, 5 << 30, 4, 128, 4096, 0, 17, 6 << 30, 1 << 20),
     -2),                                                      # splits > 16
    ((P, S1, Q, S2, R, 4, 128, 256, 0, 2, T, 4095), -8),       # workspace < 2*4*128*4
    ((P, S1, Q, S2, R, 4, 128, 256, 0, 2, None, 0), -8),
    ((P, S1, Q, S2, R, 4, 128, 256, 0, 2, T + 8, 1 << 20), -3),
    ((P, S1, Q, S2, R, 4, 128, 256, 0, 2, R, 1 << 20), -6),    # workspace overlaps C
    ((P, S1, Q, S2, R, 4, 128, 256, 0, 2, T, -1), -2),
])
def test_splitk_validation(args, want):
    assert fgq.load().fgq_gemm_fp8_blockscaled_splitk(*args, None) == want


def test_ws_validation():
    lib = fgq.load()
    # dtype and shape errors as the plain GEMM; a negative workspace size is a shape error
    assert lib.fgq_gemm_fp8_blockscaled_ws(P, S1, Q, S2, R, 4, 128, 256, 2, T, 1 << 20,
                                           None) == -4
    assert lib.fgq_gemm_fp8_blockscaled_ws(P, S1, Q, S2, R, 4, 100, 256, 0, T, 1 << 20,
                                           None) == -2
    assert lib.fgq_gemm_fp8_blockscaled_ws(P, S1, Q, S2, R, 4, 128, 256, 0, T, -5, None) == -2
    assert lib.fgq_gemm_fp8_blockscaled_ws(None, None, None, None, None, 0, 128, 256, 0, None,
                                           0, None) == 0


# Shapes that pass the argument checks but whose grid would exceed the 2^32 work-items one
# HIP dispatch can count: refused as shape errors before any launch (the fake addresses are
# far enough apart that no range overlaps).
T40, T41, T42 = 1 << 40, 1 << 41, 1 << 42


def test_grid_limit_is_a_shape_error():
    lib = fgq.load()
    # activation quantizer: 2^20 x 2^17 elements -> 2^33 work-items
    assert lib.fgq_quantize_act_1x128(P, T40, T41, 1 << 20, 1 << 17, None) == -2
    # skinny GEMM: 2^23 tiles of 768 threads
    assert lib.fgq_gemm_fp8_blockscaled_variant(P, 0x40000, T40, 0x100000, T42, 128, 1 << 28,
                                                128, 0, 4, None) == -2


# The binding has no CPU path: every entry point refuses host tensors before calling the
# library (which would otherwise dereference host pointers as device addresses).
def _host(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


def test_binding_refuses_host_tensors():
    import torch
    bf, u8, f32 = torch.bfloat16, torch.uint8, torch.float32
    calls = [
        lambda: fgq.fgq_quantize_act_1x128(_host((4, 128), bf)),
        lambda: fgq.fgq_quantize_weight_128x128(_host((128, 128), bf)),
        lambda: fgq.fgq_quantize_act_1x128_ue8m0(_host((4, 128), bf)),
        lambda: fgq.fgq_quantize_weight_128x128_ue8m0(_host((128, 128), bf)),
        lambda: fgq.fgq_quantize_nvfp4(_host((4, 32), bf)),
        lambda: fgq.fgq_gemm_fp8_blockscaled(_host((4, 128), u8), _host((4, 1), f32),
                                             _host((128, 128), u8), _host((1, 1), f32)),
        lambda: fgq.fgq_gemm_fp8_blockscaled_variant(_host((4, 128), u8), _host((4, 1), f32),
                                                     _host((128, 128), u8), _host((1, 1), f32),
                                                     variant=3),
        lambda: fgq.fgq_gemm_fp8_blockscaled_quant(_host((4, 128), u8), _host((4, 1), f32),
                                                   _host((128, 128), u8), _host((1, 1), f32)),
        lambda: fgq.fgq_gemm_fp8_blockscaled_ue8m0(_host((4, 128), u8), _host((4, 1), u8),
                                                   _host((128, 128), u8), _host((1, 1), u8)),
        lambda: fgq.fgq_gemm_nvfp4(_host((4, 64), u8), _host((4, 8), u8), _host((1,), f32),
                                   _host((128, 64), u8), _host((128, 8), u8), _host((1,), f32)),
        lambda: calib.fgq_probe_fp8_mfma_partials(_host((16, 128), u8), _host((128, 16), u8)),
    ]
    for i, call in enumerate(calls):
        with pytest.raises(TypeError, match="CUDA"):
            call()
