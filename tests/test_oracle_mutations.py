"""The pins are strong enough: each plausible mistake planted in a copy of the oracle's C
source (a wrong tie rule, scale constant, exponent bias, index, dropped term, reciprocal for
a divide) makes at least one pin fail, while the unmodified copy built the same way passes.
Each mutant is built with gcc into a temporary directory and the oracle pin tests run
against it in a subprocess (the oracle package loads the build named by FGQ_ORACLE_LIB).
CPU only; the mutations live in these copies, never in oracle/."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "fgq_oracle.c")
# fastest pins first; -x stops at the first failure.  The long domain sweep and the
# NVFP4 coder's division check (which does not use the oracle) are left out here.
PINS = ["tests/test_oracle_gemm.py", "tests/test_oracle_e4m3.py", "tests/test_oracle_quant.py",
        "tests/test_oracle_ue8m0.py", "tests/test_oracle_nvfp4.py"]
SKIP = ["tests/test_oracle_quant.py::test_domain_sweep_properties",
        "tests/test_oracle_nvfp4.py::test_coder_division_is_correctly_rounded"]

# name -> (text in fgq_oracle.c, replacement[, which occurrence, 0-based; default the first])
MUTANTS = {
    "E4M3 ties to the odd code": (
        "pick = (lo % 2 == 0) ? lo : lo + 1;", "pick = (lo % 2 == 1) ? lo : lo + 1;"),
    "E4M3 exponent bias 8": (
        "mag = ldexp(1.0 + (double)m / 8.0, e - 7);", "mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "E4M3 subnormal step 2^-10": (
        "mag = ldexp((double)m / 8.0, -6);", "mag = ldexp((double)m / 8.0, -7);"),
    "scale amax/240 (E4M3 FNUZ maximum)": (
        "float s = amax / 448.0f;", "float s = amax / 240.0f;"),
    "x * (1/s) for x / s": (
        "q[idx[i]] = oracle_e4m3_encode(v / s);", "q[idx[i]] = oracle_e4m3_encode(v * (1.0f / s));"),
    "amax misses the last element of a group": (
        "for (int64_t i = 0; i < n; ++i) {\n        float v = fabsf(",
        "for (int64_t i = 0; i + 1 < n; ++i) {\n        float v = fabsf("),
    "GEMM takes scale_A of the next K block": (
        "double a = dec[Aq[m * K + k]] * (double)sA[m * KB + k / 128];",
        "double a = dec[Aq[m * K + k]] * (double)sA[m * KB + (k / 128 + 1) % KB];"),
    "GEMM takes scale_B of column block 0": (
        "double p = a * (dec[brow[n]] * (double)sbrow[n / 128]);",
        "double p = a * (dec[brow[n]] * (double)sbrow[0]);"),
    "GEMM drops the last K block": (
        "for (int64_t k = 0; k < K; ++k) {\n            double a",
        "for (int64_t k = 0; k < K - (K > 128 ? 128 : 0); ++k) {\n            double a"),
    "UE8M0 exponent one too high": (
        "while (e < 254 && 448.0 * ldexp(1.0, e - 127) < amax)",
        "while (e < 254 && 448.0 * ldexp(1.0, e - 127) <= amax)"),
    "E2M1 ties to the odd code": (
        "best = (c % 2 == 0) ? c : c + 1;", "best = (c % 2 == 1) ? c : c + 1;"),
    "NVFP4 global scale amax/2560": (
        "float gs = amax_t / 2688.0f;", "float gs = amax_t / 2560.0f;"),
    "UE8M0 amax misses the last element of a group": (
        "for (int64_t i = 0; i < n; ++i) {\n        float v = fabsf(",
        "for (int64_t i = 0; i + 1 < n; ++i) {\n        float v = fabsf(", 1),
    "NVFP4 block amax misses the last element": (
        "for (int j = 0; j < 16; ++j) {\n                float v = fabsf(",
        "for (int j = 0; j < 15; ++j) {\n                float v = fabsf("),
    "NVFP4 tensor amax misses the last element": (
        "for (int64_t i = 0; i < R * C; ++i) {", "for (int64_t i = 0; i + 1 < R * C; ++i) {"),
    "GEMM tolerance sum of signed products": (
        "srow[n] += fabs(p);", "srow[n] += p;"),
    "UE8M0 decode bias 126": (
        "return ldexp(1.0, (int)e - 127);", "return ldexp(1.0, (int)e - 126);"),
    "NVFP4 GEMM nibble order swapped for B": (
        "uint8_t code = (k % 2 == 0) ? (byte & 15) : (byte >> 4);\n                double b",
        "uint8_t code = (k % 2 == 1) ? (byte & 15) : (byte >> 4);\n                double b"),
    "NVFP4 GEMM block scale of A one block late": (
        "oracle_e4m3_decode(sA[m * KB + k / 16])",
        "oracle_e4m3_decode(sA[m * KB + (k / 16 + 1) % KB])"),
}


def mutate(source, old, new, which=0):
    at = -1
    for _ in range(which + 1):
        at = source.find(old, at + 1)
        assert at >= 0, f"mutation site not found: {old!r} (occurrence {which})"
    return source[:at] + new + source[at + len(old):]


def build(tmp, name, text):
    c = os.path.join(tmp, name + ".c")
    lib = os.path.join(tmp, name + ".so")
    with open(c, "w") as f:
        f.write(text)
    subprocess.run(["gcc", *oracle.CFLAGS, c, "-o", lib, "-lm"], check=True,
                   capture_output=True, timeout=120)
    return lib


def run_pins(lib):
    env = dict(os.environ, FGQ_ORACLE_LIB=lib)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS]
    for s in SKIP:
        cmd += ["--deselect", s]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def source():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    with open(SRC) as f:
        return f.read()


def test_every_mutant_fails_a_pin(source, tmp_path):
    names = sorted(MUTANTS)
    libs = {"control": build(str(tmp_path), "control", source)}
    for i, name in enumerate(names):
        libs[name] = build(str(tmp_path), f"m{i}", mutate(source, *MUTANTS[name]))
    with ThreadPoolExecutor(max_workers=4) as pool:
        results = dict(zip(libs, pool.map(run_pins, libs.values())))
    rc, out = results.pop("control")
    assert rc == 0, "the unmodified copy must pass its pins:\n" + out
    survivors = [n for n, (rc, out) in results.items() if rc == 0 or "failed" not in out]
    assert not survivors, f"mutants no pin catches: {survivors}"
