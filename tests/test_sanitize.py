"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no GPU).

* The oracle (oracle/fgq_oracle.c): every entry point on small seeded inputs spanning the
  bf16 exponent range, all-zero groups, and refused shapes
  (tests/helpers/oracle_sanitize_main.c).
* The C ABI layers (fine_grained_block_fgq_amd/csrc/api.cpp and calib_api.cpp, the
  measurement library's) linked against stub launchers:
  every entry point with valid arguments reaches its launcher once and maps the launcher's
  status (success, launch failure, a grid too large for one dispatch); invalid or empty
  arguments never reach a launcher (tests/helpers/abi_stub_main.cpp).

Both are built with gcc/g++ here (host code only) and must print "ok" with no sanitizer
report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HELPERS = os.path.join(ROOT, "tests", "helpers")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _build_and_run(cmd, exe, tmp_path):
    if shutil.which(cmd[0]) is None:
        pytest.skip(f"{cmd[0]} not available")
    out = str(tmp_path / exe)
    subprocess.run(cmd + ["-o", out], check=True, capture_output=True, text=True, timeout=300)
    run = subprocess.run([out], capture_output=True, text=True, timeout=300, env=ENV)
    report = run.stdout + run.stderr
    assert run.returncode == 0, report
    assert "runtime error" not in report and "AddressSanitizer" not in report, report
    return run.stdout


def test_oracle_under_sanitizers(tmp_path):
    out = _build_and_run(["gcc", "-std=gnu99", "-ffp-contract=off", "-fno-fast-math", *SAN,
                          os.path.join(ROOT, "oracle", "fgq_oracle.c"),
                          os.path.join(HELPERS, "oracle_sanitize_main.c"), "-lm"],
                         "oracle_san", tmp_path)
    assert out.startswith("ok")


def test_abi_layer_with_stub_launchers_under_sanitizers(tmp_path):
    hip_include = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")
    if not os.path.isdir(os.path.join(hip_include, "hip")):
        pytest.skip("HIP headers not available")
    out = _build_and_run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", hip_include,
                          "-I", os.path.join(ROOT, "fine_grained_block_fgq_amd", "csrc"), *SAN,
                          os.path.join(ROOT, "fine_grained_block_fgq_amd", "csrc", "api.cpp"),
                          os.path.join(ROOT, "fine_grained_block_fgq_amd", "csrc",
                                       "calib_api.cpp"),
                          os.path.join(HELPERS, "abi_stub_main.cpp")],
                         "abi_san", tmp_path)
    assert out.strip() == "ok"
