"""Checks of the seeded input generator (not part of the method)."""
import numpy as np

import synth


def test_philox_known_answer():
    # Philox4x32-10 known-answer vector (Random123 distribution): counter 0, key 0
    assert synth.philox4x32_10(0, 0, 0) == (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)


def test_bf16_rounding_nearest_even():
    assert synth.f64_to_bf16(1.0) == 0x3F80
    assert synth.f64_to_bf16(1.0 + 2 ** -8) == 0x3F80          # tie -> even
    assert synth.f64_to_bf16(1.0 + 3 * 2 ** -8) == 0x3F82      # tie -> even (up)
    assert synth.f64_to_bf16(1.0 + 2 ** -8 + 2 ** -30) == 0x3F81
    assert synth.f64_to_bf16(-2.0) == 0xC000
    assert synth.f64_to_bf16(2.0 ** -133) == 0x0001            # bf16 min subnormal


def test_workload_statistics_and_determinism():
    A, B, n = synth.workload_inputs("tiny")
    A2, B2, n2 = synth.workload_inputs("tiny")
    assert np.array_equal(A, A2) and np.array_equal(B, B2) and n == n2
    a = (A.astype(np.uint32) << 16).view(np.float32)
    b = (B.astype(np.uint32) << 16).view(np.float32)
    assert A.shape == (128, 512) and B.shape == (512, 256)
    assert 30 <= n <= 110                      # 0.1% of 65536 = 65.5 expected
    big = int(np.sum(np.abs(a) > 20))         # an outlier is z*100: |z| < 0.2 stays small
    assert n // 2 <= big <= n
    assert abs(b.std() - 0.02) < 0.001 and abs(b.mean()) < 0.001
    # per-row magnitudes span 1e-2..1e2 for the skinny workload
    spec = synth.WORKLOADS["skinny"].a
    X, _ = synth.matrix(spec)
    rs = (X.astype(np.uint32) << 16).view(np.float32).std(axis=1)
    assert rs.min() < 0.05 and rs.max() > 20
