"""The measurement-only ceiling kernels (libfgq_calib's fgq_calib_stream / fgq_calib_mfma_f16) do
what bench.py assumes: the stream touches every input byte and writes the word XORs, and the
MFMA kernel runs to completion with a repeatable result."""
import numpy as np
import pytest
import torch

import fine_grained_block_fgq_amd as fgq
from fine_grained_block_fgq_amd import calib

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n16", [1, 511, 512, 513, 100003])
def test_calib_stream_writes_word_xors(n16):
    print(f"calib_stream n16={n16}", flush=True)
    rng = np.random.default_rng(n16)
    src_h = rng.integers(0, 2**32, size=4 * n16, dtype=np.uint32)
    src = torch.from_numpy(src_h.view(np.int32)).cuda()
    dst = torch.full((2 * n16 + 2,), -1, dtype=torch.int32, device="cuda")
    moved = calib.fgq_calib_stream(src, dst)
    torch.cuda.synchronize()
    assert moved == 24 * n16
    got = dst.cpu().numpy().view(np.uint32)
    w = src_h.reshape(n16, 4)
    want = np.stack([w[:, 0] ^ w[:, 1], w[:, 2] ^ w[:, 3]], axis=1).reshape(-1)
    assert np.array_equal(got[:2 * n16], want)
    assert np.all(got[2 * n16:] == np.uint32(0xFFFFFFFF))   # nothing written past the end


def test_calib_mfma_runs_and_repeats():
    print("calib_mfma blocks=8 iters=5", flush=True)
    out = torch.zeros((8 * 512,), dtype=torch.float32, device="cuda")
    flops = calib.fgq_calib_mfma_f16(out, 8, 5)
    torch.cuda.synchronize()
    assert flops == 8 * 8 * 5 * 16 * 16384
    first = out.clone()
    calib.fgq_calib_mfma_f16(out, 8, 5)
    torch.cuda.synchronize()
    assert torch.isfinite(first).all()
    assert torch.equal(first, out)
    assert first.abs().sum() > 0
