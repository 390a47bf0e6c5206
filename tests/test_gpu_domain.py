"""Every (x, amax) pair through the device quantizer.

Under 1x128 quantization a code depends only on the element x and its tile's amax, both
bf16 with |x| <= amax.  This test runs ALL such pairs (every positive finite bf16 amax,
every x of either sign, ~1.07e9 elements) through fgq_quantize_act_1x128 and compares
every code and scale with the oracle, so the device arithmetic (reciprocal with one
quotient correction, hardware E4M3 convert) is proven identical to fl32(x/s) + RNE E4M3
on the whole input domain (NaN/Inf inputs are outside the contract)."""
import numpy as np
import pytest

import oracle
from tests.domain import all_amax_bits, domain_tiles
from tests.gpu_util import bits_equal, free, gpu_quant_act, log

pytestmark = pytest.mark.gpu


def test_all_x_amax_pairs():
    amax = all_amax_bits()
    chunks = np.array_split(amax, 24)
    total = 0
    for ci, ch in enumerate(chunks):
        X, _, _ = domain_tiles(ch)
        X = X.reshape(-1, 128 * 64) if X.shape[0] % 64 == 0 else X.reshape(-1, 128)
        q, s = gpu_quant_act(X, sentinel=False)
        rq, rs = oracle.quantize_act(X)
        total += X.size
        assert bits_equal(s, rs), (ci, int(np.sum(s.view(np.uint32) != rs.view(np.uint32))))
        bad = q != rq
        assert not bad.any(), (ci, int(bad.sum()), X.reshape(-1)[np.argmax(bad.reshape(-1))])
        log(f"domain chunk {ci}: amax {ch[0]:#06x}..{ch[-1]:#06x} ok ({X.size} elements)")
        del X, q, s, rq, rs
    free()
    assert total > 1.0e9
