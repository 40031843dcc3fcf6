"""q4k_gemv_noalloc (the GEMV whose scratch is the library's fixed device
array) against q4k_gemv (caller workspace): same kernel and launch shape, so
the same bits; two calls in a row, the second on a smaller input, both also
within the GEMV bar of the oracle."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import assert_gemv, down, note, require_gpu, up

pytestmark = pytest.mark.gpu


def test_noalloc_gemv_matches_gemv_two_calls():
    require_gpu()
    import bit_block_quantized_gguf_amd as q4k
    for i, (M, K) in enumerate(((17408, 5120), (1000, 2048))):
        note("gemv_noalloc %dx%d (call %d)" % (M, K, i + 1))
        w = synth.q4k_weight(synth.key(15, i), M, K)
        x = synth.normal(synth.key(15, 100 + i), K)
        wd, xd = up(w), up(x)
        y0 = down(q4k.gemv_noalloc(wd, xd)).copy()
        y1 = down(q4k.gemv(wd, xd))
        assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32)), (M, K)
        yr, S = oracle.gemv(w, x, M, K)
        assert_gemv(y0.astype(np.float64), yr, S, "gemv_noalloc %dx%d" % (M, K))
