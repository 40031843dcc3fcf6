"""Q8_0 GEMV (q4k_gemv_q8_0) against the CPU oracle, through the C ABI."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import assert_gemv, bits, down, note, require_gpu, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q4k():
    require_gpu()
    import bit_block_quantized_gguf_amd as q4k
    return q4k


@pytest.mark.parametrize("M,K", [(1, 256), (63, 256), (65, 512), (300, 768), (1000, 2560),
                                 (129, 5120), (64, 17408)])
def test_q8_0_gemv_matches_oracle(q4k, M, K):
    w = synth.q8_0_weight(synth.key(7, M + K), M, K)
    x = synth.normal(synth.key(7, 3 * M + K), K)
    note("q8_0 gemv %dx%d" % (M, K))
    y = down(q4k.gemv_q8_0(up(w), up(x), M=M, K=K))
    yr, S = oracle.gemv_q8_0(w, x, M, K)
    assert_gemv(y, yr, S, "q8_0 %dx%d" % (M, K))


def test_q8_0_gemv_lm_head_sampled(q4k):
    """The lm_head shape (vocab 248320 x hidden 5120, 1.35 GB in Q8_0) on
    sampled rows, tile edges and the last rows included."""
    M, K = 248320, 5120
    w = synth.q8_0_weight(synth.key(7, 1), M, K)
    x = synth.normal(synth.key(7, 2), K)
    note("q8_0 gemv lm_head")
    y = down(q4k.gemv_q8_0(up(w), up(x), M=M, K=K))
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([rng.integers(0, M, 400), [0, 63, 64, M - 65, M - 64, M - 1]]))
    yr, S = oracle.gemv_q8_0(w, x, M, K, rows=rows)
    assert_gemv(y[rows], yr, S, "q8_0 lm_head")


def test_q8_0_gemv_zero_and_one_hot(q4k):
    M, K = 200, 1024
    w = synth.q8_0_weight(synth.key(7, 5), M, K)
    wd = up(w)
    assert np.all(down(q4k.gemv_q8_0(wd, up(np.zeros(K, np.float32)), M=M, K=K)) == 0.0)
    deq = oracle.dequant_q8_0(w, M, K)
    for k in (0, 1, 31, 32, 33, 255, 511, 512, 1023):
        x = np.zeros(K, np.float32)
        x[k] = 1.0
        y = down(q4k.gemv_q8_0(wd, up(x), M=M, K=K))
        # every other product is an exact zero and the +128 offset cancels exactly
        assert np.array_equal(y, deq[:, k]), k


def test_q8_0_gemv_deterministic_and_split_variants(q4k):
    M, K = 5120, 17408
    w = synth.q8_0_weight(synth.key(7, 9), M, K)
    x = synth.normal(synth.key(7, 10), K)
    wd, xd = up(w), up(x)
    yr, S = oracle.gemv_q8_0(w, x, M, K)
    try:
        for groups in (0, 1, 7, 80, 333, 1024, 2720):
            q4k.tune_gemv(0, groups)
            note("q8_0 groups=%d" % groups)
            y = down(q4k.gemv_q8_0(wd, xd, M=M, K=K))
            assert_gemv(y, yr, S, "q8_0 groups=%d" % groups)
            assert np.array_equal(bits(y), bits(down(q4k.gemv_q8_0(wd, xd, M=M, K=K)))), groups
    finally:
        q4k.tune_gemv(0, 0)
