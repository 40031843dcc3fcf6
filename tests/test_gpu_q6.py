"""Q6_K GEMV (q4k_gemv_q6_k) against the CPU oracle, through the C ABI."""
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


@pytest.mark.parametrize("M,K", [(1, 1024), (63, 1024), (65, 2048), (300, 3072), (129, 5120),
                                 (1000, 6144), (64, 17408)])
def test_q6_k_gemv_matches_oracle(q4k, M, K):
    w = synth.q6_k_weight(synth.key(8, M + K), M, K)
    x = synth.normal(synth.key(8, 3 * M + K), K)
    note("q6_k gemv %dx%d" % (M, K))
    y = down(q4k.gemv_q6_k(up(w), up(x), M=M, K=K))
    yr, S = oracle.gemv_q6_k(w, x, M, K)
    assert_gemv(y, yr, S, "q6_k %dx%d" % (M, K))


@pytest.mark.parametrize("M,K", [(17408, 5120), (5120, 17408)])
def test_q6_k_gemv_mlp_shapes_sampled(q4k, M, K):
    """The MLP shapes (73 MB each in Q6_K) on sampled rows, tile edges and
    the last rows included."""
    w = synth.q6_k_weight(synth.key(8, 1 + K), M, K)
    x = synth.normal(synth.key(8, 2 + K), K)
    note("q6_k gemv %dx%d" % (M, K))
    y = down(q4k.gemv_q6_k(up(w), up(x), M=M, K=K))
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([rng.integers(0, M, 300), [0, 63, 64, M - 65, M - 64, M - 1]]))
    yr, S = oracle.gemv_q6_k(w, x, M, K, rows=rows)
    assert_gemv(y[rows], yr, S, "q6_k %dx%d" % (M, K))


def test_q6_k_gemv_zero_and_one_hot(q4k):
    M, K = 200, 2048
    w = synth.q6_k_weight(synth.key(8, 5), M, K)
    wd = up(w)
    assert np.all(down(q4k.gemv_q6_k(wd, up(np.zeros(K, np.float32)), M=M, K=K)) == 0.0)
    deq = oracle.dequant_q6_k(w, M, K)
    for k in (0, 1, 15, 16, 31, 32, 127, 128, 255, 256, 1023, 2047):
        x = np.zeros(K, np.float32)
        x[k] = 1.0
        y = down(q4k.gemv_q6_k(wd, up(x), M=M, K=K))
        # one exact product, and the -32 offset cancels in integers
        assert np.array_equal(y, deq[:, k]), k


def test_q6_k_gemv_deterministic_and_split_variants(q4k):
    M, K = 5120, 17408
    w = synth.q6_k_weight(synth.key(8, 9), M, K)
    x = synth.normal(synth.key(8, 10), K)
    wd, xd = up(w), up(x)
    yr, S = oracle.gemv_q6_k(w, x, M, K)
    try:
        for groups in (0, 1, 7, 80, 333, 1024, 1360):
            q4k.tune_gemv(0, groups)
            note("q6_k groups=%d" % groups)
            y = down(q4k.gemv_q6_k(wd, xd, M=M, K=K))
            assert_gemv(y, yr, S, "q6_k groups=%d" % groups)
            assert np.array_equal(bits(y), bits(down(q4k.gemv_q6_k(wd, xd, M=M, K=K)))), groups
    finally:
        q4k.tune_gemv(0, 0)


@pytest.mark.parametrize("K", [256, 512, 1280, 5376])
def test_q6_k_gemv_rejects_k_not_multiple_of_1024(q4k, K):
    """Rows must hold a multiple of four blocks; anything else is Q4K_ESHAPE
    before any launch."""
    M = 8
    w = up(synth.q6_k_weight(synth.key(8, 20), M, K))
    x = up(np.ones(K, np.float32))
    with pytest.raises(Exception, match="1024"):
        q4k.gemv_q6_k(w, x, M=M, K=K)
