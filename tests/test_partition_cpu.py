"""Host-side bounds checks of the work partitions (no device): the kernels'
own range, owner and cut-tile arithmetic is run on the host for every
workgroup by q4k_check_partition, against the workspace each launch reserves
and the extent of its operands.  Shapes: every workload of the model, ragged
and tiny shapes, the largest the entry points accept, and sweeps of the
workgroup count (including counts above the number of work units)."""
from __future__ import annotations

import itertools

import pytest

import bit_block_quantized_gguf_amd as q4k
from synth import workloads as wl


@pytest.fixture(scope="module", autouse=True)
def lib():
    return q4k.load()


MODEL = [(wl.INTER, wl.HIDDEN), (wl.HIDDEN, wl.INTER), (16480, wl.HIDDEN), (14336, wl.HIDDEN),
         (wl.HIDDEN, 6144), (wl.VOCAB, wl.HIDDEN), (512, 1024), (1024, 512)]
RAGGED = [(1, 256), (63, 256), (64, 256), (65, 512), (777, 1536), (33, 2560), (129, 4352),
          (2047, 768)]
GROUPS = [0, 1, 2, 3, 7, 64, 255, 256, 511, 512, 513, 1000, 1024, 2048, 5000, 16384]


@pytest.mark.parametrize("M,K", MODEL + RAGGED)
def test_gemv_partitions(M, K):
    for G in GROUPS:
        q4k.check_partition(q4k.OP_GEMV, M, K, 1, G)
    for N, G in itertools.product((2, 3, 4, 8, 16, 33), (0, 5, 512, 4096)):
        q4k.check_partition(q4k.OP_GEMV_BATCH, M, K, N, G)


@pytest.mark.parametrize("inter,hidden", [(wl.INTER, wl.HIDDEN), (1024, 512), (4352, 2560),
                                          (768, 256)])
def test_mlp_partitions(inter, hidden):
    for G in GROUPS:
        q4k.check_partition(q4k.OP_MLP, inter, hidden, 1, G)


@pytest.mark.parametrize("M,K", [(wl.VOCAB, wl.HIDDEN), (777, 1536), (63, 512), (5120, 17408)])
def test_q8_q6_partitions(M, K):
    for G in (0, 1, 3, 512, 2048, 16384):
        q4k.check_partition(q4k.OP_GEMV_Q8_0, M, K, 1, G)
        if K % 1024 == 0:
            q4k.check_partition(q4k.OP_GEMV_Q6_K, M, K, 1, G)


@pytest.mark.parametrize("M,K", [(wl.INTER, wl.HIDDEN), (wl.HIDDEN, wl.INTER), (777, 1536),
                                 (300, 512), (1, 256)])
def test_gemm_partitions(M, K):
    try:
        for t, P, G in itertools.product((0, 32, 64, 128, 256), (1, 16, 22, 27, 64, 255, 256, 513,
                                                                  1024), (0, 1, 3, 256, 700)):
            q4k.tune_gemm(t, 0)
            q4k.check_partition(q4k.OP_GEMM, M, K, P, G)
    finally:
        q4k.tune_gemm(0, 0)


def test_largest_accepted_shapes():
    """M = 2^30 rows, K = 2^24 columns: 64-bit range arithmetic, 32-bit lane
    offsets at their widest."""
    for M, K in ((1 << 30, 256), (64, 1 << 24), (1 << 20, 1 << 24)):
        for G in (0, 1, 513, 16384):
            q4k.check_partition(q4k.OP_GEMV, M, K, 1, G)
            q4k.check_partition(q4k.OP_GEMV_BATCH, M, K, 16, G)
    q4k.check_partition(q4k.OP_GEMM, 1 << 20, 1 << 14, 1024, 0)


def test_refusals():
    with pytest.raises(q4k.Q4KError):
        q4k.check_partition(q4k.OP_GEMV, 64, 100)          # K not a multiple of 256
    with pytest.raises(q4k.Q4KError):
        q4k.check_partition(q4k.OP_GEMV, 64, 256, 1, -1)
    with pytest.raises(q4k.Q4KError):
        q4k.check_partition(q4k.OP_GEMV, (1 << 30) + 1, 256)
    with pytest.raises(q4k.Q4KError):
        q4k.check_partition(q4k.OP_GDN_STEP, 64, 256)
