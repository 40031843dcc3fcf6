"""HIP path vs the CPU oracle: dequant, GEMV, batched GEMV and GEMM.

Every call goes through the C ABI (the Python binding only marshals
arguments).  Inputs come from the seeded generator; expected values come
from the oracle or from the hand-worked blocks.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from synth import workloads as wl
from tests.golden_io import load_worked_blocks
from tests.gpu_util import (COS_MIN, GEMM_REL, GEMV_REL, assert_gemv, assert_within, bits,
                            cosine, down, note, require_gpu, up)

pytestmark = pytest.mark.gpu
QK, BB = 256, 144


@pytest.fixture(scope="module")
def torch():
    return require_gpu()


@pytest.fixture(scope="module")
def q4k(torch):
    import bit_block_quantized_gguf_amd as q4k
    return q4k


def _case(cfg, t, M, K):
    return synth.q4k_weight(synth.key(cfg, t), M, K), synth.normal(synth.key(cfg, 1000 + t), K)


# ---------------------------------------------------------------- dequant

def test_dequant_worked_blocks(q4k):
    items = load_worked_blocks()
    W = np.stack([it["block"] for it in items])           # M = #blocks, K = 256
    got = down(q4k.dequant(up(W), len(items), QK))
    for r, it in enumerate(items):
        for k, (val, sign) in enumerate(it["expect"]):
            exp = np.float32(float(val))
            if val == 0:
                exp = np.float32(-0.0 if sign < 0 else 0.0)
            assert bits(got[r, k]) == bits(exp), (it["id"], k, got[r, k], exp)


@pytest.mark.parametrize("M,K", [(512, 1024), (1024, 512), (1, 256), (37, 768), (130, 2560)])
def test_dequant_bit_exact(q4k, M, K):
    w, _ = _case(1, M + K, M, K)
    note("dequant %dx%d" % (M, K))
    got = down(q4k.dequant(up(w), M, K))
    assert np.array_equal(bits(got), bits(oracle.dequant(w, M, K)))


def test_dequant_all_finite_halves(q4k):
    """d and dmin over every finite binary16 class (subnormals, negatives,
    zeros): bit-exact including the sign of zero."""
    M, K = 64, 2048
    w = synth.q4k_weight(synth.key(1, 77), M, K).reshape(-1, BB).copy()
    rng = np.random.default_rng(5)
    h = rng.integers(0, 65536, size=(w.shape[0], 2), dtype=np.uint32)
    h[(h >> 10 & 31) == 31] &= 0x83FF          # keep finite: clear the exponent
    h[::7, 0] = 0x8000                          # -0 scales
    h[::5, 1] = 0x0000
    h[::11, 0] = 0x0001
    w[:, 0], w[:, 1] = h[:, 0] & 0xFF, h[:, 0] >> 8
    w[:, 2], w[:, 3] = h[:, 1] & 0xFF, h[:, 1] >> 8
    w = w.reshape(M, -1)
    got = down(q4k.dequant(up(w), M, K))
    assert np.array_equal(bits(got), bits(oracle.dequant(w, M, K)))


def test_dequant_mlp_shape_bit_exact(q4k):
    M, K = 17408, 5120
    w = synth.q4k_weight(synth.key(2, 0), M, K)
    note("dequant full %dx%d" % (M, K))
    got = down(q4k.dequant(up(w), M, K))
    assert np.array_equal(bits(got), bits(oracle.dequant(w, M, K)))


# ---------------------------------------------------------------- GEMV

@pytest.mark.parametrize("M,K", [(512, 1024), (1024, 512), (1, 256), (63, 256), (65, 512),
                                 (130, 768), (257, 2560), (1000, 4096), (64, 17408)])
def test_gemv_matches_oracle(q4k, M, K):
    w, x = _case(1, 7 * M + K, M, K)
    note("gemv %dx%d" % (M, K))
    y = down(q4k.gemv(up(w), up(x), M=M, K=K))
    yr, S = oracle.gemv(w, x, M, K)
    assert_gemv(y, yr, S, "gemv %dx%d" % (M, K))


def test_gemv_mlp_block(q4k):
    """Gate and up at 17408x5120, then down at 5120x17408 on silu(g)*u formed
    by the caller (the oracle, from the GPU's gate/up outputs)."""
    x = synth.activations(2, 1, wl.HIDDEN)[0]
    ws = {name: synth.q4k_weight(synth.key(2, i), M, K) for i, (name, M, K) in enumerate(wl.MLP)}
    outs = {}
    for name in ("gate", "up"):
        note("gemv %s" % name)
        y = down(q4k.gemv(up(ws[name]), up(x), M=wl.INTER, K=wl.HIDDEN))
        yr, S = oracle.gemv(ws[name], x, wl.INTER, wl.HIDDEN)
        assert_gemv(y, yr, S, name)
        outs[name] = y.astype(np.float64)
    g, u = outs["gate"], outs["up"]
    a = np.array([oracle.silu(v) for v in g]) * u
    a = a.astype(np.float32)
    note("gemv down")
    y = down(q4k.gemv(up(ws["down"]), up(a), M=wl.HIDDEN, K=wl.INTER))
    yr, S = oracle.gemv(ws["down"], a, wl.HIDDEN, wl.INTER)
    assert_gemv(y, yr, S, "down")


def test_gemv_zero_and_one_hot(q4k):
    M, K = 300, 1024
    w, _ = _case(1, 5, M, K)
    wd = up(w)
    y = down(q4k.gemv(wd, up(np.zeros(K, np.float32)), M=M, K=K))
    assert np.all(y == 0.0)
    deq = oracle.dequant(w, M, K)
    for k in (0, 17, 31, 32, 63, 64, 100, 255, 256, 511, 700, 1023):
        x = np.zeros(K, np.float32)
        x[k] = 1.0
        y = down(q4k.gemv(wd, up(x), M=M, K=K))
        # every term but one is an exact zero, so the column comes back exactly
        assert np.array_equal(y, deq[:, k]), k


def test_gemv_deterministic_and_split_variants(q4k):
    M, K = 5120, 17408
    w, x = _case(1, 99, M, K)
    wd, xd = up(w), up(x)
    y0 = down(q4k.gemv(wd, xd, M=M, K=K))
    y1 = down(q4k.gemv(wd, xd, M=M, K=K))
    assert np.array_equal(bits(y0), bits(y1))
    yr, S = oracle.gemv(w, x, M, K)
    try:
        for groups in (1, 7, 80, 81, 200, 333, 1024, 1360, 5000):
            q4k.tune_gemv(0, groups)
            note("gemv groups=%d" % groups)
            y = down(q4k.gemv(wd, xd, M=M, K=K))
            assert_gemv(y, yr, S, "groups=%d" % groups)
            y2 = down(q4k.gemv(wd, xd, M=M, K=K))
            assert np.array_equal(bits(y), bits(y2)), groups
    finally:
        q4k.tune_gemv(0, 0)


def test_gemv_cancellation_blocks(q4k):
    """Sub-blocks whose weights cancel to exact zero (constant nibble q with
    dmin*m = d*sc*q) exercise the factored sum: the bar still holds."""
    M, K = 128, 1024
    w = synth.q4k_weight(synth.key(1, 55), M, K).reshape(-1, BB).copy()
    # d = dmin = 2^-10, sc = m = 7 in every sub-block (packing: s[0..7] = 7, s[8..11] = 0x77)
    d = 0x1400
    w[:, 0], w[:, 1], w[:, 2], w[:, 3] = d & 0xFF, d >> 8, d & 0xFF, d >> 8
    w[:, 4:12] = 7
    w[:, 12:16] = 0x77
    w[::2, 16:] = 0x11        # q = 1 everywhere: w = 7*2^-10 - 7*2^-10 = 0 on even blocks
    w = w.reshape(M, -1)
    x = synth.normal(synth.key(1, 56), K)
    y = down(q4k.gemv(up(w), up(x), M=M, K=K))
    yr, S = oracle.gemv(w, x, M, K)
    assert_within(y, yr, S, GEMV_REL, "cancellation")


# ---------------------------------------------------------------- batched GEMV

@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 8, 16, 17, 33])
def test_gemv_batch_small(q4k, N):
    M, K = 777, 1536
    w, _ = _case(4, N, M, K)
    X = synth.activations(4, N, K, first=100)
    note("gemv_batch N=%d" % N)
    Y = down(q4k.gemv_batch(up(w), up(X), M=M, K=K))
    Yr, S = oracle.gemv_batch(w, X, M, K)
    for n in range(N):
        assert_gemv(Y[n], Yr[n], S[n], "N=%d n=%d" % (N, n))


@pytest.mark.parametrize("N", wl.BATCH_N)
def test_gemv_batch_full_shape(q4k, N):
    M, K = wl.BATCH_SHAPE
    w = synth.q4k_weight(synth.key(4, 0), M, K)
    X = synth.activations(4, N, K)
    note("gemv_batch full N=%d" % N)
    Y = down(q4k.gemv_batch(up(w), up(X), M=M, K=K))
    Yr, S = oracle.gemv_batch(w, X, M, K)
    for n in range(N):
        assert_gemv(Y[n], Yr[n], S[n], "N=%d n=%d" % (N, n))


@pytest.mark.parametrize("N", [8, 16])
def test_gemv_batch_wide_range(q4k, N):
    """Activations spread over 2^-80 .. 2^80: vector n is scaled by
    2^(8n - 60) and each column by a further 2^e, e in [-20, 20].  Sixteen
    vectors run on bf16 matrix instructions with each f32 operand split into
    two bf16 parts, which keep the full f32 exponent range; every vector must
    still meet the f32 bar."""
    M, K = 512, 2048
    w, _ = _case(4, 7, M, K)
    X = synth.activations(4, N, K, first=200)
    e = np.clip(np.round(synth.normal(synth.key(4, 77), K) * 10.0), -20, 20)
    X = (X * np.exp2(e)[None, :] * np.exp2(8.0 * np.arange(N) - 60.0)[:, None]).astype(np.float32)
    note("gemv_batch wide range N=%d" % N)
    Y = down(q4k.gemv_batch(up(w), up(X), M=M, K=K))
    Yr, S = oracle.gemv_batch(w, X, M, K)
    assert np.all(np.isfinite(Y))
    for n in range(N):
        assert_gemv(Y[n], Yr[n], S[n], "N=%d n=%d" % (N, n))


def test_gemv_batch_one_equals_gemv(q4k):
    M, K = 2000, 5120
    w, x = _case(4, 3, M, K)
    y = down(q4k.gemv(up(w), up(x), M=M, K=K))
    Y = down(q4k.gemv_batch(up(w), up(x[None, :]), M=M, K=K))
    assert np.array_equal(bits(Y[0]), bits(y))


# ---------------------------------------------------------------- GEMM

def _check_gemm(Y, w, X, M, K, rows, toks, what):
    Yr, S = oracle.gemm(w, X, M, K, rows=rows, toks=toks)
    Y16, S16 = oracle.gemm(w, X, M, K, rows=rows, toks=toks, bf16_inputs=True)
    got = Y[np.ix_(toks, rows)] if rows is not None else Y[toks]
    assert_within(got, Yr, S, GEMM_REL, what + " vs f32 reference")
    assert_within(got, Y16, S16, GEMV_REL, what + " vs bf16-input reference")
    for t in range(got.shape[0]):
        c = cosine(got[t], Y16[t])
        assert c >= COS_MIN, "%s token %d cosine %.9f" % (what, t, c)


@pytest.mark.parametrize("tile,wg", [(0, 0), (32, 1), (32, 4), (32, 5), (64, 2), (64, 9), (128, 1),
                                     (128, 3), (256, 1), (256, 2), (256, 7)])
@pytest.mark.parametrize("M,K,P", [(300, 512, 1), (300, 512, 7), (128, 256, 128), (129, 768, 130),
                                   (520, 1024, 200), (64, 4096, 33), (257, 2048, 257),
                                   (256, 1280, 128)])
def test_gemm_small(q4k, M, K, P, tile, wg):
    """Ragged rows and tokens around both tile widths; stream-K grids of one
    workgroup (everything in one range), a few workgroups whose ranges cut
    tiles at odd super-block offsets, and grids with fewer workgroups than
    tiles, where whole-tile rounds come before the stream-K ranges (32 tokens
    on 4 workgroups; 0: automatic)."""
    w, _ = _case(5, M + P, M, K)
    X = synth.activations(5, P, K, first=M)
    note("gemm %dx%d P=%d tile=%d wg=%d" % (M, K, P, tile, wg))
    try:
        q4k.tune_gemm(tile, wg)
        Y = down(q4k.gemm(up(w), up(X), M=M, K=K))
    finally:
        q4k.tune_gemm(0, 0)
    toks = np.arange(P)
    _check_gemm(Y, w, X, M, K, np.arange(M), toks,
                "gemm %dx%d P=%d tile=%d wg=%d" % (M, K, P, tile, wg))


def _sample(n, rng, k=48, tile=128):
    idx = set(rng.choice(n, size=min(k, n), replace=False).tolist())
    idx |= {0, n - 1}
    idx |= {i for i in range(tile - 1, n, tile) if i < n}       # tile edges
    idx |= {i for i in range(tile, n, tile)}
    return np.array(sorted(idx), np.int64)


@pytest.mark.parametrize("shape", wl.PREFILL_SHAPES, ids=["17408x5120", "5120x17408"])
@pytest.mark.parametrize("P", wl.PREFILL_P)
def test_gemm_prefill_sampled(q4k, shape, P):
    M, K = shape
    w = synth.q4k_weight(synth.key(5, wl.PREFILL_SHAPES.index(shape)), M, K)
    X = synth.activations(5, P, K)
    note("gemm prefill %dx%d P=%d" % (M, K, P))
    Y = down(q4k.gemm(up(w), up(X), M=M, K=K))
    assert np.all(np.isfinite(Y))
    rng = np.random.default_rng(P + M)
    rows, toks = _sample(M, rng, 40), _sample(P, rng, 16)
    _check_gemm(Y, w, X, M, K, rows, toks, "prefill %dx%d P=%d" % (M, K, P))


@pytest.mark.parametrize("shape", wl.PREFILL_SHAPES, ids=["17408x5120", "5120x17408"])
def test_gemm_prefill_every_element(q4k, shape):
    """P = 256 at full size, every one of the 4.5 million outputs against both
    references (the oracle computes all of them: 45.6 GFLOP in double, a few
    seconds on the host threads)."""
    M, K = shape
    P = wl.PREFILL_P[0]
    w = synth.q4k_weight(synth.key(5, wl.PREFILL_SHAPES.index(shape)), M, K)
    X = synth.activations(5, P, K)
    note("gemm prefill every element %dx%d P=%d" % (M, K, P))
    Y = down(q4k.gemm(up(w), up(X), M=M, K=K))
    _check_gemm(Y, w, X, M, K, None, np.arange(P), "prefill all %dx%d P=%d" % (M, K, P))


@pytest.mark.parametrize("P", [1, 16, 22, 27, 64])
def test_gemm_short_prompt_sampled(q4k, P):
    """Short prompts (the 22- and 27-token prompts among them) on the MLP
    gate shape: narrow token tiles, every CU busy through stream-K, sampled
    rows and every token."""
    M, K = wl.PREFILL_SHAPES[0]
    w = synth.q4k_weight(synth.key(5, 0), M, K)
    X = synth.activations(5, P, K)
    note("gemm short prompt %dx%d P=%d (tile %d)" % (M, K, P, q4k.gemm_config(M, K, P)[0]))
    Y = down(q4k.gemm(up(w), up(X), M=M, K=K))
    assert np.all(np.isfinite(Y))
    rng = np.random.default_rng(P + 3)
    rows = _sample(M, rng, 40)
    _check_gemm(Y, w, X, M, K, rows, np.arange(P), "short prompt P=%d" % P)


def test_gemm_bf16_exact_inputs(q4k):
    """E7-tiled weights (small integers) and x with <= 8 significant bits are
    exact in bf16, so only f32 accumulation error remains vs the exact sum."""
    blk = next(it for it in load_worked_blocks() if it["id"] == "E7")["block"]
    M, K, P = 256, 1024, 160
    w = np.ascontiguousarray(np.tile(blk, (M, K // QK)))
    rng = np.random.default_rng(9)
    X = (rng.integers(-128, 128, (P, K)) / 16.0).astype(np.float32)
    Y = down(q4k.gemm(up(w), up(X), M=M, K=K))
    Yr, S = oracle.gemm(w, X, M, K)
    assert_within(Y, Yr, S, GEMV_REL, "bf16-exact gemm")


def test_gemm_split_k_variants_agree(q4k):
    """Stream-K partitions from one workgroup to more than the CUs, at both
    tile widths: every one gives the reference within the bars, repeated
    calls give the same bits, and each call leaves the workspace's counter
    region at zero."""
    M, K, P = 5120, 17408, 256
    w = synth.q4k_weight(synth.key(5, 1), M, K)
    X = synth.activations(5, P, K)
    wd, Xd = up(w), up(X)
    rng = np.random.default_rng(3)
    rows, toks = _sample(M, rng, 24), _sample(P, rng, 8)
    try:
        outs = []
        for tt, wg in ((32, 1), (32, 256), (32, 1000), (64, 77), (64, 256), (128, 1), (128, 37),
                       (128, 256), (128, 511), (256, 1), (256, 5), (256, 256), (256, 1000)):
            q4k.tune_gemm(tt, wg)
            note("gemm tile=%d wg=%d" % (tt, wg))
            ws = q4k.Workspace(q4k.workspace_size(q4k.OP_GEMM, M, K, P))
            Y = down(q4k.gemm(wd, Xd, M=M, K=K, ws=ws))
            assert not ws.tensor[:4 * 16384].cpu().numpy().any(), "counters left non-zero"
            _check_gemm(Y, w, X, M, K, rows, toks, "tile=%d wg=%d" % (tt, wg))
            outs.append(Y)
            Y2 = down(q4k.gemm(wd, Xd, M=M, K=K, ws=ws))
            assert np.array_equal(bits(Y2), bits(Y))                 # deterministic
    finally:
        q4k.tune_gemm(0, 0)
