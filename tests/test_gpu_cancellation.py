"""GEMV-family kernels on rows whose weights cancel (HIP path vs the oracle).

A row whose dequantised weights are all exactly zero has S = sum|w*x| = 0,
so the GEMV bar |y - y_ref| <= 1e-4*S + 1e-6 leaves 1e-6 absolute.  The
kernels form every weight exactly before it meets x (see
test_kernel_order_cpu.py for the f32 emulation of the old and new orders),
so such rows must come out as exactly 0 — through the plain GEMV, the
batched GEMV, the fused MLP block, the decode stack's fused epilogues, and
the Q8_0 and Q6_K kernels.  Rows that nearly cancel (eleven bits) and
ordinary generated rows share the matrices, so tiles mix all three kinds.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests.cancel_rows import q4k_mixed, q6_zero_row, q8_zero_row
from tests.gpu_util import (GEMV_ABS, GEMV_REL, assert_gemv, assert_within, down, note,
                            require_gpu, up)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return require_gpu()


@pytest.fixture(scope="module")
def q4k(torch):
    import bit_block_quantized_gguf_amd as q4k
    return q4k


def _zero_rows(w, M, K):
    deq = oracle.dequant(w, M, K)
    return np.nonzero(~deq.any(axis=1))[0]


SHAPES = [(256, 5120), (130, 17408), (327, 6144)]


@pytest.mark.parametrize("M,K", SHAPES)
def test_gemv_cancelling_rows(q4k, M, K):
    w = q4k_mixed(synth.q4k_weight(synth.key(11, M), M, K), K)
    x = synth.normal(synth.key(11, 1000 + M), K)
    zr = _zero_rows(w, M, K)
    assert zr.size >= M // 2 - 1
    note("gemv cancelling rows %dx%d" % (M, K))
    y = down(q4k.gemv(up(w), up(x), M=M, K=K)).astype(np.float64)
    yr, S = oracle.gemv(w, x, M, K)
    assert np.all(y[zr] == 0.0), y[zr][y[zr] != 0][:4]
    assert_gemv(y, yr, S, "gemv cancelling %dx%d" % (M, K))


@pytest.mark.parametrize("N", [1, 2, 4, 16])
def test_gemv_batch_cancelling_rows(q4k, N):
    M, K = 200, 5120
    w = q4k_mixed(synth.q4k_weight(synth.key(11, 77), M, K), K)
    X = synth.activations(11, N, K)
    zr = _zero_rows(w, M, K)
    note("gemv_batch cancelling rows N=%d" % N)
    Y = down(q4k.gemv_batch(up(w), up(X), M=M, K=K)).astype(np.float64)
    Yr, S = oracle.gemv_batch(w, X, M, K)
    assert np.all(Y[:, zr] == 0.0)
    for n in range(N):
        assert_gemv(Y[n], Yr[n], S[n], "gemv_batch cancelling N=%d n=%d" % (N, n))


def test_mlp_cancelling_rows(q4k, torch):
    H, I = 512, 1024
    wg = q4k_mixed(synth.q4k_weight(synth.key(11, 301), I, H), H, every=3)
    wu = synth.q4k_weight(synth.key(11, 302), I, H)
    wd = q4k_mixed(synth.q4k_weight(synth.key(11, 303), H, I), I)
    x = synth.normal(synth.key(11, 304), H)
    r = synth.normal(synth.key(11, 305), H)
    zg, zd = _zero_rows(wg, I, H), _zero_rows(wd, H, I)
    note("mlp cancelling rows")
    act = torch.empty(I, dtype=torch.float32, device="cuda")
    y = down(q4k.mlp(up(wg), up(wu), up(wd), up(x), None, 1e-6, up(r), act=act)).astype(np.float64)
    a = down(act).astype(np.float64)
    assert np.all(a[zg] == 0.0)                      # silu(0) * v = 0
    assert np.array_equal(y[zd], r[zd].astype(np.float64))   # 0 + resid
    o = oracle.mlp(wg, wu, wd, H, I, x, None, 1e-6, r)
    # activation: the GEMV bound of g and u (with the f32 1/rms) through silu
    dg = GEMV_REL * o["Sg"] + 2e-6 * np.abs(o["g"]) + GEMV_ABS
    du = GEMV_REL * o["Su"] + 2e-6 * np.abs(o["u"]) + GEMV_ABS
    silu = o["g"] / (1.0 + np.exp(-np.clip(o["g"], -700, 700)))
    tol_a = 1.1 * np.abs(o["u"]) * dg + np.abs(silu) * du + dg * du + 4e-7 * np.abs(o["a"]) + GEMV_ABS
    assert np.all(np.abs(a - o["a"]) <= tol_a)
    # output: the down GEMV teacher-forced on the GPU's own activation
    yd, Sd = oracle.gemv(wd, a, H, I)
    tol_y = GEMV_REL * Sd + GEMV_ABS + np.abs(r) * 2.0 ** -23
    assert np.all(np.abs(y - (yd + r)) <= tol_y)


def test_stack_one_layer_cancelling(q4k):
    """One layer plus lm_head, every matrix with cancelling rows; each node is
    recomputed by the oracle from the GPU's own input (teacher-forced)."""
    import math
    H = 512
    sh = {"mix_in": (1536, H), "mix_out": (H, 1024), "gate": (1024, H), "up": (1024, H),
          "down": (H, 1024)}
    host, dev = {}, {}
    for i, name in enumerate(("mix_in", "mix_out", "gate", "up", "down")):
        M, K = sh[name]
        host[name] = q4k_mixed(synth.q4k_weight(synth.key(12, i), M, K), K)
        dev[name] = up(host[name])
    lm = q4k_mixed(synth.q4k_weight(synth.key(12, 9), 700, H), H)
    stack = q4k.DecodeStack([dev], up(lm), hidden=H)
    h0 = synth.normal(synth.key(12, 10), H)
    note("stack one layer cancelling")
    stack(up(h0))
    get = lambda l, b: down(stack.buffer(l, b)).astype(np.float64)

    def rmsn(v):
        return v / math.sqrt(np.mean(v * v) + 1e-6)

    h, u, hm = get(0, q4k.BUF_H), get(0, q4k.BUF_U), get(0, q4k.BUF_HMID)
    g, v, a, h1 = get(0, q4k.BUF_G), get(0, q4k.BUF_V), get(0, q4k.BUF_A), get(1, q4k.BUF_H)
    logits = get(0, q4k.BUF_LOGITS)

    def node(name, xin, out, resid=None):
        M, K = sh[name] if name != "lm" else (700, H)
        W = host[name] if name != "lm" else lm
        y, S = oracle.gemv(W, rmsn(xin), M, K)
        zr = _zero_rows(W, M, K)
        if resid is not None:
            assert np.array_equal(out[zr], resid[zr]), name
            y, S = y + resid, S + np.abs(resid)
        else:
            assert np.all(out[zr] == 0.0), name
        assert_within(out, y, S, GEMV_REL, "stack %s" % name)

    node("mix_in", h, u)
    node("mix_out", u[:1024], hm, resid=h)
    node("gate", hm, g)
    node("up", hm, v)
    node("down", a, h1, resid=hm)
    node("lm", h1, logits)
    stack.close()


@pytest.mark.parametrize("d", [1e-3, 1.0, 65504.0])
def test_q8_0_cancelling_rows(q4k, d):
    M, K = 192, 5120
    w = np.array(synth.q8_0_weight(synth.key(13, 1), M, K), copy=True)
    w[::2] = q8_zero_row(d, K)
    x = synth.normal(synth.key(13, 2), K)
    note("q8_0 cancelling rows d=%g" % d)
    y = down(q4k.gemv_q8_0(up(w), up(x), M=M, K=K)).astype(np.float64)
    yr, S = oracle.gemv_q8_0(w, x, M, K)
    assert np.all(y[::2] == 0.0)
    assert_gemv(y, yr, S, "q8_0 cancelling d=%g" % d)


@pytest.mark.parametrize("d", [1e-3, 1.0, 65504.0])
def test_q6_k_cancelling_rows(q4k, d):
    M, K = 192, 5120
    w = np.array(synth.q6_k_weight(synth.key(13, 3), M, K), copy=True)
    w[::2] = q6_zero_row(d, K)
    x = synth.normal(synth.key(13, 4), K)
    note("q6_k cancelling rows d=%g" % d)
    y = down(q4k.gemv_q6_k(up(w), up(x), M=M, K=K)).astype(np.float64)
    yr, S = oracle.gemv_q6_k(w, x, M, K)
    assert np.all(y[::2] == 0.0)
    assert_gemv(y, yr, S, "q6_k cancelling d=%g" % d)
