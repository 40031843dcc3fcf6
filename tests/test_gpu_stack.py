"""Decode stack (one hipGraph per token) vs the oracle chain.

Two checks per plan, as the chain is long:
  * teacher-forced, per node: each GEMV node is recomputed by the oracle from
    the GPU's own input buffer and must meet the GEMV bar (1e-4*S + 1e-6, with
    the residual magnitude added to S for residual nodes);
  * end-to-end: logits vs the oracle's double-precision chain, cosine
    >= 0.999999.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import synth
from synth import workloads as wl
from tests.gpu_util import (COS_MIN, GEMV_REL, assert_within, bits, cosine, down, note,
                            require_gpu, up)

pytestmark = pytest.mark.gpu
MATS = wl.LAYER_MATS


@pytest.fixture(scope="module")
def torch():
    return require_gpu()


@pytest.fixture(scope="module")
def q4k(torch):
    import bit_block_quantized_gguf_amd as q4k
    return q4k


def _rmsn(v):
    v = np.asarray(v, np.float64)
    return v / math.sqrt(np.mean(v * v) + 1e-6)


def _build(q4k, shapes_per_layer, lm_shape, hidden, cfg):
    host, dev = [], []
    for l, sh in enumerate(shapes_per_layer):
        hl, dl = {}, {}
        for i, name in enumerate(MATS):
            M, K = sh[name]
            hl[name] = synth.q4k_weight(synth.key(cfg, 5 * l + i), M, K)
            dl[name] = up(hl[name])
        host.append(hl)
        dev.append(dl)
    lm = synth.q4k_weight(synth.key(cfg, 5 * len(shapes_per_layer)), *lm_shape)
    stack = q4k.DecodeStack(dev, up(lm), hidden=hidden)
    return host, dev, lm, stack


def _teacher_forced(q4k, stack, host, lm, shapes, layers, rows_fn):
    """Check every node of the given layers from the GPU's own inputs."""
    get = lambda l, b: down(stack.buffer(l, b)).astype(np.float64)
    for l in layers:
        sh = shapes[l]
        h = get(l, q4k.BUF_H)
        u = get(l, q4k.BUF_U)
        hm = get(l, q4k.BUF_HMID)
        g = get(l, q4k.BUF_G)
        v = get(l, q4k.BUF_V)
        a = get(l, q4k.BUF_A)
        hn = get(l + 1, q4k.BUF_H)

        def node(name, x, out, resid=None):
            M, K = sh[name]
            rows = rows_fn(M)
            y, S = oracle.gemv(host[l][name], _rmsn(x), M, K, rows=rows)
            if resid is not None:
                y = y + resid[rows]
                S = S + np.abs(resid[rows])
            assert_within(out[rows], y, S, GEMV_REL, "layer %d %s" % (l, name))

        node("mix_in", h, u)
        node("mix_out", u[:sh["mix_out"][1]], hm, resid=h)
        node("gate", hm, g)
        node("up", hm, v)
        node("down", a, hn, resid=hm)
        ref_a = np.array([oracle.silu(t) for t in g]) * v
        assert np.all(np.abs(a - ref_a) <= 1e-5 * np.abs(ref_a) + 1e-6 * (np.abs(v) + 1e-30)), l
    L = len(shapes)
    hL = get(L, q4k.BUF_H)
    logits = get(0, q4k.BUF_LOGITS)
    rows = rows_fn(lm.shape[0])
    y, S = oracle.gemv(lm, _rmsn(hL), lm.shape[0], hL.size, rows=rows)
    assert_within(logits[rows], y, S, GEMV_REL, "lm_head")


def _small_shapes(n_layers, hidden=512, inter=1024):
    shapes = []
    for l in range(n_layers):
        attn = l % 4 == 3
        shapes.append({"mix_in": (1280 if attn else 1536, hidden),
                       "mix_out": (hidden, 768 if attn else 1024),
                       "gate": (inter, hidden), "up": (inter, hidden), "down": (hidden, inter)})
    return shapes


def test_small_stack_end_to_end_and_per_node(q4k):
    L, H, V = 4, 512, 1000
    shapes = _small_shapes(L, H)
    host, dev, lm, stack = _build(q4k, shapes, (V, H), H, cfg=30)
    assert stack.nodes() == 4 * L + 2
    h0 = synth.normal(synth.key(30, 9999), H)
    logits = down(stack(up(h0)))
    mats, shp = [], []
    for l in range(L):
        for name in MATS:
            mats.append(host[l][name])
            shp.append(shapes[l][name])
    mats.append(lm)
    shp.append((V, H))
    ref = oracle.stack(mats, shp, L, H, h0)
    c = cosine(logits, ref)
    note("small stack cosine %.12f" % c)
    assert c >= COS_MIN
    assert np.max(np.abs(logits - ref)) <= 1e-4 * np.max(np.abs(ref))
    _teacher_forced(q4k, stack, host, lm, shapes, range(L), lambda M: np.arange(M))
    stack.close()


def test_stack_replays_match_eager_and_each_other(q4k, torch):
    """The graph is replayed many times with other work and syncs in between;
    every replay of the same input returns the same bits."""
    L, H, V = 2, 512, 640
    shapes = _small_shapes(L, H)
    host, dev, lm, stack = _build(q4k, shapes, (V, H), H, cfg=31)
    hs = [synth.normal(synth.key(31, 5000 + i), H) for i in range(3)]
    first = [down(stack(up(h))) for h in hs]
    assert not np.array_equal(first[0], first[1])
    for rep in range(5):
        for i, h in enumerate(hs):
            junk = torch.randn(1 << 16, device="cuda").sum()       # eager work between replays
            out = down(stack(up(h)))
            assert np.array_equal(bits(out), bits(first[i])), (rep, i)
            del junk
    stack.close()


def test_stack_zero_layers(q4k):
    H, V = 768, 333
    host, dev, lm, stack = _build(q4k, [], (V, H), H, cfg=32)
    assert stack.nodes() == 2
    h0 = synth.normal(synth.key(32, 1), H)
    logits = down(stack(up(h0)))
    y, S = oracle.gemv(lm, _rmsn(h0), V, H)
    assert_within(logits, y, S, GEMV_REL, "lm only")
    stack.close()


def test_full_stack_sampled(q4k, torch):
    """The 64-layer, hidden-5120 chain (about 14.4 GB of Q4_K weights).

    Teacher-forced checks on sampled rows of every node of four layers and
    the lm_head, and end-to-end logits against the oracle's double chain."""
    L = wl.N_LAYERS
    shapes = [wl.layer_shapes(l) for l in range(L)]
    note("full stack: generating %.2f GB" % (wl.stack_bytes() / 1e9))
    host, dev = [], []
    for l in range(L):
        hl, dl = {}, {}
        for name in MATS:
            M, K = shapes[l][name]
            hl[name] = synth.q4k_weight(wl.stack_tensor_key(l, name), M, K)
            dl[name] = up(hl[name])
        host.append(hl)
        dev.append(dl)
    lm = synth.q4k_weight(wl.stack_tensor_key(None, "lm_head"), wl.VOCAB, wl.HIDDEN)
    note("full stack: capturing graph")
    stack = q4k.DecodeStack(dev, up(lm), hidden=wl.HIDDEN)
    assert stack.nodes() == 4 * L + 2
    h0 = synth.activations(3, 1, wl.HIDDEN)[0]
    logits = down(stack(up(h0)))
    assert np.all(np.isfinite(logits))
    rng = np.random.default_rng(1)
    rows_fn = lambda M: np.unique(np.concatenate([rng.choice(M, 256, replace=False), [0, M - 1]]))
    note("full stack: teacher-forced checks")
    _teacher_forced(q4k, stack, host, lm, shapes, [0, 3, 31, 63], rows_fn)
    note("full stack: oracle chain")
    mats, shp = [], []
    for l in range(L):
        for name in MATS:
            mats.append(host[l][name])
            shp.append(shapes[l][name])
    mats.append(lm)
    shp.append((wl.VOCAB, wl.HIDDEN))
    ref = oracle.stack(mats, shp, L, wl.HIDDEN, h0)
    c = cosine(logits, ref)
    note("full stack cosine %.12f" % c)
    assert c >= COS_MIN
    stack.close()
