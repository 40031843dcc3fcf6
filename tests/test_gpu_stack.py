"""Decode stack (one hipGraph per token, or one persistent kernel per token)
vs the oracle chain.

Two checks per plan, as the chain is long:
  * teacher-forced, per node: each GEMV node is recomputed by the oracle from
    the GPU's own input buffer and must meet the GEMV bar (1e-4*S + 1e-6, with
    the residual magnitude added to S for residual nodes);
  * end-to-end: logits vs the oracle's double-precision chain, cosine
    >= 0.999999.
The persistent plan runs the same nodes with the same unit split, so every
buffer it leaves must equal the graph plan's bit for bit.
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


def _build(q4k, shapes_per_layer, lm_shape, hidden, cfg, **kw):
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
    stack = q4k.DecodeStack(dev, up(lm), hidden=hidden, **kw)
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
    assert stack.nodes() == 4 * L + 1
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
    assert stack.nodes() == 1
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
    assert stack.nodes() == 4 * L + 1
    h0 = synth.activations(3, 1, wl.HIDDEN)[0]
    logits = down(stack(up(h0)))
    assert np.all(np.isfinite(logits))
    note("full stack: persistent plan")
    pstack = q4k.DecodeStack(dev, up(lm), hidden=wl.HIDDEN, persistent=True)
    for _ in range(2):
        plog = down(pstack(up(h0)))
        assert np.array_equal(bits(plog), bits(logits))
    assert pstack.status() == 0
    pstack.close()
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


BUFS = ("BUF_H", "BUF_U", "BUF_HMID", "BUF_G", "BUF_V", "BUF_A")


def _all_bits(q4k, stack, L):
    out = [bits(down(stack.buffer(0, q4k.BUF_LOGITS)))]
    for l in range(L + 1):
        for b in BUFS if l < L else BUFS[:1]:
            out.append(bits(down(stack.buffer(l, getattr(q4k, b)))))
    return out


@pytest.mark.parametrize("L,H,V", [(4, 512, 1000), (0, 768, 333), (3, 1024, 70000)])
def test_persistent_equals_graph(q4k, torch, L, H, V):
    """Every arena buffer of the persistent plan equals the graph plan's, bit
    for bit, over several tokens with eager work in between.  The small
    shapes give nodes with fewer work units than workgroups; the 70000-row
    head gives one with many more."""
    shapes = _small_shapes(L, H)
    host, dev, lm, graph = _build(q4k, shapes, (V, H), H, cfg=33)
    pers = q4k.DecodeStack(dev, up(lm), hidden=H, persistent=True)
    assert pers.nodes() == graph.nodes() == 4 * L + 1
    note("persistent vs graph L=%d H=%d V=%d" % (L, H, V))
    for t in range(6):
        h = up(synth.normal(synth.key(33, 7000 + t), H))
        graph(h)
        ref = _all_bits(q4k, graph, L)
        junk = torch.randn(1 << 16, device="cuda").sum()
        pers(h)
        got = _all_bits(q4k, pers, L)
        for i, (a, b) in enumerate(zip(got, ref)):
            assert np.array_equal(a, b), (t, i)
        del junk
    assert pers.status() == 0
    if L:
        _teacher_forced(q4k, pers, host, lm, shapes, range(L), lambda M: np.arange(M))
    pers.close()
    graph.close()


def test_persistent_many_tokens(q4k, torch):
    """Two hundred tokens back to back (the node counters grow by the grid
    size every token) return the same bits as the first run of each input."""
    L, H, V = 2, 512, 640
    shapes = _small_shapes(L, H)
    host, dev, lm, pers = _build(q4k, shapes, (V, H), H, cfg=34, persistent=True)
    hs = [up(synth.normal(synth.key(34, 100 + i), H)) for i in range(4)]
    first = [bits(down(pers(h))) for h in hs]
    outs = [pers(hs[t % 4]) for t in range(200)]
    torch.cuda.synchronize()
    for t in range(200):
        assert np.array_equal(bits(down(outs[t])), first[t % 4]), t
    assert pers.status() == 0
    pers.close()


def test_persistent_wait_limit_reports_and_recovers(q4k, torch):
    """With a one-poll limit a wait between nodes gives up (the kernel still
    ends); status() reports it once and clears it; a plan with the default
    limit on the same weights still matches the graph plan afterwards."""
    L, H, V = 4, 512, 1000
    shapes = _small_shapes(L, H)
    host, dev, lm, graph = _build(q4k, shapes, (V, H), H, cfg=35)
    tight = q4k.DecodeStack(dev, up(lm), hidden=H, persistent=True, spin_limit=1)
    h = up(synth.normal(synth.key(35, 1), H))
    seen = 0
    for _ in range(20):
        tight(h)
        seen = tight.status()
        if seen:
            break
    note("one-poll limit reported: %d" % seen)
    assert seen == 1
    assert tight.status() == 0          # cleared
    tight.close()
    pers = q4k.DecodeStack(dev, up(lm), hidden=H, persistent=True)
    assert np.array_equal(bits(down(pers(h))), bits(down(graph(h))))
    assert pers.status() == 0
    pers.close()
    graph.close()
