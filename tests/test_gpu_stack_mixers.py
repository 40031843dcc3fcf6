"""Decode stack with the real token mixers (Q4K_STACK_MIXERS): three Gated
DeltaNet layers and one gated-attention layer (the layout of the pages'
tiny hybrid fixture), three tokens in a row.

Per token, every node is recomputed by the oracle from the GPU's own input
(teacher-forced): the projections and MLP GEMVs under the GEMV bar, the
mixers from the GPU's mixer-in output and the GPU's state before the token
under the mixer bars of test_gpu_mixers.py, and the states after the token.
End to end, the oracle runs the whole chain in double from the same inputs,
token after token, and the logits must match by cosine.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import GEMV_REL, assert_within, cosine, down, note, require_gpu, up

pytestmark = pytest.mark.gpu
H, I, V = 512, 1024, 1000
KINDS = [0, 0, 0, 1]
GDN = dict(key_heads=2, value_heads=4)
ATT = dict(q_heads=2, kv_heads=1, rope_dim=64, rope_theta=1e7)
CAP = 8


@pytest.fixture(scope="module")
def torch():
    return require_gpu()


@pytest.fixture(scope="module")
def q4k(torch):
    import bit_block_quantized_gguf_amd as q4k
    return q4k


def _n(k, n, s=1.0):
    return (s * synth.normal(synth.key(17, k), n)).astype(np.float32)


def _shapes(kind):
    if kind == 0:
        Min = (2 * GDN["key_heads"] + 2 * GDN["value_heads"]) * 128 + 2 * GDN["value_heads"]
        Kout = GDN["value_heads"] * 128
    else:
        Min = (2 * ATT["q_heads"] + 2 * ATT["kv_heads"]) * 256
        Kout = ATT["q_heads"] * 256
    return {"mix_in": (Min, H), "mix_out": (H, Kout), "gate": (I, H), "up": (I, H),
            "down": (H, I)}


def _rmsn(v):
    v = np.asarray(v, np.float64)
    return v / np.sqrt(np.mean(v * v) + 1e-6)


def _within_heads(got, ref, nh, what, rel=2e-4):
    got = np.asarray(got, np.float64).reshape(nh, -1)
    ref = np.asarray(ref, np.float64).reshape(nh, -1)
    for h in range(nh):
        err = np.max(np.abs(got[h] - ref[h]))
        assert err <= rel * np.max(np.abs(ref[h])), (what, h, err)
        assert cosine(got[h], ref[h]) >= 0.999999, (what, h)


def test_stack_with_real_mixers(q4k, torch):
    host, dev, mats, shapes, mixers, dmix = [], [], [], [], [], []
    for l, kind in enumerate(KINDS):
        sh = _shapes(kind)
        hl, dl = {}, {}
        for i, name in enumerate(("mix_in", "mix_out", "gate", "up", "down")):
            hl[name] = synth.q4k_weight(synth.key(17, 10 * l + i), *sh[name])
            dl[name] = up(hl[name])
            mats.append(hl[name])
            shapes.append(sh[name])
        host.append(hl)
        dev.append(dl)
        if kind == 0:
            C = (2 * GDN["key_heads"] + GDN["value_heads"]) * 128
            m = dict(conv_w=_n(100 + l, 4 * C, 0.5), a_log=_n(110 + l, 4, 0.5),
                     dt_bias=_n(120 + l, 4, 0.5), norm_w=(1 + 0.1 * _n(130 + l, 128)).astype(np.float32),
                     **GDN)
        else:
            m = dict(q_norm_w=(0.2 * _n(140 + l, 256)).astype(np.float32),
                     k_norm_w=(0.2 * _n(150 + l, 256)).astype(np.float32), **ATT)
        mixers.append(m)
        dmix.append({k: (up(v) if isinstance(v, np.ndarray) else v) for k, v in m.items()})
    lm = synth.q4k_weight(synth.key(17, 99), V, H)
    mats.append(lm)
    shapes.append((V, H))
    stack = q4k.DecodeStack(dev, up(lm), hidden=H, kinds=KINDS, mixers=dmix, attn_capacity=CAP)
    # per layer four GEMVs and the mixer's kernels (GDN one, attention two;
    # each mixer also writes the sums of squares the out-projection needs),
    # then the lm_head and the position update
    L = len(KINDS)
    assert stack.nodes() == 4 * L + sum(1 if k == 0 else 2 for k in KINDS) + 2
    get = lambda l, b: down(stack.buffer(l, b)).astype(np.float64)
    # oracle states for the free-running chain
    ostates = []
    for l, kind in enumerate(KINDS):
        if kind == 0:
            C = (2 * GDN["key_heads"] + GDN["value_heads"]) * 128
            ostates.append((np.zeros(3 * C), np.zeros(4 * 128 * 128)))
        else:
            ostates.append((np.zeros((1, CAP, 256)), np.zeros((1, CAP, 256))))
    for tok in range(3):
        h0 = synth.normal(synth.key(17, 1000 + tok), H)
        before = []
        for l, kind in enumerate(KINDS):
            a, b = ((q4k.BUF_CONV_STATE, q4k.BUF_GDN_STATE) if kind == 0
                    else (q4k.BUF_K_CACHE, q4k.BUF_V_CACHE))
            before.append((get(l, a), get(l, b)))
        note("stack with mixers: token %d" % tok)
        logits = down(stack(up(h0))).astype(np.float64)
        assert stack.position() == tok + 1
        for l, kind in enumerate(KINDS):
            sh = _shapes(kind)
            W = host[l]
            h, u, o = get(l, q4k.BUF_H), get(l, q4k.BUF_U), get(l, q4k.BUF_MIX)
            hm, g, v, a, hn = (get(l, q4k.BUF_HMID), get(l, q4k.BUF_G), get(l, q4k.BUF_V),
                               get(l, q4k.BUF_A), get(l + 1, q4k.BUF_H))
            y, S = oracle.gemv(W["mix_in"], _rmsn(h), *sh["mix_in"])
            assert_within(u, y, S, GEMV_REL, "tok %d layer %d mix_in" % (tok, l))
            m = mixers[l]
            if kind == 0:
                ro, rcs, rS = oracle.gdn_step(u, m["conv_w"], m["a_log"], m["dt_bias"], m["norm_w"],
                                              before[l][0], before[l][1], Hk=2, Hv=4)
                _within_heads(o, ro, 4, "tok %d layer %d gdn" % (tok, l))
                assert np.array_equal(get(l, q4k.BUF_CONV_STATE), rcs.ravel())
                St = get(l, q4k.BUF_GDN_STATE)
                scale = np.abs(rS.ravel()) + np.sqrt(np.mean(rS * rS))
                assert np.all(np.abs(St - rS.ravel()) <= 2e-5 * scale), (tok, l)
            else:
                kc0 = before[l][0].reshape(1, CAP, 256)
                vc0 = before[l][1].reshape(1, CAP, 256)
                ro, rkc, rvc = oracle.attn_step(u, m["q_norm_w"], m["k_norm_w"], kc0, vc0, tok,
                                                Hq=2, Hkv=1, R=64, theta=1e7)
                _within_heads(o, ro, 2, "tok %d attention" % tok)
                kc = get(l, q4k.BUF_K_CACHE).reshape(1, CAP, 256)
                assert np.all(np.abs(kc[:, tok] - rkc[:, tok]) <= 2e-5 * (np.abs(rkc[:, tok]) + 1))
            y, S = oracle.gemv(W["mix_out"], _rmsn(o), *sh["mix_out"])
            assert_within(hm, y + h, S + np.abs(h), GEMV_REL, "tok %d layer %d mix_out" % (tok, l))
            y, S = oracle.gemv(W["gate"], _rmsn(hm), *sh["gate"])
            assert_within(g, y, S, GEMV_REL, "tok %d layer %d gate" % (tok, l))
            y, S = oracle.gemv(W["up"], _rmsn(hm), *sh["up"])
            assert_within(v, y, S, GEMV_REL, "tok %d layer %d up" % (tok, l))
            y, S = oracle.gemv(W["down"], _rmsn(a), *sh["down"])
            assert_within(hn, y + hm, S + np.abs(hm), GEMV_REL, "tok %d layer %d down" % (tok, l))
        y, S = oracle.gemv(lm, _rmsn(get(len(KINDS), q4k.BUF_H)), V, H)
        assert_within(logits, y, S, GEMV_REL, "tok %d lm_head" % tok)
        ref, ostates = oracle.stack_mixers_token(mats, shapes, KINDS, mixers, ostates, H, h0, tok)
        c = cosine(logits, ref)
        note("token %d logits cosine %.9f" % (tok, c))
        assert c >= 0.999999, (tok, c)
    stack.reset()
    assert stack.position() == 0
    torch.cuda.synchronize()
    assert not get(0, q4k.BUF_GDN_STATE).any() and not get(3, q4k.BUF_K_CACHE).any()
    stack.close()
