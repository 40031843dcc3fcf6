"""q4k_mlp (one MLP block: (1 + w) RMSNorm, gate|up with SwiGLU, down with the
residual) against the CPU oracle.

Every call goes through the C ABI.  The activation a = silu(g) * u is checked
against the oracle's with the GEMV bound carried through the SiLU; the output
is checked teacher-forced (the oracle's down matmul on the GPU's own
activation) under the GEMV bound, and end to end by cosine.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from synth import workloads as wl
from tests.gpu_util import COS_MIN, GEMV_ABS, GEMV_REL, bits, cosine, down, note, require_gpu, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q4k():
    require_gpu()
    import bit_block_quantized_gguf_amd as q4k
    return q4k


def _weights(cfg, H, I):
    return (synth.q4k_weight(synth.key(cfg, 1), I, H), synth.q4k_weight(synth.key(cfg, 2), I, H),
            synth.q4k_weight(synth.key(cfg, 3), H, I))


def _check(q4k, torch, H, I, cfg, gain, resid, label):
    wg, wu, wd = _weights(cfg, H, I)
    x = synth.normal(synth.key(cfg, 4), H)
    nw = (0.2 * synth.normal(synth.key(cfg, 5), H)).astype(np.float32) if gain else None
    r = synth.normal(synth.key(cfg, 6), H) if resid else None
    note("mlp %s H=%d I=%d" % (label, H, I))
    act = torch.empty(I, dtype=torch.float32, device="cuda")
    y = down(q4k.mlp(up(wg), up(wu), up(wd), up(x), up(nw) if gain else None, 1e-6,
                     up(r) if resid else None, act=act))
    a = down(act)
    o = oracle.mlp(wg, wu, wd, H, I, x, nw, 1e-6, r)
    # activation: errors of g and u (GEMV bound + 1/rms in f32) through silu
    dg = GEMV_REL * o["Sg"] + 2e-6 * np.abs(o["g"]) + GEMV_ABS
    du = GEMV_REL * o["Su"] + 2e-6 * np.abs(o["u"]) + GEMV_ABS
    sig = 1.0 / (1.0 + np.exp(-np.clip(o["g"], -700, 700)))
    silu = o["g"] * sig
    tol_a = 1.1 * np.abs(o["u"]) * dg + np.abs(silu) * du + dg * du + 4e-7 * np.abs(o["a"]) + GEMV_ABS
    err_a = np.abs(a.astype(np.float64) - o["a"])
    assert np.all(err_a <= tol_a), (label, int(np.argmax(err_a / tol_a)), float(np.max(err_a / tol_a)))
    # output, teacher-forced on the GPU's activation
    yd, Sd = oracle.gemv(wd, a, H, I)
    if resid:
        yd = yd + r.astype(np.float64)
    tol_y = GEMV_REL * Sd + GEMV_ABS + (np.abs(r) * 2.0 ** -23 if resid else 0.0)
    err_y = np.abs(y.astype(np.float64) - yd)
    assert np.all(err_y <= tol_y), (label, float(np.max(err_y / tol_y)))
    assert cosine(y, o["y"]) >= COS_MIN, label
    return y


@pytest.mark.parametrize("gain,resid", [(True, True), (False, True), (True, False), (False, False)])
def test_mlp_small(q4k, gain, resid):
    import torch
    _check(q4k, torch, 512, 768, 21, gain, resid, "small gain=%d resid=%d" % (gain, resid))


def test_mlp_ragged_tiles(q4k):
    """inter not a multiple of 32 rows of gate|up tiles, hidden not of 64."""
    import torch
    _check(q4k, torch, 1280, 2816, 22, True, True, "ragged")


def test_mlp_qwen_block(q4k):
    """The model's MLP shape: hidden 5120, intermediate 17408."""
    import torch
    _check(q4k, torch, wl.HIDDEN, wl.INTER, 23, True, True, "qwen")


def test_mlp_in_place_and_deterministic(q4k):
    """y written over resid (the residual stream updated in place) equals the
    out-of-place result bit for bit, and repeated calls agree bit for bit."""
    import torch
    H, I = 1024, 1536
    wg, wu, wd = (up(w) for w in _weights(24, H, I))
    x = up(synth.normal(synth.key(24, 4), H))
    nw = up((0.2 * synth.normal(synth.key(24, 5), H)).astype(np.float32))
    r_host = synth.normal(synth.key(24, 6), H)
    y1 = down(q4k.mlp(wg, wu, wd, x, nw, 1e-6, up(r_host)))
    y2 = down(q4k.mlp(wg, wu, wd, x, nw, 1e-6, up(r_host)))
    h = up(r_host)
    q4k.mlp(wg, wu, wd, x, nw, 1e-6, h, y=h)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y1), bits(y2))
    assert np.array_equal(bits(y1), bits(down(h)))
