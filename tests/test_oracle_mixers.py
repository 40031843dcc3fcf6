"""Pins of the mixer oracle (oracle/mixer_oracle.c) against closed forms.

Each case is chosen so that a plausible slip in the oracle changes the
result: a transposed state (S q instead of S^T q), the sign of the delta
rule, the order of the convolution taps or of the state shift, the key head
that a value head reads, the decay formula, the rotary pairing (i, i+R/2)
against (2i, 2i+1) and its frequencies, the partial-rotary boundary, the
(1 + w) RMSNorm form, the softmax scale and the output gates.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle

rng = np.random.default_rng(2026)


def silu(x):
    return x / (1.0 + np.exp(-x))


def sig(x):
    return 1.0 / (1.0 + np.exp(-x))


# ------------------------------------------------------------------ GDN

SMALL = dict(Hk=2, Hv=4, Dk=8, Dv=8)


def _gdn_inputs(Hk, Hv, Dk, Dv, taps=(0.0, 0.0, 0.0, 1.0)):
    C = 2 * Hk * Dk + Hv * Dv
    u = rng.normal(size=C + Hv * Dv + 2 * Hv)
    conv_w = np.tile(np.array(taps, np.float64), (C, 1))
    return dict(u=u, conv_w=conv_w, a_log=rng.normal(size=Hv), dt_bias=rng.normal(size=Hv),
                norm_w=rng.normal(size=Dv), conv_state=rng.normal(size=(C, 3)),
                S=np.zeros((Hv, Dv, Dk)))


def _split(u, Hk, Hv, Dk, Dv):
    nq, nv = Hk * Dk, Hv * Dv
    C = 2 * nq + nv
    return (u[:nq].reshape(Hk, Dk), u[nq:2 * nq].reshape(Hk, Dk), u[2 * nq:C].reshape(Hv, Dv),
            u[C:C + nv].reshape(Hv, Dv), u[C + nv:C + nv + Hv], u[C + nv + Hv:])


def _run(inp, dims):
    return oracle.gdn_step(inp["u"], inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["norm_w"],
                           inp["conv_state"], inp["S"], **dims)


def test_gdn_conv_state_shifts_oldest_out():
    inp = _gdn_inputs(**SMALL)
    _, cs, _ = _run(inp, SMALL)
    C = cs.shape[0]
    old = inp["conv_state"]
    assert np.array_equal(cs[:, 0], old[:, 1]) and np.array_equal(cs[:, 1], old[:, 2])
    assert np.array_equal(cs[:, 2], inp["u"][:C])


@pytest.mark.parametrize("taps,src", [((0, 0, 0, 1), "input"), ((1, 0, 0, 0), "oldest"),
                                      ((0, 0, 1, 0), "newest_state")])
def test_gdn_first_step_closed_form(taps, src):
    """From S = 0 the state after one step is beta k v^T, so the output of value
    head h is the gated norm of beta_h (k_j . q_j) v_h with j = h // (Hv/Hk)."""
    d = SMALL
    Hk, Hv, Dk, Dv = d["Hk"], d["Hv"], d["Dk"], d["Dv"]
    inp = _gdn_inputs(taps=taps, **d)
    out, _, S = _run(inp, d)
    C = 2 * Hk * Dk + Hv * Dv
    raw = {"input": inp["u"][:C], "oldest": inp["conv_state"][:, 0],
           "newest_state": inp["conv_state"][:, 2]}[src]
    c = silu(raw)
    q = c[:Hk * Dk].reshape(Hk, Dk)
    k = c[Hk * Dk:2 * Hk * Dk].reshape(Hk, Dk)
    v = c[2 * Hk * Dk:].reshape(Hv, Dv)
    _, _, _, z, b, _ = _split(inp["u"], Hk, Hv, Dk, Dv)
    qn = q / np.sqrt((q * q).sum(1, keepdims=True) + 1e-6) / math.sqrt(Dk)
    kn = k / np.sqrt((k * k).sum(1, keepdims=True) + 1e-6)
    for h in range(Hv):
        j = h // (Hv // Hk)
        beta = sig(b[h])
        np.testing.assert_allclose(S[h], beta * np.outer(v[h], kn[j]), rtol=1e-13, atol=1e-15)
        o = beta * (kn[j] @ qn[j]) * v[h]
        ref = inp["norm_w"] * o / np.sqrt(np.mean(o * o) + 1e-6) * silu(z[h])
        np.testing.assert_allclose(out[h * Dv:(h + 1) * Dv], ref, rtol=1e-12, atol=1e-14)


def test_gdn_delta_rule_replaces_the_value_of_a_key():
    """No decay (a_log -> -inf), beta = 1: after writing v1 then v2 under the
    same key, the state holds k v2^T, and the output reads v2."""
    d = SMALL
    Hk, Hv, Dk, Dv = d["Hk"], d["Hv"], d["Dk"], d["Dv"]
    inp = _gdn_inputs(**d)
    inp["a_log"] = np.full(Hv, -1e4)
    inp["conv_state"][:] = 0.0
    C = 2 * Hk * Dk + Hv * Dv
    nv = Hv * Dv
    u1 = inp["u"].copy()
    u1[C + nv:C + nv + Hv] = 40.0                   # beta = sigmoid(40) = 1 in double
    u2 = u1.copy()
    u2[2 * Hk * Dk:C] = rng.normal(size=nv)         # new values, same q and k
    _, cs, S1 = oracle.gdn_step(u1, inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["norm_w"],
                                inp["conv_state"], inp["S"], **d)
    out2, _, S2 = oracle.gdn_step(u2, inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["norm_w"],
                                  cs, S1, **d)
    k = silu(u1[Hk * Dk:2 * Hk * Dk]).reshape(Hk, Dk)
    kn = k / np.sqrt((k * k).sum(1, keepdims=True) + 1e-6)
    v2 = silu(u2[2 * Hk * Dk:C]).reshape(Hv, Dv)
    for h in range(Hv):
        j = h // (Hv // Hk)
        # |k|^2 = 1 - eps/(|k|^2 + eps): the old value is removed up to that factor
        np.testing.assert_allclose(S2[h], np.outer(v2[h], kn[j]), rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("a_log,a_plus_dt,alpha", [
    (0.0, 0.0, 0.5),                                              # -ln2
    (math.log(3.0), 2.0, (1.0 + math.e ** 2) ** -3),               # -3 softplus(2)
])
def test_gdn_decay_scales_the_state(a_log, a_plus_dt, alpha):
    """beta = 0 (b -> -inf): the step only decays, S' = exp(g) S with
    g = -exp(a_log) softplus(a + dt_bias)."""
    d = SMALL
    Hk, Hv, Dk, Dv = d["Hk"], d["Hv"], d["Dk"], d["Dv"]
    inp = _gdn_inputs(**d)
    inp["S"] = rng.normal(size=(Hv, Dv, Dk))
    inp["a_log"] = np.full(Hv, a_log)
    inp["dt_bias"] = np.full(Hv, 0.5)
    C = 2 * Hk * Dk + Hv * Dv
    nv = Hv * Dv
    inp["u"][C + nv:C + nv + Hv] = -800.0           # beta = 0 exactly
    inp["u"][C + nv + Hv:] = a_plus_dt - 0.5
    _, _, S = _run(inp, d)
    np.testing.assert_allclose(S, alpha * inp["S"], rtol=1e-14)


def test_gdn_model_dims_state_orientation():
    """At the model's sizes (16 key / 48 value heads x 128): a state with one
    nonzero entry S_h[i][j] (key index i, value index j) under beta = 0 and no
    decay puts q_i in output position j of head h before the norm."""
    d = dict(Hk=16, Hv=48, Dk=128, Dv=128)
    inp = _gdn_inputs(**d)
    inp["a_log"] = np.full(48, -1e4)
    C = 2 * 16 * 128 + 48 * 128
    nv = 48 * 128
    inp["u"][C + nv:C + nv + 48] = -800.0
    inp["norm_w"] = np.ones(128)
    inp["u"][C:C + nv] = 40.0                       # silu(z) the same positive constant everywhere
    h, i, j = 29, 5, 77
    inp["S"] = np.zeros((48, 128, 128))
    inp["S"][h, j, i] = 1.0                          # value-major storage: S[h][dv][dk]
    out, _, _ = _run(inp, d)
    oh = out[h * 128:(h + 1) * 128]
    nz = np.nonzero(np.abs(oh) > 1e-9)[0]
    assert list(nz) == [j]


# ------------------------------------------------------------------ attention

SA = dict(Hq=4, Hkv=2, D=8, R=4, theta=10000.0)


def _attn_inputs(Hq, Hkv, D, cap=6):
    u = rng.normal(size=Hq * 2 * D + 2 * Hkv * D)
    return dict(u=u, qw=rng.normal(size=D) * 0.3, kw=rng.normal(size=D) * 0.3,
                kc=np.zeros((Hkv, cap, D)), vc=np.zeros((Hkv, cap, D)))


def _rms1pw(x, w):
    return x / np.sqrt(np.mean(x * x) + 1e-6) * (1.0 + w)


def test_attn_first_position_returns_gated_value():
    """pos = 0: one key, softmax weight 1, so o_h = v_g * sigmoid(gate_h) with
    g = h // (Hq/Hkv); v is not normalised."""
    Hq, Hkv, D = SA["Hq"], SA["Hkv"], SA["D"]
    inp = _attn_inputs(Hq, Hkv, D)
    out, kc, vc = oracle.attn_step(inp["u"], inp["qw"], inp["kw"], inp["kc"], inp["vc"], 0, **SA)
    v = inp["u"][Hq * 2 * D + Hkv * D:].reshape(Hkv, D)
    for h in range(Hq):
        gate = inp["u"][h * 2 * D + D:(h + 1) * 2 * D]
        np.testing.assert_allclose(out[h * D:(h + 1) * D], v[h // (Hq // Hkv)] * sig(gate),
                                   rtol=1e-14)
    assert np.array_equal(vc[:, 0], v)


@pytest.mark.parametrize("pos", [0, 3, 5])
def test_attn_rotary_pairs_and_frequencies(pos):
    """The cached key is rope(rmsnorm(k) (1 + w)): pairs (i, i + R/2) rotated by
    pos * theta^(-2i/R); dims from R on only normalised."""
    Hq, Hkv, D, R, th = SA["Hq"], SA["Hkv"], SA["D"], SA["R"], SA["theta"]
    inp = _attn_inputs(Hq, Hkv, D)
    _, kc, _ = oracle.attn_step(inp["u"], inp["qw"], inp["kw"], inp["kc"], inp["vc"], pos, **SA)
    k = inp["u"][Hq * 2 * D:Hq * 2 * D + Hkv * D].reshape(Hkv, D)
    for g in range(Hkv):
        kn = _rms1pw(k[g], inp["kw"])
        exp = kn.copy()
        for i in range(R // 2):
            ang = pos * th ** (-2.0 * i / R)
            exp[i] = kn[i] * math.cos(ang) - kn[i + R // 2] * math.sin(ang)
            exp[i + R // 2] = kn[i + R // 2] * math.cos(ang) + kn[i] * math.sin(ang)
        np.testing.assert_allclose(kc[g, pos], exp, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(kc[g, pos, R:], kn[R:], rtol=1e-15)


def test_attn_equal_keys_average_values():
    """No rotary (R = 0), the same key at two positions: equal scores, so the
    output is the mean of the two values, gated."""
    Hq, Hkv, D = 4, 2, 8
    inp = _attn_inputs(Hq, Hkv, D)
    u0 = inp["u"].copy()
    u1 = inp["u"].copy()
    off = Hq * 2 * D + Hkv * D
    u1[off:] = rng.normal(size=Hkv * D)             # new values, same keys
    kw = dict(Hq=Hq, Hkv=Hkv, D=D, R=0, theta=1e7)
    _, kc, vc = oracle.attn_step(u0, inp["qw"], inp["kw"], inp["kc"], inp["vc"], 0, **kw)
    out, _, _ = oracle.attn_step(u1, inp["qw"], inp["kw"], kc, vc, 1, **kw)
    v0, v1 = u0[off:].reshape(Hkv, D), u1[off:].reshape(Hkv, D)
    for h in range(Hq):
        gate = u1[h * 2 * D + D:(h + 1) * 2 * D]
        g = h // (Hq // Hkv)
        np.testing.assert_allclose(out[h * D:(h + 1) * D], (v0[g] + v1[g]) / 2 * sig(gate),
                                   rtol=1e-13)


def test_attn_softmax_scale_and_one_plus_w_norm():
    """Two positions with different keys: o = softmax(q.k_t / sqrt(D)) over t;
    and with w = -1 the (1 + w) norm zeroes q, giving the plain mean."""
    Hq, Hkv, D = 2, 1, 16
    kw = dict(Hq=Hq, Hkv=Hkv, D=D, R=0, theta=1e7)
    inp = _attn_inputs(Hq, Hkv, D)
    off = Hq * 2 * D
    u1 = inp["u"].copy()
    u1[off:] = rng.normal(size=2 * Hkv * D)
    _, kc, vc = oracle.attn_step(inp["u"], inp["qw"], inp["kw"], inp["kc"], inp["vc"], 0, **kw)
    out, kc2, vc2 = oracle.attn_step(u1, inp["qw"], inp["kw"], kc, vc, 1, **kw)
    for h in range(Hq):
        q = _rms1pw(u1[h * 2 * D:h * 2 * D + D], inp["qw"])
        s = np.array([q @ kc2[0, t] for t in range(2)]) / math.sqrt(D)
        p = np.exp(s - s.max())
        p /= p.sum()
        gate = u1[h * 2 * D + D:(h + 1) * 2 * D]
        np.testing.assert_allclose(out[h * D:(h + 1) * D], (p[0] * vc2[0, 0] + p[1] * vc2[0, 1])
                                   * sig(gate), rtol=1e-12)
    out0, _, _ = oracle.attn_step(u1, np.full(D, -1.0), inp["kw"], kc, vc, 1, **kw)
    for h in range(Hq):
        gate = u1[h * 2 * D + D:(h + 1) * 2 * D]
        np.testing.assert_allclose(out0[h * D:(h + 1) * D], (vc2[0, 0] + vc2[0, 1]) / 2 * sig(gate),
                                   rtol=1e-13)


def test_attn_model_dims_gqa_mapping():
    """At the model's sizes (24 query heads, 4 key/value heads of 256, rotary
    64, theta 1e7), pos 0: query head h returns value head h // 6."""
    D, Hq, Hkv = 256, 24, 4
    u = rng.normal(size=Hq * 2 * D + 2 * Hkv * D)
    off = Hq * 2 * D + Hkv * D
    for g in range(Hkv):
        u[off + g * D:off + (g + 1) * D] = g + 1.0
    for h in range(Hq):
        u[h * 2 * D + D:(h + 1) * 2 * D] = 40.0     # gate open
    out, _, _ = oracle.attn_step(u, np.zeros(D), np.zeros(D), np.zeros((Hkv, 4, D)),
                                 np.zeros((Hkv, 4, D)), 0)
    for h in range(Hq):
        np.testing.assert_allclose(out[h * D:(h + 1) * D], h // 6 + 1.0, rtol=1e-15)
