"""Token mixers on the GPU (q4k_gdn_step, q4k_attn_step) against the double
oracle (oracle/mixer_oracle.c), at the model's sizes.

Bars (f32 kernels against the double oracle on the same f32 inputs):
  * state, conv state, caches: |x - x_ref| <= 2e-5 * (|x_ref| + rms(x_ref))
    elementwise — the dot products behind them are 128/256-term f32 sums;
  * outputs: per head, |y - y_ref| <= 2e-4 * max|y_ref of that head| and the
    head's cosine >= 0.999999 — a head's output is a normalised or
    softmax-weighted vector, whose f32 error is a small multiple of 2^-24
    times its largest element;
  * several tokens in a row: every step teacher-forced (the oracle starts
    from the GPU's own state of the previous step), plus the free-running
    chain at the end within ten times the one-step bar.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import down, note, require_gpu, up

pytestmark = pytest.mark.gpu
Hk, Hv, D = 16, 48, 128
C = (2 * Hk + Hv) * D
NU = C + Hv * D + 2 * Hv


@pytest.fixture(scope="module")
def torch():
    return require_gpu()


@pytest.fixture(scope="module")
def q4k(torch):
    import bit_block_quantized_gguf_amd as q4k
    return q4k


def _n(k, n, s=1.0):
    return (s * synth.normal(synth.key(16, k), n)).astype(np.float32)


def _close(got, ref, rel, what):
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    scale = np.abs(ref) + np.sqrt(np.mean(ref * ref))
    bad = np.abs(got - ref) > rel * scale
    assert not bad.any(), "%s: %d outside, worst %.3g" % (
        what, int(bad.sum()), float(np.max(np.abs(got - ref) / np.maximum(scale, 1e-30))))


def _heads(got, ref, nh, rel, what):
    got = np.asarray(got, np.float64).reshape(nh, -1)
    ref = np.asarray(ref, np.float64).reshape(nh, -1)
    for h in range(nh):
        m = np.max(np.abs(ref[h]))
        err = np.max(np.abs(got[h] - ref[h]))
        assert err <= rel * m, "%s head %d: err %.3g of max %.3g" % (what, h, err, m)
        c = got[h] @ ref[h] / (np.linalg.norm(got[h]) * np.linalg.norm(ref[h]))
        assert c >= 0.999999, "%s head %d cosine %.9f" % (what, h, c)


def _gdn_params():
    return dict(conv_w=_n(1, 4 * C, 0.5), a_log=_n(2, Hv, 0.5), dt_bias=_n(3, Hv, 0.5),
                norm_w=(1.0 + 0.1 * _n(4, D)).astype(np.float32))


@pytest.mark.parametrize("steps", [1, 6])
def test_gdn_steps_match_oracle(q4k, steps):
    prm = _gdn_params()
    dprm = {k: up(v) for k, v in prm.items()}
    cs = _n(5, 3 * C)
    S = _n(6, Hv * D * D, 0.05)
    cs_d, S_d = up(cs), up(S)
    cs_free, S_free = cs.astype(np.float64), S.astype(np.float64)
    note("gdn %d steps" % steps)
    for t in range(steps):
        u = _n(100 + t, NU)
        cs_prev, S_prev = down(cs_d).copy(), down(S_d).copy()
        out = down(q4k.gdn_step(up(u), dprm["conv_w"], dprm["a_log"], dprm["dt_bias"],
                                dprm["norm_w"], cs_d, S_d))
        ref, cs_ref, S_ref = oracle.gdn_step(u, prm["conv_w"], prm["a_log"], prm["dt_bias"],
                                             prm["norm_w"], cs_prev, S_prev)
        _close(down(cs_d), cs_ref, 0.0, "conv state step %d" % t)     # a shift: exact
        _close(down(S_d), S_ref, 2e-5, "state step %d" % t)
        _heads(out, ref, Hv, 2e-4, "gdn out step %d" % t)
        free, cs_free, S_free = oracle.gdn_step(u, prm["conv_w"], prm["a_log"], prm["dt_bias"],
                                                prm["norm_w"], cs_free, S_free)
    _close(down(S_d), S_free, 2e-4, "state after %d free-running steps" % steps)
    _heads(out, free, Hv, 2e-3, "gdn out after %d free-running steps" % steps)


def test_gdn_deterministic_and_counters_cleared(q4k, torch):
    """A head's 128 state rows are split over four workgroups; the last to
    arrive applies the norm, and the last reader of a key head's q and k
    channels shifts their conv state: two runs of the same steps give the
    same bits, and every call leaves the workspace's arrival counters at
    zero."""
    prm = _gdn_params()
    dprm = {k: up(v) for k, v in prm.items()}
    ws = q4k.Workspace(q4k.workspace_size(q4k.OP_GDN_STEP, Hk, Hv, 0))
    runs = []
    for _ in range(2):
        cs_d, S_d = up(_n(5, 3 * C)), up(_n(6, Hv * D * D, 0.05))
        outs = []
        for t in range(3):
            o = q4k.gdn_step(up(_n(100 + t, NU)), dprm["conv_w"], dprm["a_log"],
                             dprm["dt_bias"], dprm["norm_w"], cs_d, S_d, ws=ws)
            outs.append(down(o).copy())
            cnt = ws.tensor[:4 * (Hv + Hk)].cpu().numpy()
            assert not cnt.any(), "arrival counters left non-zero"
        runs.append((outs, down(S_d).copy()))
    for a, b in zip(runs[0][0], runs[1][0]):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(runs[0][1].view(np.uint32), runs[1][1].view(np.uint32))


def test_gdn_zero_state_first_token(q4k):
    """From a zero state and zero conv state the first token's state is the
    rank-1 beta k v^T of every head."""
    prm = _gdn_params()
    dprm = {k: up(v) for k, v in prm.items()}
    cs = np.zeros(3 * C, np.float32)
    S = np.zeros(Hv * D * D, np.float32)
    u = _n(200, NU)
    cs_d, S_d = up(cs), up(S)
    out = down(q4k.gdn_step(up(u), dprm["conv_w"], dprm["a_log"], dprm["dt_bias"],
                            dprm["norm_w"], cs_d, S_d))
    ref, _, S_ref = oracle.gdn_step(u, prm["conv_w"], prm["a_log"], prm["dt_bias"],
                                    prm["norm_w"], cs, S)
    _close(down(S_d), S_ref, 2e-5, "state")
    _heads(out, ref, Hv, 2e-4, "gdn out")
    Sg = down(S_d).reshape(Hv, D, D).astype(np.float64)
    for h in (0, 17, 47):
        sv = np.linalg.svd(Sg[h], compute_uv=False)
        assert sv[1] <= 1e-6 * sv[0]


Hq, Hkv, AD, R = 24, 4, 256, 64
NA = Hq * 2 * AD + 2 * Hkv * AD


def _attn_params():
    return dict(qw=(0.2 * _n(10, AD)).astype(np.float32), kw=(0.2 * _n(11, AD)).astype(np.float32))


def test_attn_sequence_matches_oracle(q4k, torch):
    """Positions 0..39: every step teacher-forced from the GPU's caches."""
    prm = _attn_params()
    cap = 48
    kc = torch.zeros((Hkv, cap, AD), device="cuda")
    vc = torch.zeros((Hkv, cap, AD), device="cuda")
    qw, kw = up(prm["qw"]), up(prm["kw"])
    note("attention positions 0..39")
    for pos in range(40):
        u = _n(300 + pos, NA)
        kc_prev, vc_prev = down(kc).copy(), down(vc).copy()
        out = down(q4k.attn_step(up(u), qw, kw, kc, vc, pos))
        ref, kc_ref, vc_ref = oracle.attn_step(u, prm["qw"], prm["kw"], kc_prev, vc_prev, pos)
        _close(down(kc)[:, pos], kc_ref[:, pos], 2e-5, "k cache pos %d" % pos)
        assert np.array_equal(down(vc)[:, pos], vc_ref[:, pos].astype(np.float32))
        _heads(out, ref, Hq, 2e-4, "attn out pos %d" % pos)


def test_attn_long_context(q4k, torch):
    """One step at position 1500 over caches filled with random keys/values."""
    prm = _attn_params()
    cap, pos = 1600, 1500
    kc_h = _n(400, Hkv * cap * AD).reshape(Hkv, cap, AD)
    vc_h = _n(401, Hkv * cap * AD).reshape(Hkv, cap, AD)
    kc, vc = up(kc_h), up(vc_h)
    u = _n(402, NA)
    note("attention at position %d" % pos)
    out = down(q4k.attn_step(up(u), up(prm["qw"]), up(prm["kw"]), kc, vc, pos))
    ref, kc_ref, _ = oracle.attn_step(u, prm["qw"], prm["kw"], kc_h, vc_h, pos)
    _heads(out, ref, Hq, 2e-4, "attn out long")
    _close(down(kc)[:, pos], kc_ref[:, pos], 2e-5, "k cache long")


def test_attn_deterministic(q4k, torch):
    prm = _attn_params()
    cap = 8
    u = up(_n(500, NA))
    outs = []
    for _ in range(2):
        kc = torch.zeros((Hkv, cap, AD), device="cuda")
        vc = torch.zeros((Hkv, cap, AD), device="cuda")
        for pos in range(5):
            o = q4k.attn_step(u, up(prm["qw"]), up(prm["kw"]), kc, vc, pos)
        outs.append(down(o).copy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


@pytest.mark.parametrize("pos", [63, 64, 4160, 8199])
def test_attn_split_kv_chunks(q4k, torch, pos):
    """Capacity 8200 gives 64 chunk workgroups over up to 129 chunks of 64
    positions: one partial chunk (63), a chunk of one position (64), two
    chunks for the first workgroups (4160), three with a ragged tail (8199)."""
    prm = _attn_params()
    cap = 8200
    kc_h = _n(600, Hkv * cap * AD).reshape(Hkv, cap, AD)
    vc_h = _n(601, Hkv * cap * AD).reshape(Hkv, cap, AD)
    kc, vc = up(kc_h), up(vc_h)
    u = _n(602 + pos, NA)
    note("attention split-KV at position %d of %d" % (pos, cap))
    out = down(q4k.attn_step(up(u), up(prm["qw"]), up(prm["kw"]), kc, vc, pos))
    ref, kc_ref, vc_ref = oracle.attn_step(u, prm["qw"], prm["kw"], kc_h, vc_h, pos)
    _heads(out, ref, Hq, 2e-4, "attn out pos %d" % pos)
    _close(down(kc)[:, pos], kc_ref[:, pos], 2e-5, "k cache pos %d" % pos)
    assert np.array_equal(down(vc)[:, pos], vc_ref[:, pos].astype(np.float32))
    # rows other than pos are untouched
    kd = down(kc)
    assert np.array_equal(np.delete(kd, pos, axis=1),
                          np.delete(kc_h.astype(np.float32), pos, axis=1))


@pytest.mark.parametrize("hq,hkv", [(4, 4), (16, 2), (40, 2)])
def test_attn_head_groups(q4k, torch, hq, hkv):
    """Query heads per key/value head of 1, exactly one group of 8, and 20
    (groups of 8, 8 and 4)."""
    prm = _attn_params()
    cap, pos = 330, 321
    na = hq * 2 * AD + 2 * hkv * AD
    kc_h = _n(700, hkv * cap * AD).reshape(hkv, cap, AD)
    vc_h = _n(701, hkv * cap * AD).reshape(hkv, cap, AD)
    kc, vc = up(kc_h), up(vc_h)
    u = _n(702, na)
    note("attention %d query heads over %d kv heads" % (hq, hkv))
    out = down(q4k.attn_step(up(u), up(prm["qw"]), up(prm["kw"]), kc, vc, pos, q_heads=hq,
                             kv_heads=hkv))
    ref, _, _ = oracle.attn_step(u, prm["qw"], prm["kw"], kc_h, vc_h, pos, Hq=hq, Hkv=hkv)
    _heads(out, ref, hq, 2e-4, "attn out %dx%d" % (hq, hkv))


@pytest.mark.parametrize("hk,hv", [(4, 4), (2, 8), (1, 12)])
def test_gdn_head_ratios(q4k, hk, hv):
    """Value heads per key head of 1, 4 and 12 (the conv state of a key
    head's q and k channels is read by 4, 16 and 48 workgroups; the last one
    shifts it), two steps, state and conv state and outputs against the
    oracle."""
    C = (2 * hk + hv) * D
    nu = C + hv * D + 2 * hv
    prm = dict(conv_w=_n(31, 4 * C, 0.5), a_log=_n(32, hv, 0.5), dt_bias=_n(33, hv, 0.5),
               norm_w=(1.0 + 0.1 * _n(34, D)).astype(np.float32))
    dprm = {k: up(v) for k, v in prm.items()}
    cs, S = _n(35, 3 * C), _n(36, hv * D * D, 0.05)
    cs_d, S_d = up(cs), up(S)
    note("gdn heads %d/%d" % (hk, hv))
    for t in range(2):
        u = _n(800 + t, nu)
        cs_prev, S_prev = down(cs_d).copy(), down(S_d).copy()
        out = down(q4k.gdn_step(up(u), dprm["conv_w"], dprm["a_log"], dprm["dt_bias"],
                                dprm["norm_w"], cs_d, S_d, key_heads=hk, value_heads=hv))
        ref, cs_ref, S_ref = oracle.gdn_step(u, prm["conv_w"], prm["a_log"], prm["dt_bias"],
                                             prm["norm_w"], cs_prev, S_prev, Hk=hk, Hv=hv)
        _close(down(cs_d), cs_ref, 0.0, "conv state %d/%d step %d" % (hk, hv, t))
        _close(down(S_d), S_ref, 2e-5, "state %d/%d step %d" % (hk, hv, t))
        _heads(out, ref, hv, 2e-4, "gdn out %d/%d step %d" % (hk, hv, t))


@pytest.mark.parametrize("rope_dim", [0, 2, 256])
def test_attn_rope_extremes(q4k, torch, rope_dim):
    """No rotary, one rotated pair, and every dimension rotated, at a position
    whose angles wrap many times (pos 4000 of 4096: the angle reduction
    modulo 2 pi in double)."""
    prm = _attn_params()
    cap, pos = 4096, 4000
    kc_h = _n(900, Hkv * cap * AD).reshape(Hkv, cap, AD)
    vc_h = _n(901, Hkv * cap * AD).reshape(Hkv, cap, AD)
    kc, vc = up(kc_h), up(vc_h)
    u = _n(902 + rope_dim, NA)
    note("attention rope_dim %d at position %d" % (rope_dim, pos))
    out = down(q4k.attn_step(up(u), up(prm["qw"]), up(prm["kw"]), kc, vc, pos,
                             rope_dim=rope_dim))
    ref, kc_ref, _ = oracle.attn_step(u, prm["qw"], prm["kw"], kc_h, vc_h, pos, R=rope_dim)
    _heads(out, ref, Hq, 2e-4, "attn out rope_dim %d" % rope_dim)
    _close(down(kc)[:, pos], kc_ref[:, pos], 2e-5, "k cache rope_dim %d" % rope_dim)
