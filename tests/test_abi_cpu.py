"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and rejects bad arguments before touching a device."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

import bit_block_quantized_gguf_amd as q4k

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4k.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(q4k_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(q4k.LIB_PATH):
        pytest.fail("libq4k.so is not built; run __graft_entry__.build()")
    return q4k.load()


def test_header_symbols_are_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", q4k.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    declared = _declared()
    assert declared, "no declarations parsed"
    missing = [s for s in declared if s not in exported]
    assert not missing, missing
    assert sorted(q4k.EXPORTS) == declared


def test_library_is_gfx950_only():
    """The offload bundle of the library names gfx950 as its only GPU target."""
    blob = open(q4k.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa--(gfx[0-9a-z]+)", blob))
    assert targets == {b"gfx950"}, targets


def test_version(lib):
    assert lib.q4k_version() == 10100


P = 0x10000  # fake, 16-byte aligned "device" address: never dereferenced
WS = 0x40000  # fake 256-byte aligned workspace address
BIG = 1 << 40  # a workspace size no call exceeds


@pytest.mark.parametrize("M,K,code", [(-1, 256, -2), (4, 0, -2), (4, 100, -2), (4, 257, -2),
                                      (4, -256, -2), (1 << 31, 256, -6), ((1 << 30) + 1, 256, -6),
                                      (4, (1 << 24) + 256, -6)])
def test_gemv_shape_errors(lib, M, K, code):
    """Shapes outside the contract, including the limits that keep the
    kernels' 32-bit in-tile offsets from wrapping (K <= 2^24, M <= 2^30)."""
    assert lib.q4k_gemv(P, P, P, M, K, WS, BIG, None) == code
    assert lib.q4k_last_error()


def test_null_and_alignment_errors(lib):
    assert lib.q4k_gemv(None, P, P, 4, 256, WS, BIG, None) == -1
    assert lib.q4k_gemv(P, None, P, 4, 256, WS, BIG, None) == -1
    assert lib.q4k_gemv(P, P, None, 4, 256, WS, BIG, None) == -1
    assert lib.q4k_gemv(P + 4, P, P, 4, 256, WS, BIG, None) == -3
    assert lib.q4k_gemv(P, P + 8, P, 4, 256, WS, BIG, None) == -3
    assert lib.q4k_dequant(P, P + 2, 4, 256, None) == -3
    assert b"aligned" in lib.q4k_last_error()
    assert lib.q4k_gemv_batch(P, P, P, 4, 256, -1, WS, BIG, None) == -2
    assert lib.q4k_gemm(P, P, P, 4, 256, -3, WS, BIG, None) == -2
    assert b"P must be" in lib.q4k_last_error()


def test_mlp_validation(lib):
    """q4k_mlp checks shapes, pointers, alignment and eps before any device
    work (hidden and inter must be positive multiples of 256)."""
    f = ctypes.c_float
    ok = lambda **kw: dict(dict(wg=P, wu=P, wd=P, H=512, I=768, x=P, nw=None, eps=f(1e-6),
                                r=None, y=P, act=None), **kw)
    call = lambda a: lib.q4k_mlp(a["wg"], a["wu"], a["wd"], a["H"], a["I"], a["x"], a["nw"],
                                 a["eps"], a["r"], a["y"], a["act"], WS, BIG, None)
    for kw, code in (({"H": 500}, -2), ({"I": 0}, -2), ({"I": 100}, -2), ({"H": -256}, -2),
                     ({"wg": None}, -1), ({"wu": None}, -1), ({"wd": None}, -1),
                     ({"x": None}, -1), ({"y": None}, -1), ({"eps": f(-1.0)}, -1),
                     ({"eps": f(float("nan"))}, -1), ({"eps": f(float("inf"))}, -1),
                     ({"x": P + 4}, -3), ({"act": P + 8}, -3), ({"wd": P + 2}, -3)):
        assert call(ok(**kw)) == code, kw
        assert lib.q4k_last_error()


def test_zero_sizes_are_noops(lib):
    # nothing is enqueued and no device is touched
    assert lib.q4k_gemv(None, None, None, 0, 256, None, 0, None) == 0
    assert lib.q4k_dequant(None, None, 0, 512, None) == 0
    assert lib.q4k_gemv_batch(None, None, None, 5, 256, 0, None, 0, None) == 0
    assert lib.q4k_gemm(None, None, None, 5, 256, 0, None, 0, None) == 0
    assert lib.q4k_last_error() == b""


def test_stack_create_validation(lib):
    out = ctypes.c_void_p()
    assert lib.q4k_decode_stack_create(None, None, ctypes.byref(out)) == -1
    mk = lambda M, K: q4k.MatDesc(P, M, K)
    L = (q4k.LayerDesc * 1)()
    L[0].mix_in, L[0].mix_out = mk(768, 512), mk(512, 512)
    L[0].gate, L[0].up, L[0].down = mk(1024, 512), mk(1024, 512), mk(512, 1024)
    d = q4k.StackDesc(512, 1, L, mk(300, 512), 1e-6, 0)
    bad = [
        ("flags", lambda d: setattr(d, "flags", 1), -1),
        ("hidden", lambda d: setattr(d, "hidden", 500), -2),
        ("mixout", lambda d: setattr(L[0], "mix_out", mk(512, 1024)), -2),
        ("down", lambda d: setattr(L[0], "down", mk(512, 768)), -2),
        ("lm", lambda d: setattr(d, "lm_head", mk(300, 256)), -2),
        ("align", lambda d: setattr(L[0], "gate", q4k.MatDesc(P + 4, 1024, 512)), -3),
    ]
    for name, mut, code in bad:
        L[0].mix_in, L[0].mix_out = mk(768, 512), mk(512, 512)
        L[0].gate, L[0].up, L[0].down = mk(1024, 512), mk(1024, 512), mk(512, 1024)
        d = q4k.StackDesc(512, 1, L, mk(300, 512), 1e-6, 0)
        mut(d)
        assert lib.q4k_decode_stack_create(ctypes.byref(d), None, ctypes.byref(out)) == code, name
        assert not out.value
    lib.q4k_decode_stack_destroy(None)  # NULL-safe


def test_stack_entry_points_reject_null(lib):
    n = ctypes.c_int64()
    ptr = ctypes.c_void_p()
    assert lib.q4k_decode_stack(None, P, P, None) == -1
    assert lib.q4k_decode_stack_buffer(None, 0, 0, ctypes.byref(ptr), ctypes.byref(n)) == -1
    assert lib.q4k_decode_stack_nodes(None, ctypes.byref(n)) == -1


def test_launch_shape_reports(lib):
    for (M, K) in [(17408, 5120), (5120, 17408), (5120, 6144), (16480, 5120), (248320, 5120),
                   (512, 1024), (1024, 512), (1, 256)]:
        wk, groups = q4k.gemv_config(M, K, 1)
        units = -(-M // 64) * -(-(K // 256) // 4)
        assert wk == 4 and 1 <= groups <= units
    tt, wg = q4k.gemm_config(5120, 17408, 256)
    assert tt in (32, 64, 128, 256) and wg >= 1


def test_tuning_knobs_validate(lib):
    assert lib.q4k_tune_gemv(3, 0) == -1
    assert lib.q4k_tune_gemv(8, 0) == -1
    assert lib.q4k_tune_gemv(4, -1) == -1
    assert lib.q4k_tune_gemm(0, -1) == -1
    assert lib.q4k_tune_gemm(0, 4097) == -1
    assert lib.q4k_tune_gemm(96, 0) == -1
    q4k.tune_gemm(32, 0)
    assert q4k.gemm_config(17408, 5120, 22)[0] == 32
    q4k.tune_gemm(64, 0)
    assert q4k.gemm_config(17408, 5120, 22)[0] == 64
    q4k.tune_gemm(256, 3)
    assert q4k.gemm_config(17408, 5120, 512) == (256, 3)
    q4k.tune_gemm(128, 0)
    assert q4k.gemm_config(17408, 5120, 512)[0] == 128
    q4k.tune_gemm(256, 4096)
    assert q4k.gemm_config(300, 512, 7) == (256, 4)          # capped at tiles x super-blocks
    q4k.tune_gemv(4, 300)
    assert q4k.gemv_config(17408, 5120) == (4, 300)
    q4k.tune_gemv(0, 5000)
    assert q4k.gemv_config(17408, 5120) == (4, 1360)   # at most one workgroup per unit
    q4k.tune_gemv(0, 0)
    q4k.tune_gemm(0, 0)


def test_product_path_has_no_oracle_or_fallback():
    """The package never imports the CPU reference and has no CPU fallback."""
    pkg = os.path.join(ROOT, "bit_block_quantized_gguf_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "liboracle" not in text, f
                assert "q4k_oracle" not in text, f


@pytest.mark.parametrize("M,K,code", [(-1, 1024, -2), (4, 0, -2), (4, 256, -2), (4, 512, -2),
                                      (4, 1280, -2), (4, 1000, -2), (1 << 31, 1024, -6)])
def test_gemv_q6_k_shape_errors(lib, M, K, code):
    """K must be a positive multiple of 1024 (rows of a multiple of four
    210-byte blocks); checked before the pointers and the device."""
    assert lib.q4k_gemv_q6_k(None, None, None, M, K, WS, BIG, None) == code
    assert lib.q4k_last_error()


def test_gemv_q6_k_pointer_errors_and_zero_rows(lib):
    assert lib.q4k_gemv_q6_k(None, P, P, 4, 1024, WS, BIG, None) == -1
    assert lib.q4k_gemv_q6_k(P, None, P, 4, 1024, WS, BIG, None) == -1
    assert lib.q4k_gemv_q6_k(P, P, None, 4, 1024, WS, BIG, None) == -1
    assert lib.q4k_gemv_q6_k(P + 8, P, P, 4, 1024, WS, BIG, None) == -3
    assert lib.q4k_gemv_q6_k(P, P + 4, P, 4, 1024, WS, BIG, None) == -3
    assert lib.q4k_gemv_q6_k(P, P, P + 12, 4, 1024, WS, BIG, None) == -3
    assert lib.q4k_gemv_q6_k(None, None, None, 0, 2048, None, 0, None) == 0
    assert lib.q4k_last_error() == b""


# ---------------------------------------------------------------- workspaces

OPS = [(q4k.OP_GEMV, 17408, 5120, 1), (q4k.OP_GEMV_BATCH, 17408, 5120, 16),
       (q4k.OP_GEMM, 5120, 17408, 1024), (q4k.OP_GEMV_Q8_0, 248320, 5120, 1),
       (q4k.OP_GEMV_Q6_K, 5120, 17408, 1), (q4k.OP_MLP, 17408, 5120, 0)]


@pytest.mark.parametrize("op,M,K,N", OPS)
def test_workspace_size_reports(lib, op, M, K, N):
    n = q4k.workspace_size(op, M, K, N)
    assert n > 0 and n % 256 == 0


def test_workspace_size_errors(lib):
    n = ctypes.c_size_t(7)
    assert lib.q4k_workspace_size(99, 4, 256, 1, ctypes.byref(n)) == -1
    assert lib.q4k_workspace_size(q4k.OP_GEMV, 4, 256, 1, None) == -1
    assert lib.q4k_workspace_size(q4k.OP_GEMV, 4, 100, 1, ctypes.byref(n)) == -2
    assert lib.q4k_workspace_size(q4k.OP_GEMV_Q6_K, 4, 512, 1, ctypes.byref(n)) == -2
    assert lib.q4k_workspace_size(q4k.OP_GEMV_BATCH, 4, 256, -1, ctypes.byref(n)) == -2
    assert lib.q4k_workspace_size(q4k.OP_GEMV, 0, 256, 1, ctypes.byref(n)) == 0 and n.value == 0
    # the batch needs at least the single-vector workspace and grows with N
    one = q4k.workspace_size(q4k.OP_GEMV_BATCH, 4096, 5120, 1)
    assert one == q4k.workspace_size(q4k.OP_GEMV, 4096, 5120)
    assert q4k.workspace_size(q4k.OP_GEMV_BATCH, 4096, 5120, 16) > one
    # the GEMM's workspace holds the bf16 copy of X: grows with P
    assert (q4k.workspace_size(q4k.OP_GEMM, 5120, 5120, 1024)
            > q4k.workspace_size(q4k.OP_GEMM, 5120, 5120, 256) >= 256 * 5120 * 2)


@pytest.mark.parametrize("op,M,K,N", OPS)
def test_workspace_checked_before_any_device_work(lib, op, M, K, N):
    """A NULL, misaligned or too small workspace is rejected before the
    device is touched (also here, with no GPU)."""
    need = q4k.workspace_size(op, M, K, N)
    f = ctypes.c_float(1e-6)

    def call(ws, nbytes):
        if op == q4k.OP_GEMV:
            return lib.q4k_gemv(P, P, P, M, K, ws, nbytes, None)
        if op == q4k.OP_GEMV_BATCH:
            return lib.q4k_gemv_batch(P, P, P, M, K, N, ws, nbytes, None)
        if op == q4k.OP_GEMM:
            return lib.q4k_gemm(P, P, P, M, K, N, ws, nbytes, None)
        if op == q4k.OP_GEMV_Q8_0:
            return lib.q4k_gemv_q8_0(P, P, P, M, K, ws, nbytes, None)
        if op == q4k.OP_GEMV_Q6_K:
            return lib.q4k_gemv_q6_k(P, P, P, M, K, ws, nbytes, None)
        return lib.q4k_mlp(P, P, P, K, M, P, None, f, None, P, None, ws, nbytes, None)

    assert call(None, need) == -1 and b"NULL" in lib.q4k_last_error()
    assert call(WS, need - 256) == -1 and b"workspace" in lib.q4k_last_error()
    assert call(WS + 128, need) == -3
    # with a large enough workspace the call gets as far as the device check
    assert call(WS, need) not in (-1, -2, -3)


# ---------------------------------------------------------------- binding checks

def test_binding_checks_sizes_before_the_device():
    """The binding checks the element count of every input and output (an
    undersized tensor would make a kernel write past it) before anything
    else; on this GPU-less host a correctly sized CPU tensor then fails the
    device check instead."""
    torch = pytest.importorskip("torch")
    f32, u8 = torch.float32, torch.uint8
    w = torch.zeros(64 * 2 * 144, dtype=u8)               # 64 x 512 Q4_K
    x, y = torch.zeros(512, dtype=f32), torch.zeros(64, dtype=f32)

    def raises(msg, fn):
        with pytest.raises((ValueError, TypeError)) as e:
            fn()
        assert msg in str(e.value), str(e.value)

    raises("w holds", lambda: q4k.gemv(w[:-1], x, y, M=64, K=512))
    raises("x has 511", lambda: q4k.gemv(w, x[:-1], y, M=64, K=512))
    raises("y has 63", lambda: q4k.gemv(w, x, y[:-1], M=64, K=512))
    raises("device", lambda: q4k.gemv(w, x, y, M=64, K=512))
    raises("out has", lambda: q4k.dequant(w, 64, 512, out=torch.zeros(64 * 511, dtype=f32)))
    X = torch.zeros((3, 512), dtype=f32)
    raises("Y has", lambda: q4k.gemv_batch(w, X, torch.zeros((3, 63), dtype=f32), M=64, K=512))
    raises("X must be", lambda: q4k.gemv_batch(w, torch.zeros((3, 500), dtype=f32), M=64, K=512))
    raises("Y has", lambda: q4k.gemm(w, X, torch.zeros((2, 64), dtype=f32), M=64, K=512))
    wq8 = torch.zeros(64 * 16 * 34, dtype=u8)
    raises("y has", lambda: q4k.gemv_q8_0(wq8, x, y[:10], M=64, K=512))
    wq6 = torch.zeros(64 * 4 * 210, dtype=u8)
    raises("x has", lambda: q4k.gemv_q6_k(wq6, torch.zeros(1000, dtype=f32), M=64, K=1024))
    wg = torch.zeros(256 * 2 * 144, dtype=u8)             # 256 x 512
    wd = torch.zeros(512 * 1 * 144, dtype=u8)             # 512 x 256
    h = torch.zeros(512, dtype=f32)
    for kw, msg in (({"y": torch.zeros(511, dtype=f32)}, "y has"),
                    ({"resid": torch.zeros(100, dtype=f32)}, "resid has"),
                    ({"norm_w": torch.zeros(513, dtype=f32)}, "norm_w has"),
                    ({"act": torch.zeros(255, dtype=f32)}, "act has")):
        raises(msg, lambda: q4k.mlp(wg, wg, wd, h, hidden=512, inter=256, **kw))


# ---------------------------------------------------------------- token mixers

def test_gdn_step_validation(lib):
    ok = dict(key_heads=16, value_heads=48, key_dim=128, value_dim=128, eps=1e-6,
              conv_w=P, a_log=P, dt_bias=P, norm_w=P)
    need = q4k.workspace_size(q4k.OP_GDN_STEP, 16, 48)
    # counter region (arrival counters per value head and per key head) and
    # the heads' outputs before their norm
    assert need >= 65536 + 48 * 128 * 4

    def call(ws=WS, nbytes=need, u=P, **kw):
        prm = q4k.GdnParams(**dict(ok, **kw))
        return lib.q4k_gdn_step(ctypes.byref(prm), u, P, P, P, ws, nbytes, None)

    assert lib.q4k_gdn_step(None, P, P, P, P, WS, need, None) == -1
    for kw, code in (({"value_heads": 40}, -2), ({"key_heads": 0}, -2), ({"key_dim": 64}, -2),
                     ({"value_dim": 256}, -2), ({"eps": -1.0}, -1), ({"eps": float("nan")}, -1),
                     ({"conv_w": None}, -1), ({"norm_w": P + 4}, -3), ({"u": None}, -1),
                     ({"u": P + 8}, -3), ({"ws": None}, -1), ({"nbytes": need - 256}, -1),
                     ({"ws": WS + 16}, -3)):
        assert call(**kw) == code, kw
        assert lib.q4k_last_error()
    assert call() not in (-1, -2, -3)   # valid: gets as far as the device check


def test_attn_step_validation(lib):
    ok = dict(q_heads=24, kv_heads=4, head_dim=256, rope_dim=64, rope_theta=1e7, eps=1e-6,
              q_norm_w=P, k_norm_w=P)
    need = q4k.workspace_size(q4k.OP_ATTN_STEP, 24, 4, 64)
    # one partial (256 outputs, max, sum) per head slot of every chunk
    # workgroup: 4 kv heads x 8 query-head slots at one chunk (capacity 64)
    assert need >= 4 * 8 * 258 * 4
    # the split-KV partials grow with the capacity until 64 chunk workgroups
    assert q4k.workspace_size(q4k.OP_ATTN_STEP, 24, 4, 4096) > need
    assert (q4k.workspace_size(q4k.OP_ATTN_STEP, 24, 4, 4096)
            == q4k.workspace_size(q4k.OP_ATTN_STEP, 24, 4, 1 << 20))
    for M, K, N in ((25, 4, 64), (24, 0, 64), (24, 4, 0)):
        with pytest.raises(q4k.Q4KError):
            q4k.workspace_size(q4k.OP_ATTN_STEP, M, K, N)

    def call(cap=64, pos=3, u=P, kc=P, ws=WS, nbytes=need, **kw):
        prm = q4k.AttnParams(**dict(ok, **kw))
        return lib.q4k_attn_step(ctypes.byref(prm), u, kc, P, cap, pos, P, ws, nbytes, None)

    assert lib.q4k_attn_step(None, P, P, P, 64, 0, P, WS, need, None) == -1
    for kw, code in (({"head_dim": 128}, -2), ({"q_heads": 25}, -2), ({"kv_heads": 0}, -2),
                     ({"rope_dim": 63}, -2), ({"rope_dim": 258}, -2), ({"pos": 64}, -2),
                     ({"pos": -1}, -2), ({"cap": 0}, -2), ({"rope_theta": 0.0}, -1),
                     ({"u": None}, -1), ({"kc": P + 4}, -3), ({"q_norm_w": None}, -1),
                     ({"ws": None}, -1), ({"nbytes": need - 256}, -1), ({"ws": WS + 16}, -3),
                     ({"cap": 4096, "pos": 5}, -1)):
        assert call(**kw) == code, kw
        assert lib.q4k_last_error()
    assert call() not in (-1, -2, -3)


def test_stack_create_validation_with_mixers(lib):
    """With Q4K_STACK_MIXERS the plan checks each layer's mixer sizes against
    its projections and the KV-cache capacity before touching a device."""
    out = ctypes.c_void_p()
    mk = lambda M, K: q4k.MatDesc(P, M, K)
    L = (q4k.LayerDesc * 2)()
    gdn_in = (2 * 2 + 2 * 4) * 128 + 8           # Hk = 2, Hv = 4
    att_in = (2 * 2 + 2 * 1) * 256               # Hq = 2, Hkv = 1

    def layers():
        L[0].kind, L[1].kind = 0, 1
        L[0].mix_in, L[0].mix_out = mk(gdn_in, 512), mk(512, 512)
        L[1].mix_in, L[1].mix_out = mk(att_in, 512), mk(512, 512)
        for l in (0, 1):
            L[l].gate, L[l].up, L[l].down = mk(1024, 512), mk(1024, 512), mk(512, 1024)

    mx = (q4k.MixerDesc * 2)()

    def mixers():
        mx[0].gdn = q4k.GdnParams(2, 4, 128, 128, 1e-6, P, P, P, P)
        mx[1].attn = q4k.AttnParams(2, 1, 256, 64, 1e7, 1e-6, P, P)

    bad = [
        ("flags", lambda d: setattr(d, "flags", 3), -1),
        ("mixers null", lambda d: setattr(d, "mixers", None), -1),
        ("gdn in", lambda d: setattr(L[0], "mix_in", mk(gdn_in + 1, 512)), -2),
        ("attn out", lambda d: setattr(L[1], "mix_out", mk(512, 768)), -2),
        ("gdn heads", lambda d: setattr(mx[0], "gdn", q4k.GdnParams(3, 4, 128, 128, 1e-6, P, P, P, P)), -2),
        ("attn dim", lambda d: setattr(mx[1], "attn", q4k.AttnParams(2, 1, 128, 64, 1e7, 1e-6, P, P)), -2),
        ("gdn ptr", lambda d: setattr(mx[0], "gdn", q4k.GdnParams(2, 4, 128, 128, 1e-6, None, P, P, P)), -1),
        ("capacity", lambda d: setattr(d, "attn_capacity", 0), -2),
        ("kind", lambda d: setattr(L[1], "kind", 2), -1),
    ]
    for name, mut, code in bad:
        layers()
        mixers()
        d = q4k.StackDesc(512, 2, L, mk(300, 512), 1e-6, q4k.STACK_MIXERS, mx, 16)
        mut(d)
        assert lib.q4k_decode_stack_create(ctypes.byref(d), None, ctypes.byref(out)) == code, name
        assert not out.value
    # a persistent plan takes no mixers and a non-negative poll limit
    layers()
    mixers()
    for flags, spin in ((q4k.STACK_MIXERS | q4k.STACK_PERSISTENT, 0), (q4k.STACK_PERSISTENT, -1),
                        (4, 0)):
        d = q4k.StackDesc(512, 2, L, mk(300, 512), 1e-6, flags, mx, 16, spin)
        assert lib.q4k_decode_stack_create(ctypes.byref(d), None, ctypes.byref(out)) == -1, flags
        assert not out.value
    n = ctypes.c_int64()
    st = ctypes.c_int32(7)
    assert lib.q4k_decode_stack_reset(None, None) == -1
    assert lib.q4k_decode_stack_position(None, ctypes.byref(n)) == -1
    assert lib.q4k_decode_stack_status(None, None, ctypes.byref(st)) == -1
