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
    assert lib.q4k_version() == 10000


P = 0x10000  # fake, 16-byte aligned "device" address: never dereferenced


@pytest.mark.parametrize("M,K,code", [(-1, 256, -2), (4, 0, -2), (4, 100, -2), (4, 257, -2),
                                      (4, -256, -2), (1 << 31, 256, -6)])
def test_gemv_shape_errors(lib, M, K, code):
    assert lib.q4k_gemv(P, P, P, M, K, None) == code
    assert lib.q4k_last_error()


def test_null_and_alignment_errors(lib):
    assert lib.q4k_gemv(None, P, P, 4, 256, None) == -1
    assert lib.q4k_gemv(P, None, P, 4, 256, None) == -1
    assert lib.q4k_gemv(P, P, None, 4, 256, None) == -1
    assert lib.q4k_gemv(P + 4, P, P, 4, 256, None) == -3
    assert lib.q4k_gemv(P, P + 8, P, 4, 256, None) == -3
    assert lib.q4k_dequant(P, P + 2, 4, 256, None) == -3
    assert b"aligned" in lib.q4k_last_error()
    assert lib.q4k_gemv_batch(P, P, P, 4, 256, -1, None) == -2
    assert lib.q4k_gemm(P, P, P, 4, 256, -3, None) == -2
    assert b"P must be" in lib.q4k_last_error()


def test_mlp_validation(lib):
    """q4k_mlp checks shapes, pointers, alignment and eps before any device
    work (hidden and inter must be positive multiples of 256)."""
    f = ctypes.c_float
    ok = lambda **kw: dict(dict(wg=P, wu=P, wd=P, H=512, I=768, x=P, nw=None, eps=f(1e-6),
                                r=None, y=P, act=None), **kw)
    call = lambda a: lib.q4k_mlp(a["wg"], a["wu"], a["wd"], a["H"], a["I"], a["x"], a["nw"],
                                 a["eps"], a["r"], a["y"], a["act"], None)
    for kw, code in (({"H": 500}, -2), ({"I": 0}, -2), ({"I": 100}, -2), ({"H": -256}, -2),
                     ({"wg": None}, -1), ({"wu": None}, -1), ({"wd": None}, -1),
                     ({"x": None}, -1), ({"y": None}, -1), ({"eps": f(-1.0)}, -1),
                     ({"eps": f(float("nan"))}, -1), ({"eps": f(float("inf"))}, -1),
                     ({"x": P + 4}, -3), ({"act": P + 8}, -3), ({"wd": P + 2}, -3)):
        assert call(ok(**kw)) == code, kw
        assert lib.q4k_last_error()


def test_zero_sizes_are_noops(lib):
    # nothing is enqueued and no device is touched
    assert lib.q4k_gemv(None, None, None, 0, 256, None) == 0
    assert lib.q4k_dequant(None, None, 0, 512, None) == 0
    assert lib.q4k_gemv_batch(None, None, None, 5, 256, 0, None) == 0
    assert lib.q4k_gemm(None, None, None, 5, 256, 0, None) == 0
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
    assert lib.q4k_gemv_q6_k(None, None, None, M, K, None) == code
    assert lib.q4k_last_error()


def test_gemv_q6_k_pointer_errors_and_zero_rows(lib):
    assert lib.q4k_gemv_q6_k(None, P, P, 4, 1024, None) == -1
    assert lib.q4k_gemv_q6_k(P, None, P, 4, 1024, None) == -1
    assert lib.q4k_gemv_q6_k(P, P, None, 4, 1024, None) == -1
    assert lib.q4k_gemv_q6_k(P + 8, P, P, 4, 1024, None) == -3
    assert lib.q4k_gemv_q6_k(P, P + 4, P, 4, 1024, None) == -3
    assert lib.q4k_gemv_q6_k(P, P, P + 12, 4, 1024, None) == -3
    assert lib.q4k_gemv_q6_k(None, None, None, 0, 2048, None) == 0
    assert lib.q4k_last_error() == b""
