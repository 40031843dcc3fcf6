"""Helpers shared by the GPU parity tests: device setup, uploads, and the
comparison bars.

Bars:
  * dequantisation: bit-exact (uint32 equality, signed zeros distinct);
  * GEMV / batched GEMV: |y - y_ref| <= 1e-4 * S + 1e-6 per element with
    S = sum_k |w_ik x_k|, and cosine(y, y_ref) >= 0.999999 per vector;
  * bf16 GEMM: |y - Y_ref| <= 5e-3 * S + 1e-6 against the exact f32-input
    product, |y - Y16| <= 1e-4 * S16 + 1e-6 against the product of the
    bf16-rounded inputs (only f32 accumulation error remains), and
    cosine(y, Y16) >= 0.999999 per token row.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

GEMV_REL, GEMV_ABS = 1e-4, 1e-6
GEMM_REL = 5e-3
COS_MIN = 0.999999


def require_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_block_quantized_gguf_amd as q4k
    q4k.load()  # raises if the HIP library is missing: no fallback
    return torch


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def up(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def down(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def cosine(a, b) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    if na == 0 or nb == 0:
        return 0.0
    return float(a @ b / (na * nb))


def assert_within(y, y_ref, S, rel, what, abs_=GEMV_ABS):
    y = np.asarray(y, np.float64)
    err = np.abs(y - y_ref)
    bound = rel * S + abs_
    bad = np.nonzero(~(err <= bound))
    if bad[0].size:
        i = tuple(b[0] for b in bad)
        raise AssertionError("%s: %d elements outside |err| <= %g*S + %g; first at %s: got %r "
                             "ref %r S %r (max err/S %.3g)"
                             % (what, bad[0].size, rel, abs_, i, y[i], y_ref[i], S[i],
                                float(np.max(err / np.maximum(S, 1e-30)))))


def assert_gemv(y, y_ref, S, what):
    assert_within(y, y_ref, S, GEMV_REL, what)
    c = cosine(y, y_ref)
    assert c >= COS_MIN, "%s: cosine %.9f < %g" % (what, c, COS_MIN)


def bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, np.float32).view(np.uint32)
