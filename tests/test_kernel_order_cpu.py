"""The GEMV kernels' f32 summation order, emulated on the CPU.

The stated GEMV bar is |y - y_ref| <= 1e-4 * S + 1e-6 with S = sum_k |w_ik x_k|.
A row whose weights are all exactly zero is a legal input (Q4_K: d = dmin,
sc = m, q = 1; Q8_0: every q = 0; Q6_K: every q = 32), so S = 0 there and
the bar is 1e-6 absolute.

These tests replay the kernels' order of operations in float32
(tests/kernel_order.py) and show that
  * the factored order the kernels used first (scale/min algebra applied to
    separately rounded sums of q*x and of x) misses the bar on such rows once
    the scales are large enough, and
  * the per-weight order the kernels use now gives exactly 0 there and stays
    far inside the bar on random rows.
The GPU tests (test_gpu_cancellation.py) then check the kernels themselves.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests import kernel_order as ko
from tests.cancel_rows import q4k_zero_row, q6_zero_row, q8_zero_row

K = 5120
BAR_REL, BAR_ABS = 1e-4, 1e-6


def _x():
    return synth.normal(synth.key(9, 1), K)


@pytest.mark.parametrize("d", [1.0 / 64, 1.0])
def test_q4k_factored_order_misses_bar_on_zero_rows(d):
    w, x = q4k_zero_row(d, K), _x()
    yr, S = oracle.gemv(w.reshape(1, -1), x, 1, K)
    assert S[0] == 0.0 and yr[0] == 0.0
    assert abs(ko.q4k_row(w, x, "factored")) > BAR_ABS


@pytest.mark.parametrize("d", [1e-3, 1.0 / 64, 1.0, 65504.0])
def test_q4k_per_weight_order_exact_on_zero_rows(d):
    w, x = q4k_zero_row(d, K), _x()
    assert ko.q4k_row(w, x, "per_weight") == 0.0


@pytest.mark.parametrize("d", [1.0 / 64, 1.0])
def test_q8_factored_order_misses_bar_on_zero_rows(d):
    w, x = q8_zero_row(d, K), _x()
    yr, S = oracle.gemv_q8_0(w.reshape(1, -1), x, 1, K)
    assert S[0] == 0.0 and yr[0] == 0.0
    assert abs(ko.q8_row(w, x, "factored")) > BAR_ABS


@pytest.mark.parametrize("d", [1e-3, 1.0, 65504.0])
def test_q8_per_weight_order_exact_on_zero_rows(d):
    assert ko.q8_row(q8_zero_row(d, K), _x(), "per_weight") == 0.0


@pytest.mark.parametrize("d", [1e-3, 1.0])
def test_q6_factored_order_misses_bar_on_zero_rows(d):
    w, x = q6_zero_row(d, K), _x()
    yr, S = oracle.gemv_q6_k(w.reshape(1, -1), x, 1, K)
    assert S[0] == 0.0 and yr[0] == 0.0
    assert abs(ko.q6_row(w, x, "factored")) > BAR_ABS


@pytest.mark.parametrize("d", [1e-3, 1.0, 65504.0])
def test_q6_per_weight_order_exact_on_zero_rows(d):
    assert ko.q6_row(q6_zero_row(d, K), _x(), "per_weight") == 0.0


def test_per_weight_orders_within_bar_on_random_rows():
    x = _x()
    for name, gen, ref, row in (
            ("q4k", synth.q4k_weight, oracle.gemv, ko.q4k_row),
            ("q8_0", synth.q8_0_weight, oracle.gemv_q8_0, ko.q8_row),
            ("q6_k", synth.q6_k_weight, oracle.gemv_q6_k, ko.q6_row)):
        w = gen(synth.key(9, 20), 3, K)
        yr, S = ref(w, x, 3, K)
        for r in range(3):
            err = abs(row(w[r], x, "per_weight") - yr[r])
            # the f32 error of this order is a small multiple of 2^-24 * S
            assert err <= 1e-6 * S[r], (name, r, err, S[r])


def test_q4k_per_weight_weights_equal_the_dequantised_values():
    """The per-weight order forms each weight as one rounding of
    d*sc*q - dmin*m: the oracle's dequantised value, bit for bit."""
    w = synth.q4k_weight(synth.key(9, 21), 2, 512)
    d, dmin, sc, m, q = ko.q4k_fields(w.reshape(-1, 144))
    j = np.arange(256) // 32
    vals = (d[:, None].astype(np.float64) * sc[:, j] * q
            - dmin[:, None].astype(np.float64) * m[:, j]).astype(np.float32)
    assert np.array_equal(vals.reshape(2, 512).view(np.uint32),
                          oracle.dequant(w, 2, 512).view(np.uint32))
