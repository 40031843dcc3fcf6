"""Rows whose weights cancel exactly (every dequantised weight is 0), and
rows that nearly cancel, for the three block formats (test helper).

Q4_K: d = dmin with every sc = m = 63 and q = 1 gives w = 63 d - 63 d = 0.
Q8_0: every q = 0.  Q6_K: every q = 32 (w = d * sc * (q - 32)).
"""
from __future__ import annotations

import numpy as np


def half_bits(v: float) -> int:
    return int(np.array([v], np.float16).view(np.uint16)[0])


def q4k_zero_row(d: float, K: int) -> np.ndarray:
    """d = dmin, every sc = m = 63, every q = 1: w = 63 d - 63 d = 0."""
    blk = np.zeros(144, np.uint8)
    h = half_bits(d)
    blk[0] = blk[2] = h & 0xFF
    blk[1] = blk[3] = h >> 8
    blk[4:16] = 0xFF          # all six-bit scales and mins 63
    blk[16:] = 0x11           # both nibbles of every byte 1
    return np.tile(blk, K // 256)


def q8_zero_row(d: float, K: int) -> np.ndarray:
    blk = np.zeros(34, np.uint8)
    h = half_bits(d)
    blk[0], blk[1] = h & 0xFF, h >> 8
    return np.tile(blk, K // 32)


def q6_zero_row(d: float, K: int) -> np.ndarray:
    """Every q = 32 (low nibbles 0, high bit pair 2) with scales 127."""
    blk = np.zeros(210, np.uint8)
    blk[128:192] = 0xAA
    blk[192:208] = 127
    h = half_bits(d)
    blk[208], blk[209] = h & 0xFF, h >> 8
    return np.tile(blk, K // 256)




def q4k_near_zero_row(K: int) -> np.ndarray:
    """d = 1, dmin = 1 + 2^-10 (the next binary16), sc = m = 63, q = 1:
    every weight is 63 - 63 (1 + 2^-10) = -63 / 1024, a cancellation of
    eleven bits."""
    blk = np.zeros(144, np.uint8)
    hd, hm = half_bits(1.0), half_bits(1.0 + 2.0 ** -10)
    blk[0], blk[1] = hd & 0xFF, hd >> 8
    blk[2], blk[3] = hm & 0xFF, hm >> 8
    blk[4:16] = 0xFF
    blk[16:] = 0x11
    return np.tile(blk, K // 256)


def q4k_mixed(gen_rows: np.ndarray, K: int, every: int = 2) -> np.ndarray:
    """Copy of a generated Q4_K matrix in which every `every`-th row cancels
    exactly (d cycling through 1e-3, 1/64, 1 and 65504) and the row after it
    nearly cancels."""
    w = np.array(gen_rows, np.uint8, copy=True)
    ds = (1e-3, 1.0 / 64, 1.0, 65504.0)
    for i, r in enumerate(range(0, w.shape[0], every)):
        w[r] = q4k_zero_row(ds[i % len(ds)], K)
        if r + 1 < w.shape[0] and (i % 3) == 1:
            w[r + 1] = q4k_near_zero_row(K)
    return w
