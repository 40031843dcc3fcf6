"""Seeded synthetic inputs for the Q4_K matmul path (harness code).

Produces raw Q4_K super-block bytes and f32 activations from a counter-based
SplitMix64 stream (see ``synth.c`` for the exact word-to-byte recipe).  Both
the HIP path and the CPU reference read the bytes made here, so neither side
ever generates inputs on its own.  Nothing in this module dequantises or
multiplies: it holds none of the method's arithmetic.

Keys: input set ``c`` (1..5) and tensor ``t`` map to the stream key
``(1000 + c) * 2**32 + t``; activation vector ``n`` of a set uses tensor index
``0xFFFF0000 + n``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

BLOCK_BYTES = 144
QK = 256
D_LO, D_HI = 1e-4, 1e-3
ACT_BASE = 0xFFFF0000


def build(force: bool = False) -> str:
    """Compile ``synth.c`` into ``libsynth.so`` with gcc (OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.synth_word.restype = ctypes.c_uint64
        lib.synth_word.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_half_bits.restype = ctypes.c_uint16
        lib.synth_half_bits.argtypes = [ctypes.c_double]
        lib.synth_q4k_blocks.restype = ctypes.c_int
        lib.synth_q4k_blocks.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                         ctypes.c_void_p, ctypes.c_double, ctypes.c_double]
        lib.synth_q6_k_blocks.restype = ctypes.c_int
        lib.synth_q6_k_blocks.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_void_p, ctypes.c_double, ctypes.c_double]
        lib.synth_q8_0_blocks.restype = ctypes.c_int
        lib.synth_q8_0_blocks.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_void_p, ctypes.c_double, ctypes.c_double]
        lib.synth_normal_f32.restype = None
        lib.synth_normal_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p]
        lib.synth_bytes.restype = None
        lib.synth_bytes.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p]
        _lib = lib
    return _lib


def key(cfg: int, tensor: int) -> int:
    """Stream key of tensor ``tensor`` in input set ``cfg``."""
    return ((1000 + int(cfg)) << 32) + int(tensor)


def word(k: int, i: int) -> int:
    return int(_load().synth_word(k, i))


def half_bits(v: float) -> int:
    return int(_load().synth_half_bits(v))


def q4k_weight(k: int, M: int, K: int, lo: float = D_LO, hi: float = D_HI,
               row0: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    """Rows ``row0 .. row0+M-1`` of a random Q4_K matrix with K columns.

    Returns uint8 [M, K/256*144]: row-major, each row K/256 consecutive blocks.
    Row r of the full matrix is the same bytes whatever ``row0``/``M`` slice it
    is generated in.
    """
    if K % QK:
        raise ValueError("K must be a multiple of 256")
    nb = K // QK
    if out is None:
        out = np.empty((M, nb * BLOCK_BYTES), dtype=np.uint8)
    assert out.flags.c_contiguous and out.dtype == np.uint8 and out.size == M * nb * BLOCK_BYTES
    if M:
        rc = _load().synth_q4k_blocks(k, row0 * nb, M * nb, out.ctypes.data, lo, hi)
        if rc != 0:
            raise ValueError("d/dmin range outside binary16 normals")
    return out


Q8_QK, Q8_BLOCK_BYTES = 32, 34


def q8_0_weight(k: int, M: int, K: int, lo: float = D_LO, hi: float = D_HI) -> np.ndarray:
    """A random Q8_0 matrix with K columns: uint8 [M, K/32*34], row-major, each
    row K/32 consecutive 34-byte blocks (binary16 d, then 32 int8 quants)."""
    if K % Q8_QK:
        raise ValueError("K must be a multiple of 32")
    nb = K // Q8_QK
    out = np.empty((M, nb * Q8_BLOCK_BYTES), dtype=np.uint8)
    if M:
        rc = _load().synth_q8_0_blocks(k, 0, M * nb, out.ctypes.data, lo, hi)
        if rc != 0:
            raise ValueError("d range outside binary16 normals")
    return out


Q6_QK, Q6_BLOCK_BYTES = 256, 210


def q6_k_weight(k: int, M: int, K: int, lo: float = D_LO, hi: float = D_HI) -> np.ndarray:
    """A random Q6_K matrix with K columns: uint8 [M, K/256*210], row-major, each
    row K/256 consecutive 210-byte blocks (quant low bits, quant high bits,
    sixteen int8 scales, binary16 d; all bytes uniform except d ~ U(lo, hi))."""
    if K % Q6_QK:
        raise ValueError("K must be a multiple of 256")
    nb = K // Q6_QK
    out = np.empty((M, nb * Q6_BLOCK_BYTES), dtype=np.uint8)
    if M:
        rc = _load().synth_q6_k_blocks(k, 0, M * nb, out.ctypes.data, lo, hi)
        if rc != 0:
            raise ValueError("d range outside binary16 normals")
    return out


def normal(k: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    if n:
        _load().synth_normal_f32(k, n, out.ctypes.data)
    return out


def activations(cfg: int, n_vec: int, K: int, first: int = 0) -> np.ndarray:
    """``n_vec`` standard-normal f32 vectors of length K, shape [n_vec, K]."""
    X = np.empty((n_vec, K), dtype=np.float32)
    for i in range(n_vec):
        X[i] = normal(key(cfg, ACT_BASE + first + i), K)
    return X


def raw_bytes(k: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    if n:
        _load().synth_bytes(k, n, out.ctypes.data)
    return out
