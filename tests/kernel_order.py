"""f32 emulation of the GEMV kernels' operation order (test helper, CPU only).

Each function replays, in numpy float32 with one rounding per operation,
the arithmetic one kernel lane performs for one output row, so that a
property of the summation order can be checked on the CPU before it is
checked on the GPU.  Two orders per block format:

* ``factored``: the form the kernels used first.  Per sub-block it sums
  q*x and x separately and combines them with the scales afterwards,
  e.g. for Q4_K  d*sum_j sc_j*T_j - dmin*sum_j m_j*X_j.  Its rounding
  error grows with sum (d*sc*q + dmin*m)*|x|, which a row whose weights
  cancel (w = 0 exactly, so S = sum|w*x| = 0) does not bound.
* ``per_weight``: the form the kernels use now.  Every weight is formed
  exactly rounded (Q4_K: w = fma(q, d*sc, -dmin*m)) or as an exact small
  integer times a scale applied once per group of weights (Q8_0: q,
  Q6_K: q - 32), and the sums run over w*x, so the error is a multiple of
  sum|w*x|.

The chain structure (which products share an accumulator, the order of
the final adds) follows the kernels; the decoding of the bytes is this
module's own (numpy bit slicing), and fused multiply-adds are evaluated in
double and rounded to float32.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
TWO_M24 = 2.0 ** -24


def fma32(a, b, c):
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64)
            + np.asarray(c, np.float64)).astype(F32)


def add32(a, b):
    return (np.asarray(a, F32) + np.asarray(b, F32)).astype(F32)


def mul32(a, b):
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64)).astype(F32)


def _half(lo, hi):
    return (lo.astype(np.uint16) | (hi.astype(np.uint16) << 8)).view(np.float16).astype(F32)


# ------------------------------------------------------------------ Q4_K

def q4k_fields(blocks):
    """blocks: uint8 [R, 144] -> d, dmin [R] f32; sc, m [R, 8]; q [R, 256]."""
    B = np.asarray(blocks, np.uint8)
    d = _half(B[:, 0], B[:, 1])
    dmin = _half(B[:, 2], B[:, 3])
    s = B[:, 4:16].astype(np.int64)
    sc = np.zeros((B.shape[0], 8), np.int64)
    m = np.zeros_like(sc)
    sc[:, :4] = s[:, 0:4] & 63
    m[:, :4] = s[:, 4:8] & 63
    sc[:, 4:] = (s[:, 8:12] & 15) | ((s[:, 0:4] >> 6) << 4)
    m[:, 4:] = (s[:, 8:12] >> 4) | ((s[:, 4:8] >> 6) << 4)
    qs = B[:, 16:144].astype(np.int64)
    q = np.zeros((B.shape[0], 256), np.int64)
    for g in range(4):
        q[:, 64 * g:64 * g + 32] = qs[:, 32 * g:32 * g + 32] & 15
        q[:, 64 * g + 32:64 * g + 64] = qs[:, 32 * g:32 * g + 32] >> 4
    return d, dmin, sc, m, q


def _x_subsums(xb, width):
    """Sums of x over groups of `width` values as the kernels form them: a
    lane adds its four values as (a+b)+(c+d), then an xor butterfly over
    width/4 lanes."""
    lanes = xb.astype(F32).reshape(-1, 4)
    s = add32(add32(lanes[:, 0], lanes[:, 1]), add32(lanes[:, 2], lanes[:, 3]))
    step = 1
    while step < width // 4:
        s = add32(s, s[np.arange(s.size) ^ step])
        step *= 2
    return s[:: width // 4]


def q4k_row(w_row, x, order):
    """One output row of the Q4_K GEMV: w_row uint8 [nb*144], x f32 [nb*256].
    Blocks j go to wave j % 4; the four wave sums are added in wave order."""
    nb = len(w_row) // 144
    d, dmin, sc, m, q = q4k_fields(np.asarray(w_row, np.uint8).reshape(nb, 144))
    x = np.asarray(x, F32)
    acc = [F32(0)] * 4
    for j in range(nb):
        xb = x[256 * j:256 * j + 256]
        cl = [F32(0), F32(0)]
        ch = [F32(0), F32(0)]
        A_lo = A_hi = F32(0)
        for g in range(4):
            if order == "per_weight":
                wl = (d[j] * sc[j, 2 * g] * q[j, 64 * g:64 * g + 32].astype(np.float64)
                      - np.float64(dmin[j]) * m[j, 2 * g]).astype(F32)
                wh = (d[j] * sc[j, 2 * g + 1] * q[j, 64 * g + 32:64 * g + 64].astype(np.float64)
                      - np.float64(dmin[j]) * m[j, 2 * g + 1]).astype(F32)
            else:  # binary16 subnormal nibble values, high nibbles kept as 16 q
                wl = (q[j, 64 * g:64 * g + 32] * TWO_M24).astype(F32)
                wh = (16 * q[j, 64 * g + 32:64 * g + 64] * TWO_M24).astype(F32)
            for i in range(8):
                for e in range(4):
                    l, c = 4 * i + e, e & 1
                    cl[c] = fma32(wl[l], xb[64 * g + l], cl[c])
                    ch[c] = fma32(wh[l], xb[64 * g + 32 + l], ch[c])
            if order == "factored":
                A_lo = fma32(F32(sc[j, 2 * g]), add32(cl[0], cl[1]), A_lo)
                A_hi = fma32(F32(sc[j, 2 * g + 1]), add32(ch[0], ch[1]), A_hi)
                cl = [F32(0), F32(0)]
                ch = [F32(0), F32(0)]
        if order == "per_weight":
            blk = add32(add32(cl[0], cl[1]), add32(ch[0], ch[1]))
        else:
            X = _x_subsums(xb, 32)
            Bm = F32(0)
            for s in range(8):
                Bm = fma32(F32(m[j, s]), X[s], Bm)
            inner = fma32(A_hi, F32(0.0625 * 2 ** 24), mul32(A_lo, F32(2 ** 24)))
            blk = fma32(d[j], inner, mul32(-dmin[j], Bm))
        acc[j % 4] = add32(acc[j % 4], blk)
    return float(add32(add32(add32(acc[0], acc[1]), acc[2]), acc[3]))


# ------------------------------------------------------------------ Q8_0

def q8_row(w_row, x, order):
    """One output row of the Q8_0 GEMV (34-byte blocks: binary16 d, 32 int8)."""
    B = np.asarray(w_row, np.uint8).reshape(-1, 34)
    d = _half(B[:, 0], B[:, 1])
    q = B[:, 2:34].view(np.int8).astype(np.int64)
    x = np.asarray(x, F32)
    acc = [F32(0)] * 4
    for j in range(B.shape[0]):
        wv = (j // 4) % 4  # a unit is 16 blocks; wave w takes blocks 4w .. 4w+3
        xb = x[32 * j:32 * j + 32]
        if order == "per_weight":
            vals = q[j].astype(F32)
        else:  # u = q + 128 as binary16 subnormals
            vals = ((q[j] + 128) * TWO_M24).astype(F32)
        c = [F32(0), F32(0)]
        for i in range(8):
            for e in range(4):
                c[e & 1] = fma32(vals[4 * i + e], xb[4 * i + e], c[e & 1])
        T = add32(c[0], c[1])
        if order == "per_weight":
            acc[wv] = fma32(d[j], T, acc[wv])
        else:
            X = _x_subsums(xb, 32)[0]
            acc[wv] = fma32(d[j], fma32(T, F32(2 ** 24), mul32(F32(-128), X)), acc[wv])
    return float(add32(add32(add32(acc[0], acc[1]), acc[2]), acc[3]))


# ------------------------------------------------------------------ Q6_K

def q6_fields(blocks):
    B = np.asarray(blocks, np.uint8)
    ql = B[:, 0:128].astype(np.int64)
    qh = B[:, 128:192].astype(np.int64)
    sc = B[:, 192:208].view(np.int8).astype(np.int64)
    d = _half(B[:, 208], B[:, 209])
    q = np.zeros((B.shape[0], 256), np.int64)
    for h in range(2):
        for c in range(4):
            for l in range(32):
                nib = ql[:, 64 * h + 32 * (c % 2) + l]
                nib = nib & 15 if c < 2 else nib >> 4
                q[:, 128 * h + 32 * c + l] = nib | (((qh[:, 32 * h + l] >> (2 * c)) & 3) << 4)
    return d, sc, q


def q6_row(w_row, x, order):
    """One output row of the Q6_K GEMV (210-byte blocks)."""
    nb = len(w_row) // 210
    d, sc, q = q6_fields(np.asarray(w_row, np.uint8).reshape(nb, 210))
    x = np.asarray(x, F32)
    acc = [F32(0)] * 4
    for j in range(nb):
        xb = x[256 * j:256 * j + 256]
        X = _x_subsums(xb, 16)
        A = Bs = F32(0)
        for h in range(2):
            for c in range(4):
                for half in range(2):
                    grp = 8 * h + 2 * c + half
                    t = [F32(0), F32(0)]
                    for i in range(4 * half, 4 * half + 4):
                        for e in range(4):
                            k = 128 * h + 32 * c + 4 * i + e
                            v = (F32(q[j, k] - 32) if order == "per_weight"
                                 else F32(q[j, k] * TWO_M24))
                            t[e & 1] = fma32(v, xb[k], t[e & 1])
                    A = fma32(F32(sc[j, grp]), add32(t[0], t[1]), A)
                    Bs = fma32(F32(sc[j, grp]), X[grp], Bs)
        if order == "factored":
            A = fma32(F32(-32), Bs, mul32(A, F32(2 ** 24)))
        acc[j % 4] = fma32(d[j], A, acc[j % 4])
    return float(add32(add32(add32(acc[0], acc[1]), acc[2]), acc[3]))
