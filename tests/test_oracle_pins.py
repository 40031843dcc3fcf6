"""Pins of the CPU reference (oracle) to facts outside itself.

Each test checks the oracle against something it does not compute: an
independent library (numpy's binary16, torch's bfloat16 rounding, numpy's
float64 matmul), hand-worked blocks (tests/golden/worked_blocks.txt), closed
forms, exact rational arithmetic, or invariants that a dropped term, a wrong
sign or index, or a transposed operand would break.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests.golden_io import load_worked_blocks

QK, BB = 256, 144


def _f32_bits(v: float) -> int:
    return int(np.array([v], np.float32).view(np.uint32)[0])


# ---------------------------------------------------------------- binary16

def test_half_decode_exhaustive_vs_numpy():
    """All 65,536 binary16 patterns decode as numpy's float16 does."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(h)) for h in pats], np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signs of zeros and infinities are kept
    assert math.copysign(1.0, oracle.half_to_double(0x8000)) == -1.0
    assert oracle.half_to_double(0x7C00) == math.inf
    assert oracle.half_to_double(0xFC00) == -math.inf


def test_half_decode_named_values():
    assert oracle.half_to_double(0x3C00) == 1.0
    assert oracle.half_to_double(0x0001) == 2.0 ** -24
    assert oracle.half_to_double(0x03FF) == 1023 * 2.0 ** -24
    assert oracle.half_to_double(0x0400) == 2.0 ** -14
    assert oracle.half_to_double(0x7BFF) == 65504.0
    assert oracle.half_to_double(0xC000) == -2.0
    assert oracle.half_to_double(0x3555) == 0.333251953125


# ---------------------------------------------------------------- worked blocks

WORKED = load_worked_blocks()


@pytest.mark.parametrize("item", WORKED, ids=[w["id"] for w in WORKED])
def test_worked_block_dequant(item):
    got = oracle.dequant_block(item["block"])
    for k, (val, sign) in enumerate(item["expect"]):
        exp = np.float32(float(val))
        if val == 0:
            exp = np.float32(-0.0) if sign < 0 else np.float32(0.0)
        assert _f32_bits(got[k]) == _f32_bits(float(exp)), (item["id"], k, got[k], exp)


@pytest.mark.parametrize("item", [w for w in WORKED if "sc" in w], ids=lambda w: w["id"])
def test_worked_block_scales(item):
    sc, mn = oracle.unpack_scales(item["block"][4:16])
    assert list(sc) == item["sc"]
    assert list(mn) == item["m"]


def test_scale_packing_is_a_bijection():
    """Every 12-byte pattern maps to distinct (sc, m) fields in 0..63: the 96
    bits carry 16 six-bit fields exactly once each (checked bit by bit)."""
    seen = np.zeros((16, 6), np.int64)
    for byte in range(12):
        for bit in range(8):
            s = np.zeros(12, np.uint8)
            s[byte] = 1 << bit
            sc, mn = oracle.unpack_scales(s)
            fields = list(sc) + list(mn)
            hits = [(f, v) for f, v in enumerate(fields) if v]
            assert len(hits) == 1, (byte, bit, fields)
            f, v = hits[0]
            assert v & (v - 1) == 0 and v < 64
            seen[f, int(v).bit_length() - 1] += 1
    assert (seen == 1).all()


def test_dequant_rounding_tie_is_nearest_even():
    """E5's exact value 30965759 is a tie between f32 neighbours; RNE picks the
    even significand, so truncation or round-half-up would both fail here."""
    blk = next(w for w in WORKED if w["id"] == "E5")["block"]
    got = oracle.dequant_block(blk)
    assert got[0] == np.float32(30965760.0)
    assert 32768 * 63 * 15 - 1 == 30965759


def test_dequant_matrix_places_blocks_row_major():
    M, K = 3, 512
    w = synth.q4k_weight(synth.key(9, 1), M, K)
    full = oracle.dequant(w, M, K)
    for r in range(M):
        for b in range(K // QK):
            blk = w[r, b * BB:(b + 1) * BB]
            assert np.array_equal(full[r, b * QK:(b + 1) * QK].view(np.uint32),
                                  oracle.dequant_block(blk).view(np.uint32))


def _exact_block_values(blk: np.ndarray):
    """Exact rational weights of one block, written from the format reading
    with Python integers and Fractions (no floating point)."""
    def half(h):
        s, e, f = h >> 15, (h >> 10) & 31, h & 1023
        v = Fraction(f, 1 << 24) if e == 0 else Fraction(1024 + f) * Fraction(2) ** (e - 25)
        return -v if s else v
    b = [int(t) for t in blk]
    d, dmin = half(b[0] | b[1] << 8), half(b[2] | b[3] << 8)
    s = b[4:16]
    sc = [s[j] & 63 for j in range(4)] + [(s[j + 4] & 15) | ((s[j - 4] >> 6) << 4) for j in range(4, 8)]
    mn = [s[j + 4] & 63 for j in range(4)] + [(s[j + 4] >> 4) | ((s[j] >> 6) << 4) for j in range(4, 8)]
    qs = b[16:]
    out = []
    for g in range(4):
        lo = [qs[32 * g + l] & 15 for l in range(32)]
        hi = [qs[32 * g + l] >> 4 for l in range(32)]
        out += [d * sc[2 * g] * q - dmin * mn[2 * g] for q in lo]
        out += [d * sc[2 * g + 1] * q - dmin * mn[2 * g + 1] for q in hi]
    return out


def _exact_block_values_terms(blk: np.ndarray, k: int) -> bool:
    """True if both terms of weight k (d*sc*q and dmin*m) are exactly zero."""
    b = [int(t) for t in blk]
    s = b[4:16]
    j = k // 32
    sc = (s[j] & 63) if j < 4 else ((s[j + 4] & 15) | ((s[j - 4] >> 6) << 4))
    mn = (s[j + 4] & 63) if j < 4 else ((s[j + 4] >> 4) | ((s[j] >> 6) << 4))
    g, r = k // 64, k % 64
    q = (b[16 + 32 * g + r] & 15) if r < 32 else (b[16 + 32 * g + r - 32] >> 4)
    d_zero = (b[0] | (b[1] & 0x7F) << 8) == 0
    m_zero = (b[2] | (b[3] & 0x7F) << 8) == 0
    return (d_zero or sc * q == 0) and (m_zero or mn == 0)


def test_dequant_random_blocks_vs_exact_rationals():
    """Random blocks over every finite binary16 d/dmin: the oracle's f32 equals
    the exact rational value rounded once to f32 (numpy's RNE cast of the exact
    double, which holds the rational exactly)."""
    rng = np.random.default_rng(7)
    raw = synth.raw_bytes(synth.key(9, 2), 64 * BB).reshape(64, BB)
    for i in range(64):
        blk = raw[i].copy()
        # any finite binary16 for d and dmin (exponent field != 31)
        for off in (0, 2):
            while True:
                h = int(rng.integers(0, 65536))
                if (h >> 10) & 31 != 31:
                    break
            blk[off], blk[off + 1] = h & 0xFF, h >> 8
        exact = _exact_block_values(blk)
        got = oracle.dequant_block(blk)
        d_neg, dmin_neg = bool(blk[1] & 0x80), bool(blk[3] & 0x80)
        for k in range(256):
            dv = float(exact[k])
            assert Fraction(dv) == exact[k]           # exact in double
            if dv == 0.0:
                # IEEE: x - x = +0; a zero product keeps its operand's sign, so
                # the difference is -0 only for (-0) - (+0).
                a_zero = _exact_block_values_terms(blk, k)
                neg = a_zero and d_neg and not dmin_neg
                dv = -0.0 if neg else 0.0
            assert _f32_bits(got[k]) == _f32_bits(float(np.float32(dv))), (i, k)


# ---------------------------------------------------------------- GEMV

def _rand_case(seed, M, K):
    w = synth.q4k_weight(synth.key(9, 100 + seed), M, K)
    x = synth.normal(synth.key(9, 200 + seed), K)
    return w, x


def test_gemv_zero_activation_is_exact_zero():
    M, K = 7, 768
    w, _ = _rand_case(1, M, K)
    y, S = oracle.gemv(w, np.zeros(K, np.float32), M, K)
    assert np.all(y == 0.0) and np.all(S == 0.0)


def test_gemv_one_hot_returns_dequant_column():
    M, K = 5, 512
    w, _ = _rand_case(2, M, K)
    Wd = oracle.dequant(w, M, K)
    for k in (0, 1, 31, 32, 63, 64, 200, 255, 256, 300, 511):
        x = np.zeros(K, np.float32)
        x[k] = 1.0
        y, _ = oracle.gemv(w, x, M, K)
        assert np.array_equal(y, Wd[:, k].astype(np.float64)), k


def test_gemv_all_ones_closed_form():
    """x = 1: y_i = sum over sub-blocks of d*sc*Q - 32*dmin*m, where Q is the
    integer nibble sum of the sub-block.  The oracle sums f32-rounded weights,
    so the two differ by at most 2^-24 * sum|w| (one rounding per weight)."""
    M, K = 6, 1024
    w, _ = _rand_case(3, M, K)
    y, S = oracle.gemv(w, np.ones(K, np.float32), M, K)
    for i in range(M):
        total = Fraction(0)
        for b in range(K // QK):
            blk = [int(t) for t in w[i, b * BB:(b + 1) * BB]]
            d = Fraction(oracle.half_to_double(blk[0] | blk[1] << 8))
            dmin = Fraction(oracle.half_to_double(blk[2] | blk[3] << 8))
            sc, mn = oracle.unpack_scales(np.array(blk[4:16], np.uint8))
            qs = blk[16:]
            for g in range(4):
                Qlo = sum(qs[32 * g + l] & 15 for l in range(32))
                Qhi = sum(qs[32 * g + l] >> 4 for l in range(32))
                total += d * int(sc[2 * g]) * Qlo - 32 * dmin * int(mn[2 * g])
                total += d * int(sc[2 * g + 1]) * Qhi - 32 * dmin * int(mn[2 * g + 1])
        assert abs(Fraction(y[i]) - total) <= Fraction(2) ** -24 * Fraction(S[i]) * 1.0000001


@pytest.mark.parametrize("M,K", [(1, 256), (3, 256), (4, 512), (2, 512)])
def test_gemv_bruteforce_exact_rationals(M, K):
    """Tiny matrices: y equals the exact rational sum of fl32(w)*x to 1e-15."""
    w, x = _rand_case(10 + M + K, M, K)
    y, S = oracle.gemv(w, x, M, K)
    for i in range(M):
        acc = Fraction(0)
        for b in range(K // QK):
            vals = _exact_block_values(w[i, b * BB:(b + 1) * BB])
            for k, v in enumerate(vals):
                acc += Fraction(float(np.float32(float(v)))) * Fraction(float(x[b * QK + k]))
        assert abs(Fraction(y[i]) - acc) <= Fraction(1, 10 ** 15) * Fraction(S[i])


def test_gemv_matches_library_matmul_on_dequant():
    """Non-square M != K: y equals numpy's float64 matmul of the dequantised
    matrix (a transposed operand or wrong row stride would fail)."""
    M, K = 37, 1280
    w, x = _rand_case(4, M, K)
    Wd = oracle.dequant(w, M, K).astype(np.float64)
    y, S = oracle.gemv(w, x, M, K)
    ref = Wd @ x.astype(np.float64)
    assert np.all(np.abs(y - ref) <= 1e-13 * S + 1e-300)
    assert np.allclose(S, np.abs(Wd) @ np.abs(x.astype(np.float64)), rtol=1e-13, atol=0)


def test_gemv_linearity_and_rows_subset():
    M, K = 9, 768
    w, x1 = _rand_case(5, M, K)
    x2 = synth.normal(synth.key(9, 301), K).astype(np.float64)
    x1 = x1.astype(np.float64)
    a, b = 0.75, -1.5
    y1, S1 = oracle.gemv(w, x1, M, K)
    y2, S2 = oracle.gemv(w, x2, M, K)
    y3, _ = oracle.gemv(w, a * x1 + b * x2, M, K)
    assert np.all(np.abs(y3 - (a * y1 + b * y2)) <= 1e-12 * (abs(a) * S1 + abs(b) * S2))
    rows = [8, 0, 3]
    ys, _ = oracle.gemv(w, x1, M, K, rows=rows)
    assert np.array_equal(ys, y1[rows])


def test_gemv_block_permutation_invariance():
    M, K = 4, 1536
    w, x = _rand_case(6, M, K)
    nb = K // QK
    perm = np.array([3, 0, 5, 1, 4, 2])
    wp = w.reshape(M, nb, BB)[:, perm, :].reshape(M, nb * BB).copy()
    xp = x.reshape(nb, QK)[perm].reshape(K).copy()
    y, S = oracle.gemv(w, x, M, K)
    yp, _ = oracle.gemv(wp, xp, M, K)
    assert np.all(np.abs(y - yp) <= 1e-13 * S)


def test_gemv_batch_columns_equal_single_gemv():
    M, K, N = 11, 512, 3
    w, _ = _rand_case(7, M, K)
    X = synth.activations(9, N, K)
    Y, S = oracle.gemv_batch(w, X, M, K)
    for n in range(N):
        y, s = oracle.gemv(w, X[n], M, K)
        assert np.array_equal(Y[n], y) and np.array_equal(S[n], s)


# ---------------------------------------------------------------- bf16 / GEMM

def test_bf16_round_named_ties():
    b2f = lambda b: float(np.array([b], np.uint32).view(np.float32)[0])
    assert oracle.bf16_round(b2f(0x3F808000)) == b2f(0x3F800000)   # tie, kept bit even
    assert oracle.bf16_round(b2f(0x3F818000)) == b2f(0x3F820000)   # tie, kept bit odd -> up
    assert oracle.bf16_round(b2f(0x3F808001)) == b2f(0x3F810000)   # above the tie
    assert oracle.bf16_round(b2f(0xBF818000)) == b2f(0xBF820000)   # negative tie
    assert oracle.bf16_round(1.0) == 1.0


def test_bf16_round_vs_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    bits = bits[((bits >> 23) & 0xFF) < 0xFE]                 # finite, away from overflow
    ties = (bits & 0xFFFF0000) | 0x8000
    allb = np.concatenate([bits, ties]).astype(np.uint32)
    vals = allb.view(np.float32)
    ref = torch.from_numpy(vals.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    got = np.array([oracle.bf16_round(float(v)) for v in vals], np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_gemm_rows_equal_gemv_per_token():
    M, K, P = 10, 512, 4
    w, _ = _rand_case(8, M, K)
    X = synth.activations(9, P, K, first=10)
    Y, S = oracle.gemm(w, X, M, K)
    for p in range(P):
        y, s = oracle.gemv(w, X[p], M, K)
        assert np.array_equal(Y[p], y) and np.array_equal(S[p], s)
    Ys, _ = oracle.gemm(w, X, M, K, rows=[9, 2], toks=[3, 0])
    assert np.array_equal(Ys, Y[np.ix_([3, 0], [9, 2])])


def test_gemm_bf16_inputs_vs_library_matmul():
    """bf16 reference = numpy float64 matmul of torch-rounded bf16 operands."""
    torch = pytest.importorskip("torch")
    M, K, P = 12, 768, 5
    w, _ = _rand_case(9, M, K)
    X = synth.activations(9, P, K, first=20)
    Wd = oracle.dequant(w, M, K)
    Wb = torch.from_numpy(Wd).to(torch.bfloat16).to(torch.float64).numpy()
    Xb = torch.from_numpy(X).to(torch.bfloat16).to(torch.float64).numpy()
    ref = Xb @ Wb.T
    Y16, S16 = oracle.gemm(w, X, M, K, bf16_inputs=True)
    assert np.all(np.abs(Y16 - ref) <= 1e-13 * S16)


def test_gemm_bf16_exact_inputs_equal_f32_reference():
    """E7 weights are small integers and x with <= 8 significant bits is bf16
    exact, so rounding the inputs to bf16 must change nothing."""
    blk = next(w for w in WORKED if w["id"] == "E7")["block"]
    M, K, P = 3, 512, 2
    w = np.tile(blk, (M, K // QK))
    rng = np.random.default_rng(3)
    X = (rng.integers(-128, 128, (P, K)) / 16.0).astype(np.float32)
    Y, _ = oracle.gemm(w, X, M, K)
    Y16, _ = oracle.gemm(w, X, M, K, bf16_inputs=True)
    assert np.array_equal(Y, Y16)


# ---------------------------------------------------------------- glue / stack

def test_rms_and_silu_closed_forms():
    assert oracle.rms(np.full(64, 3.0), 1e-6) == math.sqrt(9.0 + 1e-6)
    assert oracle.rms(np.array([3.0, 4.0]), 0.0) == math.sqrt(12.5)
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) == 0.0
    assert abs(oracle.silu(1.0) - 0.7310585786300049) < 1e-16
    # silu(x) - silu(-x) = x
    for g in (0.3, 2.0, 7.5):
        assert abs((oracle.silu(g) - oracle.silu(-g)) - g) < 1e-15 * (1 + g)


# ---------------------------------------------------------------- MLP block

def _worked_rows(n_rows, shift):
    """A [n_rows][256] Q4_K matrix (one super-block per row) whose row i is
    hand-worked block (i + shift) mod len(WORKED), and its known values."""
    blocks = [np.asarray(it["block"], np.uint8) for it in WORKED]
    vals = [[float(v) for v, _ in it["expect"]] for it in WORKED]
    idx = [(i + shift) % len(WORKED) for i in range(n_rows)]
    return np.stack([blocks[j] for j in idx]), [vals[j] for j in idx]


def _silu(v: float) -> float:
    # e^-v overflows past 709.78: the quotient is then v / inf = -0
    return v / (1.0 + math.exp(-v)) if -v < 709.0 else v / math.inf


@pytest.mark.parametrize("k,c", [(0, 1.0), (37, 1.0), (200, 0.75), (255, 2.5)])
def test_mlp_one_hot_closed_form(k, c):
    """x = e_k, eps = 0, gain (1 + w) = c everywhere, hidden = inter = 256:
    rms(e_k) = 1/16 exactly, so n = 16 c e_k and the gate and up outputs are
    16 c times column k of the hand-worked rows.  a = silu(g) * u, and
    y = r + W_down a as an exactly rounded sum (math.fsum) over the known
    down-row values: pins the normalisation, the gain, which product takes the
    SiLU, the down matrix orientation and the residual."""
    H = I = 256
    wg, vg = _worked_rows(I, 0)
    wu, vu = _worked_rows(I, 3)
    wd, vd = _worked_rows(H, 5)
    x = np.zeros(H, np.float32)
    x[k] = 1.0
    nw = np.full(H, c - 1.0, np.float32)
    r = np.linspace(-2, 2, H).astype(np.float32)
    out = oracle.mlp(wg, wu, wd, H, I, x, nw, 0.0, r)
    g = [16.0 * c * vg[i][k] for i in range(I)]
    u = [16.0 * c * vu[i][k] for i in range(I)]
    a = [_silu(g[i]) * u[i] for i in range(I)]
    for i in range(I):
        assert out["g"][i] == g[i] and out["u"][i] == u[i]
        assert abs(out["a"][i] - a[i]) <= 1e-15 * abs(a[i])
    for j in range(H):
        yj = float(r[j]) + math.fsum(vd[j][i] * a[i] for i in range(I))
        scale = float(abs(r[j])) + math.fsum(abs(vd[j][i] * a[i]) for i in range(I))
        assert abs(out["y"][j] - yj) <= 1e-13 * (scale + 1.0), j


def test_mlp_zero_input_and_zero_gain_give_the_residual():
    """x = 0 normalises to 0 (rms = sqrt(eps)), and a gain of 1 + w = 0 zeroes
    n: either way a = silu(0) * 0 = 0 and y is exactly the residual."""
    H, I = 512, 768
    wg = synth.q4k_weight(synth.key(9, 901), I, H)
    wu = synth.q4k_weight(synth.key(9, 902), I, H)
    wd = synth.q4k_weight(synth.key(9, 903), H, I)
    r = synth.normal(synth.key(9, 904), H)
    out = oracle.mlp(wg, wu, wd, H, I, np.zeros(H, np.float32), None, 1e-6, r)
    assert np.all(out["a"] == 0.0) and np.array_equal(out["y"], r.astype(np.float64))
    x = synth.normal(synth.key(9, 905), H)
    out = oracle.mlp(wg, wu, wd, H, I, x, np.full(H, -1.0, np.float32), 1e-6, r)
    assert np.all(out["a"] == 0.0) and np.array_equal(out["y"], r.astype(np.float64))
    out = oracle.mlp(wg, wu, wd, H, I, x, None, 1e-6, None)
    assert np.all(out["y"] != 0.0)     # no residual: y is the MLP output itself


def test_mlp_scale_invariance_without_eps():
    """With eps = 0, RMSNorm(4x) = RMSNorm(x) exactly (4 is a power of two, so
    the mean, the square root and the division all scale exactly): every
    output is bit-identical."""
    H, I = 512, 768
    wg = synth.q4k_weight(synth.key(9, 911), I, H)
    wu = synth.q4k_weight(synth.key(9, 912), I, H)
    wd = synth.q4k_weight(synth.key(9, 913), H, I)
    x = synth.normal(synth.key(9, 914), H)
    nw = (0.1 * synth.normal(synth.key(9, 915), H)).astype(np.float32)
    a = oracle.mlp(wg, wu, wd, H, I, x, nw, 0.0, None)
    b = oracle.mlp(wg, wu, wd, H, I, (4 * x).astype(np.float32), nw, 0.0, None)
    for key in ("g", "u", "a", "y"):
        assert np.array_equal(a[key], b[key]), key


def test_mlp_eps_enters_the_rms():
    """x = e_k with eps = 1/256: rms = sqrt(1/256 + 1/256) = sqrt(2)/16, so
    the gate output is 16/sqrt(2) times the hand-worked column value."""
    H = I = 256
    wg, vg = _worked_rows(I, 1)
    wu, _ = _worked_rows(I, 2)
    wd, _ = _worked_rows(H, 4)
    x = np.zeros(H, np.float32)
    x[9] = 1.0
    out = oracle.mlp(wg, wu, wd, H, I, x, None, 1.0 / 256, None)
    for i in range(I):
        assert abs(out["g"][i] - 16.0 / math.sqrt(2.0) * vg[i][9]) <= 1e-15 * (1 + abs(out["g"][i]))


def _tiny_stack(n_layers, hidden=512, mix_in=768, mix_k=512, inter=768, vocab=256, cfg=9):
    mats, shapes = [], []
    t = 500
    for _ in range(n_layers):
        for (M, K) in ((mix_in, hidden), (hidden, mix_k), (inter, hidden), (inter, hidden), (hidden, inter)):
            mats.append(synth.q4k_weight(synth.key(cfg, t), M, K))
            shapes.append((M, K))
            t += 1
    mats.append(synth.q4k_weight(synth.key(cfg, t), vocab, hidden))
    shapes.append((vocab, hidden))
    return mats, shapes


def test_stack_equals_composition_of_gemvs():
    """The chain is a composition of the pinned GEMV with rmsn/silu glue."""
    L, H = 2, 512
    mats, shapes = _tiny_stack(L, hidden=H)
    h0 = synth.normal(synth.key(9, 900), H)
    logits, hid = oracle.stack(mats, shapes, L, H, h0, want_hidden=True)

    def rmsn_gemv(i, v):
        M, K = shapes[i]
        v = np.asarray(v, np.float64)
        y, _ = oracle.gemv(mats[i], v / math.sqrt(np.mean(v * v) + 1e-6), M, K)
        return y

    h = h0.astype(np.float64)
    for l in range(L):
        b = 5 * l
        u = rmsn_gemv(b + 0, h)
        h = h + rmsn_gemv(b + 1, u[:shapes[b + 1][1]])
        g = rmsn_gemv(b + 2, h)
        a = rmsn_gemv(b + 3, h)
        act = g / (1.0 + np.exp(-g)) * a
        h = h + rmsn_gemv(b + 4, act)
        assert np.allclose(hid[l], h, rtol=1e-12, atol=1e-12)
    ref = rmsn_gemv(5 * L, h)
    assert np.allclose(logits, ref, rtol=1e-11, atol=1e-11)


def test_stack_zero_layers_is_normalised_lm_head():
    H = 256
    mats, shapes = _tiny_stack(0, hidden=H)
    h0 = synth.normal(synth.key(9, 901), H)
    logits = oracle.stack(mats, shapes, 0, H, h0)
    r = math.sqrt(np.mean(h0.astype(np.float64) ** 2) + 1e-6)
    y, S = oracle.gemv(mats[0], h0.astype(np.float64) / r, shapes[0][0], H)
    # numpy's pairwise mean and the oracle's running sum round differently
    assert np.all(np.abs(logits - y) <= 1e-13 * S)


def test_stack_rejects_broken_chain():
    mats, shapes = _tiny_stack(1, hidden=512)
    shapes = list(shapes)
    shapes[1] = (512, 1024)          # mixer-out K larger than mixer-in M
    with pytest.raises(ValueError):
        oracle.stack(mats, shapes, 1, 512, np.zeros(512, np.float32))


def test_thread_count_does_not_change_bits():
    M, K = 64, 1024
    w, x = _rand_case(12, M, K)
    oracle.set_threads(1)
    y1, _ = oracle.gemv(w, x, M, K)
    oracle.set_threads(4)
    y4, _ = oracle.gemv(w, x, M, K)
    assert np.array_equal(y1, y4)


# ---------------------------------------------------------------- Q8_0

def _q8_fixture():
    """The hand-worked Q8_0 blocks of tests/golden/q8_0_blocks.txt."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "q8_0_blocks.txt")
    out = []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        bid, dhex, qs, exp = [f.strip() for f in line.split("|")]
        if qs == "ramp":
            q = [i - 16 for i in range(32)]
        elif qs == "alt":
            q = [127 if i % 2 == 0 else -128 for i in range(32)]
        else:
            q = [int(v) for v in qs.split()]
        d = int(dhex, 16)
        blk = np.array([d & 0xFF, d >> 8] + [v & 0xFF for v in q], np.uint8)
        out.append((bid, blk, exp.split()))
    return out


@pytest.mark.parametrize("item", _q8_fixture(), ids=lambda it: it[0])
def test_q8_0_worked_blocks(item):
    """d is the first (little-endian) binary16, the quants are two's-complement
    bytes, w = d * q with the sign of zero kept."""
    bid, blk, exp = item
    got = oracle.dequant_q8_0(blk[None, :], 1, 32)[0]
    assert len(exp) == 32
    for i, e in enumerate(exp):
        want = np.float32(-0.0) if e == "-0" else np.float32(float(e))
        assert _f32_bits(got[i]) == _f32_bits(want), (bid, i, got[i], e)


def test_q8_0_dequant_vs_numpy_decoding():
    """Random blocks: numpy's own binary16 and int8 decoding of the same bytes,
    multiplied in double and rounded once, agree bit for bit."""
    w = synth.q8_0_weight(synth.key(9, 930), 37, 1024)
    blocks = w.reshape(-1, 34)
    d = blocks[:, :2].copy().view(np.float16).astype(np.float64)
    q = blocks[:, 2:].view(np.int8).astype(np.float64)
    ref = (d * q).astype(np.float32).reshape(37, 1024)
    got = oracle.dequant_q8_0(w, 37, 1024)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_q8_0_gemv_closed_forms():
    """Zero x gives exact zeros; a one-hot x returns the dequantised column; a
    row of blocks repeated k times with x = 1 sums to k times the block sum."""
    M, K = 40, 512
    w = synth.q8_0_weight(synth.key(9, 931), M, K)
    y, S = oracle.gemv_q8_0(w, np.zeros(K, np.float32), M, K)
    assert np.all(y == 0.0) and np.all(S == 0.0)
    deq = oracle.dequant_q8_0(w, M, K)
    for k in (0, 31, 32, 100, 511):
        x = np.zeros(K, np.float32)
        x[k] = 1.0
        y, _ = oracle.gemv_q8_0(w, x, M, K)
        assert np.array_equal(y, deq[:, k].astype(np.float64))
    _, blk, _ = _q8_fixture()[0]              # Q1: weights -16 .. 15
    tiled = np.tile(blk, 16)[None, :]         # 16 blocks = 512 weights
    y, _ = oracle.gemv_q8_0(tiled, np.ones(512, np.float32), 1, 512)
    assert y[0] == 16 * sum(range(-16, 16))


@pytest.mark.parametrize("M,K", [(3, 32), (2, 96)])
def test_q8_0_gemv_bruteforce_exact_rationals(M, K):
    """Tiny matrices: the exact rational sum (Fractions from the raw bytes) is
    within the double rounding of the oracle's result."""
    w = synth.q8_0_weight(synth.key(9, 932 + K), M, K)
    x = synth.normal(synth.key(9, 933), K)
    y, _ = oracle.gemv_q8_0(w, x, M, K)
    for r in range(M):
        acc = Fraction(0)
        for j in range(K // 32):
            b = w[r, 34 * j:34 * (j + 1)]
            h = int(b[0]) | (int(b[1]) << 8)
            e, m, s = (h >> 10) & 31, h & 1023, -1 if h & 0x8000 else 1
            d = s * (Fraction(m, 1024) * Fraction(2) ** -14 if e == 0 else
                     Fraction(1024 + m, 1024) * Fraction(2) ** (e - 15))
            for i in range(32):
                q = int(b[2 + i]) - 256 if b[2 + i] >= 128 else int(b[2 + i])
                acc += d * q * Fraction(float(x[32 * j + i]))
        assert abs(Fraction(y[r]) - acc) <= Fraction(1, 2 ** 40) * (1 + abs(acc))


# ---------------------------------------------------------------- Q6_K

def _q6_fixture():
    """The hand-worked Q6_K blocks of tests/golden/q6_k_blocks.txt."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "q6_k_blocks.txt")
    out = []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        bid, dhex, ql, qh, sc, exp = [f.strip() for f in line.split("|")]
        if ql == "ramp4":
            qlb = [(i % 16) | ((15 - i % 16) << 4) for i in range(128)]
        else:
            qlb = [int(ql, 16)] * 128
        qhb = [int(qh, 16)] * 64
        if sc == "idx1":
            scv = [g + 1 for g in range(16)]
        elif sc == "alt":
            scv = [-1 if g % 2 == 0 else 2 for g in range(16)]
        else:
            scv = [int(sc)] * 16
        d = int(dhex, 16)
        blk = np.array(qlb + qhb + [v & 0xFF for v in scv] + [d & 0xFF, d >> 8], np.uint8)
        assert blk.size == 210
        kind, *vals = exp.split()
        if kind == "all":
            want = vals * 256
        elif kind == "groups":
            want = [v for v in vals for _ in range(16)]
        else:
            want = vals * 2
        assert len(want) == 256, bid
        out.append((bid, blk, want))
    return out


@pytest.mark.parametrize("item", _q6_fixture(), ids=lambda it: it[0])
def test_q6_k_worked_blocks(item):
    """Scale per 16 weights, nibble order (low nibbles of ql for the first two
    32-weight quarters of each half, high nibbles for the last two), qh bit
    pairs 2c, 2c+1, d last and little-endian, subnormal d, negative d and
    scales, and the sign of zero of d * (sc * (q - 32))."""
    bid, blk, exp = item
    got = oracle.dequant_q6_k(blk[None, :], 1, 256)[0]
    for i, e in enumerate(exp):
        want = np.float32(-0.0) if e == "-0" else np.float32(float(e))
        assert _f32_bits(got[i]) == _f32_bits(want), (bid, i, got[i], e)


def test_q6_k_dequant_vs_numpy_decoding():
    """Random blocks decoded a second way: numpy's binary16 and int8 views and
    array-wide bit slicing of the same bytes, multiplied in double, agree with
    the oracle bit for bit (every value is exact in f32)."""
    M, K = 23, 1024
    w = synth.q6_k_weight(synth.key(9, 940), M, K)
    blocks = w.reshape(-1, 210)
    ql, qh = blocks[:, :128].astype(np.int64), blocks[:, 128:192].astype(np.int64)
    sc = blocks[:, 192:208].view(np.int8).astype(np.int64)
    d = blocks[:, 208:210].copy().view(np.float16).astype(np.float64)[:, 0]
    q = np.empty((blocks.shape[0], 256), np.int64)
    for h in range(2):
        for c in range(4):
            src = ql[:, 64 * h + 32 * (c % 2): 64 * h + 32 * (c % 2) + 32]
            low = (src & 15) if c < 2 else (src >> 4)
            high = (qh[:, 32 * h: 32 * h + 32] >> (2 * c)) & 3
            q[:, 128 * h + 32 * c: 128 * h + 32 * c + 32] = low | (high << 4)
    ints = np.repeat(sc, 16, axis=1) * (q - 32)
    ref = (d[:, None] * ints.astype(np.float64)).astype(np.float32).reshape(M, K)
    got = oracle.dequant_q6_k(w, M, K)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(ref.astype(np.float64), d[:, None].repeat(256, 1).reshape(M, K) *
                          ints.reshape(M, K))   # no rounding anywhere


def test_q6_k_gemv_closed_forms():
    """Zero x gives exact zeros; a one-hot x returns the dequantised column;
    the all-63 block (K2: w = 31) tiled k times with x = 1 sums to 256 k 31."""
    M, K = 40, 1024
    w = synth.q6_k_weight(synth.key(9, 941), M, K)
    y, S = oracle.gemv_q6_k(w, np.zeros(K, np.float32), M, K)
    assert np.all(y == 0.0) and np.all(S == 0.0)
    deq = oracle.dequant_q6_k(w, M, K)
    for k in (0, 15, 16, 127, 128, 255, 256, 1023):
        x = np.zeros(K, np.float32)
        x[k] = 1.0
        y, _ = oracle.gemv_q6_k(w, x, M, K)
        assert np.array_equal(y, deq[:, k].astype(np.float64))
    blk = [b for b in _q6_fixture() if b[0] == "K2"][0][1]
    tiled = np.tile(blk, 4)[None, :]
    y, _ = oracle.gemv_q6_k(tiled, np.ones(1024, np.float32), 1, 1024)
    assert y[0] == 4 * 256 * 31


@pytest.mark.parametrize("M,K", [(2, 256), (1, 512)])
def test_q6_k_gemv_bruteforce_exact_rationals(M, K):
    """Tiny matrices: the exact rational sum, decoded from the raw bytes with
    Python integers, is within the double rounding of the oracle's result."""
    w = synth.q6_k_weight(synth.key(9, 942 + K), M, K)
    x = synth.normal(synth.key(9, 943), K)
    y, _ = oracle.gemv_q6_k(w, x, M, K)
    for r in range(M):
        acc = Fraction(0)
        for j in range(K // 256):
            b = [int(v) for v in w[r, 210 * j:210 * (j + 1)]]
            h16 = b[208] | (b[209] << 8)
            e, m, s = (h16 >> 10) & 31, h16 & 1023, -1 if h16 & 0x8000 else 1
            d = s * (Fraction(m, 1024) * Fraction(2) ** -14 if e == 0 else
                     Fraction(1024 + m, 1024) * Fraction(2) ** (e - 15))
            for k in range(256):
                h, c, l = k // 128, (k % 128) // 32, k % 32
                lo = b[64 * h + 32 * (c % 2) + l]
                lo = lo & 15 if c < 2 else lo >> 4
                hi = (b[128 + 32 * h + l] >> (2 * c)) & 3
                sc = b[192 + k // 16] - 256 if b[192 + k // 16] >= 128 else b[192 + k // 16]
                acc += d * sc * ((lo | (hi << 4)) - 32) * Fraction(float(x[256 * j + k]))
        assert abs(Fraction(y[r]) - acc) <= Fraction(1, 2 ** 40) * (1 + abs(acc))
