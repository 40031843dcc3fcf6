"""CPU reference (oracle) for the Q4_K matmul path — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product (the HIP library and its
Python binding) never imports it and shares no code with it.

Thin ctypes marshalling around ``q4k_oracle.c`` (plain C, double precision);
see that file for the arithmetic and its sources.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q4k_oracle.c")
_SRC_MIX = os.path.join(_HERE, "mixer_oracle.c")
_HDR = os.path.join(_HERE, "q4k_oracle.h")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

QK = 256
BLOCK_BYTES = 144
RMS_EPS = 1e-6

_p = ctypes.c_void_p
_i64 = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (OpenMP over rows, -O2, strict IEEE)."""
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(_SRC_MIX), os.path.getmtime(_HDR))
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < newest:
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp",
                               "-ffp-contract=off", "-fno-fast-math",
                               "-o", tmp, _SRC, _SRC_MIX, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_half_to_double.restype = ctypes.c_double
        L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_unpack_scales.restype = None
        L.oracle_unpack_scales.argtypes = [_p, _p, _p]
        L.oracle_dequant_block.restype = None
        L.oracle_dequant_block.argtypes = [_p, _p]
        L.oracle_dequant.restype = ctypes.c_int
        L.oracle_dequant.argtypes = [_p, _i64, _i64, _p]
        L.oracle_gemv_rows.restype = ctypes.c_int
        L.oracle_gemv_rows.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p, _p]
        L.oracle_gemv_rows_d.restype = ctypes.c_int
        L.oracle_gemv_rows_d.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p, _p]
        L.oracle_gemv_batch_rows.restype = ctypes.c_int
        L.oracle_gemv_batch_rows.argtypes = [_p, _p, _i64, _i64, _i64, _p, _i64, _p, _p]
        L.oracle_bf16_round.restype = ctypes.c_float
        L.oracle_bf16_round.argtypes = [ctypes.c_float]
        L.oracle_gemm_sub.restype = ctypes.c_int
        L.oracle_gemm_sub.argtypes = [_p, _p, _i64, _i64, _i64, _p, _i64, _p, _i64,
                                      ctypes.c_int32, _p, _p]
        L.oracle_rms.restype = ctypes.c_double
        L.oracle_rms.argtypes = [_p, _i64, ctypes.c_double]
        L.oracle_silu.restype = ctypes.c_double
        L.oracle_silu.argtypes = [ctypes.c_double]
        L.oracle_dequant_q8_0_block.restype = None
        L.oracle_dequant_q8_0_block.argtypes = [_p, _p]
        L.oracle_dequant_q8_0.restype = ctypes.c_int
        L.oracle_dequant_q8_0.argtypes = [_p, _i64, _i64, _p]
        L.oracle_gemv_q8_0_rows_d.restype = ctypes.c_int
        L.oracle_gemv_q8_0_rows_d.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p, _p]
        i32, dbl = ctypes.c_int32, ctypes.c_double
        L.oracle_gdn_step.restype = ctypes.c_int
        L.oracle_gdn_step.argtypes = [i32, i32, i32, i32, dbl] + [_p] * 8
        L.oracle_attn_step.restype = ctypes.c_int
        L.oracle_attn_step.argtypes = [i32, i32, i32, i32, dbl, dbl, _p, _p, _p, _p, _p, _i64,
                                       _i64, _p]
        L.oracle_dequant_q6_k_block.restype = None
        L.oracle_dequant_q6_k_block.argtypes = [_p, _p]
        L.oracle_dequant_q6_k.restype = ctypes.c_int
        L.oracle_dequant_q6_k.argtypes = [_p, _i64, _i64, _p]
        L.oracle_gemv_q6_k_rows_d.restype = ctypes.c_int
        L.oracle_gemv_q6_k_rows_d.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p, _p]
        L.oracle_mlp.restype = ctypes.c_int
        L.oracle_mlp.argtypes = [_p, _p, _p, _i64, _i64, _p, _p, ctypes.c_double, _p,
                                 _p, _p, _p, _p, _p, _p, _p]
        L.oracle_stack.restype = ctypes.c_int
        L.oracle_stack.argtypes = [_p, _p, _p, ctypes.c_int32, _i64, ctypes.c_double, _p, _p, _p]
        L.oracle_set_threads.restype = None
        L.oracle_set_threads.argtypes = [ctypes.c_int32]
        L.oracle_get_threads.restype = ctypes.c_int32
        L.oracle_get_threads.argtypes = []
        _lib = L
    return _lib


def _u8(a):
    a = np.ascontiguousarray(a, dtype=np.uint8)
    return a


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _rows(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, r.size


def _check(rc):
    if rc != 0:
        raise ValueError("oracle call failed with status %d" % rc)


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().oracle_get_threads())


def half_to_double(h: int) -> float:
    return float(_load().oracle_half_to_double(int(h)))


def unpack_scales(s12) -> tuple[np.ndarray, np.ndarray]:
    s = _u8(s12)
    assert s.size == 12
    sc = np.zeros(8, np.int32)
    mn = np.zeros(8, np.int32)
    _load().oracle_unpack_scales(s.ctypes.data, sc.ctypes.data, mn.ctypes.data)
    return sc, mn


def dequant_block(blk) -> np.ndarray:
    b = _u8(blk)
    assert b.size == BLOCK_BYTES
    out = np.empty(QK, np.float32)
    _load().oracle_dequant_block(b.ctypes.data, out.ctypes.data)
    return out


def dequant(w, M: int, K: int) -> np.ndarray:
    w = _u8(w)
    assert w.size == M * (K // QK) * BLOCK_BYTES
    out = np.empty((M, K), np.float32)
    _check(_load().oracle_dequant(w.ctypes.data, M, K, out.ctypes.data))
    return out


def gemv(w, x, M: int, K: int, rows=None) -> tuple[np.ndarray, np.ndarray]:
    """(y, S) in double for the listed rows (all rows if None)."""
    w = _u8(w)
    x = np.ascontiguousarray(x)
    r, nr = _rows(rows)
    n = nr if r is not None else M
    y = np.empty(n, np.float64)
    S = np.empty(n, np.float64)
    rp = r.ctypes.data if r is not None else None
    if x.dtype == np.float64:
        assert x.size == K
        _check(_load().oracle_gemv_rows_d(w.ctypes.data, x.ctypes.data, M, K, rp, nr,
                                          y.ctypes.data, S.ctypes.data))
    else:
        x = _f32(x)
        assert x.size == K
        _check(_load().oracle_gemv_rows(w.ctypes.data, x.ctypes.data, M, K, rp, nr,
                                        y.ctypes.data, S.ctypes.data))
    return y, S


def gemv_batch(w, X, M: int, K: int, rows=None) -> tuple[np.ndarray, np.ndarray]:
    """X f32 [N][K] -> (Y, S) double [N][rows]."""
    w = _u8(w)
    X = _f32(X)
    N = X.shape[0]
    assert X.shape[1] == K
    r, nr = _rows(rows)
    n = nr if r is not None else M
    Y = np.empty((N, n), np.float64)
    S = np.empty((N, n), np.float64)
    _check(_load().oracle_gemv_batch_rows(w.ctypes.data, X.ctypes.data, M, K, N,
                                          r.ctypes.data if r is not None else None, nr,
                                          Y.ctypes.data, S.ctypes.data))
    return Y, S


def bf16_round(v: float) -> float:
    return float(_load().oracle_bf16_round(float(v)))


def gemm(w, X, M: int, K: int, rows=None, toks=None, bf16_inputs: bool = False):
    """X f32 [P][K] -> (Y, S) double [toks][rows]."""
    w = _u8(w)
    X = _f32(X)
    P = X.shape[0]
    assert X.shape[1] == K
    r, nr = _rows(rows)
    t, nt = _rows(toks)
    n_r = nr if r is not None else M
    n_t = nt if t is not None else P
    Y = np.empty((n_t, n_r), np.float64)
    S = np.empty((n_t, n_r), np.float64)
    _check(_load().oracle_gemm_sub(w.ctypes.data, X.ctypes.data, M, K, P,
                                   r.ctypes.data if r is not None else None, nr,
                                   t.ctypes.data if t is not None else None, nt,
                                   1 if bf16_inputs else 0, Y.ctypes.data, S.ctypes.data))
    return Y, S


def rms(v, eps: float = RMS_EPS) -> float:
    v = np.ascontiguousarray(v, dtype=np.float64)
    return float(_load().oracle_rms(v.ctypes.data, v.size, eps))


def silu(g: float) -> float:
    return float(_load().oracle_silu(float(g)))


def dequant_q8_0(w, M: int, K: int) -> np.ndarray:
    """Q8_0 matrix [M, K/32*34] -> f32 [M, K]."""
    w = _u8(w)
    out = np.empty((M, K), np.float32)
    _check(_load().oracle_dequant_q8_0(w.ctypes.data, M, K, out.ctypes.data))
    return out


def gemv_q8_0(w, x, M: int, K: int, rows=None) -> tuple[np.ndarray, np.ndarray]:
    """(y, S) in float64 for a Q8_0 matrix: y = W x, S = sum |w x| per row."""
    w = _u8(w)
    x = np.asarray(x)
    xd = np.ascontiguousarray(x if x.dtype == np.float64 else x.astype(np.float32), np.float64)
    assert xd.size == K
    r, nr = _rows(rows)
    n = nr if r is not None else M
    y, S = np.empty(n, np.float64), np.empty(n, np.float64)
    _check(_load().oracle_gemv_q8_0_rows_d(w.ctypes.data, xd.ctypes.data, M, K,
                                           r.ctypes.data if r is not None else None, nr,
                                           y.ctypes.data, S.ctypes.data))
    return y, S


def dequant_q6_k(w, M: int, K: int) -> np.ndarray:
    """Q6_K matrix [M, K/256*210] -> f32 [M, K] (exact)."""
    w = _u8(w)
    out = np.empty((M, K), np.float32)
    _check(_load().oracle_dequant_q6_k(w.ctypes.data, M, K, out.ctypes.data))
    return out


def gemv_q6_k(w, x, M: int, K: int, rows=None) -> tuple[np.ndarray, np.ndarray]:
    """(y, S) in float64 for a Q6_K matrix: y = W x, S = sum |w x| per row."""
    w = _u8(w)
    x = np.asarray(x)
    xd = np.ascontiguousarray(x if x.dtype == np.float64 else x.astype(np.float32), np.float64)
    assert xd.size == K
    r, nr = _rows(rows)
    n = nr if r is not None else M
    y, S = np.empty(n, np.float64), np.empty(n, np.float64)
    _check(_load().oracle_gemv_q6_k_rows_d(w.ctypes.data, xd.ctypes.data, M, K,
                                           r.ctypes.data if r is not None else None, nr,
                                           y.ctypes.data, S.ctypes.data))
    return y, S


def mlp(wg, wu, wd, hidden: int, inter: int, x, norm_w=None, eps: float = RMS_EPS,
        resid=None) -> dict:
    """One MLP block (see q4k_oracle.c): returns g, u, a [inter], y [hidden]
    and the sums of |w x| Sg, Su [inter], Sd [hidden], all float64."""
    arrs = [_u8(wg), _u8(wu), _u8(wd)]
    x = _f32(x)
    nw = _f32(norm_w) if norm_w is not None else None
    r = _f32(resid) if resid is not None else None
    assert x.size == hidden and (nw is None or nw.size == hidden) and (r is None or r.size == hidden)
    out = {k: np.empty(inter, np.float64) for k in ("g", "u", "a", "Sg", "Su")}
    out.update({k: np.empty(hidden, np.float64) for k in ("y", "Sd")})
    _check(_load().oracle_mlp(arrs[0].ctypes.data, arrs[1].ctypes.data, arrs[2].ctypes.data,
                              hidden, inter, x.ctypes.data,
                              nw.ctypes.data if nw is not None else None, float(eps),
                              r.ctypes.data if r is not None else None,
                              *[out[k].ctypes.data for k in ("g", "u", "a", "y", "Sg", "Su", "Sd")]))
    return out


def stack(mats, shapes, n_layers: int, hidden: int, h0, eps: float = RMS_EPS,
          want_hidden: bool = False):
    """Decode matmul chain.  mats: 5*n_layers+1 uint8 arrays (per layer
    mix_in, mix_out, gate, up, down; then lm_head); shapes: matching (M, K)."""
    assert len(mats) == len(shapes) == 5 * n_layers + 1
    arrs = [_u8(m) for m in mats]
    ptrs = (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    Ms = np.array([s[0] for s in shapes], np.int64)
    Ks = np.array([s[1] for s in shapes], np.int64)
    h0 = _f32(h0)
    assert h0.size == hidden
    logits = np.empty(shapes[-1][0], np.float64)
    hid = np.empty((n_layers, hidden), np.float64) if want_hidden else None
    _check(_load().oracle_stack(ptrs, Ms.ctypes.data, Ks.ctypes.data, n_layers, hidden, eps,
                                h0.ctypes.data, logits.ctypes.data,
                                hid.ctypes.data if hid is not None else None))
    return (logits, hid) if want_hidden else logits


def _d(a, n=None):
    a = np.ascontiguousarray(a, np.float64)
    assert n is None or a.size == n, (a.size, n)
    return a


def gdn_step(u, conv_w, a_log, dt_bias, norm_w, conv_state, S, Hk=16, Hv=48, Dk=128, Dv=128,
             eps=RMS_EPS):
    """One Gated DeltaNet decode step (mixer_oracle.c) in double.  Returns
    (out [Hv*Dv], new conv_state [C][3], new S [Hv][Dv][Dk]); inputs are not
    modified.  u: [2*Hk*Dk + 2*Hv*Dv + 2*Hv]."""
    C = 2 * Hk * Dk + Hv * Dv
    # every converted array is held in a local until the call returns
    u = _d(u, C + Hv * Dv + 2 * Hv)
    cw, al, dt, nw = _d(conv_w, 4 * C), _d(a_log, Hv), _d(dt_bias, Hv), _d(norm_w, Dv)
    cs = _d(conv_state, 3 * C).copy()
    St = _d(S, Hv * Dv * Dk).copy()
    out = np.empty(Hv * Dv, np.float64)
    _check(_load().oracle_gdn_step(Hk, Hv, Dk, Dv, float(eps), u.ctypes.data, cw.ctypes.data,
                                   al.ctypes.data, dt.ctypes.data, nw.ctypes.data,
                                   cs.ctypes.data, St.ctypes.data, out.ctypes.data))
    return out, cs.reshape(C, 3), St.reshape(Hv, Dv, Dk)


def attn_step(u, q_norm_w, k_norm_w, k_cache, v_cache, pos, Hq=24, Hkv=4, D=256, R=64,
              theta=1e7, eps=RMS_EPS):
    """One gated full-attention decode step at position pos (mixer_oracle.c)
    in double.  Caches [Hkv][cap][D] (positions < pos filled).  Returns (out
    [Hq*D], new k_cache, new v_cache); inputs are not modified."""
    kc = np.array(k_cache, np.float64, copy=True, order="C")
    vc = np.array(v_cache, np.float64, copy=True, order="C")
    cap = kc.shape[1]
    u = _d(u, Hq * 2 * D + 2 * Hkv * D)
    qw, kw = _d(q_norm_w, D), _d(k_norm_w, D)
    out = np.empty(Hq * D, np.float64)
    _check(_load().oracle_attn_step(Hq, Hkv, D, R, float(theta), float(eps), u.ctypes.data,
                                    qw.ctypes.data, kw.ctypes.data, kc.ctypes.data,
                                    vc.ctypes.data, cap, int(pos), out.ctypes.data))
    return out, kc, vc


def _rmsn(v, eps):
    v = np.asarray(v, np.float64)
    return v / np.sqrt(np.mean(v * v) + eps)


def stack_mixers_token(mats, shapes, kinds, mixers, states, hidden, h0, pos, eps=RMS_EPS):
    """One token of the decode chain with the real token mixers, in double:
    per layer u = W_in rmsn(h); o = gdn_step(u) or attn_step(u, pos);
    h_mid = h + W_out rmsn(o); a = silu(W_gate rmsn(h_mid)) * (W_up rmsn(h_mid));
    h = h_mid + W_down rmsn(a); then logits = W_lm rmsn(h).  A composition of
    the oracle's gemv, gdn_step and attn_step.  `states[l]` is (conv_state, S)
    for kind 0 or (k_cache, v_cache) for kind 1; returns (logits, new states)."""
    h = np.asarray(h0, np.float64)
    new_states = []
    for l, kind in enumerate(kinds):
        W = mats[5 * l:5 * l + 5]
        S = shapes[5 * l:5 * l + 5]
        u, _ = gemv(W[0], _rmsn(h, eps), *S[0])
        m = mixers[l]
        if kind == 0:
            o, cs, St = gdn_step(u, m["conv_w"], m["a_log"], m["dt_bias"], m["norm_w"],
                                 states[l][0], states[l][1], Hk=m["key_heads"],
                                 Hv=m["value_heads"], eps=m.get("eps", eps))
            new_states.append((cs, St))
        else:
            o, kc, vc = attn_step(u, m["q_norm_w"], m["k_norm_w"], states[l][0], states[l][1],
                                  pos, Hq=m["q_heads"], Hkv=m["kv_heads"], R=m["rope_dim"],
                                  theta=m["rope_theta"], eps=m.get("eps", eps))
            new_states.append((kc, vc))
        y, _ = gemv(W[1], _rmsn(o, eps), *S[1])
        hm = h + y
        g, _ = gemv(W[2], _rmsn(hm, eps), *S[2])
        v, _ = gemv(W[3], _rmsn(hm, eps), *S[3])
        a = g / (1.0 + np.exp(-g)) * v
        y, _ = gemv(W[4], _rmsn(a, eps), *S[4])
        h = hm + y
    logits, _ = gemv(mats[-1], _rmsn(h, eps), *shapes[-1])
    return logits, new_states
