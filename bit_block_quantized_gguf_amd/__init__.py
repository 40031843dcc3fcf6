"""Python binding of libq4k (MI355X / gfx950 Q4_K matmul library).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libq4k.so``.  PyTorch supplies device memory and streams; all
calls enqueue on ``torch.cuda.current_stream()`` and return without
synchronising.  If the library has not been built, importing the functions
raises instead of falling back to anything else.

The names follow the C ABI in ``include/q4k.h``:
``dequant``, ``gemv``, ``gemv_batch``, ``gemm`` and ``DecodeStack``
(``q4k_decode_stack_*``).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libq4k.so")

QK = 256
BLOCK_BYTES = 144

Q4K_OK = 0
STATUS = {0: "Q4K_OK", -1: "Q4K_EINVAL", -2: "Q4K_ESHAPE", -3: "Q4K_EALIGN",
          -4: "Q4K_ENOMEM", -5: "Q4K_EHIP", -6: "Q4K_EUNSUPPORTED"}
(BUF_H, BUF_U, BUF_HMID, BUF_G, BUF_V, BUF_A, BUF_LOGITS, BUF_MIX, BUF_CONV_STATE, BUF_GDN_STATE,
 BUF_K_CACHE, BUF_V_CACHE) = range(12)
STACK_MIXERS = 1
STACK_PERSISTENT = 2

# Every symbol include/q4k.h declares (checked by the CPU test suite).
EXPORTS = (
    "q4k_last_error", "q4k_version", "q4k_workspace_size", "q4k_dequant", "q4k_gemv",
    "q4k_gemv_q8_0", "q4k_gemv_q6_k", "q4k_mlp", "q4k_gemv_batch", "q4k_gemm",
    "q4k_decode_stack_create", "q4k_decode_stack", "q4k_decode_stack_buffer",
    "q4k_decode_stack_nodes", "q4k_decode_stack_destroy", "q4k_gemv_config", "q4k_gemm_config",
    "q4k_tune_gemv", "q4k_tune_gemm", "q4k_gemv_noalloc", "q4k_gdn_step", "q4k_attn_step",
    "q4k_decode_stack_reset", "q4k_decode_stack_position", "q4k_decode_stack_status",
    "q4k_check_partition",
)
(OP_GEMV, OP_GEMV_BATCH, OP_GEMM, OP_GEMV_Q8_0, OP_GEMV_Q6_K, OP_MLP, OP_GDN_STEP,
 OP_ATTN_STEP) = range(8)

_lib = None


class Q4KError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s (%d): %s" % (STATUS.get(code, "?"), code, msg))
        self.code = code


class MatDesc(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("M", ctypes.c_int64), ("K", ctypes.c_int64)]


class LayerDesc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("mix_in", MatDesc), ("mix_out", MatDesc),
                ("gate", MatDesc), ("up", MatDesc), ("down", MatDesc)]


class GdnParams(ctypes.Structure):
    _fields_ = [("key_heads", ctypes.c_int32), ("value_heads", ctypes.c_int32),
                ("key_dim", ctypes.c_int32), ("value_dim", ctypes.c_int32), ("eps", ctypes.c_float),
                ("conv_w", ctypes.c_void_p), ("a_log", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p), ("norm_w", ctypes.c_void_p)]


class AttnParams(ctypes.Structure):
    _fields_ = [("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("rope_dim", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("eps", ctypes.c_float),
                ("q_norm_w", ctypes.c_void_p), ("k_norm_w", ctypes.c_void_p)]


class MixerDesc(ctypes.Structure):
    _fields_ = [("gdn", GdnParams), ("attn", AttnParams)]


class StackDesc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int64), ("n_layers", ctypes.c_int32),
                ("layers", ctypes.POINTER(LayerDesc)), ("lm_head", MatDesc),
                ("eps", ctypes.c_float), ("flags", ctypes.c_int32),
                ("mixers", ctypes.POINTER(MixerDesc)), ("attn_capacity", ctypes.c_int64),
                ("spin_limit", ctypes.c_int32)]


def load(path: str | None = None):
    """Load libq4k.so (built by ``bit_block_quantized_gguf_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    try:
        # Load torch's HIP runtime first so that libq4k binds to the same
        # libamdhip64.so.7 (one runtime per process).
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise ImportError("libq4k.so is not built (run __graft_entry__.build() or "
                          "python bit_block_quantized_gguf_amd/build.py)")
    L = ctypes.CDLL(path)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.q4k_last_error.restype = ctypes.c_char_p
    L.q4k_last_error.argtypes = []
    L.q4k_version.restype = ctypes.c_int
    sz = ctypes.c_size_t
    L.q4k_workspace_size.argtypes = [i32, i64, i64, i64, ctypes.POINTER(sz)]
    L.q4k_dequant.argtypes = [p, p, i64, i64, p]
    L.q4k_gemv.argtypes = [p, p, p, i64, i64, p, sz, p]
    L.q4k_gemv_batch.argtypes = [p, p, p, i64, i64, i64, p, sz, p]
    L.q4k_gemm.argtypes = [p, p, p, i64, i64, i64, p, sz, p]
    L.q4k_mlp.argtypes = [p, p, p, i64, i64, p, p, ctypes.c_float, p, p, p, p, sz, p]
    L.q4k_gemv_q8_0.argtypes = [p, p, p, i64, i64, p, sz, p]
    L.q4k_gemv_noalloc.argtypes = [p, p, p, i64, i64, p]
    L.q4k_gemv_noalloc.restype = ctypes.c_int
    L.q4k_gdn_step.argtypes = [ctypes.POINTER(GdnParams), p, p, p, p, p, sz, p]
    L.q4k_gdn_step.restype = ctypes.c_int
    L.q4k_attn_step.argtypes = [ctypes.POINTER(AttnParams), p, p, p, i64, i64, p, p, sz, p]
    L.q4k_attn_step.restype = ctypes.c_int
    L.q4k_gemv_q6_k.argtypes = [p, p, p, i64, i64, p, sz, p]
    L.q4k_decode_stack_create.argtypes = [ctypes.POINTER(StackDesc), p, ctypes.POINTER(p)]
    L.q4k_decode_stack.argtypes = [p, p, p, p]
    L.q4k_decode_stack_buffer.argtypes = [p, i32, i32, ctypes.POINTER(p), ctypes.POINTER(i64)]
    L.q4k_decode_stack_nodes.argtypes = [p, ctypes.POINTER(i64)]
    L.q4k_decode_stack_reset.argtypes = [p, p]
    L.q4k_decode_stack_reset.restype = ctypes.c_int
    L.q4k_decode_stack_position.argtypes = [p, ctypes.POINTER(i64)]
    L.q4k_decode_stack_position.restype = ctypes.c_int
    L.q4k_decode_stack_status.argtypes = [p, p, ctypes.POINTER(i32)]
    L.q4k_decode_stack_status.restype = ctypes.c_int
    L.q4k_check_partition.argtypes = [i32, i64, i64, i64, i32]
    L.q4k_check_partition.restype = ctypes.c_int
    L.q4k_decode_stack_destroy.argtypes = [p]
    L.q4k_decode_stack_destroy.restype = None
    L.q4k_gemv_config.argtypes = [i64, i64, i64, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.q4k_gemm_config.argtypes = [i64, i64, i64, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.q4k_tune_gemv.argtypes = [i32, i32]
    L.q4k_tune_gemm.argtypes = [i32, i32]
    for name in ("q4k_workspace_size", "q4k_dequant", "q4k_gemv", "q4k_gemv_batch", "q4k_gemm",
                 "q4k_mlp", "q4k_gemv_q8_0", "q4k_gemv_q6_k",
                 "q4k_decode_stack_create", "q4k_decode_stack", "q4k_decode_stack_buffer",
                 "q4k_decode_stack_nodes", "q4k_gemv_config", "q4k_gemm_config",
                 "q4k_tune_gemv", "q4k_tune_gemm"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def check(rc: int) -> None:
    if rc != Q4K_OK:
        msg = load().q4k_last_error().decode(errors="replace")
        raise Q4KError(rc, msg)


def _torch():
    import torch
    return torch


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _tensor(t, dtype, name, numel=None):
    """Check a tensor argument's type, dtype, element count and layout (an
    undersized output would make a kernel write past it).  Device placement is
    checked separately, after every argument's size (_on_gpu)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if numel is not None and t.numel() != numel:
        raise ValueError("%s has %d elements, the call needs %d" % (name, t.numel(), numel))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _on_gpu(**tensors):
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError("%s must be a device tensor" % name)


def _dev_tensor(t, dtype, name):
    _tensor(t, dtype, name)
    _on_gpu(**{name: t})
    return t


def _weights(w, M, K, block_bytes=BLOCK_BYTES, block_weights=QK, fmt="Q4_K"):
    torch = _torch()
    if K % QK:
        raise ValueError("K must be a multiple of 256")
    need = M * (K // block_weights) * block_bytes
    if not isinstance(w, torch.Tensor):
        raise TypeError("w must be a torch.Tensor")
    if w.numel() != need:
        raise ValueError("w holds %d bytes, a %dx%d %s matrix needs %d"
                         % (w.numel(), M, K, fmt, need))
    return _tensor(w, torch.uint8, "w")


def weight_shape(w) -> tuple[int, int]:
    """(M, K) of a [M, K/256*144] uint8 super-block tensor."""
    M, rb = w.shape
    if rb % BLOCK_BYTES:
        raise ValueError("row length is not a whole number of 144-byte blocks")
    return M, rb // BLOCK_BYTES * QK


def version() -> int:
    return int(load().q4k_version())


# ---------------------------------------------------------------- workspaces

_ws_need: dict = {}


def workspace_size(op: int, M: int, K: int, N: int = 0) -> int:
    """Bytes of workspace that call `op` (OP_GEMV, ...) needs for the shape
    (memoised per shape; the tuning knobs clear the memo)."""
    key = (op, M, K, N)
    n = _ws_need.get(key)
    if n is None:
        c = ctypes.c_size_t()
        check(load().q4k_workspace_size(op, M, K, N, ctypes.byref(c)))
        n = _ws_need[key] = c.value
    return n


class Workspace:
    """Caller-owned device scratch for the calls that need one: zero-filled
    once here; every call leaves it valid for the next (see include/q4k.h).
    Calls that may run at the same time need distinct workspaces."""

    def __init__(self, nbytes: int, device=None):
        torch = _torch()
        n = max(256, (int(nbytes) + 255) // 256 * 256)
        self.tensor = torch.zeros(n, dtype=torch.uint8,
                                  device=device if device is not None else "cuda")
        if self.tensor.data_ptr() % 256:
            raise RuntimeError("workspace allocation is not 256-byte aligned")
        self.nbytes = n

    @property
    def ptr(self) -> int:
        return self.tensor.data_ptr()


# Default workspaces, one growing chain per (device, stream).  A buffer is
# never released once made: a HIP graph that captured a call keeps using the
# buffer that call was given.
_ws_cache: dict = {}


def _ws(op, M, K, N, ws):
    need = workspace_size(op, M, K, N)
    if ws is not None:
        if not isinstance(ws, Workspace):
            raise TypeError("ws must be a Workspace")
        return ws
    torch = _torch()
    key = (torch.cuda.current_device(), torch.cuda.current_stream().cuda_stream)
    chain = _ws_cache.setdefault(key, [])
    if not chain or chain[-1].nbytes < need:
        chain.append(Workspace(need))
    return chain[-1]


# ---------------------------------------------------------------- calls

def dequant(w, M: int | None = None, K: int | None = None, out=None):
    torch = _torch()
    if M is None:
        M, K = weight_shape(w)
    _weights(w, M, K)
    if out is None:
        out = torch.empty((M, K), dtype=torch.float32, device=w.device)
    _tensor(out, torch.float32, "out", M * K)
    _on_gpu(w=w, out=out)
    check(load().q4k_dequant(w.data_ptr(), out.data_ptr(), M, K, _stream()))
    return out


def gemv(w, x, y=None, M: int | None = None, K: int | None = None, ws=None):
    torch = _torch()
    if M is None:
        M, K = weight_shape(w)
    _weights(w, M, K)
    _tensor(x, torch.float32, "x", K)
    if y is None:
        y = torch.empty(M, dtype=torch.float32, device=w.device)
    _tensor(y, torch.float32, "y", M)
    _on_gpu(w=w, x=x, y=y)
    ws = _ws(OP_GEMV, M, K, 1, ws)
    check(load().q4k_gemv(w.data_ptr(), x.data_ptr(), y.data_ptr(), M, K, ws.ptr, ws.nbytes,
                          _stream()))
    return y


def gemv_noalloc(w, x, y=None, M: int | None = None, K: int | None = None):
    """q4k_gemv_noalloc: the GEMV with its scratch in the library's fixed
    per-device array (no workspace; calls on one GPU must not overlap)."""
    torch = _torch()
    if M is None:
        M, K = weight_shape(w)
    _weights(w, M, K)
    _tensor(x, torch.float32, "x", K)
    if y is None:
        y = torch.empty(M, dtype=torch.float32, device=w.device)
    _tensor(y, torch.float32, "y", M)
    _on_gpu(w=w, x=x, y=y)
    check(load().q4k_gemv_noalloc(w.data_ptr(), x.data_ptr(), y.data_ptr(), M, K, _stream()))
    return y


Q8_BLOCK_BYTES = 34


def gemv_q8_0(w, x, y=None, M: int | None = None, K: int | None = None, ws=None):
    """y = W x for a Q8_0 weight [M, K/32*34] uint8 (K a multiple of 256)."""
    torch = _torch()
    if M is None:
        M, rb = w.shape
        if rb % Q8_BLOCK_BYTES:
            raise ValueError("row length is not a whole number of 34-byte blocks")
        K = rb // Q8_BLOCK_BYTES * 32
    _weights(w, M, K, Q8_BLOCK_BYTES, 32, "Q8_0")
    _tensor(x, torch.float32, "x", K)
    if y is None:
        y = torch.empty(M, dtype=torch.float32, device=w.device)
    _tensor(y, torch.float32, "y", M)
    _on_gpu(w=w, x=x, y=y)
    ws = _ws(OP_GEMV_Q8_0, M, K, 1, ws)
    check(load().q4k_gemv_q8_0(w.data_ptr(), x.data_ptr(), y.data_ptr(), M, K, ws.ptr,
                               ws.nbytes, _stream()))
    return y


Q6_BLOCK_BYTES = 210


def gemv_q6_k(w, x, y=None, M: int | None = None, K: int | None = None, ws=None):
    """y = W x for a Q6_K weight [M, K/256*210] uint8 (K a multiple of 1024)."""
    torch = _torch()
    if M is None:
        M, rb = w.shape
        if rb % Q6_BLOCK_BYTES:
            raise ValueError("row length is not a whole number of 210-byte blocks")
        K = rb // Q6_BLOCK_BYTES * 256
    _weights(w, M, K, Q6_BLOCK_BYTES, 256, "Q6_K")
    _tensor(x, torch.float32, "x", K)
    if y is None:
        y = torch.empty(M, dtype=torch.float32, device=w.device)
    _tensor(y, torch.float32, "y", M)
    _on_gpu(w=w, x=x, y=y)
    ws = _ws(OP_GEMV_Q6_K, M, K, 1, ws)
    check(load().q4k_gemv_q6_k(w.data_ptr(), x.data_ptr(), y.data_ptr(), M, K, ws.ptr,
                               ws.nbytes, _stream()))
    return y


def mlp(w_gate, w_up, w_down, x, norm_w=None, eps: float = 1e-6, resid=None, y=None, act=None,
        hidden: int | None = None, inter: int | None = None, ws=None):
    """y = resid + W_down (silu(W_gate n) * (W_up n)), n = x / rms(x) * (1 + norm_w).

    w_gate, w_up: [inter, hidden/256*144] uint8; w_down: [hidden, inter/256*144].
    norm_w and resid may be None (gain 1, no residual); act, if given, receives
    the activation a = silu(W_gate n) * (W_up n)."""
    torch = _torch()
    if hidden is None:
        inter, hidden = weight_shape(w_gate)
    _weights(w_gate, inter, hidden)
    _weights(w_up, inter, hidden)
    _weights(w_down, hidden, inter)
    _tensor(x, torch.float32, "x", hidden)
    for name, v, n in (("norm_w", norm_w, hidden), ("resid", resid, hidden), ("act", act, inter)):
        if v is not None:
            _tensor(v, torch.float32, name, n)
    if y is None:
        y = torch.empty(hidden, dtype=torch.float32, device=x.device)
    _tensor(y, torch.float32, "y", hidden)
    _on_gpu(w_gate=w_gate, w_up=w_up, w_down=w_down, x=x, norm_w=norm_w, resid=resid, act=act, y=y)
    ws = _ws(OP_MLP, inter, hidden, 0, ws)
    ptr = lambda t: t.data_ptr() if t is not None else None
    check(load().q4k_mlp(w_gate.data_ptr(), w_up.data_ptr(), w_down.data_ptr(), hidden, inter,
                         x.data_ptr(), ptr(norm_w), float(eps), ptr(resid), y.data_ptr(),
                         ptr(act), ws.ptr, ws.nbytes, _stream()))
    return y


def gemv_batch(w, X, Y=None, M: int | None = None, K: int | None = None, ws=None):
    torch = _torch()
    if M is None:
        M, K = weight_shape(w)
    _weights(w, M, K)
    if X.dim() != 2 or X.shape[1] != K:
        raise ValueError("X must be [N, K=%d]" % K)
    N = X.shape[0]
    _tensor(X, torch.float32, "X", N * K)
    if Y is None:
        Y = torch.empty((N, M), dtype=torch.float32, device=w.device)
    _tensor(Y, torch.float32, "Y", N * M)
    _on_gpu(w=w, X=X, Y=Y)
    ws = _ws(OP_GEMV_BATCH, M, K, N, ws)
    check(load().q4k_gemv_batch(w.data_ptr(), X.data_ptr(), Y.data_ptr(), M, K, N, ws.ptr,
                                ws.nbytes, _stream()))
    return Y


def gemm(w, X, Y=None, M: int | None = None, K: int | None = None, ws=None):
    torch = _torch()
    if M is None:
        M, K = weight_shape(w)
    _weights(w, M, K)
    if X.dim() != 2 or X.shape[1] != K:
        raise ValueError("X must be [P, K=%d]" % K)
    P = X.shape[0]
    _tensor(X, torch.float32, "X", P * K)
    if Y is None:
        Y = torch.empty((P, M), dtype=torch.float32, device=w.device)
    _tensor(Y, torch.float32, "Y", P * M)
    _on_gpu(w=w, X=X, Y=Y)
    ws = _ws(OP_GEMM, M, K, P, ws)
    check(load().q4k_gemm(w.data_ptr(), X.data_ptr(), Y.data_ptr(), M, K, P, ws.ptr, ws.nbytes,
                          _stream()))
    return Y


def gdn_step(u, conv_w, a_log, dt_bias, norm_w, conv_state, state, out=None, key_heads=16,
             value_heads=48, eps: float = 1e-6, ws=None):
    """One Gated DeltaNet token (q4k_gdn_step): updates conv_state [C, 3] and
    state [Hv, 128, 128] in place, returns out [Hv*128]."""
    torch = _torch()
    Hk, Hv, D = key_heads, value_heads, 128
    C = (2 * Hk + Hv) * D
    f32 = torch.float32
    _tensor(u, f32, "u", C + Hv * D + 2 * Hv)
    _tensor(conv_w, f32, "conv_w", 4 * C)
    _tensor(a_log, f32, "a_log", Hv)
    _tensor(dt_bias, f32, "dt_bias", Hv)
    _tensor(norm_w, f32, "norm_w", D)
    _tensor(conv_state, f32, "conv_state", 3 * C)
    _tensor(state, f32, "state", Hv * D * D)
    if out is None:
        out = torch.empty(Hv * D, dtype=f32, device=u.device)
    _tensor(out, f32, "out", Hv * D)
    _on_gpu(u=u, conv_w=conv_w, a_log=a_log, dt_bias=dt_bias, norm_w=norm_w,
            conv_state=conv_state, state=state, out=out)
    ws = _ws(OP_GDN_STEP, Hk, Hv, 0, ws)
    prm = GdnParams(Hk, Hv, D, D, float(eps), conv_w.data_ptr(), a_log.data_ptr(),
                    dt_bias.data_ptr(), norm_w.data_ptr())
    check(load().q4k_gdn_step(ctypes.byref(prm), u.data_ptr(), conv_state.data_ptr(),
                              state.data_ptr(), out.data_ptr(), ws.ptr, ws.nbytes, _stream()))
    return out


def attn_step(u, q_norm_w, k_norm_w, k_cache, v_cache, pos: int, out=None, q_heads=24,
              kv_heads=4, rope_dim=64, rope_theta: float = 1e7, eps: float = 1e-6, ws=None):
    """One gated full-attention token at position pos (q4k_attn_step): writes
    position pos of k_cache/v_cache [Hkv, capacity, 256], returns out [Hq*256]."""
    torch = _torch()
    D, f32 = 256, torch.float32
    _tensor(u, f32, "u", q_heads * 2 * D + 2 * kv_heads * D)
    _tensor(q_norm_w, f32, "q_norm_w", D)
    _tensor(k_norm_w, f32, "k_norm_w", D)
    if k_cache.dim() != 3 or k_cache.shape[0] != kv_heads or k_cache.shape[2] != D:
        raise ValueError("k_cache must be [kv_heads, capacity, 256]")
    cap = k_cache.shape[1]
    _tensor(k_cache, f32, "k_cache", kv_heads * cap * D)
    _tensor(v_cache, f32, "v_cache", kv_heads * cap * D)
    if out is None:
        out = torch.empty(q_heads * D, dtype=f32, device=u.device)
    _tensor(out, f32, "out", q_heads * D)
    _on_gpu(u=u, q_norm_w=q_norm_w, k_norm_w=k_norm_w, k_cache=k_cache, v_cache=v_cache, out=out)
    ws = _ws(OP_ATTN_STEP, q_heads, kv_heads, cap, ws)
    prm = AttnParams(q_heads, kv_heads, D, rope_dim, float(rope_theta), float(eps),
                     q_norm_w.data_ptr(), k_norm_w.data_ptr())
    check(load().q4k_attn_step(ctypes.byref(prm), u.data_ptr(), k_cache.data_ptr(),
                               v_cache.data_ptr(), cap, int(pos), out.data_ptr(), ws.ptr,
                               ws.nbytes, _stream()))
    return out


def gemv_config(M: int, K: int, N: int = 1) -> tuple[int, int]:
    wk, ks = ctypes.c_int32(), ctypes.c_int32()
    check(load().q4k_gemv_config(M, K, N, ctypes.byref(wk), ctypes.byref(ks)))
    return wk.value, ks.value


def gemm_config(M: int, K: int, P: int) -> tuple[int, int]:
    """(tile_tokens, workgroups) that q4k_gemm picks for the shape."""
    tt, wg = ctypes.c_int32(), ctypes.c_int32()
    check(load().q4k_gemm_config(M, K, P, ctypes.byref(tt), ctypes.byref(wg)))
    return tt.value, wg.value


def tune_gemv(waves_per_group: int = 0, workgroups: int = 0) -> None:
    """Force the GEMV workgroup count (0: automatic); waves_per_group must be 0 or 4."""
    check(load().q4k_tune_gemv(waves_per_group, workgroups))
    _ws_need.clear()


def check_partition(op: int, M: int, K: int, N: int = 1, workgroups: int = 0) -> None:
    """Host-side check of the work partition a launch would use (no device
    needed); raises Q4KError naming the first violation."""
    check(load().q4k_check_partition(op, M, K, N, workgroups))


def tune_gemm(tile_tokens: int = 0, workgroups: int = 0) -> None:
    """Force the GEMM tile width (0, 32, 64, 128 or 256 tokens) and workgroup count (0: automatic)."""
    check(load().q4k_tune_gemm(tile_tokens, workgroups))
    _ws_need.clear()


class DecodeStack:
    """The per-token projection/MLP chain: one hipGraph launch per token, or
    with ``persistent=True`` one cooperative kernel per token (stand-in mixer
    only; ``spin_limit`` bounds each wait between nodes, 0 = default).

    ``layers``: list of dicts with keys mix_in, mix_out, gate, up, down, each a
    uint8 device tensor [M, K/256*144]; ``lm_head`` likewise.  The tensors are
    borrowed (kept referenced here) and must not be freed while the plan lives.

    ``mixers`` (optional): one dict per layer with the real token mixer's
    parameters — for kind 0 (Gated DeltaNet) conv_w, a_log, dt_bias, norm_w
    (f32 device tensors) and key_heads, value_heads; for kind 1 (attention)
    q_norm_w, k_norm_w and q_heads, kv_heads, rope_dim, rope_theta — with
    ``attn_capacity`` KV-cache positions.
    """

    def __init__(self, layers, lm_head, hidden: int, eps: float = 1e-6, kinds=None, mixers=None,
                 attn_capacity: int = 0, persistent: bool = False, spin_limit: int = 0):
        torch = _torch()
        self._keep = []
        arr = (LayerDesc * max(1, len(layers)))()
        for i, L in enumerate(layers):
            ld = arr[i]
            ld.kind = int(kinds[i]) if kinds is not None else 0
            for name in ("mix_in", "mix_out", "gate", "up", "down"):
                t = L[name]
                M, K = weight_shape(t)
                _weights(t, M, K)
                _on_gpu(**{name: t})
                self._keep.append(t)
                setattr(ld, name, MatDesc(t.data_ptr(), M, K))
        M, K = weight_shape(lm_head)
        _weights(lm_head, M, K)
        _on_gpu(lm_head=lm_head)
        self._keep.append(lm_head)
        self.hidden = hidden
        self.vocab = M
        self.n_layers = len(layers)
        flags, mix_arr = (STACK_PERSISTENT if persistent else 0), None
        if mixers is not None:
            flags |= STACK_MIXERS
            mix_arr = (MixerDesc * max(1, len(layers)))()
            f32 = torch.float32
            for i, m in enumerate(mixers):
                for t in m.values():
                    if isinstance(t, torch.Tensor):
                        _tensor(t, f32, "mixer parameter")
                        _on_gpu(mixer_parameter=t)
                        self._keep.append(t)
                ptr = lambda k: m[k].data_ptr() if k in m else None
                if arr[i].kind == 0:
                    mix_arr[i].gdn = GdnParams(m.get("key_heads", 16), m.get("value_heads", 48),
                                               128, 128, float(m.get("eps", 1e-6)), ptr("conv_w"),
                                               ptr("a_log"), ptr("dt_bias"), ptr("norm_w"))
                else:
                    mix_arr[i].attn = AttnParams(m.get("q_heads", 24), m.get("kv_heads", 4), 256,
                                                 m.get("rope_dim", 64),
                                                 float(m.get("rope_theta", 1e7)),
                                                 float(m.get("eps", 1e-6)), ptr("q_norm_w"),
                                                 ptr("k_norm_w"))
        desc = StackDesc(hidden, len(layers), arr, MatDesc(lm_head.data_ptr(), M, K),
                         float(eps), flags, mix_arr, int(attn_capacity), int(spin_limit))
        self._desc_layers = (arr, mix_arr)
        h = ctypes.c_void_p()
        check(load().q4k_decode_stack_create(ctypes.byref(desc), _stream(), ctypes.byref(h)))
        self._h = h
        self._device = torch.cuda.current_device()

    def reset(self):
        """Mixer states to zero and the position to 0."""
        check(load().q4k_decode_stack_reset(self._h, _stream()))

    def position(self) -> int:
        n = ctypes.c_int64()
        check(load().q4k_decode_stack_position(self._h, ctypes.byref(n)))
        return n.value

    def status(self) -> int:
        """0 if every wait between nodes ended normally since the last call
        (persistent plans; synchronises the current stream), else 1."""
        st = ctypes.c_int32()
        check(load().q4k_decode_stack_status(self._h, _stream(), ctypes.byref(st)))
        return st.value

    def __call__(self, h_in, logits=None):
        torch = _torch()
        _tensor(h_in, torch.float32, "h_in", self.hidden)
        if logits is None:
            logits = torch.empty(self.vocab, dtype=torch.float32, device=h_in.device)
        _tensor(logits, torch.float32, "logits", self.vocab)
        _on_gpu(h_in=h_in, logits=logits)
        check(load().q4k_decode_stack(self._h, h_in.data_ptr(), logits.data_ptr(), _stream()))
        return logits

    def run_no_copy(self, h_in):
        """Launch one token and leave the logits in the arena (see ``buffer``)."""
        torch = _torch()
        _tensor(h_in, torch.float32, "h_in", self.hidden)
        _on_gpu(h_in=h_in)
        check(load().q4k_decode_stack(self._h, h_in.data_ptr(), None, _stream()))

    def buffer_ptr(self, layer: int, which: int) -> tuple[int, int]:
        ptr, n = ctypes.c_void_p(), ctypes.c_int64()
        check(load().q4k_decode_stack_buffer(self._h, layer, which, ctypes.byref(ptr),
                                             ctypes.byref(n)))
        return ptr.value, n.value

    def buffer(self, layer: int, which: int):
        """Device tensor viewing an arena buffer (valid until the next token)."""
        torch = _torch()
        ptr, n = self.buffer_ptr(layer, which)
        view = _DeviceView(ptr, n)
        return torch.as_tensor(view, device="cuda")

    def nodes(self) -> int:
        n = ctypes.c_int64()
        check(load().q4k_decode_stack_nodes(self._h, ctypes.byref(n)))
        return n.value

    def close(self):
        if getattr(self, "_h", None):
            load().q4k_decode_stack_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class _DeviceView:
    """Zero-copy description of a device float32 buffer for torch.as_tensor."""

    def __init__(self, ptr: int, n: int):
        self.__cuda_array_interface__ = {"shape": (n,), "typestr": "<f4", "data": (ptr, False),
                                         "version": 2, "strides": None}
