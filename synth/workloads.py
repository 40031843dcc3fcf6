"""Shapes and stream keys of the synthetic workloads (harness code).

Shapes are those of Qwen3.6-27B as the parity page lists it ("Qwen3.6-27B on
Apple M3 Pro — the llama.cpp parity bar", architecture list: 64 layers, hidden
5120, intermediate 17408, vocab 248320, 48 Gated-DeltaNet + 16 full-attention
layers with full_attention_interval 4) and the per-phase matmuls of the
decode profile ("Mac Qwen3.6-27B Metal Q4_K perf diagnosis", §2).  Derived
projection widths: attention qkv 14336 = 24*256*2 + 4*256*2, o K = 24*256;
GDN in_proj 16480 = 2*16*128 + 2*48*128 + 2*48, out_proj K = 48*128.

Weights are random Q4_K super-blocks from ``synth.q4k_weight`` (d, dmin
~U(1e-4, 1e-3) in binary16, uniform scale/min bytes and nibbles); activations
are N(0, 1) f32.  They stand in for the real q4_k_m weights and chat prompts,
which are not available here.
"""
from __future__ import annotations

from . import key

HIDDEN = 5120
INTER = 17408
VOCAB = 248320
N_LAYERS = 64
ATTN_EVERY = 4

SINGLE = [(512, 1024), (1024, 512)]            # input set 1, both readings of "2 blocks/row"
MLP = [("gate", 17408, 5120), ("up", 17408, 5120), ("down", 5120, 17408)]   # set 2
BATCH_SHAPE = (17408, 5120)                    # set 4
BATCH_N = [1, 2, 4, 8, 16]
PREFILL_SHAPES = [(17408, 5120), (5120, 17408)]  # set 5
PREFILL_P = [256, 512, 1024]

GDN_SHAPES = {"mix_in": (16480, HIDDEN), "mix_out": (HIDDEN, 6144)}
ATTN_SHAPES = {"mix_in": (14336, HIDDEN), "mix_out": (HIDDEN, 6144)}
MLP_SHAPES = {"gate": (INTER, HIDDEN), "up": (INTER, HIDDEN), "down": (HIDDEN, INTER)}
LAYER_MATS = ("mix_in", "mix_out", "gate", "up", "down")


def is_attention(layer: int) -> bool:
    """Layer pattern: every fourth layer is full attention (offset 3)."""
    return layer % ATTN_EVERY == ATTN_EVERY - 1


def layer_shapes(layer: int) -> dict:
    sh = dict(ATTN_SHAPES if is_attention(layer) else GDN_SHAPES)
    sh.update(MLP_SHAPES)
    return sh


def stack_tensor_key(layer: int | None, mat: str, cfg: int = 3) -> int:
    """Key of a decode-stack matrix (layer None: lm_head)."""
    if layer is None:
        return key(cfg, 5 * N_LAYERS)
    return key(cfg, 5 * layer + LAYER_MATS.index(mat))


def stack_bytes(n_layers: int = N_LAYERS) -> int:
    total = 0
    for l in range(n_layers):
        for M, K in layer_shapes(l).values():
            total += M * (K // 256) * 144
    return total + VOCAB * (HIDDEN // 256) * 144
