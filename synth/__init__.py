"""Seeded synthetic inputs for the looped weight-shared transformer.

This module only draws random numbers in the shapes and distributions of the
model family (TinyLoop docs, "TinyLoop Framework" intro page: embed, pre-blocks,
one shared loop block, final norm and head). It holds none of the forward
pass's arithmetic, so both the CPU oracle and the GPU library can take their
inputs from here without sharing any computation.

Weight format handed out (the canonical layout):
  qweight  uint32 [N][K/8]   eight signed 4-bit values per word along K,
                              element k%8 in bits 4*(k%8)..4*(k%8)+3
  scales   float16 [N][ceil(K/g)]  one scale per g=128 input channels

Random 32-bit words are drawn directly: every nibble of a uniform word is
uniform on 0..15, which is exactly a uniform signed 4-bit value on [-8, 7]
under two's complement, and nibbles are independent.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["Shape", "SHAPES", "make_weights", "make_tokens", "block_linear_shapes",
           "weights_nbytes"]


@dataclasses.dataclass(frozen=True)
class Shape:
    vocab: int
    d_model: int
    n_heads: int
    head_dim: int
    ffn_dim: int
    n_pre: int
    group_size: int = 128
    rope_base: float = 10000.0
    rms_eps: float = 1e-5


SHAPES = {
    # tiny looped transformer: 1 pre-block + 1 loop block, d 256, 4 heads x 64, ffn 704
    "tiny": Shape(vocab=1024, d_model=256, n_heads=4, head_dim=64, ffn_dim=704, n_pre=1),
    # 407M-shaped model: 2 pre-blocks + 1 loop block, d 2048, 16 heads x 128, ffn 5632
    "m407": Shape(vocab=50304, d_model=2048, n_heads=16, head_dim=128, ffn_dim=5632, n_pre=2),
    # very small shape for brute-force checks
    "micro": Shape(vocab=64, d_model=32, n_heads=2, head_dim=16, ffn_dim=48, n_pre=1, group_size=16),
}

LINEARS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def block_linear_shapes(s: Shape) -> dict:
    """(N_out, K_in) of every linear in one transformer block."""
    d, f = s.d_model, s.ffn_dim
    return {"wq": (d, d), "wk": (d, d), "wv": (d, d), "wo": (d, d),
            "w_gate": (f, d), "w_up": (f, d), "w_down": (d, f)}


def _draw_linear(rng, n, k, g, scale_mult=1.0):
    if k % 8:
        raise ValueError("K must be a multiple of 8")
    qweight = rng.integers(0, 2**32, size=(n, k // 8), dtype=np.uint32)
    ng = -(-k // g)
    scales = (0.02 / 7.0 * scale_mult) * rng.uniform(0.5, 1.5, size=(n, ng))
    return {"qweight": qweight, "scales": scales.astype(np.float16)}


def make_weights(s: Shape, seed: int = 0, gains: str = "ones", q_scale_mult: float = 1.0) -> dict:
    """Seeded synthetic model.

    Draw order from default_rng(seed): embed, then for each block (pre..., loop)
    the seven linears in LINEARS order (words, then scales), then head.
    gains="ones" gives unit RMSNorm gains; gains="random" draws
    fp16(1 + U(-0.1, 0.1)) from default_rng(seed + 7) so the INT4 weights are the
    same in both modes. q_scale_mult multiplies the W_q scales (sharper
    attention, so masking mistakes change the output visibly).
    """
    rng = np.random.default_rng(seed)
    d, V = s.d_model, s.vocab
    embed = rng.normal(0.0, 0.02, size=(V, d)).astype(np.float16)
    shapes = block_linear_shapes(s)
    blocks = []
    for _ in range(s.n_pre + 1):
        blk = {}
        for name in LINEARS:
            n, k = shapes[name]
            blk[name] = _draw_linear(rng, n, k, s.group_size,
                                     q_scale_mult if name == "wq" else 1.0)
        blocks.append(blk)
    head = rng.normal(0.0, 0.02, size=(V, d)).astype(np.float16)
    grng = np.random.default_rng(seed + 7)

    def gain():
        if gains == "ones":
            return np.ones(d, dtype=np.float16)
        if gains == "random":
            return (1.0 + grng.uniform(-0.1, 0.1, size=d)).astype(np.float16)
        raise ValueError(gains)

    for blk in blocks:
        blk["attn_norm"] = gain()
        blk["mlp_norm"] = gain()
    final_norm = gain()
    return {"shape": s, "embed": embed, "pre": blocks[:s.n_pre], "loop": blocks[s.n_pre],
            "final_norm": final_norm, "head": head}


def make_tokens(vocab: int, n: int, seed: int = 0, lane: int = 0) -> np.ndarray:
    """Prompt token ids, uniform on [0, vocab), from default_rng(seed + 1000 + lane)."""
    rng = np.random.default_rng(seed + 1000 + lane)
    return rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def weights_nbytes(s: Shape) -> dict:
    """Byte counts of the canonical tensors (packed words + fp16 scales)."""
    per_block = 0
    for n, k in block_linear_shapes(s).values():
        per_block += n * k // 2 + n * math.ceil(k / s.group_size) * 2
    return {"block_w4": per_block, "embed": s.vocab * s.d_model * 2,
            "head": s.vocab * s.d_model * 2}
