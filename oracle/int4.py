"""Packed signed INT4 weights: unpack, pack, exact dequantization.

The pages run the loop block on low-bit weights ("TinyLoop Framework" intro
page, "What Makes It Different": INT2/INT4 execution) but print no layout. The
layout followed here is the plainest reading of "eight values per 32-bit word
along K, one FP16 scale per 128 input channels, symmetric values in [-8, 7]":

  * element k of a row lives in word k // 8, bits 4*(k % 8) .. 4*(k % 8) + 3,
    least significant nibble first;
  * a nibble is a two's-complement 4-bit integer (no zero point);
  * matrices are [N_out][K_in] (one output row's K contiguous), scales are
    [N_out][ceil(K / g)], and a partial last group covers the leftover columns.
"""
import numpy as np


def unpack_int4(qweight: np.ndarray) -> np.ndarray:
    """uint32 [..., K/8] -> int8 [..., K] with values in [-8, 7]."""
    w = np.asarray(qweight, dtype=np.uint32)
    out = np.empty(w.shape[:-1] + (w.shape[-1] * 8,), dtype=np.int8)
    for j in range(8):
        nib = ((w >> np.uint32(4 * j)) & np.uint32(0xF)).astype(np.int16)
        out[..., j::8] = np.where(nib >= 8, nib - 16, nib).astype(np.int8)
    return out


def pack_int4(q: np.ndarray) -> np.ndarray:
    """int [..., K] in [-8, 7] -> uint32 [..., K/8]; inverse of unpack_int4."""
    q = np.asarray(q)
    if q.shape[-1] % 8:
        raise ValueError("K must be a multiple of 8")
    if q.min(initial=0) < -8 or q.max(initial=0) > 7:
        raise ValueError("values must lie in [-8, 7]")
    nib = (q.astype(np.int64) & 0xF).astype(np.uint32)
    out = np.zeros(q.shape[:-1] + (q.shape[-1] // 8,), dtype=np.uint32)
    for j in range(8):
        out |= nib[..., j::8] << np.uint32(4 * j)
    return out


def dequantize(qweight: np.ndarray, scales: np.ndarray, group_size: int = 128) -> np.ndarray:
    """W[n, k] = int4(n, k) * scale[n, k // g], as float64.

    The product of an integer of at most 4 bits and an FP16 scale (11-bit
    significand) is exact in float32 and float64, so this is the exact weight
    matrix the model is defined by.
    """
    q = unpack_int4(qweight).astype(np.float64)
    k = q.shape[-1]
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    if s.shape[-1] != -(-k // group_size):
        raise ValueError("scales must have ceil(K/g) columns")
    return q * np.repeat(s, group_size, axis=-1)[..., :k]
