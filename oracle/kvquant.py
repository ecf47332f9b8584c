"""Per-token, per-head symmetric INT8 KV quantization.

"Performance and Memory" page, section "KV cache INT8 -- 2x context at matched
VRAM": each cached K or V row of one (token, head) is stored as INT8 with one
FP16 scale. The scale is max|x| / 127 stored in FP16.

Reading of the steps (the page names the scheme, not its rounding):
  amax = max |x| over the head_dim values (float32, exact);
  s    = fp16(amax / 127), the float32 quotient correctly rounded, then
         rounded to nearest-even FP16;
  q    = clamp(rint(x / f32(s)), -127, 127), the float32 quotient correctly
         rounded and rint rounding half to even; q = 0 when s == 0;
  x^   = f32(q) * f32(s)  (exact in float32).
These decisions are taken in float32 on purpose: a quantized code is an
integer decided by floating point, and both implementations must decide it in
the same precision.
"""
import numpy as np


def kv_quantize(x: np.ndarray):
    """x: float16 [..., hd] -> (int8 [..., hd], float16 [...])."""
    x32 = np.asarray(x, dtype=np.float16).astype(np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    s16 = np.divide(amax, np.float32(127.0), dtype=np.float32).astype(np.float16)
    s32 = s16.astype(np.float32)[..., None]
    ratio = np.divide(x32, s32, out=np.zeros_like(x32), where=s32 > 0)
    q = np.clip(np.rint(ratio), -127, 127)
    q = np.where(s32 > 0, q, 0).astype(np.int8)
    return q, s16


def kv_dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """(int8 [..., hd], float16 [...]) -> float64 values f32(q) * f32(s)."""
    v = q.astype(np.float32) * np.asarray(s, dtype=np.float16).astype(np.float32)[..., None]
    return v.astype(np.float64)


def kv_cache_bytes(n_layers: int, max_seq: int, n_heads: int, head_dim: int, int8: bool) -> int:
    """Bytes of one lane's K and V cache over n_layers effective layers.

    FP16: 2 (K and V) * layers * max_seq * heads * head_dim * 2 bytes.
    INT8: 2 * layers * max_seq * heads * (head_dim bytes + one 2-byte scale).
    The same page prints 167.8 MB vs 85.2 MB at max_seq=2048 over 10 layers.
    """
    per_row = head_dim + 2 if int8 else head_dim * 2
    return 2 * n_layers * max_seq * n_heads * per_row


# ---------------------------------------------------------------- store-h INT8
# "Current Status" page, KV-cache table: Store-h (INT8), 66-75% less memory than
# FP16 K/V. The page names the mode and its saving, not the scheme. Reading:
# each 128-element group of an h row is quantized exactly like one INT8 K/V
# row above (symmetric, one FP16 scale per group); the rows K and V are rebuilt
# from are h^ = fp16(q * s), the FP16 A operand of the rebuild product. With
# d = 2048 that keeps d + 2 d / 128 bytes per position and layer against
# 4 d for FP16 K and V: 74.6% less, inside the page's range.
H_GROUP = 128


def h_quantize(h: np.ndarray):
    """h: float16-valued [n][d] (d a multiple of 128) -> (int8 [n][d],
    float16 [n][d / 128]), each 128-element group quantized as kv_quantize does."""
    h = np.asarray(h)
    n, d = h.shape
    if d % H_GROUP:
        raise ValueError("d must be a multiple of 128")
    q, s = kv_quantize(h.astype(np.float16).reshape(n, d // H_GROUP, H_GROUP))
    return q.reshape(n, d), s


def h_dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """(int8 [n][d], float16 [n][d / 128]) -> float64 values of fp16(q * s).
    The product of an int8 and an fp16 is exact in float64 (and float32);
    it is rounded once, to nearest-even FP16."""
    n, d = q.shape
    v = q.reshape(n, d // H_GROUP, H_GROUP).astype(np.float64) * \
        np.asarray(s, dtype=np.float16).astype(np.float64)[..., None]
    return v.astype(np.float16).astype(np.float64).reshape(n, d)


def store_h_bytes(n_layers: int, max_seq: int, d_model: int, int8: bool) -> int:
    """Bytes of one lane's store-h cache over n_layers effective layers:
    FP16 h: d_model * 2 per position; INT8 h: d_model codes + d_model / 128
    fp16 scales per position."""
    per_pos = d_model + 2 * (d_model // H_GROUP) if int8 else 2 * d_model
    return n_layers * max_seq * per_pos
