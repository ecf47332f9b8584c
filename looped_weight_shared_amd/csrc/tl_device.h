// Device-side helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

#define TL_WAVE 64

namespace tl {

// ---------------------------------------------------------------------------
// Packed INT4 layout (see pack.hip): a tile covers 16 output rows x 128 input
// columns, 1 KiB, and lane l of a wave owns the 16-byte slot l of the tile:
// word s (0..3) of the slot holds the 8 values of row 16*nb + l%16 at columns
// 128*g + 32*s + 8*(l/16) + 0..7, which is exactly the B operand of one
// v_mfma_f32_16x16x32_f16 k-step. Nibble p holds column 2p and nibble p+4
// column 2p+1 (so each 16-bit half of (w >> 4p) & 0x000F000F is one element
// of a consecutive pair), stored offset-binary u = q + 8.
// ---------------------------------------------------------------------------
constexpr int kTileBytes = 1024;
constexpr int kTileBytesF16 = 4096;  // dense fp16 body tile
constexpr int kGroup = 128;

// 8 signed 4-bit values of one packed word -> 8 exact fp16 integers in
// column order. The nibble pairs (0,4) and (2,6) of the word (the latter after
// a shift by 8) sit at bits 0 and 16, where OR-ing them into the mantissa of
// 1024.0h gives 1024 + u exactly; the pairs (1,5) and (3,7) sit at bits 4 and
// 20, which gives 1024 + 16u exactly. One packed subtract of 1032, or one
// packed fma by 1/16 minus 72, then gives q = u - 8 exactly (every
// intermediate is an integer below 2048 or a power-of-two multiple of one).
// The mask-and-or is one v_and_or_b32 (its constants come from registers:
// this encoding cannot carry literals).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(c));
  return r;
}
__device__ __forceinline__ half8_t dequant_word(uint32_t w) {
  const uint32_t magic = 0x64006400u, lo = 0x000F000Fu, hi = 0x00F000F0u;
  const uint32_t w8 = w >> 8;
  const half2_t t0 = __builtin_bit_cast(half2_t, and_or(w, lo, magic));   // 1024 + u, nibbles 0, 4
  const half2_t t1 = __builtin_bit_cast(half2_t, and_or(w, hi, magic));   // 1024 + 16u, nibbles 1, 5
  const half2_t t2 = __builtin_bit_cast(half2_t, and_or(w8, lo, magic));  // nibbles 2, 6
  const half2_t t3 = __builtin_bit_cast(half2_t, and_or(w8, hi, magic));  // nibbles 3, 7
  const half2_t bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const half2_t k16 = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t b72 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const half2_t a0 = t0 + bias, a2 = t2 + bias;
  const half2_t a1 = __builtin_elementwise_fma(t1, k16, b72), a3 = __builtin_elementwise_fma(t3, k16, b72);
  half8_t r = {a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
  return r;
}

__device__ __forceinline__ float4_t mfma16(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ uint16_t f2h(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);  // round to nearest even
}

// Reductions over the 16 lanes of one row of the wave (lanes 16r..16r+15)
// and over the whole wave, on DPP lane moves instead of LDS permutes: swap
// neighbours, swap pairs (quad_perm), then half-row and row mirrors add the
// other quad and the other half, so every lane of the row ends with the same
// bits (each step adds two equal-order operands: a + b on one side, b + a on
// the other). The wave-wide forms read the four row results with readlane
// and combine them in row order (a uniform value). Callers run them with the
// whole wave active.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7 - i within each 8
constexpr int kDppMirror = 0x140;      // lane i <- lane 15 - i within each 16
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<kDppXor1>(v);
  v += dpp_mov<kDppXor2>(v);
  v += dpp_mov<kDppHalfMirror>(v);
  v += dpp_mov<kDppMirror>(v);
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_mov<kDppXor1>(v));
  v = fmaxf(v, dpp_mov<kDppXor2>(v));
  v = fmaxf(v, dpp_mov<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_mov<kDppMirror>(v));
  return v;
}
// Max and sum over the four rows' copies of a lane's value (lanes n, n + 16,
// n + 32, n + 48), on gfx950's row swaps instead of LDS permutes:
// v_permlane16_swap with both operands holding x leaves rows (0, 0, 2, 2) in
// the one and (1, 1, 3, 3) in the other, so their elementwise max (sum) is
// the xor-16 butterfly step in every lane; v_permlane32_swap does the same
// for the halves. Both operands of every step are the same two values in
// each lane of a query, so all four lanes end with the same bits.
__device__ __forceinline__ float rows4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// The same over aligned groups of N = 8 or 16 lanes.
template <int N>
__device__ __forceinline__ float lanes_sum(float v) {
  static_assert(N == 8 || N == 16, "groups of 8 or 16 lanes");
  if constexpr (N == 16) return row16_sum(v);
  v += dpp_mov<kDppXor1>(v);
  v += dpp_mov<kDppXor2>(v);
  return v + dpp_mov<kDppHalfMirror>(v);
}
template <int N>
__device__ __forceinline__ float lanes_max(float v) {
  static_assert(N == 8 || N == 16, "groups of 8 or 16 lanes");
  if constexpr (N == 16) return row16_max(v);
  v = fmaxf(v, dpp_mov<kDppXor1>(v));
  v = fmaxf(v, dpp_mov<kDppXor2>(v));
  return fmaxf(v, dpp_mov<kDppHalfMirror>(v));
}
// (value, index) maximum with ties to the lower index (a total order, so both
// lanes of an exchange keep the same winner) over the 16 lanes of a row, and
// over the wave (uniform result).
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
  const float ov = dpp_mov<CTRL>(v);
  const int oi = __builtin_amdgcn_mov_dpp(i, CTRL, 0xF, 0xF, true);
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}
__device__ __forceinline__ void row16_argmax(float& v, int& i) {
  argmax_step<kDppXor1>(v, i);
  argmax_step<kDppXor2>(v, i);
  argmax_step<kDppHalfMirror>(v, i);
  argmax_step<kDppMirror>(v, i);
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  row16_argmax(v, i);
  float bv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float rv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16 * r));
    const int ri = __builtin_amdgcn_readlane(i, 16 * r);
    if (rv > bv || (rv == bv && ri < bi)) {
      bv = rv;
      bi = ri;
    }
  }
  v = bv;
  i = bi;
}
constexpr int kDppRor8 = 0x128;  // lane i <- lane (i + 8) mod 16 within each 16: the xor-8 partner
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
}

// e^-z as 2^(-z log2 e): one v_exp_f32 (saturates to +inf for very negative z,
// where the quotient is -0, as with expf)
__device__ __forceinline__ float silu(float z) { return z / (1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z)); }

// RoPE-pair packing of the QKV rows: within each head of hd rows, packed
// row 16j + r holds natural row 8j + r (r < 8, first half of rotation pair
// 8j + r) or hd/2 + 8j + r - 8 (r >= 8, its second half).
__host__ __device__ __forceinline__ int rope_pair_row(int p, int hd) {
  const int j = p >> 4, r = p & 15;
  return r < 8 ? 8 * j + r : hd / 2 + 8 * j + (r - 8);
}
__host__ __device__ __forceinline__ int qkv_natural_col(int n, int hd) {
  const int p = n % hd;
  return n - p + rope_pair_row(p, hd);
}

// Rotary embedding of one pair (x1 = dim i, x2 = dim i + hd/2) by the angle
// whose cos/sin are c, s; both results are rounded to fp16 (Q and K cast
// points). Every kernel that rotates uses this one expression.
__device__ __forceinline__ void rope_pair(float x1, float x2, float c, float s, _Float16* r1, _Float16* r2) {
  *r1 = (_Float16)(x1 * c - x2 * s);
  *r2 = (_Float16)(x2 * c + x1 * s);
}

// INT8 KV quantizer of one (token, head) row: scale = fp16(amax / 127) with a
// correctly rounded fp32 division, code = clamp(rint(x / f32(scale)), -127,
// 127) with a correctly rounded division and round-half-even, 0 when the
// scale is 0.
__device__ __forceinline__ _Float16 kv_scale(float amax) { return (_Float16)__fdiv_rn(amax, 127.0f); }
__device__ __forceinline__ int kv_code(float x, float sf) {
  if (!(sf > 0.f)) return 0;
  return (int)fminf(fmaxf(rintf(__fdiv_rn(x, sf)), -127.f), 127.f);
}

// Decode attention writes, per (row, head, key part), the part's softmax
// state: weighted value sums [hd], then the running max and the sum of
// weights, in a row of hd + kAttnPartExtra floats (16-byte aligned rows).
// Scores and maxima are in log2 units (log2 e folded into the softmax scale),
// so a weight is 2^(score - max), one v_exp_f32.
// Parts are combined in part order by attn_merge_step; a part with max -inf
// (beyond the row's context) is skipped. The merge kernel and the O-projection
// GEMV both use this, so either path gives the same bits.
constexpr int kAttnPartExtra = 4;
__device__ __forceinline__ void attn_merge_step(float gm, float mp, float lp, float nump, float& num, float& den) {
  if (mp != -INFINITY) {
    const float w = __builtin_amdgcn_exp2f(mp - gm);
    num = fmaf(w, nump, num);
    den = fmaf(w, lp, den);
  }
}

}  // namespace tl
