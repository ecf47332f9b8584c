// W4A16 matrix kernels on MFMA (gfx950, v_mfma_f32_16x16x32_f16): the
// epilogue helpers and the LDS barrier that the decode GEMV (w4gemv.hip) and
// the prefill GEMM (w4mm.hip) share.
//
// Both kernels compute C[m][n] = sum_k A[m][k] * W[n][k] with
// W[n][k] = q[n][k] * s[n][k/128] (the loop block's INT4 weights, one FP16
// scale per 128 inputs). The packed weight tile of one (16-row n-block,
// 128-column group) is loaded straight from HBM into registers, 16 bytes per
// lane, already in MFMA B-operand order; its 4-bit values are turned into
// exact fp16 integers in registers; the four 32-deep MFMA k-steps of the group
// accumulate q * a exactly into a fresh fp32 tile, which is then scaled by
// the group scale and added to the running fp32 sum. The scale is therefore
// applied in fp32 after an exact integer-weight contraction, so the only
// rounding is fp32 accumulation.
#pragma once
#include "tl_device.h"
#include "tl_kernels.h"

namespace tl {

// ---------------------------------------------------------------- epilogue
__device__ __forceinline__ size_t epi_index(const Epi& e, int m, int n) {
  return (size_t)m * e.ldo + (e.perm_hd ? qkv_natural_col(n, e.perm_hd) : n);
}
__device__ __forceinline__ void epi_swiglu(const Epi& e, int m, int c, float g, float u) {
  e.out_f16[(size_t)m * e.ldo + c] = f2h(silu(g) * u);
}

// Waits for this wave's LDS accesses, then the block barrier (LDS only:
// global requests stay in flight across it).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace tl
