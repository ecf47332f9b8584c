// Causal attention over the per-layer KV cache (gfx950).
//
// Cache layout of one (lane, effective layer): K then V, each [H][S][hd]
// fp16; or, in INT8 mode, Kq int8 [H][S][hd], Ks fp16 [H][S], Vq, Vs (one
// FP16 scale per token and head: "Performance and Memory" page, "KV cache
// INT8"). Attention always reads what the cache holds, so an INT8 cache is
// read back as q * s in the prefill too (cached and uncached paths agree).
//
// Prefill: a block takes 64 queries of one head (4 waves x 16 rows) and walks
// 64-key tiles up to its causal limit: K tile and transposed V tile staged in
// LDS, S = Q K^T and O += P V on v_mfma_f32_16x16x32_f16, online softmax in
// fp32 (running max and sum per row). INT8 codes are exact in fp16, so the
// MFMAs run on the codes and the per-key scales multiply the score columns
// and the probabilities (P is rounded to fp16 for the PV MFMA).
//
// Decode: one query per lane; the context is cut in 128-key chunks, each
// block (2 waves) scores its chunk with 16 lanes per key (8 dims each), keeps
// the chunk max/sum and the unnormalised P V in fp32, and a combine pass
// merges the chunks of a head in chunk order.
#include "tl_device.h"
#include "tl_kernels.h"

namespace tl {

struct CachePtrs {
  const uint8_t* k;   // fp16 [S][hd] or int8 [S][hd] of this head
  const uint8_t* v;
  const uint16_t* ks;  // int8 mode: fp16 scales [S]
  const uint16_t* vs;
};

__device__ __forceinline__ CachePtrs cache_ptrs(const KvGeom& kv, int lane, int layer, int h) {
  const uint8_t* base = kv.base + ((size_t)lane * kv.n_layers + layer) * kv.layer_bytes;
  const size_t HS = (size_t)kv.H * kv.S;
  CachePtrs c;
  if (kv.int8) {
    c.k = base + (size_t)h * kv.S * kv.hd;
    c.ks = reinterpret_cast<const uint16_t*>(base + HS * kv.hd) + (size_t)h * kv.S;
    c.v = base + HS * kv.hd + HS * 2 + (size_t)h * kv.S * kv.hd;
    c.vs = reinterpret_cast<const uint16_t*>(base + 2 * HS * kv.hd + HS * 2) + (size_t)h * kv.S;
  } else {
    c.k = base + (size_t)h * kv.S * kv.hd * 2;
    c.v = base + HS * kv.hd * 2 + (size_t)h * kv.S * kv.hd * 2;
    c.ks = c.vs = nullptr;
  }
  return c;
}

// 8 cache values of one row as fp16 (INT8 codes are exact in fp16).
__device__ __forceinline__ u32x4_t load8_as_f16(const uint8_t* row, int d0, int int8) {
  if (!int8) return *reinterpret_cast<const u32x4_t*>(row + d0 * 2);
  const uint2 c = *reinterpret_cast<const uint2*>(row + d0);
  half8_t h;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = (_Float16)(float)(int8_t)((c.x >> (8 * j)) & 0xFF);
    h[4 + j] = (_Float16)(float)(int8_t)((c.y >> (8 * j)) & 0xFF);
  }
  return __builtin_bit_cast(u32x4_t, h);
}

// ------------------------------------------------------------------ prefill
template <int HD>
__global__ __launch_bounds__(256) void attn_prefill_kernel(const uint16_t* __restrict__ q, int M, int lane_id,
                                                           int p0, KvGeom kv, int layer, uint16_t* __restrict__ o) {
  constexpr int KS = HD / 32;     // k-steps of S = Q K^T
  constexpr int DB = HD / 16;     // 16-wide d blocks of O
  constexpr int LK = HD + 8;      // LDS row stride of the K tile (halves)
  constexpr int LV = 64 + 8;      // LDS row stride of the transposed V tile
  __shared__ __align__(16) _Float16 Ks[64 * LK];
  __shared__ __align__(16) _Float16 Vt[HD * LV];
  __shared__ __align__(16) _Float16 Ps[4][16 * LV];
  __shared__ float ksc[64], vsc[64];

  const int tid = threadIdx.x, wave = tid >> 6, ln = tid & 63;
  const int l16 = ln & 15, lq = ln >> 4;
  const int h = blockIdx.y;
  const int q0 = blockIdx.x * 64;
  const int d = kv.H * HD;
  const int kend = p0 + min(q0 + 64, M);  // keys [0, kend) can be visible to this block
  const CachePtrs cp = cache_ptrs(kv, lane_id, layer, h);
  const float scale = 1.0f / sqrtf((float)HD);

  // Q fragments (A operand of S): row q0 + 16*wave + l16, dims 32s + 8lq .. +7
  half8_t qf[KS];
  {
    const int qr = q0 + 16 * wave + l16;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4_t v = {0, 0, 0, 0};
      if (qr < M) v = *reinterpret_cast<const u32x4_t*>(q + (size_t)qr * d + h * HD + 32 * s + 8 * lq);
      qf[s] = __builtin_bit_cast(half8_t, v);
    }
  }
  float mrow[4], lrow[4];
  float4_t oacc[DB];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    mrow[r] = -INFINITY;
    lrow[r] = 0.f;
  }
#pragma unroll
  for (int b = 0; b < DB; ++b) oacc[b] = (float4_t){0.f, 0.f, 0.f, 0.f};
  const int qpos_base = p0 + q0 + 16 * wave + 4 * lq;  // + r

  const int nkt = (kend + 63) / 64;
  for (int kt = 0; kt < nkt; ++kt) {
    const int key0 = kt * 64;
    // ---- stage K (row-major) and V (transposed) for keys key0..key0+63
    for (int c = tid; c < 64 * HD / 8; c += 256) {
      const int kr = c / (HD / 8), d0 = (c % (HD / 8)) * 8;
      const int key = key0 + kr;
      u32x4_t kvv = {0, 0, 0, 0}, vvv = {0, 0, 0, 0};
      if (key < kend) {
        const size_t roff = (size_t)key * HD * (kv.int8 ? 1 : 2);
        kvv = load8_as_f16(cp.k + roff, d0, kv.int8);
        vvv = load8_as_f16(cp.v + roff, d0, kv.int8);
      }
      *reinterpret_cast<u32x4_t*>(&Ks[kr * LK + d0]) = kvv;
      const half8_t vh = __builtin_bit_cast(half8_t, vvv);
#pragma unroll
      for (int j = 0; j < 8; ++j) Vt[(d0 + j) * LV + kr] = vh[j];
    }
    if (tid < 64) {
      const int key = key0 + tid;
      float a = 1.f, b = 1.f;
      if (kv.int8) {
        a = key < kend ? h2f(cp.ks[key]) : 0.f;
        b = key < kend ? h2f(cp.vs[key]) : 0.f;
      }
      ksc[tid] = a * scale;
      vsc[tid] = b;
    }
    __syncthreads();

    // ---- S = Q K^T for 16 rows x 64 keys (lane: rows 4lq+r, key 16kb + l16)
    float sv[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float4_t t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const half8_t bf = *reinterpret_cast<const half8_t*>(&Ks[(kb * 16 + l16) * LK + 32 * s + 8 * lq]);
        t = mfma16(qf[s], bf, t);
      }
      const int key = key0 + kb * 16 + l16;
      const float ks = ksc[kb * 16 + l16];
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[kb][r] = (key <= qpos_base + r) ? t[r] * ks : -INFINITY;
    }
    // ---- online softmax per row
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float mx = fmaxf(fmaxf(sv[0][r], sv[1][r]), fmaxf(sv[2][r], sv[3][r]));
      mx = row16_max(mx);
      const float mnew = fmaxf(mrow[r], mx);
      const float alpha = expf(mrow[r] - mnew);  // 0 on the first tile (mrow = -inf)
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float p = expf(sv[kb][r] - mnew);
        ps += p;
        sv[kb][r] = p;
      }
      ps = row16_sum(ps);
      lrow[r] = lrow[r] * alpha + ps;
      mrow[r] = mnew;
#pragma unroll
      for (int b = 0; b < DB; ++b) oacc[b][r] *= alpha;
    }
    // ---- P (fp16, value scale folded in) through LDS into A-operand order
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const float vs = vsc[kb * 16 + l16];
#pragma unroll
      for (int r = 0; r < 4; ++r) Ps[wave][(4 * lq + r) * LV + kb * 16 + l16] = (_Float16)(sv[kb][r] * vs);
    }
    __syncthreads();
    half8_t pa[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) pa[s] = *reinterpret_cast<const half8_t*>(&Ps[wave][l16 * LV + 32 * s + 8 * lq]);
    // ---- O += P V
#pragma unroll
    for (int b = 0; b < DB; ++b) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const half8_t bf = *reinterpret_cast<const half8_t*>(&Vt[(b * 16 + l16) * LV + 32 * s + 8 * lq]);
        oacc[b] = mfma16(pa[s], bf, oacc[b]);
      }
    }
    __syncthreads();
  }
  // ---- normalise and store rows q0 + 16*wave + 4lq + r
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int qr = q0 + 16 * wave + 4 * lq + r;
    if (qr >= M) continue;
    const float inv = 1.0f / lrow[r];
#pragma unroll
    for (int b = 0; b < DB; ++b) o[(size_t)qr * d + h * HD + b * 16 + l16] = f2h(oacc[b][r] * inv);
  }
}

hipError_t launch_attn_prefill(const uint16_t* q, int M, int lane, int p0, const KvGeom& kv, int layer,
                               uint16_t* o, hipStream_t s) {
  dim3 grid((M + 63) / 64, kv.H);
  if (kv.hd == 128)
    hipLaunchKernelGGL(attn_prefill_kernel<128>, grid, dim3(256), 0, s, q, M, lane, p0, kv, layer, o);
  else if (kv.hd == 64)
    hipLaunchKernelGGL(attn_prefill_kernel<64>, grid, dim3(256), 0, s, q, M, lane, p0, kv, layer, o);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ------------------------------------------------------------------ decode
constexpr int kChunk = 128;  // keys per decode block (2 waves x 64)

size_t attn_decode_scratch_floats(int max_rows, int H, int hd, int S) {
  const int nch = (S + kChunk - 1) / kChunk;
  return (size_t)max_rows * H * nch * (hd + 2);
}

template <int HD>
__global__ __launch_bounds__(128) void attn_decode_kernel(const uint16_t* __restrict__ q, RowMap rm, KvGeom kv,
                                                          int layer, float* __restrict__ part) {
  constexpr int LPK = HD / 8;    // lanes per key
  constexpr int KPP = 64 / LPK;  // keys per wave pass
  constexpr int NP = 64 / KPP;   // passes per wave (64 keys per wave)
  __shared__ float red_m[2], red_l[2];
  __shared__ float red_o[2][HD];

  const int chunk = blockIdx.x, h = blockIdx.y, m = blockIdx.z;
  const int nch = gridDim.x;
  const int lane_id = rm.row_lane[m];
  const int ctx = rm.row_pos[m] + 1;
  const int c0 = chunk * kChunk;
  if (c0 >= ctx) return;  // whole block exits: nothing to do for this chunk
  const int tid = threadIdx.x, wave = tid >> 6, ln = tid & 63;
  const int sub = ln % LPK, kg = ln / LPK;
  const int d0 = sub * 8;
  const int d = kv.H * HD;
  const CachePtrs cp = cache_ptrs(kv, lane_id, layer, h);
  const float scale = 1.0f / sqrtf((float)HD);

  float qv[8];
  {
    const half8_t qh =
        __builtin_bit_cast(half8_t, *reinterpret_cast<const u32x4_t*>(q + (size_t)m * d + h * HD + d0));
#pragma unroll
    for (int j = 0; j < 8; ++j) qv[j] = (float)qh[j];
  }
  const int rowb = kv.int8 ? HD : HD * 2;
  float sc[NP];
  float mx = -INFINITY;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int key = c0 + wave * 64 + p * KPP + kg;
    float s = -INFINITY;
    if (key < ctx) {
      const half8_t kh = __builtin_bit_cast(half8_t, load8_as_f16(cp.k + (size_t)key * rowb, d0, kv.int8));
      float t = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) t = fmaf(qv[j], (float)kh[j], t);
#pragma unroll
      for (int off = LPK / 2; off >= 1; off >>= 1) t += __shfl_xor(t, off, 64);
      s = t * scale * (kv.int8 ? h2f(cp.ks[key]) : 1.0f);
    }
    sc[p] = s;
    mx = fmaxf(mx, s);
  }
  mx = wave_max(mx);
  if (ln == 0) red_m[wave] = mx;
  __syncthreads();
  const float cm = fmaxf(red_m[0], red_m[1]);  // chunk max (finite: key c0 < ctx)
  float lsum = 0.f;
  float ov[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) ov[j] = 0.f;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int key = c0 + wave * 64 + p * KPP + kg;
    if (key < ctx) {
      const float pr = expf(sc[p] - cm);
      if (sub == 0) lsum += pr;
      const float pv = pr * (kv.int8 ? h2f(cp.vs[key]) : 1.0f);
      const half8_t vh = __builtin_bit_cast(half8_t, load8_as_f16(cp.v + (size_t)key * rowb, d0, kv.int8));
#pragma unroll
      for (int j = 0; j < 8; ++j) ov[j] = fmaf(pv, (float)vh[j], ov[j]);
    }
  }
  lsum = wave_sum(lsum);
  // reduce ov over the KPP key groups of the wave (lanes with equal `sub`)
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1)
#pragma unroll
    for (int j = 0; j < 8; ++j) ov[j] += __shfl_xor(ov[j], off, 64);
  if (ln == 0) red_l[wave] = lsum;
  if (kg == 0)
#pragma unroll
    for (int j = 0; j < 8; ++j) red_o[wave][d0 + j] = ov[j];
  __syncthreads();
  float* dst = part + ((size_t)(m * kv.H + h) * nch + chunk) * (HD + 2);
  for (int i = tid; i < HD; i += 128) dst[i] = red_o[0][i] + red_o[1][i];
  if (tid == 0) {
    dst[HD] = cm;
    dst[HD + 1] = red_l[0] + red_l[1];
  }
}

__global__ void attn_combine_kernel(const float* __restrict__ part, RowMap rm, int H, int hd, int nch,
                                    uint16_t* __restrict__ o) {
  const int h = blockIdx.x, m = blockIdx.y;
  const int ctx = rm.row_pos[m] + 1;
  const int used = (ctx + kChunk - 1) / kChunk;
  const float* base = part + (size_t)(m * H + h) * nch * (hd + 2);
  float gm = -INFINITY;
  for (int c = 0; c < used; ++c) gm = fmaxf(gm, base[c * (hd + 2) + hd]);
  for (int i = threadIdx.x; i < hd; i += blockDim.x) {
    float num = 0.f, den = 0.f;
    for (int c = 0; c < used; ++c) {
      const float w = expf(base[c * (hd + 2) + hd] - gm);
      num = fmaf(w, base[c * (hd + 2) + i], num);
      den = fmaf(w, base[c * (hd + 2) + hd + 1], den);
    }
    o[(size_t)m * H * hd + h * hd + i] = f2h(num / den);
  }
}

hipError_t launch_attn_decode(const uint16_t* q, int M, const RowMap& rm, const KvGeom& kv, int layer,
                              float* part, uint16_t* o, hipStream_t s) {
  int maxctx = 0;
  for (int m = 0; m < M; ++m) maxctx = max(maxctx, rm.row_pos[m] + 1);
  const int nch = (kv.S + kChunk - 1) / kChunk;
  const int used = (maxctx + kChunk - 1) / kChunk;
  // Blocks beyond a row's context exit at once; the grid spans the longest row.
  dim3 grid(used, kv.H, M);
  (void)nch;
  if (kv.hd == 128)
    hipLaunchKernelGGL(attn_decode_kernel<128>, grid, dim3(128), 0, s, q, rm, kv, layer, part);
  else if (kv.hd == 64)
    hipLaunchKernelGGL(attn_decode_kernel<64>, grid, dim3(128), 0, s, q, rm, kv, layer, part);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(kv.H, M), dim3(128), 0, s, part, rm, kv.H, kv.hd, used, o);
  return hipGetLastError();
}

}  // namespace tl
