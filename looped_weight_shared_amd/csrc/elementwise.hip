// Small kernels of the forward pass: embedding gather, RMSNorm + fp16 cast,
// RoPE + KV-cache write (FP16 or INT8), head projection, argmax, row scatter
// and the INT8 KV row quantizer.
#include "tl_device.h"
#include "tl_kernels.h"

namespace tl {

__device__ __forceinline__ int row_lane(const RowMap& rm, int m) { return rm.per_row ? rm.row_lane[m] : rm.lane; }
__device__ __forceinline__ int row_pos(const RowMap& rm, int m) { return rm.per_row ? rm.row_pos[m] : rm.p0 + m; }
// Output row of per-row results: the lane in decode, the call row in prefill.
__device__ __forceinline__ int out_row(const RowMap& rm, int m) { return rm.per_row ? rm.row_lane[m] : m; }

// ------------------------------------------------------------------ embed
// x[m] = f32(E[token]); decode rows read the token of their lane.
__global__ void embed_kernel(const uint16_t* __restrict__ E, const int32_t* __restrict__ tokens, RowMap rm, int d,
                             float* __restrict__ x) {
  const int m = blockIdx.x;
  const int tok = tokens[rm.per_row ? rm.row_lane[m] : m];
  const uint16_t* er = E + (size_t)tok * d;
  for (int k = threadIdx.x; k < d; k += blockDim.x) x[(size_t)m * d + k] = h2f(er[k]);
}

hipError_t launch_embed(const uint16_t* embed, const int32_t* tokens, int M, const RowMap& rm, int d, float* x,
                        hipStream_t s) {
  hipLaunchKernelGGL(embed_kernel, dim3(M), dim3(256), 0, s, embed, tokens, rm, d, x);
  return hipGetLastError();
}

// ------------------------------------------------------------------ RMSNorm
// h[m] = fp16(gamma * x[m] / sqrt(mean(x[m]^2) + eps)); one block per row.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, const uint16_t* __restrict__ g,
                                                      float eps, int d, uint16_t* __restrict__ h) {
  __shared__ float part[4];
  const int m = blockIdx.x, tid = threadIdx.x;
  const float* xr = x + (size_t)m * d;
  float acc = 0.f;
  for (int k = tid; k < d; k += 256) acc += xr[k] * xr[k];
  acc = wave_sum(acc);
  if ((tid & 63) == 0) part[tid >> 6] = acc;
  __syncthreads();
  const float ss = part[0] + part[1] + part[2] + part[3];
  const float rinv = 1.0f / sqrtf(ss / (float)d + eps);
  for (int k = tid; k < d; k += 256) h[(size_t)m * d + k] = f2h((xr[k] * rinv) * h2f(g[k]));
}

hipError_t launch_rmsnorm(const float* x, const uint16_t* gamma, float eps, int M, int d, uint16_t* h,
                          hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(M), dim3(256), 0, s, x, gamma, eps, d, h);
  return hipGetLastError();
}

// ------------------------------------------------------------------ INT8 KV quantizer
// One wave quantizes one row of hd <= 128 values, 2 per lane (lane i holds
// elements i and i + hd/2). Bit-exact definition: amax = max|x|;
// s = fp16(amax / 127) (correctly rounded fp32 division, then RNE);
// q = clamp(rint(x / f32(s)), -127, 127), 0 when s == 0.
__device__ __forceinline__ void quant_pair(float a, float b, bool valid, int8_t* qa, int8_t* qb, uint16_t* sc) {
  float am = valid ? fmaxf(fabsf(a), fabsf(b)) : 0.f;
  am = wave_max(am);
  const _Float16 s16 = (_Float16)__fdiv_rn(am, 127.0f);
  const float sf = (float)s16;
  if (valid) {
    float x0 = 0.f, x1 = 0.f;
    if (sf > 0.f) {
      x0 = fminf(fmaxf(rintf(__fdiv_rn(a, sf)), -127.f), 127.f);
      x1 = fminf(fmaxf(rintf(__fdiv_rn(b, sf)), -127.f), 127.f);
    }
    *qa = (int8_t)(int)x0;
    *qb = (int8_t)(int)x1;
  }
  *sc = __builtin_bit_cast(uint16_t, s16);
}

__global__ void kv_quant_rows_kernel(const uint16_t* __restrict__ x, int rows, int hd, int8_t* __restrict__ q,
                                     uint16_t* __restrict__ sc) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wave exits together
  const int ln = threadIdx.x & 63, half = hd / 2;
  const bool valid = ln < half;
  float a = 0.f, b = 0.f;
  if (valid) {
    a = h2f(x[(size_t)row * hd + ln]);
    b = h2f(x[(size_t)row * hd + ln + half]);
  }
  int8_t qa = 0, qb = 0;
  uint16_t s;
  quant_pair(a, b, valid, &qa, &qb, &s);
  if (valid) {
    q[(size_t)row * hd + ln] = qa;
    q[(size_t)row * hd + ln + half] = qb;
  }
  if (ln == 0) sc[row] = s;
}

hipError_t launch_kv_quantize_rows(const uint16_t* x, int rows, int hd, int8_t* q, uint16_t* sc, hipStream_t s) {
  hipLaunchKernelGGL(kv_quant_rows_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, x, rows, hd, q, sc);
  return hipGetLastError();
}

// ------------------------------------------------------------------ RoPE + KV write
// One wave per (row, head). Lane i < hd/2 rotates the pair (i, i + hd/2) of q
// and k by angle pos * base^(-2i/hd) (cos/sin table computed on the host in
// double precision), rounds Q, K, V to fp16, writes Q and stores K, V in the
// cache of the row's lane at its position (FP16, or INT8 + scale).
__global__ __launch_bounds__(256) void rope_kv_kernel(const float* __restrict__ qkv, int M, RowMap rm,
                                                      const float* __restrict__ rope_cs, KvGeom kv, int layer,
                                                      uint16_t* __restrict__ qout) {
  const int m = blockIdx.y;
  const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (h >= kv.H) return;
  const int ln = threadIdx.x & 63;
  const int hd = kv.hd, half = hd / 2, d = kv.H * hd;
  const bool valid = ln < half;
  const int lane = row_lane(rm, m), pos = row_pos(rm, m);
  const float* row = qkv + (size_t)m * 3 * d;
  float c = 0.f, sn = 0.f;
  float q1 = 0.f, q2 = 0.f, k1 = 0.f, k2 = 0.f, v1 = 0.f, v2 = 0.f;
  if (valid) {
    c = rope_cs[(size_t)pos * half + ln];
    sn = rope_cs[(size_t)kv.S * half + (size_t)pos * half + ln];
    q1 = row[h * hd + ln];
    q2 = row[h * hd + ln + half];
    k1 = row[d + h * hd + ln];
    k2 = row[d + h * hd + ln + half];
    v1 = row[2 * d + h * hd + ln];
    v2 = row[2 * d + h * hd + ln + half];
  }
  const _Float16 Q1 = (_Float16)(q1 * c - q2 * sn), Q2 = (_Float16)(q2 * c + q1 * sn);
  const _Float16 K1 = (_Float16)(k1 * c - k2 * sn), K2 = (_Float16)(k2 * c + k1 * sn);
  const _Float16 V1 = (_Float16)v1, V2 = (_Float16)v2;
  if (valid) {
    qout[(size_t)m * d + h * hd + ln] = __builtin_bit_cast(uint16_t, Q1);
    qout[(size_t)m * d + h * hd + ln + half] = __builtin_bit_cast(uint16_t, Q2);
  }
  uint8_t* base = kv.base + ((size_t)lane * kv.n_layers + layer) * kv.layer_bytes;
  const size_t HS = (size_t)kv.H * kv.S;
  const size_t rowi = (size_t)h * kv.S + pos;
  if (!kv.int8) {
    uint16_t* K = reinterpret_cast<uint16_t*>(base) + rowi * hd;
    uint16_t* V = reinterpret_cast<uint16_t*>(base) + HS * hd + rowi * hd;
    if (valid) {
      K[ln] = __builtin_bit_cast(uint16_t, K1);
      K[ln + half] = __builtin_bit_cast(uint16_t, K2);
      V[ln] = __builtin_bit_cast(uint16_t, V1);
      V[ln + half] = __builtin_bit_cast(uint16_t, V2);
    }
  } else {
    int8_t* Kq = reinterpret_cast<int8_t*>(base) + rowi * hd;
    uint16_t* Ks = reinterpret_cast<uint16_t*>(base + HS * hd) + rowi;
    int8_t* Vq = reinterpret_cast<int8_t*>(base + HS * hd + HS * 2) + rowi * hd;
    uint16_t* Vs = reinterpret_cast<uint16_t*>(base + 2 * HS * hd + HS * 2) + rowi;
    int8_t a, b;
    uint16_t s;
    quant_pair((float)K1, (float)K2, valid, &a, &b, &s);
    if (valid) {
      Kq[ln] = a;
      Kq[ln + half] = b;
    }
    if (ln == 0) *Ks = s;
    quant_pair((float)V1, (float)V2, valid, &a, &b, &s);
    if (valid) {
      Vq[ln] = a;
      Vq[ln + half] = b;
    }
    if (ln == 0) *Vs = s;
  }
}

hipError_t launch_rope_kv(const float* qkv, int M, const RowMap& rm, const float* rope_cs, const KvGeom& kv,
                          int layer, uint16_t* q_out, hipStream_t s) {
  if (kv.hd > 128 || kv.hd % 2) return hipErrorInvalidValue;
  dim3 grid((kv.H + 3) / 4, M);
  hipLaunchKernelGGL(rope_kv_kernel, grid, dim3(256), 0, s, qkv, M, rm, rope_cs, kv, layer, q_out);
  return hipGetLastError();
}

// ------------------------------------------------------------------ head
// logits[row][v] = sum_k z[m][k] * Head[v][k] for M <= 16 normed rows z (fp16
// [M][d], produced by rmsnorm_kernel). A wave owns one 16-row block of the
// head and walks K in 32-deep MFMA steps, 8 steps of loads in flight.
__global__ __launch_bounds__(256) void head_kernel(const uint16_t* __restrict__ z, int M,
                                                   const uint16_t* __restrict__ head, int V, int d,
                                                   float* __restrict__ logits, RowMap rm) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int lda = d + 8;
  _Float16* Z = reinterpret_cast<_Float16*>(smem);
  const int tid = threadIdx.x, wave = tid >> 6, ln = tid & 63;
  const int l16 = ln & 15, lq = ln >> 4;
  for (int i = tid; i < M * (d / 8); i += 256) {
    const int m = i / (d / 8), c = (i % (d / 8)) * 8;
    *reinterpret_cast<u32x4_t*>(Z + m * lda + c) = *reinterpret_cast<const u32x4_t*>(z + (size_t)m * d + c);
  }
  __syncthreads();
  const int nb = blockIdx.x * 4 + wave;
  const int v = nb * 16 + l16;
  const bool vrow = v < V;
  const bool arow = l16 < M;
  const half8_t hz = {0, 0, 0, 0, 0, 0, 0, 0};
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  const int nsteps = d / 32;
  for (int s0 = 0; s0 < nsteps; s0 += 8) {
    u32x4_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      w[j] = (u32x4_t){0, 0, 0, 0};
      if (vrow && s0 + j < nsteps)
        w[j] = *reinterpret_cast<const u32x4_t*>(head + (size_t)v * d + (s0 + j) * 32 + 8 * lq);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (s0 + j < nsteps) {
        const half8_t af =
            arow ? *reinterpret_cast<const half8_t*>(Z + l16 * lda + (s0 + j) * 32 + 8 * lq) : hz;
        acc = mfma16(af, __builtin_bit_cast(half8_t, w[j]), acc);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * lq + r;
    if (m < M && vrow) logits[(size_t)out_row(rm, m) * V + v] = acc[r];
  }
}

hipError_t launch_head_z(const uint16_t* z, int M, const uint16_t* head, int V, int d, float* logits,
                         const RowMap& rm, hipStream_t s) {
  if (M < 1 || M > 16 || d % 32) return hipErrorInvalidValue;
  const size_t lds = (size_t)M * (d + 8) * 2;
  const int nblk = (V + 15) / 16;
  hipLaunchKernelGGL(head_kernel, dim3((nblk + 3) / 4), dim3(256), lds, s, z, M, head, V, d, logits, rm);
  return hipGetLastError();
}

// ------------------------------------------------------------------ argmax
// Greedy next token per row: the largest logit, ties to the lowest index.
__global__ __launch_bounds__(1024) void argmax_kernel(const float* __restrict__ logits, int V, RowMap rm,
                                                      int32_t* __restrict__ next) {
  __shared__ float bv[16];
  __shared__ int bi[16];
  const int m = blockIdx.x, tid = threadIdx.x;
  const float* lg = logits + (size_t)out_row(rm, m) * V;
  float best = -INFINITY;
  int idx = 0x7fffffff;
  for (int v = tid; v < V; v += 1024) {
    const float x = lg[v];
    if (x > best) {
      best = x;
      idx = v;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ob = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(idx, o, 64);
    if (ob > best || (ob == best && oi < idx)) {
      best = ob;
      idx = oi;
    }
  }
  if ((tid & 63) == 0) {
    bv[tid >> 6] = best;
    bi[tid >> 6] = idx;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 16; ++w)
      if (bv[w] > best || (bv[w] == best && bi[w] < idx)) {
        best = bv[w];
        idx = bi[w];
      }
    next[out_row(rm, m)] = idx == 0x7fffffff ? 0 : idx;
  }
}

hipError_t launch_argmax(const float* logits, int M, int V, const RowMap& rm, int32_t* next, hipStream_t s) {
  hipLaunchKernelGGL(argmax_kernel, dim3(M), dim3(1024), 0, s, logits, V, rm, next);
  return hipGetLastError();
}

// ------------------------------------------------------------------ scatter
__global__ void scatter_rows_kernel(const float* __restrict__ src, int d, RowMap rm, float* __restrict__ dst) {
  const int m = blockIdx.x;
  const int r = out_row(rm, m);
  for (int k = threadIdx.x; k < d; k += blockDim.x) dst[(size_t)r * d + k] = src[(size_t)m * d + k];
}

hipError_t launch_scatter_rows(const float* src, int M, int d, const RowMap& rm, float* dst, hipStream_t s) {
  hipLaunchKernelGGL(scatter_rows_kernel, dim3(M), dim3(256), 0, s, src, d, rm, dst);
  return hipGetLastError();
}

}  // namespace tl
