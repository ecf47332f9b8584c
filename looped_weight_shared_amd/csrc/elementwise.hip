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
                             int V, float* __restrict__ x) {
  const int m = blockIdx.x;
  const int tok = min(max(tokens[rm.per_row ? rm.row_lane[m] : m], 0), V - 1);  // ids outside [0, V) clamped
  const uint16_t* er = E + (size_t)tok * d;
  for (int k = threadIdx.x; k < d; k += blockDim.x) x[(size_t)m * d + k] = h2f(er[k]);
}

hipError_t launch_embed(const uint16_t* embed, const int32_t* tokens, int M, const RowMap& rm, int d, int V, float* x,
                        hipStream_t s) {
  launch(embed_kernel, dim3(M), dim3(256), 0, s, embed, tokens, rm, d, V, x);
  return hipGetLastError();
}

// ------------------------------------------------------------------ RMSNorm
// One block (kNormThreads threads) per row: x += the pending split-K partials
// of the residual GEMM that produced x (split order), then h = fp16(gamma * x
// / sqrt(mean(x^2) + eps)). Thread t owns the float4 chunks t, t + 512, ...
// (CH of them); every load is issued before the first store.
constexpr int kMaxSplits = kMaxSplitK;
// 512 threads per row (one float4 of a 2048-wide row each) measured 0.3%
// faster per prefill than 256; the 8 wave sums are added pairwise.
constexpr int kNormThreads = 512;
__device__ __forceinline__ float norm_parts(const float* part) {
  return ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
}

// One block per row. Every load is issued first (clamped addresses, no
// branches): the row of x, the SP pending split partials (SP = 0: none; a
// power of two >= the actual count S, the extra ones read in bounds and
// selected out), and the gains. x += the partials summed in split order,
// then h = fp16(x * rinv * gamma).
template <int CH, int SP>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(float* __restrict__ x, Pending pend, int M,
                                                      const uint16_t* __restrict__ g, float eps, int d,
                                                      uint16_t* __restrict__ h) {
  __shared__ float part[kNormThreads / 64];
  const int m = blockIdx.x, tid = threadIdx.x;
  float4* xr = reinterpret_cast<float4*>(x + (size_t)m * d);
  const int nc = d / 4;
  int cc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) cc[c] = min(tid + kNormThreads * c, nc - 1);
  float4 v[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) v[c] = xr[cc[c]];
  constexpr int SPN = SP > 0 ? SP : 1;
  float4 p[CH][SPN];
  if constexpr (SP > 0) {
    const float4* pp = reinterpret_cast<const float4*>(pend.part) + (size_t)m * nc;
    const size_t split = (size_t)M * nc;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int s = 0; s < SP; ++s) p[c][s] = pp[(size_t)min(s, pend.S - 1) * split + cc[c]];
  }
  uint2 gr[CH];
  if (h) {
#pragma unroll
    for (int c = 0; c < CH; ++c) gr[c] = *reinterpret_cast<const uint2*>(g + 4 * cc[c]);
  }
  if constexpr (SP > 0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      float4 a = p[c][0];
#pragma unroll
      for (int s = 1; s < SP; ++s) {
        const bool on = s < pend.S;
        a.x += on ? p[c][s].x : 0.f;
        a.y += on ? p[c][s].y : 0.f;
        a.z += on ? p[c][s].z : 0.f;
        a.w += on ? p[c][s].w : 0.f;
      }
      v[c].x += a.x;
      v[c].y += a.y;
      v[c].z += a.z;
      v[c].w += a.w;
      if (tid + kNormThreads * c < nc) xr[cc[c]] = v[c];
    }
  }
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c)
    if (tid + kNormThreads * c < nc) acc += v[c].x * v[c].x + v[c].y * v[c].y + v[c].z * v[c].z + v[c].w * v[c].w;
  acc = wave_sum(acc);
  if ((tid & 63) == 0) part[tid >> 6] = acc;
  __syncthreads();
  const float ss = norm_parts(part);
  const float rinv = 1.0f / sqrtf(ss / (float)d + eps);
  if (!h) return;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ci = tid + kNormThreads * c;
    if (ci >= nc) continue;
    const int k = ci * 4;
    const float g0 = h2f(gr[c].x & 0xFFFF), g1 = h2f(gr[c].x >> 16), g2 = h2f(gr[c].y & 0xFFFF), g3 = h2f(gr[c].y >> 16);
    const uint32_t lo = (uint32_t)f2h((v[c].x * rinv) * g0) | ((uint32_t)f2h((v[c].y * rinv) * g1) << 16);
    const uint32_t hi = (uint32_t)f2h((v[c].z * rinv) * g2) | ((uint32_t)f2h((v[c].w * rinv) * g3) << 16);
    *reinterpret_cast<uint2*>(h + (size_t)m * d + k) = make_uint2(lo, hi);
  }
}

// First layer of a prefill: x[m] = f32(E[tokens[m]]) and h[m] =
// fp16(RMSNorm(x[m]) * gamma) in one pass (the same arithmetic as the embed
// kernel followed by rmsnorm_kernel<CH, 0>, so the same bits).
template <int CH>
__global__ __launch_bounds__(kNormThreads) void embed_rmsnorm_kernel(const uint16_t* __restrict__ E,
                                                            const int32_t* __restrict__ tokens, int V,
                                                            float* __restrict__ x, const uint16_t* __restrict__ g,
                                                            float eps, int d, uint16_t* __restrict__ h) {
  __shared__ float part[kNormThreads / 64];
  const int m = blockIdx.x, tid = threadIdx.x;
  const int nc = d / 4;
  int cc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) cc[c] = min(tid + kNormThreads * c, nc - 1);
  uint2 gr[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) gr[c] = *reinterpret_cast<const uint2*>(g + 4 * cc[c]);
  const int tok = min(max(tokens[m], 0), V - 1);  // ids outside [0, V) clamped
  const uint2* er = reinterpret_cast<const uint2*>(E + (size_t)tok * d);
  float4 v[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const uint2 e4 = er[cc[c]];
    v[c] = make_float4(h2f(e4.x & 0xFFFF), h2f(e4.x >> 16), h2f(e4.y & 0xFFFF), h2f(e4.y >> 16));
  }
  float4* xr = reinterpret_cast<float4*>(x + (size_t)m * d);
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c)
    if (tid + kNormThreads * c < nc) {
      xr[cc[c]] = v[c];
      acc += v[c].x * v[c].x + v[c].y * v[c].y + v[c].z * v[c].z + v[c].w * v[c].w;
    }
  acc = wave_sum(acc);
  if ((tid & 63) == 0) part[tid >> 6] = acc;
  __syncthreads();
  const float ss = norm_parts(part);
  const float rinv = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ci = tid + kNormThreads * c;
    if (ci >= nc) continue;
    const int k = ci * 4;
    const float g0 = h2f(gr[c].x & 0xFFFF), g1 = h2f(gr[c].x >> 16), g2 = h2f(gr[c].y & 0xFFFF), g3 = h2f(gr[c].y >> 16);
    const uint32_t lo = (uint32_t)f2h((v[c].x * rinv) * g0) | ((uint32_t)f2h((v[c].y * rinv) * g1) << 16);
    const uint32_t hi = (uint32_t)f2h((v[c].z * rinv) * g2) | ((uint32_t)f2h((v[c].w * rinv) * g3) << 16);
    *reinterpret_cast<uint2*>(h + (size_t)m * d + k) = make_uint2(lo, hi);
  }
}

hipError_t launch_embed_rmsnorm(const uint16_t* embed, const int32_t* tokens, int V, int M, int d, float* x,
                                const uint16_t* gamma, float eps, uint16_t* h, hipStream_t s) {
  if (M < 1) return hipSuccess;
  if (d % 4 || d < 4 || d > 8192) return hipErrorInvalidValue;
  const int ch = (d / 4 + kNormThreads - 1) / kNormThreads;
  if (ch <= 1)
    launch(embed_rmsnorm_kernel<1>, dim3(M), dim3(kNormThreads), 0, s, embed, tokens, V, x, gamma, eps, d, h);
  else if (ch <= 2)
    launch(embed_rmsnorm_kernel<2>, dim3(M), dim3(kNormThreads), 0, s, embed, tokens, V, x, gamma, eps, d, h);
  else if (ch <= 4)
    launch(embed_rmsnorm_kernel<4>, dim3(M), dim3(kNormThreads), 0, s, embed, tokens, V, x, gamma, eps, d, h);
  else
    launch(embed_rmsnorm_kernel<8>, dim3(M), dim3(kNormThreads), 0, s, embed, tokens, V, x, gamma, eps, d, h);
  return hipGetLastError();
}

template <int CH>
static hipError_t rmsnorm_splits(float* x, Pending pend, const uint16_t* gamma, float eps, int M, int d, uint16_t* h,
                                 hipStream_t s) {
  const int S = pend.part ? pend.S : 0;
  if (S == 0)
    launch(rmsnorm_kernel<CH, 0>, dim3(M), dim3(kNormThreads), 0, s, x, pend, M, gamma, eps, d, h);
  else if (S <= 2)
    launch(rmsnorm_kernel<CH, 2>, dim3(M), dim3(kNormThreads), 0, s, x, pend, M, gamma, eps, d, h);
  else if (S <= 4)
    launch(rmsnorm_kernel<CH, 4>, dim3(M), dim3(kNormThreads), 0, s, x, pend, M, gamma, eps, d, h);
  else if (S <= 8)
    launch(rmsnorm_kernel<CH, 8>, dim3(M), dim3(kNormThreads), 0, s, x, pend, M, gamma, eps, d, h);
  else
    launch(rmsnorm_kernel<CH, 16>, dim3(M), dim3(kNormThreads), 0, s, x, pend, M, gamma, eps, d, h);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(float* x, Pending pend, const uint16_t* gamma, float eps, int M, int d, uint16_t* h,
                          hipStream_t s) {
  if (M < 1) return hipSuccess;
  if (d % 4 || d < 4 || d > 8192 || (pend.part && (pend.S < 1 || pend.S > kMaxSplits))) return hipErrorInvalidValue;
  const int ch = (d / 4 + kNormThreads - 1) / kNormThreads;
  if (ch <= 1) return rmsnorm_splits<1>(x, pend, gamma, eps, M, d, h, s);
  if (ch <= 2) return rmsnorm_splits<2>(x, pend, gamma, eps, M, d, h, s);
  if (ch <= 4) return rmsnorm_splits<4>(x, pend, gamma, eps, M, d, h, s);
  return rmsnorm_splits<8>(x, pend, gamma, eps, M, d, h, s);
}

// ------------------------------------------------------------------ INT8 KV quantizer
// One wave quantizes one row of hd <= 128 values, 2 per lane (lane i holds
// elements i and i + hd/2). Bit-exact definition: amax = max|x|;
// s = fp16(amax / 127) (correctly rounded fp32 division, then RNE);
// q = clamp(rint(x / f32(s)), -127, 127), 0 when s == 0.
__device__ __forceinline__ void quant_pair(float a, float b, bool valid, int8_t* qa, int8_t* qb, uint16_t* sc) {
  float am = valid ? fmaxf(fabsf(a), fabsf(b)) : 0.f;
  am = wave_max(am);
  const _Float16 s16 = kv_scale(am);
  const float sf = (float)s16;
  if (valid) {
    *qa = (int8_t)kv_code(a, sf);
    *qb = (int8_t)kv_code(b, sf);
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
  launch(kv_quant_rows_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, x, rows, hd, q, sc);
  return hipGetLastError();
}

// ------------------------------------------------------------------ RoPE + KV write
// One wave per (row, head). Lane i < hd/2 rotates the pair (i, i + hd/2) of q
// and k by angle pos * base^(-2i/hd) (cos/sin table computed on the host in
// double precision), rounds Q, K, V to fp16, writes Q and stores K, V in the
// cache of the row's lane at its position (FP16, or INT8 + scale).
__global__ __launch_bounds__(256) void rope_kv_kernel(const float* __restrict__ qkv, int S, int M, RowMap rm,
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
  const size_t split = (size_t)M * 3 * d;  // stride between split-K partials
  auto val = [&](int col) {
    float v = row[col];
    for (int s = 1; s < S; ++s) v += row[s * split + col];
    return v;
  };
  float c = 0.f, sn = 0.f;
  float q1 = 0.f, q2 = 0.f, k1 = 0.f, k2 = 0.f, v1 = 0.f, v2 = 0.f;
  if (valid) {
    c = rope_cs[(size_t)pos * half + ln];
    sn = rope_cs[(size_t)kv.S * half + (size_t)pos * half + ln];
    q1 = val(h * hd + ln);
    q2 = val(h * hd + ln + half);
    k1 = val(d + h * hd + ln);
    k2 = val(d + h * hd + ln + half);
    v1 = val(2 * d + h * hd + ln);
    v2 = val(2 * d + h * hd + ln + half);
  }
  _Float16 Q1, Q2, K1, K2;
  rope_pair(q1, q2, c, sn, &Q1, &Q2);
  rope_pair(k1, k2, c, sn, &K1, &K2);
  const _Float16 V1 = (_Float16)v1, V2 = (_Float16)v2;
  if (valid) {
    qout[(size_t)m * d + h * hd + ln] = __builtin_bit_cast(uint16_t, Q1);
    qout[(size_t)m * d + h * hd + ln + half] = __builtin_bit_cast(uint16_t, Q2);
  }
  uint8_t* base = kv.base + ((size_t)lane * kv.n_layers + layer) * kv.layer_bytes;
  const size_t HS = (size_t)kv.H * kv.cap;
  const size_t rowi = (size_t)h * kv.cap + kv_slot(kv, pos);
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
    const Int8Planes pl = int8_planes(kv.H, kv.cap, hd);
    int8_t* Kq = reinterpret_cast<int8_t*>(base + pl.kq) + rowi * hd;
    uint16_t* Ks = reinterpret_cast<uint16_t*>(base + pl.ks) + rowi;
    int8_t* Vq = reinterpret_cast<int8_t*>(base + pl.vq) + rowi * hd;
    uint16_t* Vs = reinterpret_cast<uint16_t*>(base + pl.vs) + rowi;
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

hipError_t launch_rope_kv(const float* qkv, int S, int M, const RowMap& rm, const float* rope_cs, const KvGeom& kv,
                          int layer, uint16_t* q_out, hipStream_t s) {
  if (kv.hd > 128 || kv.hd % 2 || S < 1) return hipErrorInvalidValue;
  dim3 grid((kv.H + 3) / 4, M);
  launch(rope_kv_kernel, grid, dim3(256), 0, s, qkv, S, M, rm, rope_cs, kv, layer, q_out);
  return hipGetLastError();
}

// ------------------------------------------------------------------ head
// Final RMSNorm and head projection in one launch, plus per-block argmax
// candidates. Block b owns vocab rows 16b..16b+15; its 4 waves split the
// d/32 MFMA k-steps into 4 contiguous quarters, so each wave streams one
// contiguous run of 1 KiB tiles (the head is stored in tile order: lane l of
// step s holds row l%16, columns 32s + 8(l/16)..+7). Order of work, so that
// no wait covers the head stream: the residual rows and gamma are requested
// first, then the first batch of tiles; the block normalises the M <= MR
// rows into LDS (z = fp16(gamma x / rms)); then batches of kHeadBatch steps
// are streamed double-buffered. The quarters are summed in wave order. Head
// tiles are read non-temporally: streamed once, they should not displace the
// loop-block weights from the caches. Each block writes its logits and, per
// row, its (max, lowest index) candidate.
constexpr int kHeadBatch = 4;  // k-steps per batch and wave (two batches in flight)
constexpr int kHeadXpt = 8;    // residual elements per thread (d <= 2048)

__device__ __forceinline__ void head_lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int MR, int PER>
__global__ __launch_bounds__(256) void head_kernel(const float* __restrict__ x, int M, const uint16_t* __restrict__ gamma,
                                                   float eps, const uint8_t* __restrict__ tiles, int V, int d,
                                                   float* __restrict__ logits, RowMap rm, float* __restrict__ cval,
                                                   int* __restrict__ cidx) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int lda = d + 8;
  _Float16* Z = reinterpret_cast<_Float16*>(smem);
  __shared__ float red[4][MR];
  __shared__ float4_t qsum[4][64];
  const int tid = threadIdx.x, wave = tid >> 6, ln = tid & 63;
  const int l16 = ln & 15, lq = ln >> 4;
  const int nb = blockIdx.x;
  const int nsteps = d / 32, per = (nsteps + 3) / 4, sb = wave * per;  // per <= PER
  const u32x4_t* tp = reinterpret_cast<const u32x4_t*>(tiles) + (size_t)nb * nsteps * 64 + ln;

  // ---- residual rows and gamma: this thread's 8 columns k8 .. k8+7
  const int k8 = kHeadXpt * tid, kc = min(k8, d - 8);
  float4_t xv[MR][2];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const float4_t* xp = reinterpret_cast<const float4_t*>(x + (size_t)min(m, M - 1) * d + kc);
    xv[m][0] = xp[0];
    xv[m][1] = xp[1];
  }
  u32x4_t gr = *reinterpret_cast<const u32x4_t*>(gamma + kc);
  asm volatile("" ::: "memory");

  // ---- first batch of this wave's quarter
  constexpr int NB = (PER + kHeadBatch - 1) / kHeadBatch;  // batches per wave
  u32x4_t wbuf[2][kHeadBatch];
  auto load_w = [&](u32x4_t (&w)[kHeadBatch], int s0) {
#pragma unroll
    for (int j = 0; j < kHeadBatch; ++j)
      w[j] = __builtin_nontemporal_load(tp + (size_t)min(sb + min(s0 + j, per - 1), nsteps - 1) * 64);
  };
  load_w(wbuf[0], 0);
  asm volatile("" ::: "memory");
#pragma unroll
  for (int m = 0; m < MR; ++m) asm volatile("" : "+v"(xv[m][0]), "+v"(xv[m][1]));
  asm volatile("" : "+v"(gr));

  // ---- z = fp16(RMSNorm(x)) for the M rows
  const bool kin = k8 < d;
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    float a = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < 4; ++c) a = fmaf(xv[m][h][c], xv[m][h][c], a);
    a = wave_sum(kin ? a : 0.f);
    if (ln == 0) red[wave][m] = a;
  }
  head_lds_barrier();
  const half8_t gh = __builtin_bit_cast(half8_t, gr);
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (m < M && kin) {
      const float rinv = 1.0f / sqrtf((red[0][m] + red[1][m] + red[2][m] + red[3][m]) / (float)d + eps);
      half8_t zv;
#pragma unroll
      for (int c = 0; c < 8; ++c) zv[c] = (_Float16)((xv[m][c >> 2][c & 3] * rinv) * (float)gh[c]);
      *reinterpret_cast<half8_t*>(Z + m * lda + k8) = zv;
    }
  }
  head_lds_barrier();

  // ---- stream the quarter, double-buffered; steps past it meet zero activations
  const bool arow = l16 < M;
  const half8_t hz = {0, 0, 0, 0, 0, 0, 0, 0};
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  auto consume = [&](const u32x4_t (&w)[kHeadBatch], int s0) {
#pragma unroll
    for (int j = 0; j < kHeadBatch; ++j) {
      const int st = sb + s0 + j;
      const bool ok = arow && s0 + j < per && st < nsteps;
      const half8_t z8 = *reinterpret_cast<const half8_t*>(Z + l16 * lda + min(st, nsteps - 1) * 32 + 8 * lq);
      acc = mfma16(ok ? z8 : hz, __builtin_bit_cast(half8_t, w[j]), acc);
    }
  };
  // straight-line pipeline: batch b+1 is requested before batch b is consumed
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b + 1 < NB) load_w(wbuf[(b + 1) & 1], (b + 1) * kHeadBatch);
    asm volatile("" ::: "memory");
    consume(wbuf[b & 1], b * kHeadBatch);
  }

  // ---- quarters summed in wave order; logits and per-row candidates
  qsum[wave][ln] = acc;
  head_lds_barrier();
  if (wave == 0) {
    const float4_t t = ((qsum[0][ln] + qsum[1][ln]) + qsum[2][ln]) + qsum[3][ln];
    const int v = nb * 16 + l16;
    const int nblk = gridDim.x;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * lq + r;  // lane holds row m = 4lq + r, vocab v
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      if (m < M && v < V) {
        logits[(size_t)out_row(rm, m) * V + v] = t[r];
        bv = t[r];
        bi = v;
      }
      // max over the 16 vocab rows, ties to the lowest index
      row16_argmax(bv, bi);
      if (l16 == 0 && m < M) {
        cval[(size_t)m * nblk + nb] = bv;
        cidx[(size_t)m * nblk + nb] = bi;
      }
    }
  }
}

// Greedy next token of each row from the head blocks' candidates: the
// largest logit, ties to the lowest index (a total order, so the result does
// not depend on the scan order).
__global__ __launch_bounds__(256) void argmax_kernel(const float* __restrict__ cval, const int* __restrict__ cidx,
                                                     int nblk, RowMap rm, int32_t* __restrict__ next,
                                                     int* __restrict__ advance) {
  __shared__ float bv_s[4];
  __shared__ int bi_s[4];
  const int m = blockIdx.x, tid = threadIdx.x;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  // kArgPer candidates per thread are requested before any is compared
  // (clamped indices, out-of-range ones dropped), so the scan costs one
  // round trip per 256 * kArgPer candidates
  constexpr int kArgPer = 16;
  for (int base = 0; base < nblk; base += 256 * kArgPer) {
    float cv[kArgPer];
    int ci[kArgPer];
#pragma unroll
    for (int j = 0; j < kArgPer; ++j) {
      const int b = min(base + tid + 256 * j, nblk - 1);
      cv[j] = cval[(size_t)m * nblk + b];
      ci[j] = cidx[(size_t)m * nblk + b];
    }
#pragma unroll
    for (int j = 0; j < kArgPer; ++j) {
      const bool in = base + tid + 256 * j < nblk;
      if (in && (cv[j] > bv || (cv[j] == bv && ci[j] < bi))) {
        bv = cv[j];
        bi = ci[j];
      }
    }
  }
  wave_argmax(bv, bi);
  if ((tid & 63) == 0) {
    bv_s[tid >> 6] = bv;
    bi_s[tid >> 6] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w)
      if (bv_s[w] > bv_s[0] || (bv_s[w] == bv_s[0] && bi_s[w] < bi_s[0])) {
        bv_s[0] = bv_s[w];
        bi_s[0] = bi_s[w];
      }
    next[out_row(rm, m)] = bi_s[0] == 0x7fffffff ? 0 : bi_s[0];
    if (advance) advance[rm.row_lane[m]] += 1;  // a graph-replayed decode step's last kernel
  }
}

size_t head_scratch_bytes(int max_rows, int V) { return (size_t)max_rows * ((V + 15) / 16) * 8; }

template <int PER>
static void head_rows(dim3 g, size_t lds, hipStream_t s, const float* x, int M, const uint16_t* gamma, float eps,
                      const uint8_t* t, int V, int d, float* logits, const RowMap& rm, float* cval, int* cidx) {
  if (M == 1)
    launch(head_kernel<1, PER>, g, dim3(256), lds, s, x, M, gamma, eps, t, V, d, logits, rm, cval, cidx);
  else if (M == 2)
    launch(head_kernel<2, PER>, g, dim3(256), lds, s, x, M, gamma, eps, t, V, d, logits, rm, cval, cidx);
  else if (M <= 4)
    launch(head_kernel<4, PER>, g, dim3(256), lds, s, x, M, gamma, eps, t, V, d, logits, rm, cval, cidx);
  else
    launch(head_kernel<8, PER>, g, dim3(256), lds, s, x, M, gamma, eps, t, V, d, logits, rm, cval, cidx);
}

hipError_t launch_head(const float* x, int M, const uint16_t* gamma, float eps, const uint8_t* head_tiles, int V,
                       int d, float* logits, const RowMap& rm, void* scratch, hipStream_t s) {
  if (M < 1 || M > 8 || d % 32 || d > 256 * kHeadXpt) return hipErrorInvalidValue;
  const size_t lds = (size_t)M * (d + 8) * 2;
  const int nblk = (V + 15) / 16;
  float* cval = static_cast<float*>(scratch);
  int* cidx = reinterpret_cast<int*>(cval + (size_t)M * nblk);
  const int per = (d / 32 + 3) / 4;  // k-steps per wave
  const dim3 g(nblk);
  if (per <= 4)
    head_rows<4>(g, lds, s, x, M, gamma, eps, head_tiles, V, d, logits, rm, cval, cidx);
  else if (per <= 8)
    head_rows<8>(g, lds, s, x, M, gamma, eps, head_tiles, V, d, logits, rm, cval, cidx);
  else
    head_rows<16>(g, lds, s, x, M, gamma, eps, head_tiles, V, d, logits, rm, cval, cidx);
  return hipGetLastError();
}

hipError_t launch_argmax(int M, int V, const RowMap& rm, const void* scratch, int32_t* next, hipStream_t s,
                         int* advance) {
  if (M < 1 || M > 8) return hipErrorInvalidValue;
  const int nblk = (V + 15) / 16;
  const float* cval = static_cast<const float*>(scratch);
  const int* cidx = reinterpret_cast<const int*>(cval + (size_t)M * nblk);
  launch(argmax_kernel, dim3(M), dim3(256), 0, s, cval, cidx, nblk, rm, next, advance);
  return hipGetLastError();
}

// ------------------------------------------------------------------ store-h rows
// h row m (fp16 [d]) -> the h cache of its lane and layer at its position.
__global__ void store_h_kernel(const uint16_t* __restrict__ h, int d, RowMap rm, uint8_t* __restrict__ base,
                               size_t layer_bytes, int n_layers, int layer) {
  const int m = blockIdx.x;
  uint16_t* dst = reinterpret_cast<uint16_t*>(base + ((size_t)row_lane(rm, m) * n_layers + layer) * layer_bytes) +
                  (size_t)row_pos(rm, m) * d;
  const uint4* src4 = reinterpret_cast<const uint4*>(h + (size_t)m * d);
  uint4* dst4 = reinterpret_cast<uint4*>(dst);
  for (int k = threadIdx.x; k < d / 8; k += blockDim.x) dst4[k] = src4[k];
}

hipError_t launch_store_h(const uint16_t* h, int M, int d, const RowMap& rm, uint8_t* base, size_t layer_bytes,
                          int n_layers, int layer, hipStream_t s) {
  if (d % 8) return hipErrorInvalidValue;
  launch(store_h_kernel, dim3(M), dim3(256), 0, s, h, d, rm, base, layer_bytes, n_layers, layer);
  return hipGetLastError();
}

// ------------------------------------------------------------------ INT8 store-h rows
// One wave per 128-element group of an h row ("Current Status" page, KV-cache
// table: Store-h INT8): amax over the group (fp32, exact), scale fp16(amax /
// 127) and codes clamp(rint(x / s), -127, 127), the same decisions as the
// INT8 K/V quantizer per (token, head) (kv_scale, kv_code); lane l holds
// elements 2l and 2l + 1 of the group.
__global__ __launch_bounds__(256) void store_h8_kernel(const uint16_t* __restrict__ h, int d, int G, RowMap rm,
                                                       uint8_t* __restrict__ base, size_t hs_off,
                                                       size_t layer_bytes, int n_layers, int layer,
                                                       uint16_t* __restrict__ hhat) {
  const int m = blockIdx.x, g = blockIdx.y * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  if (g >= G) return;
  const uint32_t two = *reinterpret_cast<const uint32_t*>(h + (size_t)m * d + g * 128 + 2 * l);
  const float x0 = h2f((uint16_t)(two & 0xffffu)), x1 = h2f((uint16_t)(two >> 16));
  float amax = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const _Float16 sc = kv_scale(amax);
  const float sf = (float)sc;
  const int q0 = kv_code(x0, sf), q1 = kv_code(x1, sf);
  const int pos = row_pos(rm, m);
  uint8_t* lb = base + ((size_t)row_lane(rm, m) * n_layers + layer) * layer_bytes;
  *reinterpret_cast<uint16_t*>(lb + (size_t)pos * d + g * 128 + 2 * l) =
      (uint16_t)((q0 & 0xff) | ((q1 & 0xff) << 8));
  if (l == 0) *reinterpret_cast<_Float16*>(lb + hs_off + ((size_t)pos * G + g) * 2) = sc;
  if (hhat) {
    const _Float16 y0 = (_Float16)((float)q0 * sf), y1 = (_Float16)((float)q1 * sf);
    *reinterpret_cast<uint32_t*>(hhat + (size_t)m * d + g * 128 + 2 * l) =
        (uint32_t)__builtin_bit_cast(uint16_t, y0) | ((uint32_t)__builtin_bit_cast(uint16_t, y1) << 16);
  }
}

hipError_t launch_store_h8(const uint16_t* h, int M, int d, int S, const RowMap& rm, uint8_t* base,
                           size_t layer_bytes, int n_layers, int layer, uint16_t* hhat, hipStream_t s) {
  if (d % 128 || M < 1) return hipErrorInvalidValue;
  const int G = d / 128;
  launch(store_h8_kernel, dim3(M, (G + 3) / 4), dim3(256), 0, s, h, d, G, rm, base, h8_planes(S, d).hs,
         layer_bytes, n_layers, layer, hhat);
  return hipGetLastError();
}

// fp16(q * s) of rows 0 .. rows-1: 8 consecutive elements (one group's) per thread.
__global__ __launch_bounds__(256) void dequant_h8_kernel(const uint8_t* __restrict__ lb, size_t hs_off, int rows,
                                                         int d, uint16_t* __restrict__ out) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;  // index of an 8-element run
  if (i >= (size_t)rows * d / 8) return;
  const size_t e0 = i * 8;
  const size_t r = e0 / d, c = e0 - r * d;
  const float sf = (float)*reinterpret_cast<const _Float16*>(lb + hs_off + (r * (d / 128) + c / 128) * 2);
  const uint2 q8 = *reinterpret_cast<const uint2*>(lb + e0);
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t src = k < 2 ? q8.x : q8.y;
    const int sh = (k & 1) * 16;
    const int qa = (int)(int8_t)((src >> sh) & 0xff), qb = (int)(int8_t)((src >> (sh + 8)) & 0xff);
    const _Float16 ya = (_Float16)((float)qa * sf), yb = (_Float16)((float)qb * sf);
    w[k] = (uint32_t)__builtin_bit_cast(uint16_t, ya) | ((uint32_t)__builtin_bit_cast(uint16_t, yb) << 16);
  }
  *reinterpret_cast<uint4*>(out + e0) = make_uint4(w[0], w[1], w[2], w[3]);
}

hipError_t launch_dequant_h8(const uint8_t* layer_base, int rows, int d, int S, uint16_t* out, hipStream_t s) {
  if (d % 128 || rows < 0 || rows > S) return hipErrorInvalidValue;
  if (rows == 0) return hipSuccess;
  const size_t runs = (size_t)rows * d / 8;
  launch(dequant_h8_kernel, dim3((unsigned)((runs + 255) / 256)), dim3(256), 0, s, layer_base, h8_planes(S, d).hs,
         rows, d, out);
  return hipGetLastError();
}

// ------------------------------------------------------------------ safety check
// Residual L2 norm of each row (x plus any pending split partials, x itself
// untouched); a row whose norm is not <= max_norm (NaN included) records
// code_base + row with an atomic min, so the first (iteration, row) wins.
__global__ __launch_bounds__(256) void safety_check_kernel(const float* __restrict__ x, Pending pend, int M, int d,
                                                          float max_norm, int code_base, int* __restrict__ result) {
  __shared__ float part[4];
  const int m = blockIdx.x, tid = threadIdx.x;
  const float* xr = x + (size_t)m * d;
  float acc = 0.f;
  for (int k = tid; k < d; k += 256) {
    float v = xr[k];
    if (pend.part)
      for (int s = 0; s < pend.S; ++s) v += pend.part[((size_t)s * M + m) * d + k];
    acc = fmaf(v, v, acc);
  }
  acc = wave_sum(acc);
  if ((tid & 63) == 0) part[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    const float nrm = sqrtf(part[0] + part[1] + part[2] + part[3]);
    if (!(nrm <= max_norm)) atomicMin(result, code_base + m);
  }
}

__global__ void safety_reset_kernel(int* result) {
  if (threadIdx.x == 0) *result = 0x7fffffff;
}

hipError_t launch_safety_reset(int* result, hipStream_t s) {
  launch(safety_reset_kernel, dim3(1), dim3(64), 0, s, result);
  return hipGetLastError();
}

hipError_t launch_safety_check(const float* x, Pending pend, int M, int d, float max_norm, int code_base, int* result,
                               hipStream_t s) {
  if (M < 1) return hipSuccess;
  launch(safety_check_kernel, dim3(M), dim3(256), 0, s, x, pend, M, d, max_norm, code_base, result);
  return hipGetLastError();
}

// ------------------------------------------------------------------ scatter
__global__ void scatter_rows_kernel(const float* __restrict__ src, int d, RowMap rm, float* __restrict__ dst) {
  const int m = blockIdx.x;
  const int r = out_row(rm, m);
  for (int k = threadIdx.x; k < d; k += blockDim.x) dst[(size_t)r * d + k] = src[(size_t)m * d + k];
}

hipError_t launch_scatter_rows(const float* src, int M, int d, const RowMap& rm, float* dst, hipStream_t s) {
  launch(scatter_rows_kernel, dim3(M), dim3(256), 0, s, src, d, rm, dst);
  return hipGetLastError();
}

// ------------------------------------------------------------------ decode positions
__global__ void set_pos_kernel(int* __restrict__ dpos, PosArgs a) {
  const int i = threadIdx.x;
  if (i < a.n) dpos[i] = a.v[i];
}

hipError_t launch_set_pos(int* dpos, const PosArgs& a, hipStream_t s) {
  if (a.n < 0 || a.n > 8) return hipErrorInvalidValue;
  launch(set_pos_kernel, dim3(1), dim3(64), 0, s, dpos, a);
  return hipGetLastError();
}

__global__ void advance_pos_kernel(int* __restrict__ dpos, RowMap rm, int M) {
  const int m = threadIdx.x;
  if (m < M) dpos[rm.row_lane[m]] += 1;
}

hipError_t launch_advance_pos(int* dpos, const RowMap& rm, int M, hipStream_t s) {
  if (M < 1 || M > 8) return hipErrorInvalidValue;
  launch(advance_pos_kernel, dim3(1), dim3(64), 0, s, dpos, rm, M);
  return hipGetLastError();
}

}  // namespace tl
