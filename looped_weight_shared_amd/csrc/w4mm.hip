// W4A16 matrix kernels on MFMA (gfx950, v_mfma_f32_16x16x32_f16).
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
//
// Decode GEMV (M <= 16): one m-block; a block owns 1 or 2 n-blocks and its
// waves split the K groups round-robin; partial tiles are summed across
// waves in LDS in fixed wave order (the result does not depend on M or on
// which rows are present). The activation rows are staged in LDS once,
// optionally RMS-normalised from the fp32 residual on the way in.
//
// Prefill GEMM: a block is 4 waves side by side along N, each owning NBW
// n-blocks for all BM = 16*MB rows; the fp16 activation tile of each group is
// double-buffered through LDS (global loads of group g+1 overlap the MFMAs of
// group g) and shared by the 4 waves, while each wave streams its own weight
// tiles one group ahead.
#include <type_traits>

#include "tl_device.h"
#include "tl_kernels.h"

namespace tl {

// ---------------------------------------------------------------- epilogue
__device__ __forceinline__ void epi_store(const Epi& e, int m, int n, float v) {
  if (e.perm_hd) n = qkv_natural_col(n, e.perm_hd);
  if (e.mode == EPI_RESID)
    e.out_f32[(size_t)m * e.ldo + n] += v;
  else
    e.out_f32[(size_t)m * e.ldo + n] = v;
}
__device__ __forceinline__ void epi_swiglu(const Epi& e, int m, int c, float g, float u) {
  e.out_f16[(size_t)m * e.ldo + c] = f2h(silu(g) * u);
}

// ---------------------------------------------------------------- GEMV
// Decode-shaped products (M <= 8 rows). A block owns NBB n-blocks of 16
// output rows; its 8 waves split the K groups (wave w takes groups w, w+8,
// ...). The block stages the M activation rows in LDS as fp16 (the MFMA A
// operand; rows >= M read as zero) and every wave reads its fragments from
// there. Order of work, chosen so no wait ever covers the weight requests:
//   1. each thread requests its activation elements (coalesced), then
//   2. each wave requests all its weight tiles and scales;
//   3. activation math (NORM: per-row sums of squares, one LDS exchange,
//      h = fp16(x * rinv * gamma)) and the LDS stores, barrier (LDS only);
//   4. dequant + MFMA as the tiles arrive; fixed-order cross-wave sum.
// The vmcnt counter is in order, so the activation requests go first; the
// empty asm statements keep the compiler from hoisting the activation math
// (and its waits) above the weight requests.
constexpr int kGemvWaves = 8;
constexpr int kGemvThreads = kGemvWaves * 64;
constexpr int kGemvIt = 8;        // groups per wave at most: K <= 8 * 8 * 128
constexpr int kGemvAChunks = 16;  // fp16 16-byte chunks per thread at most: M * K <= 8 * 8192

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// GI: groups requested per wave (ceil(G / 8) rounded up to 2 or 8; a wave
// with fewer groups re-requests its last one and skips it in the math). APT:
// fp16 activation chunks per thread (fp16 input). All requests are
// unconditional with clamped addresses, so the code between them is
// straight-line and the compiler's waits stay exact.
enum GemvSrc { SRC_A16 = 0, SRC_NORM = 1, SRC_ATT = 2, SRC_EMB = 3 };

template <int NBB, int SRC, int MR, int GI, int APT, bool F16>
__global__ __launch_bounds__(kGemvThreads) void w4_gemv_kernel(const uint8_t* __restrict__ tiles,
                                                               const uint16_t* __restrict__ scales, int N, int K,
                                                               int G, ASrc a, int M, Epi e) {
  constexpr int WK = kGemvWaves;
  // SRC_EMB: the rows are the embedding rows of the tokens (first layer),
  // normalised as SRC_NORM does; block 0 also writes them to x32
  constexpr bool EMB = SRC == SRC_EMB, NORM = SRC == SRC_NORM || EMB, ATT = SRC == SRC_ATT;
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ float red[WK * NBB * 256];
  __shared__ float nrm[WK][MR];
  const int lda = G * 128 + 8;  // LDS row stride in halves (16-byte pad)
  _Float16* As = reinterpret_cast<_Float16*>(smem);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int nb0 = blockIdx.x * NBB;
  const int Kp = G * 128;

  // ---- 1. activation requests
  float4_t xv[NORM ? MR : (ATT ? APT : 1)];
  float2 ml[ATT ? APT : 1];
  uint2 gr = {0, 0};
  u32x4_t av[SRC == SRC_A16 ? APT : 1];
  const int k4 = 4 * tid;  // NORM/ATT: this thread's 4 columns (K <= 2048)
  const int kc = min(k4, K - 4);
  const int chunks = K / 8, nch = M * chunks;
  const int npairs = M * a.att_np;  // ATT: (row, part) pairs, row-major
  if constexpr (EMB) {
    int tk[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) tk[m] = min(max(a.tok[a.tok_idx[min(m, M - 1)]], 0), a.vocab - 1);
    gr = *reinterpret_cast<const uint2*>(a.gamma + kc);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const uint2 e4 = *reinterpret_cast<const uint2*>(a.emb + (size_t)tk[m] * K + kc);
      xv[m] = (float4_t){h2f(e4.x & 0xFFFF), h2f(e4.x >> 16), h2f(e4.y & 0xFFFF), h2f(e4.y >> 16)};
    }
  } else if constexpr (NORM) {
#pragma unroll
    for (int m = 0; m < MR; ++m) xv[m] = *reinterpret_cast<const float4_t*>(a.x32 + (size_t)min(m, M - 1) * K + kc);
    gr = *reinterpret_cast<const uint2*>(a.gamma + kc);
  } else if constexpr (ATT) {
    const int H = K / a.att_hd, hh = kc / a.att_hd, i = kc - hh * a.att_hd;
    const int stride = a.att_hd + kAttnPartExtra;
#pragma unroll
    for (int q = 0; q < APT; ++q) {
      const int qq = min(q, npairs - 1);
      const int m = qq / a.att_np, p = qq - m * a.att_np;
      const float* b = a.att + ((size_t)(m * H + hh) * a.att_np_max + p) * stride;
      xv[q] = *reinterpret_cast<const float4_t*>(b + i);
      ml[q] = *reinterpret_cast<const float2*>(b + a.att_hd);
    }
  } else {
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      const int c = min(tid + kGemvThreads * i, nch - 1);
      const int m = c / chunks, kk = (c - m * chunks) * 8;
      av[i] = *reinterpret_cast<const u32x4_t*>(a.a16 + (size_t)m * K + kk);
    }
  }
  asm volatile("" ::: "memory");  // activation requests strictly before the weight requests
  // ---- 2. weight requests (F16: four 16-byte slots per tile and lane, no scales)
  constexpr int WS = F16 ? 4 : 1;
  u32x4_t wv[GI][NBB][WS];
  uint32_t sc[GI][NBB];  // raw fp16 bits: converting at load time would force a wait
#pragma unroll
  for (int it = 0; it < GI; ++it) {
    const int g = min(wave + it * WK, G - 1);
#pragma unroll
    for (int j = 0; j < NBB; ++j) {
      const size_t tile = (size_t)(nb0 + j) * G + g;
      if constexpr (F16) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          wv[it][j][s] = *(reinterpret_cast<const u32x4_t*>(tiles + tile * kTileBytesF16) + s * 64 + lane);
      } else {
        wv[it][j][0] = *(reinterpret_cast<const u32x4_t*>(tiles + tile * kTileBytes) + lane);
        sc[it][j] = scales[tile * 16 + l16];
      }
    }
  }
  asm volatile("" ::: "memory");
  if constexpr (NORM) {
#pragma unroll
    for (int m = 0; m < MR; ++m) asm volatile("" : "+v"(xv[m]));
  } else if constexpr (ATT) {
#pragma unroll
    for (int q = 0; q < APT; ++q) asm volatile("" : "+v"(xv[q]), "+v"(ml[q]));
  } else {
#pragma unroll
    for (int i = 0; i < APT; ++i) asm volatile("" : "+v"(av[i]));
  }

  // ---- 3. activations into LDS
  if constexpr (EMB) {  // the first layer's residual rows
    if (blockIdx.x == 0 && k4 < K)
#pragma unroll
      for (int m = 0; m < MR; ++m)
        if (m < M) *reinterpret_cast<float4_t*>(const_cast<float*>(a.x32) + (size_t)m * K + k4) = xv[m];
  }
  if constexpr (NORM) {
    const bool kin = k4 < K;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) ss = fmaf(xv[m][c], xv[m][c], ss);
      ss = wave_sum(kin ? ss : 0.f);
      if (lane == 0) nrm[wave][m] = ss;
    }
    lds_barrier();
    const half2_t* gh = reinterpret_cast<const half2_t*>(&gr);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (m < M && k4 < Kp) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < WK; ++w) t += nrm[w][m];
        const float rinv = 1.0f / sqrtf(t / (float)K + a.eps);
        half2_t h01, h23;
        h01.x = (_Float16)((xv[m][0] * rinv) * (float)gh[0].x);
        h01.y = (_Float16)((xv[m][1] * rinv) * (float)gh[0].y);
        h23.x = (_Float16)((xv[m][2] * rinv) * (float)gh[1].x);
        h23.y = (_Float16)((xv[m][3] * rinv) * (float)gh[1].y);
        const half2_t z2 = {0, 0};
        *reinterpret_cast<half2_t*>(As + m * lda + k4) = kin ? h01 : z2;
        *reinterpret_cast<half2_t*>(As + m * lda + k4 + 2) = kin ? h23 : z2;
      }
    }
  } else if constexpr (ATT) {
    // merge each row's parts in part order (attn_merge_step), as the merge kernel does
    const bool kin = k4 < K;
    for (int m = 0; m < M; ++m) {
      float gm = -INFINITY;
#pragma unroll
      for (int q = 0; q < APT; ++q)
        if (q < npairs && q / a.att_np == m) gm = fmaxf(gm, ml[q].x);
      float num[4] = {0.f, 0.f, 0.f, 0.f}, den[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < APT; ++q)
        if (q < npairs && q / a.att_np == m)
#pragma unroll
          for (int c = 0; c < 4; ++c) attn_merge_step(gm, ml[q].x, ml[q].y, xv[q][c], num[c], den[c]);
      if (k4 < Kp) {
        half2_t h01, h23;
        h01.x = (_Float16)(num[0] / den[0]);
        h01.y = (_Float16)(num[1] / den[1]);
        h23.x = (_Float16)(num[2] / den[2]);
        h23.y = (_Float16)(num[3] / den[3]);
        const half2_t z2 = {0, 0};
        *reinterpret_cast<half2_t*>(As + m * lda + k4) = kin ? h01 : z2;
        *reinterpret_cast<half2_t*>(As + m * lda + k4 + 2) = kin ? h23 : z2;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      const int c = tid + kGemvThreads * i;
      if (c < nch) {
        const int m = c / chunks, kk = (c - m * chunks) * 8;
        *reinterpret_cast<u32x4_t*>(As + m * lda + kk) = av[i];
      }
    }
    // zero columns K..Kp-1 of the M rows (K not a multiple of 128)
    const int padc = (Kp - K) / 8;
    for (int c = tid; c < M * padc; c += kGemvThreads) {
      const int m = c / padc;
      *reinterpret_cast<u32x4_t*>(As + m * lda + K + (c - m * padc) * 8) = (u32x4_t){0, 0, 0, 0};
    }
  }
  lds_barrier();

  // ---- 4. dequant + MFMA per group, scaled once per group
  float4_t acc[NBB];
#pragma unroll
  for (int j = 0; j < NBB; ++j) acc[j] = (float4_t){0.f, 0.f, 0.f, 0.f};
  const bool arow = l16 < M;
  const half8_t hz = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int it = 0; it < GI; ++it) {
    const int g = wave + it * WK;
    if (g < G) {
      half8_t af[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        af[s] = arow ? *reinterpret_cast<const half8_t*>(As + l16 * lda + g * 128 + 32 * s + 8 * lq) : hz;
#pragma unroll
      for (int j = 0; j < NBB; ++j) {
        if constexpr (F16) {
#pragma unroll
          for (int s = 0; s < 4; ++s) acc[j] = mfma16(af[s], __builtin_bit_cast(half8_t, wv[it][j][s]), acc[j]);
        } else {
          float4_t t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s) t = mfma16(af[s], dequant_word(wv[it][j][0][s]), t);
          const float scf = h2f((uint16_t)sc[it][j]);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[j][r] = fmaf(t[r], scf, acc[j][r]);
        }
      }
    }
  }

  // ---- sum the per-wave tiles in fixed wave order, then the epilogue
#pragma unroll
  for (int j = 0; j < NBB; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[((wave * NBB + j) * 64 + lane) * 4 + r] = acc[j][r];
  __syncthreads();
  if (tid < 256) {
    const int ln = tid >> 2, r = tid & 3;
    const int m = 4 * (ln >> 4) + r, col = ln & 15;
    if (m < M) {
      float v[NBB];
#pragma unroll
      for (int j = 0; j < NBB; ++j) {
        float t = 0.f;
        for (int w = 0; w < WK; ++w) t += red[((w * NBB + j) * 64 + ln) * 4 + r];
        v[j] = t;
      }
      if (e.mode == EPI_SWIGLU) {
        if constexpr (NBB == 2) epi_swiglu(e, m, blockIdx.x * 16 + col, v[0], v[1]);
      } else {
#pragma unroll
        for (int j = 0; j < NBB; ++j) epi_store(e, m, (nb0 + j) * 16 + col, v[j]);
      }
    }
  }
}

bool gemv_supported(int M, int K, const ASrc& a) {
  const int G = (K + 127) / 128;
  if (M < 1 || M > 8 || K < 8 || K % 8) return false;
  if (a.x32) return K <= 4 * kGemvThreads && (!a.emb || (a.tok && a.vocab > 0));  // one float4 per thread and row
  if (a.att)
    return K <= 4 * kGemvThreads && a.att_hd >= 4 && a.att_hd % 4 == 0 && K % a.att_hd == 0 && a.att_np >= 1 &&
           M * a.att_np <= 16;
  return G <= kGemvWaves * kGemvIt && M * (K / 8) <= kGemvThreads * kGemvAChunks;
}

template <int NBB, int SRC, int MR, int GI, int APT, bool F16>
static hipError_t gemv_launch_t(const Packed& w, const ASrc& a, int M, const Epi& e, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&w4_gemv_kernel<NBB, SRC, MR, GI, APT, F16>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  const size_t lds = (size_t)M * (w.G * 128 + 8) * 2;
  launch((w4_gemv_kernel<NBB, SRC, MR, GI, APT, F16>), dim3(w.N / 16 / NBB), dim3(kGemvThreads), lds, s, w.tiles,
         w.scales, w.N, w.K, w.G, a, M, e);
  return hipGetLastError();
}
template <int NBB, int SRC, int MR, int GI, int APT>
static hipError_t gemv_launch(const Packed& w, const ASrc& a, int M, const Epi& e, hipStream_t s) {
  return w.f16 ? gemv_launch_t<NBB, SRC, MR, GI, APT, true>(w, a, M, e, s)
               : gemv_launch_t<NBB, SRC, MR, GI, APT, false>(w, a, M, e, s);
}

// the first layer's rows from the embedding (x written by block 0)
template <int NBB>
static hipError_t gemv_emb_rows(const Packed& w, const ASrc& a, int M, const Epi& e, hipStream_t s) {
  if (M == 1) return gemv_launch<NBB, SRC_EMB, 1, 2, 1>(w, a, M, e, s);
  if (M == 2) return gemv_launch<NBB, SRC_EMB, 2, 2, 1>(w, a, M, e, s);
  if (M <= 4) return gemv_launch<NBB, SRC_EMB, 4, 2, 1>(w, a, M, e, s);
  return gemv_launch<NBB, SRC_EMB, 8, 2, 1>(w, a, M, e, s);
}

// fused RMSNorm: K <= 2048, so at most 2 groups per wave
template <int NBB>
static hipError_t gemv_norm_rows(const Packed& w, const ASrc& a, int M, const Epi& e, hipStream_t s) {
  if (M == 1) return gemv_launch<NBB, SRC_NORM, 1, 2, 1>(w, a, M, e, s);
  if (M == 2) return gemv_launch<NBB, SRC_NORM, 2, 2, 1>(w, a, M, e, s);
  if (M <= 4) return gemv_launch<NBB, SRC_NORM, 4, 2, 1>(w, a, M, e, s);
  return gemv_launch<NBB, SRC_NORM, 8, 2, 1>(w, a, M, e, s);
}

// merged attention parts: K <= 2048; (row, part) pairs per thread
static hipError_t gemv_att(const Packed& w, const ASrc& a, int M, const Epi& e, hipStream_t s) {
  const int pairs = M * a.att_np;
  if (pairs <= 1) return gemv_launch<1, SRC_ATT, 1, 2, 1>(w, a, M, e, s);
  if (pairs <= 2) return gemv_launch<1, SRC_ATT, 1, 2, 2>(w, a, M, e, s);
  if (pairs <= 4) return gemv_launch<1, SRC_ATT, 1, 2, 4>(w, a, M, e, s);
  if (pairs <= 8) return gemv_launch<1, SRC_ATT, 1, 2, 8>(w, a, M, e, s);
  return gemv_launch<1, SRC_ATT, 1, 2, 16>(w, a, M, e, s);
}

template <int GI>
static hipError_t gemv_a16(const Packed& w, const ASrc& a, int M, const Epi& e, hipStream_t s) {
  const int apt = (M * (w.K / 8) + kGemvThreads - 1) / kGemvThreads;
  if (apt <= 1) return gemv_launch<1, SRC_A16, 1, GI, 1>(w, a, M, e, s);
  if (apt <= 2) return gemv_launch<1, SRC_A16, 1, GI, 2>(w, a, M, e, s);
  if (apt <= 4) return gemv_launch<1, SRC_A16, 1, GI, 4>(w, a, M, e, s);
  if (apt <= 8) return gemv_launch<1, SRC_A16, 1, GI, 8>(w, a, M, e, s);
  return gemv_launch<1, SRC_A16, 1, GI, 16>(w, a, M, e, s);
}

hipError_t launch_w4_gemv(const Packed& w, const ASrc& a, int M, const Epi& e, hipStream_t s) {
  if (!gemv_supported(M, w.K, a) || e.mode == EPI_QKV_ROPE) return hipErrorInvalidValue;
  if (a.emb) return e.mode == EPI_SWIGLU ? hipErrorInvalidValue : gemv_emb_rows<1>(w, a, M, e, s);
  if (a.x32) return e.mode == EPI_SWIGLU ? gemv_norm_rows<2>(w, a, M, e, s) : gemv_norm_rows<1>(w, a, M, e, s);
  if (e.mode == EPI_SWIGLU) return hipErrorInvalidValue;
  if (a.att) return gemv_att(w, a, M, e, s);
  return w.G <= 2 * kGemvWaves ? gemv_a16<2>(w, a, M, e, s) : gemv_a16<8>(w, a, M, e, s);
}

// ---------------------------------------------------------------- GEMM
// Prefill-shaped products (any M). A block of 4 waves computes a tile of
// 16*MB rows x 64*NBW columns: the waves share the activation rows (staged
// in LDS) and each owns NBW 16-column n-blocks, whose weight tiles and
// scales it streams straight into registers. Every 128-column group's
// activations (16 bytes per thread and m-block, in MFMA fragment order:
// block (mb, s) of a stage holds at byte 16*l row m0 + 16mb + l%16, columns
// 128g + 32s + 8(l/16)..+7) and weights are requested kGemmAhead groups before
// use into a register ring. Per group g:
//   - the activations of group g+1 are written to the other LDS stage;
//   - group g is computed from LDS and the weight registers of group g
//     (dequant in registers, v_mfma_f32_16x16x32_f16 into a per-group tile,
//     scaled once per group in fp32);
//   - group g + kGemmAhead is requested into the ring slot just freed; one
//     barrier (LDS only).
// At these sizes the loop is latency-bound, so the depth of the ring (not
// the tile shape) sets the speed. Plain vector loads (LDS-DMA measured about
// half the per-CU throughput); addresses clamped at the end of the K range
// and out-of-range groups meeting zero weights, so the unrolled loop body is
// straight-line code and the compiler's waits stay exact. Rows >= M and
// columns >= K read in-bounds elements: those rows are never stored and those
// columns meet zero weights. When the plan splits K over S blocks, each
// writes an fp32 partial tile and the consumer sums the S partials in order.
constexpr int kGemmAhead = 2;  // groups of loads in flight per wave (the loop is unrolled by it)

// Epilogue kinds, a template parameter so that each kind's kernel is
// register-allocated for its own epilogue: fp32 out (split-K partials,
// STORE, RESID), QKV_ROPE, SWIGLU.
enum GemmEp { GEP_F32 = 0, GEP_QKV = 1, GEP_SWIGLU = 2 };

template <int MB, int NBW, bool F16, int EP>
__global__ __launch_bounds__(256) void w4_gemm_kernel(const uint8_t* __restrict__ tiles,
                                                      const uint16_t* __restrict__ scales, int N, int K, int G,
                                                      const uint16_t* __restrict__ A, int M, Epi e, GemmPlan pl) {
  constexpr int kA = MB * 4 * 1024;  // one group's activation stage
  __shared__ __align__(16) uint8_t As[2][kA];
  const int L = blockIdx.x;
  const int U = pl.gy * pl.S;
  const int xcd = L & 7, r = L >> 3;
  const int cl = r / U, u = r - cl * U;
  const int cb = cl * 8 + xcd;
  if (cb >= pl.gx) return;  // padding block of the XCD mapping
  const int my = u / pl.S, sp = u - my * pl.S;
  const int kg0 = sp * pl.gps, kg1 = min(G, kg0 + pl.gps);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int NB = N / 16;
  const int nbw0 = (cb * 4 + wave) * NBW;
  const int m0 = my * 16 * MB;

  // this thread copies k-step s = wave of every m-block of a stage
  const uint16_t* arow[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) arow[i] = A + (size_t)min(m0 + i * 16 + l16, M - 1) * K;
  const int acol = 32 * wave + 8 * lq;
  const u32x4_t* btile[NBW];
  const uint16_t* bscale[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    const size_t nb = (size_t)min(nbw0 + j, NB - 1) * G;
    btile[j] = reinterpret_cast<const u32x4_t*>(tiles + nb * (F16 ? kTileBytesF16 : kTileBytes)) + lane;
    bscale[j] = F16 ? scales : scales + nb * 16 + l16;
  }

  constexpr int D = kGemmAhead;
  constexpr int WS = F16 ? 4 : 1;  // 16-byte weight slots per tile and lane
  u32x4_t ar[D][MB];
  u32x4_t br[D][NBW][WS];
  uint32_t bs[D][NBW];  // raw fp16 bits (W4 only)
  auto load_a = [&](u32x4_t (&ra)[MB], int g) {
    const int col = min(min(g, kg1 - 1) * 128 + acol, K - 8);
#pragma unroll
    for (int i = 0; i < MB; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(arow[i] + col);
  };
  auto load_b = [&](u32x4_t (&rb)[NBW][WS], uint32_t (&rs)[NBW], int g) {
    const int gc = min(g, kg1 - 1);
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      if constexpr (F16) {
#pragma unroll
        for (int s = 0; s < 4; ++s) rb[j][s] = btile[j][((size_t)gc * 4 + s) * 64];
        rs[j] = 0;
      } else {
        rb[j][0] = btile[j][(size_t)gc * 64];
        rs[j] = bscale[j][(size_t)gc * 16];
      }
    }
  };
  auto store_a = [&](const u32x4_t (&ra)[MB], int buf) {
#pragma unroll
    for (int i = 0; i < MB; ++i) *reinterpret_cast<u32x4_t*>(&As[buf][(i * 4 + wave) * 1024 + lane * 16]) = ra[i];
  };

  float4_t acc[MB][NBW];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf, const u32x4_t (&bw)[NBW][WS], const uint32_t (&bsc)[NBW], bool valid) {
    if constexpr (F16) {  // dense fp16 weights: straight into the accumulators
      const half8_t hz = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        half8_t af[MB], bf[NBW];
#pragma unroll
        for (int i = 0; i < MB; ++i)
          af[i] = *reinterpret_cast<const half8_t*>(&As[buf][(i * 4 + s) * 1024 + lane * 16]);
#pragma unroll
        for (int j = 0; j < NBW; ++j) bf[j] = valid ? __builtin_bit_cast(half8_t, bw[j][s]) : hz;
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NBW; ++j) acc[i][j] = mfma16(af[i], bf[j], acc[i][j]);
      }
      return;
    }
    float4_t t[MB][NBW];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NBW; ++j) t[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8_t af[MB], bf[NBW];
#pragma unroll
      for (int i = 0; i < MB; ++i) af[i] = *reinterpret_cast<const half8_t*>(&As[buf][(i * 4 + s) * 1024 + lane * 16]);
#pragma unroll
      for (int j = 0; j < NBW; ++j) bf[j] = dequant_word(valid ? bw[j][0][s] : 0x88888888u);  // 0x8: q = 0
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j) t[i][j] = mfma16(af[i], bf[j], t[i][j]);
    }
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const float sc = h2f((uint16_t)bsc[j]);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) acc[i][j][rr] = fmaf(t[i][j][rr], sc, acc[i][j][rr]);
    }
  };

  // prologue: groups kg0 .. kg0+D-1 requested; group kg0's activations staged
#pragma unroll
  for (int k = 0; k < D; ++k) {
    load_a(ar[k], kg0 + k);
    load_b(br[k], bs[k], kg0 + k);
  }
  store_a(ar[0], 0);
  lds_barrier();
  // D groups per trip (D even), so every ring slot and LDS stage is static
#pragma unroll 1
  for (int g = kg0; g < kg1; g += D) {
#pragma unroll
    for (int k = 0; k < D; ++k) {
      load_a(ar[k], g + k + D);                          // group g+k+D -> slot k (staged one step ago)
      store_a(ar[(k + 1) % D], (k + 1) & 1);            // group g+k+1 -> LDS
      compute(k & 1, br[k], bs[k], g + k < kg1);         // group g+k
      load_b(br[k], bs[k], g + k + D);
      lds_barrier();
    }
  }

  // ---- split-K: publish this split's partial tile; the kernel that consumes
  // the result sums the S partials in split order (kernel boundaries make
  // them visible; no in-kernel cross-block traffic).
  // Every epilogue stages each n-block's 16 columns of the wave's 16*MB rows
  // in the wave's own LDS slot (the activation stages are free once the last
  // group's barrier has passed), so that each lane then stores one 16-byte
  // run of consecutive output columns instead of scattered 2- or 4-byte
  // stores. Lane (lq, l16) holds C[m0 + 16i + 4lq + rr][16(nbw0 + j) + l16].
  float* stf = reinterpret_cast<float*>(&As[0][0]) + wave * (MB * 16 * 16);
  uint16_t* stg = reinterpret_cast<uint16_t*>(&As[0][0]) + wave * (MB * 16 * 16);
  auto stage = [&](int i, int rr, uint16_t v) { stg[(i * 16 + 4 * lq + rr) * 16 + l16] = v; };

  // ---- fp32 out: split-K partial tiles (the consumer sums the S partials in
  // split order; kernel boundaries make them visible), STORE, RESID
  if constexpr (EP == GEP_F32) {
    const bool resid = pl.S == 1 && e.mode == EPI_RESID;
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) stf[(i * 16 + 4 * lq + rr) * 16 + l16] = acc[i][j][rr];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's staging writes land before its reads
      if (nbw0 + j < NB) {
#pragma unroll
        for (int c = lane; c < MB * 64; c += 64) {  // 4 runs of 4 columns per row
          const int r = c >> 2, q4 = c & 3;
          const int m = m0 + r;
          float4_t v = *reinterpret_cast<const float4_t*>(stf + r * 16 + q4 * 4);
          if (m < M) {
            // 4 consecutive packed columns stay consecutive in natural order
            const int n = (nbw0 + j) * 16 + q4 * 4;
            const int nn = e.perm_hd ? qkv_natural_col(n, e.perm_hd) : n;
            float* dst = pl.S > 1 ? pl.part + ((size_t)sp * M + m) * N + nn : e.out_f32 + (size_t)m * e.ldo + nn;
            if (resid) v = *reinterpret_cast<const float4_t*>(dst) + v;
            *reinterpret_cast<float4_t*>(dst) = v;
          }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next n-block's writes
    }
    return;
  }

  // ---- QKV with RoPE, fp16 Q and the K/V cache rows (RoPE-pair packing:
  // lane l16 < 8 holds the first half of rotation pair t, lane l16 + 8 the
  // second half; both halves are rotated as rope_pair does)
  if constexpr (EP == GEP_QKV) {
    const int hd = e.kv.hd, half = hd / 2, d = e.kv.H * hd;
    uint8_t* base = e.kv.base + ((size_t)e.lane * e.kv.n_layers + e.layer) * e.kv.layer_bytes;
    const size_t HS = (size_t)e.kv.H * e.kv.cap;
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int n = min(nbw0 + j, NB - 1) * 16 + l16;
      const int sec = e.sec_base + n / d, p = n % hd;
      const bool first = (p & 15) < 8;
      const int t = 8 * (p >> 4) + (p & 7);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int m = m0 + i * 16 + 4 * lq + rr;
          const int pos = e.p0 + min(m, M - 1);
          const float v = acc[i][j][rr];
          const float other = dpp_mov<kDppRor8>(v);  // the pair partner, 8 lanes away
          float y = v;
          if (sec < 2) {
            const float c = e.rope[(size_t)pos * half + t];
            const float sn = e.rope[(size_t)e.kv.S * half + (size_t)pos * half + t];
            _Float16 y1, y2;
            rope_pair(first ? v : other, first ? other : v, c, sn, &y1, &y2);
            y = (float)(first ? y1 : y2);
          }
          stage(i, rr, f2h(y));
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's staging writes land before its reads
      if (nbw0 + j < NB) {
        // columns 0..7 of the n-block are dims t0..t0+7 of its head, 8..15 are half+t0..
        const int n0 = (nbw0 + j) * 16;
        const int sec0 = e.sec_base + n0 / d, hh = (n0 % d) / hd, t0 = 8 * ((n0 % hd) >> 4);
#pragma unroll
        for (int c = lane; c < MB * 32; c += 64) {
          const int r = c >> 1, hl = c & 1;
          const int m = m0 + r;
          const u32x4_t v8 = *reinterpret_cast<const u32x4_t*>(stg + r * 16 + hl * 8);
          if (m < M) {
            const int dim0 = hl ? half + t0 : t0;
            uint16_t* dst = sec0 == 0 ? e.qout + (size_t)m * d + hh * hd + dim0
                                      : reinterpret_cast<uint16_t*>(base) + (sec0 == 2 ? HS * hd : 0) +
                                            ((size_t)hh * e.kv.cap + kv_slot(e.kv, e.p0 + m)) * hd + dim0;
            *reinterpret_cast<u32x4_t*>(dst) = v8;
          }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next n-block's writes
    }
    return;
  }

  if constexpr (EP == GEP_SWIGLU) {
    if constexpr (NBW % 2 == 0) {
#pragma unroll
      for (int j = 0; j < NBW; j += 2) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) stage(i, rr, f2h(silu(acc[i][j][rr]) * acc[i][j + 1][rr]));
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (nbw0 + j < NB) {
          const int c0 = ((nbw0 + j) >> 1) * 16;
#pragma unroll
          for (int c = lane; c < MB * 32; c += 64) {
            const int r = c >> 1, hl = c & 1;
            const int m = m0 + r;
            const u32x4_t v8 = *reinterpret_cast<const u32x4_t*>(stg + r * 16 + hl * 8);
            if (m < M) *reinterpret_cast<u32x4_t*>(e.out_f16 + (size_t)m * e.ldo + c0 + hl * 8) = v8;
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
    }
    return;
  }
}

// Tile shape and K split. Sweeping every (rows, columns, split) on the
// 407M shapes at M = 128 and 1024 put the best tile at 32 rows x 128
// columns (2 x 2 MFMA tiles per wave) almost everywhere, the loop being
// bound by latency and VALU rather than bytes: more blocks in flight beat
// bigger tiles. K is split (fp32 partials, summed by the consumer) until
// there are 384 blocks, keeping at least 4 groups per split; the columns
// narrow to 64 only when even the split grid stays below 256 blocks (at
// M = 128 the down projection then runs 8 splits of 32 x 128 tiles instead
// of 4 splits of 32 x 64: 10.5 -> 9.8 us, partials included).
GemmPlan plan_w4_gemm(int N, int K, int M, bool swiglu, bool unsplit) {
  const int NB = N / 16, G = (K + 127) / 128;
  GemmPlan p{};
  p.mb = M <= 16 ? 1 : 2;
  p.gy = (M + 16 * p.mb - 1) / (16 * p.mb);
  auto splits = [&](int gx) {
    int S = 1;
    if (!swiglu && !unsplit)
      while (S < kMaxSplitK && gx * p.gy * S < 384 && G / (2 * S) >= 4) S *= 2;
    return S;
  };
  p.nbw = 2;
  p.gx = (NB + 4 * p.nbw - 1) / (4 * p.nbw);
  int S = splits(p.gx);
  if (!swiglu && p.gx * p.gy * S < 256) {
    p.nbw = 1;
    p.gx = (NB + 3) / 4;
    S = splits(p.gx);
  }
  p.gps = (G + S - 1) / S;
  p.S = (G + p.gps - 1) / p.gps;
  p.blocks = ((p.gx + 7) / 8) * 8 * p.gy * p.S;
  return p;
}

size_t w4_gemm_scratch_bytes(int N, int K, int M, bool swiglu) {
  const GemmPlan p = plan_w4_gemm(N, K, M, swiglu, false);
  if (p.S == 1) return 0;
  return (size_t)p.S * M * N * 4;
}

// out[m][n] (= or +=) sum_s part[s][m][n], summed in split order.
__global__ void reduce_partials_kernel(const float* __restrict__ part, int S, int M, int N, float* __restrict__ out,
                                       int accumulate) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t MN = (size_t)M * N;
  if (i >= MN) return;
  float v = part[i];
  for (int s = 1; s < S; ++s) v += part[s * MN + i];
  out[i] = accumulate ? out[i] + v : v;
}

hipError_t launch_reduce_partials(const float* part, int S, int M, int N, float* out, int accumulate, hipStream_t s) {
  const size_t MN = (size_t)M * N;
  launch(reduce_partials_kernel, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, s, part, S, M, N, out,
                     accumulate);
  return hipGetLastError();
}

template <int MB, int NBW, int EP>
static hipError_t gemm_launch_ep(const Packed& w, const uint16_t* A, int M, const Epi& e, const GemmPlan& pl,
                                 hipStream_t s) {
  if (w.f16)
    launch((w4_gemm_kernel<MB, NBW, true, EP>), dim3(pl.blocks), dim3(256), 0, s, w.tiles, w.scales, w.N, w.K, w.G,
           A, M, e, pl);
  else
    launch((w4_gemm_kernel<MB, NBW, false, EP>), dim3(pl.blocks), dim3(256), 0, s, w.tiles, w.scales, w.N, w.K, w.G,
           A, M, e, pl);
  return hipGetLastError();
}
template <int MB, int NBW>
static hipError_t gemm_launch(const Packed& w, const uint16_t* A, int M, const Epi& e, const GemmPlan& pl,
                              hipStream_t s) {
  if (pl.S > 1 || e.mode == EPI_STORE || e.mode == EPI_RESID) return gemm_launch_ep<MB, NBW, GEP_F32>(w, A, M, e, pl, s);
  if (e.mode == EPI_QKV_ROPE) return gemm_launch_ep<MB, NBW, GEP_QKV>(w, A, M, e, pl, s);
  if constexpr (NBW % 2 == 0)
    if (e.mode == EPI_SWIGLU) return gemm_launch_ep<MB, NBW, GEP_SWIGLU>(w, A, M, e, pl, s);
  return hipErrorInvalidValue;
}

hipError_t launch_w4_gemm(const Packed& w, const uint16_t* A, int M, const Epi& e, float* part, hipStream_t s) {
  if (M < 1) return hipErrorInvalidValue;
  GemmPlan pl = plan_w4_gemm(w.N, w.K, M, e.mode == EPI_SWIGLU, e.mode == EPI_QKV_ROPE);
  if (pl.S > 1 && !part) return hipErrorInvalidValue;
  if (e.mode == EPI_QKV_ROPE) {
    const int d = e.kv.H * e.kv.hd;
    if (e.kv.int8 || e.perm_hd != e.kv.hd || w.N % d || e.sec_base < 0 || e.sec_base + w.N / d > 3)
      return hipErrorInvalidValue;
  }
  pl.part = part;
  if (pl.nbw == 2) return pl.mb == 2 ? gemm_launch<2, 2>(w, A, M, e, pl, s) : gemm_launch<1, 2>(w, A, M, e, pl, s);
  return pl.mb == 2 ? gemm_launch<2, 1>(w, A, M, e, pl, s) : gemm_launch<1, 1>(w, A, M, e, pl, s);
}

}  // namespace tl
