// Decode GEMV of the W4 loop block (gfx950, v_mfma_f32_16x16x32_f16); the
// arithmetic shared with the prefill GEMM is described in w4_epi.h.
//
// M <= 16 rows: one m-block; a block owns 1 or 2 n-blocks and its waves split
// the K groups round-robin; partial tiles are summed across waves in LDS in
// fixed wave order (the result does not depend on M or on which rows are
// present). The activation rows are staged in LDS once, optionally
// RMS-normalised from the fp32 residual on the way in.
//
// This translation unit is compiled with the memory-clause machine scheduler
// (build.py): it keeps each wave's weight requests together ahead of the
// math, which measured 1.1-1.5% faster decode steps than the default
// schedule, with the same instructions and results.
#include <type_traits>

#include "w4_epi.h"

namespace tl {

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

// GI: groups requested per wave (ceil(G / 8) rounded up to 2, 6 or 8; a wave
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
  // the residual values the epilogue adds to (EPI_RESID), requested last: the
  // epilogue thread (row em, column ecol of each n-block) owns them, so they
  // need no wait until the end and no dependent load remains there
  const int eln = tid >> 2, er = tid & 3;
  const int em = 4 * (eln >> 4) + er, ecol = eln & 15;
  const bool eout = tid < 256 && em < M;
  float rx[NBB];
#pragma unroll
  for (int j = 0; j < NBB; ++j) {
    rx[j] = 0.f;
    if (e.mode == EPI_RESID && eout) rx[j] = e.out_f32[epi_index(e, em, (nb0 + j) * 16 + ecol)];
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
      // row m's parts are pairs q0 .. q1-1 (row-major); one weight and one
      // sum per part, shared by the thread's 4 columns (the merge kernel's
      // per-element arithmetic, attn_merge_step, in the same order)
      const int q0 = m * a.att_np, q1 = min(q0 + a.att_np, npairs);
      float gm = -INFINITY;
#pragma unroll
      for (int q = 0; q < APT; ++q)
        if (q >= q0 && q < q1) gm = fmaxf(gm, ml[q].x);
      float num[4] = {0.f, 0.f, 0.f, 0.f}, den = 0.f;
#pragma unroll
      for (int q = 0; q < APT; ++q)
        if (q >= q0 && q < q1 && ml[q].x != -INFINITY) {
          const float w = __builtin_amdgcn_exp2f(ml[q].x - gm);
          den = fmaf(w, ml[q].y, den);
#pragma unroll
          for (int c = 0; c < 4; ++c) num[c] = fmaf(w, xv[q][c], num[c]);
        }
      if (k4 < Kp) {
        half2_t h01, h23;
        h01.x = (_Float16)(num[0] / den);
        h01.y = (_Float16)(num[1] / den);
        h23.x = (_Float16)(num[2] / den);
        h23.y = (_Float16)(num[3] / den);
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
  if (eout) {
    float v[NBB];
#pragma unroll
    for (int j = 0; j < NBB; ++j) {
      float t = 0.f;
      for (int w = 0; w < WK; ++w) t += red[((w * NBB + j) * 64 + eln) * 4 + er];
      v[j] = t;
    }
    if (e.mode == EPI_SWIGLU) {
      if constexpr (NBB == 2) epi_swiglu(e, em, blockIdx.x * 16 + ecol, v[0], v[1]);
    } else {
#pragma unroll
      for (int j = 0; j < NBB; ++j)
        e.out_f32[epi_index(e, em, (nb0 + j) * 16 + ecol)] = e.mode == EPI_RESID ? rx[j] + v[j] : v[j];
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
  // two n-blocks per block where they pair up: half the blocks repeat the
  // fused RMSNorm (QKV at the 407M shape: decode 0.2617 -> 0.2608 ms/token,
  // INT8 context 2048 0.317 -> 0.316, three lanes 1.203 -> 1.195, same bits)
  if (a.x32)
    return e.mode == EPI_SWIGLU || (w.N / 16) % 2 == 0 ? gemv_norm_rows<2>(w, a, M, e, s)
                                                       : gemv_norm_rows<1>(w, a, M, e, s);
  if (e.mode == EPI_SWIGLU) return hipErrorInvalidValue;
  if (a.att) return gemv_att(w, a, M, e, s);
  if (w.G <= 2 * kGemvWaves) return gemv_a16<2>(w, a, M, e, s);
  return w.G <= 6 * kGemvWaves ? gemv_a16<6>(w, a, M, e, s) : gemv_a16<8>(w, a, M, e, s);
}

}  // namespace tl
