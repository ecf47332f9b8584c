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
#include "tl_device.h"
#include "tl_kernels.h"

namespace tl {

// ---------------------------------------------------------------- epilogue
__device__ __forceinline__ void epi_store(const Epi& e, int m, int n, float v) {
  if (e.mode == EPI_RESID)
    e.out_f32[(size_t)m * e.ldo + n] += v;
  else
    e.out_f32[(size_t)m * e.ldo + n] = v;
}
__device__ __forceinline__ void epi_swiglu(const Epi& e, int m, int c, float g, float u) {
  e.out_f16[(size_t)m * e.ldo + c] = f2h(silu(g) * u);
}

// ---------------------------------------------------------------- GEMV
constexpr int kGemvMaxIt = 8;  // weight tiles kept in flight per wave and n-block

template <int WK, int NBB>
__global__ __launch_bounds__(WK * 64) void w4_gemv_kernel(const uint8_t* __restrict__ tiles,
                                                          const uint16_t* __restrict__ scales, int N, int K,
                                                          int G, ASrc a, int M, Epi e) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int lda = G * 128 + 8;  // LDS row stride in halves (16-byte pad)
  _Float16* As = reinterpret_cast<_Float16*>(smem);
  float* red = reinterpret_cast<float*>(smem + (((size_t)M * lda * 2 + 15) & ~(size_t)15));
  float* nrm = red + WK * NBB * 256;  // [WK][16] sum-of-squares partials, then [16] rinv

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int nb0 = blockIdx.x * NBB;
  const int Kp = G * 128;

  // ---- stage the M activation rows (fp16) into LDS
  if (a.x32) {
    for (int m = 0; m < M; ++m) {
      const float* xr = a.x32 + (size_t)m * K;
      float acc = 0.f;
      for (int k = tid; k < K; k += WK * 64) acc += xr[k] * xr[k];
      acc = wave_sum(acc);
      if (lane == 0) nrm[wave * 16 + m] = acc;
    }
    __syncthreads();
    if (tid < M) {
      float t = 0.f;
      for (int w = 0; w < WK; ++w) t += nrm[w * 16 + tid];
      nrm[WK * 16 + tid] = 1.0f / sqrtf(t / (float)K + a.eps);
    }
    __syncthreads();
    for (int m = 0; m < M; ++m) {
      const float rinv = nrm[WK * 16 + m];
      const float* xr = a.x32 + (size_t)m * K;
      for (int k = tid; k < Kp; k += WK * 64) {
        float v = 0.f;
        if (k < K) v = (xr[k] * rinv) * h2f(a.gamma[k]);
        As[m * lda + k] = (_Float16)v;
      }
    }
  } else {
    const int chunks = Kp / 8;
    for (int i = tid; i < M * chunks; i += WK * 64) {
      const int m = i / chunks, c = (i - m * chunks) * 8;
      u32x4_t v = {0, 0, 0, 0};
      if (c < K) v = *reinterpret_cast<const u32x4_t*>(a.a16 + (size_t)m * K + c);
      *reinterpret_cast<u32x4_t*>(As + m * lda + c) = v;
    }
  }
  __syncthreads();

  // ---- K groups g = wave, wave + WK, ... ; up to kGemvMaxIt tiles in flight
  float4_t acc[NBB];
#pragma unroll
  for (int j = 0; j < NBB; ++j) acc[j] = (float4_t){0.f, 0.f, 0.f, 0.f};
  const bool arow = l16 < M;
  const half8_t hz = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int gb = wave; gb < G; gb += WK * kGemvMaxIt) {
    u32x4_t wv[kGemvMaxIt][NBB];
    float sc[kGemvMaxIt][NBB];
#pragma unroll
    for (int it = 0; it < kGemvMaxIt; ++it) {
      const int g = gb + it * WK;
#pragma unroll
      for (int j = 0; j < NBB; ++j) {
        if (g < G) {
          const size_t tile = (size_t)(nb0 + j) * G + g;
          wv[it][j] = *reinterpret_cast<const u32x4_t*>(tiles + tile * kTileBytes + lane * 16);
          sc[it][j] = h2f(scales[tile * 16 + l16]);
        }
      }
    }
#pragma unroll
    for (int it = 0; it < kGemvMaxIt; ++it) {
      const int g = gb + it * WK;
      if (g < G) {
        half8_t af[4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
          af[s] = arow ? *reinterpret_cast<const half8_t*>(As + l16 * lda + g * 128 + 32 * s + 8 * lq) : hz;
#pragma unroll
        for (int j = 0; j < NBB; ++j) {
          float4_t t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s) t = mfma16(af[s], dequant_word(wv[it][j][s]), t);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[j][r] = fmaf(t[r], sc[it][j], acc[j][r]);
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

template <int WK, int NBB>
static hipError_t gemv_launch(const Packed& w, const ASrc& a, int M, const Epi& e, hipStream_t s) {
  const size_t lds = (((size_t)M * (w.G * 128 + 8) * 2 + 15) & ~(size_t)15) + (size_t)WK * NBB * 256 * 4 +
                     (size_t)(WK + 1) * 16 * 4;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&w4_gemv_kernel<WK, NBB>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  const int blocks = w.N / 16 / NBB;
  hipLaunchKernelGGL((w4_gemv_kernel<WK, NBB>), dim3(blocks), dim3(WK * 64), lds, s, w.tiles, w.scales, w.N,
                     w.K, w.G, a, M, e);
  return hipGetLastError();
}

hipError_t launch_w4_gemv(const Packed& w, const ASrc& a, int M, const Epi& e, hipStream_t s) {
  if (M < 1 || M > 16) return hipErrorInvalidValue;
  if (e.mode == EPI_SWIGLU) return gemv_launch<8, 2>(w, a, M, e, s);
  return gemv_launch<8, 1>(w, a, M, e, s);
}

// ---------------------------------------------------------------- GEMM
constexpr int kLdsA = 136;  // halves per LDS row of the A tile (128 + 8 pad)

template <int MB, int NBW>
__global__ __launch_bounds__(256) void w4_gemm_kernel(const uint8_t* __restrict__ tiles,
                                                      const uint16_t* __restrict__ scales, int N, int K, int G,
                                                      const uint16_t* __restrict__ A, int M, Epi e) {
  constexpr int BM = 16 * MB;
  __shared__ __align__(16) _Float16 As[2][BM * kLdsA];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int NB = N / 16;
  const int nbw0 = (blockIdx.x * 4 + wave) * NBW;
  const int m0 = blockIdx.y * BM;

  // A loader: BM rows x 16 chunks of 8 halves = MB chunks per thread.
  u32x4_t an[MB];
  auto load_a = [&](int g) {
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int c = tid + 256 * i, row = c >> 4, col = g * 128 + (c & 15) * 8;
      const int m = m0 + row;
      u32x4_t v = {0, 0, 0, 0};
      if (m < M && col < K) v = *reinterpret_cast<const u32x4_t*>(A + (size_t)m * K + col);
      an[i] = v;
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int c = tid + 256 * i, row = c >> 4;
      *reinterpret_cast<u32x4_t*>(&As[buf][row * kLdsA + (c & 15) * 8]) = an[i];
    }
  };
  u32x4_t bw[NBW], bn[NBW];
  float bs[NBW], bsn[NBW];
  auto load_b = [&](int g, u32x4_t* w, float* sc) {
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int nb = nbw0 + j;
      if (nb < NB) {
        const size_t tile = (size_t)nb * G + g;
        w[j] = *reinterpret_cast<const u32x4_t*>(tiles + tile * kTileBytes + lane * 16);
        sc[j] = h2f(scales[tile * 16 + l16]);
      } else {
        w[j] = (u32x4_t){0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
        sc[j] = 0.f;
      }
    }
  };

  float4_t acc[MB][NBW];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};

  load_a(0);
  store_a(0);
  load_b(0, bw, bs);
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    if (g + 1 < G) {
      load_a(g + 1);
      load_b(g + 1, bn, bsn);
    }
    float4_t t[MB][NBW];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NBW; ++j) t[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8_t bf[NBW];
#pragma unroll
      for (int j = 0; j < NBW; ++j) bf[j] = dequant_word(bw[j][s]);
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const half8_t af =
            *reinterpret_cast<const half8_t*>(&As[buf][(i * 16 + l16) * kLdsA + 32 * s + 8 * lq]);
#pragma unroll
        for (int j = 0; j < NBW; ++j) t[i][j] = mfma16(af, bf[j], t[i][j]);
      }
    }
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(t[i][j][r], bs[j], acc[i][j][r]);
    if (g + 1 < G) {
      store_a(buf ^ 1);
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        bw[j] = bn[j];
        bs[j] = bsn[j];
      }
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds C[m0 + 16i + 4lq + r][16*(nbw0 + j) + l16]
#pragma unroll
  for (int i = 0; i < MB; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + i * 16 + 4 * lq + r;
      if (m >= M) continue;
      if (e.mode == EPI_SWIGLU) {
        if constexpr (NBW % 2 == 0) {
#pragma unroll
          for (int j = 0; j < NBW; j += 2)
            if (nbw0 + j < NB) epi_swiglu(e, m, ((nbw0 + j) >> 1) * 16 + l16, acc[i][j][r], acc[i][j + 1][r]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NBW; ++j)
          if (nbw0 + j < NB) epi_store(e, m, (nbw0 + j) * 16 + l16, acc[i][j][r]);
      }
    }
  }
}

template <int MB, int NBW>
static hipError_t gemm_launch(const Packed& w, const uint16_t* A, int M, const Epi& e, hipStream_t s) {
  const int NB = w.N / 16;
  dim3 grid((NB + 4 * NBW - 1) / (4 * NBW), (M + 16 * MB - 1) / (16 * MB));
  hipLaunchKernelGGL((w4_gemm_kernel<MB, NBW>), grid, dim3(256), 0, s, w.tiles, w.scales, w.N, w.K, w.G, A, M, e);
  return hipGetLastError();
}

hipError_t launch_w4_gemm(const Packed& w, const uint16_t* A, int M, const Epi& e, hipStream_t s) {
  if (M < 1) return hipErrorInvalidValue;
  const int NB = w.N / 16;
  const bool swiglu = e.mode == EPI_SWIGLU;
  // Two n-blocks per wave when the shape allows (SwiGLU needs the gate/up pair).
  const int nbw = (swiglu || NB % 8 == 0) ? 2 : 1;
  // Largest row tile that still gives about one block per CU.
  int mb = M > 64 ? 8 : (M > 32 ? 4 : (M > 16 ? 2 : 1));
  auto blocks = [&](int mbv) { return ((NB + 4 * nbw - 1) / (4 * nbw)) * ((M + 16 * mbv - 1) / (16 * mbv)); };
  while (mb > 1 && blocks(mb) < 240) mb >>= 1;
  if (nbw == 2) {
    switch (mb) {
      case 8: return gemm_launch<8, 2>(w, A, M, e, s);
      case 4: return gemm_launch<4, 2>(w, A, M, e, s);
      case 2: return gemm_launch<2, 2>(w, A, M, e, s);
      default: return gemm_launch<1, 2>(w, A, M, e, s);
    }
  }
  switch (mb) {
    case 8: return gemm_launch<8, 1>(w, A, M, e, s);
    case 4: return gemm_launch<4, 1>(w, A, M, e, s);
    case 2: return gemm_launch<2, 1>(w, A, M, e, s);
    default: return gemm_launch<1, 1>(w, A, M, e, s);
  }
}

}  // namespace tl
