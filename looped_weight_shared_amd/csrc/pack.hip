// Weight ingest: canonical INT4 linear -> packed MFMA-fragment tiles.
//
// Canonical input (the model family's INT4 weights: eight signed 4-bit values
// per 32-bit word along K, least significant nibble first, one FP16 scale per
// 128 input channels): qweight uint32 [N][K/8], scales fp16 [N][ceil(K/128)].
//
// Packed output, per 16-row n-block nb and 128-column group g (1 KiB tile):
// lane slot l (16 bytes) holds row 16*nb + l%16, word s of the slot the 8
// columns 128*g + 32*s + 8*(l/16) + 0..7. Inside a word, nibble p is column
// 2p and nibble p + 4 column 2p + 1, each stored offset-binary (q + 8).
// Columns at or beyond K are stored as q = 0. Scales follow all tiles as
// fp16 [N/16][G][16].
#include "tl_device.h"
#include "tl_kernels.h"

namespace tl {

// Canonical word (nibble j = column j, two's complement) -> packed word.
__device__ __forceinline__ uint32_t repack_word(uint32_t cw) {
  uint32_t out = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t even = (cw >> (8 * p)) & 0xFu;      // column 2p
    uint32_t odd = (cw >> (8 * p + 4)) & 0xFu;   // column 2p+1
    out |= even << (4 * p);
    out |= odd << (16 + 4 * p);
  }
  return out ^ 0x88888888u;  // two's complement -> offset binary
}

// One thread per packed word.
__global__ void pack_kernel(const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc, int N, int K,
                            uint32_t* __restrict__ dst, uint16_t* __restrict__ dst_sc, int G, int nb_offset,
                            int nb_stride, int perm_hd) {
  const int G_src = (K + 127) / 128;
  const long long total = (long long)(N / 16) * G_src * 256;  // words
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int s = (int)(i & 3);
  const int l = (int)((i >> 2) & 63);
  const long long tile = i >> 8;
  const int g = (int)(tile % G_src);
  const int nb = (int)(tile / G_src);
  const int n = perm_hd ? qkv_natural_col(nb * 16 + (l & 15), perm_hd) : nb * 16 + (l & 15);
  const int k0 = g * 128 + 32 * s + 8 * (l >> 4);
  uint32_t w = 0x88888888u;  // all zeros
  if (k0 < K) w = repack_word(qw[(size_t)n * (K / 8) + k0 / 8]);
  const int dnb = nb_offset + nb * nb_stride;
  dst[(((size_t)dnb * G + g) * 64 + l) * 4 + s] = w;
  if (s == 0 && l < 16) dst_sc[((size_t)dnb * G + g) * 16 + l] = sc[(size_t)n * G_src + g];
}

hipError_t launch_pack(const uint32_t* qweight, const uint16_t* scales, int N, int K, uint8_t* dst_tiles,
                       uint16_t* dst_scales, int dst_G, int nb_offset, int nb_stride, int perm_hd, hipStream_t s) {
  if (perm_hd && (perm_hd % 16 || N % perm_hd)) return hipErrorInvalidValue;
  const long long total = (long long)(N / 16) * ((K + 127) / 128) * 256;
  const int threads = 256;
  const long long blocks = (total + threads - 1) / threads;
  launch(pack_kernel, dim3((unsigned)blocks), dim3(threads), 0, s, qweight, scales, N, K,
                     reinterpret_cast<uint32_t*>(dst_tiles), dst_scales, dst_G, nb_offset, nb_stride, perm_hd);
  return hipGetLastError();
}

// FP16 body tiles: one thread per 16-byte slot (8 columns of one row).
__global__ void pack_f16_kernel(const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc, int N, int K,
                                uint32_t* __restrict__ dst, int G, int nb_offset, int nb_stride, int perm_hd) {
  const int G_src = (K + 127) / 128;
  const long long total = (long long)(N / 16) * G_src * 256;  // slots
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int l = (int)(i & 63);
  const int s = (int)((i >> 6) & 3);
  const long long tile = i >> 8;
  const int g = (int)(tile % G_src);
  const int nb = (int)(tile / G_src);
  const int n = perm_hd ? qkv_natural_col(nb * 16 + (l & 15), perm_hd) : nb * 16 + (l & 15);
  const int k0 = g * 128 + 32 * s + 8 * (l >> 4);
  uint32_t out[4] = {0, 0, 0, 0};
  if (k0 < K) {
    const uint32_t cw = qw[(size_t)n * (K / 8) + k0 / 8];
    const float scale = (float)__builtin_bit_cast(_Float16, sc[(size_t)n * G_src + g]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int q = (int)((cw >> (4 * e)) & 0xFu) - (((cw >> (4 * e)) & 0x8u) ? 16 : 0);  // two's complement nibble
      const uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)((float)q * scale));    // exact product, one rounding
      out[e >> 1] |= h << (16 * (e & 1));
    }
  }
  const int dnb = nb_offset + nb * nb_stride;
  uint32_t* d = dst + ((((size_t)dnb * G + g) * 4 + s) * 64 + l) * 4;
  d[0] = out[0];
  d[1] = out[1];
  d[2] = out[2];
  d[3] = out[3];
}

hipError_t launch_pack_f16(const uint32_t* qweight, const uint16_t* scales, int N, int K, uint8_t* dst_tiles, int dst_G,
                           int nb_offset, int nb_stride, int perm_hd, hipStream_t s) {
  if (perm_hd && (perm_hd % 16 || N % perm_hd)) return hipErrorInvalidValue;
  const long long total = (long long)(N / 16) * ((K + 127) / 128) * 256;
  launch(pack_f16_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, qweight, scales, N, K,
         reinterpret_cast<uint32_t*>(dst_tiles), dst_G, nb_offset, nb_stride, perm_hd);
  return hipGetLastError();
}

// Inverse view: packed -> int8 [N][K] values and fp16 [N][G] scales.
__global__ void unpack_kernel(const uint32_t* __restrict__ src, const uint16_t* __restrict__ src_sc, int N, int K,
                              int G, int8_t* __restrict__ q, uint16_t* __restrict__ sc) {
  const long long total = (long long)(N / 16) * G * 256;
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int s = (int)(i & 3);
  const int l = (int)((i >> 2) & 63);
  const long long tile = i >> 8;
  const int g = (int)(tile % G);
  const int nb = (int)(tile / G);
  const int n = nb * 16 + (l & 15);
  const int k0 = g * 128 + 32 * s + 8 * (l >> 4);
  const uint32_t w = src[i];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int even = (int)((w >> (4 * p)) & 0xFu) - 8;
    const int odd = (int)((w >> (16 + 4 * p)) & 0xFu) - 8;
    if (k0 + 2 * p < K) q[(size_t)n * K + k0 + 2 * p] = (int8_t)even;
    if (k0 + 2 * p + 1 < K) q[(size_t)n * K + k0 + 2 * p + 1] = (int8_t)odd;
  }
  if (s == 0 && l < 16) sc[(size_t)n * G + g] = src_sc[tile * 16 + l];
}

hipError_t launch_unpack(const Packed& p, int8_t* q, uint16_t* scales, hipStream_t s) {
  const long long total = (long long)(p.N / 16) * p.G * 256;
  const int threads = 256;
  const long long blocks = (total + threads - 1) / threads;
  launch(unpack_kernel, dim3((unsigned)blocks), dim3(threads), 0, s,
                     reinterpret_cast<const uint32_t*>(p.tiles), p.scales, p.N, p.K, p.G, q, scales);
  return hipGetLastError();
}

// FP16 head [V][d] -> tiles [ceil(V/16)][d/32][64 lanes][16 B]: lane l of
// tile (nb, s) holds row 16nb + l%16, columns 32s + 8(l/16)..+7 -- the B
// operand of one v_mfma_f32_16x16x32_f16 step, read by a wave as one
// contiguous 1 KiB. Rows past V are zero.
__global__ void pack_head_kernel(const uint16_t* __restrict__ head, int V, int d, uint8_t* __restrict__ dst,
                                 size_t n_slots) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_slots) return;
  const int nsteps = d / 32;
  const int l = (int)(i & 63);
  const size_t t = i >> 6;
  const int st = (int)(t % nsteps);
  const size_t nb = t / nsteps;
  const size_t row = nb * 16 + (l & 15);
  u32x4_t v = {0, 0, 0, 0};
  if (row < (size_t)V) v = *reinterpret_cast<const u32x4_t*>(head + row * d + st * 32 + 8 * (l >> 4));
  *reinterpret_cast<u32x4_t*>(dst + i * 16) = v;
}

hipError_t launch_pack_head(const uint16_t* head, int V, int d, uint8_t* dst, hipStream_t s) {
  if (V < 1 || d < 32 || d % 32) return hipErrorInvalidValue;
  const size_t n_slots = head_packed_bytes(V, d) / 16;
  launch(pack_head_kernel, dim3((unsigned)((n_slots + 255) / 256)), dim3(256), 0, s, head, V, d, dst, n_slots);
  return hipGetLastError();
}

}  // namespace tl
