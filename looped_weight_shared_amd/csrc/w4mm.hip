// Prefill GEMM of the W4 loop block (gfx950, v_mfma_f32_16x16x32_f16); the
// arithmetic shared with the decode GEMV is described in w4_epi.h.
//
// A block is 4 waves side by side along N, each owning NBW n-blocks for all
// BM = 16*MB rows; the fp16 activation tile of each group is double-buffered
// through LDS (global loads of group g+1 overlap the MFMAs of group g) and
// shared by the 4 waves, while each wave streams its own weight tiles one
// group ahead.
#include <type_traits>

#include "w4_epi.h"

namespace tl {

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

// MB m-blocks x NBW n-blocks per wave, the block's 4 waves side by side along
// N: a block tile is 16*MB rows x 64*NBW columns. The small tiles (MB <= 2)
// request activations two groups ahead; the large-M tile (MB = 8, NBW = 2:
// 128 x 128 per block, 128 x 32 per wave) feeds each dequantized weight word
// to 8 MFMAs instead of 2, requests its 32 KiB activation stage one group
// ahead and runs 2 waves per SIMD (2 blocks per CU).
template <int MB, int NBW, bool F16, int EP>
__global__ __launch_bounds__(256, MB > 2 ? 2 : 1) void w4_gemm_kernel(const uint8_t* __restrict__ tiles,
                                                                      const uint16_t* __restrict__ scales, int N,
                                                                      int K, int G, const uint16_t* __restrict__ A,
                                                                      int M, Epi e, GemmPlan pl) {
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

  // The large-M tile (MB > 2) keeps its addresses in scalar registers where it
  // can (the wave index is uniform) and its rows as 32-bit offsets: eight
  // 64-bit row pointers per lane would not fit its register budget. The small
  // tiles keep per-lane pointers (measured ~1% faster in the forward pass).
  constexpr bool kBig = MB > 2;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = kBig ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int NB = N / 16;
  const int nbw0 = (cb * 4 + wave) * NBW;
  const int m0 = my * 16 * MB;

  // this thread copies k-step s = wave of every m-block of a stage (rows past
  // M read row M-1; they are never stored)
  const uint16_t* arow[kBig ? 1 : MB];
  if constexpr (!kBig) {
#pragma unroll
    for (int i = 0; i < MB; ++i) arow[i] = A + (size_t)min(m0 + i * 16 + l16, M - 1) * K;
  }
  const int arow0 = (m0 + l16) * K, arow_last = (M - 1) * K;  // large tile: element offsets
  const int acol = 32 * wave + 8 * lq;
  const uint8_t* btile[NBW];  // large tile: per-wave (uniform) bases; small: this lane's slot
  const uint16_t* bscale[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    const size_t nb = (size_t)min(nbw0 + j, NB - 1) * G;
    btile[j] = tiles + nb * (F16 ? kTileBytesF16 : kTileBytes) + (kBig ? 0 : lane * 16);
    bscale[j] = F16 ? scales : scales + nb * 16 + (kBig ? 0 : l16);
  }
  const int bl16 = kBig ? lane * 16 : 0, sl16 = kBig ? l16 : 0;

  constexpr int D = kGemmAhead;
  // activation groups held in registers ahead of their LDS stage: 2 for the
  // small tiles, 1 for the large-M tile (its stage is 4x larger, and one
  // group's 64 MFMAs per wave cover the loads of the next)
  constexpr int DA = MB <= 2 ? D : 1;
  constexpr int WS = F16 ? 4 : 1;  // 16-byte weight slots per tile and lane
  u32x4_t ar[DA][MB];
  u32x4_t br[D][NBW][WS];
  uint32_t bs[D][NBW];  // raw fp16 bits (W4 only)
  auto load_a = [&](u32x4_t (&ra)[MB], int g) {
    const int col = min(min(g, kg1 - 1) * 128 + acol, K - 8);
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if constexpr (kBig)
        ra[i] = *reinterpret_cast<const u32x4_t*>(A + (min(arow0 + i * 16 * K, arow_last) + col));
      else
        ra[i] = *reinterpret_cast<const u32x4_t*>(arow[i] + col);
    }
  };
  auto load_b = [&](u32x4_t (&rb)[NBW][WS], uint32_t (&rs)[NBW], int g) {
    const int gc = min(g, kg1 - 1);
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      if constexpr (F16) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          rb[j][s] = *reinterpret_cast<const u32x4_t*>(btile[j] + ((size_t)gc * 4 + s) * 1024 + bl16);
        rs[j] = 0;
      } else {
        rb[j][0] = *reinterpret_cast<const u32x4_t*>(btile[j] + (size_t)gc * kTileBytes + bl16);
        rs[j] = bscale[j][(size_t)gc * 16 + sl16];
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
    // The small tiles pin the group's weight words and scales here, after
    // the previous group's barrier: left free, the scheduler hoists the next
    // group's zero-select and dequantization above that barrier, and the wait
    // for those registers then covers the loads requested one step earlier
    // (a vmcnt(0) per trip) instead of two (seq-128 prefill 0.591 -> 0.582
    // ms/step, same bits). The large-M tiles measured slower pinned.
    u32x4_t wv[NBW];
    uint32_t sv[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      wv[j] = bw[j][0];
      sv[j] = bsc[j];
      if constexpr (!kBig) asm volatile("" : "+v"(wv[j]), "+v"(sv[j]));
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8_t af[MB], bf[NBW];
#pragma unroll
      for (int i = 0; i < MB; ++i) af[i] = *reinterpret_cast<const half8_t*>(&As[buf][(i * 4 + s) * 1024 + lane * 16]);
#pragma unroll
      for (int j = 0; j < NBW; ++j) bf[j] = dequant_word(valid ? wv[j][s] : 0x88888888u);  // 0x8: q = 0
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j) t[i][j] = mfma16(af[i], bf[j], t[i][j]);
    }
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const float sc = h2f((uint16_t)sv[j]);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) acc[i][j][rr] = fmaf(t[i][j][rr], sc, acc[i][j][rr]);
    }
  };

  // QKV epilogue of the small tiles: the RoPE cos/sin of every output this
  // lane writes, requested with the first groups rather than after the loop
  // (they depend on nothing the loop computes)
  constexpr bool kRopePre = EP == GEP_QKV && !kBig;
  float rcs[kRopePre ? NBW : 1][kRopePre ? MB : 1][4][2];
  auto rope_at = [&](int j, int i, int rr) {
    const int half = e.kv.hd / 2;
    const int n = min(nbw0 + j, NB - 1) * 16 + l16, p = n % e.kv.hd;
    const int t = 8 * (p >> 4) + (p & 7);
    const int pos = e.p0 + min(m0 + i * 16 + 4 * lq + rr, M - 1);
    return (size_t)pos * half + t;
  };

  if constexpr (DA == D) {
    // prologue: groups kg0 .. kg0+D-1 requested; group kg0's activations staged
#pragma unroll
    for (int k = 0; k < D; ++k) {
      load_a(ar[k], kg0 + k);
      load_b(br[k], bs[k], kg0 + k);
    }
    if constexpr (kRopePre) {
      const size_t sin_off = (size_t)e.kv.S * (e.kv.hd / 2);
#pragma unroll
      for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const size_t o = rope_at(j, i, rr);
            rcs[j][i][rr][0] = e.rope[o];
            rcs[j][i][rr][1] = e.rope[sin_off + o];
          }
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
  } else {
    // one activation group in registers: group g+1 is requested before group
    // g is computed and written to the other LDS stage right after it
    load_a(ar[0], kg0);
#pragma unroll
    for (int k = 0; k < D; ++k) load_b(br[k], bs[k], kg0 + k);
    store_a(ar[0], 0);
    load_a(ar[0], kg0 + 1);
    lds_barrier();
#pragma unroll 1
    for (int g = kg0; g < kg1; g += D) {
#pragma unroll
      for (int k = 0; k < D; ++k) {
        compute(k & 1, br[k], bs[k], g + k < kg1);         // group g+k from stage k
        store_a(ar[0], (k + 1) & 1);                      // group g+k+1 -> the other stage
        load_a(ar[0], g + k + 2);
        load_b(br[k], bs[k], g + k + D);
        lds_barrier();
      }
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
            float c, sn;
            if constexpr (kRopePre) {
              c = rcs[j][i][rr][0];
              sn = rcs[j][i][rr][1];
            } else {
              c = e.rope[(size_t)pos * half + t];
              sn = e.rope[(size_t)e.kv.S * half + (size_t)pos * half + t];
            }
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
//
// Large M: when even 128 x 128 blocks make at least 512 of them (gate/up from
// M = 641; at M = 1024 704 blocks), 128 x 32 wave tiles (kernel <8, 2>) are
// used: each dequantized weight word then feeds 8 MFMAs and each weight tile
// is read by M/128 row tiles instead of M/32 (gate/up at M = 1024: 73.7 ->
// 68.5 us in the seq-1024 forward pass). With fewer blocks the 2-blocks-per-CU
// tile leaves CUs unevenly loaded: QKV at M = 1024 (384 blocks) measured 47.8
// -> 52.8 us in situ, so it and the O and down projections stay on 32-row
// tiles. K is never split on this path.
//
// From M = 512 the other linears take 64-row tiles (kernel <4, 2>, 64 x 128
// blocks, the large-M code path): half the dequantization per output of the
// 32-row tiles. At M = 1024 (seq-1024 forward, one box, two alternations)
// QKV 47.7 -> 42.5 us, down 42.6 -> 36.9 (now split-K 2), O 18.9 -> 17.6,
// the step 3.58-3.60 -> 3.52-3.54 ms; unsplit O and down on 256 such blocks
// were slower (21, 46 us).
GemmPlan plan_w4_gemm(int N, int K, int M, bool swiglu, bool unsplit, bool folded) {
  const int NB = N / 16, G = (K + 127) / 128;
  GemmPlan p{};
  if ((long long)((NB + 7) / 8) * ((M + 127) / 128) >= 512) {
    p.mb = 8;
    p.nbw = 2;
    p.gx = (NB + 7) / 8;
    p.gy = (M + 127) / 128;
    p.S = 1;
    p.gps = G;
    p.blocks = ((p.gx + 7) / 8) * 8 * p.gy;
    return p;
  }
  auto tiles = [&](int mb) {
    GemmPlan q{};
    q.mb = mb;
    q.gy = (M + 16 * mb - 1) / (16 * mb);
    auto splits = [&](int gx) {
      int S = 1;
      if (!swiglu && !unsplit)
        while (S < kMaxSplitK && gx * q.gy * S < 384 && G / (2 * S) >= 4) S *= 2;
      return S;
    };
    q.nbw = 2;
    q.gx = (NB + 4 * q.nbw - 1) / (4 * q.nbw);
    int S = splits(q.gx);
    if (!swiglu && mb <= 2 && q.gx * q.gy * S < 256) {
      q.nbw = 1;
      q.gx = (NB + 3) / 4;
      S = splits(q.gx);
    }
    q.gps = (G + S - 1) / S;
    q.S = (G + q.gps - 1) / q.gps;
    q.blocks = ((q.gx + 7) / 8) * 8 * q.gy * q.S;
    return q;
  };
  // 64-row tiles from M = 512, unless they would split K for a caller that
  // must sum the partials in a pass of its own (the standalone linear)
  if (M >= 512) {
    const GemmPlan q = tiles(4);
    if (folded || q.S == 1) return q;
  }
  return tiles(M <= 16 ? 1 : 2);
}

size_t w4_gemm_scratch_bytes(int N, int K, int M, bool swiglu, bool folded) {
  const GemmPlan p = plan_w4_gemm(N, K, M, swiglu, false, folded);
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

hipError_t launch_w4_gemm(const Packed& w, const uint16_t* A, int M, const Epi& e, float* part, hipStream_t s,
                          bool folded) {
  if (M < 1) return hipErrorInvalidValue;
  GemmPlan pl = plan_w4_gemm(w.N, w.K, M, e.mode == EPI_SWIGLU, e.mode == EPI_QKV_ROPE, folded);
  if (pl.S > 1 && !part) return hipErrorInvalidValue;
  if (e.mode == EPI_QKV_ROPE) {
    const int d = e.kv.H * e.kv.hd;
    if (e.kv.int8 || e.perm_hd != e.kv.hd || w.N % d || e.sec_base < 0 || e.sec_base + w.N / d > 3)
      return hipErrorInvalidValue;
  }
  pl.part = part;
  if (pl.mb == 8) return gemm_launch<8, 2>(w, A, M, e, pl, s);
  if (pl.mb == 4) return gemm_launch<4, 2>(w, A, M, e, pl, s);
  if (pl.nbw == 2) return pl.mb == 2 ? gemm_launch<2, 2>(w, A, M, e, pl, s) : gemm_launch<1, 2>(w, A, M, e, pl, s);
  return pl.mb == 2 ? gemm_launch<2, 1>(w, A, M, e, pl, s) : gemm_launch<1, 1>(w, A, M, e, pl, s);
}

}  // namespace tl
