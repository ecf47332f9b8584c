// Causal attention over the per-layer KV cache (gfx950).
//
// Cache layout of one (lane, effective layer): K then V, each [H][S][hd]
// fp16; or, in INT8 mode, Kq int8 [H][S][hd], Ks fp16 [H][S], Vq, Vs (one
// FP16 scale per token and head: "Performance and Memory" page, "KV cache
// INT8"), each plane 256-byte aligned (int8_planes). Attention always reads what the cache holds, so an INT8 cache is
// read back as q * s in the prefill too (cached and uncached paths agree).
//
// Prefill: a block takes 64 queries of one head (8 waves: 4 groups of 16
// rows x 2 halves of each key tile; without a sliding window the rows are two
// mirrored 32-row tiles, which evens the causal work of the blocks) and walks
// 128-key tiles up to its causal limit: K and V tiles staged row-major in LDS (V's MFMA fragments read back
// with gfx950's transposing LDS read), S^T = K Q^T and O^T += V^T P^T on
// v_mfma_f32_16x16x32_f16 (the transposed score tile is already in the PV
// MFMA's operand layout, so P stays in registers), online softmax in
// fp32 (running max and sum per query). INT8 codes are exact in fp16, so the
// MFMAs run on the codes and the per-key scales multiply the score columns
// and the probabilities. P enters the PV MFMA as two fp16 parts (high part and
// the rounded remainder), so the weights keep about 22 significant bits.
//
// Decode: one query per lane; see attn_decode_kernel below.
#include <type_traits>

#include "tl_device.h"
#include "tl_kernels.h"

namespace tl {

typedef float float2_t __attribute__((ext_vector_type(2)));

// Workgroups go to the 8 XCDs round-robin by linear index and each XCD has
// its own L2. Renumbering block b of an n-block grid so that the blocks one
// XCD receives are consecutive indices lets a (head, query tile) grid put
// whole heads on one XCD: a head's K/V rows then enter one L2 instead of all
// eight. A bijection on [0, n) for any n.
__device__ __forceinline__ int xcd_contiguous(int b, int n) {
  const int x = b & 7, per = n >> 3, extra = n & 7;
  return x * per + min(x, extra) + (b >> 3);
}

struct CachePtrs {
  const uint8_t* k;   // fp16 [S][hd] or int8 [S][hd] of this head
  const uint8_t* v;
  const uint16_t* ks;  // int8 mode: fp16 scales [S]
  const uint16_t* vs;
};

__device__ __forceinline__ CachePtrs cache_ptrs(const KvGeom& kv, int lane, int layer, int h) {
  const uint8_t* base = kv.base + ((size_t)lane * kv.n_layers + layer) * kv.layer_bytes;
  const size_t HS = (size_t)kv.H * kv.cap;
  CachePtrs c;
  if (kv.int8) {
    const Int8Planes pl = int8_planes(kv.H, kv.cap, kv.hd);
    c.k = base + pl.kq + (size_t)h * kv.cap * kv.hd;
    c.ks = reinterpret_cast<const uint16_t*>(base + pl.ks) + (size_t)h * kv.cap;
    c.v = base + pl.vq + (size_t)h * kv.cap * kv.hd;
    c.vs = reinterpret_cast<const uint16_t*>(base + pl.vs) + (size_t)h * kv.cap;
  } else {
    c.k = base + (size_t)h * kv.cap * kv.hd * 2;
    c.v = base + HS * kv.hd * 2 + (size_t)h * kv.cap * kv.hd * 2;
    c.ks = c.vs = nullptr;
  }
  return c;
}


// ------------------------------------------------------------------ prefill
// gfx950 transposing LDS read (ds_read_b64_tr_b16), in groups of 16 lanes:
// lane 16g + 4a + b receives element b of the 4-element (8-byte) chunks
// addressed by lanes 16g + a, 16g + a + 4, 16g + a + 8 and 16g + a + 12, in
// that order. Two reads (rows r and r + 4) give a lane 8 values of one column.
typedef short short4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ half8_t lds_read_tr16x8(const _Float16* p0, const _Float16* p1) {
  typedef __attribute__((address_space(3))) short4_t lds_short4;
  const short4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p0));
  const short4_t c = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p1));
  const short4_t lo = a, hi = c;
  typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
  const half4_t l4 = __builtin_bit_cast(half4_t, lo), h4 = __builtin_bit_cast(half4_t, hi);
  return (half8_t){l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
}

__device__ __forceinline__ void attn_lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// K/V tile t (keys KT*t .. KT*t + KT-1) is requested into registers while
// tile t-1 is computed (raw: fp16 rows, or INT8 codes and scales, converted
// when written to LDS so the request never waits), then written to LDS as
// 16-byte row chunks, K and V alike. The block barriers wait on LDS only, so the next
// tile's requests stay in flight across them. KT = 128 keys per tile: a
// 128-token call takes one tile per block.
//
// The block's 8 waves are 4 query groups (16 rows each) x 2 key halves: wave
// (g, k) runs the online softmax of rows 16g.. over keys 64k..64k+63 of every
// tile, and at the end the k = 1 wave hands its (max, sum, weighted values)
// to the k = 0 wave through LDS, which merges the two halves and stores the
// rows. Splitting the keys halves each wave's dependent MFMA/softmax chain and
// puts two waves on every SIMD (9.1 -> 8.6 us per layer at 128 tokens, where
// a block sees a single tile; longer calls walk more tiles per wave).
// Blocks per head of the tiled prefill kernel. Without a window (fold) a
// block takes two 32-row query tiles, j and its mirror nq - 1 - j, as query
// groups 0-1 and 2-3: every pair has about the same causal work, so the
// blocks end together instead of the last tile's block walking twice the
// average number of key tiles (a group whose queries all precede a key part
// skips it). With a window a block takes 64 consecutive rows.
__host__ __device__ inline int attn_prefill_blocks(int M, bool fold) {
  return fold ? ((M + 31) / 32 + 1) / 2 : (M + 63) / 64;
}
constexpr int kAttnKT = 128;
constexpr int kAttnKSplit = 2;
constexpr int kAttnThreads = 256 * kAttnKSplit;
template <int HD, bool I8>
__global__ __launch_bounds__(kAttnThreads) void attn_prefill_kernel(const uint16_t* __restrict__ q, int M,
                                                                    int lane_id, int p0, KvGeom kv, int layer,
                                                                    uint16_t* __restrict__ o) {
  constexpr int KT = kAttnKT;     // keys per tile
  constexpr int KH = KT / kAttnKSplit;  // keys per wave and tile
  constexpr int KB = KH / 16;     // 16-key blocks of S
  constexpr int PS = KH / 32;     // k-steps of O += P V
  constexpr int KS = HD / 32;     // k-steps of S = Q K^T
  constexpr int DB = HD / 16;     // 16-wide d blocks of O
  constexpr int LK = HD + 8;      // LDS row stride of the K tile (halves)
  // LDS row stride of the V tile: each 16-lane group of a transposing read
  // covers 4 rows x 16 dims, conflict-free with rows 8 dwords apart mod 64
  constexpr int LV = HD + 16;
  constexpr int CPT = KT * HD / 8 / kAttnThreads;  // 8-element chunks of K (and of V) per thread and tile
  static_assert(KB >= 1 && PS >= 1 && CPT >= 1, "tile shape");
  using Raw = typename std::conditional<I8, uint2, u32x4_t>::type;
  // K tile, then the V tile, both row-major (key rows of HD + 8 halves), in
  // one array (reused by the merge)
  // floats per lane of the key-half merge: m, l, 2 of padding, o[DB][4] (a
  // stride of 4 mod 8 dwords keeps each 16-lane pass of 16-byte accesses on
  // distinct banks); the merge reuses the K/V array
  constexpr int RW = 4 + 4 * DB;
  constexpr int KVH = KT * (LK + LV) > 4 * 64 * RW * 2 ? KT * (LK + LV) : 4 * 64 * RW * 2;
  __shared__ __align__(16) _Float16 KVs[KVH];
  _Float16* const Ks = KVs;
  _Float16* const Vs = KVs + KT * LK;
  __shared__ __align__(16) float ksc[KT];
  __shared__ __align__(16) float vsc[KT];

  const int tid = threadIdx.x, wave = tid >> 6, ln = tid & 63;
  const int qg = wave & 3, kh = wave >> 2;  // query group, key half
  const int l16 = ln & 15, lq = ln >> 4;
  // 1-D grid of H x nqb blocks, head-major per XCD (attn_prefill_blocks).
  // r0: first row of this wave's query group (M: the group has no rows).
  const bool fold = kv.window == 0;
  const int nqb = attn_prefill_blocks(M, fold);
  const int id = xcd_contiguous(blockIdx.x, gridDim.x);
  const int h = id / nqb;
  const int j = id - h * nqb;
  int r0, rlo, rhi;  // rows [rlo, rhi) bound the block's queries
  if (fold) {
    const int nq = (M + 31) / 32, ta = j, tb = nq - 1 - j;
    r0 = qg < 2 ? 32 * ta + 16 * qg : (tb > ta ? 32 * tb + 16 * (qg - 2) : M);
    rlo = 32 * ta;
    rhi = min(32 * max(ta, tb) + 32, M);
  } else {
    rlo = (nqb - 1 - j) * 64;  // the causally longest tile first
    r0 = rlo + 16 * qg;
    rhi = min(rlo + 64, M);
  }
  const int d = kv.H * HD;
  const int kend = p0 + rhi;               // keys [kbeg, kend) can be visible to this block
  const int kbeg = kv_first(kv, p0 + rlo);  // the window of the block's first query
  const CachePtrs cp = cache_ptrs(kv, lane_id, layer, h);
  // scores in log2 units (softmax scale times log2 e folded into the key
  // scales), so every weight is one v_exp_f32: exp(x) = 2^(x log2 e)
  const float scale = 1.4426950408889634f / sqrtf((float)HD);
  const int nkt = (kend + KT - 1) / KT;
  const int kt0 = kbeg / KT;

  Raw kreg[CPT], vreg[CPT];
  uint32_t kscr = 0, vscr = 0;  // raw fp16 scales (INT8), threads < KT
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + kAttnThreads * i;
      const int kr = c / (HD / 8), d0 = (c % (HD / 8)) * 8;
      const int key = min(max(kt * KT + kr, kbeg), kend - 1);
      const size_t roff = (size_t)kv_slot(kv, key) * HD * (I8 ? 1 : 2) + d0 * (I8 ? 1 : 2);
      kreg[i] = *reinterpret_cast<const Raw*>(cp.k + roff);
      vreg[i] = *reinterpret_cast<const Raw*>(cp.v + roff);
    }
    if constexpr (I8) {
      const int key = min(max(kt * KT + (tid & (KT - 1)), kbeg), kend - 1);
      kscr = cp.ks[kv_slot(kv, key)];
      vscr = cp.vs[kv_slot(kv, key)];
    }
  };
  auto to_f16 = [&](const Raw& r) -> half8_t {
    if constexpr (I8) {
      half8_t hv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hv[j] = (_Float16)(float)(int8_t)((r.x >> (8 * j)) & 0xFF);
        hv[4 + j] = (_Float16)(float)(int8_t)((r.y >> (8 * j)) & 0xFF);
      }
      return hv;
    } else {
      return __builtin_bit_cast(half8_t, r);
    }
  };
  // Rows outside [kbeg, kend) hold the clamped edge row, a finite cache row:
  // their scores are masked to -inf, so their weights are exactly 0.
  auto store_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + kAttnThreads * i;
      const int kr = c / (HD / 8), d0 = (c % (HD / 8)) * 8;
      *reinterpret_cast<half8_t*>(&Ks[kr * LK + d0]) = to_f16(kreg[i]);
      *reinterpret_cast<half8_t*>(&Vs[kr * LV + d0]) = to_f16(vreg[i]);
    }
    if constexpr (I8) {  // an FP16 cache takes the softmax scale as a constant
      if (tid < KT) {
        ksc[tid] = h2f((uint16_t)kscr) * scale;
        vsc[tid] = h2f((uint16_t)vscr);
      }
    }
  };

  load_tile(kt0);
  // Q fragments (A operand of S): row r0 + l16, dims 32s + 8lq .. +7
  half8_t qf[KS];
  {
    const int qr = r0 + l16;
    const int qc = min(qr, M - 1);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(q + (size_t)qc * d + h * HD + 32 * s + 8 * lq);
      qf[s] = qr < M ? __builtin_bit_cast(half8_t, v) : (half8_t){0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  // Scores are computed transposed (S^T = K Q^T), so a lane holds 4 keys of
  // one query: lane (lq, n) has query 16*qg + n and keys 16kb + 4lq + r of
  // every 16-key block, which is the B-operand layout O^T = V^T P^T needs;
  // P never leaves registers. Each lane keeps its query's running max and
  // sum (the 4 lanes of a query hold the same values) and O^T: dims
  // 16b + 4lq + r of its query.
  float mrow = -INFINITY, lrow = 0.f;
  float4_t oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) oacc[b] = (float4_t){0.f, 0.f, 0.f, 0.f};
  const int qpos = p0 + r0 + l16;
  const int kfirst = kv_first(kv, qpos);
  // a key part in [kfull0, kfull1] is visible to all 16 queries of the group;
  // one that starts after kvis (or a group without rows) is visible to none
  const int kfull0 = kv_first(kv, p0 + r0 + 15), kfull1 = p0 + r0;
  const int kvis = r0 < M ? p0 + r0 + 15 : -1;

  for (int kt = kt0; kt < nkt; ++kt) {
    const int key0 = kt * KT + kh * KH;  // this wave's keys key0 .. key0 + KH - 1
    store_tile(kt);
    attn_lds_barrier();
    if (kt + 1 < nkt) load_tile(kt + 1);  // the next tile is in flight during this tile's math
    asm volatile("" ::: "memory");
    if (key0 <= kvis) {  // wave-uniform: otherwise the group's state would not change

      // ---- S^T = K Q^T for KH keys x 16 queries (lane: keys 16kb + 4lq + r, query n)
      float sv[KB][4];
      float4_t st[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float4_t t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const half8_t kf = *reinterpret_cast<const half8_t*>(&Ks[(kh * KH + kb * 16 + l16) * LK + 32 * s + 8 * lq]);
          t = mfma16(kf, qf[s], t);
        }
        const float4_t ks = I8 ? *reinterpret_cast<const float4_t*>(&ksc[kh * KH + kb * 16 + 4 * lq])
                               : (float4_t){scale, scale, scale, scale};
        st[kb] = t * ks;
      }
      if (key0 >= kfull0 && key0 + KH - 1 <= kfull1) {  // wave-uniform: no key of the part is masked
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) sv[kb][r] = st[kb][r];
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = key0 + kb * 16 + 4 * lq + r;
            sv[kb][r] = (key <= qpos && key >= kfirst) ? st[kb][r] : -INFINITY;
          }
      }
      // ---- online softmax of the lane's query (its keys are spread over the
      // lanes n, n+16, n+32, n+48)
      {
        float mx = sv[0][0];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sv[kb][r]);
        mx = rows4_max(mx);
        const float mnew = fmaxf(mrow, mx);
        // a query with no visible key so far (a sliding window that starts in a
        // later tile, or a key half beyond the query) keeps mnew = -inf:
        // subtract 0 instead, so its weights are exp(-inf) = 0 rather than NaN
        const float mref = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(mrow - mref);  // 0 while mrow = -inf
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float pr = __builtin_amdgcn_exp2f(sv[kb][r] - mref);
            ps += pr;
            sv[kb][r] = pr;
          }
        ps = rows4_sum(ps);
        lrow = lrow * alpha + ps;
        mrow = mnew;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) oacc[b][r] *= alpha;
      }
      // ---- O^T += V^T P^T over this wave's keys, 32 keys per MFMA. A k-step
      // pairs key blocks 2j and 2j+1: lane (lq, n) holds P^T for keys
      // 32j + 4lq + (0..3) and 32j + 16 + 4lq + (0..3) of query n, and reads V^T
      // for the same 8 keys of dim 16b + n with two transposing reads (lane
      // (lq, n) addressing key row +4lq + n/4 at dims 16b + 4(n%4) .. +3), so
      // both operands enumerate k in the same order. P (value scale folded in)
      // enters as an fp16 high part and the fp16 rounding of the remainder: the
      // two MFMAs apply it with about 22 significant bits instead of 11. (INT8:
      // a weight near 1 is then the fp16 scale itself, held exactly; weights
      // far below it fall into fp16's subnormal range and keep fewer bits, on
      // terms that carry little of O.)
#pragma unroll
      for (int j = 0; j < PS; ++j) {
        half8_t ph, pl;
#pragma unroll
        for (int hblk = 0; hblk < 2; ++hblk) {
          const int kb = 2 * j + hblk;
          const float4_t vs = I8 ? *reinterpret_cast<const float4_t*>(&vsc[kh * KH + kb * 16 + 4 * lq])
                                 : (float4_t){1.f, 1.f, 1.f, 1.f};
#pragma unroll
          for (int r = 0; r < 4; r += 2) {  // pairs: one packed conversion per part
            float2_t x = {sv[kb][r], sv[kb][r + 1]};
            if constexpr (I8) x *= (float2_t){vs[r], vs[r + 1]};
            const half2_t hi = __builtin_convertvector(x, half2_t);
            const half2_t lo = __builtin_convertvector(x - __builtin_convertvector(hi, float2_t), half2_t);
            ph[4 * hblk + r] = hi[0];
            ph[4 * hblk + r + 1] = hi[1];
            pl[4 * hblk + r] = lo[0];
            pl[4 * hblk + r + 1] = lo[1];
          }
        }
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          const _Float16* vp = &Vs[(kh * KH + 32 * j + 4 * lq + (l16 >> 2)) * LV + b * 16 + 4 * (l16 & 3)];
          const half8_t vf = lds_read_tr16x8(vp, vp + 16 * LV);
          oacc[b] = mfma16(vf, ph, oacc[b]);
          oacc[b] = mfma16(vf, pl, oacc[b]);
        }
      }
    }
    attn_lds_barrier();  // every wave is done with this K/V tile before the next is written
  }

  // ---- merge the key halves: wave (g, 1) -> LDS (the K/V tiles are free
  // after the loop's last barrier) -> wave (g, 0), which scales both by
  // exp(m_half - m) and adds them in half order
  static_assert((size_t)4 * 64 * RW * 4 <= sizeof(KVs), "merge buffer");
  float* const mb = reinterpret_cast<float*>(KVs);
  if (kh == 1) {
    float* dst = mb + (size_t)(qg * 64 + ln) * RW;
    dst[0] = mrow;
    dst[1] = lrow;
#pragma unroll
    for (int b = 0; b < DB; ++b) *reinterpret_cast<float4_t*>(dst + 4 + 4 * b) = oacc[b];
  }
  attn_lds_barrier();
  if (kh == 1) return;
  const float* src = mb + (size_t)(qg * 64 + ln) * RW;
  // ---- normalise and store query r0 + n, dims 16b + 4lq .. +3
  const float m2 = src[0], l2 = src[1];
  const float m = fmaxf(mrow, m2);
  const float mref = m == -INFINITY ? 0.f : m;
  const float a1 = __builtin_amdgcn_exp2f(mrow - mref), a2 = __builtin_amdgcn_exp2f(m2 - mref);
  const float inv = 1.0f / (lrow * a1 + l2 * a2);
  const int qr = r0 + l16;
  if (qr >= M) return;
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    const float4_t o2 = *reinterpret_cast<const float4_t*>(src + 4 + 4 * b);
    uint2 w;
    w.x = (uint32_t)f2h((oacc[b][0] * a1 + o2[0] * a2) * inv) | ((uint32_t)f2h((oacc[b][1] * a1 + o2[1] * a2) * inv) << 16);
    w.y = (uint32_t)f2h((oacc[b][2] * a1 + o2[2] * a2) * inv) | ((uint32_t)f2h((oacc[b][3] * a1 + o2[3] * a2) * inv) << 16);
    *reinterpret_cast<uint2*>(o + (size_t)qr * d + h * HD + b * 16 + 4 * lq) = w;
  }
}

// Short calls (M <= kShortMaxM rows: the 128-token benchmark step, chunked
// prefill tails, speculative verification): one block per (16 queries, head),
// so a 128-token call has 128 blocks instead of 32. Its 4 waves take the
// block's visible keys in 32-key chunks round-robin, each with its own online
// softmax, and need no block barrier until the final merge: a wave requests
// its K rows straight from the cache in MFMA A-operand order (key row, 8
// dims per lane), stages its V chunk in its own LDS slot (row-major, read back
// with the transposing LDS read as in the tiled kernel) and keeps P in
// registers; causally invisible chunks are never loaded. The 4 wave states
// are merged in wave order at the end.
constexpr int kShortQ = 16;       // queries per block
constexpr int kShortChunk = 32;   // keys per wave step
constexpr int kShortMaxM = 128;   // and at most 8 chunks (256 keys) visible to the call
template <int HD, bool I8>
__global__ __launch_bounds__(256) void attn_prefill_short_kernel(const uint16_t* __restrict__ q, int M, int lane_id,
                                                                 int p0, KvGeom kv, int layer,
                                                                 uint16_t* __restrict__ o) {
  constexpr int KS = HD / 32;                  // k-steps of S^T = K Q^T
  constexpr int DB = HD / 16;                  // 16-dim blocks of O
  constexpr int LV = HD + 16;                  // LDS row stride of a wave's V chunk (halves)
  constexpr int VCH = kShortChunk * HD / 8 / 64;  // 8-element V chunks per lane and key chunk
  constexpr int RW = 4 + 4 * DB;               // floats per lane in the merge
  static_assert(64 * RW * 4 <= kShortChunk * LV * 2, "merge state fits a wave's V slot");
  using Raw = typename std::conditional<I8, uint2, u32x4_t>::type;
  constexpr int ESZ = I8 ? 1 : 2;              // bytes per cached element
  __shared__ __align__(16) _Float16 Vw[4][kShortChunk * LV];

  const int tid = threadIdx.x, wave = tid >> 6, ln = tid & 63;
  const int l16 = ln & 15, lq = ln >> 4;
  const int nq = (M + kShortQ - 1) / kShortQ;  // 1-D grid of H x nq blocks, as in the tiled kernel
  const int id = xcd_contiguous(blockIdx.x, gridDim.x);
  const int h = id / nq;
  const int q0 = (nq - 1 - (id - h * nq)) * kShortQ;
  const int d = kv.H * HD;
  const int kend = p0 + min(q0 + kShortQ, M);  // keys [kbeg, kend) can be visible to this block
  const int kbeg = kv_first(kv, p0 + q0);
  const CachePtrs cp = cache_ptrs(kv, lane_id, layer, h);
  const float scale = 1.4426950408889634f / sqrtf((float)HD);  // log2 units: weights are 2^x
  const int nch = (kend - kbeg + kShortChunk - 1) / kShortChunk;

  // Q fragments (B operand): query q0 + l16, dims 32s + 8lq .. +7
  half8_t qf[KS];
  {
    const int qr = q0 + l16, qc = min(qr, M - 1);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(q + (size_t)qc * d + h * HD + 32 * s + 8 * lq);
      qf[s] = qr < M ? __builtin_bit_cast(half8_t, v) : (half8_t){0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  const int qpos = p0 + q0 + l16;
  const int kfirst = kv_first(kv, qpos);
  auto to_f16 = [&](const Raw& r) -> half8_t {
    if constexpr (I8) {
      half8_t hv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hv[j] = (_Float16)(float)(int8_t)((r.x >> (8 * j)) & 0xFF);
        hv[4 + j] = (_Float16)(float)(int8_t)((r.y >> (8 * j)) & 0xFF);
      }
      return hv;
    } else {
      return __builtin_bit_cast(half8_t, r);
    }
  };

  float mrow = -INFINITY, lrow = 0.f;
  float4_t oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) oacc[b] = (float4_t){0.f, 0.f, 0.f, 0.f};
  _Float16* const vw = Vw[wave];

  for (int c = wave; c < nch; c += 4) {
    const int key0 = kbeg + c * kShortChunk;  // this chunk: keys key0 .. key0 + 31
    // ---- requests: K fragments (key row key0 + 16kb + l16, dims 32s + 8lq ..),
    // V rows (linear chunk e = ln + 64i: key e / (HD/8), dims 8 (e % (HD/8)) ..),
    // INT8 scales of the keys this lane scores (16kb + 4lq + r)
    Raw kr[2][KS], vr[VCH];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const size_t row = (size_t)kv_slot(kv, min(key0 + 16 * kb + l16, kend - 1)) * HD * ESZ;
#pragma unroll
      for (int s = 0; s < KS; ++s) kr[kb][s] = *reinterpret_cast<const Raw*>(cp.k + row + (32 * s + 8 * lq) * ESZ);
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int e = ln + 64 * i, r = e / (HD / 8), d0 = (e % (HD / 8)) * 8;
      vr[i] = *reinterpret_cast<const Raw*>(cp.v + (size_t)kv_slot(kv, min(key0 + r, kend - 1)) * HD * ESZ + d0 * ESZ);
    }
    uint32_t ksr[I8 ? 8 : 1], vsr[I8 ? 8 : 1];
    if constexpr (I8) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int slot = kv_slot(kv, min(key0 + 16 * kb + 4 * lq + r, kend - 1));
          ksr[4 * kb + r] = cp.ks[slot];
          vsr[4 * kb + r] = cp.vs[slot];
        }
    }
    // ---- the V chunk into this wave's LDS slot (fp16; INT8 codes are exact in fp16)
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int e = ln + 64 * i, r = e / (HD / 8), d0 = (e % (HD / 8)) * 8;
      *reinterpret_cast<half8_t*>(&vw[r * LV + d0]) = to_f16(vr[i]);
    }
    // ---- S^T = K Q^T (lane: keys 16kb + 4lq + r of query l16)
    float sv[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float4_t t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) t = mfma16(to_f16(kr[kb][s]), qf[s], t);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = key0 + 16 * kb + 4 * lq + r;
        float ks = scale;
        if constexpr (I8) ks *= h2f((uint16_t)ksr[4 * kb + r]);
        sv[kb][r] = (key < kend && key <= qpos && key >= kfirst) ? t[r] * ks : -INFINITY;
      }
    }
    // ---- online softmax of the lane's query (its 32 keys are spread over the
    // lanes n, n+16, n+32, n+48)
    {
      float mx = sv[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sv[kb][r]);
      mx = rows4_max(mx);
      const float mnew = fmaxf(mrow, mx);
      // no visible key so far (a window starting later, or keys beyond the
      // query): subtract 0, so the weights are exp(-inf) = 0, not NaN
      const float mref = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = __builtin_amdgcn_exp2f(mrow - mref);
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pr = __builtin_amdgcn_exp2f(sv[kb][r] - mref);
          ps += pr;
          sv[kb][r] = pr;
        }
      ps = rows4_sum(ps);
      lrow = lrow * alpha + ps;
      mrow = mnew;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[b][r] *= alpha;
    }
    // ---- O^T += V^T P^T over the chunk's 32 keys (one k-step; P in two fp16
    // parts, value scales folded in), V^T from this wave's slot
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's V writes land before its reads
    {
      half8_t ph, pl;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {  // pairs: one packed conversion per part
          float2_t x = {sv[kb][r], sv[kb][r + 1]};
          if constexpr (I8) x *= (float2_t){h2f((uint16_t)vsr[4 * kb + r]), h2f((uint16_t)vsr[4 * kb + r + 1])};
          const half2_t hi = __builtin_convertvector(x, half2_t);
          const half2_t lo = __builtin_convertvector(x - __builtin_convertvector(hi, float2_t), half2_t);
          ph[4 * kb + r] = hi[0];
          ph[4 * kb + r + 1] = hi[1];
          pl[4 * kb + r] = lo[0];
          pl[4 * kb + r + 1] = lo[1];
        }
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const _Float16* vp = &vw[(4 * lq + (l16 >> 2)) * LV + b * 16 + 4 * (l16 & 3)];
        const half8_t vf = lds_read_tr16x8(vp, vp + 16 * LV);
        oacc[b] = mfma16(vf, ph, oacc[b]);
        oacc[b] = mfma16(vf, pl, oacc[b]);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next chunk's writes
  }

  // ---- merge the 4 waves' states in wave order (waves 1..3 through their own
  // LDS slot), normalise and store query q0 + l16, dims 16b + 4lq .. +3
  if (wave > 0) {
    float* dst = reinterpret_cast<float*>(vw) + ln * RW;
    dst[0] = mrow;
    dst[1] = lrow;
#pragma unroll
    for (int b = 0; b < DB; ++b) *reinterpret_cast<float4_t*>(dst + 4 + 4 * b) = oacc[b];
  }
  attn_lds_barrier();
  if (wave > 0) return;
  float mw[4], lw[4];
  mw[0] = mrow;
  lw[0] = lrow;
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    const float* src = reinterpret_cast<const float*>(Vw[w]) + ln * RW;
    mw[w] = src[0];
    lw[w] = src[1];
  }
  float m = mw[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) m = fmaxf(m, mw[w]);
  const float mref = m == -INFINITY ? 0.f : m;
  float a[4], den = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    a[w] = __builtin_amdgcn_exp2f(mw[w] - mref);
    den += lw[w] * a[w];
  }
  const float inv = 1.0f / den;
  const int qr = q0 + l16;
  if (qr >= M) return;
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    float4_t acc = oacc[b] * a[0];
#pragma unroll
    for (int w = 1; w < 4; ++w)
      acc += *reinterpret_cast<const float4_t*>(reinterpret_cast<const float*>(Vw[w]) + ln * RW + 4 + 4 * b) * a[w];
    uint2 wv;
    wv.x = (uint32_t)f2h(acc[0] * inv) | ((uint32_t)f2h(acc[1] * inv) << 16);
    wv.y = (uint32_t)f2h(acc[2] * inv) | ((uint32_t)f2h(acc[3] * inv) << 16);
    *reinterpret_cast<uint2*>(o + (size_t)qr * d + h * HD + b * 16 + 4 * lq) = wv;
  }
}

hipError_t launch_attn_prefill(const uint16_t* q, int M, int lane, int p0, const KvGeom& kv, int layer,
                               uint16_t* o, hipStream_t s) {
  // short calls over a short visible span (each wave walks at most 2 chunks;
  // a long context reached by a short call is better served by the tiled
  // kernel, which requests the next key tile during the current one)
  if (M <= kShortMaxM && p0 + M - kv_first(kv, p0) <= 8 * kShortChunk) {
    const dim3 g((M + kShortQ - 1) / kShortQ * kv.H);
    if (kv.hd == 128 && kv.int8)
      launch(attn_prefill_short_kernel<128, true>, g, dim3(256), 0, s, q, M, lane, p0, kv, layer, o);
    else if (kv.hd == 128)
      launch(attn_prefill_short_kernel<128, false>, g, dim3(256), 0, s, q, M, lane, p0, kv, layer, o);
    else if (kv.hd == 64 && kv.int8)
      launch(attn_prefill_short_kernel<64, true>, g, dim3(256), 0, s, q, M, lane, p0, kv, layer, o);
    else if (kv.hd == 64)
      launch(attn_prefill_short_kernel<64, false>, g, dim3(256), 0, s, q, M, lane, p0, kv, layer, o);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  const dim3 grid(attn_prefill_blocks(M, kv.window == 0) * kv.H);
  if (kv.hd == 128 && kv.int8)
    launch(attn_prefill_kernel<128, true>, grid, dim3(kAttnThreads), 0, s, q, M, lane, p0, kv, layer, o);
  else if (kv.hd == 128)
    launch(attn_prefill_kernel<128, false>, grid, dim3(kAttnThreads), 0, s, q, M, lane, p0, kv, layer, o);
  else if (kv.hd == 64 && kv.int8)
    launch(attn_prefill_kernel<64, true>, grid, dim3(kAttnThreads), 0, s, q, M, lane, p0, kv, layer, o);
  else if (kv.hd == 64)
    launch(attn_prefill_kernel<64, false>, grid, dim3(kAttnThreads), 0, s, q, M, lane, p0, kv, layer, o);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ------------------------------------------------------------------ decode
// A block of BW waves (4 or 8) covers BW * 32 keys of the visible context of
// one row's lane for one head; wave w takes the 32-key chunk
// BW*blockIdx.x + w (4 waves of 32 keys measured 4.5 us per layer at context
// 256-384 against 5.4 us for 2 waves of 64; smaller parts shorten the
// attention further but cost the O projection more to merge). Lanes are 16
// per key (8 dims each) x 4 keys per pass (HD 128). Order of work, so that no
// wait covers the cache reads:
//   1. the row's q, k, v projections for this lane's 8 dims (and their RoPE
//      partners) and the cos/sin of position pos;
//   2. every K and V row of the chunk (positions < pos; addresses clamped,
//      values outside the context replaced by zeros);
//   3. Q = fp16(RoPE(q)); the wave whose chunk holds pos also rotates/rounds
//      (INT8: quantizes) the new K and V, stores them in the cache and scores
//      that key from registers; scores, softmax, P V.
// The waves of each part merge in LDS in wave order and the block writes each
// part's softmax state (a part beyond the row's context: max = -inf, sum 0);
// the parts are combined in part order either by attn_merge_kernel or inside
// the O-projection GEMV.
constexpr int kDecChunk = 32;
constexpr int kDecPart = kDecChunk * 4;  // keys of the smallest part (4 waves)

// Waves per part of a row with `ctx` visible keys: parts of 128 keys up to
// context 1024, 256 beyond, so a row has at most 8 parts to context 2048.
// The O-projection GEMV merges every part of the call's rows in each of its
// blocks, so fewer parts make it cheaper, while larger parts leave fewer
// blocks to the attention (measured at context 1920-2048, INT8 cache, one
// lane: 16 parts of 128 keys 0.333 ms/token, 8 of 256 keys 0.324, 4 of 512
// keys (16-wave blocks) 0.376). The split depends on the row's own context
// only, so a lane's result does not depend on the other rows of the call.
__host__ __device__ inline int dec_part_waves(int ctx) { return ctx <= 1024 ? 4 : 8; }

size_t attn_decode_scratch_floats(int max_rows, int H, int hd, int S) {
  const int np = (S + kDecPart - 1) / kDecPart;
  return (size_t)max_rows * H * np * (hd + kAttnPartExtra);
}

int attn_decode_np_max(int S) { return (S + kDecPart - 1) / kDecPart; }

int attn_decode_parts(int M, const RowMap& rm, const KvGeom& kv) {
  int np = 0;
  for (int m = 0; m < M; ++m) {
    const int ctx = rm.row_pos[m] + 1 - kv_first(kv, rm.row_pos[m]);
    const int pk = kDecChunk * dec_part_waves(ctx);
    np = max(np, (ctx + pk - 1) / pk);
  }
  return np;
}

void attn_decode_shape(int M, const RowMap& rm, const KvGeom& kv, int* out) {
  int maxctx = 1, bw = 4;
  for (int m = 0; m < M; ++m) {
    const int ctx = rm.row_pos[m] + 1 - kv_first(kv, rm.row_pos[m]);
    const int w = dec_part_waves(ctx);
    maxctx = max(maxctx, ctx);
    bw = max(bw, w);
    out[3 + 2 * m] = w;
    out[4 + 2 * m] = (ctx + kDecChunk * w - 1) / (kDecChunk * w);
  }
  out[0] = bw;
  out[1] = (maxctx + bw * kDecChunk - 1) / (bw * kDecChunk);
  out[2] = attn_decode_parts(M, rm, kv);
}

// BW waves per block (the largest part of the call's rows): a block covers
// BW * 32 keys and writes BW / W parts of a row whose parts have W waves.
template <int HD, bool I8, int BW>
__global__ __launch_bounds__(BW * 64) void attn_decode_kernel(const float* __restrict__ qkv, RowMap rm,
                                                              const float* __restrict__ rope_cs, KvGeom kv,
                                                              int layer, float* __restrict__ part, int np_max) {
  constexpr int LPK = HD / 8;    // lanes per key
  constexpr int KPP = 64 / LPK;  // keys per pass
  constexpr int NP = kDecChunk / KPP;
  constexpr int HALF = HD / 2;
  __shared__ float red_o[BW][64 / (HD / 8)][HD];  // per wave and key row of a pass
  __shared__ float red_m[BW], red_l[BW];
  const int bp = blockIdx.x, h = blockIdx.y, m = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, ln = tid & 63;
  const int sub = ln % LPK, kg = ln / LPK, d0 = sub * 8;
  const int d = kv.H * HD;
  // ---- 1. projections of this row (8 dims + their RoPE partners): they do
  // not depend on the position, so they are requested before it is known (a
  // graph-replayed step reads the position from device memory)
  const bool lo = d0 < HALF;
  const int i0 = lo ? d0 : d0 - HALF;  // pair index of the first dim
  const float* row = qkv + (size_t)m * 3 * d;
  const float4_t* q1p = reinterpret_cast<const float4_t*>(row + h * HD + i0);
  const float4_t* q2p = reinterpret_cast<const float4_t*>(row + h * HD + i0 + HALF);
  const float4_t* k1p = reinterpret_cast<const float4_t*>(row + d + h * HD + i0);
  const float4_t* k2p = reinterpret_cast<const float4_t*>(row + d + h * HD + i0 + HALF);
  const float4_t* vp = reinterpret_cast<const float4_t*>(row + 2 * d + h * HD + d0);
  float4_t q1[2] = {q1p[0], q1p[1]}, q2[2] = {q2p[0], q2p[1]};
  float4_t k1[2] = {k1p[0], k1p[1]}, k2[2] = {k2p[0], k2p[1]};
  float4_t vv[2] = {vp[0], vp[1]};
  const int pos = rm.dpos ? rm.dpos[rm.row_lane[m]] : rm.row_pos[m];
  const int kbeg = kv_first(kv, pos);  // keys kbeg .. pos are visible
  const int ctx = pos + 1 - kbeg;
  const int W = BW == 4 ? 4 : dec_part_waves(ctx), ppb = BW / W;  // waves per part, parts per block
  const int nparts = (ctx + kDecChunk * W - 1) / (kDecChunk * W);
  const int pb0 = bp * ppb;  // this block's first part
  if (pb0 >= nparts) {  // beyond this row's context: empty parts
    if ((int)threadIdx.x < ppb && pb0 + (int)threadIdx.x < np_max) {
      float* dst = part + ((size_t)(m * kv.H + h) * np_max + pb0 + threadIdx.x) * (HD + kAttnPartExtra);
      dst[HD] = -INFINITY;
      dst[HD + 1] = 0.f;
    }
    return;
  }
  const int lane_id = rm.row_lane[m];
  const CachePtrs cp = cache_ptrs(kv, lane_id, layer, h);
  const int rowb = I8 ? HD : 2 * HD;
  const int k0 = kbeg + (bp * BW + wave) * kDecChunk;
  const bool active = k0 <= pos;
  // cos/sin of the position
  const float4_t* cp4 = reinterpret_cast<const float4_t*>(rope_cs + (size_t)pos * HALF + i0);
  const float4_t* sp4 = reinterpret_cast<const float4_t*>(rope_cs + (size_t)kv.S * HALF + (size_t)pos * HALF + i0);
  float4_t cs[2] = {cp4[0], cp4[1]}, sn[2] = {sp4[0], sp4[1]};

  // ---- 2. the chunk's cached keys and values (positions < pos)
  using Row = typename std::conditional<I8, uint2, u32x4_t>::type;
  Row kr[NP], vr[NP];
  uint32_t ksr[I8 ? NP : 1], vsr[I8 ? NP : 1];  // raw fp16 scales
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int key = kv_slot(kv, max(min(k0 + p * KPP + kg, pos - 1), kbeg));
    kr[p] = *reinterpret_cast<const Row*>(cp.k + (size_t)key * rowb + d0 * (I8 ? 1 : 2));
    vr[p] = *reinterpret_cast<const Row*>(cp.v + (size_t)key * rowb + d0 * (I8 ? 1 : 2));
    if constexpr (I8) {
      ksr[p] = cp.ks[key];
      vsr[p] = cp.vs[key];
    }
  }
  asm volatile("" ::: "memory");
#pragma unroll
  for (int i = 0; i < 2; ++i)
    asm volatile("" : "+v"(q1[i]), "+v"(q2[i]), "+v"(k1[i]), "+v"(k2[i]), "+v"(vv[i]), "+v"(cs[i]), "+v"(sn[i]));

  // ---- 3. Q = fp16(RoPE(q)) for dims d0..d0+7 (pair partner is dim +-HALF)
  float qv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    _Float16 r1, r2;
    rope_pair(q1[j >> 2][j & 3], q2[j >> 2][j & 3], cs[j >> 2][j & 3], sn[j >> 2][j & 3], &r1, &r2);
    qv[j] = (float)(lo ? r1 : r2);
  }
  // ---- the new key/value (only the chunk that holds pos)
  const bool own = (pos >= k0) && (pos < k0 + kDecChunk);
  float kn[8], vn[8], ksn = 1.f, vsn = 1.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) kn[j] = vn[j] = 0.f;
  if (own) {
    _Float16 kf[8], vf[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      _Float16 r1, r2;
      rope_pair(k1[j >> 2][j & 3], k2[j >> 2][j & 3], cs[j >> 2][j & 3], sn[j >> 2][j & 3], &r1, &r2);
      kf[j] = lo ? r1 : r2;
      vf[j] = (_Float16)vv[j >> 2][j & 3];
    }
    const bool writer = (kg == 0);
    if constexpr (I8) {
      float ka = 0.f, va = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        ka = fmaxf(ka, fabsf((float)kf[j]));
        va = fmaxf(va, fabsf((float)vf[j]));
      }
      ka = lanes_max<LPK>(ka);
      va = lanes_max<LPK>(va);
      const _Float16 s16k = kv_scale(ka), s16v = kv_scale(va);
      ksn = (float)s16k;
      vsn = (float)s16v;
      uint32_t kw[2] = {0, 0}, vw[2] = {0, 0};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int qk = kv_code((float)kf[j], ksn), qvv = kv_code((float)vf[j], vsn);
        kn[j] = (float)qk;
        vn[j] = (float)qvv;
        kw[j >> 2] |= ((uint32_t)(qk & 0xFF)) << (8 * (j & 3));
        vw[j >> 2] |= ((uint32_t)(qvv & 0xFF)) << (8 * (j & 3));
      }
      if (writer) {
        const int ps = kv_slot(kv, pos);
        uint8_t* K = const_cast<uint8_t*>(cp.k) + (size_t)ps * rowb + d0;
        uint8_t* V = const_cast<uint8_t*>(cp.v) + (size_t)ps * rowb + d0;
        *reinterpret_cast<uint2*>(K) = make_uint2(kw[0], kw[1]);
        *reinterpret_cast<uint2*>(V) = make_uint2(vw[0], vw[1]);
        if (sub == 0) {
          const_cast<uint16_t*>(cp.ks)[ps] = __builtin_bit_cast(uint16_t, s16k);
          const_cast<uint16_t*>(cp.vs)[ps] = __builtin_bit_cast(uint16_t, s16v);
        }
      }
    } else {
      half8_t kh8, vh8;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        kh8[j] = kf[j];
        vh8[j] = vf[j];
        kn[j] = (float)kf[j];
        vn[j] = (float)vf[j];
      }
      if (writer) {
        const int ps = kv_slot(kv, pos);
        *reinterpret_cast<half8_t*>(const_cast<uint8_t*>(cp.k) + (size_t)ps * rowb + d0 * 2) = kh8;
        *reinterpret_cast<half8_t*>(const_cast<uint8_t*>(cp.v) + (size_t)ps * rowb + d0 * 2) = vh8;
      }
    }
  }

  // ---- scores, chunk max
  const float scale = 1.4426950408889634f / sqrtf((float)HD);  // log2 units: weights are 2^x
  float sc[NP];
  float mx = -INFINITY;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int key = k0 + p * KPP + kg;
    float t = 0.f, tn = 0.f;
    if constexpr (I8) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t w = j < 4 ? kr[p].x : kr[p].y;
        t = fmaf(qv[j], (float)(int8_t)((w >> (8 * (j & 3))) & 0xFF), t);
      }
    } else {
      const half8_t kh8 = __builtin_bit_cast(half8_t, kr[p]);
#pragma unroll
      for (int j = 0; j < 8; ++j) t = fmaf(qv[j], (float)kh8[j], t);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) tn = fmaf(qv[j], kn[j], tn);
    t = key < pos ? t : (key == pos ? tn : 0.f);
    t = lanes_sum<LPK>(t);
    float kscale = ksn;
    if constexpr (I8) kscale = key < pos ? h2f((uint16_t)ksr[p]) : ksn;
    sc[p] = key <= pos ? t * scale * kscale : -INFINITY;
    mx = fmaxf(mx, sc[p]);
  }
  mx = wave_max(mx);  // -inf only for a wave whose chunk starts after pos
  float lsum = 0.f, ov[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) ov[j] = 0.f;
  if (active) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int key = k0 + p * KPP + kg;
      const float pr = key <= pos ? __builtin_amdgcn_exp2f(sc[p] - mx) : 0.f;
      if (sub == 0) lsum += pr;
      float vrow[8];
      if constexpr (I8) {
        const float vsc = h2f((uint16_t)vsr[p]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t w = j < 4 ? vr[p].x : vr[p].y;
          vrow[j] = (float)(int8_t)((w >> (8 * (j & 3))) & 0xFF) * vsc;
        }
      } else {
        const half8_t vh8 = __builtin_bit_cast(half8_t, vr[p]);
#pragma unroll
        for (int j = 0; j < 8; ++j) vrow[j] = (float)vh8[j];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float vj = key < pos ? vrow[j] : (key == pos ? vn[j] * vsn : 0.f);
        ov[j] = fmaf(pr, vj, ov[j]);
      }
    }
  }
  lsum = wave_sum(lsum);
#pragma unroll
  for (int j = 0; j < 8; ++j) red_o[wave][kg][d0 + j] = ov[j];
  if (ln == 0) {
    red_m[wave] = mx;
    red_l[wave] = lsum;
  }
  __syncthreads();
  // ---- each part merges its W waves in wave order (a part whose waves all
  // lie beyond the context comes out empty: max -inf, sum 0)
  for (int j = 0; j < ppb && pb0 + j < np_max; ++j) {
    float* dst = part + ((size_t)(m * kv.H + h) * np_max + pb0 + j) * (HD + kAttnPartExtra);
    float bm = -INFINITY;
#pragma unroll
    for (int w = j * W; w < (j + 1) * W; ++w) bm = fmaxf(bm, red_m[w]);
    if (tid < HD) {
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int w = j * W; w < (j + 1) * W; ++w) {
        if (red_m[w] == -INFINITY) continue;  // chunk beyond the context
        const float sw = __builtin_amdgcn_exp2f(red_m[w] - bm);
        float o = red_o[w][0][tid];
#pragma unroll
        for (int g = 1; g < KPP; ++g) o += red_o[w][g][tid];  // key rows in order
        num = fmaf(sw, o, num);
        den = fmaf(sw, red_l[w], den);
      }
      dst[tid] = num;
      if (tid == 0) {
        dst[HD] = bm;
        dst[HD + 1] = den;
      }
    }
  }
}

// Combine the np parts of every (row, head) in part order into fp16 O.
template <int HD>
__global__ __launch_bounds__(HD) void attn_merge_kernel(const float* __restrict__ part, int H, int np, int np_max,
                                                        uint16_t* __restrict__ o) {
  const int h = blockIdx.x, m = blockIdx.y;
  const float* base = part + (size_t)(m * H + h) * np_max * (HD + kAttnPartExtra);
  float gm = -INFINITY;
  for (int q = 0; q < np; ++q) gm = fmaxf(gm, base[(size_t)q * (HD + kAttnPartExtra) + HD]);
  const int i = threadIdx.x;
  float num = 0.f, den = 0.f;
  for (int q = 0; q < np; ++q) {
    const float* pq = base + (size_t)q * (HD + kAttnPartExtra);
    attn_merge_step(gm, pq[HD], pq[HD + 1], pq[i], num, den);
  }
  o[(size_t)m * H * HD + h * HD + i] = f2h(num / den);
}

template <int HD, bool I8, int BW>
static void decode_launch_bw(int M, const float* qkv, const RowMap& rm, const float* rope_cs, const KvGeom& kv,
                             int layer, float* part, int np_max, int maxctx, int nparts, hipStream_t s) {
  // Enough blocks for the longest context, and for every row to write its
  // first `nparts` parts (the merge reads that many of each row; a row with
  // W = BW writes one part per block).
  const dim3 grid(max((maxctx + BW * kDecChunk - 1) / (BW * kDecChunk), nparts), kv.H, M);
  launch((attn_decode_kernel<HD, I8, BW>), grid, dim3(BW * 64), 0, s, qkv, rm, rope_cs, kv, layer, part, np_max);
}

template <int HD, bool I8>
static void decode_launch(int M, const float* qkv, const RowMap& rm, const float* rope_cs, const KvGeom& kv,
                          int layer, float* part, int np_max, uint16_t* o, hipStream_t s) {
  int maxctx = 1, bw = 4;
  for (int m = 0; m < M; ++m) {
    const int ctx = rm.row_pos[m] + 1 - kv_first(kv, rm.row_pos[m]);
    maxctx = max(maxctx, ctx);
    bw = max(bw, dec_part_waves(ctx));
  }
  const int nparts = attn_decode_parts(M, rm, kv);
  if (bw == 4)
    decode_launch_bw<HD, I8, 4>(M, qkv, rm, rope_cs, kv, layer, part, np_max, maxctx, nparts, s);
  else
    decode_launch_bw<HD, I8, 8>(M, qkv, rm, rope_cs, kv, layer, part, np_max, maxctx, nparts, s);
  if (o) launch(attn_merge_kernel<HD>, dim3(kv.H, M), dim3(HD), 0, s, part, kv.H, nparts, np_max, o);
}

hipError_t launch_attn_decode(const float* qkv, int M, const RowMap& rm, const float* rope_cs, const KvGeom& kv,
                              int layer, float* part, uint16_t* o, hipStream_t s) {
  const int np_max = attn_decode_np_max(kv.S);
  if (attn_decode_parts(M, rm, kv) > np_max) return hipErrorInvalidValue;
  if (kv.hd == 128 && kv.int8)
    decode_launch<128, true>(M, qkv, rm, rope_cs, kv, layer, part, np_max, o, s);
  else if (kv.hd == 128)
    decode_launch<128, false>(M, qkv, rm, rope_cs, kv, layer, part, np_max, o, s);
  else if (kv.hd == 64 && kv.int8)
    decode_launch<64, true>(M, qkv, rm, rope_cs, kv, layer, part, np_max, o, s);
  else if (kv.hd == 64)
    decode_launch<64, false>(M, qkv, rm, rope_cs, kv, layer, part, np_max, o, s);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tl
