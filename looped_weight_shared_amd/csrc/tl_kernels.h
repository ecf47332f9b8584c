// Host-side launchers of the gfx950 kernels (internal to libtl).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tl {

// Kernel timing. While a timing window is open on the calling thread, every
// launch takes the next event pair and attaches it to its own dispatch
// (hipExtLaunchKernel), so the pair measures that kernel alone, under the
// kind the caller set.
struct LaunchTimer {
  hipEvent_t* ev = nullptr;  // 2 per launch
  int* kind = nullptr;
  int cap = 0, used = 0, cur_kind = 0;
};
extern thread_local LaunchTimer* t_launch_timer;

template <typename F, typename... Args>
inline void launch(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t s, Args... args) {
  LaunchTimer* t = t_launch_timer;
  if (t && t->used < t->cap) {
    const int i = t->used++;
    t->kind[i] = t->cur_kind;
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, t->ev[2 * i], t->ev[2 * i + 1], 0u, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
  }
}

// A linear in the packed layout: tiles [N/16][G][64 lanes][16 B], then
// scales fp16 [N/16][G][16]. G = ceil(K / 128).
struct Packed {
  const uint8_t* tiles;
  const uint16_t* scales;  // W4 only
  int N, K, G;
  int f16 = 0;  // 1: dense fp16 tiles (4 KiB per 16 rows x 128 columns), no scales
};

inline size_t packed_tile_bytes(int N, int K) { return (size_t)(N / 16) * ((K + 127) / 128) * 1024; }
inline size_t packed_scale_bytes(int N, int K) { return (size_t)(N / 16) * ((K + 127) / 128) * 32; }
inline size_t packed_bytes(int N, int K) { return packed_tile_bytes(N, K) + packed_scale_bytes(N, K); }
// FP16 head in MFMA tile order (see launch_pack_head).
inline size_t head_packed_bytes(int V, int d) { return (size_t)((V + 15) / 16) * (d / 32) * 1024; }
hipError_t launch_pack_head(const uint16_t* head, int V, int d, uint8_t* dst, hipStream_t s);

// Repack a canonical [N][K/8] / [N][ceil(K/128)] linear into the packed
// buffer of a (possibly fused) destination: source n-block b goes to
// destination n-block nb_offset + b * nb_stride. perm_hd > 0 (a multiple of
// 16) stores the rows of every perm_hd-row head in RoPE-pair order
// (qkv_natural_col): each n-block then holds 8 rotation pairs, the first
// halves in its rows 0..7 and the second halves in rows 8..15.
hipError_t launch_pack(const uint32_t* qweight, const uint16_t* scales, int N, int K, uint8_t* dst_tiles,
                       uint16_t* dst_scales, int dst_G, int nb_offset, int nb_stride, int perm_hd, hipStream_t s);
hipError_t launch_unpack(const Packed& p, int8_t* q, uint16_t* scales, hipStream_t s);
// FP16 body: the same canonical linear dequantized to fp16(q * s) (one
// rounding of the exact product) in the MFMA B-operand order of the W4 tile
// (slot s of lane l = word s of the W4 slot), 4 KiB per 16-row x 128-column
// tile laid out [s][lane][16 B]; same n-block placement and row order options.
inline size_t packed_f16_bytes(int N, int K) { return (size_t)(N / 16) * ((K + 127) / 128) * 4096; }
hipError_t launch_pack_f16(const uint32_t* qweight, const uint16_t* scales, int N, int K, uint8_t* dst_tiles, int dst_G,
                           int nb_offset, int nb_stride, int perm_hd, hipStream_t s);

struct KvGeom {
  uint8_t* base;        // start of all caches
  size_t layer_bytes;   // one lane, one layer
  int n_layers;         // layers per lane
  int H, hd, S;         // heads, head_dim, max_seq (positions; RoPE table rows)
  int int8;
  int cap;              // cache rows per (lane, layer, head): S, or the window's ring
  int window;           // 0: full cache; W: queries see the last W positions
};
// INT8 cache of one (lane, layer): K codes int8 [H][cap][hd], K scales fp16
// [H][cap], V codes, V scales, each plane starting on a 256-byte boundary so
// that every 8- and 16-byte access to a code row stays aligned whatever
// H * cap is. (At H * cap a multiple of 128 there is no padding.)
struct Int8Planes {
  size_t kq, ks, vq, vs, bytes;
};
__host__ __device__ inline size_t kv_al256(size_t x) { return (x + 255) & ~(size_t)255; }
__host__ __device__ inline Int8Planes int8_planes(int H, int cap, int hd) {
  const size_t codes = kv_al256((size_t)H * cap * hd), scales = kv_al256((size_t)H * cap * 2);
  Int8Planes p;
  p.kq = 0;
  p.ks = codes;
  p.vq = codes + scales;
  p.vs = 2 * codes + scales;
  p.bytes = 2 * (codes + scales);
  return p;
}

// One layer of an INT8 store-h cache (TL_KV_H8): codes int8 [S][d] at 0, then
// the fp16 scale of each 128-element group, [S][d / 128], both planes
// 256-byte aligned.
struct H8Planes {
  size_t hs, bytes;
};
__host__ __device__ inline H8Planes h8_planes(int S, int d) {
  H8Planes p;
  p.hs = kv_al256((size_t)S * d);
  p.bytes = p.hs + kv_al256((size_t)S * (d / 128) * 2);
  return p;
}

// Cache row of position pos (a ring when windowed) and the first position
// a query at pos sees.
__host__ __device__ inline int kv_slot(const KvGeom& kv, int pos) { return kv.window ? pos % kv.cap : pos; }
__host__ __device__ inline int kv_first(const KvGeom& kv, int pos) {
  return kv.window ? (pos - kv.window + 1 > 0 ? pos - kv.window + 1 : 0) : 0;
}

// Epilogue of the W4 matrix kernels.
//   STORE / RESID: fp32 out[m*ldo + n] = / += v;
//   SWIGLU: fp16 out[m*ldo + c] = silu(gate) * up (gate/up n-blocks paired);
//   QKV_ROPE (GEMM, K never split, FP16 cache, one lane's rows at p0 + m):
//     the columns of a RoPE-pair packed QKV (perm_hd = head_dim) are rotated
//     in registers (the pair partner sits 8 lanes away), rounded to fp16 and
//     written as Q to qout [M][d] and as K, V rows into cache layer `layer`.
//     The weight may be a section view: its column n belongs to section
//     sec_base + n / d (0 Q, 1 K, 2 V).
// perm_hd > 0: the packed columns are in RoPE-pair order; STORE / RESID and
// split partials write column qkv_natural_col(n).
enum EpiMode { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_QKV_ROPE = 3 };
struct Epi {
  int mode;
  float* out_f32;
  uint16_t* out_f16;
  int ldo;
  int perm_hd = 0;
  const float* rope = nullptr;  // cos [S][hd/2] then sin [S][hd/2]
  uint16_t* qout = nullptr;
  KvGeom kv{};
  int layer = 0, lane = 0, p0 = 0;
  int sec_base = 0;
};

// Activation source of the matrix kernels: fp16 rows, or fp32 residual rows
// normalised on the fly (h = fp16(gamma * x / sqrt(mean(x^2) + eps))).
struct ASrc {
  const uint16_t* a16;  // fp16 [M][K] (used when x32 and att are null)
  const float* x32;     // fp32 [M][K] residual rows to RMS-normalise
  const uint16_t* gamma;
  float eps;
  // decode attention parts to merge into fp16 A rows (K = H * att_hd)
  const float* att = nullptr;
  int att_np = 0, att_np_max = 0, att_hd = 0;
  // with x32 and emb set (GEMV, first layer): row m is f32(emb[tok[tok_idx[m]]])
  // instead of x32's row, and the kernel writes it to x32 (the residual)
  const uint16_t* emb = nullptr;
  const int32_t* tok = nullptr;  // ids outside [0, vocab) are clamped
  int tok_idx[8] = {};
  int vocab = 0;
};

// C = A * W^T for M <= 8 rows (decode GEMV shape); K split across waves.
// With a.x32 set the A operand is fp16(RMSNorm(x32) * gamma); with a.att
// set it is the merged decode attention output. Both need K <= 2048 (and
// att M * np <= 16); gemv_supported tells whether a call can run here.
bool gemv_supported(int M, int K, const ASrc& a);
hipError_t launch_w4_gemv(const Packed& w, const ASrc& a, int M, const Epi& e, hipStream_t s);
// Launch plan of the prefill GEMM: row tile 16*mb, nbw n-blocks per wave,
// gx column blocks x gy row tiles x S K-splits of gps groups each.
struct GemmPlan {
  int mb, nbw, gx, gy, S, gps, blocks;
  float* part;  // S > 1: fp32 partial tiles [S][M][N], summed by the consumer
};
constexpr int kMaxSplitK = 16;  // consumers sum at most this many partials
// swiglu: gate/up pairs per wave and no K split; unsplit: no K split
// folded: the caller sums split-K partials within a pass it makes anyway
// (false: the standalone linear, which needs an extra reduction pass)
GemmPlan plan_w4_gemm(int N, int K, int M, bool swiglu, bool unsplit = false, bool folded = true);
size_t w4_gemm_scratch_bytes(int N, int K, int M, bool swiglu, bool folded = true);
// C = A * W^T for any M (prefill GEMM shape); A fp16 [M][K]. When the plan
// splits K (S > 1, never for SwiGLU) the kernel writes the S partials to
// `part` instead of running the epilogue; the caller passes them on.
hipError_t launch_w4_gemm(const Packed& w, const uint16_t* A, int M, const Epi& e, float* part, hipStream_t s,
                          bool folded = true);
// out (= or +=) sum of S partials [S][M][N], in split order.
hipError_t launch_reduce_partials(const float* part, int S, int M, int N, float* out, int accumulate, hipStream_t s);

// Pending split-K partials of a residual GEMM: x += sum_s part[s] (split
// order) before x is used.
struct Pending {
  const float* part;  // [S][M][d] or null
  int S;
};
// First layer of a prefill: x [M][d] = f32(embed[tokens[m]]) and fp16 h =
// RMSNorm(x) * gamma, bit-identical to launch_embed then launch_rmsnorm.
hipError_t launch_embed_rmsnorm(const uint16_t* embed, const int32_t* tokens, int V, int M, int d, float* x,
                                const uint16_t* gamma, float eps, uint16_t* h, hipStream_t s);
// x += pending (if any), then fp16 h [M][d] = RMSNorm(x) (prefill path).
hipError_t launch_rmsnorm(float* x, Pending pend, const uint16_t* gamma, float eps, int M, int d, uint16_t* h,
                          hipStream_t s);

// Per-row placement of the rows of one call: row m belongs to lane
// row_lane[m] at absolute position row_pos[m]. Prefill rows are all one
// lane at p0 + m (per_row == 0); decode rows use the arrays (M <= 8).
struct RowMap {
  int per_row;
  int lane, p0;
  int row_lane[8];
  int row_pos[8];
  // Decode steps replayed from a graph read row m's position on the device,
  // dpos[row_lane[m]] (advanced by launch_advance_pos at the end of each
  // step), so one captured step serves every position with the same launch
  // shape; row_pos keeps the host's values, which plan the launches.
  const int* dpos = nullptr;
};

// Device copy of the lanes' positions for graph-replayed decode steps.
struct PosArgs {
  int v[8];
  int n;
};
hipError_t launch_set_pos(int* dpos, const PosArgs& a, hipStream_t s);
// dpos[row_lane[m]] += 1 for the M rows of a decode step.
hipError_t launch_advance_pos(int* dpos, const RowMap& rm, int M, hipStream_t s);

// RoPE on q and k of qkv fp32 [M][3d] (the sum of S split-K partials, each
// [M][3d], in split order), fp16 Q out [M][d], K/V into cache layer.
hipError_t launch_rope_kv(const float* qkv, int S, int M, const RowMap& rm, const float* rope_cs, const KvGeom& kv,
                          int layer, uint16_t* q_out, hipStream_t s);

// Causal attention of M new rows of one lane (prefill) over cache rows
// 0..p0+M-1 of one layer. Q fp16 [M][d] -> O fp16 [M][d].
hipError_t launch_attn_prefill(const uint16_t* q, int M, int lane, int p0, const KvGeom& kv, int layer,
                               uint16_t* o, hipStream_t s);
// Single-query attention for M decode rows (one per lane) over each lane's
// rows 0..row_pos[m], from the raw QKV projection qkv fp32 [M][3d]: applies
// RoPE, writes the new K/V row into cache layer `layer` and attends in
// parts of 128 keys (256 for a row with more than 1024 visible keys): part
// receives, per (row, head, part), the part's softmax state (np_max =
// ceil(S / 128) slots per (row, head), rows of hd + 4 floats; each row's
// first attn_decode_parts() slots are written, empty ones with max -inf).
// With o non-null the parts are also merged into O fp16 [M][d]; otherwise
// the O projection merges them (ASrc::att).
size_t attn_decode_scratch_floats(int max_rows, int H, int hd, int S);
int attn_decode_parts(int M, const RowMap& rm, const KvGeom& kv);  // parts written per (row, head) this call
// Everything the decode attention's launch depends on besides the positions
// themselves (grid, block width, parts per row): equal shapes let a captured
// decode step be replayed at the next positions. Writes 3 + 2 * M ints.
void attn_decode_shape(int M, const RowMap& rm, const KvGeom& kv, int* out);
int attn_decode_np_max(int S);                  // part slots per (row, head)
hipError_t launch_attn_decode(const float* qkv, int M, const RowMap& rm, const float* rope_cs, const KvGeom& kv,
                              int layer, float* part, uint16_t* o, hipStream_t s);

// Token ids outside [0, V) are clamped into range (no out-of-bounds read).
hipError_t launch_embed(const uint16_t* embed, const int32_t* tokens, int M, const RowMap& rm, int d, int V,
                        float* x, hipStream_t s);
// Final RMSNorm of the residual rows x [M][d] (M <= 8, d <= 2048), logits
// against the head in tile order (launch_pack_head) written at
// logits[out_row(m) * V] (out_row = the row's lane in decode, m in prefill),
// and per 16-row block argmax candidates in scratch (head_scratch_bytes).
size_t head_scratch_bytes(int max_rows, int V);
hipError_t launch_head(const float* x, int M, const uint16_t* gamma, float eps, const uint8_t* head_tiles, int V,
                       int d, float* logits, const RowMap& rm, void* scratch, hipStream_t s);
// next[out_row(m)] = argmax of row m's logits, from the head's per-block
// candidates in `scratch` (ties: lowest index). advance (optional): also
// advance[row_lane[m]] += 1 (the device positions of a graph-replayed decode
// step, so that it needs no kernel of its own for them).
hipError_t launch_argmax(int M, int V, const RowMap& rm, const void* scratch, int32_t* next, hipStream_t s,
                         int* advance = nullptr);
// dst[row_lane[m] * d] = src[m * d] for m < M (decode output rows by lane).
hipError_t launch_scatter_rows(const float* src, int M, int d, const RowMap& rm, float* dst, hipStream_t s);

// Store-h: fp16 h rows [M][d] -> h cache [lane][layer][pos][d] at each row's
// lane and position.
hipError_t launch_store_h(const uint16_t* h, int M, int d, const RowMap& rm, uint8_t* base, size_t layer_bytes,
                          int n_layers, int layer, hipStream_t s);
// INT8 store-h rows: h row m (fp16 [d]) -> codes and per-128-group scales at
// its position in its lane's cache layer (h8_planes with S = max_seq); with
// hhat, fp16(q * s) of the row is also written to hhat[m][d].
hipError_t launch_store_h8(const uint16_t* h, int M, int d, int S, const RowMap& rm, uint8_t* base,
                           size_t layer_bytes, int n_layers, int layer, uint16_t* hhat, hipStream_t s);
// fp16(q * s) of positions 0 .. rows-1 of one INT8 store-h cache layer -> out [rows][d].
hipError_t launch_dequant_h8(const uint8_t* layer_base, int rows, int d, int S, uint16_t* out, hipStream_t s);

// Per-iteration residual-norm check: result = min(result, code_base + m) for
// each row m of x (+ pending partials) whose L2 norm is not <= max_norm.
constexpr int kSafetyRowBits = 20;  // code = iteration << kSafetyRowBits | row
hipError_t launch_safety_reset(int* result, hipStream_t s);
hipError_t launch_safety_check(const float* x, Pending pend, int M, int d, float max_norm, int code_base, int* result,
                               hipStream_t s);

hipError_t launch_kv_quantize_rows(const uint16_t* x, int rows, int hd, int8_t* q, uint16_t* sc,
                                   hipStream_t s);

}  // namespace tl
