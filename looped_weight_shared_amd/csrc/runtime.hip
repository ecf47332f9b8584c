// Host runtime of the C ABI declared in include/tl.h: argument and state
// validation, workspace carving, weight repacking at create time, and the
// layer sequence of prefill and cached decode.
//
// The forward pass follows the TinyLoop docs ("TinyLoop Framework" intro
// page): embed, n_pre distinct pre-blocks, then ONE loop block applied L
// times, then final norm and head. Effective layer l uses pre-block l for
// l < n_pre and the loop block otherwise, and writes KV cache layer l.
// In a decode step the lanes are ordered by descending L so that the lanes
// still running at loop iteration i are always the first rows of the batch
// (the "L-aware batching" of the "Current Status" page: each lane keeps its
// own depth).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "tl.h"
#include "tl_kernels.h"

namespace {

thread_local std::string g_err;

tl_status fail(tl_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

#define TL_HIP(expr)                                                                          \
  do {                                                                                        \
    hipError_t e_ = (expr);                                                                   \
    if (e_ != hipSuccess) return fail(TL_E_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct BlockW {
  tl::Packed qkv, o, gu, down;
  const uint16_t* attn_norm;
  const uint16_t* mlp_norm;
};

bool check_cfg(const tl_config* c, tl_status* st, std::string* why) {
  *st = TL_E_INVAL;
  if (!c) return *why = "cfg is NULL", false;
  if (c->head_dim != 64 && c->head_dim != 128) return *why = "head_dim must be 64 or 128", false;
  if (c->n_heads < 1 || c->d_model != c->n_heads * c->head_dim) return *why = "d_model != n_heads*head_dim", false;
  if (c->d_model % 32 || c->ffn_dim < 16 || c->ffn_dim % 16) return *why = "d_model % 32 or ffn_dim % 16 != 0", false;
  if (c->d_model > 2048) return *why = "d_model must be <= 2048 (one residual row per 256 threads in registers)", false;
  if (c->group_size != 128) return *why = "group_size must be 128", false;
  if (c->vocab < 1 || c->n_pre < 0) return *why = "vocab < 1 or n_pre < 0", false;
  if (c->kv_dtype != TL_KV_FP16 && c->kv_dtype != TL_KV_INT8 && c->kv_dtype != TL_KV_H16 &&
      c->kv_dtype != TL_KV_H8)
    return *why = "bad kv_dtype", false;
  if (c->kv_dtype == TL_KV_H8 && c->d_model % 128)
    return *why = "store-h INT8 (TL_KV_H8) needs d_model % 128 == 0 (128-element groups)", false;
  if (!(c->rms_eps >= 0.f) || !(c->rope_base > 0.f)) return *why = "bad rms_eps or rope_base", false;
  *st = TL_E_RANGE;
  if (c->max_loops < 1 || c->max_loops > 64) return *why = "max_loops must be in 1..64", false;
  if (c->n_lanes < 1 || c->n_lanes > 8) return *why = "n_lanes must be in 1..8", false;
  if (c->max_seq < 1 || c->max_tokens < 1) return *why = "max_seq and max_tokens must be >= 1", false;
  if (c->cache_window < 0) return *why = "cache_window must be >= 0", false;
  if (c->fp16_body != 0 && c->fp16_body != 1) return *why = "fp16_body must be 0 or 1", false;
  if ((c->kv_dtype == TL_KV_H16 || c->kv_dtype == TL_KV_H8) && c->cache_window > 0) {
    *st = TL_E_UNSUPPORTED;
    return *why = "store-h (TL_KV_H16, TL_KV_H8) does not combine with cache_window", false;
  }
  *st = TL_OK;
  return true;
}

// one linear in the block store: packed W4 (tiles + scales) or the FP16 body
size_t linear_bytes(const tl_config* c, int N, int K) {
  return c->fp16_body ? tl::packed_f16_bytes(N, K) : tl::packed_bytes(N, K);
}
size_t block_bytes(const tl_config* c) {
  const int d = c->d_model, f = c->ffn_dim;
  if (c->fp16_body)
    return al256(linear_bytes(c, 3 * d, d)) + al256(linear_bytes(c, d, d)) + al256(linear_bytes(c, 2 * f, d)) +
           al256(linear_bytes(c, d, f));
  return al256(tl::packed_bytes(3 * d, d)) + al256(tl::packed_bytes(d, d)) + al256(tl::packed_bytes(2 * f, d)) +
         al256(tl::packed_bytes(d, f));
}
// Cache rows per (lane, layer, head): max_seq, or with a window W a ring of
// W + max_tokens rows (a prefill chunk never overwrites a row one of its own
// queries still sees) when that is shorter.
int kv_rows(const tl_config* c) {
  if (c->cache_window <= 0) return c->max_seq;
  return (int)std::min<long long>(c->max_seq, (long long)c->cache_window + c->max_tokens);
}
size_t rope_bytes(const tl_config* c) { return al256((size_t)2 * c->max_seq * (c->head_dim / 2) * 4); }

int tokens_cap(const tl_config* c) { return std::max(c->max_tokens, c->n_lanes); }

// Largest split-K partial buffer any prefill GEMM of this model can need.
size_t gemm_scratch_bytes(const tl_config* c) {
  const int d = c->d_model, f = c->ffn_dim, T = tokens_cap(c);
  size_t mx = 0;
  for (int M = 1; M <= T; ++M) {
    mx = std::max(mx, tl::w4_gemm_scratch_bytes(3 * d, d, M, false));
    mx = std::max(mx, tl::w4_gemm_scratch_bytes(d, d, M, false));
    mx = std::max(mx, tl::w4_gemm_scratch_bytes(2 * f, d, M, true));
    mx = std::max(mx, tl::w4_gemm_scratch_bytes(d, f, M, false));
  }
  return mx;
}

// Self-speculative decode drafts at most this many tokens per round, so the
// verify prefill (draft + 1 rows) fits the head kernel's row limit.
constexpr int kSpecMaxDraft = 7;
int head_rows_cap(const tl_config* c) { return std::max(c->n_lanes, kSpecMaxDraft + 1); }

struct ActLayout {
  size_t x, h, qkv, q, o, a, part, logits, gpart, hscr, spec, safety, dpos, hkv, hdq, total;
};
ActLayout act_layout(const tl_config* c) {
  const size_t T = (size_t)tokens_cap(c), d = c->d_model, f = c->ffn_dim;
  ActLayout L;
  size_t off = 0;
  L.x = off; off += al256(T * d * 4);
  L.h = off; off += al256(T * d * 2);
  L.qkv = off; off += al256(T * 3 * d * 4);
  L.q = off; off += al256(T * d * 2);
  L.o = off; off += al256(T * d * 2);
  L.a = off; off += al256(T * f * 2);
  L.part = off; off += al256(tl::attn_decode_scratch_floats(c->n_lanes, c->n_heads, c->head_dim, c->max_seq) * 4);
  L.logits = off; off += al256((size_t)head_rows_cap(c) * c->vocab * 4);
  L.gpart = off; off += al256(gemm_scratch_bytes(c));
  L.hscr = off; off += al256(tl::head_scratch_bytes(head_rows_cap(c), c->vocab));
  // speculative tokens: draft chain [kSpecMaxDraft + 2][n_lanes], verify
  // tokens and verifier argmaxes [kSpecMaxDraft + 1] each
  L.spec = off; off += al256(((size_t)(kSpecMaxDraft + 2) * c->n_lanes + 2 * (kSpecMaxDraft + 1)) * 4);
  L.safety = off; off += al256(4);  // first tripped (iteration, row) code of the safety check
  L.dpos = off; off += al256(8 * 4);  // lane positions read by graph-replayed decode steps
  // store-h: K/V rebuilt for one layer, FP16 [lane][K|V][H][max_seq][hd]
  const bool hmode = c->kv_dtype == TL_KV_H16 || c->kv_dtype == TL_KV_H8;
  L.hkv = off;
  if (hmode) off += al256((size_t)c->n_lanes * 2 * c->max_seq * c->d_model * 2);
  // store-h INT8: fp16(q * s) rows of one lane's h cache for the rebuild, FP16 [max_seq][d]
  L.hdq = off;
  if (c->kv_dtype == TL_KV_H8) off += al256((size_t)c->max_seq * c->d_model * 2);
  L.total = off;
  return L;
}

// The GEMV kernel keeps all M activation rows of K in LDS.

}  // namespace

struct tl_ctx {
  tl_config cfg;
  std::vector<BlockW> blocks;  // n_pre pre-blocks, then the loop block
  const uint16_t* embed;
  const uint8_t* head;  // head repacked in MFMA tile order
  const uint16_t* final_norm;
  float* rope;
  tl::KvGeom kv;
  float* x;
  uint16_t* h;
  float* qkv;
  uint16_t* q;
  uint16_t* o;
  uint16_t* a;
  float* part;
  float* logits;
  float* gpart;      // split-K partial tiles of the prefill GEMM
  tl::Pending pend;  // residual partials not yet added to x
  void* hscr;        // head/argmax per-block candidates
  int32_t* spec_chain;  // [kSpecMaxDraft + 2][n_lanes]
  int32_t* spec_ver;    // [kSpecMaxDraft + 1]
  int32_t* spec_next;   // [kSpecMaxDraft + 1]
  // store-h: h cache [lane][layer][max_seq][d] (in d_kv); kv then describes the scratch.
  // h8: the cache holds INT8 codes and per-128-group fp16 scales (tl::h8_planes)
  // and hdq the fp16(q * s) rows a rebuild reads
  bool hmode = false;
  bool h8 = false;
  uint16_t* hdq = nullptr;
  uint8_t* hc_base = nullptr;
  size_t hc_layer_bytes = 0;
  int hc_layers = 0;
  // per-iteration residual-norm check (off while safety_max <= 0)
  float safety_max = 0.f;
  int* safety_res = nullptr;
  int32_t safety_host = 0x7fffffff;
  int safety_iter = -1, safety_row = -1;  // last trip reported
  std::vector<int> len, loops, depth;  // depth: effective layers every cached token has
  int32_t spec_host[16];               // host side of the speculative token exchange
  // optional: launch sequences captured as HIP graphs and replayed when a
  // later call has the same shape and pointers (cuts host enqueue time):
  // bit 0 prefill, bit 1 decode steps (tl_set_graphs)
  int graph_mask = 0;
  // decode graphs read the lane positions from here (device int32 [n_lanes]);
  // dpos_synced: it equals len[] as of the stream's tail
  int32_t* dpos = nullptr;
  bool dpos_synced = false;
  bool force_eager = false;  // self-speculative drafting: plain launches
  struct DecodeGraph {
    std::vector<long long> key;
    hipGraphExec_t exec = nullptr;
    hipEvent_t done = nullptr;  // recorded after each replay
    unsigned long long used = 0;
  };
  std::vector<DecodeGraph> dgraphs;
  unsigned long long dgraph_clock = 0;
  bool h_ready = false;  // c->h holds the next linear's normalised input (fused embed + RMSNorm)
  // the first layer's rows are still the embedding rows of these tokens (the
  // first GEMV reads them directly and writes x); emb_rm maps row -> token
  const int32_t* emb_tokens = nullptr;
  tl::RowMap emb_rm{};
  hipStream_t cap_stream = nullptr;  // capture only; default priority
  struct PrefillGraph {
    bool valid = false;
    int lane = -1, n = 0, p0 = 0, loops = 0;
    const void *tokens = nullptr, *hidden = nullptr, *logits = nullptr, *next = nullptr;
    hipGraphExec_t exec = nullptr;
  } pg;
  hipEvent_t pg_done = nullptr;  // recorded after each replay; waited on before the exec is destroyed
  // kernel timing window
  bool prof_on = false;
  std::vector<hipEvent_t> prof_ev;  // 2 per launch
  std::vector<int> prof_kind;
  tl::LaunchTimer timer;
};

namespace tl {
thread_local LaunchTimer* t_launch_timer = nullptr;
}

namespace {

// Sets the kind under which the launches inside the scope are timed while a
// timing window is open (each launch records its own event pair).
void drop_prefill_graph(tl_ctx* ctx);
void drop_decode_graphs(tl_ctx* ctx);

struct KScope {
  KScope(tl_ctx* ctx, int kind, hipStream_t) {
    tl::t_launch_timer = ctx->prof_on ? &ctx->timer : nullptr;
    ctx->timer.cur_kind = kind;
  }
  ~KScope() { tl::t_launch_timer = nullptr; }
};

// Decode-shaped calls (M <= 8) use the split-K-in-block GEMV with the RMSNorm
// fused; larger M uses the MFMA GEMM, whose K-split partials (if the plan
// splits) are left for the consumer: *S_out receives the split count. The
// GEMM uses *gemm_epi instead of e when one is given (an epilogue that needs
// K unsplit: the plan then never splits); *used_gemm_epi tells whether it did.
tl_status linear(tl_ctx* c, int kind, const tl::Packed& w, const tl::ASrc& src, int M, const tl::Epi& e,
                 int* S_out, hipStream_t s, const tl::Epi* gemm_epi = nullptr, bool* used_gemm_epi = nullptr) {
  *S_out = 1;
  if (used_gemm_epi) *used_gemm_epi = false;
  // the GEMV's fused RMSNorm reads x as is: pending split-K residual partials
  // (left by a GEMM) must go through the RMSNorm kernel first
  const bool pending = src.x32 && c->pend.part;
  if (c->emb_tokens && src.x32) {  // first layer: the GEMV gathers the embedding rows itself
    tl::ASrc se = src;
    se.emb = c->embed;
    se.tok = c->emb_tokens;
    se.vocab = c->cfg.vocab;
    for (int m = 0; m < M && m < 8; ++m) se.tok_idx[m] = c->emb_rm.per_row ? c->emb_rm.row_lane[m] : m;
    c->emb_tokens = nullptr;
    if (!pending && tl::gemv_supported(M, w.K, se)) {
      KScope k(c, kind, s);
      TL_HIP(tl::launch_w4_gemv(w, se, M, e, s));
      return TL_OK;
    }
    KScope k(c, TL_K_EMBED, s);
    TL_HIP(tl::launch_embed(c->embed, se.tok, M, c->emb_rm, w.K, c->cfg.vocab, c->x, s));
  }
  if (c->h_ready && src.x32) {  // h = fp16(RMSNorm(x) * gamma) is already in place
    c->h_ready = false;
    const bool alt = gemm_epi != nullptr;
    const int S = alt ? 1 : tl::plan_w4_gemm(w.N, w.K, M, e.mode == tl::EPI_SWIGLU).S;
    KScope k(c, kind, s);
    TL_HIP(tl::launch_w4_gemm(w, c->h, M, alt ? *gemm_epi : e, c->gpart, s));
    *S_out = S;
    if (used_gemm_epi) *used_gemm_epi = alt;
    return TL_OK;
  }
  if (!pending && tl::gemv_supported(M, w.K, src)) {
    KScope k(c, kind, s);
    TL_HIP(tl::launch_w4_gemv(w, src, M, e, s));
    return TL_OK;
  }
  const uint16_t* A = src.a16;
  if (src.x32) {
    // x += pending residual partials, then h = fp16(RMSNorm(x))
    KScope k(c, TL_K_NORM, s);
    TL_HIP(tl::launch_rmsnorm(c->x, c->pend, src.gamma, src.eps, M, w.K, c->h, s));
    c->pend = tl::Pending{nullptr, 1};
    A = c->h;
  }
  const bool alt = gemm_epi != nullptr;
  const int S = alt ? 1 : tl::plan_w4_gemm(w.N, w.K, M, e.mode == tl::EPI_SWIGLU).S;
  KScope k(c, kind, s);
  TL_HIP(tl::launch_w4_gemm(w, A, M, alt ? *gemm_epi : e, c->gpart, s));
  *S_out = S;
  if (used_gemm_epi) *used_gemm_epi = alt;
  return TL_OK;
}

// One effective layer over M rows (prefill rows of one lane, or the first M
// decode rows).
// Store-h attention input of one layer (TL_KV_H16, TL_KV_H8; "Current
// Status" page, KV-cache table: Store-h FP16 and INT8; "Claims & Data
// Sources": h-mode KV reconstruction from the shared W_k / W_v):
//   1. h = fp16(RMSNorm(x)) (pending split partials summed), each row also
//      stored at its position in its lane's h cache for this layer (H8: as
//      INT8 codes with one fp16 scale per 128-element group, and K, V are
//      rebuilt from fp16(q * s), the new rows' included);
//   2. prefill: Q = fp16(RoPE(h W_q^T)) by the Q section of the packed QKV
//      (GEMM, RoPE epilogue); decode: q, k, v of the new rows (GEMV) for the
//      decode attention, which rotates them itself;
//   3. K, V of the lane's positions 0 .. end-1 (prefill: through the new
//      rows; decode: the cached ones) rebuilt from the h cache by the K/V
//      section (GEMM with the RoPE epilogue, K never split) into the scratch
//      that c->kv describes, one slot per lane.
tl_status hmode_qkv(tl_ctx* c, const BlockW& B, int layer, int M, const tl::RowMap& rm, bool decode, hipStream_t s) {
  const int d = c->cfg.d_model, hd = c->cfg.head_dim;
  {
    KScope k(c, TL_K_NORM, s);
    TL_HIP(tl::launch_rmsnorm(c->x, c->pend, B.attn_norm, c->cfg.rms_eps, M, d, c->h, s));
    c->pend = tl::Pending{nullptr, 1};
  }
  {
    KScope k(c, TL_K_COPY, s);
    if (c->h8)  // decode: the new rows' fp16(q * s) also go to hdq for their K/V
      TL_HIP(tl::launch_store_h8(c->h, M, d, c->cfg.max_seq, rm, c->hc_base, c->hc_layer_bytes, c->hc_layers, layer,
                                 decode ? c->hdq : nullptr, s));
    else
      TL_HIP(tl::launch_store_h(c->h, M, d, rm, c->hc_base, c->hc_layer_bytes, c->hc_layers, layer, s));
  }
  const int nbd = d / 16;  // n-blocks per section
  const size_t tb = B.qkv.f16 ? 4096 : 1024;  // tile bytes
  const tl::Packed qsec{B.qkv.tiles, B.qkv.scales, d, d, B.qkv.G, B.qkv.f16};
  const tl::Packed kvsec{B.qkv.tiles + (size_t)nbd * B.qkv.G * tb,
                         B.qkv.f16 ? nullptr : B.qkv.scales + (size_t)nbd * B.qkv.G * 16, 2 * d, d, B.qkv.G,
                         B.qkv.f16};
  tl::Epi er{tl::EPI_QKV_ROPE, nullptr, nullptr, 0};
  er.perm_hd = hd;
  er.rope = c->rope;
  er.qout = c->q;
  er.kv = c->kv;
  er.layer = 0;
  if (decode && c->h8) {
    // q from h; k, v of the new rows from the fp16(q * s) rows the cache will
    // give back, as for every cached position
    tl::Epi eq{tl::EPI_STORE, c->qkv, nullptr, 3 * d};
    eq.perm_hd = hd;
    tl::Epi ekv{tl::EPI_STORE, c->qkv + d, nullptr, 3 * d};
    ekv.perm_hd = hd;
    KScope k(c, TL_K_QKV, s);
    TL_HIP(tl::launch_w4_gemv(qsec, tl::ASrc{c->h, nullptr, nullptr, 0.f}, M, eq, s));
    TL_HIP(tl::launch_w4_gemv(kvsec, tl::ASrc{c->hdq, nullptr, nullptr, 0.f}, M, ekv, s));
  } else if (decode) {
    tl::Epi eq{tl::EPI_STORE, c->qkv, nullptr, 3 * d};
    eq.perm_hd = hd;
    KScope k(c, TL_K_QKV, s);
    TL_HIP(tl::launch_w4_gemv(B.qkv, tl::ASrc{c->h, nullptr, nullptr, 0.f}, M, eq, s));
  } else {
    er.lane = rm.lane;
    er.p0 = rm.p0;
    KScope k(c, TL_K_QKV, s);
    TL_HIP(tl::launch_w4_gemm(qsec, c->h, M, er, c->gpart, s));
  }
  // rebuild, per lane: rows are positions 0 .. end-1 of the lane's h cache
  er.sec_base = 1;
  er.p0 = 0;
  const int nrows = decode ? M : 1;
  for (int m = 0; m < nrows; ++m) {
    const int lane = decode ? rm.row_lane[m] : rm.lane;
    const int end = decode ? rm.row_pos[m] : rm.p0 + M;
    if (end < 1) continue;
    er.lane = lane;
    const uint8_t* lb = c->hc_base + ((size_t)lane * c->hc_layers + layer) * c->hc_layer_bytes;
    const uint16_t* hrows = reinterpret_cast<const uint16_t*>(lb);
    if (c->h8) {
      KScope k(c, TL_K_COPY, s);
      TL_HIP(tl::launch_dequant_h8(lb, end, d, c->cfg.max_seq, c->hdq, s));
      hrows = c->hdq;
    }
    KScope k(c, TL_K_ROPE_KV, s);
    TL_HIP(tl::launch_w4_gemm(kvsec, hrows, end, er, c->gpart, s));
  }
  return TL_OK;
}

// Split-K partials [S][M][d] of a residual GEMM (O or down projection). A
// prefill keeps them pending: the next RMSNorm (or resolve()) adds them to x
// in split order, saving a pass over x. A decode step adds them right away:
// its row count shrinks from layer to layer as lanes reach their L, and the
// head reads x directly, so partials left for later would be summed with the
// wrong row stride or not at all. (Decode reaches the GEMM only when the
// GEMV cannot take the shape, e.g. ffn_dim above 8192 for the down projection.)
tl_status keep_partials(tl_ctx* c, int kind, int S, int M, bool decode, hipStream_t s) {
  if (S <= 1) return TL_OK;
  if (!decode) {
    c->pend = tl::Pending{c->gpart, S};
    return TL_OK;
  }
  KScope k(c, kind, s);
  TL_HIP(tl::launch_reduce_partials(c->gpart, S, M, c->cfg.d_model, c->x, 1, s));
  return TL_OK;
}

tl_status run_layer(tl_ctx* c, const BlockW& B, int layer, int M, const tl::RowMap& rm, bool decode,
                    hipStream_t s) {
  const int d = c->cfg.d_model, f = c->cfg.ffn_dim;
  const float eps = c->cfg.rms_eps;
  tl_status st;
  int S = 1;
  tl::ASrc osrc{c->o, nullptr, nullptr, 0.f};
  // store-h: attention reads the rebuilt scratch as cache layer 0
  const int alayer = c->hmode ? 0 : layer;
  if (c->hmode) {
    st = hmode_qkv(c, B, layer, M, rm, decode, s);
    if (st != TL_OK) return st;
  }
  // h = fp16(RMSNorm(x)); [q;k;v] = h W_qkv^T (packed in RoPE-pair order).
  // A prefill GEMM with unsplit K and an FP16 cache applies RoPE and writes
  // Q and the K/V rows in its epilogue; otherwise qkv goes out in fp32.
  tl::Epi eq{tl::EPI_STORE, c->qkv, nullptr, 3 * d};
  eq.perm_hd = c->cfg.head_dim;
  tl::Epi er = eq;
  er.mode = tl::EPI_QKV_ROPE;
  er.rope = c->rope;
  er.qout = c->q;
  er.kv = c->kv;
  er.layer = layer;
  er.lane = rm.lane;
  er.p0 = rm.p0;
  bool roped = c->hmode;  // store-h: Q (prefill) or q, k, v (decode) are done
  if (!c->hmode) {
    st = linear(c, TL_K_QKV, B.qkv, tl::ASrc{nullptr, c->x, B.attn_norm, eps}, M, eq, &S, s,
                (!decode && !c->kv.int8) ? &er : nullptr, &roped);
    if (st != TL_OK) return st;
  }
  const float* qkv = S > 1 ? c->gpart : c->qkv;
  if (decode) {
    if (S > 1) {
      // the decode attention reads whole projections: sum a split GEMM's partials first
      KScope k(c, TL_K_QKV, s);
      TL_HIP(tl::launch_reduce_partials(c->gpart, S, M, 3 * d, c->qkv, 0, s));
      qkv = c->qkv;
    }
    // RoPE, new K/V into cache layer `layer`, single-query attention in key
    // parts; the O projection merges the parts itself when its GEMV can
    tl::ASrc att{nullptr, nullptr, nullptr, 0.f, c->part, tl::attn_decode_parts(M, rm, c->kv),
                 tl::attn_decode_np_max(c->cfg.max_seq), c->cfg.head_dim};
    const bool fuse = tl::gemv_supported(M, d, att);
    KScope k(c, TL_K_ATTN, s);
    TL_HIP(tl::launch_attn_decode(qkv, M, rm, c->rope, c->kv, alayer, c->part, fuse ? nullptr : c->o, s));
    if (fuse) osrc = att;
  } else {
    // RoPE on q, k (summing the split-K partials); fp16 Q; K, V into cache layer `layer`
    if (!roped) {
      KScope k(c, TL_K_ROPE_KV, s);
      TL_HIP(tl::launch_rope_kv(qkv, S, M, rm, c->rope, c->kv, layer, c->q, s));
    }
    KScope k(c, TL_K_ATTN, s);
    TL_HIP(tl::launch_attn_prefill(c->q, M, rm.lane, rm.p0, c->kv, alayer, c->o, s));
  }
  // x += O W_o^T (deferred to the next RMSNorm when K is split)
  st = linear(c, TL_K_O, B.o, osrc, M, tl::Epi{tl::EPI_RESID, c->x, nullptr, d}, &S, s);
  if (st != TL_OK) return st;
  st = keep_partials(c, TL_K_O, S, M, decode, s);
  if (st != TL_OK) return st;
  // a = fp16(silu(h2 W_gate^T) * h2 W_up^T), h2 = fp16(RMSNorm(x))
  st = linear(c, TL_K_GATE_UP, B.gu, tl::ASrc{nullptr, c->x, B.mlp_norm, eps}, M,
              tl::Epi{tl::EPI_SWIGLU, nullptr, c->a, f}, &S, s);
  if (st != TL_OK) return st;
  // x += a W_down^T (deferred likewise)
  st = linear(c, TL_K_DOWN, B.down, tl::ASrc{c->a, nullptr, nullptr, 0.f}, M,
              tl::Epi{tl::EPI_RESID, c->x, nullptr, d}, &S, s);
  if (st != TL_OK) return st;
  return keep_partials(c, TL_K_DOWN, S, M, decode, s);
}

// Apply any pending residual partials to x (after the last layer).
tl_status resolve(tl_ctx* c, int M, hipStream_t s) {
  if (!c->pend.part) return TL_OK;
  KScope k(c, TL_K_NORM, s);
  TL_HIP(tl::launch_rmsnorm(c->x, c->pend, c->final_norm, c->cfg.rms_eps, M, c->cfg.d_model, nullptr, s));
  c->pend = tl::Pending{nullptr, 1};
  return TL_OK;
}

tl_status check_lane(const tl_ctx* c, int lane) {
  if (!c) return fail(TL_E_INVAL, "ctx is NULL");
  if (lane < 0 || lane >= c->cfg.n_lanes) return fail(TL_E_INVAL, "lane index out of range");
  return TL_OK;
}

}  // namespace

extern "C" {

const char* tl_last_error(void) { return g_err.c_str(); }

size_t tl_weights_ws_bytes(const tl_config* cfg) {
  tl_status st;
  std::string why;
  if (!check_cfg(cfg, &st, &why)) return 0;
  return (size_t)(cfg->n_pre + 1) * block_bytes(cfg) + al256(tl::head_packed_bytes(cfg->vocab, cfg->d_model)) +
         rope_bytes(cfg);
}

size_t tl_kv_layer_bytes(const tl_config* cfg) {
  tl_status st;
  std::string why;
  if (!check_cfg(cfg, &st, &why)) return 0;
  const size_t rows = (size_t)kv_rows(cfg) * cfg->n_heads;
  if (cfg->kv_dtype == TL_KV_INT8) return tl::int8_planes(cfg->n_heads, kv_rows(cfg), cfg->head_dim).bytes;
  if (cfg->kv_dtype == TL_KV_H16) return (size_t)cfg->max_seq * cfg->d_model * 2;
  if (cfg->kv_dtype == TL_KV_H8) return tl::h8_planes(cfg->max_seq, cfg->d_model).bytes;
  return 2 * rows * cfg->head_dim * 2;
}

size_t tl_kv_bytes(const tl_config* cfg) {
  return (size_t)(cfg ? cfg->n_lanes : 0) * (size_t)(cfg ? cfg->n_pre + cfg->max_loops : 0) *
         tl_kv_layer_bytes(cfg);
}

size_t tl_act_ws_bytes(const tl_config* cfg) {
  tl_status st;
  std::string why;
  if (!check_cfg(cfg, &st, &why)) return 0;
  return act_layout(cfg).total;
}

tl_status tl_create(const tl_config* cfg, const tl_weights* w, void* d_weights_ws, void* d_kv, void* d_act_ws,
                    void* stream, tl_ctx** out) {
  tl_status st;
  std::string why;
  if (!out) return fail(TL_E_INVAL, "out is NULL");
  *out = nullptr;
  if (!check_cfg(cfg, &st, &why)) return fail(st, why);
  if (!w || !w->embed || !w->head || !w->final_norm || (cfg->n_pre > 0 && !w->pre))
    return fail(TL_E_INVAL, "missing weight pointer");
  if (!d_weights_ws || !d_kv || !d_act_ws) return fail(TL_E_INVAL, "workspace pointer is NULL");
  if (!aligned(d_weights_ws, 256) || !aligned(d_kv, 256) || !aligned(d_act_ws, 256))
    return fail(TL_E_INVAL, "workspaces must be 256-byte aligned");
  if (!aligned(w->embed, 16) || !aligned(w->head, 16) || !aligned(w->final_norm, 16))
    return fail(TL_E_INVAL, "embed/head/final_norm must be 16-byte aligned");
  auto block_ok = [](const tl_block& b) {
    const tl_qlinear* ls[7] = {&b.wq, &b.wk, &b.wv, &b.wo, &b.w_gate, &b.w_up, &b.w_down};
    for (auto* l : ls)
      if (!l->qweight || !l->scales || !aligned(l->qweight, 4) || !aligned(l->scales, 2)) return false;
    return b.attn_norm && b.mlp_norm && aligned(b.attn_norm, 16) && aligned(b.mlp_norm, 16);
  };
  for (int i = 0; i < cfg->n_pre; ++i)
    if (!block_ok(w->pre[i])) return fail(TL_E_INVAL, "pre-block weight pointer missing or misaligned");
  if (!block_ok(w->loop)) return fail(TL_E_INVAL, "loop-block weight pointer missing or misaligned");

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  tl_ctx* c = new tl_ctx();
  c->cfg = *cfg;
  c->embed = w->embed;

  c->final_norm = w->final_norm;
  const int d = cfg->d_model, f = cfg->ffn_dim;
  uint8_t* p = static_cast<uint8_t*>(d_weights_ws);
  auto carve = [&](int N, int K) {
    tl::Packed pk;
    pk.tiles = p;
    pk.scales = cfg->fp16_body ? nullptr : reinterpret_cast<const uint16_t*>(p + tl::packed_tile_bytes(N, K));
    pk.N = N;
    pk.K = K;
    pk.G = (K + 127) / 128;
    pk.f16 = cfg->fp16_body ? 1 : 0;
    p += al256(linear_bytes(cfg, N, K));
    return pk;
  };
  auto pack = [&](const tl_qlinear& l, int N, int K, const tl::Packed& dst, int off, int stride, int perm = 0) {
    if (dst.f16)
      return tl::launch_pack_f16(l.qweight, l.scales, N, K, const_cast<uint8_t*>(dst.tiles), dst.G, off, stride, perm,
                                 s);
    return tl::launch_pack(l.qweight, l.scales, N, K, const_cast<uint8_t*>(dst.tiles),
                           const_cast<uint16_t*>(dst.scales), dst.G, off, stride, perm, s);
  };
  for (int b = 0; b <= cfg->n_pre; ++b) {
    const tl_block& src = b < cfg->n_pre ? w->pre[b] : w->loop;
    BlockW B;
    B.qkv = carve(3 * d, d);
    B.o = carve(d, d);
    B.gu = carve(2 * f, d);
    B.down = carve(d, f);
    B.attn_norm = src.attn_norm;
    B.mlp_norm = src.mlp_norm;
    hipError_t e = hipSuccess;
    // q, k, v rows of each head in RoPE-pair order (the QKV epilogues rely on it)
    const int hd = cfg->head_dim;
    if (e == hipSuccess) e = pack(src.wq, d, d, B.qkv, 0, 1, hd);
    if (e == hipSuccess) e = pack(src.wk, d, d, B.qkv, d / 16, 1, hd);
    if (e == hipSuccess) e = pack(src.wv, d, d, B.qkv, 2 * d / 16, 1, hd);
    if (e == hipSuccess) e = pack(src.wo, d, d, B.o, 0, 1);
    if (e == hipSuccess) e = pack(src.w_gate, f, d, B.gu, 0, 2);  // gate/up n-blocks interleaved
    if (e == hipSuccess) e = pack(src.w_up, f, d, B.gu, 1, 2);
    if (e == hipSuccess) e = pack(src.w_down, d, f, B.down, 0, 1);
    if (e != hipSuccess) {
      delete c;
      return fail(TL_E_HIP, std::string("weight repack: ") + hipGetErrorString(e));
    }
    c->blocks.push_back(B);
  }
  // the head in MFMA tile order (streamed once per decode step)
  {
    c->head = p;
    hipError_t e = tl::launch_pack_head(w->head, cfg->vocab, d, p, s);
    p += al256(tl::head_packed_bytes(cfg->vocab, d));
    if (e != hipSuccess) {
      delete c;
      return fail(TL_E_HIP, std::string("head repack: ") + hipGetErrorString(e));
    }
  }
  // RoPE table: cos then sin of pos * base^(-2i/hd), computed in double.
  c->rope = reinterpret_cast<float*>(p);
  {
    const int half = cfg->head_dim / 2, S = cfg->max_seq;
    std::vector<float> tab((size_t)2 * S * half);
    for (int pos = 0; pos < S; ++pos)
      for (int i = 0; i < half; ++i) {
        const double th = std::pow((double)cfg->rope_base, -2.0 * i / cfg->head_dim);
        tab[(size_t)pos * half + i] = (float)std::cos(pos * th);
        tab[(size_t)S * half + (size_t)pos * half + i] = (float)std::sin(pos * th);
      }
    hipError_t e = hipMemcpyAsync(c->rope, tab.data(), tab.size() * 4, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      delete c;
      return fail(TL_E_HIP, std::string("rope table upload: ") + hipGetErrorString(e));
    }
  }
  c->hmode = cfg->kv_dtype == TL_KV_H16 || cfg->kv_dtype == TL_KV_H8;
  c->h8 = cfg->kv_dtype == TL_KV_H8;
  c->kv.base = static_cast<uint8_t*>(d_kv);
  c->kv.layer_bytes = tl_kv_layer_bytes(cfg);
  c->kv.n_layers = cfg->n_pre + cfg->max_loops;
  if (c->hmode) {  // d_kv holds h rows; attention reads the rebuilt one-layer scratch
    c->hc_base = static_cast<uint8_t*>(d_kv);
    c->hc_layer_bytes = tl_kv_layer_bytes(cfg);
    c->hc_layers = cfg->n_pre + cfg->max_loops;
    c->kv.base = static_cast<uint8_t*>(d_act_ws) + act_layout(cfg).hkv;
    c->kv.layer_bytes = (size_t)2 * cfg->max_seq * cfg->d_model * 2;
    c->kv.n_layers = 1;
  }
  c->kv.H = cfg->n_heads;
  c->kv.hd = cfg->head_dim;
  c->kv.S = cfg->max_seq;
  c->kv.cap = kv_rows(cfg);
  c->kv.window = cfg->cache_window;
  c->kv.int8 = cfg->kv_dtype == TL_KV_INT8;
  const ActLayout L = act_layout(cfg);
  uint8_t* ab = static_cast<uint8_t*>(d_act_ws);
  c->x = reinterpret_cast<float*>(ab + L.x);
  c->h = reinterpret_cast<uint16_t*>(ab + L.h);
  c->qkv = reinterpret_cast<float*>(ab + L.qkv);
  c->q = reinterpret_cast<uint16_t*>(ab + L.q);
  c->o = reinterpret_cast<uint16_t*>(ab + L.o);
  c->a = reinterpret_cast<uint16_t*>(ab + L.a);
  c->part = reinterpret_cast<float*>(ab + L.part);
  c->logits = reinterpret_cast<float*>(ab + L.logits);
  c->gpart = reinterpret_cast<float*>(ab + L.gpart);
  c->hscr = ab + L.hscr;
  c->hdq = c->h8 ? reinterpret_cast<uint16_t*>(ab + L.hdq) : nullptr;
  c->spec_chain = reinterpret_cast<int32_t*>(ab + L.spec);
  c->spec_ver = c->spec_chain + (size_t)(kSpecMaxDraft + 2) * cfg->n_lanes;
  c->spec_next = c->spec_ver + (kSpecMaxDraft + 1);
  c->safety_res = reinterpret_cast<int*>(ab + L.safety);
  c->dpos = reinterpret_cast<int32_t*>(ab + L.dpos);
  c->pend = tl::Pending{nullptr, 1};
  c->len.assign(cfg->n_lanes, 0);
  c->loops.assign(cfg->n_lanes, 1);
  c->depth.assign(cfg->n_lanes, INT_MAX);
  *out = c;
  return TL_OK;
}

tl_status tl_destroy(tl_ctx* ctx) {
  if (!ctx) return fail(TL_E_INVAL, "ctx is NULL");
  for (auto& e : ctx->prof_ev) (void)hipEventDestroy(e);
  drop_prefill_graph(ctx);
  drop_decode_graphs(ctx);
  if (ctx->pg_done) (void)hipEventDestroy(ctx->pg_done);
  if (ctx->cap_stream) (void)hipStreamDestroy(ctx->cap_stream);
  delete ctx;
  return TL_OK;
}

tl_status tl_set_loops(tl_ctx* ctx, int32_t lane, int32_t loops) {
  if (!ctx) return fail(TL_E_INVAL, "ctx is NULL");
  if (lane < -1 || lane >= ctx->cfg.n_lanes) return fail(TL_E_INVAL, "lane index out of range");
  if (loops < 1 || loops > ctx->cfg.max_loops) return fail(TL_E_RANGE, "loops outside 1..max_loops");
  const int lo = lane < 0 ? 0 : lane, hi = lane < 0 ? ctx->cfg.n_lanes : lane + 1;
  for (int l = lo; l < hi; ++l)
    if (ctx->len[l] > 0 && ctx->cfg.n_pre + loops > ctx->depth[l])
      return fail(TL_E_STATE, "lane holds tokens computed to a smaller depth");
  for (int l = lo; l < hi; ++l) ctx->loops[l] = loops;
  return TL_OK;
}

tl_status tl_get_loops(const tl_ctx* ctx, int32_t lane, int32_t* loops) {
  tl_status st = check_lane(ctx, lane);
  if (st != TL_OK) return st;
  if (!loops) return fail(TL_E_INVAL, "loops is NULL");
  *loops = ctx->loops[lane];
  return TL_OK;
}

tl_status tl_reset(tl_ctx* ctx, int32_t lane) {
  if (!ctx) return fail(TL_E_INVAL, "ctx is NULL");
  if (lane < -1 || lane >= ctx->cfg.n_lanes) return fail(TL_E_INVAL, "lane index out of range");
  const int lo = lane < 0 ? 0 : lane, hi = lane < 0 ? ctx->cfg.n_lanes : lane + 1;
  for (int l = lo; l < hi; ++l) {
    ctx->len[l] = 0;
    ctx->depth[l] = INT_MAX;
  }
  ctx->dpos_synced = false;
  return TL_OK;
}

int32_t tl_length(const tl_ctx* ctx, int32_t lane) {
  if (!ctx || lane < 0 || lane >= ctx->cfg.n_lanes) return -1;
  return ctx->len[lane];
}

}  // extern "C"

namespace {

// The launches of one prefill call (the state update is the caller's).
tl_status enqueue_prefill(tl_ctx* ctx, int lane, const int32_t* d_tokens, int n, float* d_hidden, float* d_logits,
                          int32_t* d_next, int p0, int L, hipStream_t s, bool head_all_rows = false) {
  const tl_config& C = ctx->cfg;
  tl_status st;
  tl::RowMap rm{};
  rm.per_row = 0;
  rm.lane = lane;
  rm.p0 = p0;
  const int d = C.d_model;
  const bool safe = ctx->safety_max > 0.f;
  ctx->h_ready = false;
  ctx->emb_tokens = nullptr;
  ctx->pend = tl::Pending{nullptr, 1};  // nothing carries over from an earlier call
  if (safe) {
    KScope k(ctx, TL_K_SAFETY, s);
    TL_HIP(tl::launch_safety_reset(ctx->safety_res, s));
  }
  // embedding gather; when the first layer's QKV runs as a GEMM (n > 8 rows,
  // K/V stored), fused with that layer's RMSNorm
  const tl::ASrc first{nullptr, ctx->x, ctx->blocks[0].attn_norm, C.rms_eps};
  if (C.n_pre + L > 0 && !ctx->hmode && !tl::gemv_supported(n, d, first)) {
    KScope k(ctx, TL_K_EMBED, s);
    TL_HIP(tl::launch_embed_rmsnorm(ctx->embed, d_tokens, C.vocab, n, d, ctx->x, ctx->blocks[0].attn_norm, C.rms_eps,
                                    ctx->h, s));
    ctx->h_ready = true;
  } else if (C.n_pre + L > 0 && !ctx->hmode) {
    ctx->emb_tokens = d_tokens;  // the first layer's QKV GEMV gathers the rows
    ctx->emb_rm = rm;
  } else {
    KScope k(ctx, TL_K_EMBED, s);
    TL_HIP(tl::launch_embed(ctx->embed, d_tokens, n, rm, d, C.vocab, ctx->x, s));
  }
  for (int layer = 0; layer < C.n_pre + L; ++layer) {
    const BlockW& B = ctx->blocks[std::min(layer, C.n_pre)];
    st = run_layer(ctx, B, layer, n, rm, false, s);
    if (st != TL_OK) return st;
    if (safe && layer >= C.n_pre) {
      KScope k(ctx, TL_K_SAFETY, s);
      TL_HIP(tl::launch_safety_check(ctx->x, ctx->pend, n, d, ctx->safety_max, (layer - C.n_pre) << tl::kSafetyRowBits,
                                     ctx->safety_res, s));
    }
  }
  st = resolve(ctx, n, s);
  if (st != TL_OK) return st;
  if (d_hidden) {
    KScope k(ctx, TL_K_COPY, s);
    TL_HIP(hipMemcpyAsync(d_hidden, ctx->x, (size_t)n * d * 4, hipMemcpyDeviceToDevice, s));
  }
  if (d_logits || d_next) {
    // the last row, or every row (n <= the head's row limit): logits row m
    // at lg + m * vocab, argmax at d_next[m]
    float* lg = d_logits ? d_logits : ctx->logits;
    tl::RowMap one{};
    const int rows = head_all_rows ? n : 1;
    {
      KScope k(ctx, TL_K_HEAD, s);
      TL_HIP(tl::launch_head(ctx->x + (size_t)(n - rows) * d, rows, ctx->final_norm, C.rms_eps, ctx->head, C.vocab,
                             d, lg, one, ctx->hscr, s));
    }
    if (d_next) {
      KScope k(ctx, TL_K_ARGMAX, s);
      TL_HIP(tl::launch_argmax(rows, C.vocab, one, ctx->hscr, d_next, s));
    }
  }
  return TL_OK;
}

// Reads the safety check's result (one synchronisation of the stream). rows,
// if given, maps a result row to the lane reported.
tl_status safety_verdict(tl_ctx* ctx, hipStream_t s, const std::vector<int>* rows) {
  hipError_t e = hipMemcpyAsync(&ctx->safety_host, ctx->safety_res, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(TL_E_HIP, std::string("reading the safety check: ") + hipGetErrorString(e));
  const int code = ctx->safety_host;
  if (code == 0x7fffffff) return TL_OK;
  const int it = code >> tl::kSafetyRowBits, row = code & ((1 << tl::kSafetyRowBits) - 1);
  ctx->safety_iter = it;
  ctx->safety_row = rows ? (*rows)[row] : row;
  return fail(TL_E_SAFETY, "residual norm above the safety threshold after loop iteration " + std::to_string(it) +
                               (rows ? " on lane " : " on row ") + std::to_string(ctx->safety_row));
}

void drop_prefill_graph(tl_ctx* ctx) {
  if (ctx->pg.exec) {
    (void)hipEventSynchronize(ctx->pg_done);  // the last replay may still run
    (void)hipGraphExecDestroy(ctx->pg.exec);
  }
  ctx->pg = tl_ctx::PrefillGraph{};
}

// The launches of one decode step over `rows` (the state update is the
// caller's). replay: the step is being captured for graph replay, so the
// decode attention reads the positions from ctx->dpos and a last kernel
// advances them.
tl_status enqueue_decode(tl_ctx* ctx, const std::vector<int>& rows, tl::RowMap rm, const int32_t* d_tokens,
                         float* d_hidden, float* d_logits, int32_t* d_next, hipStream_t s, bool replay) {
  const tl_config& C = ctx->cfg;
  const int M = (int)rows.size(), d = C.d_model;
  const bool safe = ctx->safety_max > 0.f;
  if (replay) rm.dpos = ctx->dpos;
  ctx->h_ready = false;
  ctx->emb_tokens = nullptr;
  ctx->pend = tl::Pending{nullptr, 1};  // nothing carries over from an earlier call
  if (safe) {
    KScope k(ctx, TL_K_SAFETY, s);
    TL_HIP(tl::launch_safety_reset(ctx->safety_res, s));
  }
  const int Lmax = ctx->loops[rows[0]];
  if (C.n_pre + Lmax > 0 && !ctx->hmode) {
    ctx->emb_tokens = d_tokens;  // the first layer's QKV GEMV gathers the rows
    ctx->emb_rm = rm;
  } else {
    KScope k(ctx, TL_K_EMBED, s);
    TL_HIP(tl::launch_embed(ctx->embed, d_tokens, M, rm, d, C.vocab, ctx->x, s));
  }
  for (int layer = 0; layer < C.n_pre + Lmax; ++layer) {
    int Ml = 0;
    while (Ml < M && C.n_pre + ctx->loops[rows[Ml]] > layer) ++Ml;
    const BlockW& B = ctx->blocks[std::min(layer, C.n_pre)];
    tl_status st = run_layer(ctx, B, layer, Ml, rm, true, s);
    if (st != TL_OK) return st;
    if (safe && layer >= C.n_pre) {
      KScope k(ctx, TL_K_SAFETY, s);
      TL_HIP(tl::launch_safety_check(ctx->x, ctx->pend, Ml, d, ctx->safety_max,
                                     (layer - C.n_pre) << tl::kSafetyRowBits, ctx->safety_res, s));
    }
  }
  if (d_logits || d_next) {
    float* lg = d_logits ? d_logits : ctx->logits;
    {
      KScope k(ctx, TL_K_HEAD, s);
      TL_HIP(tl::launch_head(ctx->x, M, ctx->final_norm, C.rms_eps, ctx->head, C.vocab, d, lg, rm, ctx->hscr, s));
    }
  }
  if (d_hidden) {
    KScope k(ctx, TL_K_COPY, s);
    TL_HIP(tl::launch_scatter_rows(ctx->x, M, d, rm, d_hidden, s));
  }
  // argmax last: a replayed step advances the device positions in it
  if (d_next) {
    KScope k(ctx, TL_K_ARGMAX, s);
    TL_HIP(tl::launch_argmax(M, C.vocab, rm, ctx->hscr, d_next, s, replay ? ctx->dpos : nullptr));
  } else if (replay) {
    KScope k(ctx, TL_K_COPY, s);
    TL_HIP(tl::launch_advance_pos(ctx->dpos, rm, M, s));
  }
  return TL_OK;
}

constexpr int kMaxDecodeGraphs = 4;  // e.g. alternating token buffers, or a few lane sets

void drop_decode_graphs(tl_ctx* ctx) {
  for (auto& g : ctx->dgraphs) {
    if (g.done) (void)hipEventSynchronize(g.done);  // its last replay may still run
    if (g.exec) (void)hipGraphExecDestroy(g.exec);
    if (g.done) (void)hipEventDestroy(g.done);
  }
  ctx->dgraphs.clear();
}

// One decode step from a captured graph. The graph is keyed by everything
// its launches depend on except the lane positions: the rows (lanes, in
// order) and their L, the decode attention's launch shape (grid, block width
// and parts per row, which change every 128 or 256 keys) and the caller's
// pointers. The positions are read on the device from ctx->dpos, which the
// host sets only when its own view changed since the last replay (prefill,
// reset, eager steps); each replay advances them itself.
tl_status decode_graph_launch(tl_ctx* ctx, const std::vector<int>& rows, const tl::RowMap& rm,
                              const int32_t* d_tokens, float* d_hidden, float* d_logits, int32_t* d_next,
                              hipStream_t s) {
  const int M = (int)rows.size();
  std::vector<long long> key;
  key.push_back(M);
  for (int m = 0; m < M; ++m) {
    key.push_back(rows[m]);
    key.push_back(ctx->loops[rows[m]]);
  }
  int shape[3 + 2 * 8];
  tl::attn_decode_shape(M, rm, ctx->kv, shape);
  key.insert(key.end(), shape, shape + 3 + 2 * M);
  for (const void* p : {(const void*)d_tokens, (const void*)d_hidden, (const void*)d_logits, (const void*)d_next})
    key.push_back((long long)reinterpret_cast<uintptr_t>(p));
  if (!ctx->dpos_synced) {
    tl::PosArgs a{};
    a.n = ctx->cfg.n_lanes;
    for (int l = 0; l < a.n; ++l) a.v[l] = ctx->len[l];
    KScope k(ctx, TL_K_COPY, s);
    TL_HIP(tl::launch_set_pos(ctx->dpos, a, s));
    ctx->dpos_synced = true;
  }
  tl_ctx::DecodeGraph* g = nullptr;
  for (auto& e : ctx->dgraphs)
    if (e.key == key) g = &e;
  if (!g) {
    if (!ctx->cap_stream) TL_HIP(hipStreamCreateWithFlags(&ctx->cap_stream, hipStreamNonBlocking));
    hipGraph_t graph = nullptr;
    TL_HIP(hipStreamBeginCapture(ctx->cap_stream, hipStreamCaptureModeThreadLocal));
    tl_status st = enqueue_decode(ctx, rows, rm, d_tokens, d_hidden, d_logits, d_next, ctx->cap_stream, true);
    const hipError_t ce = hipStreamEndCapture(ctx->cap_stream, &graph);
    if (st != TL_OK || ce != hipSuccess) {
      if (graph) (void)hipGraphDestroy(graph);
      return st != TL_OK ? st : fail(TL_E_HIP, std::string("decode graph capture: ") + hipGetErrorString(ce));
    }
    tl_ctx::DecodeGraph e;
    const hipError_t ie = hipGraphInstantiate(&e.exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (ie != hipSuccess) return fail(TL_E_HIP, std::string("decode graph instantiate: ") + hipGetErrorString(ie));
    const hipError_t ee = hipEventCreateWithFlags(&e.done, hipEventDisableTiming);
    if (ee != hipSuccess) {
      (void)hipGraphExecDestroy(e.exec);
      return fail(TL_E_HIP, std::string("hipEventCreate: ") + hipGetErrorString(ee));
    }
    e.key = std::move(key);
    if ((int)ctx->dgraphs.size() >= kMaxDecodeGraphs) {  // evict the least recently replayed
      auto lru = std::min_element(ctx->dgraphs.begin(), ctx->dgraphs.end(),
                                  [](const tl_ctx::DecodeGraph& a, const tl_ctx::DecodeGraph& b) { return a.used < b.used; });
      (void)hipEventSynchronize(lru->done);
      (void)hipGraphExecDestroy(lru->exec);
      (void)hipEventDestroy(lru->done);
      ctx->dgraphs.erase(lru);
    }
    ctx->dgraphs.push_back(std::move(e));
    g = &ctx->dgraphs.back();
  }
  g->used = ++ctx->dgraph_clock;
  TL_HIP(hipGraphLaunch(g->exec, s));
  TL_HIP(hipEventRecord(g->done, s));
  return TL_OK;
}

}  // namespace

extern "C" {

tl_status tl_prefill(tl_ctx* ctx, int32_t lane, const int32_t* d_tokens, int32_t n, float* d_hidden,
                     float* d_logits, int32_t* d_next, void* stream) {
  tl_status st = check_lane(ctx, lane);
  if (st != TL_OK) return st;
  if (!d_tokens) return fail(TL_E_INVAL, "d_tokens is NULL");
  const tl_config& C = ctx->cfg;
  if (n < 1 || n > C.max_tokens) return fail(TL_E_RANGE, "n outside 1..max_tokens");
  const int p0 = ctx->len[lane];
  if (p0 + n > C.max_seq) return fail(TL_E_RANGE, "prefill would exceed max_seq");
  const int L = ctx->loops[lane];
  if (p0 > 0 && C.n_pre + L > ctx->depth[lane]) return fail(TL_E_STATE, "lane's L is deeper than its cache");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  ctx->dpos_synced = false;  // the lane's length changes
  if (!(ctx->graph_mask & 1) || ctx->prof_on || ctx->safety_max > 0.f) {
    st = enqueue_prefill(ctx, lane, d_tokens, n, d_hidden, d_logits, d_next, p0, L, s);
    if (st != TL_OK) return st;
  } else {
    auto& g = ctx->pg;
    const bool same = g.valid && g.lane == lane && g.n == n && g.p0 == p0 && g.loops == L && g.tokens == d_tokens &&
                      g.hidden == d_hidden && g.logits == d_logits && g.next == d_next;
    if (!same) {
      drop_prefill_graph(ctx);
      if (!ctx->cap_stream) TL_HIP(hipStreamCreateWithFlags(&ctx->cap_stream, hipStreamNonBlocking));
      if (!ctx->pg_done) TL_HIP(hipEventCreateWithFlags(&ctx->pg_done, hipEventDisableTiming));
      hipGraph_t graph = nullptr;
      TL_HIP(hipStreamBeginCapture(ctx->cap_stream, hipStreamCaptureModeThreadLocal));
      st = enqueue_prefill(ctx, lane, d_tokens, n, d_hidden, d_logits, d_next, p0, L, ctx->cap_stream);
      const hipError_t ce = hipStreamEndCapture(ctx->cap_stream, &graph);
      if (st != TL_OK || ce != hipSuccess) {
        if (graph) (void)hipGraphDestroy(graph);
        return st != TL_OK ? st : fail(TL_E_HIP, std::string("graph capture: ") + hipGetErrorString(ce));
      }
      const hipError_t ie = hipGraphInstantiate(&g.exec, graph, nullptr, nullptr, 0);
      (void)hipGraphDestroy(graph);
      if (ie != hipSuccess) {
        g.exec = nullptr;
        return fail(TL_E_HIP, std::string("graph instantiate: ") + hipGetErrorString(ie));
      }
      g.valid = true;
      g.lane = lane;
      g.n = n;
      g.p0 = p0;
      g.loops = L;
      g.tokens = d_tokens;
      g.hidden = d_hidden;
      g.logits = d_logits;
      g.next = d_next;
    }
    TL_HIP(hipGraphLaunch(g.exec, s));
    TL_HIP(hipEventRecord(ctx->pg_done, s));
  }
  ctx->len[lane] = p0 + n;
  ctx->depth[lane] = std::min(ctx->depth[lane], C.n_pre + L);
  if (ctx->safety_max > 0.f) return safety_verdict(ctx, s, nullptr);
  return TL_OK;
}

tl_status tl_set_safety(tl_ctx* ctx, float max_norm) {
  if (!ctx) return fail(TL_E_INVAL, "ctx is NULL");
  if (!(max_norm >= 0.f)) return fail(TL_E_RANGE, "max_norm must be >= 0 (0: off)");
  ctx->safety_max = max_norm;
  ctx->safety_iter = ctx->safety_row = -1;
  return TL_OK;
}

tl_status tl_safety_last(const tl_ctx* ctx, int32_t* iteration, int32_t* row) {
  if (!ctx || !iteration || !row) return fail(TL_E_INVAL, "NULL argument");
  *iteration = ctx->safety_iter;
  *row = ctx->safety_row;
  return TL_OK;
}

tl_status tl_set_graphs(tl_ctx* ctx, int32_t enable) {
  if (!ctx) return fail(TL_E_INVAL, "ctx is NULL");
  if (enable < 0 || enable > 3) return fail(TL_E_RANGE, "enable must be 0..3 (bit 0 prefill, bit 1 decode)");
  ctx->graph_mask = enable;
  if (!(enable & 1)) drop_prefill_graph(ctx);
  if (!(enable & 2)) drop_decode_graphs(ctx);
  return TL_OK;
}

tl_status tl_decode_step(tl_ctx* ctx, const int32_t* d_tokens, const uint8_t* h_active, float* d_hidden,
                         float* d_logits, int32_t* d_next, void* stream) {
  if (!ctx) return fail(TL_E_INVAL, "ctx is NULL");
  if (!d_tokens) return fail(TL_E_INVAL, "d_tokens is NULL");
  const tl_config& C = ctx->cfg;
  std::vector<int> rows;
  for (int l = 0; l < C.n_lanes; ++l)
    if (!h_active || h_active[l]) rows.push_back(l);
  for (int l : rows) {
    if (ctx->len[l] < 1) return fail(TL_E_STATE, "decode on a lane with no cached token");
    if (ctx->len[l] >= C.max_seq) return fail(TL_E_RANGE, "lane is at max_seq");
    if (C.n_pre + ctx->loops[l] > ctx->depth[l]) return fail(TL_E_STATE, "lane's L is deeper than its cache");
  }
  if (rows.empty()) return TL_OK;
  std::stable_sort(rows.begin(), rows.end(), [&](int a, int b) { return ctx->loops[a] > ctx->loops[b]; });
  const int M = (int)rows.size();
  tl::RowMap rm{};
  rm.per_row = 1;
  for (int m = 0; m < M; ++m) {
    rm.row_lane[m] = rows[m];
    rm.row_pos[m] = ctx->len[rows[m]];
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool safe = ctx->safety_max > 0.f;
  // graph replay (tl_set_graphs bit 1) unless a timing window or the safety
  // check is on, the cache is store-h (its launch shapes change every step)
  // or a self-speculative round is drafting
  const bool replay = (ctx->graph_mask & 2) && !ctx->prof_on && !safe && !ctx->hmode && !ctx->force_eager;
  tl_status st = replay ? decode_graph_launch(ctx, rows, rm, d_tokens, d_hidden, d_logits, d_next, s)
                        : enqueue_decode(ctx, rows, rm, d_tokens, d_hidden, d_logits, d_next, s, false);
  if (st != TL_OK) return st;
  if (!replay) ctx->dpos_synced = false;  // eager steps do not advance the device positions
  for (int l : rows) {
    ctx->len[l] += 1;
    ctx->depth[l] = std::min(ctx->depth[l], C.n_pre + ctx->loops[l]);
  }
  if (safe) return safety_verdict(ctx, s, &rows);
  return TL_OK;
}

// Self-speculative greedy decode of one lane: draft with cached decode steps
// at draft_loops, verify with one appended prefill of the k + 1 tokens at
// the lane's own L, every row's greedy token from the head; accept drafts up
// to the first that differs from the verifier's token, then emit the
// verifier's token there. The cache is shared: verification rewrites the
// drafted positions at full depth and the length is set back past the
// accepted ones.
tl_status tl_spec_decode(tl_ctx* ctx, int32_t lane, int32_t token, int32_t draft_loops, int32_t k_draft,
                         int32_t n_new, int32_t* h_out, tl_spec_stats* stats, void* stream) {
  tl_status st = check_lane(ctx, lane);
  if (st != TL_OK) return st;
  const tl_config& C = ctx->cfg;
  if (!h_out && n_new > 0) return fail(TL_E_INVAL, "h_out is NULL");
  if (token < 0 || token >= C.vocab) return fail(TL_E_RANGE, "token outside 0..vocab-1");
  const int Lv = ctx->loops[lane];
  if (draft_loops < 1 || draft_loops > Lv) return fail(TL_E_RANGE, "draft_loops outside 1..L of the lane");
  if (k_draft < 1 || k_draft > kSpecMaxDraft || k_draft + 1 > C.max_tokens)
    return fail(TL_E_RANGE, "k_draft outside 1..min(7, max_tokens - 1)");
  if (ctx->len[lane] < 1) return fail(TL_E_STATE, "speculative decode on a lane with no cached token");
  if (C.n_pre + Lv > ctx->depth[lane]) return fail(TL_E_STATE, "lane's L is deeper than its cache");
  if (n_new > 0 && ctx->len[lane] >= C.max_seq) return fail(TL_E_RANGE, "lane is at max_seq");
  if (ctx->prof_on) return fail(TL_E_STATE, "not inside a timing window");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  tl_spec_stats acc{0, 0, 0, 0};
  const int nl = C.n_lanes;
  std::vector<uint8_t> active(nl, 0);
  active[lane] = 1;
  int32_t* chain = ctx->spec_chain;  // row i: the token decode step i consumes, at [lane]
  ctx->spec_host[0] = token;
  TL_HIP(hipMemcpyAsync(chain + lane, ctx->spec_host, 4, hipMemcpyHostToDevice, s));
  const int depth0 = ctx->depth[lane];
  int emitted = 0;
  while (emitted < n_new) {
    const int p = ctx->len[lane];
    if (p >= C.max_seq) {
      st = fail(TL_E_RANGE, "lane reached max_seq");
      break;
    }
    const int k = std::min(k_draft, C.max_seq - p - 1);  // positions p .. p+k must fit
    // draft: k cached decode steps at draft_loops (plain launches: each step
    // reads another row of the token chain, which a graph would key on)
    ctx->loops[lane] = draft_loops;
    ctx->force_eager = true;
    for (int i = 0; i < k && st == TL_OK; ++i)
      st = tl_decode_step(ctx, chain + (size_t)i * nl, active.data(), nullptr, nullptr, chain + (size_t)(i + 1) * nl,
                          stream);
    ctx->force_eager = false;
    ctx->loops[lane] = Lv;
    // verify: tokens t0..tk as one prefill at p with the head on every row
    // (after a failure: the drafted rows are dropped the same way)
    ctx->len[lane] = p;
    ctx->depth[lane] = depth0;
    if (st != TL_OK) break;
    hipError_t he = hipMemcpy2DAsync(ctx->spec_ver, 4, chain + lane, (size_t)nl * 4, 4, k + 1,
                                     hipMemcpyDeviceToDevice, s);
    if (he != hipSuccess) {
      st = fail(TL_E_HIP, std::string("hipMemcpy2DAsync: ") + hipGetErrorString(he));
      break;
    }
    st = enqueue_prefill(ctx, lane, ctx->spec_ver, k + 1, nullptr, nullptr, ctx->spec_next, p, Lv, s, true);
    if (st != TL_OK) break;
    int32_t* hv = ctx->spec_host;  // [0, k]: t0..tk, [8, 8+k]: v0..vk
    he = hipMemcpyAsync(hv, ctx->spec_ver, (size_t)(k + 1) * 4, hipMemcpyDeviceToHost, s);
    if (he == hipSuccess) he = hipMemcpyAsync(hv + 8, ctx->spec_next, (size_t)(k + 1) * 4, hipMemcpyDeviceToHost, s);
    if (he == hipSuccess) he = hipStreamSynchronize(s);
    if (he != hipSuccess) {
      st = fail(TL_E_HIP, std::string("reading the verify tokens: ") + hipGetErrorString(he));
      break;
    }
    if (ctx->safety_max > 0.f) {  // the verify pass tripped the check: keep nothing of this round
      st = safety_verdict(ctx, s, nullptr);
      if (st != TL_OK) break;
    }
    int a = 0;
    while (a < k && hv[1 + a] == hv[8 + a]) ++a;
    // emitted this round: t1..ta, then v_a; the cache keeps t0..t(r-1)
    const int r = std::min(a + 1, n_new - emitted);
    for (int j = 0; j < r; ++j) h_out[emitted + j] = j < a ? hv[1 + j] : hv[8 + a];
    emitted += r;
    ctx->len[lane] = p + r;
    acc.rounds += 1;
    acc.drafted += k;
    acc.accepted += a;
    // the next round starts from the last emitted token (not cached)
    if (emitted < n_new) {
      he = hipMemcpyAsync(chain + lane, ctx->spec_next + a, 4, hipMemcpyDeviceToDevice, s);
      if (he != hipSuccess) {
        st = fail(TL_E_HIP, std::string("hipMemcpyAsync: ") + hipGetErrorString(he));
        break;
      }
    }
  }
  ctx->loops[lane] = Lv;
  ctx->depth[lane] = depth0;
  ctx->dpos_synced = false;  // the lane's length was set back and forth
  acc.emitted = emitted;
  if (stats) *stats = acc;
  return st;
}

tl_status tl_profile_begin(tl_ctx* ctx, int32_t max_launches) {
  if (!ctx) return fail(TL_E_INVAL, "ctx is NULL");
  if (ctx->prof_on) return fail(TL_E_STATE, "a timing window is already open");
  if (max_launches < 1 || max_launches > 1000000) return fail(TL_E_RANGE, "max_launches outside 1..1000000");
  ctx->prof_ev.assign((size_t)2 * max_launches, nullptr);
  for (auto& e : ctx->prof_ev) {
    hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) {
      for (auto& x : ctx->prof_ev)
        if (x) (void)hipEventDestroy(x);
      ctx->prof_ev.clear();
      return fail(TL_E_HIP, std::string("hipEventCreate: ") + hipGetErrorString(err));
    }
  }
  ctx->prof_kind.assign(max_launches, 0);
  ctx->timer = tl::LaunchTimer{ctx->prof_ev.data(), ctx->prof_kind.data(), max_launches, 0, 0};
  ctx->prof_on = true;
  return TL_OK;
}

tl_status tl_profile_end(tl_ctx* ctx, double* total_ms, int32_t* count) {
  if (!ctx) return fail(TL_E_INVAL, "ctx is NULL");
  if (!ctx->prof_on) return fail(TL_E_STATE, "no timing window is open");
  if (!total_ms || !count) return fail(TL_E_INVAL, "output arrays are NULL");
  for (int k = 0; k < TL_K_COUNT; ++k) {
    total_ms[k] = 0.0;
    count[k] = 0;
  }
  hipError_t err = hipSuccess;
  for (int i = 0; i < ctx->timer.used && err == hipSuccess; ++i) {
    err = hipEventSynchronize(ctx->prof_ev[2 * i + 1]);
    float ms = 0.f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, ctx->prof_ev[2 * i], ctx->prof_ev[2 * i + 1]);
    total_ms[ctx->prof_kind[i]] += ms;
    count[ctx->prof_kind[i]] += 1;
  }
  for (auto& e : ctx->prof_ev) (void)hipEventDestroy(e);
  ctx->prof_ev.clear();
  ctx->timer = tl::LaunchTimer{};
  ctx->prof_on = false;
  if (err != hipSuccess) return fail(TL_E_HIP, std::string("event timing: ") + hipGetErrorString(err));
  return TL_OK;
}

// ---------------------------------------------------------------- single kernels
}  // extern "C"

namespace {
__global__ void empty_kernel() {}
}  // namespace

extern "C" {

tl_status tl_launch_empty(int32_t n, void* stream) {
  if (n < 0 || n > 1000000) return fail(TL_E_RANGE, "n outside 0..1000000");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (int i = 0; i < n; ++i) hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, s);
  TL_HIP(hipGetLastError());
  return TL_OK;
}

size_t tl_qlinear_packed_bytes(int32_t N, int32_t K) {
  if (N < 16 || N % 16 || K < 8 || K % 8) return 0;
  return tl::packed_bytes(N, K);
}

tl_status tl_qlinear_pack(const uint32_t* d_qweight, const uint16_t* d_scales, int32_t N, int32_t K, void* d_packed,
                          void* stream) {
  if (N < 16 || N % 16 || K < 8 || K % 8) return fail(TL_E_INVAL, "need N % 16 == 0 and K % 8 == 0");
  if (!d_qweight || !d_scales || !d_packed || !aligned(d_packed, 256)) return fail(TL_E_INVAL, "bad pointer");
  uint8_t* t = static_cast<uint8_t*>(d_packed);
  TL_HIP(tl::launch_pack(d_qweight, d_scales, N, K, t, reinterpret_cast<uint16_t*>(t + tl::packed_tile_bytes(N, K)),
                         (K + 127) / 128, 0, 1, 0, reinterpret_cast<hipStream_t>(stream)));
  return TL_OK;
}

size_t tl_qlinear_packed_f16_bytes(int32_t N, int32_t K) {
  if (N < 16 || N % 16 || K < 8 || K % 8) return 0;
  return tl::packed_f16_bytes(N, K);
}

tl_status tl_qlinear_pack_f16(const uint32_t* d_qweight, const uint16_t* d_scales, int32_t N, int32_t K,
                              void* d_packed, void* stream) {
  if (N < 16 || N % 16 || K < 8 || K % 8) return fail(TL_E_INVAL, "need N % 16 == 0 and K % 8 == 0");
  if (!d_qweight || !d_scales || !d_packed || !aligned(d_packed, 256)) return fail(TL_E_INVAL, "bad pointer");
  TL_HIP(tl::launch_pack_f16(d_qweight, d_scales, N, K, static_cast<uint8_t*>(d_packed), (K + 127) / 128, 0, 1, 0,
                             reinterpret_cast<hipStream_t>(stream)));
  return TL_OK;
}

static tl::Packed packed_view(const void* d_packed, int N, int K) {
  tl::Packed p;
  p.tiles = static_cast<const uint8_t*>(d_packed);
  p.scales = reinterpret_cast<const uint16_t*>(p.tiles + tl::packed_tile_bytes(N, K));
  p.N = N;
  p.K = K;
  p.G = (K + 127) / 128;
  return p;
}

tl_status tl_qlinear_unpack(const void* d_packed, int32_t N, int32_t K, int8_t* d_q, uint16_t* d_scales,
                            void* stream) {
  if (N < 16 || N % 16 || K < 8 || K % 8) return fail(TL_E_INVAL, "need N % 16 == 0 and K % 8 == 0");
  if (!d_packed || !d_q || !d_scales) return fail(TL_E_INVAL, "bad pointer");
  TL_HIP(tl::launch_unpack(packed_view(d_packed, N, K), d_q, d_scales, reinterpret_cast<hipStream_t>(stream)));
  return TL_OK;
}

size_t tl_w4_linear_ws_bytes(int32_t N, int32_t K, int32_t M) {
  if (N < 16 || N % 16 || K < 8 || K % 8 || M < 1) return 0;
  return al256(tl::w4_gemm_scratch_bytes(N, K, M, false, false));
}

tl_status tl_w4_linear(const void* d_packed, int32_t N, int32_t K, const uint16_t* d_A, int32_t M, float* d_C,
                       void* d_ws, void* stream) {
  if (N < 16 || N % 16 || K < 8 || K % 8) return fail(TL_E_INVAL, "need N % 16 == 0 and K % 8 == 0");
  if (M < 1) return fail(TL_E_RANGE, "M < 1");
  if (!d_packed || !d_A || !d_C || !aligned(d_A, 16) || !aligned(d_C, 16)) return fail(TL_E_INVAL, "bad pointer");
  const tl::Packed p = packed_view(d_packed, N, K);
  const tl::Epi e{tl::EPI_STORE, d_C, nullptr, N};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (tl::gemv_supported(M, K, tl::ASrc{d_A, nullptr, nullptr, 0.f})) {
    TL_HIP(tl::launch_w4_gemv(p, tl::ASrc{d_A, nullptr, nullptr, 0.f}, M, e, s));
    return TL_OK;
  }
  const int S = tl::plan_w4_gemm(N, K, M, false, false, false).S;
  if (S > 1 && (!d_ws || !aligned(d_ws, 256))) return fail(TL_E_INVAL, "this shape needs d_ws");
  float* part = static_cast<float*>(d_ws);
  TL_HIP(tl::launch_w4_gemm(p, d_A, M, e, part, s, false));
  if (S > 1) TL_HIP(tl::launch_reduce_partials(part, S, M, N, d_C, 0, s));
  return TL_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free W4 linear
// Split-K partials of tl_w4_linear_noalloc live in this file-scope device
// array (one copy per GPU, held until the process ends). Host code never
// passes the array's name to a kernel: its per-device address comes from
// hipGetSymbolAddress, taken once per device on the first call there.
namespace {
constexpr size_t kNoallocScratchBytes = (size_t)16 << 20;
__device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

tl_status scratch_for_current_device(void** out) {
  int dev = -1;
  TL_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(TL_E_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    TL_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TL_OK;
}
}  // namespace

extern "C" {

size_t tl_w4_linear_noalloc_max_bytes(void) { return kNoallocScratchBytes; }

tl_status tl_w4_linear_noalloc(const void* d_packed, int32_t N, int32_t K, const uint16_t* d_A, int32_t M, float* d_C,
                               void* stream) {
  if (N < 16 || N % 16 || K < 8 || K % 8) return fail(TL_E_INVAL, "need N % 16 == 0 and K % 8 == 0");
  if (M < 1) return fail(TL_E_RANGE, "M < 1");
  if (!d_packed || !d_A || !d_C || !aligned(d_A, 16) || !aligned(d_C, 16)) return fail(TL_E_INVAL, "bad pointer");
  const size_t need = tl_w4_linear_ws_bytes(N, K, M);
  if (need > kNoallocScratchBytes)
    return fail(TL_E_RANGE, "this shape needs " + std::to_string(need) + " bytes of split-K scratch, above the " +
                                std::to_string(kNoallocScratchBytes) + "-byte static buffer");
  void* ws = nullptr;
  if (need > 0) {
    const tl_status st = scratch_for_current_device(&ws);
    if (st != TL_OK) return st;
  }
  return tl_w4_linear(d_packed, N, K, d_A, M, d_C, ws, stream);
}

tl_status tl_kv_quantize_rows(const uint16_t* d_x, int32_t rows, int32_t hd, int8_t* d_q, uint16_t* d_s,
                              void* stream) {
  if (rows < 1 || hd < 2 || hd > 128 || hd % 2) return fail(TL_E_INVAL, "need rows >= 1, hd even and <= 128");
  if (!d_x || !d_q || !d_s) return fail(TL_E_INVAL, "bad pointer");
  TL_HIP(tl::launch_kv_quantize_rows(d_x, rows, hd, d_q, d_s, reinterpret_cast<hipStream_t>(stream)));
  return TL_OK;
}

}  // extern "C"
