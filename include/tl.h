/*
 * tl.h -- C ABI of the looped weight-shared transformer forward pass on
 * MI355X (gfx950).
 *
 * The model family (TinyLoop docs, "TinyLoop Framework" intro page, opening
 * list): embed tokens, run a few pre-blocks, reuse ONE shared loop block L
 * times, then final RMSNorm and the output head. L is a per-lane runtime
 * argument (same page, "What Makes It Different": loop count is a runtime
 * knob; weight memory is tied to unique blocks, not effective depth). Every
 * pre-block and every loop iteration is an "effective layer" with its own KV
 * cache ("Performance and Memory" page, INT8-KV table: 10 layers at 2
 * pre-blocks and L=8). Cached decode is the default path and an uncached
 * recompute is its parity reference ("Performance and Memory" page, "Key
 * Runtime Switches", TINYLOOP_DISABLE_KV_CACHE).
 *
 * Conventions for every call:
 *  - Device pointers ("d_" prefix) are caller-owned device memory; host
 *    pointers ("h_" prefix, and every struct passed by pointer) are host
 *    memory read during the call only. The library never allocates or frees
 *    device memory: workspace sizes come from the *_bytes queries and the
 *    caller passes the buffers in, aligned to 256 bytes.
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *    on it and the call returns without synchronising, except tl_create,
 *    which also uploads small tables and synchronises the stream once.
 *  - Every call returns a tl_status. Argument and state errors are detected
 *    on the host before anything is enqueued and leave all state unchanged;
 *    a failing HIP call returns TL_E_HIP. tl_last_error() gives a message for
 *    the last failure on the calling thread. No C++ exception crosses the ABI.
 *  - Token ids in device buffers are not checked against [0, vocab) by the
 *    host; the kernels clamp an id outside that range into it (no
 *    out-of-bounds read), and the result is then that of the clamped id.
 *  - A tl_ctx is not thread-safe. Identical calls give bit-identical results;
 *    a lane's results do not depend on which other lanes run in the same
 *    decode step.
 *  - FP16 values are passed as uint16_t bit patterns (IEEE binary16).
 */
#ifndef TL_H
#define TL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TL_OK = 0,
  TL_E_INVAL = 1,        /* bad pointer, alignment, shape or lane index */
  TL_E_RANGE = 2,        /* L, token count or sequence length out of range */
  TL_E_STATE = 3,        /* call not valid in the lane's current state */
  TL_E_HIP = 4,          /* a HIP runtime call failed */
  TL_E_UNSUPPORTED = 5,  /* valid request the library does not implement */
  TL_E_SAFETY = 6        /* the residual-norm safety check tripped (tl_set_safety) */
} tl_status;

/* TL_KV_H16 (store-h: "Current Status" page, KV-cache table; "Claims & Data
 * Sources": h-mode KV reconstruction from the shared W_k / W_v): each layer's
 * cache keeps the block's normed attention input h = fp16(RMSNorm(x)) per
 * position, half the bytes of FP16 K and V; every call rebuilds K and V of
 * the visible positions with the block's own W_k, W_v (one W4 GEMM per
 * layer, RoPE in its epilogue) into a one-layer FP16 scratch that attention
 * then reads. Prefill results are bit-identical to TL_KV_FP16 (the same
 * GEMM arithmetic produces K and V either way); decode differs from it only
 * in rounding (its stored K/V rows come from the decode GEMV there). Not
 * combinable with cache_window. */
/* TL_KV_H8 (store-h INT8, the same table's Store-h INT8 row: 66-75% less
 * memory than FP16 K/V): as TL_KV_H16, but each 128-element group of an h
 * row is kept as INT8 codes with one fp16 scale, quantized with the INT8 K/V
 * rule (scale fp16(amax / 127), codes rint(x / scale) clamped to +-127), and
 * K, V of every visible position, the call's new rows included, are rebuilt
 * from fp16(code * scale); Q comes from h itself. 74.6% less than FP16 K/V at
 * d_model = 2048. Needs d_model % 128 == 0; not combinable with
 * cache_window. */
typedef enum { TL_KV_FP16 = 0, TL_KV_INT8 = 1, TL_KV_H16 = 2, TL_KV_H8 = 3 } tl_kv_dtype;

/* Model shape and runtime limits. */
typedef struct {
  int32_t vocab, d_model, n_heads, head_dim, ffn_dim;
  int32_t n_pre;        /* number of pre-blocks (distinct weights each) */
  int32_t group_size;   /* INT4 scale group along K; must be 128 */
  float rope_base;      /* rotary base, e.g. 10000 */
  float rms_eps;        /* RMSNorm epsilon, e.g. 1e-5 */
  int32_t max_seq;      /* positions per lane (KV rows per lane and layer unless windowed) */
  int32_t max_loops;    /* largest L; KV layers per lane = n_pre + max_loops */
  int32_t n_lanes;      /* independent sequences (each with its own L and KV) */
  int32_t kv_dtype;     /* tl_kv_dtype */
  int32_t max_tokens;   /* largest token count of one tl_prefill call */
  /* Sliding-window cache ("Performance and Memory" page, "Sliding-Window
   * Cache"): 0 keeps the full cache; W > 0 keeps only the last W cached
   * tokens, i.e. a query at position q attends to positions q-W+1 .. q. The
   * cache then holds a ring of min(max_seq, W + max_tokens) rows per lane,
   * layer and head (position p in row p mod that), so KV memory no longer
   * grows with max_seq; positions still run up to max_seq. */
  int32_t cache_window;
  /* FP16 body ("Performance and Memory" page, "FP16 body cache" and "Key
   * Runtime Switches": body weights dequantized to persistent FP16 at load
   * time): 0 keeps the loop and pre-blocks as packed W4 (the default); 1
   * stores each block linear as fp16(q * s) tiles (4x the bytes, no scales)
   * and runs the same GEMM/GEMV kernels without the dequantization. */
  int32_t fp16_body;
} tl_config;

/* One INT4 linear layer in the canonical layout (device pointers):
 *   qweight uint32 [N][K/8]: element k of row n is nibble k%8 of word k/8,
 *           least significant nibble first, two's complement in [-8, 7];
 *   scales  fp16   [N][ceil(K/group_size)]; W[n][k] = q * scales[n][k/g]. */
typedef struct {
  const uint32_t* qweight;
  const uint16_t* scales;
} tl_qlinear;

/* One transformer block: pre-norm attention then pre-norm SwiGLU MLP.
 * wq, wk, wv, wo: N = K = d_model; w_gate, w_up: N = ffn, K = d_model;
 * w_down: N = d_model, K = ffn. Norm gains are fp16 [d_model]. */
typedef struct {
  const uint16_t* attn_norm;
  tl_qlinear wq, wk, wv, wo;
  const uint16_t* mlp_norm;
  tl_qlinear w_gate, w_up, w_down;
} tl_block;

typedef struct {
  const uint16_t* embed;       /* fp16 [vocab][d_model], used in place */
  const tl_block* pre;         /* host array of n_pre blocks */
  tl_block loop;               /* the shared loop block */
  const uint16_t* final_norm;  /* fp16 [d_model] */
  const uint16_t* head;        /* fp16 [vocab][d_model], repacked by tl_create */
} tl_weights;

typedef struct tl_ctx tl_ctx;

/* ---- sizes ------------------------------------------------------------- */

/* Repacked block weights, the head in MFMA tile order and the RoPE table.
 * Independent of max_loops: the loop block is stored once however many
 * times it runs. */
size_t tl_weights_ws_bytes(const tl_config* cfg);
/* K and V of one lane for one effective layer, with R = max_seq rows (or,
 * with cache_window W > 0, R = min(max_seq, W + max_tokens) ring rows):
 *   FP16: 2 * R * n_heads * head_dim * 2
 *   INT8: 2 * (A(R * n_heads * head_dim) + A(R * n_heads * 2)), A(x) = x
 *         rounded up to a multiple of 256 (codes + one fp16 scale per token
 *         and head, "Performance and Memory" page, INT8-KV; equal to
 *         2 * R * n_heads * (head_dim + 2) when R * n_heads % 128 == 0).
 *   H16:  max_seq * d_model * 2               (h rows [max_seq][d_model]).
 *   H8:   A(max_seq * d_model) + A(max_seq * d_model / 128 * 2): codes int8
 *         [max_seq][d_model] at offset 0, then the fp16 scale of each
 *         128-element group [max_seq][d_model / 128].
 * Layout per layer: K then V planes [n_heads][R][head_dim]; INT8: K codes
 * int8 [n_heads][R][head_dim] at offset 0, K scales fp16 [n_heads][R] at
 * A(codes), V codes at A(codes) + A(scales), V scales after them, every
 * plane 256-byte aligned. Position p lives in row p (p mod R with a
 * window). 0 for an invalid config. */
size_t tl_kv_layer_bytes(const tl_config* cfg);
/* n_lanes * (n_pre + max_loops) * tl_kv_layer_bytes. */
size_t tl_kv_bytes(const tl_config* cfg);
/* Activations and scratch for calls of up to max_tokens tokens. */
size_t tl_act_ws_bytes(const tl_config* cfg);

/* ---- context ----------------------------------------------------------- */

/* Validates cfg and pointers, repacks every INT4 linear of the pre-blocks and
 * the loop block into d_weights_ws (so the canonical buffers may be freed
 * afterwards), copies the head into MFMA tile order there too, and clears
 * the per-lane state. embed and the norm gains are read in place and must
 * outlive the context. d_kv holds the caches of
 * all lanes; d_act_ws the activations. Every lane starts empty with L = 1.
 * Pointers: embed, head and the norm gains 16-byte aligned; workspaces
 * 256-byte aligned.
 * Errors: TL_E_INVAL (null/misaligned pointer, head_dim not 64 or 128,
 * d_model != n_heads*head_dim, d_model not a multiple of 32 or above 2048,
 * ffn_dim not a multiple of 16, group_size != 128), TL_E_RANGE (max_loops outside 1..64, n_lanes outside
 * 1..8, max_seq or max_tokens < 1), TL_E_HIP. */
tl_status tl_create(const tl_config* cfg, const tl_weights* w, void* d_weights_ws, void* d_kv,
                    void* d_act_ws, void* stream, tl_ctx** out);
tl_status tl_destroy(tl_ctx* ctx);

/* Loop count of one lane (lane = -1: every lane). 1 <= loops <= max_loops.
 * A lane holding cached tokens may only run as deep as every cached token
 * was computed (its KV for deeper layers does not exist): TL_E_STATE if
 * n_pre + loops exceeds that depth. Host-only; enqueues nothing. */
tl_status tl_set_loops(tl_ctx* ctx, int32_t lane, int32_t loops);
tl_status tl_get_loops(const tl_ctx* ctx, int32_t lane, int32_t* loops);
/* Empties a lane (lane = -1: every lane); its L is kept. Host-only. */
tl_status tl_reset(tl_ctx* ctx, int32_t lane);
/* Cached tokens of a lane, or -1 for a bad lane index. */
int32_t tl_length(const tl_ctx* ctx, int32_t lane);

/* ---- forward ----------------------------------------------------------- */

/* Appends n tokens (d_tokens int32 [n]) to `lane` at its current length p0
 * and runs all n_pre + L effective layers over them: embed, per layer
 * RMSNorm -> W4 QKV GEMM -> RoPE -> KV write (FP16 or INT8) -> causal
 * attention over cache rows 0..p0+n-1 -> W4 O GEMM + residual -> RMSNorm ->
 * W4 gate/up GEMM + SwiGLU -> W4 down GEMM + residual.
 * Optional outputs (NULL to skip):
 *   d_hidden float [n][d_model]: final residual of every position (before
 *            the final norm);
 *   d_logits float [vocab]: head logits of the last position;
 *   d_next   int32 [1]: argmax of those logits (ties -> lowest index).
 * With d_logits and d_next both NULL the head is not run ("no logits
 * materialization", "Performance and Memory" page, benchmark shape).
 * Errors: TL_E_INVAL (bad lane or pointer), TL_E_RANGE (n < 1,
 * n > max_tokens, p0 + n > max_seq), TL_E_STATE (lane's L deeper than its
 * cached tokens).
 * Launches: eager by default. After tl_set_graphs(ctx, 1) the call's kernel
 * sequence is captured once as a HIP graph (on a stream the context owns)
 * and replayed on `stream` by later calls with the same lane, n, p0, L and
 * pointers; any other call re-captures. A replay does exactly what the
 * eager launches would (same kernels, arguments and order, no memset
 * nodes), so results are bit-identical either way. While a timing window is
 * open, calls launch eagerly. */
tl_status tl_prefill(tl_ctx* ctx, int32_t lane, const int32_t* d_tokens, int32_t n, float* d_hidden,
                     float* d_logits, int32_t* d_next, void* stream);

/* Graph capture/replay, off by default. enable is a bit mask: bit 0
 * (value 1) prefill, bit 1 (value 2) decode steps. Replay cuts the host's
 * enqueue time (about 0.2-0.5 -> 0.06 ms for the ~80 launches of a 10-layer
 * prefill; decode steps, ~52 launches, likewise) but not the GPU time, which
 * the kernels and the per-dispatch gap set.
 * Decode: a step is captured once per (active lanes in order, their L, the
 * decode attention's launch shape, which changes every 128 keys (256 beyond
 * 1024), and the d_tokens/d_hidden/d_logits/d_next pointers) and replayed
 * for later steps with the same key; up to 4 such graphs are kept (least
 * recently replayed evicted). The lane positions are then read on the device
 * from a copy in d_act_ws that each replay advances and that the call
 * re-initialises (one small kernel) when prefill, reset, an eager step or a
 * self-speculative round changed the lengths. Steps launch eagerly while a
 * timing window or the safety check is on, for store-h caches, and inside
 * tl_spec_decode's drafting. Results are bit-identical either way.
 * Switching a kind off frees its graphs after their last replay finished.
 * Errors: TL_E_INVAL (ctx NULL), TL_E_RANGE (enable outside 0..3). */
tl_status tl_set_graphs(tl_ctx* ctx, int32_t enable);

/* One cached decode step for every lane with h_active[lane] != 0 (h_active
 * NULL: all lanes). Consumes d_tokens[lane] (int32 [n_lanes], entries of
 * inactive lanes ignored) at position tl_length(lane), runs each active lane
 * through its own n_pre + L layers (loop iteration i runs only the lanes with
 * L > i, "Current Status" page, L-aware batching with per_lane_loops), then
 * final norm, head and argmax. Outputs, indexed by lane, NULL to skip:
 *   d_hidden float [n_lanes][d_model], d_logits float [n_lanes][vocab],
 *   d_next int32 [n_lanes]. Rows of inactive lanes are left untouched.
 * Errors: TL_E_INVAL, TL_E_RANGE (a lane at max_seq), TL_E_STATE (an active
 * lane with no cached token, or deeper than its cache). */
tl_status tl_decode_step(tl_ctx* ctx, const int32_t* d_tokens, const uint8_t* h_active,
                         float* d_hidden, float* d_logits, int32_t* d_next, void* stream);

/* ---- self-speculative decode -------------------------------------------
 * Greedy generation on one lane where the same weights draft at a shallow
 * depth and verify at the lane's own L ("Introduction" page, "What Makes It
 * Different": draft and verify share the weights; "Current Status" page,
 * speculative decode table: L=2 draft, L=8 verify; "Claims & Data Sources":
 * draft_loops vs verify_loops). Each round:
 *   1. drafts k = min(k_draft, max_seq - p - 1) tokens with cached decode
 *      steps at draft_loops (p = tl_length(lane) at the round's start; the
 *      first step consumes the round's input token at position p);
 *   2. verifies the input token and the k drafts in one appended prefill at
 *      p with the lane's L, taking every row's greedy token from the head;
 *   3. accepts the drafts up to the first one that differs from the
 *      verifier's token at its position, and emits them followed by the
 *      verifier's token there (all k accepted: its token after the last
 *      draft), i.e. 1..k+1 tokens, each the verifier's greedy choice.
 * The cache is shared between draft and verify: the verify prefill rewrites
 * the drafted positions at full depth and the lane's length is set back to
 * just past the accepted ones. The host reads 2(k+1) token ids per round
 * (one stream synchronisation per round).
 * token: the lane's last token, not yet in the cache (as for
 *   tl_decode_step). Exactly n_new tokens go to h_out (host int32 [n_new]);
 *   afterwards the last of them is not in the cache (the next call's token)
 *   and tl_length(lane) has grown by n_new.
 * stats (may be NULL): rounds, drafted tokens, accepted drafts, tokens
 * emitted (n_new unless an error stopped the call).
 * Errors: TL_E_INVAL (bad lane, h_out NULL with n_new > 0), TL_E_RANGE
 * (token outside the vocabulary, draft_loops outside 1..L, k_draft outside
 * 1..min(7, max_tokens - 1), the lane reaching max_seq), TL_E_STATE (lane
 * empty or deeper than its cache, or a timing window open). After an error
 * the tokens emitted so far are in h_out and the lane holds them as above. */
typedef struct {
  int32_t rounds;
  int32_t drafted;
  int32_t accepted;
  int32_t emitted;
} tl_spec_stats;
tl_status tl_spec_decode(tl_ctx* ctx, int32_t lane, int32_t token, int32_t draft_loops, int32_t k_draft,
                         int32_t n_new, int32_t* h_out, tl_spec_stats* stats, void* stream);

/* ---- per-iteration safety check ----------------------------------------
 * "Current Status" page, architecture-unique features table: the residual
 * stream's L2 norm is checked after every loop iteration and the forward is
 * stopped when it exceeds a threshold (L checkpoints per token). With
 * max_norm > 0, tl_prefill, tl_decode_step and tl_spec_decode compute, after
 * each loop iteration (not after pre-blocks), every row's ||x||_2 (x plus any
 * pending split partials) in one small kernel, and at the end of the call
 * read the first (iteration, row) whose norm is not <= max_norm (NaN trips
 * too); if there is one the call returns TL_E_SAFETY. The call's work is
 * complete when it reports (outputs written, lane length advanced, except
 * that tl_spec_decode drops a tripped round), so the caller decides: reset
 * the lane, lower L, or stop. Costs one launch per loop iteration plus one
 * stream synchronisation per call; prefill graph replay is not used while
 * it is on. max_norm 0 switches it off (the default).
 * Errors: TL_E_INVAL (ctx NULL), TL_E_RANGE (max_norm < 0 or NaN). */
tl_status tl_set_safety(tl_ctx* ctx, float max_norm);
/* The last trip since tl_set_safety: loop iteration (0-based) and row (the
 * call's row in prefill, the lane in decode), or -1, -1 if none. */
tl_status tl_safety_last(const tl_ctx* ctx, int32_t* iteration, int32_t* row);

/* Message of the last failed call on this thread ("" if none). */
const char* tl_last_error(void);

/* ---- kernel timing ------------------------------------------------------
 * For measurement ("Performance and Memory" page, "How To Publish Numbers
 * Responsibly" and the phase timings of TINYLOOP_CUDA_PROFILE): while a
 * window is open, every kernel the context launches (up to max_launches)
 * carries a pair of HIP events attached to its own dispatch
 * (hipExtLaunchKernel), so each pair spans that kernel's execution alone.
 * Windows are per context; launches are attributed on the calling thread.
 * tl_profile_end waits for the recorded events and returns, per kernel kind,
 * the number of launches and their summed durations (TL_K_COPY counts the
 * row scatter of decode hidden states; plain memory copies are not timed). */
typedef enum {
  TL_K_EMBED = 0, TL_K_NORM, TL_K_QKV, TL_K_ROPE_KV, TL_K_ATTN, TL_K_O, TL_K_GATE_UP, TL_K_DOWN,
  TL_K_HEAD, TL_K_ARGMAX, TL_K_COPY, TL_K_SAFETY, TL_K_COUNT
} tl_kernel_kind;
/* Errors: TL_E_STATE if a window is already open, TL_E_RANGE for
 * max_launches outside 1..1000000, TL_E_HIP if events cannot be created. */
tl_status tl_profile_begin(tl_ctx* ctx, int32_t max_launches);
/* total_ms double[TL_K_COUNT], count int32[TL_K_COUNT] (host arrays).
 * Errors: TL_E_STATE if no window is open, TL_E_HIP. */
tl_status tl_profile_end(tl_ctx* ctx, double* total_ms, int32_t* count);

/* Enqueues n empty kernels (one 64-thread block each) on `stream`: the
 * per-dispatch floor of the stack, against which the short kernels of the
 * forward pass are measured. Errors: TL_E_RANGE (n outside 0..1000000),
 * TL_E_HIP. */
tl_status tl_launch_empty(int32_t n, void* stream);

/* ---- single kernels ----------------------------------------------------
 * The same kernels the forward pass runs, exposed for per-kernel parity
 * tests and bandwidth/throughput measurement. */

/* Bytes of one linear in the library's packed layout: 16-row x 128-column
 * tiles of 1 KiB (MFMA fragment order, offset-binary nibbles, K padded with
 * zeros to a multiple of 128) followed by fp16 scales [N/16][ceil(K/128)][16]. */
size_t tl_qlinear_packed_bytes(int32_t N, int32_t K);
/* Repacks a canonical linear (N % 16 == 0, K % 8 == 0) into d_packed. */
tl_status tl_qlinear_pack(const uint32_t* d_qweight, const uint16_t* d_scales, int32_t N, int32_t K,
                          void* d_packed, void* stream);
/* FP16 body layout of one linear ("Performance and Memory" page, "FP16 body
 * cache": body weights dequantized to persistent FP16 at load time), the
 * form tl_create builds when cfg->fp16_body is 1: per 16-row n-block nb and
 * 128-column group g a 4 KiB tile of fp16 [4][64 lanes][8], where element j
 * of lane l in slot s is W[16 nb + l%16][128 g + 32 s + 8 (l/16) + j] =
 * fp16(q * scale), the exact product rounded once to nearest even (columns at
 * or beyond K are +0). Tiles are ordered [nb][g]. Bytes: N/16 * ceil(K/128) *
 * 4096, or 0 unless N % 16 == 0 and K % 8 == 0. */
size_t tl_qlinear_packed_f16_bytes(int32_t N, int32_t K);
/* Builds that layout from a canonical linear into d_packed (256-byte
 * aligned). Errors: TL_E_INVAL (shape or pointer), TL_E_HIP. */
tl_status tl_qlinear_pack_f16(const uint32_t* d_qweight, const uint16_t* d_scales, int32_t N, int32_t K,
                              void* d_packed, void* stream);
/* Exact inverse view of the packed layout: d_q int8 [N][K] receives the
 * signed 4-bit values, d_scales fp16 [N][ceil(K/128)] the scales. Used to
 * check the repack bit for bit. */
tl_status tl_qlinear_unpack(const void* d_packed, int32_t N, int32_t K, int8_t* d_q,
                            uint16_t* d_scales, void* stream);
/* C[m][n] = sum_k A[m][k] * W[n][k] over a packed linear, fp32 out [M][N].
 * A is fp16 [M][K] row-major; d_A and d_C 16-byte aligned (TL_E_INVAL
 * otherwise). M >= 1: M <= 8 runs the decode GEMV kernel,
 * larger M the prefill GEMM kernel with the launch plan the forward pass
 * uses for that shape (including its K split); fp32 accumulation.
 * d_ws: scratch of tl_w4_linear_ws_bytes(N, K, M) bytes (may be NULL when
 * that is 0), 256-byte aligned, owned by the caller; calls sharing one d_ws
 * must not overlap. */
size_t tl_w4_linear_ws_bytes(int32_t N, int32_t K, int32_t M);
tl_status tl_w4_linear(const void* d_packed, int32_t N, int32_t K, const uint16_t* d_A, int32_t M,
                       float* d_C, void* d_ws, void* stream);
/* Allocation-free variant of tl_w4_linear, for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). Same arguments, kernels
 * and results as tl_w4_linear, minus d_ws: split-K partials go to a static
 * device buffer inside the library, one per GPU, of
 * tl_w4_linear_noalloc_max_bytes() bytes (16 MiB), held until the process
 * ends; its address on a device is looked up on the first call made on that
 * device (make that call outside graph capture). Nothing in it has to start
 * at zero: every call writes every partial it later sums. Calls on one GPU
 * share the buffer, so calls that may overlap on one GPU (different streams
 * without ordering) race; calls on one stream do not. Calls no
 * hipMalloc/hipFree. Errors: as tl_w4_linear, plus TL_E_RANGE when
 * tl_w4_linear_ws_bytes(N, K, M) exceeds the static buffer, TL_E_HIP. */
size_t tl_w4_linear_noalloc_max_bytes(void);
tl_status tl_w4_linear_noalloc(const void* d_packed, int32_t N, int32_t K, const uint16_t* d_A, int32_t M,
                               float* d_C, void* stream);
/* Per-row symmetric INT8 quantizer of the KV cache (bit-exact definition:
 * amax = max|x|; s = fp16(amax / 127) with a correctly rounded float32
 * division; q = clamp(rint_half_even(x / float(s)), -127, 127), 0 if s == 0).
 * d_x fp16 [rows][hd] -> d_q int8 [rows][hd], d_s fp16 [rows]. hd <= 128,
 * hd % 2 == 0. */
tl_status tl_kv_quantize_rows(const uint16_t* d_x, int32_t rows, int32_t hd, int8_t* d_q,
                              uint16_t* d_s, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TL_H */
