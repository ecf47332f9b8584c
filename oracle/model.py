"""Plain float64 forward pass of the looped weight-shared transformer.

Structure ("TinyLoop Framework" intro page, opening list): embed tokens, run a
small number of pre-blocks, reuse ONE shared loop block L times, then
normalise and project to the output head. L is a runtime argument ("What
Makes It Different": loop count is a runtime knob; weight memory is tied to
unique blocks, not effective depth). Every pre-block and every loop iteration
is an effective layer with its own KV cache ("Performance and Memory" page,
INT8-KV table: max_seq 2048 over 10 layers at 2 pre-blocks and L=8).

Block ("Current Status" page, model-architecture table): pre-norm RMSNorm,
rotary position embedding on q and k, full multi-head causal attention, and a
gated SiLU MLP (GeLU and post-norm are opt-in there, so not used); the
residual stream is FP32 by default (core-inference table, FP16 residual is
opt-in) and is carried here in float64.

Float16 activation cast points (a reading: FP16 activations with FP32
residual and accumulation): the normed block inputs, Q/K/V after RoPE, the
attention output and the gated-MLP product, and the final normed vector before
the head. With casts=False every cast is the identity (the pure high-precision
variant used to compare against a library transformer).

Readings where the pages are silent: RMSNorm eps 1e-5; rotate-half RoPE
pairing dimension i with i + hd/2, theta_i = base^(-2i/hd), 0-based absolute
positions; attention scale 1/sqrt(hd) with the causal mask including the
diagonal; cache layer of pre-block b is b and of loop iteration i is
n_pre + i; logits are float64 and argmax ties go to the lowest index.
"""
from __future__ import annotations

import math

import numpy as np

from .int4 import dequantize
from .kvquant import kv_quantize, kv_dequantize, h_quantize, h_dequantize, H_GROUP

_LINEARS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def fp16(a):
    """Round to nearest-even binary16 and return float64 (direct, no float32 step)."""
    with np.errstate(over="ignore"):
        return np.asarray(a, dtype=np.float64).astype(np.float16).astype(np.float64)


def _identity(a):
    return np.asarray(a, dtype=np.float64)


def rmsnorm(x, gamma, eps):
    """gamma_i * x_i / sqrt(mean(x^2) + eps) over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


def rope_cos_sin(positions, head_dim, base):
    """cos/sin [n][hd/2] of angle pos * base^(-2i/hd), in float64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang), np.sin(ang)


def apply_rope(x, cos, sin):
    """Rotate each pair (x_i, x_{i+hd/2}) of x [n][H][hd] by its angle."""
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention(Q, K, V, q_pos, window=0):
    """Causal softmax attention per head.

    Q [n][H][hd]; K, V [S][H][hd] hold cache rows 0..S-1; query m sees keys
    j <= q_pos[m], and with window W > 0 only keys j > q_pos[m] - W (the
    last W cached tokens: "Performance and Memory" page, "Sliding-Window
    Cache"; 0 means the full cache). Scores are scaled by 1/sqrt(hd); softmax
    subtracts the row maximum. Returns [n][H][hd].
    """
    n, H, hd = Q.shape
    S = K.shape[0]
    Qh = np.ascontiguousarray(Q.transpose(1, 0, 2))          # H n hd
    Kh = np.ascontiguousarray(K.transpose(1, 2, 0))          # H hd S
    Vh = np.ascontiguousarray(V.transpose(1, 0, 2))          # H S hd
    scores = np.matmul(Qh, Kh) / math.sqrt(hd)               # H n S
    masked = np.arange(S)[None, :] > np.asarray(q_pos)[:, None]
    if window > 0:
        masked |= np.arange(S)[None, :] <= np.asarray(q_pos)[:, None] - window
    scores[:, masked] = -np.inf
    scores -= scores.max(axis=-1, keepdims=True)
    p = np.exp(scores)
    p /= p.sum(axis=-1, keepdims=True)
    return np.matmul(p, Vh).transpose(1, 0, 2)               # n H hd


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


class OracleModel:
    """Dequantized float64 weights of the pre-blocks, the loop block, embed and head.

    fp16_body=True rounds every block weight q * s to float16 once, as the
    FP16 body keeps them ("Performance and Memory" page, "FP16 body cache":
    body weights dequantized to persistent FP16 at load time)."""

    def __init__(self, weights: dict, fp16_body: bool = False):
        s = weights["shape"]
        self.shape = s
        self.fp16_body = fp16_body
        self.embed = np.asarray(weights["embed"], dtype=np.float16)
        self.pre = [self._block(b) for b in weights["pre"]]
        self.loop = self._block(weights["loop"])
        self.final_norm = np.asarray(weights["final_norm"], dtype=np.float16).astype(np.float64)
        self.head16 = np.asarray(weights["head"], dtype=np.float16)
        self._head64 = None

    def _block(self, b):
        g = self.shape.group_size
        out = {name: dequantize(b[name]["qweight"], b[name]["scales"], g) for name in _LINEARS}
        if self.fp16_body:
            out = {name: w.astype(np.float16).astype(np.float64) for name, w in out.items()}
        out["attn_norm"] = np.asarray(b["attn_norm"], dtype=np.float16).astype(np.float64)
        out["mlp_norm"] = np.asarray(b["mlp_norm"], dtype=np.float16).astype(np.float64)
        return out

    @property
    def head64(self):
        if self._head64 is None:
            self._head64 = self.head16.astype(np.float64)
        return self._head64


class Cache:
    """KV cache of one lane: one K and one V store per effective layer.

    Rows hold the values attention reads: the FP16 K/V, or in INT8 mode the
    dequantized f32(q) * f32(s); the raw codes and scales are kept as well.
    depth[t] is the number of effective layers token t was computed through.
    """

    def __init__(self, shape, max_seq, kv_int8=False, window=0, store_h=False, h_int8=False):
        self.shape = shape
        self.max_seq = max_seq
        self.kv_int8 = kv_int8
        self.window = window  # cache_window: > 0 keeps only the last `window` tokens visible
        # store-h: keep the block's normed input h per position instead of K/V
        # and rebuild K, V from it with the block's own W_k, W_v when read
        self.store_h = store_h or h_int8
        if self.store_h and kv_int8:
            raise ValueError("store-h keeps h rows; INT8 K/V does not apply")
        # store-h INT8: h kept as per-128-group INT8 codes and FP16 scales
        # (kvquant.h_quantize); self.h then holds the rows K and V are rebuilt
        # from, fp16(q * s)
        self.h_int8 = h_int8
        self.h = {}
        self.hq, self.hs = {}, {}
        self.length = 0
        self.k, self.v = {}, {}
        self.kq, self.ks, self.vq, self.vs = {}, {}, {}, {}
        self.depth = np.zeros(max_seq, dtype=np.int64)

    def _store(self, d, layer, dtype, tail=()):
        if layer not in d:
            s = self.shape
            d[layer] = np.zeros((self.max_seq, s.n_heads) + tail, dtype=dtype)
        return d[layer]

    def write(self, layer, pos, K, V, raw=None):
        s = self.shape
        self._store(self.k, layer, np.float64, (s.head_dim,))[pos] = K
        self._store(self.v, layer, np.float64, (s.head_dim,))[pos] = V
        if raw is not None:
            kq, ks, vq, vs = raw
            self._store(self.kq, layer, np.int8, (s.head_dim,))[pos] = kq
            self._store(self.ks, layer, np.float16)[pos] = ks
            self._store(self.vq, layer, np.int8, (s.head_dim,))[pos] = vq
            self._store(self.vs, layer, np.float16)[pos] = vs

    def read(self, layer, upto):
        return self.k[layer][:upto], self.v[layer][:upto]

    def write_h(self, layer, pos, h):
        if layer not in self.h:
            self.h[layer] = np.zeros((self.max_seq, self.shape.d_model), dtype=np.float64)
        if self.h_int8:
            d = self.shape.d_model
            if layer not in self.hq:
                self.hq[layer] = np.zeros((self.max_seq, d), dtype=np.int8)
                self.hs[layer] = np.zeros((self.max_seq, d // H_GROUP), dtype=np.float16)
            q, s = h_quantize(np.atleast_2d(h).astype(np.float16))
            self.hq[layer][pos], self.hs[layer][pos] = q, s
            h = h_dequantize(q, s)
        self.h[layer][pos] = h


def _block_forward(x, B, cache, layer, positions, s, casts, rec=None):
    """One pre-norm block on residual rows x [n][d] at absolute positions.

    rec (a dict, optional) receives the tensors at the block's cast sites as
    they flow on: h, Q, K, V (after RoPE and the cast), O, h2, a, the
    residual after attention x_attn and after the MLP x_out, and in INT8 mode
    the K, V values attention reads (Khat, Vhat)."""
    c = fp16 if casts else _identity
    n = x.shape[0]
    H, hd = s.n_heads, s.head_dim
    h = c(rmsnorm(x, B["attn_norm"], s.rms_eps))
    q = (h @ B["wq"].T).reshape(n, H, hd)
    k = (h @ B["wk"].T).reshape(n, H, hd)
    v = (h @ B["wv"].T).reshape(n, H, hd)
    cos, sin = rope_cos_sin(positions, hd, s.rope_base)
    Q, K, V = c(apply_rope(q, cos, sin)), c(apply_rope(k, cos, sin)), c(v)
    if cache.store_h:
        # store-h ("Current Status" page, KV-cache table; "Claims & Data
        # Sources": h-mode KV reconstruction from the shared W_k / W_v): the
        # cache keeps h (FP16, or INT8 codes whose fp16(q * s) it reads back);
        # K and V of every visible position, the new ones included, are
        # rebuilt from what the cache holds; Q comes from h itself
        if cache.h_int8 and not casts:
            raise ValueError("INT8 store-h quantizes FP16 rows; it needs the FP16 cast points")
        upto = int(positions[-1]) + 1
        cache.write_h(layer, positions, h)
        hall = cache.h[layer][:upto]
        ka = (hall @ B["wk"].T).reshape(upto, H, hd)
        va = (hall @ B["wv"].T).reshape(upto, H, hd)
        ca, sa = rope_cos_sin(np.arange(upto), hd, s.rope_base)
        Kall, Vall = c(apply_rope(ka, ca, sa)), c(va)
        O = c(attention(Q, Kall, Vall, positions, cache.window)).reshape(n, H * hd)
        x1 = x + O @ B["wo"].T
        h2 = c(rmsnorm(x1, B["mlp_norm"], s.rms_eps))
        a = c(silu(h2 @ B["w_gate"].T) * (h2 @ B["w_up"].T))
        x2 = x1 + a @ B["w_down"].T
        if rec is not None:
            rec.update(h=h, Q=Q, K=K, V=V, O=O, x_attn=x1, h2=h2, a=a, x_out=x2)
        return x2
    if cache.kv_int8:
        if not casts:
            raise ValueError("INT8 KV quantizes FP16 rows; it needs the FP16 cast points")
        kq, ks = kv_quantize(K.astype(np.float16))
        vq, vs = kv_quantize(V.astype(np.float16))
        cache.write(layer, positions, kv_dequantize(kq, ks), kv_dequantize(vq, vs),
                    raw=(kq, ks, vq, vs))
    else:
        cache.write(layer, positions, K, V)
    Kall, Vall = cache.read(layer, int(positions[-1]) + 1)
    O = c(attention(Q, Kall, Vall, positions, cache.window)).reshape(n, H * hd)
    x1 = x + O @ B["wo"].T
    h2 = c(rmsnorm(x1, B["mlp_norm"], s.rms_eps))
    a = c(silu(h2 @ B["w_gate"].T) * (h2 @ B["w_up"].T))
    x2 = x1 + a @ B["w_down"].T
    if rec is not None:
        rec.update(h=h, Q=Q, K=K, V=V, O=O, x_attn=x1, h2=h2, a=a, x_out=x2)
        if cache.kv_int8:
            rec.update(Khat=Kall[positions], Vhat=Vall[positions])
    return x2


def head_logits(model, x_rows, casts=True, rec=None):
    """Final RMSNorm, cast, and the head projection: [m][d] -> [m][V] float64.
    rec (a dict, optional) receives the normed, cast head input as 'z'."""
    c = fp16 if casts else _identity
    z = c(rmsnorm(np.atleast_2d(x_rows), model.final_norm, model.shape.rms_eps))
    if rec is not None:
        rec["z"] = z
    return z @ model.head64.T


def forward(model, tokens, L, cache=None, casts=True, logits="last", trace=False,
            max_seq=None, kv_int8=False, window=0, store_h=False, h_int8=False, sites=None):
    """Append `tokens` to a lane at its current length and run all n_pre + L layers.

    Returns a dict with the final residual rows 'hidden' [n][d] (before the
    final norm), 'logits' (last position [V], all positions [n][V], or None),
    the 'cache' and, if trace, 'trace': the residual after every effective layer.
    sites (a list, optional) receives one dict per effective layer with the
    tensors at that layer's cast sites (see _block_forward), then one dict
    with the head input 'z' when logits are computed.
    """
    s = model.shape
    tokens = np.asarray(tokens, dtype=np.int64)
    n = tokens.shape[0]
    if L < 1:
        raise ValueError("L must be >= 1")
    if cache is None:
        cache = Cache(s, max_seq or max(n, 1), kv_int8=kv_int8, window=window, store_h=store_h,
                      h_int8=h_int8)
    p0 = cache.length
    if p0 + n > cache.max_seq:
        raise ValueError("sequence exceeds max_seq")
    if p0 > 0 and s.n_pre + L > int(cache.depth[:p0].min()):
        raise ValueError("earlier tokens were not computed to this depth")
    positions = p0 + np.arange(n)
    x = model.embed[tokens].astype(np.float64)
    states = []
    def rec():
        if sites is None:
            return None
        sites.append({})
        return sites[-1]

    for b in range(s.n_pre):
        x = _block_forward(x, model.pre[b], cache, b, positions, s, casts, rec())
        states.append(x)
    for i in range(L):  # the same loop-block weights on every iteration
        x = _block_forward(x, model.loop, cache, s.n_pre + i, positions, s, casts, rec())
        states.append(x)
    cache.length = p0 + n
    cache.depth[positions] = s.n_pre + L
    out = {"hidden": x, "cache": cache, "logits": None}
    if logits == "last":
        out["logits"] = head_logits(model, x[-1:], casts, rec())[0]
    elif logits == "all":
        out["logits"] = head_logits(model, x, casts, rec())
    if trace:
        out["trace"] = states
    return out


def decode_step(model, cache, token, L, casts=True):
    """Cached decode: one new token at position cache.length; next-token logits [V]."""
    r = forward(model, [int(token)], L, cache=cache, casts=casts, logits="last")
    return r["logits"], r["hidden"][0]


def forward_uncached(model, tokens, L, casts=True, kv_int8=False):
    """Uncached recompute of the whole sequence; logits of the last position."""
    return forward(model, tokens, L, cache=None, casts=casts, logits="last",
                   kv_int8=kv_int8)


def generate_greedy(model, prompt, L, steps, max_seq, kv_int8=False, casts=True, window=0):
    """Prefill the prompt, then `steps` cached decode steps, greedy (argmax).

    Returns (tokens generated: steps + 1 of them, list of logits per call:
    the prefill's last position then one per decode step, the cache).
    """
    r = forward(model, prompt, L, cache=Cache(model.shape, max_seq, kv_int8, window), casts=casts)
    cache = r["cache"]
    logits = [r["logits"]]
    toks = [int(np.argmax(r["logits"]))]
    for _ in range(steps):
        lg, _ = decode_step(model, cache, toks[-1], L, casts)
        logits.append(lg)
        toks.append(int(np.argmax(lg)))
    return toks, logits, cache
