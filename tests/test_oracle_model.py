"""Pins of the oracle's forward pass (CPU only).

The pages print no forward values, so the oracle is pinned to library
implementations of the textbook pieces (PyTorch's RMSNorm, SiLU and scaled
dot-product attention; Hugging Face's Llama decoder, a pre-norm RMSNorm /
rotate-half RoPE / SwiGLU transformer), to closed forms, and to the
invariants the pages claim for this model family (cached decode equals
uncached recompute; the loop is one block's weights applied L times;
variable-L results are prefixes of each other).
"""
import copy

import numpy as np
import pytest
import torch

import oracle
import synth


def rel_rows(a, b):
    a = np.atleast_2d(a)
    b = np.atleast_2d(b)
    return float((np.abs(a - b).max(axis=-1) / np.abs(b).max(axis=-1)).max())


# ---------------------------------------------------------------- pieces
def test_fp16_rounding_is_direct_from_float64():
    one = 1.0
    tie = one + 2.0 ** -11                   # halfway between 1 and 1 + 2^-10
    assert oracle.fp16(tie) == 1.0           # ties to even
    assert oracle.fp16(tie + 2.0 ** -40) == 1.0 + 2.0 ** -10   # a float32 step would lose this
    assert oracle.fp16(1.0 + 3 * 2.0 ** -11) == 1.0 + 2 * 2.0 ** -10
    assert oracle.fp16(70000.0) == np.inf


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((5, 48)) * 3
    g = rng.uniform(0.5, 1.5, 48)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (48,), torch.from_numpy(g), eps=1e-5)
    assert np.allclose(oracle.rmsnorm(x, g, 1e-5), ref.numpy(), rtol=1e-13, atol=0)
    # scale invariance (eps aside)
    assert rel_rows(oracle.rmsnorm(1e3 * x, g, 0.0), oracle.rmsnorm(x, g, 0.0)) < 1e-14


def test_silu_matches_torch():
    z = np.linspace(-60, 60, 1001)
    assert np.allclose(oracle.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(),
                       rtol=1e-14, atol=1e-300)
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(-1000.0) == 0.0


def test_rope_is_complex_rotation():
    rng = np.random.default_rng(11)
    n, H, hd = 7, 3, 16
    x = rng.standard_normal((n, H, hd))
    pos = np.array([0, 1, 2, 5, 100, 1023, 2047])
    cos, sin = oracle.rope_cos_sin(pos, hd, 10000.0)
    y = oracle.apply_rope(x, cos, sin)
    half = hd // 2
    z = x[..., :half] + 1j * x[..., half:]
    theta = 10000.0 ** (-np.arange(half) * 2.0 / hd)
    zr = z * np.exp(1j * pos[:, None, None] * theta[None, None, :])
    assert np.allclose(y[..., :half], zr.real, atol=1e-12)
    assert np.allclose(y[..., half:], zr.imag, atol=1e-12)
    assert np.array_equal(y[0], x[0])        # position 0 is the identity


def test_rope_scores_depend_on_offset_only():
    rng = np.random.default_rng(12)
    hd = 32
    q = rng.standard_normal((1, 1, hd))
    k = rng.standard_normal((1, 1, hd))

    def score(m, n):
        cq, sq = oracle.rope_cos_sin([m], hd, 10000.0)
        ck, sk = oracle.rope_cos_sin([n], hd, 10000.0)
        return float((oracle.apply_rope(q, cq, sq) * oracle.apply_rope(k, ck, sk)).sum())

    assert abs(score(10, 3) - score(107, 100)) < 1e-10
    assert abs(score(5, 5) - score(0, 0)) < 1e-10


def _sdpa(Q, K, V, q_pos):
    S = K.shape[0]
    mask = torch.from_numpy(np.arange(S)[None, :] <= np.asarray(q_pos)[:, None])
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q.transpose(1, 0, 2)), torch.from_numpy(K.transpose(1, 0, 2)),
        torch.from_numpy(V.transpose(1, 0, 2)), attn_mask=mask)
    return out.numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("p0,n", [(0, 9), (5, 4), (12, 1)])
def test_attention_matches_torch_sdpa(p0, n):
    rng = np.random.default_rng(13 + p0)
    H, hd = 3, 16
    S = p0 + n
    Q = rng.standard_normal((n, H, hd)) * 2
    K = rng.standard_normal((S, H, hd)) * 2
    V = rng.standard_normal((S, H, hd))
    pos = p0 + np.arange(n)
    assert np.allclose(oracle.attention(Q, K, V, pos), _sdpa(Q, K, V, pos), rtol=1e-12, atol=1e-13)
    if p0 == 0:
        ref = torch.nn.functional.scaled_dot_product_attention(
            *(torch.from_numpy(a.transpose(1, 0, 2)) for a in (Q, K, V)), is_causal=True)
        assert np.allclose(oracle.attention(Q, K, V, pos), ref.numpy().transpose(1, 0, 2),
                           rtol=1e-12, atol=1e-13)


def test_attention_special_cases():
    rng = np.random.default_rng(14)
    Q = rng.standard_normal((1, 2, 8))
    K = rng.standard_normal((1, 2, 8))
    V = rng.standard_normal((1, 2, 8))
    assert np.allclose(oracle.attention(Q, K, V, [0]), V)          # one key returns V
    Q0 = np.zeros((1, 2, 8))
    K5 = rng.standard_normal((5, 2, 8))
    V5 = rng.standard_normal((5, 2, 8))
    assert np.allclose(oracle.attention(Q0, K5, V5, [4])[0], V5.mean(axis=0))   # uniform
    # future keys do not matter
    Qm = rng.standard_normal((3, 2, 8))
    a = oracle.attention(Qm, K5, V5, [0, 1, 2])
    K5b, V5b = K5.copy(), V5.copy()
    K5b[3:] += 100
    V5b[3:] -= 7
    assert np.array_equal(a, oracle.attention(Qm, K5b, V5b, [0, 1, 2]))


# ---------------------------------------------------------------- whole model vs a library transformer
def _llama_from(weights, L):
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaForCausalLM

    s = weights["shape"]
    cfg = LlamaConfig(vocab_size=s.vocab, hidden_size=s.d_model, intermediate_size=s.ffn_dim,
                      num_hidden_layers=s.n_pre + L, num_attention_heads=s.n_heads,
                      num_key_value_heads=s.n_heads, head_dim=s.head_dim, rms_norm_eps=s.rms_eps,
                      rope_theta=s.rope_base, max_position_embeddings=4096,
                      tie_word_embeddings=False, attention_bias=False, mlp_bias=False,
                      hidden_act="silu")
    cfg._attn_implementation = "eager"
    m = LlamaForCausalLM(cfg).double().eval()
    om = oracle.OracleModel(weights)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    with torch.no_grad():
        m.model.embed_tokens.weight.copy_(T(weights["embed"].astype(np.float64)))
        blocks = om.pre + [om.loop] * L
        for layer, B in zip(m.model.layers, blocks):
            layer.self_attn.q_proj.weight.copy_(T(B["wq"]))
            layer.self_attn.k_proj.weight.copy_(T(B["wk"]))
            layer.self_attn.v_proj.weight.copy_(T(B["wv"]))
            layer.self_attn.o_proj.weight.copy_(T(B["wo"]))
            layer.mlp.gate_proj.weight.copy_(T(B["w_gate"]))
            layer.mlp.up_proj.weight.copy_(T(B["w_up"]))
            layer.mlp.down_proj.weight.copy_(T(B["w_down"]))
            layer.input_layernorm.weight.copy_(T(B["attn_norm"]))
            layer.post_attention_layernorm.weight.copy_(T(B["mlp_norm"]))
        m.model.norm.weight.copy_(T(om.final_norm))
        m.lm_head.weight.copy_(T(weights["head"].astype(np.float64)))
    return m, om


@pytest.mark.parametrize("shape,L,n", [("micro", 3, 11), ("tiny", 2, 6)])
def test_uncast_model_equals_llama_with_tied_layers(shape, L, n):
    s = synth.SHAPES[shape]
    w = synth.make_weights(s, seed=3, gains="random", q_scale_mult=8.0)
    llama, om = _llama_from(w, L)
    toks = synth.make_tokens(s.vocab, n, seed=3)
    with torch.no_grad():
        out = llama(torch.from_numpy(toks.astype(np.int64))[None], output_hidden_states=True)
    r = oracle.forward(om, toks, L, casts=False, logits="all", trace=True)
    ref_logits = out.logits[0].numpy()
    # HF computes RMSNorm and the rotary angles in float32 internally
    assert rel_rows(r["logits"], ref_logits) < 1e-5
    # hidden_states[i] is the input of layer i; the last entry is after the final norm
    for i in range(1, s.n_pre + L):
        assert rel_rows(r["trace"][i - 1], out.hidden_states[i][0].numpy()) < 1e-5


def test_cast_points_stay_close_to_uncast():
    s = synth.SHAPES["tiny"]
    w = synth.make_weights(s, seed=4, gains="random")
    om = oracle.OracleModel(w)
    toks = synth.make_tokens(s.vocab, 16, seed=4)
    a = oracle.forward(om, toks, 4, casts=True, logits="all")
    b = oracle.forward(om, toks, 4, casts=False, logits="all")
    assert 0 < rel_rows(a["hidden"], b["hidden"]) < 5e-3
    assert 0 < rel_rows(a["logits"], b["logits"]) < 5e-3
    # the stored FP16 K/V rows are FP16 numbers
    k = a["cache"].k[0][:16]
    assert np.array_equal(k, k.astype(np.float16).astype(np.float64))


def _is_fp16(a):
    a = np.asarray(a, dtype=np.float64)
    return bool(np.array_equal(a, a.astype(np.float16).astype(np.float64)))


_CAST_SITES = ("h", "Q", "K", "V", "O", "h2", "a")


@pytest.mark.parametrize("kv_int8", [False, True])
def test_cast_sites_are_fp16_and_the_residual_is_not(kv_int8):
    """The definition rounds to fp16 exactly at the normed block inputs h and
    h2, Q/K/V after RoPE, the attention output O, the gated-MLP product a and
    the head input z, and keeps the residual stream in high precision (FP32
    residual: "Current Status" page, core-inference table). Every tensor at a
    cast site, as it flows on, must therefore be an fp16 number, and the
    residual after attention and after the MLP must not be (a missing cast or
    a rounded residual fails here)."""
    s = synth.SHAPES["tiny"]
    w = synth.make_weights(s, seed=5, gains="random")
    om = oracle.OracleModel(w)
    toks = synth.make_tokens(s.vocab, 24, seed=5)
    sites = []
    r = oracle.forward(om, toks, 3, logits="all", sites=sites, kv_int8=kv_int8, max_seq=32)
    assert len(sites) == s.n_pre + 3 + 1
    for layer, rec in enumerate(sites[:-1]):
        for name in _CAST_SITES:
            assert _is_fp16(rec[name]), (layer, name)
            assert np.abs(rec[name]).max() > 0, (layer, name)
        for name in ("x_attn", "x_out"):
            assert not _is_fp16(rec[name]), (layer, name)
        if kv_int8:   # attention reads f32(q) * f32(s), not the fp16 rows themselves
            kq, ks = r["cache"].kq[layer][:24], r["cache"].ks[layer][:24]
            assert np.array_equal(rec["Khat"], oracle.kv_dequantize(kq, ks))
            assert not np.array_equal(rec["Khat"], rec["K"])
    assert _is_fp16(sites[-1]["z"])
    assert np.array_equal(sites[-2]["x_out"], r["hidden"])
    # without the casts none of the sites is an fp16 number (the check has teeth)
    raw = []
    oracle.forward(om, toks, 3, logits="all", sites=raw, casts=False)
    for rec in raw[:-1]:
        for name in _CAST_SITES:
            assert not _is_fp16(rec[name]), name
    assert not _is_fp16(raw[-1]["z"])


# ---------------------------------------------------------------- loop structure invariants
@pytest.fixture(scope="module")
def tiny():
    s = synth.SHAPES["tiny"]
    w = synth.make_weights(s, seed=0, gains="random", q_scale_mult=8.0)
    return w, oracle.OracleModel(w), synth.make_tokens(s.vocab, 20, seed=0)


def _unrolled(w, L):
    """L-1 extra pre-blocks that are copies of the loop block, then L=1."""
    w2 = dict(w)
    w2["pre"] = list(w["pre"]) + [copy.deepcopy(w["loop"]) for _ in range(L - 1)]
    w2["shape"] = synth.Shape(**{**w["shape"].__dict__, "n_pre": w["shape"].n_pre + L - 1})
    return oracle.OracleModel(w2)


@pytest.mark.parametrize("L", [1, 3, 5])
def test_loop_equals_unrolled_copies(tiny, L):
    w, om, toks = tiny
    a = oracle.forward(om, toks, L, logits="all")
    b = oracle.forward(_unrolled(w, L), toks, 1, logits="all")
    assert np.array_equal(a["hidden"], b["hidden"])
    assert np.array_equal(a["logits"], b["logits"])


def test_prefix_property(tiny):
    _, om, toks = tiny
    full = oracle.forward(om, toks, 8, trace=True)
    n_pre = om.shape.n_pre
    for k in (1, 2, 5, 8):
        r = oracle.forward(om, toks, k)
        assert np.array_equal(full["trace"][n_pre + k - 1], r["hidden"])


@pytest.mark.parametrize("kv_int8", [False, True])
def test_cached_decode_equals_uncached(tiny, kv_int8):
    _, om, toks = tiny
    L = 3
    gen, logits, cache = oracle.generate_greedy(om, toks[:12], L, steps=6, max_seq=64,
                                                kv_int8=kv_int8)
    seq = list(toks[:12]) + gen
    for t in range(7):
        ref = oracle.forward_uncached(om, seq[:12 + t], L, kv_int8=kv_int8)["logits"]
        assert rel_rows(logits[t], ref) < 1e-9
    assert cache.length == 12 + 6


def test_chunked_prefill_equals_one_shot(tiny):
    _, om, toks = tiny
    one = oracle.forward(om, toks, 4, logits="all", max_seq=32)
    c = oracle.Cache(om.shape, 32)
    a = oracle.forward(om, toks[:7], 4, cache=c, logits="all")
    b = oracle.forward(om, toks[7:], 4, cache=c, logits="all")
    assert rel_rows(np.concatenate([a["hidden"], b["hidden"]]), one["hidden"]) < 1e-9


def test_int8_cache_holds_quantized_rows(tiny):
    _, om, toks = tiny
    r = oracle.forward(om, toks, 2, kv_int8=True, max_seq=32)
    c = r["cache"]
    for layer in range(om.shape.n_pre + 2):
        d = oracle.kv_dequantize(c.kq[layer][:20], c.ks[layer][:20])
        assert np.array_equal(d, c.k[layer][:20])
    assert sorted(c.k) == list(range(om.shape.n_pre + 2))   # one cache per effective layer


def test_depth_rules(tiny):
    _, om, toks = tiny
    c = oracle.Cache(om.shape, 32)
    oracle.forward(om, toks[:5], 4, cache=c)
    with pytest.raises(ValueError):
        oracle.forward(om, toks[5:6], 5, cache=c)           # deeper than cached tokens
    oracle.forward(om, toks[5:6], 2, cache=c)               # shallower is allowed
    with pytest.raises(ValueError):
        oracle.forward(om, toks, 0)
    with pytest.raises(ValueError):
        oracle.forward(om, toks, 2, cache=oracle.Cache(om.shape, 4))


def test_argmax_ties_lowest_index():
    assert int(np.argmax(np.array([1.0, 3.0, 3.0, 2.0]))) == 1
