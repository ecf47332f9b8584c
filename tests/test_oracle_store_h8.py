"""Pins of the oracle's INT8 store-h cache (CPU only).

"Current Status" page, KV-cache table: Store-h (INT8) keeps the block's
normed input h instead of K and V, 66-75% smaller than FP16 K/V. The oracle
reads it as per-128-element-group INT8 (the INT8 K/V rule per group) with K and
V rebuilt from fp16(q * s). Pinned here by hand-worked values (the fp16 cast
of the product, ties to even, subnormal scales; two groups that must not mix),
an exact round trip on representable rows, the per-element error bound, the
page's memory range, and the forward pass's use of the cache.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from tests.conftest import GOLDEN

G = json.load(open(os.path.join(GOLDEN, "h_int8_worked.json")))


@pytest.mark.parametrize("case", G["dequant"], ids=lambda c: str(c["q"]))
def test_worked_products(case):
    q = np.zeros((1, 128), np.int8)
    q[0, 0] = case["q"]
    s = np.array([[case["s"]]], np.float16)
    assert float(s[0, 0]) == case["s"]
    assert oracle.h_dequantize(q, s)[0, 0] == case["hhat"]


def test_groups_are_128_consecutive_elements():
    g = G["groups"]
    x = np.zeros((1, g["d"]), np.float16)
    for k, v in g["x"].items():
        x[0, int(k)] = v
    q, s = oracle.h_quantize(x)
    assert s.shape == (1, g["d"] // 128)
    assert [float(v) for v in s[0]] == g["scales"]
    for k, v in g["codes"].items():
        assert q[0, int(k)] == v
    assert np.count_nonzero(q) == len(g["codes"])


def test_round_trip_is_exact_on_representable_rows():
    """Rows whose every group is c * 2^-e with a code of magnitude 127 in it
    quantize to exactly (c, 2^-e) and read back unchanged."""
    rng = np.random.default_rng(3)
    n, d = 40, 512
    c = rng.integers(-127, 128, (n, d))
    c[:, ::128] = 127 * rng.choice([-1, 1], (n, d // 128))  # amax = 127 * scale in every group
    e = rng.integers(2, 14, (n, d // 128))
    scale = np.ldexp(1.0, -e)
    h = (c.reshape(n, d // 128, 128) * scale[..., None]).reshape(n, d)
    assert np.array_equal(h.astype(np.float16).astype(np.float64), h)
    q, s = oracle.h_quantize(h.astype(np.float16))
    assert np.array_equal(q, c) and np.array_equal(s.astype(np.float64), scale)
    assert np.array_equal(oracle.h_dequantize(q, s), h)


def test_error_bound():
    """|h - h^| <= s/2 (the code's rounding) + half an fp16 ulp of h^ (the cast)."""
    rng = np.random.default_rng(4)
    for spread in (1e-3, 1.0, 40.0):
        h = (rng.standard_normal((300, 2048)) * spread).astype(np.float16)
        q, s = oracle.h_quantize(h)
        hh = oracle.h_dequantize(q, s)
        s64 = np.repeat(s.astype(np.float64), 128, axis=1)
        ulp = np.spacing(np.abs(hh).astype(np.float16)).astype(np.float64)
        assert (np.abs(h.astype(np.float64) - hh) <= s64 / 2 + ulp / 2 + 1e-300).all()
        assert np.abs(q).max() == 127


def test_memory_saving_within_the_pages_ranges():
    layers, S, d, H, hd = 10, 2048, 2048, 16, 128
    kv = oracle.kv_cache_bytes(layers, S, H, hd, False)
    h16 = oracle.store_h_bytes(layers, S, d, False)
    h8 = oracle.store_h_bytes(layers, S, d, True)
    assert 1 - h16 / kv == 0.5                      # FP16 row: 43-50%
    assert 0.66 <= 1 - h8 / kv <= 0.75              # INT8 row: 66-75%
    assert h8 == layers * S * (d + 2 * d // 128)


@pytest.fixture(scope="module")
def tiny():
    s = synth.SHAPES["tiny"]
    w = synth.make_weights(s, seed=1, gains="random", q_scale_mult=8.0)
    return s, oracle.OracleModel(w)


def test_forward_keeps_the_quantized_h_and_rebuilds_from_it(tiny):
    s, om = tiny
    toks = synth.make_tokens(s.vocab, 23, seed=5)
    sites = []
    r = oracle.forward(om, toks, 3, logits=None, max_seq=32, h_int8=True, sites=sites)
    cache = r["cache"]
    for layer, rec in enumerate(sites[:s.n_pre + 3]):
        q, sc = oracle.h_quantize(rec["h"].astype(np.float16))
        assert np.array_equal(cache.hq[layer][:23], q) and np.array_equal(cache.hs[layer][:23], sc)
        assert np.array_equal(cache.h[layer][:23], oracle.h_dequantize(q, sc))
    with pytest.raises(ValueError):
        oracle.forward(om, toks, 3, logits=None, max_seq=32, h_int8=True, casts=False)


def test_int8_h_is_close_to_fp16_h_and_not_equal(tiny):
    s, om = tiny
    toks = synth.make_tokens(s.vocab, 40, seed=6)
    a = oracle.forward(om, toks, 4, logits=None, max_seq=48, store_h=True)["hidden"]
    b = oracle.forward(om, toks, 4, logits=None, max_seq=48, h_int8=True)["hidden"]
    err = (np.linalg.norm(a - b, axis=1) / np.linalg.norm(a, axis=1)).max()
    print(f"INT8 vs FP16 store-h, tiny L=4: max row rel diff {err:.2e}")
    assert 0 < err < 2e-2


def test_cached_steps_equal_one_prefill(tiny):
    """K and V of every position come from the cache's h^ rows, so decoding
    token by token sees the same keys and values as one prefill."""
    s, om = tiny
    toks = synth.make_tokens(s.vocab, 20, seed=7)
    one = oracle.forward(om, toks, 3, logits=None, max_seq=24, h_int8=True)["hidden"]
    cache = oracle.Cache(s, 24, h_int8=True)
    rows = [oracle.forward(om, toks[:12], 3, cache=cache, logits=None)["hidden"]]
    for t in toks[12:]:
        rows.append(oracle.forward(om, [t], 3, cache=cache, logits=None)["hidden"])
    steps = np.concatenate(rows)
    assert np.abs(steps - one).max() <= 1e-9 * np.abs(one).max()
