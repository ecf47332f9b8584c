"""Pins of the oracle's sliding-window cache (cache_window).

"Performance and Memory" page, "Sliding-Window Cache": cache_window 0 keeps
the full cache, W > 0 keeps only the last W cached tokens. The reading taken:
a query at position q attends to keys q-W+1 .. q. Pins:
  - a window at least as long as the sequence is the full cache (exactly);
  - W = 1: the only visible key is the query's own, so the attention output
    is the query's own V row (a closed form);
  - masking equals slicing: for every query, the windowed attention equals
    plain causal attention over the explicitly sliced last W keys;
  - cached decode with a window equals the uncached recompute with it, and a
    window shorter than the sequence changes the result.
"""
import numpy as np
import pytest

import oracle
import synth


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_window_one_returns_own_value():
    rng = np.random.default_rng(0)
    n, H, hd = 9, 3, 8
    Q, K, V = _rand(rng, n, H, hd), _rand(rng, n, H, hd), _rand(rng, n, H, hd)
    out = oracle.attention(Q, K, V, np.arange(n), window=1)
    assert np.allclose(out, V, rtol=0, atol=1e-15)


@pytest.mark.parametrize("W", [1, 2, 5, 11])
def test_window_mask_equals_slicing(W):
    rng = np.random.default_rng(W)
    n, H, hd, p0 = 13, 2, 16, 4          # queries at positions p0..p0+n-1
    S = p0 + n
    Q, K, V = _rand(rng, n, H, hd), _rand(rng, S, H, hd), _rand(rng, S, H, hd)
    pos = p0 + np.arange(n)
    got = oracle.attention(Q, K, V, pos, window=W)
    for i, q in enumerate(pos):
        lo = max(0, q - W + 1)
        ref = oracle.attention(Q[i:i + 1], K[lo:q + 1], V[lo:q + 1], [q - lo])
        assert np.allclose(got[i], ref[0], rtol=1e-12, atol=1e-14)


def test_long_window_is_full_cache():
    rng = np.random.default_rng(3)
    n, H, hd = 10, 2, 8
    Q, K, V = _rand(rng, n, H, hd), _rand(rng, n, H, hd), _rand(rng, n, H, hd)
    full = oracle.attention(Q, K, V, np.arange(n))
    assert np.array_equal(oracle.attention(Q, K, V, np.arange(n), window=n), full)
    assert np.array_equal(oracle.attention(Q, K, V, np.arange(n), window=10 * n), full)


def test_windowed_decode_equals_uncached_and_differs_from_full():
    s = synth.SHAPES["micro"]
    om = oracle.OracleModel(synth.make_weights(s, seed=6))
    toks = synth.make_tokens(s.vocab, 20, seed=2)
    W, L = 5, 3
    # cached: prefill 12, then 8 single-token steps
    cache = oracle.Cache(s, 32, window=W)
    oracle.forward(om, toks[:12], L, cache=cache)
    hid = [oracle.forward(om, [t], L, cache=cache, logits=None)["hidden"][0] for t in toks[12:]]
    ref = oracle.forward(om, toks, L, logits=None, max_seq=32, window=W)["hidden"][12:]
    assert np.allclose(np.array(hid), ref, rtol=0, atol=1e-12)
    full = oracle.forward(om, toks, L, logits=None, max_seq=32)["hidden"][12:]
    assert np.abs(full - ref).max() > 1e-3
    same = oracle.forward(om, toks, L, logits=None, max_seq=32, window=20)["hidden"][12:]
    assert np.array_equal(same, full)
