"""Pins of the oracle's store-h cache (h-mode KV reconstruction).

"Current Status" page, KV-cache table (Store-h FP16: bit-exact) and "Claims &
Data Sources" (h-mode KV reconstruction from the shared W_k / W_v): keeping
each position's normed block input h and rebuilding K and V from it when
attention reads them gives the same attention inputs as storing K and V, so
the forward is unchanged. The store-h path rebuilds K/V for all visible
positions at every call (one matmul over the stored rows) while the K/V path
computes each position's K/V once when it is written: two code paths that
must agree, for prefill, chunked prefill and cached decode, at several L.
"""
import numpy as np
import pytest

import oracle
import synth


@pytest.fixture(scope="module")
def micro():
    s = synth.SHAPES["micro"]
    return s, oracle.OracleModel(synth.make_weights(s, seed=7, gains="random", q_scale_mult=8.0))


@pytest.mark.parametrize("L", [1, 3])
def test_store_h_equals_kv_storage(micro, L):
    s, om = micro
    toks = synth.make_tokens(s.vocab, 17, seed=3)
    ref = oracle.forward(om, toks, L, logits="all", max_seq=32)
    got = oracle.forward(om, toks, L, logits="all", max_seq=32, store_h=True)
    assert np.allclose(got["hidden"], ref["hidden"], rtol=0, atol=1e-12)
    # chunked prefill then cached decode steps, both caches side by side
    ck, ch = oracle.Cache(s, 32), oracle.Cache(s, 32, store_h=True)
    for lo, hi in [(0, 9), (9, 13), (13, 14), (14, 15), (15, 17)]:
        a = oracle.forward(om, toks[lo:hi], L, cache=ck, logits="last")
        b = oracle.forward(om, toks[lo:hi], L, cache=ch, logits="last")
        assert np.allclose(b["hidden"], a["hidden"], rtol=0, atol=1e-12)
        assert np.allclose(b["logits"], a["logits"], rtol=0, atol=1e-12)
    assert len(ch.k) == 0 and len(ch.h) == s.n_pre + L   # only h rows are kept


def test_store_h_rejects_int8():
    s = synth.SHAPES["micro"]
    with pytest.raises(ValueError):
        oracle.Cache(s, 8, kv_int8=True, store_h=True)
