"""Pins of the oracle's INT4 unpack/pack and dequantization (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle
from tests.conftest import GOLDEN


def _golden():
    with open(os.path.join(GOLDEN, "int4_words.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["word"])
def test_fixed_words(case):
    w = np.array([[int(case["word"], 16)]], dtype=np.uint32)
    assert oracle.unpack_int4(w)[0].tolist() == case["values"]
    assert oracle.pack_int4(np.array([case["values"]]))[0, 0] == w[0, 0]


def test_every_value_at_every_position():
    # each of the 16 nibble values at each of the 8 positions, other nibbles random
    rng = np.random.default_rng(1)
    for pos in range(8):
        for nib in range(16):
            base = rng.integers(0, 2**32, size=64, dtype=np.uint32)
            mask = np.uint32(0xF) << np.uint32(4 * pos)
            w = (base & ~mask) | (np.uint32(nib) << np.uint32(4 * pos))
            vals = oracle.unpack_int4(w[:, None])[:, pos]
            expect = nib - 16 if nib >= 8 else nib
            assert (vals == expect).all()


def test_exhaustive_low_and_high_halfwords():
    # all 2^16 patterns of the low half-word and of the high half-word
    pats = np.arange(2**16, dtype=np.uint32)
    for shift in (0, 16):
        w = (pats << np.uint32(shift))[:, None]
        q = oracle.unpack_int4(w)
        assert (oracle.pack_int4(q) == w).all()
        # value of nibble j is the two's-complement reading of bits 4j..4j+3
        for j in range(8):
            nib = (w[:, 0] >> np.uint32(4 * j)) & np.uint32(0xF)
            assert (q[:, j] == np.where(nib >= 8, nib.astype(np.int64) - 16, nib)).all()


def test_random_round_trip_and_range():
    rng = np.random.default_rng(2)
    w = rng.integers(0, 2**32, size=(1000, 128), dtype=np.uint32)
    q = oracle.unpack_int4(w)
    assert q.min() == -8 and q.max() == 7
    assert (oracle.pack_int4(q) == w).all()
    # uniform random words give every value about equally often
    counts = np.bincount(q.ravel().astype(np.int64) + 8, minlength=16)
    assert counts.min() > 0.9 * q.size / 16


def test_pack_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.pack_int4(np.zeros((1, 7), dtype=np.int64))
    with pytest.raises(ValueError):
        oracle.pack_int4(np.full((1, 8), 8))
    with pytest.raises(ValueError):
        oracle.pack_int4(np.full((1, 8), -9))


def test_dequant_closed_forms():
    # all codes 1: W equals the scales spread over their groups, partial last group
    n, k, g = 3, 704, 128
    q = np.ones((n, k), dtype=np.int64)
    rng = np.random.default_rng(3)
    s = rng.uniform(0.001, 0.004, size=(n, 6)).astype(np.float16)
    W = oracle.dequantize(oracle.pack_int4(q), s, g)
    for kk in range(k):
        assert (W[:, kk] == s[:, kk // g].astype(np.float64)).all()
    # the last group covers channels 640..703 only
    assert (W[:, 640:] == s[:, 5:6].astype(np.float64)).all()
    with pytest.raises(ValueError):
        oracle.dequantize(oracle.pack_int4(q), s[:, :5], g)


def test_dequant_exact_product():
    # int * fp16 scale is exact: compare with exact rational arithmetic
    from fractions import Fraction
    rng = np.random.default_rng(4)
    qw = rng.integers(0, 2**32, size=(4, 4), dtype=np.uint32)
    s = (0.02 / 7 * rng.uniform(0.5, 1.5, size=(4, 2))).astype(np.float16)
    W = oracle.dequantize(qw, s, 16)
    q = oracle.unpack_int4(qw)
    for i in range(4):
        for kk in range(32):
            exact = Fraction(int(q[i, kk])) * Fraction(float(s[i, kk // 16]))
            assert Fraction(float(W[i, kk])) == exact
            assert Fraction(float(np.float32(W[i, kk]))) == exact
