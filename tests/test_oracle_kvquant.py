"""Pins of the oracle's per-(token, head) INT8 KV quantizer and KV sizes (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle
from tests.conftest import GOLDEN


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _load("kv_int8_worked.json")["cases"], ids=lambda c: c["why"][:30])
def test_worked_rows(case):
    x = np.array(case["x"], dtype=np.float16)
    q, s = oracle.kv_quantize(x[None])
    assert float(s[0]) == case["scale"]
    assert q[0].tolist() == case["q"]
    # the value attention reads back, worked by hand as q times the scale
    assert oracle.kv_dequantize(q, s)[0].tolist() == case["xhat"]
    # the per-element bound |x - xhat| <= s/2 holds on the worked rows too
    assert (np.abs(x.astype(np.float64) - np.array(case["xhat"])) <= case["scale"] / 2).all()


def _rows(rng, n, hd=128, spread=1.0):
    return (rng.standard_normal((n, hd)) * spread).astype(np.float16)


def test_amax_maps_to_127_and_error_bound():
    rng = np.random.default_rng(5)
    for spread in (0.01, 0.3, 1.0, 30.0, 3000.0):
        x = _rows(rng, 20000, spread=spread)
        q, s = oracle.kv_quantize(x)
        x32 = x.astype(np.float32)
        s32 = s.astype(np.float32)
        assert (s32 > 0).all()
        # normal FP16 scale: the largest magnitude maps to exactly +-127
        normal = s32 >= np.float32(2.0 ** -14)
        am = np.argmax(np.abs(x32), axis=1)
        picked = q[np.arange(len(q)), am]
        assert (np.abs(picked[normal]) == 127).all()
        # |x - q*s| <= s/2 per element (the quotient is rounded once in float32)
        err = np.abs(x32.astype(np.float64) - q.astype(np.float64) * s32[:, None])
        assert (err <= s32[:, None] * (0.5 + 2.0 ** -20)).all()


def test_symmetry_and_power_of_two_scaling():
    rng = np.random.default_rng(6)
    x = _rows(rng, 2000)
    q, s = oracle.kv_quantize(x)
    qn, sn = oracle.kv_quantize(-x)
    assert (qn == -q).all() and (sn == s).all()
    q2, s2 = oracle.kv_quantize((x.astype(np.float32) * 4).astype(np.float16))
    assert (q2 == q).all() and (s2.astype(np.float32) == 4 * s.astype(np.float32)).all()


def test_zero_and_subnormal_scales():
    x = np.zeros((1, 128), dtype=np.float16)
    q, s = oracle.kv_quantize(x)
    assert (q == 0).all() and s[0] == 0
    # amax so small that amax/127 is a subnormal FP16: codes may pass 127 and must clamp
    x = np.zeros((1, 128), dtype=np.float16)
    x[0, 0] = np.float16(2.0 ** -10)
    x[0, 1] = np.float16(-(2.0 ** -10))
    q, s = oracle.kv_quantize(x)
    assert 0 < float(s[0]) < 2.0 ** -14
    assert q[0, 0] == 127 and q[0, 1] == -127
    ratio = np.float32(x[0, 0]) / np.float32(s[0])
    assert ratio > 127.0   # the clamp did fire here


def test_dequantize_is_exact_product():
    rng = np.random.default_rng(7)
    x = _rows(rng, 100)
    q, s = oracle.kv_quantize(x)
    d = oracle.kv_dequantize(q, s)
    assert (d == q.astype(np.float64) * s.astype(np.float64)[:, None]).all()


def test_kv_bytes_match_printed_page_numbers():
    g = _load("kv_cache_memory.json")
    fp16 = oracle.kv_cache_bytes(g["n_layers"], g["max_seq"], g["n_heads"], g["head_dim"], False)
    int8 = oracle.kv_cache_bytes(g["n_layers"], g["max_seq"], g["n_heads"], g["head_dim"], True)
    assert round(fp16 / 1e6, 1) == g["fp16_mb_printed"]
    assert round(int8 / 1e6, 1) == g["int8_mb_printed"]
    assert round(100.0 * (int8 - fp16) / fp16, 1) == g["delta_pct_printed"]
    per_token_int8 = int8 // g["max_seq"]
    assert fp16 // per_token_int8 == g["int8_context_printed"]
    assert fp16 // (fp16 // g["max_seq"]) == g["fp16_context_printed"]


def test_dequantize_worked_rows():
    """Hand-worked values: each row's codes times that row's scale (not another row's), exactly,
    including a subnormal fp16 scale."""
    q = np.array([[127, -127, 1, 0], [3, -2, 0, 64]], dtype=np.int8)
    s = np.array([0.5, 2.0 ** -20], dtype=np.float16)
    d = oracle.kv_dequantize(q, s)
    assert d.dtype == np.float64
    assert d[0].tolist() == [63.5, -63.5, 0.5, 0.0]
    assert d[1].tolist() == [3 * 2.0 ** -20, -2 * 2.0 ** -20, 0.0, 64 * 2.0 ** -20]
