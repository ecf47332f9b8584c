"""Pins of the oracle's FP16 body (weights q * s rounded to float16 once).

"Performance and Memory" page, "FP16 body cache": the body weights are
dequantized to persistent FP16 at load time. Pins: with power-of-two scales
every q * s is exact in float16, so the FP16 body equals the W4 oracle exactly;
with the usual scales each weight moves by at most half an fp16 ulp (checked
against numpy's own float16 rounding of the float64 product, weight by
weight); the forward pass then stays within the fp16 rounding of its inputs.
"""
import copy

import numpy as np

import oracle
import synth


def test_power_of_two_scales_are_exact():
    s = synth.SHAPES["micro"]
    w = synth.make_weights(s, seed=3)
    w2 = copy.deepcopy(w)
    for b in w2["pre"] + [w2["loop"]]:
        for name in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
            b[name]["scales"] = np.full_like(b[name]["scales"], np.float16(2.0 ** -7))
    toks = synth.make_tokens(s.vocab, 9, seed=2)
    a = oracle.forward(oracle.OracleModel(w2), toks, 3, logits="all")
    b = oracle.forward(oracle.OracleModel(w2, fp16_body=True), toks, 3, logits="all")
    assert np.array_equal(a["hidden"], b["hidden"]) and np.array_equal(a["logits"], b["logits"])


def test_weights_round_once_within_half_ulp():
    s = synth.SHAPES["micro"]
    w = synth.make_weights(s, seed=4)
    exact, body = oracle.OracleModel(w), oracle.OracleModel(w, fp16_body=True)
    for name in ("wq", "w_down"):
        e, h = exact.loop[name], body.loop[name]
        assert np.array_equal(h, e.astype(np.float16).astype(np.float64))
        ulp = np.spacing(np.abs(e).astype(np.float16)).astype(np.float64)
        assert np.all(np.abs(h - e) <= 0.5 * ulp + 1e-30)
        assert np.any(h != e)                       # the rounding is not a no-op here
    toks = synth.make_tokens(s.vocab, 9, seed=2)
    a = oracle.forward(exact, toks, 3, logits=None)["hidden"]
    b = oracle.forward(body, toks, 3, logits=None)["hidden"]
    rel = np.max(np.abs(a - b), axis=1) / np.max(np.abs(a), axis=1)
    assert 0 < rel.max() < 1e-2
