"""Pins of the oracle's per-iteration residual-norm safety check.

The residual after loop iteration k of a depth-L run is the final residual of
a depth-(k+1) run (the prefix property, pinned in test_oracle_model), so the
norms the check compares are recomputed here from separate shallower runs with
math.fsum, and the check must trip exactly at the first (iteration, row) whose
norm exceeds the threshold: never for a threshold above every norm, and at a
chosen iteration when the loop block's down-projection scales are multiplied
so that the residual grows with depth.
"""
import copy
import math

import numpy as np
import pytest

import oracle
import synth


def _norms_by_depth(om, toks, L):
    out = []
    for k in range(1, L + 1):
        x = oracle.forward(om, toks, k, logits=None)["hidden"]
        out.append([math.sqrt(math.fsum(float(v) * float(v) for v in row)) for row in x])
    return np.array(out)          # [iteration][row]


@pytest.fixture(scope="module")
def grown():
    """micro model, and a copy whose loop block has 8x the down-projection
    scales (the residual norm grows from iteration to iteration)."""
    s = synth.SHAPES["micro"]
    w = synth.make_weights(s, seed=5)
    w2 = copy.deepcopy(w)
    w2["loop"]["w_down"]["scales"] = (w2["loop"]["w_down"]["scales"].astype(np.float32) * 8.0).astype(np.float16)
    return s, oracle.OracleModel(w), oracle.OracleModel(w2)


def test_no_trip_above_every_norm(grown):
    s, om, _ = grown
    toks = synth.make_tokens(s.vocab, 7, seed=1)
    nrm = _norms_by_depth(om, toks, 4)
    assert oracle.safety_trip(om, toks, 4, nrm.max() * 1.001) is None


def test_trips_at_first_iteration_over_threshold(grown):
    s, _, om2 = grown
    toks = synth.make_tokens(s.vocab, 7, seed=1)
    L = 5
    nrm = _norms_by_depth(om2, toks, L)
    peak = nrm.max(axis=1)
    assert np.all(np.diff(peak) > 0), "the scaled model's residual should grow with depth"
    for j in range(1, L):
        thr = 0.5 * (peak[j - 1] + peak[j])      # between iterations j-1 and j
        it, row, val = oracle.safety_trip(om2, toks, L, thr)
        assert it == j
        first = int(np.nonzero(nrm[j] > thr)[0][0])
        assert row == first and abs(val - nrm[j, row]) <= 1e-9 * val


def test_nan_trips():
    s = synth.SHAPES["micro"]
    w = synth.make_weights(s, seed=2)
    w2 = copy.deepcopy(w)
    w2["loop"]["w_down"]["scales"][0, 0] = np.float16(np.inf)
    om = oracle.OracleModel(w2)
    toks = synth.make_tokens(s.vocab, 3, seed=1)
    with np.errstate(all="ignore"):
        r = oracle.safety_trip(om, toks, 2, 1e30)
    assert r is not None and r[0] == 0
