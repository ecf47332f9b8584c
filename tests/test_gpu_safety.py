"""GPU per-iteration residual-norm safety check against the oracle.

"Current Status" page, architecture-unique features table: the residual's L2
norm is checked after every loop iteration and the forward stops above a
threshold. The oracle (oracle.safety_trip) gives the first (iteration, row)
over the threshold; the GPU must report the same one (thresholds are chosen
at least 1% away from every row norm so a correct fp32 evaluation cannot
decide differently), trip earlier when the loop block's down-projection
scales are multiplied, and not trip (nor change any result) below the
threshold.
"""
import copy

import numpy as np
import pytest

import oracle
import synth
from tests.conftest import ensure_library

pytestmark = pytest.mark.gpu
tl = ensure_library()


def _torch():
    import torch
    return torch


def _model(weights, **kw):
    from looped_weight_shared_amd.model import Model
    return Model(weights, **kw)


def _dev(a):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.fixture(scope="module")
def models():
    s = synth.SHAPES["tiny"]
    w = synth.make_weights(s, seed=0)
    w8 = copy.deepcopy(w)
    w8["loop"]["w_down"]["scales"] = (w8["loop"]["w_down"]["scales"].astype(np.float32) * 8).astype(np.float16)
    return s, {"plain": (w, oracle.OracleModel(w)), "x8": (w8, oracle.OracleModel(w8))}


def _norms(om, toks, L):
    r = oracle.forward(om, toks, L, logits=None, trace=True)
    s = om.shape
    return np.array([np.sqrt((r["trace"][s.n_pre + i] ** 2).sum(1)) for i in range(L)])


def _threshold(nrm, j):
    """A threshold between the largest norm of iterations < j and the largest
    of iteration j (j = None: above every norm), at least 1% away from every
    norm that decides the first trip."""
    if j is None:
        return float(nrm.max()) * 1.5
    lo = float(nrm[:j].max()) if j > 0 else 0.0
    cand = np.sort(nrm[j][nrm[j] > lo])
    for hi in cand[::-1]:
        thr = float(np.sqrt(max(lo, 1e-6) * hi)) if lo > 0 else float(hi) * 0.5
        if np.min(np.abs(nrm[:j + 1] / thr - 1)) > 0.01:
            return thr
    pytest.skip("no well-conditioned threshold for this case")


@pytest.mark.parametrize("name,L,j", [("plain", 6, 5), ("plain", 6, 3), ("x8", 6, 2), ("x8", 6, 1), ("plain", 4, None)])
def test_prefill_trips_where_the_oracle_does(models, name, L, j):
    s, mdl = models
    w, om = mdl[name]
    toks = synth.make_tokens(s.vocab, 20, seed=1)
    nrm = _norms(om, toks, L)
    thr = _threshold(nrm, j)
    ref = oracle.safety_trip(om, toks, L, thr)
    assert (ref is None) == (j is None) and (ref is None or ref[0] == j)
    m = _model(w, max_seq=64, max_loops=L, max_tokens=32)
    m.set_loops(0, L)
    m.set_safety(thr)
    torch = _torch()
    hid = torch.empty((20, s.d_model), dtype=torch.float32, device="cuda")
    if ref is None:
        m.prefill(_dev(toks), hidden=hid)
        assert m.safety_last() == (-1, -1)
    else:
        with pytest.raises(tl.TLError) as e:
            m.prefill(_dev(toks), hidden=hid)
        assert e.value.status == tl.TL_E_SAFETY
        assert m.safety_last() == (ref[0], ref[1])
        assert m.length(0) == 20                     # the call's work is done
    print(f"{name} L={L} thr={thr:.3f}: oracle {ref}, gpu {m.safety_last()}")
    m.close()


def test_safety_off_and_on_give_identical_results(models):
    s, mdl = models
    w, _ = mdl["plain"]
    toks = synth.make_tokens(s.vocab, 20, seed=2)
    torch = _torch()
    out = []
    for thr in (0.0, 1e6):
        m = _model(w, max_seq=64, max_loops=4, max_tokens=32)
        m.set_loops(0, 4)
        m.set_safety(thr)
        hid = torch.empty((20, s.d_model), dtype=torch.float32, device="cuda")
        m.prefill(_dev(toks), hidden=hid)
        nx = torch.zeros((1,), dtype=torch.int32, device="cuda")
        m.decode_step(_dev([5]), next_tok=nx)
        torch.cuda.synchronize()
        out.append((hid.cpu().numpy(), int(nx.item())))
        assert m.safety_last() == (-1, -1)
        m.close()
    assert np.array_equal(out[0][0], out[1][0]) and out[0][1] == out[1][1]
    m = _model(w, max_seq=64, max_loops=4, max_tokens=32)
    with pytest.raises(tl.TLError) as e:
        m.set_safety(-1.0)
    assert e.value.status == tl.TL_E_RANGE
    m.close()


def test_decode_reports_the_lane(models):
    """Two lanes, L = 2 and 6 on the scaled model: only the deep lane's later
    iterations exceed the threshold, and the trip names that lane."""
    s, mdl = models
    w, om = mdl["x8"]
    P = 12
    toks = [synth.make_tokens(s.vocab, P + 1, seed=4, lane=i) for i in range(2)]
    Ls = [2, 6]
    thr = 24.0   # above lane 0's norms (<= 18.3), below lane 1's from iteration 4 (29.9)
    ref = []
    for i in range(2):
        cache = oracle.Cache(s, 64)
        oracle.forward(om, toks[i][:P], Ls[i], cache=cache, logits=None)
        nrm = _norms_from_cache(om, cache, toks[i][P], Ls[i])
        ref.append(nrm)
    assert ref[0].max() < thr * 0.99 and ref[1].max() > thr * 1.01
    first_it = int(np.nonzero(ref[1] > thr)[0][0])
    m = _model(w, max_seq=64, max_loops=6, n_lanes=2, max_tokens=32)
    for i in range(2):
        m.set_loops(i, Ls[i])
        m.prefill(_dev(toks[i][:P]), lane=i)
    m.set_safety(thr)
    with pytest.raises(tl.TLError) as e:
        m.decode_step(_dev([toks[0][P], toks[1][P]]))
    assert e.value.status == tl.TL_E_SAFETY
    assert m.safety_last() == (first_it, 1)
    assert m.length(0) == P + 1 and m.length(1) == P + 1
    m.close()


def _norms_from_cache(om, cache, token, L):
    """Residual norm after each loop iteration of one cached decode step."""
    r = oracle.forward(om, [token], L, cache=cache, logits=None, trace=True)
    s = om.shape
    return np.array([float(np.sqrt((r["trace"][s.n_pre + i][0] ** 2).sum())) for i in range(L)])
