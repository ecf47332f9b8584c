"""GPU sliding-window cache (cache_window) against the oracle.

"Performance and Memory" page, "Sliding-Window Cache": with W > 0 only the
last W cached tokens stay visible. The library keeps them in a ring of
W + max_tokens rows per (lane, layer, head), so the cases below wrap the
ring several times: chunked prefills, decode steps past the ring size, two
lanes at different positions, FP16 caches at the tiny shape (sharpened
attention, windows of 1, 16 and 40) and FP16 and INT8 caches at the 407M
shape. Floating-point results
are compared with the oracle (same window) at the 2e-3 row-relative bound,
teacher-forced; a window at least max_seq long must give the same bits as
the full cache.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.conftest import ensure_library, rel_rows

pytestmark = pytest.mark.gpu
tl = ensure_library()
TOL = 2e-3


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
def sharp():
    s = synth.SHAPES["tiny"]
    w = synth.make_weights(s, seed=1, gains="random", q_scale_mult=8.0)
    return s, w, oracle.OracleModel(w)


@pytest.fixture(scope="module")
def plain():
    s = synth.SHAPES["tiny"]
    w = synth.make_weights(s, seed=0)
    return s, w, oracle.OracleModel(w)


def _run(m, s, lanes_tokens, chunks, steps):
    """Prefill each lane's tokens in `chunks`-sized pieces, then `steps` decode
    steps on all lanes with each lane's next tokens. Returns per lane the hidden
    rows of every position and the logits of every decode step."""
    torch = _torch()
    n_l = len(lanes_tokens)
    hid = [[] for _ in range(n_l)]
    lgs = [[] for _ in range(n_l)]
    for lane, toks in enumerate(lanes_tokens):
        pre = toks[:len(toks) - steps]
        for c0 in range(0, len(pre), chunks[lane]):
            part = pre[c0:c0 + chunks[lane]]
            h = torch.empty((len(part), s.d_model), dtype=torch.float32, device="cuda")
            m.prefill(_dev(part), lane=lane, hidden=h)
            hid[lane].append(h.cpu().numpy())
    for t in range(steps):
        h = torch.zeros((n_l, s.d_model), dtype=torch.float32, device="cuda")
        lg = torch.zeros((n_l, s.vocab), dtype=torch.float32, device="cuda")
        tok = [lanes_tokens[l][len(lanes_tokens[l]) - steps + t] for l in range(n_l)]
        m.decode_step(_dev(tok), hidden=h, logits=lg)
        for lane in range(n_l):
            hid[lane].append(h[lane:lane + 1].cpu().numpy())
            lgs[lane].append(lg[lane].cpu().numpy())
    torch.cuda.synchronize()
    return [np.concatenate(x) for x in hid], [np.array(x) for x in lgs]


@pytest.mark.parametrize("W,L", [(16, 3), (1, 2), (40, 4)])
def test_window_matches_oracle_fp16(sharp, W, L):
    s, w, om = sharp
    _window_case(s, w, om, W, L, kv_int8=False, max_seq=160, max_tokens=24, lens=[110, 73], chunks=[24, 11],
                 steps=40)


@pytest.mark.parametrize("W", [2, 16])
def test_short_window_within_one_prefill_over_two_key_tiles(sharp, W):
    """A 150-token prefill in one call: with W = 16, queries 143..149 see no
    key of the first 128-key tile, so the online softmax must skip that tile
    for them (regression: their rows came out NaN)."""
    s, w, om = sharp
    _window_case(s, w, om, W, 3, kv_int8=False, max_seq=200, max_tokens=150, lens=[160, 150], chunks=[150, 150],
                 steps=10)


# INT8 windows are checked at the 407M shape. At the tiny shape (d = 256) a
# code decided differently on a one-ulp fp16 difference between two correct
# evaluations of a K/V row is a large part of a short dot product: a CPU run
# of the oracle with fp32 group-wise projections (the GPU's accumulation)
# already differs from the float64 oracle by 1.4e-3 at INT8, window or not,
# and the GPU measured 2.3e-3 with W = 16. At d = 2048 the same flips average
# out (the 2048-context INT8 tests stay below 1e-3).
@pytest.mark.slow
@pytest.mark.parametrize("kv_int8", [True, False])
def test_window_407m(kv_int8):
    s = synth.SHAPES["m407"]
    w = synth.make_weights(s, seed=0)
    om = oracle.OracleModel(w)
    _window_case(s, w, om, 128, 4, kv_int8=kv_int8, max_seq=512, max_tokens=96, lens=[264, 200],
                 chunks=[96, 70], steps=64)


def _window_case(s, w, om, W, L, kv_int8, max_seq, max_tokens, lens, chunks, steps):
    kv = tl.TL_KV_INT8 if kv_int8 else tl.TL_KV_FP16
    m = _model(w, max_seq=max_seq, max_loops=L, n_lanes=2, kv_dtype=kv, max_tokens=max_tokens,
               cache_window=W)
    for lane in range(2):
        m.set_loops(lane, L)
    toks = [synth.make_tokens(s.vocab, n, seed=3, lane=i) for i, n in enumerate(lens)]
    hid, lgs = _run(m, s, toks, chunks=chunks, steps=steps)
    m.close()
    for lane in range(2):
        ro = oracle.forward(om, toks[lane], L, logits=None, max_seq=max_seq, kv_int8=kv_int8, window=W)
        ref_l = oracle.head_logits(om, ro["hidden"][-steps:])
        e_h = rel_rows(hid[lane], ro["hidden"])
        e_l = rel_rows(lgs[lane], ref_l)
        print(f"W={W} L={L} int8={kv_int8} lane {lane}: hidden {e_h:.2e} logits {e_l:.2e}")
        assert e_h < TOL and e_l < TOL


@pytest.mark.parametrize("kv", [0, 1])
def test_long_window_is_the_full_cache(sharp, kv):
    """W >= max_seq: no ring, no masking: the same bits as cache_window 0."""
    s, w, om = sharp
    toks = [synth.make_tokens(s.vocab, 60, seed=8)]
    out = []
    for W in (0, 96, 500):
        m = _model(w, max_seq=96, max_loops=3, max_tokens=32, cache_window=W,
                   kv_dtype=tl.TL_KV_INT8 if kv else tl.TL_KV_FP16)
        m.set_loops(0, 3)
        out.append(_run(m, s, toks, chunks=[32], steps=8))
        m.close()
    for o in out[1:]:
        assert np.array_equal(o[0][0], out[0][0][0]) and np.array_equal(o[1][0], out[0][1][0])
