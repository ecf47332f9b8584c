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


def _int8_planes(H, R, hd):
    """Offsets of the INT8 planes in one (lane, layer) region, as include/tl.h
    documents them: K codes, K scales, V codes, V scales, each 256-byte aligned."""
    a = lambda x: (x + 255) // 256 * 256
    codes, scales = a(H * R * hd), a(H * R * 2)
    return {"kq": 0, "ks": codes, "vq": codes + scales, "vs": 2 * codes + scales, "bytes": 2 * (codes + scales)}


def _check_int8_ring(kv_host, layer_bytes, n_layers, s, R, lane, length, n_used, cache, sites):
    """The GPU ring of one lane against the oracle, layer by layer: ring row r
    must hold the latest position p < length with p mod R == r, coded as the
    oracle codes that position's K and V rows. The two sides compute the fp16
    K/V rows in different (correct) accumulation orders, and their residual
    streams drift apart by ~1e-3 (relative) over the layers, so a code decided
    near a rounding tie may come out one step apart and a scale (amax / 127)
    a few fp16 ulps apart. A ring, position, head or plane mistake instead puts
    unrelated rows side by side: codes many steps apart, scales far apart, and
    differences everywhere. So: codes at most one step apart, scales at most 4
    ulps apart, at most 4% of the codes flipped, and the flips clustered at
    ties (the oracle's quotient x / s within 0.35 of a half-integer, 0.08 on
    average; uniform placement would average 0.25). Returns (flips, codes,
    mean tie distance of the flips)."""
    H, hd = s.n_heads, s.head_dim
    pl = _int8_planes(H, R, hd)
    assert pl["bytes"] == layer_bytes
    flips = total = 0
    ties = []
    for layer in range(n_used):
        base = (lane * n_layers + layer) * layer_bytes
        reg = kv_host[base:base + layer_bytes]
        for kind in ("k", "v"):
            codes = reg[pl[kind + "q"]:pl[kind + "q"] + H * R * hd].view(np.int8).reshape(H, R, hd)
            scal = reg[pl[kind + "s"]:pl[kind + "s"] + H * R * 2].view(np.float16).reshape(H, R)
            oq = getattr(cache, kind + "q")[layer]                 # codes [pos][H][hd]
            osc = getattr(cache, kind + "s")[layer]                # scales [pos][H]
            ox = sites[layer][kind.upper()]                        # fp16 rows [pos][H][hd]
            for r in range(min(R, length)):
                p = r + (length - 1 - r) // R * R                  # latest position with p mod R == r
                gq, gs = codes[:, r, :].astype(np.int64), scal[:, r]
                qo, so = oq[p].astype(np.int64), osc[p]
                ulps = np.abs(gs.view(np.uint16).astype(np.int64) - so.view(np.uint16).astype(np.int64))
                assert (ulps <= 4).all(), (layer, kind, r, p, int(ulps.max()))
                d = np.abs(gq - qo)
                assert d.max() <= 1, (layer, kind, r, p, int(d.max()))
                if d.any():
                    ratio = ox[p].astype(np.float32) / so.astype(np.float32)[:, None]
                    ties.append(np.abs(np.abs(ratio - np.floor(ratio)) - 0.5)[d > 0])
                total += d.size
                flips += int((d > 0).sum())
    ties = np.concatenate(ties) if ties else np.zeros(0)
    assert flips <= 0.04 * total, (flips, total)
    if flips:
        assert ties.max() < 0.35 and ties.mean() < 0.08, (float(ties.max()), float(ties.mean()))
    return flips, total, float(ties.mean()) if flips else 0.0


# INT8 windows at the tiny shape (d = 256). The ring check reads the GPU's
# codes and scales back from the caller's KV buffer and compares them with
# the oracle's position by position: the only differences are one-step code
# flips where the two sides' fp16 K/V rows straddle a rounding tie (mean
# distance of the quotient from a tie ~0.03, against 0.25 for misplaced rows).
# Such a flip is a legitimate evaluation of the definition on either side,
# and in a window of W keys one K/V row carries ~1/W of a query's attention:
# with W <= 16 the flips alone move rows by up to 2.3e-3 at this width, so
# these cases are held to 3e-3; W = 40 and the named configurations (INT8 at
# the 407M shape, the tiny shape with FP16 KV) keep 2e-3.
TOL_INT8_SHORT_WINDOW = 3e-3


@pytest.mark.parametrize("W,L", [(16, 3), (1, 2), (40, 4)])
def test_window_matches_oracle_int8(sharp, W, L):
    """INT8 cache with a window at the tiny shape: the ring's codes and scales
    against the oracle's, then hidden states and logits."""
    s, w, om = sharp
    _window_case(s, w, om, W, L, kv_int8=True, max_seq=160, max_tokens=24, lens=[110, 73], chunks=[24, 11],
                 steps=40, check_ring=True, tol=TOL if W >= 40 else TOL_INT8_SHORT_WINDOW)


def test_window_int8_ring_plain_weights(plain):
    s, w, om = plain
    _window_case(s, w, om, 16, 3, kv_int8=True, max_seq=160, max_tokens=24, lens=[110, 73], chunks=[24, 11],
                 steps=40, check_ring=True, tol=TOL_INT8_SHORT_WINDOW)


@pytest.mark.slow
@pytest.mark.parametrize("kv_int8", [True, False])
def test_window_407m(kv_int8):
    s = synth.SHAPES["m407"]
    w = synth.make_weights(s, seed=0)
    om = oracle.OracleModel(w)
    _window_case(s, w, om, 128, 4, kv_int8=kv_int8, max_seq=512, max_tokens=96, lens=[264, 200],
                 chunks=[96, 70], steps=64)


def _window_case(s, w, om, W, L, kv_int8, max_seq, max_tokens, lens, chunks, steps, check_ring=False, tol=TOL):
    kv = tl.TL_KV_INT8 if kv_int8 else tl.TL_KV_FP16
    m = _model(w, max_seq=max_seq, max_loops=L, n_lanes=2, kv_dtype=kv, max_tokens=max_tokens,
               cache_window=W)
    for lane in range(2):
        m.set_loops(lane, L)
    toks = [synth.make_tokens(s.vocab, n, seed=3, lane=i) for i, n in enumerate(lens)]
    hid, lgs = _run(m, s, toks, chunks=chunks, steps=steps)
    kv_host = m.kv.cpu().numpy() if check_ring else None
    layer_bytes, n_layers = tl.tl_kv_layer_bytes(m.cfg), s.n_pre + L
    m.close()
    R = min(max_seq, W + max_tokens)
    for lane in range(2):
        sites = [] if check_ring else None
        ro = oracle.forward(om, toks[lane], L, logits=None, max_seq=max_seq, kv_int8=kv_int8, window=W,
                            sites=sites)
        ref_l = oracle.head_logits(om, ro["hidden"][-steps:])
        e_h = rel_rows(hid[lane], ro["hidden"])
        e_l = rel_rows(lgs[lane], ref_l)
        print(f"W={W} L={L} int8={kv_int8} lane {lane}: hidden {e_h:.2e} logits {e_l:.2e}", flush=True)
        if check_ring:
            fl, tot, tie = _check_int8_ring(kv_host, layer_bytes, n_layers, s, R, lane, len(toks[lane]),
                                            s.n_pre + L, ro["cache"], sites)
            print(f"  ring rows: codes equal to the oracle's except {fl} one-step flips of {tot} "
                  f"(mean distance of their quotient from a tie {tie:.3f})", flush=True)
        assert e_h < tol and e_l < tol


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
