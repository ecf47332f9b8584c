"""Prefill and decode graph replay give the same bits as eager launches.

tl_prefill captures its launch sequence once per (lane, n, p0, L, pointers)
and replays it. A replay must behave exactly like the eager call with the
same arguments: it reads the token buffer as it is when the replay runs,
writes the same outputs and KV rows, and leaves the lane in the same state.
Each replay here is separated by the program's own eager work (output
buffers poisoned with NaN, decode steps, synchronizations) and is checked
against a context that launches eagerly.
"""
import numpy as np
import pytest

import synth
from tests.conftest import ensure_library

pytestmark = pytest.mark.gpu
tl = ensure_library()


def _torch():
    import torch
    return torch


def _model(weights, graphs, **kw):
    from looped_weight_shared_amd.model import Model
    m = Model(weights, **kw)
    m.set_graphs(graphs)
    return m


class Bufs:
    """Fixed device buffers, so that repeated calls hit the cached graph."""

    def __init__(self, shape, n, n_lanes=1):
        torch = _torch()
        self.tok = torch.zeros((n,), dtype=torch.int32, device="cuda")
        self.hid = torch.empty((n, shape.d_model), dtype=torch.float32, device="cuda")
        self.lg = torch.empty((shape.vocab,), dtype=torch.float32, device="cuda")
        self.nx = torch.empty((1,), dtype=torch.int32, device="cuda")
        self.dtok = torch.zeros((n_lanes,), dtype=torch.int32, device="cuda")
        self.dhid = torch.empty((n_lanes, shape.d_model), dtype=torch.float32, device="cuda")
        self.dlg = torch.empty((n_lanes, shape.vocab), dtype=torch.float32, device="cuda")
        self.dnx = torch.empty((n_lanes,), dtype=torch.int32, device="cuda")

    def poison(self):
        for t in (self.hid, self.lg, self.dhid, self.dlg):
            t.fill_(float("nan"))
        self.nx.fill_(-1)
        self.dnx.fill_(-1)


def _prefill(m, b, tokens, lane=0):
    torch = _torch()
    n = len(tokens)
    b.tok[:n].copy_(torch.from_numpy(np.asarray(tokens, dtype=np.int32)))
    m.prefill(b.tok[:n], lane=lane, hidden=b.hid[:n], logits=b.lg, next_tok=b.nx)
    torch.cuda.synchronize()
    return b.hid[:n].cpu().numpy().copy(), b.lg.cpu().numpy().copy(), int(b.nx.item())


def _step(m, b, token):
    torch = _torch()
    b.dtok.fill_(token)
    m.decode_step(b.dtok, hidden=b.dhid, logits=b.dlg, next_tok=b.dnx)
    torch.cuda.synchronize()
    return b.dhid.cpu().numpy().copy(), b.dlg.cpu().numpy().copy()


def _same(a, b):
    assert len(a) == len(b)
    for x, y in zip(a, b):
        if isinstance(x, np.ndarray):
            # rows a call leaves untouched keep their NaN poison on both sides
            assert np.array_equal(x, y, equal_nan=True), "graph replay differs from eager launches"
        else:
            assert x == y


@pytest.fixture(scope="module")
def tiny():
    s = synth.SHAPES["tiny"]
    return s, synth.make_weights(s, seed=3)


def test_replays_match_eager_with_work_between(tiny):
    s, w = tiny
    kw = dict(max_seq=256, max_loops=4, max_tokens=96)
    eager, graph = _model(w, False, **kw), _model(w, True, **kw)
    be, bg = Bufs(s, 96), Bufs(s, 96)
    prompt = synth.make_tokens(s.vocab, 80, seed=5)
    for m in (eager, graph):
        m.set_loops(0, 3)
    ref = _prefill(eager, be, prompt)
    ref_steps = [_step(eager, be, t) for t in (7, 11)]
    for rep in range(4):
        graph.reset(0)
        bg.poison()
        got = _prefill(graph, bg, prompt)          # rep 0 captures, later reps replay
        _same(got, ref)
        assert graph.length(0) == 80
        for t, r in zip((7, 11), ref_steps):       # eager decode on the replayed cache
            _same(_step(graph, bg, t), r)
        assert graph.length(0) == 82
    eager.close()
    graph.close()


def test_replay_reads_current_tokens(tiny):
    """Same pointers, new token values: the replay must see the new ones."""
    s, w = tiny
    kw = dict(max_seq=128, max_loops=2, max_tokens=64)
    eager, graph = _model(w, False, **kw), _model(w, True, **kw)
    be, bg = Bufs(s, 64), Bufs(s, 64)
    for seed in (1, 2, 3):
        prompt = synth.make_tokens(s.vocab, 64, seed=seed)
        eager.reset(0)
        graph.reset(0)
        bg.poison()
        _same(_prefill(graph, bg, prompt), _prefill(eager, be, prompt))
    eager.close()
    graph.close()


def test_changing_keys_recapture(tiny):
    """Chunked prefill (p0 changes), another L, another lane and another n each
    need their own capture; alternating between them must stay exact."""
    s, w = tiny
    kw = dict(max_seq=256, max_loops=4, n_lanes=2, max_tokens=64)
    eager, graph = _model(w, False, **kw), _model(w, True, **kw)
    be, bg = Bufs(s, 64, 2), Bufs(s, 64, 2)
    toks = synth.make_tokens(s.vocab, 112, seed=9)
    plan = [(0, 4, [toks[:64], toks[64:112]]),       # two chunks: p0 = 0, 64
            (1, 2, [toks[:48]]),
            (0, 1, [toks[:64], toks[64:100]]),
            (0, 4, [toks[:64], toks[64:112]])]        # first key again
    for lane, L, chunks in plan:
        for m, b in ((eager, be), (graph, bg)):
            m.reset(lane)
            m.set_loops(lane, L)
        for c in chunks:
            bg.poison()
            _same(_prefill(graph, bg, c, lane=lane), _prefill(eager, be, c, lane=lane))
        assert graph.length(lane) == eager.length(lane) == sum(len(c) for c in chunks)
    eager.close()
    graph.close()


def test_timing_window_launches_eagerly(tiny):
    """Inside a timing window every kernel is timed, so prefill runs eagerly
    even when a graph for the same call is cached; results stay identical."""
    s, w = tiny
    m = _model(w, True, max_seq=128, max_loops=2, max_tokens=32)
    b = Bufs(s, 32)
    prompt = synth.make_tokens(s.vocab, 32, seed=4)
    m.set_loops(0, 2)
    ref = _prefill(m, b, prompt)                      # captures
    m.reset(0)
    tl.tl_profile_begin(m.ctx, 1000)
    got = _prefill(m, b, prompt)
    prof = tl.tl_profile_end(m.ctx)
    _same(got, ref)
    assert prof["embed"][0] == 1 and prof["attn"][0] == s.n_pre + 2
    m.reset(0)
    _same(_prefill(m, b, prompt), ref)               # replay after the window
    m.close()


# ------------------------------------------------------------------ decode steps
def _decode_run(m, s, n_lanes, tokens_per_step, bufs, active=None):
    """One decode step on every lane with tokens[lane]; returns hidden, logits, next."""
    torch = _torch()
    tb, hid, lg, nx = bufs
    tb.copy_(torch.tensor(tokens_per_step, dtype=torch.int32))
    for t in (hid, lg):
        t.fill_(float("nan"))
    nx.fill_(-1)
    m.decode_step(tb, active=active, hidden=hid, logits=lg, next_tok=nx)
    torch.cuda.synchronize()
    return hid.cpu().numpy().copy(), lg.cpu().numpy().copy(), nx.cpu().numpy().copy()


def _dbufs(s, n_lanes, k):
    torch = _torch()
    return [(torch.zeros((n_lanes,), dtype=torch.int32, device="cuda"),
             torch.empty((n_lanes, s.d_model), dtype=torch.float32, device="cuda"),
             torch.empty((n_lanes, s.vocab), dtype=torch.float32, device="cuda"),
             torch.empty((n_lanes,), dtype=torch.int32, device="cuda")) for _ in range(k)]


@pytest.mark.parametrize("window", [0, 48])
def test_decode_replays_match_eager(tiny, window):
    """Two lanes at L = 3 and 1, decoded together for 40 steps across the
    128-key part boundary (a new capture there), with three alternating
    output/token buffer sets (three graphs, within the cache of four), a
    prefill chunk on one lane mid-way (device positions re-initialised) and a
    reset; every step bit for bit against an eager context."""
    s, w = tiny
    kw = dict(max_seq=256, max_loops=4, n_lanes=2, max_tokens=64, cache_window=window)
    eager, graph = _model(w, False, **kw), _model(w, 2, **kw)
    be, bg = Bufs(s, 64, 2), Bufs(s, 64, 2)
    de, dg = _dbufs(s, 2, 3), _dbufs(s, 2, 3)
    prompts = [synth.make_tokens(s.vocab, 110, seed=21), synth.make_tokens(s.vocab, 97, seed=22)]
    rng = np.random.default_rng(5)
    for m, b in ((eager, be), (graph, bg)):
        m.set_loops(0, 3)
        m.set_loops(1, 1)
        for lane in (0, 1):
            for c0 in range(0, len(prompts[lane]), 64):
                _prefill(m, b, prompts[lane][c0:c0 + 64], lane=lane)
    for t in range(40):
        toks = [int(x) for x in rng.integers(0, s.vocab, 2)]
        _same(_decode_run(graph, s, 2, toks, dg[t % 3]), _decode_run(eager, s, 2, toks, de[t % 3]))
        if t == 17:   # a prefill chunk on lane 1 between decode steps
            extra = synth.make_tokens(s.vocab, 9, seed=23)
            _same(_prefill(graph, bg, extra, lane=1), _prefill(eager, be, extra, lane=1))
        if t == 29:   # lane 0 starts over
            for m, b in ((eager, be), (graph, bg)):
                m.reset(0)
            _same(_prefill(graph, bg, prompts[0][:50], lane=0), _prefill(eager, be, prompts[0][:50], lane=0))
    assert [graph.length(l) for l in (0, 1)] == [eager.length(l) for l in (0, 1)]
    eager.close()
    graph.close()


def test_decode_replay_single_lane_and_timing_window(tiny):
    """One active lane of two; a timing window in the middle launches eagerly
    and the replays after it continue exactly."""
    s, w = tiny
    kw = dict(max_seq=128, max_loops=2, n_lanes=2, max_tokens=32)
    eager, graph = _model(w, False, **kw), _model(w, 2, **kw)
    be, bg = Bufs(s, 32, 2), Bufs(s, 32, 2)
    de, dg = _dbufs(s, 2, 1), _dbufs(s, 2, 1)
    prompt = synth.make_tokens(s.vocab, 30, seed=31)
    for m, b in ((eager, be), (graph, bg)):
        m.set_loops(1, 2)
        _prefill(m, b, prompt, lane=1)
    act = [False, True]
    for t in range(12):
        if t == 5:
            tl.tl_profile_begin(graph.ctx, 10000)
        _same(_decode_run(graph, s, 2, [0, 100 + t], dg[0], act), _decode_run(eager, s, 2, [0, 100 + t], de[0], act))
        if t == 5:
            prof = tl.tl_profile_end(graph.ctx)
            assert prof["attn"][0] == s.n_pre + 2      # eager inside the window
    assert graph.length(1) == eager.length(1) == 42 and graph.length(0) == 0
    eager.close()
    graph.close()


def test_spec_decode_with_decode_graphs(tiny):
    """Self-speculative decoding drafts with plain launches and rolls the
    lane back; plain decode steps replayed from graphs afterwards continue
    from the right positions."""
    s, w = tiny
    kw = dict(max_seq=128, max_loops=4, max_tokens=32)
    eager, graph = _model(w, False, **kw), _model(w, 2, **kw)
    be, bg = Bufs(s, 32), Bufs(s, 32)
    de, dg = _dbufs(s, 1, 2), _dbufs(s, 1, 2)
    prompt = synth.make_tokens(s.vocab, 24, seed=41)
    outs = []
    for m, b, db in ((eager, be, de), (graph, bg, dg)):
        m.set_loops(0, 4)
        _, _, first = _prefill(m, b, prompt)
        for t in range(3):
            _decode_run(m, s, 1, [first + t], db[t % 2])
        toks, _ = m.spec_decode(first, 10, draft_loops=2, k_draft=3)
        after = [_decode_run(m, s, 1, [toks[-1] + t], db[t % 2]) for t in range(4)]
        outs.append((toks, after, m.length(0)))
    assert outs[0][0] == outs[1][0] and outs[0][2] == outs[1][2]
    for a, b in zip(outs[0][1], outs[1][1]):
        _same(a, b)
    eager.close()
    graph.close()
