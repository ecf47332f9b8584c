"""GPU parity of the whole forward pass through the C ABI against the oracle.

Floating-point results must agree with the float64 oracle within a maximum
row-relative error of 2e-3 (per row: max|gpu - oracle| / max|oracle|) on the
final hidden states and on the logits. Decode comparisons are teacher-forced:
both sides consume the oracle's greedy tokens, because near-tied logits can
legitimately pick different continuations. GPU-vs-GPU properties that the
model family promises (variable-L results, lanes with their own depth,
repeated runs) are checked bit for bit.
"""
import gc

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


def _toks(a):
    torch = _torch()
    return torch.from_numpy(np.asarray(a, dtype=np.int32)).cuda()


class GpuRun:
    """Prefill + teacher-forced decode on one lane, collecting outputs."""

    def __init__(self, model, lane=0):
        torch = _torch()
        self.m, self.lane = model, lane
        s = model.shape
        self.d, self.V, self.n_lanes = s.d_model, s.vocab, model.cfg.n_lanes
        self.torch = torch

    def prefill(self, prompt):
        t = self.torch
        n = len(prompt)
        hid = t.empty((n, self.d), dtype=t.float32, device="cuda")
        lg = t.empty((self.V,), dtype=t.float32, device="cuda")
        nx = t.empty((1,), dtype=t.int32, device="cuda")
        self.m.prefill(_toks(prompt), lane=self.lane, hidden=hid, logits=lg, next_tok=nx)
        t.cuda.synchronize()
        return hid.cpu().numpy(), lg.cpu().numpy(), int(nx.item())

    def step(self, token, active=None):
        t = self.torch
        toks = np.zeros(self.n_lanes, dtype=np.int32)
        toks[self.lane] = token
        hid = t.zeros((self.n_lanes, self.d), dtype=t.float32, device="cuda")
        lg = t.zeros((self.n_lanes, self.V), dtype=t.float32, device="cuda")
        nx = t.zeros((self.n_lanes,), dtype=t.int32, device="cuda")
        if active is None:
            active = [i == self.lane for i in range(self.n_lanes)]
        self.m.decode_step(_toks(toks), active=active, hidden=hid, logits=lg, next_tok=nx)
        t.cuda.synchronize()
        return hid.cpu().numpy()[self.lane], lg.cpu().numpy()[self.lane], int(nx.cpu().numpy()[self.lane])


def _argmax_valid(tok, ref_logits):
    """The GPU's greedy token is a maximiser of the oracle logits up to the tolerance."""
    return ref_logits[tok] >= ref_logits.max() - TOL * np.abs(ref_logits).max()


def _parity(weights, om, prompt, L, steps, kv_int8, max_seq, label):
    kv = tl.TL_KV_INT8 if kv_int8 else tl.TL_KV_FP16
    m = _model(weights, max_seq=max_seq, max_loops=L, kv_dtype=kv, max_tokens=len(prompt))
    m.set_loops(0, L)
    g = GpuRun(m)
    cache = oracle.Cache(om.shape, max_seq, kv_int8)
    ro = oracle.forward(om, prompt, L, cache=cache)
    hid, lg, nx = g.prefill(prompt)
    e_h, e_l = rel_rows(hid, ro["hidden"]), rel_rows(lg, ro["logits"])
    print(f"{label} prefill: hidden {e_h:.2e} logits {e_l:.2e} argmax gpu={nx} oracle={int(np.argmax(ro['logits']))}")
    assert e_h < TOL and e_l < TOL
    assert _argmax_valid(nx, ro["logits"])
    tok = int(np.argmax(ro["logits"]))
    for t in range(steps):
        lo, ho = oracle.decode_step(om, cache, tok, L)
        hg, lgg, nxg = g.step(tok)
        e_h, e_l = rel_rows(hg, ho), rel_rows(lgg, lo)
        print(f"{label} step {t}: hidden {e_h:.2e} logits {e_l:.2e} argmax gpu={nxg} oracle={int(np.argmax(lo))}")
        assert e_h < TOL and e_l < TOL
        assert _argmax_valid(nxg, lo)
        tok = int(np.argmax(lo))
    assert m.length(0) == len(prompt) + steps
    m.close()


# ------------------------------------------------------------------ tiny model
@pytest.fixture(scope="module")
def tiny():
    s = synth.SHAPES["tiny"]
    w = synth.make_weights(s, seed=0)
    return w, oracle.OracleModel(w)


@pytest.fixture(scope="module")
def tiny_sharp():
    s = synth.SHAPES["tiny"]
    w = synth.make_weights(s, seed=1, gains="random", q_scale_mult=8.0)
    return w, oracle.OracleModel(w)


def test_tiny_prompt32_L4_8_decode_steps(tiny):
    w, om = tiny
    prompt = synth.make_tokens(w["shape"].vocab, 32, seed=0)
    _parity(w, om, prompt, L=4, steps=8, kv_int8=False, max_seq=64, label="tiny")


@pytest.mark.parametrize("kv_int8", [False, True])
@pytest.mark.parametrize("L,n", [(1, 1), (3, 70), (6, 130)])
def test_tiny_sharpened(tiny_sharp, kv_int8, L, n):
    w, om = tiny_sharp
    prompt = synth.make_tokens(w["shape"].vocab, n, seed=2)
    _parity(w, om, prompt, L=L, steps=3, kv_int8=kv_int8, max_seq=160, label=f"sharp L={L} n={n} int8={kv_int8}")


# ------------------------------------------------------------------ 407M-shaped model
@pytest.fixture(scope="module")
def m407():
    s = synth.SHAPES["m407"]
    w = synth.make_weights(s, seed=0)
    return w, oracle.OracleModel(w)


def test_407m_prefill_seq128_L8_full_size(m407):
    """The prefill-throughput shape: 128 tokens, L=8, every position compared."""
    w, om = m407
    prompt = synth.make_tokens(w["shape"].vocab, 128, seed=0)
    m = _model(w, max_seq=2048, max_loops=8, max_tokens=1024)
    m.set_loops(0, 8)
    hid, lg, nx = GpuRun(m).prefill(prompt)
    ro = oracle.forward(om, prompt, 8)
    e_h, e_l = rel_rows(hid, ro["hidden"]), rel_rows(lg, ro["logits"])
    print(f"407M seq128 L8: hidden {e_h:.2e} logits {e_l:.2e}")
    assert e_h < TOL and e_l < TOL
    m.close()


@pytest.mark.parametrize("n", [512, 600])
def test_407m_prefill_64_row_tiles(m407, n):
    """From 512 rows the QKV (RoPE epilogue), gate/up (SwiGLU epilogue), O and
    down (split-K partials summed by the next RMSNorm) GEMMs run 64-row tiles;
    below 641 rows gate/up has not yet switched to the 128-row tile. Every
    position against the oracle at L=2."""
    w, om = m407
    prompt = synth.make_tokens(w["shape"].vocab, n, seed=3)
    m = _model(w, max_seq=1024, max_loops=2, max_tokens=n)
    m.set_loops(0, 2)
    hid, lg, nx = GpuRun(m).prefill(prompt)
    ro = oracle.forward(om, prompt, 2)
    e_h, e_l = rel_rows(hid, ro["hidden"]), rel_rows(lg, ro["logits"])
    print(f"407M n={n} L2: hidden {e_h:.2e} logits {e_l:.2e}")
    assert e_h < TOL and e_l < TOL
    m.close()


@pytest.mark.parametrize("L", [8, 32])
@pytest.mark.parametrize("kv_int8", [False, True])
def test_407m_prefill_and_decode(m407, L, kv_int8):
    w, om = m407
    prompt = synth.make_tokens(w["shape"].vocab, 64, seed=0)
    _parity(w, om, prompt, L=L, steps=4, kv_int8=kv_int8, max_seq=256, label=f"407M L={L} int8={kv_int8}")


# ------------------------------------------------------------------ GPU-vs-GPU properties
def _tiny_model(w, **kw):
    kw.setdefault("max_seq", 128)
    kw.setdefault("max_loops", 8)
    return _model(w, **kw)


@pytest.mark.parametrize("kv", [0, 1])
def test_cached_decode_equals_uncached_recompute(tiny_sharp, kv):
    torch = _torch()
    w, _ = tiny_sharp
    prompt = synth.make_tokens(w["shape"].vocab, 40, seed=5)
    m = _tiny_model(w, n_lanes=2, kv_dtype=kv)
    m.set_loops(-1, 5)
    g = GpuRun(m, lane=0)
    _, lg, nx = g.prefill(prompt)
    seq = list(prompt)
    for _ in range(6):
        seq.append(nx)
        _, lg, nx = g.step(nx, active=[True, False])
    # uncached: the whole sequence in one prefill on lane 1
    g1 = GpuRun(m, lane=1)
    _, lg_u, nx_u = g1.prefill(seq)
    err = rel_rows(lg, lg_u)
    print(f"cached vs uncached kv={kv}: logits {err:.2e}")
    assert err < TOL
    m.close()


def test_variable_L_is_bit_exact(tiny_sharp):
    """A lane prefilled at L=8 and then run at L=3 equals a lane run at L=3 throughout."""
    w, _ = tiny_sharp
    prompt = synth.make_tokens(w["shape"].vocab, 33, seed=6)
    a = _tiny_model(w)
    a.set_loops(0, 8)
    ga = GpuRun(a)
    ga.prefill(prompt)
    a.set_loops(0, 3)
    b = _tiny_model(w)
    b.set_loops(0, 3)
    gb = GpuRun(b)
    gb.prefill(prompt)
    tok = 17
    for _ in range(4):
        ha, la, na = ga.step(tok)
        hb, lb, nb = gb.step(tok)
        assert np.array_equal(ha, hb) and np.array_equal(la, lb) and na == nb
        tok = na
    a.close()
    b.close()


def test_lanes_with_own_depth_are_batch_invariant(tiny_sharp):
    """Three lanes at L = 4, 16, 32 decoded together equal each lane decoded alone."""
    w, _ = tiny_sharp
    torch = _torch()
    loops = [4, 16, 32]
    prompts = [synth.make_tokens(w["shape"].vocab, 20 + 7 * i, seed=0, lane=i) for i in range(3)]

    def build():
        m = _tiny_model(w, n_lanes=3, max_loops=32, kv_dtype=tl.TL_KV_INT8)
        for i in range(3):
            m.set_loops(i, loops[i])
            GpuRun(m, lane=i).prefill(prompts[i])
        return m

    together, alone = build(), build()
    d, V = w["shape"].d_model, w["shape"].vocab
    tok = np.array([3, 5, 7], dtype=np.int32)
    for _ in range(3):
        hid = torch.zeros((3, d), dtype=torch.float32, device="cuda")
        lg = torch.zeros((3, V), dtype=torch.float32, device="cuda")
        nx = torch.zeros((3,), dtype=torch.int32, device="cuda")
        together.decode_step(_toks(tok), hidden=hid, logits=lg, next_tok=nx)
        for i in range(3):
            h1 = torch.zeros((3, d), dtype=torch.float32, device="cuda")
            l1 = torch.zeros((3, V), dtype=torch.float32, device="cuda")
            n1 = torch.zeros((3,), dtype=torch.int32, device="cuda")
            alone.decode_step(_toks(tok), active=[j == i for j in range(3)], hidden=h1, logits=l1, next_tok=n1)
            torch.cuda.synchronize()
            assert torch.equal(h1[i], hid[i]) and torch.equal(l1[i], lg[i]) and int(n1[i]) == int(nx[i])
        tok = nx.cpu().numpy().astype(np.int32)
    together.close()
    alone.close()


@pytest.mark.parametrize("kv", [0, 1])
def test_decode_lanes_across_part_size_thresholds(tiny_sharp, kv):
    """Five lanes whose contexts straddle the decode attention's part sizes
    (128 keys up to context 1024, 256 beyond), decoded together for 8 steps
    so that one lane crosses the threshold: each lane equals itself decoded
    alone, bit for bit (the together call merges 5 x 8 parts in the merge
    kernel, the lone calls inside the O-projection GEMV), and with FP16
    caches every row matches the oracle (teacher-forced)."""
    w, om = tiny_sharp
    s = w["shape"]
    torch = _torch()
    L, steps, max_seq = 2, 8, 1200
    lens = [100, 506, 700, 1019, 1100]
    n = len(lens)
    streams = [synth.make_tokens(s.vocab, P + steps, seed=5, lane=i) for i, P in enumerate(lens)]
    kvd = tl.TL_KV_INT8 if kv else tl.TL_KV_FP16

    def build():
        m = _model(w, max_seq=max_seq, max_loops=L, n_lanes=n, kv_dtype=kvd, max_tokens=max(lens))
        for i in range(n):
            m.set_loops(i, L)
            m.prefill(_toks(streams[i][:lens[i]]), lane=i)
        return m

    together, alone = build(), build()
    hid = torch.zeros((steps, n, s.d_model), dtype=torch.float32, device="cuda")
    lg = torch.zeros((steps, n, s.vocab), dtype=torch.float32, device="cuda")
    for t in range(steps):
        tok = [streams[i][lens[i] + t] for i in range(n)]
        together.decode_step(_toks(tok), hidden=hid[t], logits=lg[t])
        for i in range(n):
            h1 = torch.zeros((n, s.d_model), dtype=torch.float32, device="cuda")
            l1 = torch.zeros((n, s.vocab), dtype=torch.float32, device="cuda")
            alone.decode_step(_toks(tok), active=[j == i for j in range(n)], hidden=h1, logits=l1)
            torch.cuda.synchronize()
            assert torch.equal(h1[i], hid[t, i]) and torch.equal(l1[i], lg[t, i]), (t, i)
    torch.cuda.synchronize()
    together.close()
    alone.close()
    if kv:
        return
    hid, lg = hid.cpu().numpy(), lg.cpu().numpy()
    for i in range(n):
        ro = oracle.forward(om, streams[i], L, logits=None, max_seq=max_seq)
        ref_h = ro["hidden"][lens[i]:]
        e_h = rel_rows(hid[:, i], ref_h)
        e_l = rel_rows(lg[:, i], oracle.head_logits(om, ref_h))
        print(f"lane {i} ctx {lens[i]}..{lens[i] + steps}: hidden {e_h:.2e} logits {e_l:.2e}")
        assert e_h < TOL and e_l < TOL


def test_lanes_match_oracle(tiny_sharp):
    w, om = tiny_sharp
    loops = [4, 16, 32]
    prompts = [synth.make_tokens(w["shape"].vocab, 24 + 5 * i, seed=0, lane=i) for i in range(3)]
    m = _tiny_model(w, n_lanes=3, max_loops=32, kv_dtype=tl.TL_KV_INT8)
    caches = []
    for i in range(3):
        m.set_loops(i, loops[i])
        GpuRun(m, lane=i).prefill(prompts[i])
        c = oracle.Cache(om.shape, 128, kv_int8=True)
        oracle.forward(om, prompts[i], loops[i], cache=c)
        caches.append(c)
    torch = _torch()
    d, V = w["shape"].d_model, w["shape"].vocab
    tok = [11, 22, 33]
    for step in range(2):
        hid = torch.zeros((3, d), dtype=torch.float32, device="cuda")
        lg = torch.zeros((3, V), dtype=torch.float32, device="cuda")
        m.decode_step(_toks(tok), hidden=hid, logits=lg)
        torch.cuda.synchronize()
        for i in range(3):
            lo, ho = oracle.decode_step(om, caches[i], tok[i], loops[i])
            e_h, e_l = rel_rows(hid[i].cpu().numpy(), ho), rel_rows(lg[i].cpu().numpy(), lo)
            print(f"lane {i} L={loops[i]} step {step}: hidden {e_h:.2e} logits {e_l:.2e}")
            assert e_h < TOL and e_l < TOL
    m.close()


def test_wide_ffn_decode_with_split_down_projection():
    """ffn_dim 8320 is past the decode GEMV's limit for the down projection
    (more than 64 groups along K), so decode runs it on the prefill GEMM with
    K split over 8 blocks. Two lanes at L = 3 and 1 make the step's row count
    shrink from 2 to 1 after the first loop iteration; the split partials must
    reach x before that and before the head (a prefill keeps them pending for
    the next RMSNorm instead)."""
    import dataclasses
    s = dataclasses.replace(synth.SHAPES["tiny"], ffn_dim=8320)
    w = synth.make_weights(s, seed=3, gains="random")
    om = oracle.OracleModel(w)
    loops = [3, 1]
    m = _model(w, max_seq=64, max_loops=3, n_lanes=2, kv_dtype=tl.TL_KV_FP16, max_tokens=20)
    caches = []
    for i in range(2):
        m.set_loops(i, loops[i])
        prompt = synth.make_tokens(s.vocab, 12 + 5 * i, seed=3, lane=i)
        hid, lg, _ = GpuRun(m, lane=i).prefill(prompt)
        c = oracle.Cache(s, 64)
        ro = oracle.forward(om, prompt, loops[i], cache=c)
        assert rel_rows(hid, ro["hidden"]) < TOL and rel_rows(lg, ro["logits"]) < TOL
        caches.append(c)
    torch = _torch()
    tok = [5, 900]
    for step in range(4):
        hid = torch.zeros((2, s.d_model), dtype=torch.float32, device="cuda")
        lg = torch.zeros((2, s.vocab), dtype=torch.float32, device="cuda")
        m.decode_step(_toks(tok), hidden=hid, logits=lg)
        torch.cuda.synchronize()
        for i in range(2):
            lo, ho = oracle.decode_step(om, caches[i], tok[i], loops[i])
            e_h, e_l = rel_rows(hid[i].cpu().numpy(), ho), rel_rows(lg[i].cpu().numpy(), lo)
            print(f"ffn 8320 lane {i} L={loops[i]} step {step}: hidden {e_h:.2e} logits {e_l:.2e}")
            assert e_h < TOL and e_l < TOL
            tok[i] = int(np.argmax(lo))
    # a prefill after the decode steps starts clean (nothing pending carries over)
    m.reset(1)
    prompt = synth.make_tokens(s.vocab, 9, seed=4)
    hid, lg, _ = GpuRun(m, lane=1).prefill(prompt)
    ro = oracle.forward(om, prompt, loops[1], max_seq=64)
    assert rel_rows(hid, ro["hidden"]) < TOL and rel_rows(lg, ro["logits"]) < TOL
    m.close()


def test_repeated_runs_are_bit_identical(tiny_sharp):
    w, _ = tiny_sharp
    prompt = synth.make_tokens(w["shape"].vocab, 50, seed=9)
    outs = []
    for _ in range(2):
        m = _tiny_model(w)
        m.set_loops(0, 6)
        g = GpuRun(m)
        h, l, n = g.prefill(prompt)
        h2, l2, n2 = g.step(n)
        outs.append((h, l, h2, l2))
        m.close()
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_error_paths_leave_state_unchanged(tiny):
    w, _ = tiny
    m = _tiny_model(w, max_seq=40, max_loops=8, max_tokens=32)
    g = GpuRun(m)
    with pytest.raises(tl.TLError) as e:
        g.step(1)                                            # decode before any prefill
    assert e.value.status == tl.TL_E_STATE
    m.set_loops(0, 4)
    g.prefill(synth.make_tokens(w["shape"].vocab, 30, seed=1))
    with pytest.raises(tl.TLError) as e:
        m.set_loops(0, 5)                                    # deeper than the cached tokens
    assert e.value.status == tl.TL_E_STATE
    assert m.get_loops(0) == 4
    with pytest.raises(tl.TLError) as e:
        g.prefill(synth.make_tokens(w["shape"].vocab, 11, seed=1))   # 30 + 11 > max_seq
    assert e.value.status == tl.TL_E_RANGE
    with pytest.raises(tl.TLError) as e:
        m.set_loops(0, 9)
    assert e.value.status == tl.TL_E_RANGE
    with pytest.raises(tl.TLError) as e:
        m.set_loops(3, 2)
    assert e.value.status == tl.TL_E_INVAL
    assert m.length(0) == 30
    m.set_loops(0, 2)                                        # shallower is allowed
    g.step(5)
    assert m.length(0) == 31
    m.reset(0)
    assert m.length(0) == 0
    m.set_loops(0, 8)                                        # empty lane: any depth
    m.close()


def test_no_device_memory_growth(tiny):
    torch = _torch()
    w, _ = tiny
    prompt = _toks(synth.make_tokens(w["shape"].vocab, 16, seed=3))
    torch.cuda.synchronize()
    base = None
    for i in range(12):
        m = _tiny_model(w, max_seq=32)
        m.set_loops(0, 3)
        m.prefill(prompt)
        m.decode_step(_toks([1]))
        m.close()
        del m
        gc.collect()   # objects of earlier tests freed by a collection are not growth
        torch.cuda.synchronize()
        if i == 1:
            base = torch.cuda.memory_allocated()
    assert torch.cuda.memory_allocated() == base


def test_out_of_range_token_ids_are_clamped(tiny):
    """Token ids outside [0, vocab) read the row of the clamped id (the
    kernels never index the embedding out of bounds): the same bits as ids 0
    and vocab - 1, through the short-prefill GEMV path (5 rows), the GEMM
    path (20 rows) and a decode step."""
    w, _ = tiny
    V = w["shape"].vocab
    for n in (5, 20):
        good = synth.make_tokens(V, n, seed=3)
        bad, fix = good.copy(), good.copy()
        bad[0], bad[-1] = -5, V + 7
        fix[0], fix[-1] = 0, V - 1
        outs = []
        for toks, nxt in ((bad, V + 100), (fix, V - 1)):
            m = _tiny_model(w)
            m.set_loops(0, 2)
            g = GpuRun(m)
            h, lg, _ = g.prefill(toks)
            h2, lg2, _ = g.step(nxt)
            outs.append((h, lg, h2, lg2))
            m.close()
        for a, b in zip(*outs):
            assert np.array_equal(a, b)
