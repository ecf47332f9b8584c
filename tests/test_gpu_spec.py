"""GPU self-speculative decode (tl_spec_decode) against the oracle.

The emitted tokens must be the verify depth's greedy tokens: teacher-forced,
the oracle recomputes the consumed sequence at the verify depth, and every
emitted token must be an argmax of the oracle's logits at its position up to
the 2e-3 bound (a near-tie may resolve either way). The GPU's acceptance
bookkeeping is checked for consistency (rounds, drafted, accepted, emitted),
against plain GPU greedy decoding at the same depth, and the lane's state
afterwards (length, and the cache: a decode step after the call matches the
oracle too).
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


def _argmax_ok(tok, ref):
    return ref[tok] >= ref.max() - TOL * np.abs(ref).max()


def _prefill_next(m, prompt, lane=0):
    torch = _torch()
    nx = torch.zeros((m.cfg.n_lanes,), dtype=torch.int32, device="cuda")
    m.prefill(_dev(prompt), lane=lane, next_tok=nx[lane:lane + 1])
    torch.cuda.synchronize()
    return int(nx[lane].item())


def _check_vs_oracle(om, prompt, first, toks, L, max_seq):
    """first: the prefill's greedy token; toks: the n emitted after it."""
    gen = [first] + list(toks)
    seq = np.concatenate([prompt, gen[:-1]]).astype(np.int32)
    ro = oracle.forward(om, seq, L, logits=None, max_seq=max_seq)
    ref = oracle.head_logits(om, ro["hidden"][len(prompt) - 1:])
    bad = [t for t in range(len(gen)) if not _argmax_ok(gen[t], ref[t])]
    assert not bad, f"positions whose token is not the verify depth's greedy choice: {bad[:8]}"


@pytest.fixture(scope="module")
def tiny():
    s = synth.SHAPES["tiny"]
    w = synth.make_weights(s, seed=3)
    return s, w, oracle.OracleModel(w)


@pytest.mark.parametrize("ld,k", [(2, 4), (1, 1), (3, 7), (4, 3)])
def test_spec_decode_emits_verify_depth_greedy_tokens(tiny, ld, k):
    s, w, om = tiny
    L, P, n = 4, 24, 40
    prompt = synth.make_tokens(s.vocab, P, seed=1)
    m = _model(w, max_seq=128, max_loops=L, max_tokens=32)
    m.set_loops(0, L)
    t0 = _prefill_next(m, prompt)
    toks, st = m.spec_decode(t0, n, draft_loops=ld, k_draft=k)
    print(f"ld={ld} k={k}: rounds {st.rounds} drafted {st.drafted} accepted {st.accepted}")
    assert len(toks) == n and st.emitted == n
    assert m.length(0) == P + n and m.get_loops(0) == L
    assert 0 <= st.accepted <= st.drafted <= st.rounds * k
    assert st.accepted + st.rounds >= n
    if ld == L:
        assert st.accepted >= 0.9 * st.drafted   # same depth: drafts are the verifier's tokens
    # the cache afterwards: one more plain decode step from the last token
    torch = _torch()
    nx = torch.zeros((1,), dtype=torch.int32, device="cuda")
    m.decode_step(_dev([toks[-1]]), next_tok=nx)
    torch.cuda.synchronize()
    last = int(nx.item())
    m.close()
    _check_vs_oracle(om, prompt, t0, toks + [last], L, 128)


def test_spec_matches_plain_gpu_greedy(tiny):
    """Plain cached greedy decoding at the verify depth gives the same tokens
    (up to near-ties, which the oracle check above arbitrates)."""
    s, w, om = tiny
    L, P, n = 4, 24, 32
    prompt = synth.make_tokens(s.vocab, P, seed=5)
    torch = _torch()
    m = _model(w, max_seq=128, max_loops=L, max_tokens=32)
    m.set_loops(0, L)
    t0 = _prefill_next(m, prompt)
    nx = torch.zeros((n + 1, 1), dtype=torch.int32, device="cuda")
    nx[0, 0] = t0
    for t in range(n):
        m.decode_step(nx[t], next_tok=nx[t + 1])
    torch.cuda.synchronize()
    plain = [int(v) for v in nx[1:, 0].cpu().numpy()]
    m.reset(0)
    t0b = _prefill_next(m, prompt)
    spec, _ = m.spec_decode(t0b, n, draft_loops=2, k_draft=4)
    m.close()
    assert t0b == t0
    if spec != plain:
        i = next(j for j in range(n) if spec[j] != plain[j])
        seq = np.concatenate([prompt, [t0] + spec[:i]]).astype(np.int32)
        ref = oracle.head_logits(om, oracle.forward(om, seq, L, logits=None)["hidden"][-1:])[0]
        assert _argmax_ok(spec[i], ref) and _argmax_ok(plain[i], ref), "divergence is not a near-tie"


def test_spec_decode_to_max_seq_and_errors(tiny):
    s, w, om = tiny
    L, P = 3, 20
    max_seq = 36
    prompt = synth.make_tokens(s.vocab, P, seed=2)
    m = _model(w, max_seq=max_seq, max_loops=L, n_lanes=2, max_tokens=24)
    m.set_loops(0, L)
    m.set_loops(1, L)
    with pytest.raises(tl.TLError) as e:                       # empty lane
        m.spec_decode(1, 4, draft_loops=1, k_draft=2)
    assert e.value.status == tl.TL_E_STATE
    t0 = _prefill_next(m, prompt)
    for kw, status in [(dict(draft_loops=0, k_draft=2), tl.TL_E_RANGE),
                       (dict(draft_loops=L + 1, k_draft=2), tl.TL_E_RANGE),
                       (dict(draft_loops=1, k_draft=8), tl.TL_E_RANGE)]:
        with pytest.raises(tl.TLError) as e:
            m.spec_decode(t0, 4, **kw)
        assert e.value.status == status and m.length(0) == P
    with pytest.raises(tl.TLError) as e:
        m.spec_decode(s.vocab, 4, draft_loops=1, k_draft=2)
    assert e.value.status == tl.TL_E_RANGE
    # the other lane is untouched by lane 0's speculation
    p1 = synth.make_tokens(s.vocab, 8, seed=9)
    t1 = _prefill_next(m, p1, lane=1)
    n = max_seq - P                                            # fills every position
    toks, st = m.spec_decode(t0, n, draft_loops=1, k_draft=5)
    assert len(toks) == n and m.length(0) == max_seq and m.length(1) == 8
    with pytest.raises(tl.TLError) as e:                       # the lane is full
        m.spec_decode(toks[-1], 1, draft_loops=1, k_draft=2)
    assert e.value.status == tl.TL_E_RANGE and e.value.tokens == []
    more, _ = m.spec_decode(t1, 6, draft_loops=2, k_draft=3, lane=1)
    m.close()
    _check_vs_oracle(om, prompt, t0, toks, L, max_seq)
    _check_vs_oracle(om, p1, t1, more, L, max_seq)


@pytest.mark.slow
def test_407m_spec_decode_prompt256_L8():
    s = synth.SHAPES["m407"]
    w = synth.make_weights(s, seed=0)
    om = oracle.OracleModel(w)
    P, n, L = 256, 48, 8
    prompt = synth.make_tokens(s.vocab, P, seed=0)
    m = _model(w, max_seq=2048, max_loops=L, max_tokens=P)
    m.set_loops(0, L)
    t0 = _prefill_next(m, prompt)
    toks, st = m.spec_decode(t0, n, draft_loops=2, k_draft=4)
    print(f"407M L=8 draft L=2 k=4: rounds {st.rounds} drafted {st.drafted} accepted {st.accepted}")
    m.close()
    _check_vs_oracle(om, prompt, t0, toks, L, 2048)
