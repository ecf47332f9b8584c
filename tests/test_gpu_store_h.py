"""GPU store-h cache (TL_KV_H16) against FP16 K/V storage and the oracle.

"Current Status" page, KV-cache table (Store-h FP16: bit-exact, 43-50% less
KV memory) and "Claims & Data Sources" (h-mode KV reconstruction from the
shared W_k / W_v). The library keeps h per position and layer and rebuilds K
and V with the same W4 GEMM arithmetic the FP16 mode's prefill uses (K never
split, the RoPE epilogue), so prefills must be bit-identical to TL_KV_FP16
(one-shot and chunked, tiny and 407M shapes). Decode steps write K/V from the
decode GEMV in FP16 mode but rebuild them by GEMM here, so decode is compared
with the oracle (teacher-forced, 2e-3), with lanes at different depths, and
through self-speculative decode.
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


def _prefill_chunks(m, s, toks, chunks, lane=0):
    torch = _torch()
    hs, lg = [], None
    for c0 in range(0, len(toks), chunks):
        part = toks[c0:c0 + chunks]
        h = torch.empty((len(part), s.d_model), dtype=torch.float32, device="cuda")
        lgt = torch.empty((s.vocab,), dtype=torch.float32, device="cuda")
        m.prefill(_dev(part), lane=lane, hidden=h, logits=lgt)
        hs.append(h.cpu().numpy())
        lg = lgt.cpu().numpy()
    return np.concatenate(hs), lg


@pytest.mark.parametrize("n,chunks,L", [(40, 40, 3), (40, 24, 3), (57, 16, 5), (9, 9, 2)])
def test_prefill_bit_identical_to_fp16(sharp, n, chunks, L):
    s, w, _ = sharp
    toks = synth.make_tokens(s.vocab, n, seed=2)
    out = []
    for kv in (tl.TL_KV_FP16, tl.TL_KV_H16):
        m = _model(w, max_seq=128, max_loops=L, kv_dtype=kv, max_tokens=64)
        m.set_loops(0, L)
        out.append(_prefill_chunks(m, s, toks, chunks))
        m.close()
    assert np.array_equal(out[0][0], out[1][0]) and np.array_equal(out[0][1], out[1][1])


@pytest.mark.slow
def test_407m_prefill_seq128_L8_bit_identical():
    s = synth.SHAPES["m407"]
    w = synth.make_weights(s, seed=0)
    toks = synth.make_tokens(s.vocab, 128, seed=0)
    out = []
    for kv in (tl.TL_KV_FP16, tl.TL_KV_H16):
        m = _model(w, max_seq=512, max_loops=8, kv_dtype=kv, max_tokens=128)
        m.set_loops(0, 8)
        out.append(_prefill_chunks(m, s, toks, 128))
        m.close()
    assert np.array_equal(out[0][0], out[1][0]) and np.array_equal(out[0][1], out[1][1])


def test_decode_matches_oracle_two_depths(sharp):
    s, w, om = sharp
    Ls, P, steps = [2, 5], [20, 31], 16
    toks = [synth.make_tokens(s.vocab, P[i] + steps, seed=4, lane=i) for i in range(2)]
    m = _model(w, max_seq=96, max_loops=5, n_lanes=2, kv_dtype=tl.TL_KV_H16, max_tokens=32)
    torch = _torch()
    for i in range(2):
        m.set_loops(i, Ls[i])
        m.prefill(_dev(toks[i][:P[i]]), lane=i)
    hid = np.zeros((steps, 2, s.d_model), np.float32)
    lgs = np.zeros((steps, 2, s.vocab), np.float32)
    for t in range(steps):
        h = torch.zeros((2, s.d_model), dtype=torch.float32, device="cuda")
        lg = torch.zeros((2, s.vocab), dtype=torch.float32, device="cuda")
        m.decode_step(_dev([toks[0][P[0] + t], toks[1][P[1] + t]]), hidden=h, logits=lg)
        hid[t], lgs[t] = h.cpu().numpy(), lg.cpu().numpy()
    m.close()
    for i in range(2):
        ro = oracle.forward(om, toks[i], Ls[i], logits=None, max_seq=96, store_h=True)
        ref_h = ro["hidden"][P[i]:]
        ref_l = oracle.head_logits(om, ref_h)
        e_h, e_l = rel_rows(hid[:, i], ref_h), rel_rows(lgs[:, i], ref_l)
        print(f"store-h decode lane {i} L={Ls[i]}: hidden {e_h:.2e} logits {e_l:.2e}")
        assert e_h < TOL and e_l < TOL


def test_spec_decode_in_store_h_mode(sharp):
    s, w, om = sharp
    L, P, n = 4, 24, 24
    prompt = synth.make_tokens(s.vocab, P, seed=1)
    m = _model(w, max_seq=128, max_loops=L, kv_dtype=tl.TL_KV_H16, max_tokens=32)
    m.set_loops(0, L)
    torch = _torch()
    nx = torch.zeros((1,), dtype=torch.int32, device="cuda")
    m.prefill(_dev(prompt), next_tok=nx)
    t0 = int(nx.item())
    toks, st = m.spec_decode(t0, n, draft_loops=2, k_draft=4)
    m.close()
    gen = [t0] + toks
    seq = np.concatenate([prompt, gen[:-1]]).astype(np.int32)
    ref = oracle.head_logits(om, oracle.forward(om, seq, L, logits=None, store_h=True)["hidden"][P - 1:])
    ok = [ref[t][gen[t]] >= ref[t].max() - TOL * np.abs(ref[t]).max() for t in range(len(gen))]
    assert all(ok)
