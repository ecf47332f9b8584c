"""GPU INT8 store-h cache (TL_KV_H8) against the oracle.

"Current Status" page, KV-cache table: Store-h INT8 (66-75% less memory than
FP16 K/V). The cache keeps each 128-element group of h as INT8 codes with one
fp16 scale (the INT8 K/V rule) and every call rebuilds K and V of the visible
positions from fp16(code * scale). Checked here: the codes and scales the GPU
stores are bit-identical to the oracle's quantizer applied to the GPU's own h
(read from a TL_KV_H16 run of the same tokens, whose first layer sees the same
h), prefill (one-shot and chunked) and teacher-forced decode against the
oracle's INT8 store-h forward, lanes at different depths, self-speculative
decode, and the 407M shape.
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


def _layer(m, lane, layer):
    """(raw bytes of one cache layer of one lane) as a host uint8 array."""
    lb = tl.tl_kv_layer_bytes(m.cfg)
    n_layers = m.cfg.n_pre + m.cfg.max_loops
    off = (lane * n_layers + layer) * lb
    return m.kv[off:off + lb].cpu().numpy()


def _h8(raw, S, d):
    hs = -(-S * d // 256) * 256
    q = raw[:S * d].view(np.int8).reshape(S, d)
    sc = raw[hs:hs + S * (d // 128) * 2].view(np.float16).reshape(S, d // 128)
    return q, sc


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


def test_first_layer_codes_are_the_quantizer_of_h(sharp):
    """Layer 0's h is the same in FP16 and INT8 store-h runs (the embedding's
    RMSNorm); the INT8 codes and scales must be exactly the oracle quantizer
    of the FP16 run's stored h rows, after a prefill and after decode steps."""
    s, w, _ = sharp
    S, n, L = 64, 37, 2
    toks = synth.make_tokens(s.vocab, n + 5, seed=8)
    rows = {}
    for kv in (tl.TL_KV_H16, tl.TL_KV_H8):
        m = _model(w, max_seq=S, max_loops=L, kv_dtype=kv, max_tokens=64)
        m.set_loops(0, L)
        m.prefill(_dev(toks[:n]))
        for t in range(5):
            m.decode_step(_dev([toks[n + t]]))
        _torch().cuda.synchronize()
        rows[kv] = _layer(m, 0, 0)
        m.close()
    h = rows[tl.TL_KV_H16][:S * s.d_model * 2].view(np.float16).reshape(S, s.d_model)[:n + 5]
    q, sc = _h8(rows[tl.TL_KV_H8], S, s.d_model)
    qo, so = oracle.h_quantize(h)
    assert np.array_equal(sc[:n + 5].view(np.uint16), so.view(np.uint16))
    assert np.array_equal(q[:n + 5], qo)
    assert np.abs(qo).max() == 127


@pytest.mark.parametrize("n,chunks,L", [(40, 40, 3), (57, 16, 5), (9, 9, 2)])
def test_prefill_matches_oracle(sharp, n, chunks, L):
    s, w, om = sharp
    toks = synth.make_tokens(s.vocab, n, seed=2)
    m = _model(w, max_seq=128, max_loops=L, kv_dtype=tl.TL_KV_H8, max_tokens=64)
    m.set_loops(0, L)
    hid, lg = _prefill_chunks(m, s, toks, chunks)
    m.close()
    ref = oracle.forward(om, toks, L, logits="last", max_seq=128, h_int8=True)
    e_h, e_l = rel_rows(hid, ref["hidden"]), rel_rows(lg[None], ref["logits"][None])
    print(f"H8 prefill n={n} chunks={chunks} L={L}: hidden {e_h:.2e} logits {e_l:.2e}")
    assert e_h < TOL and e_l < TOL


def test_decode_matches_oracle_two_depths(sharp):
    s, w, om = sharp
    Ls, P, steps = [2, 5], [20, 31], 16
    toks = [synth.make_tokens(s.vocab, P[i] + steps, seed=4, lane=i) for i in range(2)]
    m = _model(w, max_seq=96, max_loops=5, n_lanes=2, kv_dtype=tl.TL_KV_H8, max_tokens=32)
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
        ro = oracle.forward(om, toks[i], Ls[i], logits=None, max_seq=96, h_int8=True)
        ref_h = ro["hidden"][P[i]:]
        ref_l = oracle.head_logits(om, ref_h)
        e_h, e_l = rel_rows(hid[:, i], ref_h), rel_rows(lgs[:, i], ref_l)
        print(f"H8 decode lane {i} L={Ls[i]}: hidden {e_h:.2e} logits {e_l:.2e}")
        assert e_h < TOL and e_l < TOL


def test_spec_decode_in_h8_mode(sharp):
    s, w, om = sharp
    L, P, n = 4, 24, 24
    prompt = synth.make_tokens(s.vocab, P, seed=1)
    m = _model(w, max_seq=128, max_loops=L, kv_dtype=tl.TL_KV_H8, max_tokens=32)
    m.set_loops(0, L)
    torch = _torch()
    nx = torch.zeros((1,), dtype=torch.int32, device="cuda")
    m.prefill(_dev(prompt), next_tok=nx)
    t0 = int(nx.item())
    toks, st = m.spec_decode(t0, n, draft_loops=2, k_draft=4)
    m.close()
    gen = [t0] + toks
    seq = np.concatenate([prompt, gen[:-1]]).astype(np.int32)
    ref = oracle.head_logits(om, oracle.forward(om, seq, L, logits=None, h_int8=True)["hidden"][P - 1:])
    ok = [ref[t][gen[t]] >= ref[t].max() - TOL * np.abs(ref[t]).max() for t in range(len(gen))]
    assert all(ok)


def test_407m_prefill_and_decode_L8():
    s = synth.SHAPES["m407"]
    w = synth.make_weights(s, seed=0)
    om = oracle.OracleModel(w)
    P, steps, L = 128, 8, 8
    toks = synth.make_tokens(s.vocab, P + steps, seed=3)
    m = _model(w, max_seq=256, max_loops=L, kv_dtype=tl.TL_KV_H8, max_tokens=128)
    m.set_loops(0, L)
    torch = _torch()
    hp = torch.empty((P, s.d_model), dtype=torch.float32, device="cuda")
    m.prefill(_dev(toks[:P]), hidden=hp)
    hid = np.zeros((steps, s.d_model), np.float32)
    for t in range(steps):
        h = torch.zeros((1, s.d_model), dtype=torch.float32, device="cuda")
        m.decode_step(_dev([toks[P + t]]), hidden=h)
        hid[t] = h.cpu().numpy()[0]
    hp = hp.cpu().numpy()
    m.close()
    ref = oracle.forward(om, toks, L, logits=None, max_seq=256, h_int8=True)["hidden"]
    e_p, e_d = rel_rows(hp, ref[:P]), rel_rows(hid, ref[P:])
    print(f"407M H8 L=8: prefill {e_p:.2e} decode {e_d:.2e}")
    assert e_p < TOL and e_d < TOL
