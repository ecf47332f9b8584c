"""Full-size GPU parity at the 407M shape, in the launch configurations the
benchmark and the workload sweep use.

- cached greedy decode: prompt 256, then 128 steps at L=8 with FP16 KV and the
  argmax fed back on the device, exactly as timed; the oracle recomputes the
  same 384-token sequence (cached decode equals uncached recompute);
- long prefill: 1024 tokens at L=16 and L=32 (18 and 34 effective layers);
  one oracle run at L=32 gives both references, because the residual after
  loop iteration k of any run is the final residual of a run at L=k;
- long context with INT8 KV: prompt 1920 + 128 decode steps, reaching
  max_seq = 2048; one lane at L=8, and three lanes with L = 4, 16, 32 decoded
  together. Every lane is checked against its own oracle run (its 2048-token
  stream at its own depth), and the deeper lanes also bit for bit against the
  same lane run alone (batch invariance).

Decode inputs are fixed token streams (teacher forcing): both sides consume
the same tokens. Errors are max row-relative errors (per position:
max|gpu - oracle| / max|oracle|) on the final residual and on the logits.
The INT8 cases are the most sensitive: a code decided on an fp16 value that
differs by one ulp between two correct evaluations moves by a whole step, and
a few residual rows of the synthetic model nearly cancel after the
pre-blocks; they stay within the bound because the prefill attention applies
the softmax weights with ~22 significant bits (an fp16-rounded P took the
1920-token INT8 prefill to 3.3e-3).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.conftest import ensure_library, rel_rows

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
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


@pytest.fixture(scope="module")
def m407():
    s = synth.SHAPES["m407"]
    w = synth.make_weights(s, seed=0)
    return w, oracle.OracleModel(w)


def _decode_stream(m, lanes, first, tokens, steps, greedy):
    """Runs `steps` decode steps on `lanes` (all active). Token of lane i at
    step t: tokens[i][t], or, if greedy, the device-side argmax of the previous
    call (first[i] is the device tensor the prefill wrote it to). Returns hidden
    [steps][n_lanes][d], logits [steps][n_lanes][V] and next tokens
    [steps][n_lanes]."""
    torch = _torch()
    s, n = m.shape, m.cfg.n_lanes
    hid = torch.zeros((steps, n, s.d_model), dtype=torch.float32, device="cuda")
    lg = torch.zeros((steps, n, s.vocab), dtype=torch.float32, device="cuda")
    nx = torch.zeros((steps + 1, n), dtype=torch.int32, device="cuda")
    if greedy:
        nx[0].copy_(first)
    active = [i in lanes for i in range(n)]
    for t in range(steps):
        if greedy:
            tok = nx[t]
        else:
            tok = _dev([tokens[i][t] if i in lanes else 0 for i in range(n)])
        m.decode_step(tok, active=active, hidden=hid[t], logits=lg[t], next_tok=nx[t + 1])
    torch.cuda.synchronize()
    return hid.cpu().numpy(), lg.cpu().numpy(), nx.cpu().numpy()[1:]


def _prefill(m, prompt, lane=0):
    torch = _torch()
    s = m.shape
    hid = torch.empty((len(prompt), s.d_model), dtype=torch.float32, device="cuda")
    lg = torch.empty((s.vocab,), dtype=torch.float32, device="cuda")
    nx = torch.zeros((m.cfg.n_lanes,), dtype=torch.int32, device="cuda")
    m.prefill(_dev(prompt), lane=lane, hidden=hid, logits=lg, next_tok=nx[lane:lane + 1])
    torch.cuda.synchronize()
    return hid.cpu().numpy(), lg.cpu().numpy(), nx


def test_407m_greedy_decode_prompt256_128_steps_L8(m407):
    """The decode leg of the benchmark: same context, same launches, greedy on the device."""
    w, om = m407
    s = w["shape"]
    P, D, L = 256, 128, 8
    prompt = synth.make_tokens(s.vocab, P, seed=0)
    m = _model(w, max_seq=2048, max_loops=L, kv_dtype=tl.TL_KV_FP16, max_tokens=P)
    m.set_loops(0, L)
    hp, lp, nx0 = _prefill(m, prompt)
    hid, lg, nx = _decode_stream(m, [0], nx0, None, D, greedy=True)
    assert m.length(0) == P + D
    m.close()
    gen = np.concatenate([[int(nx0[0].item())], nx[:, 0]])      # tokens the GPU chose
    seq = np.concatenate([prompt, gen[:D]]).astype(np.int32)   # positions 0 .. P+D-1
    ro = oracle.forward(om, seq, L, logits=None)
    ref_h = ro["hidden"]
    ref_l = oracle.head_logits(om, ref_h[P - 1:])               # prefill's last + every step
    e = [rel_rows(hp, ref_h[:P]), rel_rows(lp, ref_l[0]), rel_rows(hid[:, 0], ref_h[P:]),
         rel_rows(lg[:, 0], ref_l[1:])]
    print(f"greedy decode 256+128 L8: prefill hidden {e[0]:.2e} logits {e[1]:.2e}; "
          f"decode hidden {e[2]:.2e} logits {e[3]:.2e}")
    assert max(e) < TOL
    assert all(_argmax_ok(int(gen[t]), ref_l[t]) for t in range(D + 1))


def test_407m_long_prefill_seq1024_L16_L32(m407):
    w, om = m407
    s = w["shape"]
    prompt = synth.make_tokens(s.vocab, 1024, seed=0)
    ro = oracle.forward(om, prompt, 32, logits=None, trace=True)
    m = _model(w, max_seq=1024, max_loops=32, max_tokens=1024)
    for L in (16, 32):
        m.reset(0)
        m.set_loops(0, L)
        hid, lg, nx = _prefill(m, prompt)
        ref_h = ro["trace"][s.n_pre + L - 1]
        ref_l = oracle.head_logits(om, ref_h[-1:])[0]
        e_h, e_l = rel_rows(hid, ref_h), rel_rows(lg, ref_l)
        print(f"seq1024 L={L}: hidden {e_h:.2e} logits {e_l:.2e}")
        assert e_h < TOL and e_l < TOL
        assert _argmax_ok(int(nx[0].item()), ref_l)
    m.close()


def _int8_lane_vs_oracle(om, stream, L, hp, lp, hid, lg, label):
    """stream: the lane's 2048 tokens (1920 prompt + 128 decode inputs)."""
    P = 1920
    ro = oracle.forward(om, stream, L, logits=None, max_seq=2048, kv_int8=True)
    ref_h = ro["hidden"]
    ref_l = oracle.head_logits(om, ref_h[P - 1:])             # prefill's last row, then every step
    e = [rel_rows(hp, ref_h[:P]), rel_rows(lp, ref_l[0]), rel_rows(hid, ref_h[P:]),
         rel_rows(lg, ref_l[1:])]
    print(f"{label}: prefill hidden {e[0]:.2e} logits {e[1]:.2e}; decode hidden {e[2]:.2e} "
          f"logits {e[3]:.2e}")
    assert max(e) < TOL


def test_407m_int8_kv_ctx2048_L8(m407):
    w, om = m407
    s = w["shape"]
    stream = synth.make_tokens(s.vocab, 2048, seed=0, lane=0)
    m = _model(w, max_seq=2048, max_loops=8, kv_dtype=tl.TL_KV_INT8, max_tokens=1920)
    m.set_loops(0, 8)
    hp, lp, _ = _prefill(m, stream[:1920])
    hid, lg, _ = _decode_stream(m, [0], None, [stream[1920:]], 128, greedy=False)
    assert m.length(0) == 2048
    with pytest.raises(tl.TLError) as e:                      # the lane is full
        m.decode_step(_dev([0]))
    assert e.value.status == tl.TL_E_RANGE and m.length(0) == 2048
    m.close()
    _int8_lane_vs_oracle(om, stream, 8, hp, lp, hid[:, 0], lg[:, 0], "INT8 ctx2048 L=8")


def test_407m_int8_kv_ctx2048_lanes_4_16_32(m407):
    w, om = m407
    s = w["shape"]
    Ls = [4, 16, 32]
    streams = [synth.make_tokens(s.vocab, 2048, seed=0, lane=i) for i in range(3)]
    m = _model(w, max_seq=2048, max_loops=32, n_lanes=3, kv_dtype=tl.TL_KV_INT8, max_tokens=1920)
    pre = []
    for i, L in enumerate(Ls):
        m.set_loops(i, L)
        pre.append(_prefill(m, streams[i][:1920], lane=i)[:2])
    hid, lg, _ = _decode_stream(m, [0, 1, 2], None, [st[1920:] for st in streams], 128, greedy=False)
    assert [m.length(i) for i in range(3)] == [2048] * 3
    m.close()
    # each deeper lane alone, in its own context, gives the same bits
    for i in (1, 2):
        m1 = _model(w, max_seq=2048, max_loops=32, n_lanes=1, kv_dtype=tl.TL_KV_INT8, max_tokens=1920)
        m1.set_loops(0, Ls[i])
        hp1, lp1, _ = _prefill(m1, streams[i][:1920])
        h1, l1, _ = _decode_stream(m1, [0], None, [streams[i][1920:]], 128, greedy=False)
        m1.close()
        assert np.array_equal(hp1, pre[i][0]) and np.array_equal(lp1, pre[i][1])
        assert np.array_equal(h1[:, 0], hid[:, i]) and np.array_equal(l1[:, 0], lg[:, i])
    for i, L in enumerate(Ls):
        _int8_lane_vs_oracle(om, streams[i], L, pre[i][0], pre[i][1], hid[:, i], lg[:, i],
                             f"INT8 ctx2048 lanes[4,16,32] lane {i} L={L}")
