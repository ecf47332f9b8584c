"""GPU FP16 body (tl_config.fp16_body) against the oracle with fp16 weights.

"Performance and Memory" page, "FP16 body cache" / "Key Runtime Switches":
the body weights are dequantized once to persistent FP16 and the body GEMMs
run on them. The reference is the oracle with every block weight rounded to
float16 once (OracleModel(fp16_body=True)); prefill and teacher-forced decode
must agree to the 2e-3 row-relative bound, at the tiny shape (several M, so
the GEMM, its K-split plans and the GEMV all run on FP16 tiles) and at the
407M shape, with FP16, INT8 and store-h caches.
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


def _run(m, s, toks, P, steps):
    torch = _torch()
    h = torch.empty((P, s.d_model), dtype=torch.float32, device="cuda")
    lg = torch.empty((s.vocab,), dtype=torch.float32, device="cuda")
    m.prefill(_dev(toks[:P]), hidden=h, logits=lg)
    hid, lgs = [h.cpu().numpy()], [lg.cpu().numpy()]
    for t in range(steps):
        hd = torch.zeros((1, s.d_model), dtype=torch.float32, device="cuda")
        ld = torch.zeros((1, s.vocab), dtype=torch.float32, device="cuda")
        m.decode_step(_dev([toks[P + t]]), hidden=hd, logits=ld)
        hid.append(hd.cpu().numpy())
        lgs.append(ld[0].cpu().numpy())
    torch.cuda.synchronize()
    return np.concatenate(hid), np.array(lgs)


def _check(w, om16, s, P, steps, L, kv, max_tokens):
    toks = synth.make_tokens(s.vocab, P + steps, seed=6)
    m = _model(w, max_seq=P + steps + 8, max_loops=L, kv_dtype=kv, max_tokens=max_tokens, fp16_body=True)
    m.set_loops(0, L)
    hid, lgs = _run(m, s, toks, P, steps)
    m.close()
    ro = oracle.forward(om16, toks, L, logits=None, max_seq=P + steps + 8, kv_int8=kv == tl.TL_KV_INT8,
                        store_h=kv == tl.TL_KV_H16, h_int8=kv == tl.TL_KV_H8)
    ref_l = oracle.head_logits(om16, ro["hidden"][P - 1:])
    e_h, e_l = rel_rows(hid, ro["hidden"]), rel_rows(lgs, ref_l)
    print(f"fp16 body P={P} L={L} kv={kv}: hidden {e_h:.2e} logits {e_l:.2e}")
    assert e_h < TOL and e_l < TOL


@pytest.fixture(scope="module")
def tiny():
    s = synth.SHAPES["tiny"]
    w = synth.make_weights(s, seed=1, gains="random", q_scale_mult=8.0)
    return s, w, oracle.OracleModel(w, fp16_body=True)


@pytest.mark.parametrize("P,L,kv", [(5, 3, 0), (40, 3, 0), (130, 2, 0), (40, 3, 2), (40, 3, 3)])
def test_tiny_fp16_body(tiny, P, L, kv):
    s, w, om16 = tiny
    _check(w, om16, s, P, 6, L, kv, max_tokens=P)


@pytest.mark.slow
@pytest.mark.parametrize("kv", [0, 1])
def test_407m_fp16_body_prompt128_L8(kv):
    s = synth.SHAPES["m407"]
    w = synth.make_weights(s, seed=0)
    _check(w, oracle.OracleModel(w, fp16_body=True), s, 128, 8, 8, kv, max_tokens=128)


def test_fp16_body_weight_bytes():
    s = synth.SHAPES["m407"]
    from looped_weight_shared_amd.model import make_config
    w4 = tl.tl_weights_ws_bytes(make_config(s, 2048, 8))
    f16 = tl.tl_weights_ws_bytes(make_config(s, 2048, 8, fp16_body=True))
    head = ((s.vocab + 15) // 16) * (s.d_model // 32) * 1024
    print(f"weights workspace: W4 {w4} B, FP16 body {f16} B")
    assert f16 - head > 3.5 * (w4 - head)
