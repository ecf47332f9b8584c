"""tl_w4_linear_noalloc: the W4 linear without a caller workspace (its split-K
partials live in a static device buffer inside the library). Through the C
ABI against tl_w4_linear on the same inputs (same kernels: bit-identical)
and against the oracle, on two calls in a row, the second with a smaller
input, with no device memory allocated by the calls."""
import numpy as np
import pytest

import oracle
from tests.conftest import ensure_library, rel_rows

pytestmark = pytest.mark.gpu
tl = ensure_library()


def _torch():
    import torch
    return torch


def _dev(a):
    torch = _torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.float16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def _case(rng, N, K):
    from looped_weight_shared_amd.model import device_bytes
    qw = rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint32)
    sc = (0.02 / 7 * rng.uniform(0.5, 1.5, size=(N, -(-K // 128)))).astype(np.float16)
    p = device_bytes(tl.tl_qlinear_packed_bytes(N, K))
    tl.tl_qlinear_pack(_dev(qw), _dev(sc), N, K, p)
    return qw, sc, p


def test_noalloc_matches_workspace_entry_point_twice_shrinking():
    torch = _torch()
    from looped_weight_shared_amd.model import device_bytes
    rng = np.random.default_rng(21)
    N, K = 2048, 5632                         # the down projection: K split 8 ways at M = 128
    qw, sc, p = _case(rng, N, K)
    W = oracle.dequantize(qw, sc)
    assert tl.tl_w4_linear_ws_bytes(N, K, 128) > 0
    assert tl.tl_w4_linear_ws_bytes(N, K, 128) <= tl.tl_w4_linear_noalloc_max_bytes()
    A = rng.standard_normal((128, K)).astype(np.float16)
    dA = _dev(A)
    Ms = (128, 40)                            # the second call is smaller
    outs = {M: torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda") for M in Ms}
    refs = {M: torch.empty((M, N), dtype=torch.float32, device="cuda") for M in Ms}
    wss = {M: device_bytes(max(256, tl.tl_w4_linear_ws_bytes(N, K, M))) for M in Ms}
    for M in Ms:
        tl.tl_w4_linear(p, N, K, dA, M, refs[M], wss[M])
    # set-up: the first call on a device looks up (and so maps) the static buffer
    tl.tl_w4_linear_noalloc(p, N, K, dA, 1, outs[Ms[1]])
    torch.cuda.synchronize()
    # every buffer exists before the no-alloc calls: free device memory must not move
    free0 = torch.cuda.mem_get_info()[0]
    for M in Ms:
        tl.tl_w4_linear_noalloc(p, N, K, dA, M, outs[M])
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0, M
    for M in Ms:
        assert torch.equal(outs[M], refs[M]), M
        err = rel_rows(outs[M].cpu().numpy(), A[:M].astype(np.float64) @ W.T)
        print(f"noalloc N={N} K={K} M={M}: bit-identical to tl_w4_linear; oracle row error {err:.2e}")
        assert err < 1e-4


def test_noalloc_gemv_and_unsplit_shapes_and_errors():
    torch = _torch()
    rng = np.random.default_rng(22)
    N, K = 256, 704
    qw, sc, p = _case(rng, N, K)
    W = oracle.dequantize(qw, sc)
    for M in (5, 33):                          # decode GEMV, then the GEMM
        A = rng.standard_normal((M, K)).astype(np.float16)
        C = torch.empty((M, N), dtype=torch.float32, device="cuda")
        tl.tl_w4_linear_noalloc(p, N, K, _dev(A), M, C)
        torch.cuda.synchronize()
        assert rel_rows(C.cpu().numpy(), A.astype(np.float64) @ W.T) < 1e-4
    with pytest.raises(tl.TLError) as e:
        tl.tl_w4_linear_noalloc(p, N, K, _dev(np.zeros((1, K), np.float16)), 0, C)
    assert e.value.status == tl.TL_E_RANGE
    with pytest.raises(tl.TLError) as e:
        tl.tl_w4_linear_noalloc(p, 250, K, _dev(np.zeros((1, K), np.float16)), 1, C)
    assert e.value.status == tl.TL_E_INVAL
