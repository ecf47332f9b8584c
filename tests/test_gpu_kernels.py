"""GPU parity of single kernels through the C ABI: the INT4 repack and the
INT8 KV quantizer bit for bit against the oracle, and the W4 linear (decode
GEMV and prefill GEMM kernels) against the oracle's exact dequantize-then-matmul."""
import json
import os

import numpy as np
import pytest

import oracle
from tests.conftest import GOLDEN, ensure_library, rel_rows

pytestmark = pytest.mark.gpu
tl = ensure_library()


def _torch():
    import torch
    return torch


def dev(a):
    torch = _torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.float16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t, dtype=None):
    a = t.cpu().numpy()
    return a.view(dtype) if dtype is not None else a


def _linear(rng, N, K):
    qw = rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint32)
    sc = (0.02 / 7 * rng.uniform(0.5, 1.5, size=(N, -(-K // 128)))).astype(np.float16)
    return qw, sc


def _ws(N, K, M):
    from looped_weight_shared_amd.model import device_bytes
    return device_bytes(max(256, tl.tl_w4_linear_ws_bytes(N, K, M)))


def _packed(qw, sc, N, K):
    from looped_weight_shared_amd.model import device_bytes
    p = device_bytes(tl.tl_qlinear_packed_bytes(N, K))
    tl.tl_qlinear_pack(dev(qw), dev(sc), N, K, p)
    return p


@pytest.mark.parametrize("N,K", [(16, 8), (32, 704), (256, 256), (2048, 5632), (6144, 2048)])
def test_repack_is_bit_exact(N, K):
    torch = _torch()
    rng = np.random.default_rng(N + K)
    qw, sc = _linear(rng, N, K)
    p = _packed(qw, sc, N, K)
    q = torch.empty((N, K), dtype=torch.int8, device="cuda")
    s = torch.empty((N, -(-K // 128)), dtype=torch.int16, device="cuda")
    tl.tl_qlinear_unpack(p, N, K, q, s)
    torch.cuda.synchronize()
    assert np.array_equal(host(q), oracle.unpack_int4(qw))
    assert np.array_equal(host(s, np.float16).view(np.uint16), sc.view(np.uint16))


# 407M shapes at M = 100 and 130: ragged last row tiles, with and without K
# splits (the consumer sums the partials); QKV and gate/up shapes at M = 512,
# 700 (a ragged last row tile) and 1024, the long prefill's sizes; gate/up at
# M = 1000 and 1024 and QKV at M = 1400 take the large-M 128 x 128 blocks
# (ragged last row tiles at 1000 and 1400)
LIN_CASES = [(6144, 2048, m) for m in (1, 3, 8, 16, 17, 128, 130, 512, 700, 1024, 1400)] + \
            [(2048, 5632, m) for m in (1, 2, 64, 100, 1024)] + [(2048, 2048, 128), (2048, 2048, 1024)] + \
            [(256, 704, m) for m in (1, 5, 32, 33)] + [(11264, 2048, m) for m in (1, 100, 256, 600, 1000, 1024)] + \
            [(2048, 2048, 512)] + \
            [(1040, 2048, 600), (1040, 704, 130), (1040, 2048, 17), (16, 128, 40)]  # n-blocks not a multiple of the tile


@pytest.mark.parametrize("N,K,M", LIN_CASES)
def test_w4_linear_matches_oracle(N, K, M):
    torch = _torch()
    rng = np.random.default_rng(7 * N + K + M)
    qw, sc = _linear(rng, N, K)
    p = _packed(qw, sc, N, K)
    A = rng.standard_normal((M, K)).astype(np.float16)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = _ws(N, K, M)
    tl.tl_w4_linear(p, N, K, dev(A), M, C, ws)
    torch.cuda.synchronize()
    ref = A.astype(np.float64) @ oracle.dequantize(qw, sc).T
    err = rel_rows(host(C), ref)
    print(f"N={N} K={K} M={M} rel_row_err={err:.2e}")
    assert err < 1e-4
    # run twice: bit-identical
    C2 = torch.empty_like(C)
    tl.tl_w4_linear(p, N, K, dev(A), M, C2, ws)
    torch.cuda.synchronize()
    assert torch.equal(C, C2)


def test_gemm_tile_shapes_give_the_same_bits():
    """Without a K split every output element is summed in the same order (4
    MFMA k-steps per 128-column group, then one fp32 scale-and-add per group,
    groups in order) whatever the block tile, so the large-M 128 x 128 blocks
    and the 32-row blocks agree bit for bit on the rows they share."""
    torch = _torch()
    N, K = 11264, 2048
    rng = np.random.default_rng(12)
    qw, sc = _linear(rng, N, K)
    p = _packed(qw, sc, N, K)
    A = rng.standard_normal((1024, K)).astype(np.float16)
    big = torch.empty((1024, N), dtype=torch.float32, device="cuda")
    tl.tl_w4_linear(p, N, K, dev(A), 1024, big, _ws(N, K, 1024))      # 88 x 8 = 704 large blocks
    small = torch.empty((300, N), dtype=torch.float32, device="cuda")
    tl.tl_w4_linear(p, N, K, dev(A[:300]), 300, small, _ws(N, K, 300))  # 32-row tiles, K unsplit
    torch.cuda.synchronize()
    assert torch.equal(big[:300], small)


def test_gemv_rows_do_not_depend_on_batch():
    torch = _torch()
    N, K = 2048, 2048
    rng = np.random.default_rng(11)
    qw, sc = _linear(rng, N, K)
    p = _packed(qw, sc, N, K)
    A = rng.standard_normal((8, K)).astype(np.float16)
    full = torch.empty((8, N), dtype=torch.float32, device="cuda")
    ws = _ws(N, K, 8)
    tl.tl_w4_linear(p, N, K, dev(A), 8, full, ws)
    for m in range(8):
        one = torch.empty((1, N), dtype=torch.float32, device="cuda")
        tl.tl_w4_linear(p, N, K, dev(A[m:m + 1]), 1, one, ws)
        torch.cuda.synchronize()
        assert torch.equal(one[0], full[m])


def _quant_gpu(x):
    torch = _torch()
    rows, hd = x.shape
    q = torch.empty((rows, hd), dtype=torch.int8, device="cuda")
    s = torch.empty((rows,), dtype=torch.int16, device="cuda")
    tl.tl_kv_quantize_rows(dev(x), rows, hd, q, s)
    torch.cuda.synchronize()
    return host(q), host(s, np.float16)


def _adversarial_rows():
    rows = []
    # exact ties: scale 1/16 (amax 127/16), values (k + 1/2)/16
    k = np.arange(-127, 127)
    for start in range(0, len(k), 127):
        r = np.zeros(128)
        vals = (k[start:start + 127] + 0.5) / 16.0
        r[:len(vals)] = vals
        r[127] = 127 / 16.0
        rows.append(r)
    rows.append(np.zeros(128))                                    # zero row, scale 0
    r = np.zeros(128); r[0] = 2.0 ** -10; r[1] = -(2.0 ** -10); r[2] = 2.0 ** -24
    rows.append(r)                                                # subnormal scale, clamp
    r = np.full(128, 65504.0); r[::2] = -65504.0
    rows.append(r)                                                # largest finite fp16
    return np.array(rows).astype(np.float16)


@pytest.mark.parametrize("hd", [128, 64])
def test_kv_quantizer_bit_exact(hd):
    rng = np.random.default_rng(hd)
    parts = [(rng.standard_normal((4000, hd)) * sp).astype(np.float16) for sp in (0.01, 1.0, 40.0)]
    if hd == 128:
        parts.append(_adversarial_rows())
    x = np.concatenate(parts)
    q, s = _quant_gpu(x)
    qo, so = oracle.kv_quantize(x)
    assert np.array_equal(s.view(np.uint16), so.view(np.uint16))
    assert np.array_equal(q, qo)


def test_kv_quantizer_worked_rows():
    cases = json.load(open(os.path.join(GOLDEN, "kv_int8_worked.json")))["cases"]
    x = np.array([c["x"] for c in cases], dtype=np.float16)
    q, s = _quant_gpu(x)
    for i, c in enumerate(cases):
        assert float(s[i]) == c["scale"]
        assert q[i].tolist() == c["q"]


def _f16_tiles_to_matrix(raw, N, K):
    """FP16-body tiles ([nb][g][slot s][lane l][8], see tl_qlinear_pack_f16)
    -> fp16 [N][K]: element j of lane l in slot s is row 16nb + l%16, column
    128g + 32s + 8(l//16) + j."""
    G = -(-K // 128)
    t = raw.view(np.float16).reshape(N // 16, G, 4, 4, 16, 8)    # nb, g, s, l//16, l%16, j
    w = t.transpose(0, 4, 1, 2, 3, 5).reshape(N, G * 128)       # nb, l%16 | g, s, l//16, j
    return w[:, :K], w[:, K:]


def test_fp16_body_dequant_bit_exact_all_nibbles_all_finite_scales():
    """Each FP16-body weight is the exact product q * s rounded once to
    nearest even ("Performance and Memory" page, "FP16 body cache": weights
    dequantized to persistent FP16 at load time): every one of the 63,488
    finite fp16 scales (both signs, subnormals, the largest, where q * s
    overflows to inf) meets all 16 nibble values."""
    torch = _torch()
    from looped_weight_shared_amd.model import device_bytes
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    sc16 = bits[(bits & 0x7C00) != 0x7C00].view(np.float16)     # all finite fp16 values
    N, K = sc16.size, 128                                       # 63,488 rows = 3,968 n-blocks
    assert N % 16 == 0
    nib = (np.arange(K)[None, :] + np.arange(N)[:, None]) % 16  # every value 8x per row, shifted per row
    qw = np.zeros((N, K // 8), dtype=np.uint32)
    for j in range(8):
        qw |= nib[:, j::8].astype(np.uint32) << np.uint32(4 * j)
    sc = sc16.reshape(N, 1)
    p = device_bytes(tl.tl_qlinear_packed_f16_bytes(N, K))
    tl.tl_qlinear_pack_f16(dev(qw), dev(sc), N, K, p)
    torch.cuda.synchronize()
    got, pad = _f16_tiles_to_matrix(host(p), N, K)
    with np.errstate(over="ignore"):
        want = oracle.dequantize(qw, sc).astype(np.float16)     # exact product, one RNE rounding
    assert pad.size == 0
    g, w_ = got.view(np.uint16), want.view(np.uint16)
    # an exact product of 0 may carry either sign (0 * s with s < 0, q < 0 * +0):
    # both are the number fp16(q * s); everything else must match bit for bit
    zero = ((g & 0x7FFF) == 0) & ((w_ & 0x7FFF) == 0)
    print(f"{int((g != w_).sum())} elements differ, {int(((g != w_) & zero).sum())} of them signed zeros")
    assert ((g == w_) | zero).all()
    assert (g[~zero] == w_[~zero]).all() and zero.sum() < g.size // 8


@pytest.mark.parametrize("N,K", [(32, 40), (48, 704)])
def test_fp16_body_tiles_ragged_k(N, K):
    """Columns past K are +0 in the FP16-body tiles; the rest is RNE(q * s)."""
    torch = _torch()
    from looped_weight_shared_amd.model import device_bytes
    rng = np.random.default_rng(N * K)
    qw, sc = _linear(rng, N, K)
    p = device_bytes(tl.tl_qlinear_packed_f16_bytes(N, K))
    tl.tl_qlinear_pack_f16(dev(qw), dev(sc), N, K, p)
    torch.cuda.synchronize()
    got, pad = _f16_tiles_to_matrix(host(p), N, K)
    want = oracle.dequantize(qw, sc).astype(np.float16)
    g, w_ = got.view(np.uint16), want.view(np.uint16)
    assert ((g == w_) | (((g & 0x7FFF) == 0) & ((w_ & 0x7FFF) == 0))).all()
    assert not (pad.view(np.uint16) & 0x7FFF).any()
