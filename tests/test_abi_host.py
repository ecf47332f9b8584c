"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point include/tl.h declares, and its size queries and argument
checks behave as documented."""
import ctypes
import json
import os
import re

import pytest

import synth
from tests.conftest import GOLDEN, ROOT, ensure_library

tl = ensure_library()


def _declared():
    text = open(os.path.join(ROOT, "include", "tl.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tl_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound():
    names = _declared()
    assert len(names) >= 18
    for n in names:
        assert hasattr(tl.lib, n), n
        assert n in tl.EXPORTED, n
        assert callable(getattr(tl, n)), n


def _cfg(shape="m407", max_seq=2048, max_loops=8, lanes=1, kv=0, max_tokens=128):
    from looped_weight_shared_amd.model import make_config
    return make_config(synth.SHAPES[shape], max_seq, max_loops, lanes, kv, max_tokens)


def test_kv_bytes_match_printed_page_numbers():
    g = json.load(open(os.path.join(GOLDEN, "kv_cache_memory.json")))
    fp16 = tl.tl_kv_layer_bytes(_cfg(kv=tl.TL_KV_FP16)) * g["n_layers"]
    int8 = tl.tl_kv_layer_bytes(_cfg(kv=tl.TL_KV_INT8)) * g["n_layers"]
    assert round(fp16 / 1e6, 1) == g["fp16_mb_printed"]
    assert round(int8 / 1e6, 1) == g["int8_mb_printed"]
    assert fp16 // (int8 // g["max_seq"]) == g["int8_context_printed"]
    # 2 pre-blocks + L=8 = 10 effective layers per lane
    assert tl.tl_kv_bytes(_cfg(kv=0)) == fp16
    assert tl.tl_kv_bytes(_cfg(kv=0, lanes=3)) == 3 * fp16


def test_weight_bytes_do_not_depend_on_loop_count():
    a = tl.tl_weights_ws_bytes(_cfg(max_loops=1))
    b = tl.tl_weights_ws_bytes(_cfg(max_loops=64))
    assert a == b > 0
    # three unique blocks of packed INT4 (close to 3 x 26.5 MB), the fp16 head
    # copied into tile order (206 MB: vocab is a multiple of 16) and the RoPE table
    nb = synth.weights_nbytes(synth.SHAPES["m407"])
    blk, head = nb["block_w4"], nb["head"]
    assert 3 * blk + head <= a < 3 * blk * 1.01 + head + 2 * 2048 * 64 * 4 + 4096


def test_packed_bytes():
    assert tl.tl_qlinear_packed_bytes(6144, 2048) == 6144 * 2048 // 2 + 6144 * 16 * 2
    assert tl.tl_qlinear_packed_bytes(256, 704) == 16 * 6 * (1024 + 32)   # K padded to 768
    assert tl.tl_qlinear_packed_bytes(8, 64) == 0
    assert tl.tl_qlinear_packed_bytes(16, 12) == 0


def test_bad_configs_are_rejected_without_a_gpu():
    bad = [dict(head_dim=96), dict(d_model=1000), dict(max_loops=0), dict(max_loops=65),
           dict(n_lanes=9), dict(group_size=64), dict(kv_dtype=4), dict(max_seq=0),
           dict(kv_dtype=3, n_heads=3, head_dim=64, d_model=192)]
    for kw in bad:
        c = _cfg()
        for k, v in kw.items():
            setattr(c, k, v)
        assert tl.tl_weights_ws_bytes(c) == 0, kw
        out = ctypes.c_void_p()
        w = tl.TlWeights()
        st = tl.lib.tl_create(ctypes.byref(c), ctypes.byref(w), None, None, None, None, ctypes.byref(out))
        assert st in (tl.TL_E_INVAL, tl.TL_E_RANGE), kw
        assert tl.tl_last_error()


def test_null_arguments_are_rejected():
    c = _cfg()
    out = ctypes.c_void_p()
    w = tl.TlWeights()
    assert tl.lib.tl_create(ctypes.byref(c), ctypes.byref(w), None, None, None, None,
                            ctypes.byref(out)) == tl.TL_E_INVAL
    assert tl.lib.tl_set_loops(None, 0, 4) == tl.TL_E_INVAL
    assert tl.lib.tl_prefill(None, 0, None, 1, None, None, None, None) == tl.TL_E_INVAL
    assert tl.lib.tl_decode_step(None, None, None, None, None, None, None) == tl.TL_E_INVAL
    assert tl.lib.tl_length(None, 0) == -1
    assert tl.lib.tl_qlinear_pack(None, None, 15, 8, None, None) == tl.TL_E_INVAL
    assert tl.lib.tl_kv_quantize_rows(None, 1, 130, None, None, None) == tl.TL_E_INVAL
    with pytest.raises(tl.TLError):
        tl.tl_set_loops(None, 0, 4)


def test_window_bounds_kv_memory():
    """cache_window W keeps a ring of W + max_tokens rows instead of max_seq
    ("Performance and Memory" page, "Sliding-Window Cache")."""
    import synth
    from looped_weight_shared_amd.model import make_config
    s = synth.SHAPES["tiny"]
    full = tl.tl_kv_layer_bytes(make_config(s, 2048, 4, max_tokens=64))
    win = tl.tl_kv_layer_bytes(make_config(s, 2048, 4, max_tokens=64, cache_window=256))
    assert win * 2048 == full * (256 + 64)
    assert tl.tl_kv_layer_bytes(make_config(s, 2048, 4, max_tokens=64, cache_window=4096)) == full
    assert tl.tl_kv_layer_bytes(make_config(s, 2048, 4, max_tokens=64, cache_window=-1)) == 0


def test_store_h_halves_kv_memory():
    """TL_KV_H16 keeps h [max_seq][d_model] per layer: half of FP16 K and V
    ("Current Status" page, KV-cache table: Store-h); not with a window."""
    import synth
    from looped_weight_shared_amd.model import make_config
    s = synth.SHAPES["m407"]
    fp16 = tl.tl_kv_layer_bytes(make_config(s, 2048, 8, kv_dtype=tl.TL_KV_FP16))
    h16 = tl.tl_kv_layer_bytes(make_config(s, 2048, 8, kv_dtype=tl.TL_KV_H16))
    assert 2 * h16 == fp16 and h16 == 2048 * 2048 * 2
    assert tl.tl_kv_layer_bytes(make_config(s, 2048, 8, kv_dtype=tl.TL_KV_H16, cache_window=64)) == 0


def test_store_h_int8_layer_bytes():
    """TL_KV_H8 keeps d_model codes and d_model / 128 fp16 scales per position,
    each plane 256-byte aligned ("Current Status" page, KV-cache table: Store-h
    INT8, 66-75% less than FP16 K/V); needs 128-element groups; no window."""
    import oracle
    import synth
    from looped_weight_shared_amd.model import make_config
    s = synth.SHAPES["m407"]
    fp16 = tl.tl_kv_layer_bytes(make_config(s, 2048, 8, kv_dtype=tl.TL_KV_FP16))
    h8 = tl.tl_kv_layer_bytes(make_config(s, 2048, 8, kv_dtype=tl.TL_KV_H8))
    assert h8 == 2048 * 2048 + 2048 * 16 * 2
    assert h8 * 10 == oracle.store_h_bytes(10, 2048, 2048, True)
    assert 0.66 <= 1 - h8 / fp16 <= 0.75
    odd = make_config(s, 100, 8, kv_dtype=tl.TL_KV_H8)
    assert tl.tl_kv_layer_bytes(odd) == -(-100 * 2048 // 256) * 256 + -(-100 * 16 * 2 // 256) * 256
    assert tl.tl_kv_layer_bytes(make_config(s, 2048, 8, kv_dtype=tl.TL_KV_H8, cache_window=64)) == 0
    t = synth.SHAPES["tiny"]
    if t.d_model % 128:
        assert tl.tl_kv_layer_bytes(make_config(t, 64, 2, kv_dtype=tl.TL_KV_H8)) == 0
