"""Python binding of libtl, the MI355X (gfx950) looped weight-shared transformer library.

Argument marshalling only: every function below calls the C entry point of the
same name in libtl.so (declared in include/tl.h). PyTorch supplies device
memory (tensor.data_ptr()) and streams (torch.cuda.current_stream()); all
computation runs in the library's HIP kernels. There is no CPU fallback:
importing this package fails loudly when libtl.so has not been built.
"""
from __future__ import annotations

import ctypes
import os

# PyTorch ships its own HIP runtime (soname libamdhip64.so.7). Loading torch
# first makes libtl.so bind to that same runtime, so the device pointers and
# stream handles torch hands over are valid inside the library; loading
# libtl.so first would map a second HIP runtime into the process.
import torch  # noqa: F401  (must precede the CDLL below)

__all__ = [
    "TLError", "TlConfig", "TlQLinear", "TlBlock", "TlWeights", "lib", "LIB_PATH",
    "TL_OK", "TL_E_INVAL", "TL_E_RANGE", "TL_E_STATE", "TL_E_HIP", "TL_E_UNSUPPORTED", "TL_E_SAFETY",
    "tl_set_safety", "tl_safety_last",
    "TL_KV_FP16", "TL_KV_INT8", "TL_KV_H16", "TL_KV_H8",
    "tl_weights_ws_bytes", "tl_kv_layer_bytes", "tl_kv_bytes", "tl_act_ws_bytes", "tl_create",
    "tl_destroy", "tl_set_loops", "tl_get_loops", "tl_reset", "tl_length", "tl_prefill", "tl_set_graphs", "tl_spec_decode", "TlSpecStats",
    "tl_decode_step", "tl_last_error", "tl_qlinear_packed_bytes", "tl_qlinear_pack",
    "tl_qlinear_packed_f16_bytes", "tl_qlinear_pack_f16",
    "tl_qlinear_unpack", "tl_w4_linear_ws_bytes", "tl_w4_linear", "tl_w4_linear_noalloc_max_bytes",
    "tl_w4_linear_noalloc", "tl_kv_quantize_rows", "tl_profile_begin", "tl_profile_end", "tl_launch_empty",
    "KERNEL_KINDS", "EXPORTED",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtl.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with python looped_weight_shared_amd/build.py")
lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes():
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


if len(_hip_runtimes()) > 1:
    raise ImportError("two HIP runtimes are mapped (libtl.so was loaded before torch): "
                      + ", ".join(_hip_runtimes()))

TL_OK, TL_E_INVAL, TL_E_RANGE, TL_E_STATE, TL_E_HIP, TL_E_UNSUPPORTED, TL_E_SAFETY = range(7)
TL_KV_FP16, TL_KV_INT8, TL_KV_H16, TL_KV_H8 = 0, 1, 2, 3

_i32, _f32, _sz, _vp = ctypes.c_int32, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


class TlConfig(ctypes.Structure):
    _fields_ = [("vocab", _i32), ("d_model", _i32), ("n_heads", _i32), ("head_dim", _i32),
                ("ffn_dim", _i32), ("n_pre", _i32), ("group_size", _i32), ("rope_base", _f32),
                ("rms_eps", _f32), ("max_seq", _i32), ("max_loops", _i32), ("n_lanes", _i32),
                ("kv_dtype", _i32), ("max_tokens", _i32), ("cache_window", _i32), ("fp16_body", _i32)]


class TlQLinear(ctypes.Structure):
    _fields_ = [("qweight", _vp), ("scales", _vp)]


class TlBlock(ctypes.Structure):
    _fields_ = [("attn_norm", _vp), ("wq", TlQLinear), ("wk", TlQLinear), ("wv", TlQLinear),
                ("wo", TlQLinear), ("mlp_norm", _vp), ("w_gate", TlQLinear), ("w_up", TlQLinear),
                ("w_down", TlQLinear)]


class TlWeights(ctypes.Structure):
    _fields_ = [("embed", _vp), ("pre", ctypes.POINTER(TlBlock)), ("loop", TlBlock),
                ("final_norm", _vp), ("head", _vp)]


class TlSpecStats(ctypes.Structure):
    _fields_ = [("rounds", _i32), ("drafted", _i32), ("accepted", _i32), ("emitted", _i32)]


_CFG = ctypes.POINTER(TlConfig)
_SIGS = {
    "tl_weights_ws_bytes": (_sz, [_CFG]),
    "tl_kv_layer_bytes": (_sz, [_CFG]),
    "tl_kv_bytes": (_sz, [_CFG]),
    "tl_act_ws_bytes": (_sz, [_CFG]),
    "tl_create": (ctypes.c_int, [_CFG, ctypes.POINTER(TlWeights), _vp, _vp, _vp, _vp, ctypes.POINTER(_vp)]),
    "tl_destroy": (ctypes.c_int, [_vp]),
    "tl_set_loops": (ctypes.c_int, [_vp, _i32, _i32]),
    "tl_get_loops": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(_i32)]),
    "tl_reset": (ctypes.c_int, [_vp, _i32]),
    "tl_length": (_i32, [_vp, _i32]),
    "tl_prefill": (ctypes.c_int, [_vp, _i32, _vp, _i32, _vp, _vp, _vp, _vp]),
    "tl_decode_step": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "tl_set_graphs": (ctypes.c_int, [_vp, _i32]),
    "tl_set_safety": (ctypes.c_int, [_vp, _f32]),
    "tl_safety_last": (ctypes.c_int, [_vp, ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "tl_spec_decode": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_i32),
                                      ctypes.POINTER(TlSpecStats), _vp]),
    "tl_last_error": (ctypes.c_char_p, []),
    "tl_qlinear_packed_bytes": (_sz, [_i32, _i32]),
    "tl_qlinear_pack": (ctypes.c_int, [_vp, _vp, _i32, _i32, _vp, _vp]),
    "tl_qlinear_packed_f16_bytes": (_sz, [_i32, _i32]),
    "tl_qlinear_pack_f16": (ctypes.c_int, [_vp, _vp, _i32, _i32, _vp, _vp]),
    "tl_qlinear_unpack": (ctypes.c_int, [_vp, _i32, _i32, _vp, _vp, _vp]),
    "tl_w4_linear_ws_bytes": (_sz, [_i32, _i32, _i32]),
    "tl_w4_linear": (ctypes.c_int, [_vp, _i32, _i32, _vp, _i32, _vp, _vp, _vp]),
    "tl_w4_linear_noalloc_max_bytes": (_sz, []),
    "tl_w4_linear_noalloc": (ctypes.c_int, [_vp, _i32, _i32, _vp, _i32, _vp, _vp]),
    "tl_kv_quantize_rows": (ctypes.c_int, [_vp, _i32, _i32, _vp, _vp, _vp]),
    "tl_profile_begin": (ctypes.c_int, [_vp, _i32]),
    "tl_launch_empty": (ctypes.c_int, [_i32, _vp]),
    "tl_profile_end": (ctypes.c_int, [_vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i32)]),
}
EXPORTED = tuple(_SIGS)
for _name, (_res, _args) in _SIGS.items():
    try:
        _fn = getattr(lib, _name)
    except AttributeError as _e:
        raise ImportError(f"{LIB_PATH} lacks {_name}: it is older than the sources, rebuild it") from _e
    _fn.restype = _res
    _fn.argtypes = _args


class TLError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


def _ptr(t):
    """Device address of a tensor (or None/int passthrough)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status):
    if status != TL_OK:
        raise TLError(status, lib.tl_last_error().decode())


def tl_last_error() -> str:
    return lib.tl_last_error().decode()


def tl_weights_ws_bytes(cfg: TlConfig) -> int:
    return lib.tl_weights_ws_bytes(ctypes.byref(cfg))


def tl_kv_layer_bytes(cfg: TlConfig) -> int:
    return lib.tl_kv_layer_bytes(ctypes.byref(cfg))


def tl_kv_bytes(cfg: TlConfig) -> int:
    return lib.tl_kv_bytes(ctypes.byref(cfg))


def tl_act_ws_bytes(cfg: TlConfig) -> int:
    return lib.tl_act_ws_bytes(ctypes.byref(cfg))


def tl_create(cfg: TlConfig, weights: TlWeights, weights_ws, kv, act_ws, stream=None):
    out = _vp()
    _check(lib.tl_create(ctypes.byref(cfg), ctypes.byref(weights), _ptr(weights_ws), _ptr(kv), _ptr(act_ws),
                         _stream(stream), ctypes.byref(out)))
    return out.value


def tl_destroy(ctx) -> None:
    _check(lib.tl_destroy(ctx))


def tl_set_loops(ctx, lane: int, loops: int) -> None:
    _check(lib.tl_set_loops(ctx, lane, loops))


def tl_set_safety(ctx, max_norm: float) -> None:
    _check(lib.tl_set_safety(ctx, max_norm))


def tl_safety_last(ctx):
    """(iteration, row) of the last trip, or (-1, -1)."""
    it, row = _i32(), _i32()
    _check(lib.tl_safety_last(ctx, ctypes.byref(it), ctypes.byref(row)))
    return it.value, row.value


def tl_set_graphs(ctx, enable) -> None:
    """enable: bit mask, 1 = prefill, 2 = decode steps (True = 1, False = 0)."""
    _check(lib.tl_set_graphs(ctx, int(enable)))


def tl_get_loops(ctx, lane: int) -> int:
    v = _i32()
    _check(lib.tl_get_loops(ctx, lane, ctypes.byref(v)))
    return v.value


def tl_reset(ctx, lane: int = -1) -> None:
    _check(lib.tl_reset(ctx, lane))


def tl_length(ctx, lane: int) -> int:
    return lib.tl_length(ctx, lane)


def tl_prefill(ctx, lane: int, tokens, n: int, hidden=None, logits=None, next_tok=None, stream=None) -> None:
    _check(lib.tl_prefill(ctx, lane, _ptr(tokens), n, _ptr(hidden), _ptr(logits), _ptr(next_tok),
                          _stream(stream)))


def tl_spec_decode(ctx, lane: int, token: int, draft_loops: int, k_draft: int, n_new: int, stream=None):
    """Returns (tokens: list of n_new ints, TlSpecStats). On an error the
    TLError carries the tokens emitted before it as .tokens."""
    out = (_i32 * max(n_new, 1))()
    st = TlSpecStats()
    rc = lib.tl_spec_decode(ctx, lane, token, draft_loops, k_draft, n_new, out, ctypes.byref(st), _stream(stream))
    toks = list(out[:n_new])
    if rc != TL_OK:
        err = TLError(rc, lib.tl_last_error().decode())
        err.tokens = toks[:st.emitted]
        raise err
    return toks, st


def tl_decode_step(ctx, tokens, active=None, hidden=None, logits=None, next_tok=None, stream=None) -> None:
    act = None
    if active is not None:
        act = (ctypes.c_uint8 * len(active))(*[1 if a else 0 for a in active])
    _check(lib.tl_decode_step(ctx, _ptr(tokens), act, _ptr(hidden), _ptr(logits), _ptr(next_tok),
                              _stream(stream)))


def tl_qlinear_packed_bytes(N: int, K: int) -> int:
    return lib.tl_qlinear_packed_bytes(N, K)


def tl_qlinear_pack(qweight, scales, N: int, K: int, packed, stream=None) -> None:
    _check(lib.tl_qlinear_pack(_ptr(qweight), _ptr(scales), N, K, _ptr(packed), _stream(stream)))


def tl_qlinear_packed_f16_bytes(N: int, K: int) -> int:
    return lib.tl_qlinear_packed_f16_bytes(N, K)


def tl_qlinear_pack_f16(qweight, scales, N: int, K: int, packed, stream=None) -> None:
    _check(lib.tl_qlinear_pack_f16(_ptr(qweight), _ptr(scales), N, K, _ptr(packed), _stream(stream)))


def tl_qlinear_unpack(packed, N: int, K: int, q, scales, stream=None) -> None:
    _check(lib.tl_qlinear_unpack(_ptr(packed), N, K, _ptr(q), _ptr(scales), _stream(stream)))


def tl_w4_linear_ws_bytes(N: int, K: int, M: int) -> int:
    return lib.tl_w4_linear_ws_bytes(N, K, M)


def tl_w4_linear(packed, N: int, K: int, A, M: int, C, ws, stream=None) -> None:
    _check(lib.tl_w4_linear(_ptr(packed), N, K, _ptr(A), M, _ptr(C), _ptr(ws), _stream(stream)))


def tl_w4_linear_noalloc_max_bytes() -> int:
    return lib.tl_w4_linear_noalloc_max_bytes()


def tl_w4_linear_noalloc(packed, N: int, K: int, A, M: int, C, stream=None) -> None:
    _check(lib.tl_w4_linear_noalloc(_ptr(packed), N, K, _ptr(A), M, _ptr(C), _stream(stream)))


def tl_kv_quantize_rows(x, rows: int, hd: int, q, s, stream=None) -> None:
    _check(lib.tl_kv_quantize_rows(_ptr(x), rows, hd, _ptr(q), _ptr(s), _stream(stream)))


KERNEL_KINDS = ("embed", "norm", "qkv", "rope_kv", "attn", "o", "gate_up", "down", "head", "argmax", "copy",
                "safety")


def tl_launch_empty(n: int, stream=None) -> None:
    _check(lib.tl_launch_empty(n, _stream(stream)))


def tl_profile_begin(ctx, max_launches: int) -> None:
    _check(lib.tl_profile_begin(ctx, max_launches))


def tl_profile_end(ctx) -> dict:
    """{kind: (launches, total_ms)} for the window that just closed."""
    n = len(KERNEL_KINDS)
    tot = (ctypes.c_double * n)()
    cnt = (_i32 * n)()
    _check(lib.tl_profile_end(ctx, tot, cnt))
    return {k: (int(cnt[i]), float(tot[i])) for i, k in enumerate(KERNEL_KINDS)}
