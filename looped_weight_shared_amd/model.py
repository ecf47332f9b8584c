"""Device-memory plumbing around the C ABI.

`Model` uploads canonical weights to device tensors, sizes and allocates the
three workspaces with the library's own *_bytes queries, and holds the tl_ctx.
Its methods forward to tl_prefill / tl_decode_step / tl_set_loops. Nothing is
computed here.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import (TL_KV_FP16, TlBlock, TlConfig, TlQLinear, TlWeights, tl_act_ws_bytes, tl_create,
               tl_decode_step, tl_destroy, tl_get_loops, tl_kv_bytes, tl_length, tl_prefill, tl_reset,
               tl_safety_last, tl_set_graphs, tl_set_loops, tl_set_safety, tl_spec_decode, tl_weights_ws_bytes)

_LINEARS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def make_config(shape, max_seq, max_loops, n_lanes=1, kv_dtype=TL_KV_FP16, max_tokens=None,
                cache_window=0, fp16_body=0) -> TlConfig:
    """TlConfig from a shape object with vocab/d_model/n_heads/... attributes."""
    return TlConfig(vocab=shape.vocab, d_model=shape.d_model, n_heads=shape.n_heads,
                    head_dim=shape.head_dim, ffn_dim=shape.ffn_dim, n_pre=shape.n_pre,
                    group_size=shape.group_size, rope_base=shape.rope_base, rms_eps=shape.rms_eps,
                    max_seq=max_seq, max_loops=max_loops, n_lanes=n_lanes, kv_dtype=kv_dtype,
                    max_tokens=max_tokens or max_seq, cache_window=cache_window,
                    fp16_body=1 if fp16_body else 0)


def device_bytes(nbytes: int, device="cuda") -> torch.Tensor:
    """A uint8 device buffer whose data_ptr() is 256-byte aligned."""
    t = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-t.data_ptr()) % 256
    return t[off:off + nbytes]


def _dev(a, device):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.float16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class Model:
    """A tl_ctx over synthetic canonical weights (dict as produced by synth.make_weights)."""

    def __init__(self, weights: dict, max_seq: int, max_loops: int, n_lanes: int = 1,
                 kv_dtype: int = TL_KV_FP16, max_tokens: int | None = None, device="cuda",
                 cache_window: int = 0, fp16_body: bool = False):
        self.shape = weights["shape"]
        self.cfg = make_config(self.shape, max_seq, max_loops, n_lanes, kv_dtype, max_tokens, cache_window,
                               fp16_body)
        self.device = device
        keep = []

        def up(a):
            t = _dev(a, device)
            keep.append(t)
            return t.data_ptr()

        def block(b):
            ql = {n: TlQLinear(up(b[n]["qweight"]), up(b[n]["scales"])) for n in _LINEARS}
            return TlBlock(attn_norm=up(b["attn_norm"]), mlp_norm=up(b["mlp_norm"]), **ql)

        pre = (TlBlock * max(1, len(weights["pre"])))(*[block(b) for b in weights["pre"]])
        loop = block(weights["loop"])
        # embed, head and norm gains are used in place by the library: keep them alive
        self._embed = _dev(weights["embed"], device)
        self._head = _dev(weights["head"], device)
        self._final_norm = _dev(weights["final_norm"], device)
        self._norms = [t for t in keep]  # attn/mlp norms are among these; all kept below
        w = TlWeights(embed=self._embed.data_ptr(), pre=ctypes.cast(pre, ctypes.POINTER(TlBlock)), loop=loop,
                      final_norm=self._final_norm.data_ptr(), head=self._head.data_ptr())
        self.weights_ws = device_bytes(tl_weights_ws_bytes(self.cfg), device)
        self.kv = device_bytes(tl_kv_bytes(self.cfg), device)
        self.act_ws = device_bytes(tl_act_ws_bytes(self.cfg), device)
        self.ctx = tl_create(self.cfg, w, self.weights_ws, self.kv, self.act_ws)
        torch.cuda.synchronize()
        # canonical INT4 words and scales were repacked; norms stay referenced
        self._keep = keep

    # -- forwarding -------------------------------------------------------
    def set_loops(self, lane, loops):
        tl_set_loops(self.ctx, lane, loops)

    def set_safety(self, max_norm: float):
        tl_set_safety(self.ctx, max_norm)

    def safety_last(self):
        return tl_safety_last(self.ctx)

    def set_graphs(self, enable):
        """bit mask: 1 = prefill, 2 = decode steps (True = 1)."""
        tl_set_graphs(self.ctx, enable)

    def get_loops(self, lane):
        return tl_get_loops(self.ctx, lane)

    def reset(self, lane=-1):
        tl_reset(self.ctx, lane)

    def length(self, lane=0):
        return tl_length(self.ctx, lane)

    def prefill(self, tokens: torch.Tensor, lane=0, hidden=None, logits=None, next_tok=None, stream=None):
        tl_prefill(self.ctx, lane, tokens, int(tokens.numel()), hidden, logits, next_tok, stream)

    def spec_decode(self, token: int, n_new: int, draft_loops: int, k_draft: int, lane=0, stream=None):
        """Self-speculative greedy decode: (tokens, TlSpecStats)."""
        return tl_spec_decode(self.ctx, lane, token, draft_loops, k_draft, n_new, stream)

    def decode_step(self, tokens: torch.Tensor, active=None, hidden=None, logits=None, next_tok=None,
                    stream=None):
        tl_decode_step(self.ctx, tokens, active, hidden, logits, next_tok, stream)

    def close(self):
        if self.ctx:
            tl_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
