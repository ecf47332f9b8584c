"""CPU oracle for the looped weight-shared transformer forward pass.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only the tests, the smoke check and the CPU-baseline leg
of the benchmark use it. It shares no code with the GPU library; the two meet
only in the seeded input generators of the ``synth`` package.

The oracle is deliberately plain: float64 NumPy, dequantize-then-matmul,
naive masked softmax attention, and an explicit Python loop that applies the
one shared loop block L times. Rounding to float16 happens only at the
activation cast points of the model definition, and the INT8 KV quantizer takes
its rounding decisions in float32, the precision the definition fixes for it.

Sources (the TinyLoop documentation pages):
  * "TinyLoop Framework" intro page: the four-step forward (embed, pre-blocks,
    one shared loop block reused L times, final norm + head); loop count as a
    runtime knob; weight memory tied to unique blocks.
  * "Current Status" page (zh-TW), model-architecture table: RoPE on all
    forward paths, GeLU opt-in (SwiGLU otherwise), post-norm opt-in (pre-norm
    otherwise), FP32 residual stream by default (core-inference table).
  * "Performance and Memory" page, section "KV cache INT8 -- 2x context at
    matched VRAM": per-token per-head symmetric INT8 with one FP16 scale;
    section "Key Runtime Switches" (TINYLOOP_DISABLE_KV_CACHE): the uncached
    recompute is the parity reference for cached decode.
  * "Current Status" page, KV-cache table: store-h (the cache keeps the
    block's normed input h, FP16 or INT8 per 128-element group, and K, V are
    rebuilt from it): Cache(store_h=..., h_int8=...), kvquant.h_quantize.
  * Self-speculative decode ("Introduction" page, "What Makes It Different";
    "Current Status" page, speculative decode table): speculative.py.
  * Per-iteration residual-norm safety check ("Current Status" page,
    architecture-unique features table): safety.py.
"""
from .int4 import pack_int4, unpack_int4, dequantize
from .kvquant import kv_quantize, kv_dequantize, kv_cache_bytes, h_quantize, h_dequantize, store_h_bytes
from .model import (OracleModel, Cache, rmsnorm, rope_cos_sin, apply_rope, attention,
                    silu, fp16, forward, decode_step, generate_greedy, forward_uncached,
                    head_logits)
from .speculative import speculative_greedy
from .safety import safety_trip

__all__ = ["pack_int4", "unpack_int4", "dequantize", "kv_quantize", "kv_dequantize",
           "kv_cache_bytes", "h_quantize", "h_dequantize", "store_h_bytes", "OracleModel", "Cache", "rmsnorm", "rope_cos_sin", "apply_rope",
           "attention", "silu", "fp16", "forward", "decode_step", "generate_greedy",
           "forward_uncached", "head_logits", "speculative_greedy", "safety_trip"]
