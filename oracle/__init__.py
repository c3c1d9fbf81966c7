"""fp64 CPU oracle for causal attention with RoPE and a KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no kernels, headers, helpers, tables or constants) and never
imports it.

Every function is the plain definition the pages give, evaluated in float64
with no blocking, fusion or reordering.  Inputs arrive as fp32 or bf16-valued
arrays and are widened exactly to float64; no GPU intermediate rounding is
emulated.

Pages cited (titles as published):

* [Guide]     "手写LLM推理引擎：从黑盒到白盒的底层实现指南"
              (hand-writing an LLM inference engine: from black box to white box)
* [Intuition] "手写LLM推理引擎：重建对Tokenizer、KV Cache与RoPE的底层直觉"
              (rebuilding intuition for the tokenizer, KV cache and RoPE)
* [Scratch]   "从零手搓AI推理引擎：告别调包思维，深入底层构建与优化"
              (building an AI inference engine from scratch)
* [NanoVLLM]  "以 Nano-vLLM 为例，深入理解 LLM 推理引擎（Part 2）"
              (understanding LLM inference engines through Nano-vLLM, part 2)

Pin status of each function (what fixes it other than itself) is listed in
``oracle/attention.py`` and, for the INT8 cache, ``oracle/int8_cache.py``.  One convention is *parity unpinned* by any check
on synthetic data and is fixed only by the text: the RoPE pair layout
(adjacent pairs (2i, 2i+1), [Intuition] §4) and the GQA head grouping
(contiguous groups, hk = hq // (Hq/Hkv)).
"""

from .attention import (  # noqa: F401
    rope_inv_freq,
    rope_pair_index,
    rope_rotate,
    causal_attention,
    attn_prefill,
    kv_cache_append,
    cache_rows,
    attn_decode,
    attn_prefill_cached,
    paged_slot,
)
from .int8_cache import (  # noqa: F401
    int8_scale,
    int8_quantize,
    int8_dequantize,
    int8_calibrate,
    kv_cache_append_int8,
    attn_decode_int8,
    attn_prefill_cached_int8,
)
