"""Plain CPU oracle for the paged KV-cache decode path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package imports this
package.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call it.  It shares no
code with the HIP path: no kernels, headers, helpers, tables or constants.

Sources (the three web pages on PagedAttention):

* "Memory Optimization in LLM Serving with PagedAttention" (grasp.study),
  sections "How PagedAttention Works" and "Advanced Capabilities: Memory
  Sharing with Copy-on-Write".
* "vLLM and PagedAttention: How Ideas from Operating Systems Accelerated LLM
  Inference" (polomodov.tech), the paragraphs on the paged solution, on
  sharing, and on the engine.
* "Scaling LLM Inference: Memory Management with PagedAttention and vLLM"
  (jackhb1970 blog), section "The KV Cache Bottleneck".

Every function here is pinned by CPU tests (``tests/test_oracle_pins.py``,
``tests/test_oracle_fp8.py``, ``tests/test_oracle_prefill.py``) to something other than itself: a library
attention routine on contiguous data, torch's float8_e4m3fn conversions,
closed forms, invariants and hand-worked fixtures.
"""

from .paged_attention import decode, decode_one, kv_head_of
from .cache_ops import copy_blocks, reshape_and_cache, swap_blocks
from . import fp8
from .fp8 import decode_fp8, prefill_fp8, reshape_and_cache_fp8
from .prefill import prefill

__all__ = ["decode", "decode_one", "kv_head_of", "copy_blocks", "reshape_and_cache",
           "swap_blocks", "fp8", "decode_fp8", "reshape_and_cache_fp8", "prefill", "prefill_fp8"]
