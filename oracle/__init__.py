"""CPU oracle for paged attention over an FP8 E4M3 KV cache (TEST INFRASTRUCTURE ONLY).

This package is the slow, plain reference that the GPU library is checked
against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it.  The product path
(``fp8_kv_cache_e4m3_amd``) never imports it, and it never imports the product.
The two share no code.  The only common module is ``workloads`` (the seeded
input generators), which holds none of the arithmetic below.

Sources (cited by page and section):

* vLLM PR #63139 (FA4 native FP8 forward on SM90 for all Gemma-4 layers),
  Overview.  Sliding-window layers (head dim 256) quantize Q to E4M3 and run
  attention on E4M3 Q/K/V.
* vLLM PR #60372 "[Kernel] Integrate FA4 SM90 FP8 MMA for Gemma-4 full
  attention", Overview and Claims.  Full-attention layers (head dim 512) keep
  BF16 Q over an FP8 KV cache, with normalized descale layouts, 64-token pages
  and an automatic split-KV count.  Its review thread says the kernel supports
  causal and local masks only.
* prhub digest of vLLM PR #48666, Implementation items 1-3 and the
  ``flash_attn_varlen_func`` excerpt under Key code.  The paged
  ``float8_e4m3fn`` K/V are dequantized by the kernel with per-tensor K/V
  descales folded in, Q stays BF16, and the call returns ``out`` and
  ``softmax_lse``.

Modules:
  e4m3       OCP E4M3 decode table, RNE+saturating quantizer, descale recipe
  attention  page gather, causal/window mask, masked softmax attention in fp64,
             log-sum-exp combine of split partials
  brute      pure-Python loops (math.exp / math.fsum) for tiny cases
  cache_write  the paged KV-cache write: quantize new K/V and store them at their slots

Parity pins: every function here is pinned in ``tests/test_oracle_*.py`` by a
closed form, the torch ``float8_e4m3fn`` cast, brute force or an invariant.
The pages print no worked numeric example, so no value from the pages pins
the attention outputs directly.
"""
from . import e4m3, attention, brute, cache_write  # noqa: F401
from .e4m3 import E4M3_TABLE, e4m3_decode, quantize_e4m3, dequantize_e4m3, descale_from_amax  # noqa: F401
from .attention import (gather_pages, visible_mask, paged_attention, combine_splits,  # noqa: F401
                        split_attention, query_values)
from .cache_write import slots_for_new_tokens  # noqa: F401
