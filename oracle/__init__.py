"""Plain, slow CPU oracle for paged decode attention over a block-table KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library in ``paged_kv_cache_21_amd/`` and imports nothing from it.

Everything here is written from the source pages:

* "The Reasoning Engine Meltdown" (atozofsoftwareengineering.blog), §2.1 for the
  attention definition, the decode step and the KV-size formula; §5 and §6 for
  the page table with reference counts, fork, copy-on-write and free.
* "Dismantling the Memory Wall" (blog.bako.co), section "PagedAttention: The
  Virtual Memory Analogy for GPUs" for the 16-token block and the
  token -> logical-block arithmetic; section "Copy-on-Write and Advanced
  Decoding Strategies" for sharing prompt blocks and allocating on divergence;
  section "Chunked Prefill" (with the verification pass of "RKSC", §1) for
  several new tokens attending causally at once; section "RadixAttention" for
  the prefix cache (with "RKSC", §2 C "RSBCM" for its score/depth eviction
  order); section "Cross-Tier Memory Offloading" for moving blocks to host
  memory and back.

Floating point is fp64.  fp16/bf16 inputs arrive as raw 16-bit patterns and
are decoded here, independently of the GPU code.

Parity pins: every function is checked by ``tests/test_oracle_*.py`` against
values the pages print, closed forms, brute force on tiny inputs and
invariants; none of them is "parity unpinned".
"""

from .kvsize import kv_bytes, kv_bytes_per_token
from .attention import decode_bits, ref_decode, ref_decode_rows, bruteforce_decode
from .extend import extend_query_positions, ref_extend
from .fp8 import (apply_append_fp8, dequantize_heads, dequantize_pages, e4m3_decode, e4m3_encode,
                  pow2_scale_exponent, quantize_heads, ref_decode_fp8, ref_extend_fp8)
from .pool import RefPool, RefPoolError, apply_append, apply_swap
from .radix import RadixCache, RadixError

__all__ = [
    "kv_bytes",
    "kv_bytes_per_token",
    "decode_bits",
    "ref_decode",
    "ref_decode_rows",
    "bruteforce_decode",
    "extend_query_positions",
    "ref_extend",
    "apply_append_fp8",
    "dequantize_heads",
    "dequantize_pages",
    "e4m3_decode",
    "e4m3_encode",
    "pow2_scale_exponent",
    "quantize_heads",
    "ref_decode_fp8",
    "ref_extend_fp8",
    "RefPool",
    "RefPoolError",
    "apply_append",
    "apply_swap",
    "RadixCache",
    "RadixError",
]
