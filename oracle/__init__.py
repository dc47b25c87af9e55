"""CPU oracle for the attention of one packed continuous-batching tick.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product
library (``paged_kv_cache_page_amd``) never imports it, links it or runs it,
and this package imports nothing from the product either. The two share no
kernels, helpers, tables or constants; only the seeded input generator
(``paged_kv_cache_page_amd.workloads``, which holds none of the method's
arithmetic) feeds both sides.

What it computes, and where the pages state it
----------------------------------------------
* KV pages: a shared pool of fixed-size pages, one page table per request
  (Helios blog, "Paged attention"; mini-vLLM page, "Paged KV-cache"), pool
  laid out as ``[blocks, block_size, kv_heads, head_dim]`` per layer and K/V
  (llm-serving-engine README, component table row "KV Cache").
* New K/V go into their page slots before attention reads them
  (llm-serving-engine README, the ``_step_prefill`` / ``_step_decode`` flow;
  Helios README, "Paged attention").
* RoPE on Q and K from cached cos/sin tables (Helios blog, "torch.sdpa and
  Flash Attention"; llm-serving-engine README, row "RoPE from scratch").
* Attention is ``softmax(Q K^T / sqrt(d)) V`` (Helios blog, "torch.sdpa and
  Flash Attention") with several query heads sharing one KV head (GQA, same
  section; llm-serving-engine README, row "GQA"), causal, and for a chunk with
  earlier pages a rectangular causal mask (llm-serving-engine README,
  ``_step_prefill``). Paged attention equals dense attention (mini-vLLM page,
  "Test suites").

Precision
---------
* RoPE runs in float32 with every product and sum rounded on its own (numpy
  float32 elementwise arithmetic never fuses), then rounds to the storage
  dtype. The rounded K is the value the cache write stores, so both sides take
  that quantisation decision in the same float32 arithmetic.
* Attention runs in float64 on the stored (already rounded) values.

``blocks.py`` is the reference paged block manager (free list, page tables
with reservations, refcounts, the prefix cache of chained complete blocks,
leaf-first eviction); its pins and the library's step-by-step comparison are
in ``tests/test_block_manager.py``.

Every function has at least one pin in ``tests/test_oracle_*.py`` that does
not re-type its formula: brute-force loops, closed forms, invariants, a worked
number from the pages, or a library routine (torch CPU SDPA in float64).
"""

from .numerics import bf16_bits_to_f32, f32_to_bf16_bits, storage_to_f32, f32_to_storage
from .rope import rope_inv_freq, rope_table, rope_rotate
from .paging import slot_of_token, slot_mapping, write_cache, gather_sequence, pool_bytes
from .attention import attend_sequence, paged_attention_varlen, dense_causal_attention
from .tick import run_tick

__all__ = [
    "bf16_bits_to_f32", "f32_to_bf16_bits", "storage_to_f32", "f32_to_storage",
    "rope_inv_freq", "rope_table", "rope_rotate",
    "slot_of_token", "slot_mapping", "write_cache", "gather_sequence", "pool_bytes",
    "attend_sequence", "paged_attention_varlen", "dense_causal_attention",
    "run_tick",
]
