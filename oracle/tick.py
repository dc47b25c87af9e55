"""One packed tick end to end: RoPE, slot mapping, page write, paged attention
(test infrastructure only).

Order follows the pages: project, RoPE on Q and K (Helios blog, "torch.sdpa and
Flash Attention"), write the new K/V into their page slots, then attend through
the page tables (Helios blog, "Paged attention": prefill and decode write K and
V into the pages, then run attention with the page table).
"""

from .numerics import storage_to_f32, f32_to_storage
from .rope import rope_rotate
from .paging import slot_mapping, write_cache
from .attention import paged_attention_varlen


def run_tick(dtype, q, k, v, positions, block_tables, query_start_loc, seq_lens,
             k_pool, v_pool, table, scale, slots=None):
    """Return a dict with the rotated-and-stored ``q``/``k``, the ``slots``, the
    updated pools and the float64 attention output ``out``.

    ``table`` is the oracle's own float32 cos/sin table, or None for no RoPE.
    ``slots`` defaults to the oracle's own slot mapping from the page tables.
    """
    if table is not None:
        q_st = f32_to_storage(rope_rotate(storage_to_f32(q, dtype), positions, table), dtype)
        k_st = f32_to_storage(rope_rotate(storage_to_f32(k, dtype), positions, table), dtype)
    else:
        q_st, k_st = q.copy(), k.copy()
    P = k_pool.shape[1]
    if slots is None:
        slots = slot_mapping(block_tables, query_start_loc, positions, P)
    kp, vp = write_cache(k_pool, v_pool, slots, k_st, v)
    out = paged_attention_varlen(q_st, kp, vp, block_tables, seq_lens, query_start_loc,
                                 scale, dtype)
    return {"q": q_st, "k": k_st, "slots": slots, "k_pool": kp, "v_pool": vp, "out": out}
