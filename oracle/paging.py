"""Page-table indexing, the KV page write and the gather (test infrastructure only).

* The pool is a fixed set of pages of ``P`` token slots; each sequence's page
  table maps its logical block ``j // P`` to a physical page (Helios blog,
  "Paged attention"; mini-vLLM page, "Paged KV-cache": a block table per
  sequence maps positions to blocks, like virtual memory).
* One layer's pool for K (and one for V) is ``[num_pages, P, Hkv, D]``
  (llm-serving-engine README, row "KV Cache" and "KV cache memory layout",
  which list ``[layers, 2, blocks, block_size, kv_heads, head_dim]``).
* A new token at absolute position ``p`` of sequence ``s`` lives in slot
  ``bt[s][p // P] * P + p % P``; its K/V are written there before attention
  reads the pages (llm-serving-engine README, ``_step_prefill`` writes K/V at
  the chunk start; Helios README, "Paged attention": decode writes directly to
  the shared pool).
"""

import numpy as np


def slot_of_token(block_table_row, pos, P):
    """Flat slot index of absolute position ``pos`` for one sequence's page table."""
    page = int(block_table_row[pos // P])
    return page * P + pos % P


def slot_mapping(block_tables, query_start_loc, positions, P):
    """Slot of every new token of a packed tick.

    Token t belongs to the sequence s with ``qsl[s] <= t < qsl[s+1]``; its slot
    follows from that sequence's page table and its absolute position.
    """
    block_tables = np.asarray(block_tables)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    positions = np.asarray(positions, dtype=np.int64)
    T = int(qsl[-1])
    out = np.empty(T, dtype=np.int32)
    for s in range(len(qsl) - 1):
        for t in range(int(qsl[s]), int(qsl[s + 1])):
            out[t] = slot_of_token(block_tables[s], int(positions[t]), P)
    return out


def write_cache(k_pool, v_pool, slots, k_rows, v_rows):
    """Store each token's K and V rows in its slot; a negative slot means
    "no write" (a padding row). Returns new pools; the inputs are not changed.

    ``k_pool``/``v_pool``: ``[num_pages, P, Hkv, D]`` in the storage
    representation; ``k_rows``/``v_rows``: ``[T, Hkv, D]`` same representation.
    """
    k_new = np.array(k_pool, copy=True)
    v_new = np.array(v_pool, copy=True)
    P = k_new.shape[1]
    for t, slot in enumerate(np.asarray(slots, dtype=np.int64)):
        if slot < 0:
            continue
        k_new[slot // P, slot % P] = k_rows[t]
        v_new[slot // P, slot % P] = v_rows[t]
    return k_new, v_new


def gather_sequence(pool, block_table_row, n):
    """Keys (or values) ``0..n-1`` of one sequence, read through its page table:
    ``out[j] = pool[bt[j // P], j % P]``; shape ``[n, Hkv, D]``."""
    P = pool.shape[1]
    n_blocks = (n + P - 1) // P
    pages = np.asarray(block_table_row[:n_blocks], dtype=np.int64)
    blocks = pool[pages]                       # [n_blocks, P, Hkv, D]
    flat = blocks.reshape((n_blocks * P,) + pool.shape[2:])
    return flat[:n]


def pool_bytes(layers, blocks, block_size, kv_heads, head_dim, elem_bytes):
    """Bytes of a pre-allocated K+V pool ``[layers, 2, blocks, block_size,
    kv_heads, head_dim]`` (llm-serving-engine README, "KV cache memory
    layout")."""
    return layers * 2 * blocks * block_size * kv_heads * head_dim * elem_bytes
