"""Dense causal GQA attention over each sequence's gathered K/V (test infrastructure only).

The attention a paged kernel computes is exactly the dense one over the keys
gathered through the page table (mini-vLLM page, "Test suites": paged attention
with grouped-query heads matches dense attention; Helios README, "Paged
attention": pages are read through the page table instead of a padded dense
batch). So the oracle gathers, then applies the plain definition
``softmax(q K^T * scale) V`` (Helios blog, "torch.sdpa and Flash Attention",
with scale = 1/sqrt(d)) per query head, in float64.

Readings where the pages leave a step open:

* GQA: query head ``h`` reads KV head ``h // (Hq // Hkv)`` (contiguous groups,
  the layout of the Llama/Qwen3 weights the pages load; Helios blog, same
  section: query heads share the smaller set of KV heads).
* Causality for a sequence with ``n`` keys (this tick's included) and ``L``
  query rows: row ``i`` sees keys ``j <= n - L + i`` (bottom-right aligned).
  A decode row (L = 1) sees all n keys; a chunk sees every earlier page in full
  and itself causally (llm-serving-engine README, ``_step_prefill``:
  "rectangular causal mask"; ``_step_decode``: single-query attention over the
  full K/V).
"""

import numpy as np

from .numerics import storage_to_f32
from .paging import gather_sequence


def attend_sequence(q, K, V, scale):
    """q ``[L, Hq, D]``, K/V ``[n, Hkv, D]`` (float64) -> ``[L, Hq, D]`` float64.

    Query row i of the L rows attends keys ``0 .. n-L+i``.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L, Hq, D = q.shape
    n, Hkv, _ = K.shape
    if L == 0:
        return np.zeros((0, Hq, D))
    if L > n:
        raise ValueError("a sequence cannot have more query rows than keys")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    rows = np.arange(L)[:, None]
    keys = np.arange(n)[None, :]
    visible = keys <= (n - L + rows)            # [L, n]
    out = np.empty((L, Hq, D), dtype=np.float64)
    for h in range(Hq):
        g = h // group
        scores = (q[:, h, :] @ K[:, g, :].T) * scale          # [L, n]
        scores = np.where(visible, scores, -np.inf)
        top = scores.max(axis=1, keepdims=True)
        w = np.exp(scores - top)
        w = w / w.sum(axis=1, keepdims=True)
        out[:, h, :] = w @ V[:, g, :]
    return out


def dense_causal_attention(q, K, V, scale):
    """The dense-KV reference path: the same definition on contiguous K/V."""
    return attend_sequence(q, K, V, scale)


def paged_attention_varlen(q, k_pool, v_pool, block_tables, seq_lens, query_start_loc,
                           scale, dtype):
    """Attention of a packed tick, float64 ``[T, Hq, D]``.

    ``q``: stored ``[T, Hq, D]``; pools: stored ``[num_pages, P, Hkv, D]``;
    sequence s owns rows ``qsl[s] .. qsl[s+1]-1`` of ``q`` and has
    ``seq_lens[s]`` keys in its pages (this tick's included).
    """
    qf = storage_to_f32(q, dtype).astype(np.float64)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    T = int(qsl[-1])
    Hq, D = qf.shape[1], qf.shape[2]
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for s in range(len(qsl) - 1):
        a, b = int(qsl[s]), int(qsl[s + 1])
        if b == a:
            continue
        n = int(seq_lens[s])
        K = storage_to_f32(gather_sequence(k_pool, block_tables[s], n), dtype).astype(np.float64)
        V = storage_to_f32(gather_sequence(v_pool, block_tables[s], n), dtype).astype(np.float64)
        out[a:b] = attend_sequence(qf[a:b], K, V, scale)
    return out
