"""Property tests on the GPU: random small valid ticks (hypothesis, a fixed
example budget, derandomised so every run draws the same cases) run through
pa_tick_forward and compared with the oracle at the stated tolerances, the
pools bit for bit.

Shapes: S <= 8 sequences of 1..300 keys, each a decode row, a chunk of 2..n
rows or no rows this tick; GQA groups 1, 2, 4, 8; head_dim 64 or 128 (bf16)
and 16, 64 or 128 (float32); 16-, 32- and 256-token pages; automatic or fixed
split-KV partitions; with and without RoPE (mini-vLLM page, "Test suites":
paged attention matches dense attention across shapes)."""

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

import oracle
import paged_kv_cache_page_amd as pa
from paged_kv_cache_page_amd import workloads as W
from _gpu import DEV, DevTick, check_attention, host_storage, say

pytestmark = pytest.mark.gpu


@st.composite
def ticks(draw):
    dtype = draw(st.sampled_from([W.BF16, W.BF16, W.BF16, W.F32]))
    D = draw(st.sampled_from([64, 128] if dtype == W.BF16 else [16, 64, 128]))
    G = draw(st.sampled_from([1, 2, 4, 8]))
    Hkv = draw(st.sampled_from([1, 2]))
    P = draw(st.sampled_from([16, 32, 256]))
    S = draw(st.integers(1, 8))
    seq_lens, query_lens = [], []
    for _ in range(S):
        n = draw(st.integers(1, 300))
        kind = draw(st.sampled_from(["decode", "decode", "chunk", "none"]))
        if kind == "decode" or n == 1 and kind == "chunk":
            L = 1
        elif kind == "chunk":
            L = draw(st.integers(2, n))
        else:
            L = 0
        seq_lens.append(n)
        query_lens.append(L)
    if sum(query_lens) == 0:
        query_lens[0] = 1
    rope = draw(st.booleans())
    split = draw(st.sampled_from([0, 0, 16, 64, 512]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    return dtype, D, G, Hkv, P, seq_lens, query_lens, rope, split, seed


@settings(max_examples=40, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(ticks())
def test_random_small_ticks_match_the_oracle(case):
    dtype, D, G, Hkv, P, sl, ql, rope, split, seed = case
    rng = np.random.default_rng(seed)
    t = W.build_tick(rng, name="prop", dtype=dtype, Hq=G * Hkv, Hkv=Hkv, D=D, P=P,
                     seq_lens=sl, query_lens=ql, theta=1e4 if rope else None, poison=True)
    say("prop", dtype, D, G, Hkv, P, sl, ql, rope, split)
    d = DevTick(t)
    out = pa.pa_tick_forward(d.q, d.k, d.v, d.positions, d.block_tables, d.seq_lens, d.qsl,
                             d.oracle_table(), d.k_pool, d.v_pool, t.max_query_len,
                             t.max_seq_len, scale=t.scale, kv_split_tokens=split)
    torch.cuda.synchronize()
    table = oracle.rope_table(t.max_pos, t.D, t.theta) if rope else None
    res = oracle.run_tick(t.dtype, t.q, t.k, t.v, t.positions, t.block_tables, t.qsl,
                          t.seq_lens, t.k_pool, t.v_pool, table, t.scale)
    check_attention(out, res["out"], t.dtype, "prop")
    bits = (lambda a: a.view(np.uint32)) if dtype == W.F32 else (lambda a: a)
    assert np.array_equal(bits(host_storage(d.k_pool, dtype)), bits(res["k_pool"]))
    assert np.array_equal(bits(host_storage(d.v_pool, dtype)), bits(res["v_pool"]))
