"""pa_tick_forward_noalloc on the GPU, through the C ABI: the same tick as
pa_tick_forward bit for bit (out, slots, rotated q/k, both pools) on two calls
in a row, the second with a smaller tick, so that what the first call left in
the shared fixed scratch cannot leak into the second; a third call repeats the
first. An oversized tick is refused with nothing launched."""

import numpy as np
import pytest
import torch

import paged_kv_cache_page_amd as pa
from paged_kv_cache_page_amd import workloads as W
from _gpu import DEV, DevTick, say

pytestmark = pytest.mark.gpu


def _bits(x):
    return x.view(torch.int16 if x.element_size() == 2 else torch.int32).cpu().numpy()


def _both(t, split=0):
    """The tick through pa_tick_forward (binding-allocated workspace) and through
    pa_tick_forward_noalloc, each on its own copy of the inputs."""
    a, b = DevTick(t), DevTick(t)
    table = a.oracle_table()
    ref = pa.pa_tick_forward(a.q, a.k, a.v, a.positions, a.block_tables, a.seq_lens, a.qsl,
                             table, a.k_pool, a.v_pool, t.max_query_len, t.max_seq_len,
                             scale=t.scale, kv_split_tokens=split)
    slots = torch.full((t.T,), -7, dtype=torch.int32, device=DEV)
    out = torch.empty_like(b.q)
    pa.pa_tick_forward_noalloc(b.q, b.k, b.v, b.positions, b.block_tables, b.seq_lens, b.qsl,
                               table, b.k_pool, b.v_pool, t.max_query_len, t.max_seq_len, out,
                               slots, scale=t.scale, kv_split_tokens=split)
    torch.cuda.synchronize()
    ref_slots = pa.pa_compute_slot_mapping(a.block_tables, a.qsl, a.positions, t.P, t.num_pages)
    torch.cuda.synchronize()
    for name, x, y in (("out", ref, out), ("slots", ref_slots, slots), ("q", a.q, b.q),
                       ("k", a.k, b.k), ("k_pool", a.k_pool, b.k_pool),
                       ("v_pool", a.v_pool, b.v_pool)):  # (q, k: as each call leaves them)
        assert np.array_equal(_bits(x), _bits(y)), f"{t.name}: {name} differs"


def test_noalloc_equals_tick_forward_on_two_calls_the_second_smaller():
    big = W.make_config(4, poison=True)          # packed mixed tick, about 37 MiB of scratch
    small = W.make_config(2, poison=True)        # TinyLlama decode tick, under 1 MiB
    say("noalloc: packed mixed tick")
    _both(big)
    say("noalloc: smaller decode tick after it")
    _both(small)
    say("noalloc: the packed tick again, fixed split")
    _both(big, split=512)


def test_noalloc_refuses_a_tick_past_its_scratch_and_launches_nothing():
    t = W.make_config(3, poison=False)
    d = DevTick(t)
    out = torch.empty_like(d.q)
    slots = torch.empty(t.T, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    say("noalloc: oversized tick")
    pa.pa_profile_start(16)
    with pytest.raises(pa.PaError) as e:
        # 16-key partitions over rows of up to 3983 keys: about 270 MB of partials
        pa.pa_tick_forward_noalloc(d.q, d.k, d.v, d.positions, d.block_tables, d.seq_lens, d.qsl,
                                   d.oracle_table(), d.k_pool, d.v_pool, t.max_query_len,
                                   t.max_seq_len, out, slots, scale=t.scale, kv_split_tokens=16)
    rec = pa.pa_profile_stop()
    pa.pa_profile_reset()
    assert e.value.status == 3 and "needs" in str(e.value)
    assert rec == []
