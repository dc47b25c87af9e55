"""The opt-in validation mode (pa_set_validation) on the GPU: every
precondition on device metadata that the kernels take on trust is checked on
the host before anything is enqueued. A bad tick returns PA_ERR_INVALID_ARG,
launches no kernel and names the offending sequence or token; a good tick runs
exactly as without validation."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_page_amd as pa
from paged_kv_cache_page_amd import workloads as W
from _gpu import DEV, DevTick, i32, say

pytestmark = pytest.mark.gpu

INVALID = 1


def _tick(seed=300):
    rng = np.random.default_rng(seed)
    return W.build_tick(rng, name="valid", dtype=W.BF16, Hq=8, Hkv=2, D=64, P=16,
                        seq_lens=[40, 70, 33, 20], query_lens=[1, 1, 17, 1], theta=1e4,
                        poison=True)


@pytest.fixture
def validation():
    pa.pa_set_validation(True)
    yield
    pa.pa_set_validation(False)


def _tick_call(t, bt=None, sl=None, qsl=None, pos=None, max_seq_len=None, max_query_len=None):
    d = DevTick(t)
    table = torch.from_numpy(oracle.rope_table(t.max_pos, t.D, t.theta)).to(DEV)
    return pa.pa_tick_forward(
        d.q, d.k, d.v, i32(t.positions if pos is None else pos),
        i32(t.block_tables if bt is None else bt), i32(t.seq_lens if sl is None else sl),
        i32(t.qsl if qsl is None else qsl), table, d.k_pool, d.v_pool,
        t.max_query_len if max_query_len is None else max_query_len,
        t.max_seq_len if max_seq_len is None else max_seq_len, scale=t.scale)


def _attn_call(t, bt=None, sl=None, qsl=None, max_seq_len=None):
    d = DevTick(t)
    return pa.pa_paged_attention_varlen(
        d.q, d.k_pool, d.v_pool, i32(t.block_tables if bt is None else bt),
        i32(t.seq_lens if sl is None else sl), i32(t.qsl if qsl is None else qsl),
        t.max_query_len, t.max_seq_len if max_seq_len is None else max_seq_len, scale=t.scale)


def _rejected(fn, words):
    """fn() must raise PaError(PA_ERR_INVALID_ARG) naming `words`, and enqueue
    no kernel."""
    torch.cuda.synchronize()
    pa.pa_profile_start(64)
    with pytest.raises(pa.PaError) as e:
        fn()
    rec = pa.pa_profile_stop()
    pa.pa_profile_reset()
    assert e.value.status == INVALID
    msg = str(e.value)
    for w in words:
        assert w in msg, msg
    assert rec == [], rec


def test_good_tick_passes_and_matches_the_unvalidated_call(validation):
    t = _tick()
    say("validation: good tick")
    a = _tick_call(t)
    assert pa.pa_validation_message() == ""
    pa.pa_set_validation(False)
    b = _tick_call(t)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_page_id_out_of_range(validation):
    t = _tick()
    bt = t.block_tables.copy()
    bt[1, 2] = t.num_pages + 5
    say("validation: page id out of range")
    _rejected(lambda: _tick_call(t, bt=bt), ["sequence 1", "block_tables[1][2]"])
    _rejected(lambda: _attn_call(t, bt=bt), ["sequence 1"])
    bt[1, 2] = -1
    _rejected(lambda: _attn_call(t, bt=bt), ["sequence 1"])


def test_query_start_loc_not_monotone(validation):
    t = _tick()
    qsl = t.qsl.copy()
    qsl[2], qsl[3] = qsl[3], qsl[2]
    say("validation: qsl not monotone")
    _rejected(lambda: _tick_call(t, qsl=qsl), ["query_start_loc decreases"])
    _rejected(lambda: _attn_call(t, qsl=qsl), ["query_start_loc decreases"])


def test_more_query_rows_than_keys(validation):
    t = _tick()
    sl = t.seq_lens.copy()
    sl[2] = 10                   # 17 rows
    say("validation: L > seq_len")
    _rejected(lambda: _attn_call(t, sl=sl), ["sequence 2", "17 query rows > seq_len 10"])


def test_seq_len_above_the_host_bound(validation):
    t = _tick()
    say("validation: seq_len > max_seq_len")
    _rejected(lambda: _attn_call(t, max_seq_len=50), ["sequence 1", "max_seq_len 50"])
    _rejected(lambda: _tick_call(t, max_seq_len=50), ["sequence 1", "max_seq_len 50"])


def test_tick_positions_and_shared_written_page(validation):
    t = _tick()
    pos = t.positions.copy()
    pos[0] += 1
    say("validation: position not the last key")
    _rejected(lambda: _tick_call(t, pos=pos), ["token 0", "sequence 0"])
    bt = t.block_tables.copy()
    bt[3, 1] = bt[0, 2]           # sequence 0 writes its last page, which sequence 3 also uses
    _rejected(lambda: _tick_call(t, bt=bt), ["another sequence"])


def test_cache_write_duplicate_slots(validation):
    t = _tick()
    d = DevTick(t)
    slots = oracle.slot_mapping(t.block_tables, t.qsl, t.positions, t.P).copy()
    slots[5] = slots[2]
    say("validation: duplicate slots")
    _rejected(lambda: pa.pa_rope_and_cache_write(d.q, d.k, d.v, d.positions, i32(slots), None,
                                                 d.k_pool, d.v_pool), ["same slot"])
