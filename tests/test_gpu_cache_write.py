"""GPU parity of the write side of a tick: the cos/sin table, the slot mapping
and RoPE + page write (K1), against the oracle. Integer/bit work is compared
bit for bit."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_page_amd as pa
from paged_kv_cache_page_amd import workloads as W
from _gpu import DEV, DevTick, host_storage, say, storage_tensor, i32

pytestmark = pytest.mark.gpu


def _ulp_diff_f32(a, b):
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_write_with_the_library_table_matches_the_oracle_table_write(cfg):
    """The library's own table (K0) in K1: wherever a table row equals the
    oracle's, the rotated rows are the oracle's bit for bit; elsewhere (a row
    whose float64 value sat at a float32 rounding boundary, so one entry
    differs by one float32 ulp) they agree to one bf16 rounding step, plus
    the table's own 1-ulp difference times |x| where the rotation cancels."""
    t = W.make_config(cfg, poison=True)
    say("rope+cache write with the library table, cfg", cfg)
    d = DevTick(t)
    table = pa.pa_rope_cos_sin_table(t.max_pos, t.D, t.theta, device=DEV)
    slots = pa.pa_compute_slot_mapping(d.block_tables, d.qsl, d.positions, t.P, t.num_pages)
    pa.pa_rope_and_cache_write(d.q, d.k, d.v, d.positions, slots, table, d.k_pool, d.v_pool)
    torch.cuda.synchronize()
    ref_table = oracle.rope_table(t.max_pos, t.D, t.theta)
    same = np.all(table.cpu().numpy()[t.positions] == ref_table[t.positions], axis=1)
    res = oracle.run_tick(t.dtype, t.q, t.k, t.v, t.positions, t.block_tables, t.qsl,
                          t.seq_lens, t.k_pool, t.v_pool, ref_table, t.scale)
    for name, got in (("q", host_storage(d.q, t.dtype)), ("k", host_storage(d.k, t.dtype))):
        want = res[name]
        assert np.array_equal(got[same], want[same]), name
        a = oracle.bf16_bits_to_f32(got).astype(np.float64)
        b = oracle.bf16_bits_to_f32(want).astype(np.float64)
        assert (np.abs(a - b) <= 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + 1e-6).all(), name


@pytest.mark.parametrize("max_pos,D,theta", [(1024, 64, 1e4), (32768, 128, 1e6), (64, 16, 1e4)])
def test_rope_table_matches_oracle(max_pos, D, theta):
    say("rope table", max_pos, D, theta)
    gpu = pa.pa_rope_cos_sin_table(max_pos, D, theta, device=DEV).cpu().numpy()
    ref = oracle.rope_table(max_pos, D, theta)
    d = _ulp_diff_f32(gpu, ref)
    # both evaluate cos/sin in float64 and round once; they can differ only when the
    # float64 value sits within a few float64 ulps of a float32 rounding boundary
    assert d.max() <= 1, d.max()
    assert (d == 0).mean() >= 0.9999, (d == 0).mean()


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_slot_mapping_bit_exact(cfg):
    t = W.make_config(cfg, poison=True)
    say("slot mapping cfg", cfg)
    d = DevTick(t)
    got = pa.pa_compute_slot_mapping(d.block_tables, d.qsl, d.positions, t.P, t.num_pages)
    ref = oracle.slot_mapping(t.block_tables, t.qsl, t.positions, t.P)
    assert np.array_equal(got.cpu().numpy(), ref)


def test_slot_mapping_out_of_range_rows_are_minus_one():
    t = W.make_config(2, poison=True)
    pos = t.positions.copy()
    pos[0] = -5                                  # negative position
    pos[1] = t.block_tables.shape[1] * t.P       # beyond the table row
    bt = t.block_tables.copy()
    s2 = 2
    bt[s2, int(t.positions[s2]) // t.P] = t.num_pages + 3   # page id out of range
    got = pa.pa_compute_slot_mapping(i32(bt), i32(t.qsl), i32(pos), t.P, t.num_pages).cpu().numpy()
    assert got[0] == -1 and got[1] == -1 and got[2] == -1
    ref = oracle.slot_mapping(t.block_tables, t.qsl, t.positions, t.P)
    assert np.array_equal(got[3:], ref[3:])


def _check_write(t, d):
    """Compare q/k after RoPE, the slots and both pools with the oracle, bit
    for bit, for every token. The device ran with the oracle's cos/sin table
    (the call input both sides share), so nothing is left to chance."""
    table_ref = oracle.rope_table(t.max_pos, t.D, t.theta) if t.theta is not None else None
    res = oracle.run_tick(t.dtype, t.q, t.k, t.v, t.positions, t.block_tables, t.qsl,
                          t.seq_lens, t.k_pool, t.v_pool, table_ref, t.scale)
    as_bits = (lambda a: a.view(np.uint32)) if t.dtype == W.F32 else (lambda a: a)
    assert np.array_equal(d.slots.cpu().numpy(), res["slots"])
    q_gpu = host_storage(d.q, t.dtype)
    k_gpu = host_storage(d.k, t.dtype)
    assert np.array_equal(as_bits(q_gpu), as_bits(res["q"]))
    assert np.array_equal(as_bits(k_gpu), as_bits(res["k"]))
    kp = host_storage(d.k_pool, t.dtype)
    vp = host_storage(d.v_pool, t.dtype)
    # every slot other than the written ones is bitwise unchanged (NaN bits included)
    written = np.zeros((t.num_pages, t.P), bool)
    for slot in res["slots"]:
        if slot >= 0:
            written[slot // t.P, slot % t.P] = True
    assert np.array_equal(as_bits(kp[~written]), as_bits(t.k_pool[~written]))
    assert np.array_equal(as_bits(vp[~written]), as_bits(t.v_pool[~written]))
    # written slots hold the rotated K and V's exact bits; the whole pools equal
    # the oracle's written pools
    for tok, slot in enumerate(res["slots"]):
        if slot < 0:
            continue
        pg, row = slot // t.P, slot % t.P
        assert np.array_equal(as_bits(vp[pg, row]), as_bits(t.v[tok]))
        assert np.array_equal(as_bits(kp[pg, row]), as_bits(res["k_pool"][pg, row]))
    assert np.array_equal(as_bits(kp), as_bits(res["k_pool"]))
    assert np.array_equal(as_bits(vp), as_bits(res["v_pool"]))


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_rope_and_cache_write_bit_exact(cfg):
    t = W.make_config(cfg, poison=True)
    say("rope+cache write cfg", cfg)
    d = DevTick(t).write()
    torch.cuda.synchronize()
    _check_write(t, d)


# (D = 48 bf16 and 80 fp32: 3 and 10 vectors per half row, so the workgroup is
# 255 and 250 threads)
@pytest.mark.parametrize("dtype,D", [(W.F32, 16), (W.F32, 128), (W.BF16, 64), (W.BF16, 48),
                                     (W.F32, 80)])
def test_rope_and_cache_write_small_shapes(dtype, D):
    rng = np.random.default_rng(50 + D)
    t = W.build_tick(rng, name="small", dtype=dtype, Hq=8, Hkv=2, D=D, P=16,
                     seq_lens=[1, 17, 40, 16], query_lens=[1, 17, 5, 1], theta=1e4)
    say("rope+cache write small", dtype, D)
    d = DevTick(t).write()
    torch.cuda.synchronize()
    _check_write(t, d)


def test_cache_write_without_rope_and_skipped_rows():
    rng = np.random.default_rng(60)
    t = W.build_tick(rng, name="norope", dtype=W.BF16, Hq=4, Hkv=4, D=128, P=16,
                     seq_lens=[20, 33], query_lens=[3, 2], theta=None)
    d = DevTick(t)
    slots = oracle.slot_mapping(t.block_tables, t.qsl, t.positions, t.P).copy()
    slots[1] = -1                        # a padding row: no pool write
    slots[4] = t.num_pages * t.P         # out of range: no pool write
    say("cache write without rope")
    q_before = d.q.clone()
    pa.pa_rope_and_cache_write(d.q, d.k, d.v, d.positions, i32(slots), None, d.k_pool, d.v_pool)
    torch.cuda.synchronize()
    assert torch.equal(d.q.view(torch.int16), q_before.view(torch.int16))
    kp = host_storage(d.k_pool, t.dtype)
    vp = host_storage(d.v_pool, t.dtype)
    ref_k, ref_v = oracle.write_cache(t.k_pool, t.v_pool, np.where((slots >= 0) & (slots < t.num_pages * t.P), slots, -1), t.k, t.v)
    assert np.array_equal(kp, ref_k) and np.array_equal(vp, ref_v)


def test_cache_write_q_null_rotates_only_k():
    rng = np.random.default_rng(61)
    t = W.build_tick(rng, name="konly", dtype=W.BF16, Hq=4, Hkv=2, D=64, P=16,
                     seq_lens=[9], query_lens=[4], theta=1e4)
    d = DevTick(t)
    table = d.oracle_table()
    slots = pa.pa_compute_slot_mapping(d.block_tables, d.qsl, d.positions, t.P, t.num_pages)
    say("cache write q=None")
    pa.pa_rope_and_cache_write(None, d.k, d.v, d.positions, slots, table, d.k_pool, d.v_pool)
    torch.cuda.synchronize()
    ref_table = oracle.rope_table(t.max_pos, t.D, t.theta)
    k_ref = oracle.f32_to_bf16_bits(oracle.rope_rotate(oracle.bf16_bits_to_f32(t.k), t.positions, ref_table))
    assert np.array_equal(host_storage(d.k, t.dtype), k_ref)
    assert np.array_equal(host_storage(d.q, t.dtype), t.q)
