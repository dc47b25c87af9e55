"""GPU parity of paged attention over packed ticks (decode K2/K3, prefill K4 and
the per-token VALU path) against the oracle, plus the invariants that must hold
exactly on the GPU: page relabelling, shared prefix pages, packing order and
the one-hot position probe."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_page_amd as pa
from paged_kv_cache_page_amd import workloads as W
from _gpu import (BF16_MAX_ABS, BF16_MEAN_ABS, DEV, DevTick, check_attention, host_f32,
                  host_storage, i32, run_gpu_tick, say, storage_tensor)
import _pins

pytestmark = pytest.mark.gpu


def oracle_tick(t):
    table = oracle.rope_table(t.max_pos, t.D, t.theta) if t.theta is not None else None
    if t.new_in_pool:
        return oracle.paged_attention_varlen(t.q, t.k_pool, t.v_pool, t.block_tables,
                                             t.seq_lens, t.qsl, t.scale, t.dtype)
    return oracle.run_tick(t.dtype, t.q, t.k, t.v, t.positions, t.block_tables, t.qsl,
                           t.seq_lens, t.k_pool, t.v_pool, table, t.scale)["out"]


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_config_parity(cfg):
    """The five workloads end to end (table, slots, RoPE + write, attention),
    unused slots and pages poisoned with NaN."""
    t = W.make_config(cfg, poison=True)
    say("config", cfg, t.name, "S", t.S, "T", t.T)
    _, out = run_gpu_tick(t)
    stats = check_attention(out, oracle_tick(t), t.dtype, t.name)
    say("config", cfg, stats)


@pytest.mark.parametrize("cfg", [3, 5])
def test_full_size_bench_launch_unpoisoned(cfg):
    """The bench's launch configuration (default split, unpoisoned pools)."""
    t = W.make_config(cfg, poison=False)
    say("unpoisoned config", cfg)
    _, out = run_gpu_tick(t)
    check_attention(out, oracle_tick(t), t.dtype, t.name)


def _small(seed, dtype=W.BF16, Hq=8, Hkv=2, D=128, P=16, seq_lens=(40, 300, 17, 129),
           query_lens=(1, 1, 17, 33), theta=1e4, poison=True):
    rng = np.random.default_rng(seed)
    return W.build_tick(rng, name=f"small{seed}", dtype=dtype, Hq=Hq, Hkv=Hkv, D=D, P=P,
                        seq_lens=list(seq_lens), query_lens=list(query_lens), theta=theta,
                        poison=poison)


SMALL_CASES = [
    # (dtype, Hq, Hkv, D, P, seq_lens, query_lens)
    (W.BF16, 8, 2, 128, 16, (40, 300, 17, 129), (1, 1, 17, 33)),      # mixed, chunk from scratch
    (W.BF16, 32, 4, 64, 16, (33, 500, 64, 47), (1, 1, 30, 47)),       # TinyLlama shape
    (W.BF16, 8, 8, 128, 256, (1, 257, 600, 1000), (1, 1, 88, 129)),   # group 1, n = 1
    (W.BF16, 16, 2, 64, 32, (5, 70, 200), (5, 1, 131)),               # group 8
    (W.BF16, 4, 2, 128, 16, (16, 32, 48), (16, 16, 16)),              # page-aligned chunks
    (W.BF16, 32, 4, 64, 16, (3000, 1, 700), (200, 1, 64)),            # long items cut into pieces
    (W.BF16, 16, 8, 128, 256, (5000, 2600), (300, 40)),               # pieces, group 2
    (W.BF16, 8, 1, 128, 16, (500, 1, 300), (1, 1, 70)),               # one KV head, group 8
    (W.BF16, 4, 4, 64, 32, (70, 900, 45), (1, 100, 45)),              # head_dim 64, group 1
    # 16-token pages cap a chunk at 63 pages (1008 keys): 160 k decode keys per KV head
    # make more chunks than the 128 decode waves of a head, claimed from the counter
    (W.BF16, 16, 8, 64, 16, (40000, 40000, 40000, 40000), (1, 1, 1, 1)),
    (W.F32, 4, 2, 16, 16, (5, 17, 33, 64), (1, 3, 1, 20)),            # fp32 prefill (token path)
    (W.F32, 8, 1, 64, 16, (100, 3, 700), (1, 3, 65)),
    (W.F32, 8, 4, 128, 32, (90, 190), (1, 45)),
]


@pytest.mark.parametrize("case", range(len(SMALL_CASES)))
def test_small_packed_ticks(case):
    dtype, Hq, Hkv, D, P, sl, ql = SMALL_CASES[case]
    t = _small(100 + case, dtype, Hq, Hkv, D, P, sl, ql, theta=1e4 if case % 2 else 1e6)
    say("small case", case, dtype, Hq, Hkv, D, P, sl, ql)
    _, out = run_gpu_tick(t)
    check_attention(out, oracle_tick(t), t.dtype, f"case{case}")


@pytest.mark.parametrize("split", [16, 32, 112, 512, 4096, 65536])
def test_split_count_invariance(split):
    t = _small(7, seq_lens=(2000, 1, 700, 300), query_lens=(1, 1, 1, 120))
    say("split", split)
    _, out = run_gpu_tick(t, kv_split_tokens=split)
    check_attention(out, oracle_tick(t), t.dtype, f"split{split}")


def _one_partition_tick(seed, Hq, Hkv, D, P, chunks):
    """Decode rows of 241..256 keys: each pads to 256 keys on the decode key
    axis, so with the automatic split (chunks of at least 256 keys, here
    exactly 256 since the tick has fewer rows than decode waves per KV head)
    every row is exactly one chunk, one partition; with chunks, two short
    prefill chunks (at most 4 key tiles, never cut into pieces) share the
    tick."""
    rng = np.random.default_rng(seed)
    S = 40
    sl = [int(x) for x in rng.integers(241, 257, size=S)]
    ql = [1] * S
    if chunks:
        sl += [200, 90]
        ql += [64, 90]
    return W.build_tick(rng, name="one-partition", dtype=W.BF16, Hq=Hq, Hkv=Hkv, D=D, P=P,
                        seq_lens=sl, query_lens=ql, theta=1e4, poison=True)


@pytest.mark.parametrize("Hq,Hkv,D,P,chunks", [(8, 2, 128, 16, False), (32, 8, 128, 256, False),
                                               (32, 4, 64, 16, True), (8, 8, 128, 256, True)])
def test_single_partition_rows_equal_the_merge_free_run_bitwise(Hq, Hkv, D, P, chunks):
    """Split-KV pin: rows that are one partition under the automatic split
    give the same bits as a run with partitions of 65536 keys, whose every row
    is one partition and which launches no merge kernel at all."""
    t = _one_partition_tick(140 + D + Hkv, Hq, Hkv, D, P, chunks)
    say("one-partition pin", Hq, Hkv, D, P, chunks)
    d = DevTick(t).write()
    auto = d.attend(0)
    torch.cuda.synchronize()
    pa.pa_profile_start(64)
    whole = d.attend(65536)
    rec = pa.pa_profile_stop()
    pa.pa_profile_reset()
    names = [n for n, _ in rec]
    assert not any("reduce" in n for n in names), names
    assert np.array_equal(_bits(auto), _bits(whole))
    check_attention(whole, oracle_tick(t), t.dtype, "one-partition")


def test_page_permutation_bitwise():
    t = W.make_config(4, poison=True)
    say("page permutation")
    _, a = run_gpu_tick(t)
    u = W.permute_pages(t, np.random.default_rng(5))
    _, b = run_gpu_tick(u)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def _attend_with_plan(d, kv_split_tokens=0):
    """Attention with a workspace of our own; returns (out, decode rows in the
    plan's row list), the count the plan writes first (group rows included)."""
    t = d.t
    dt = pa.PA_BF16 if t.dtype == W.BF16 else pa.PA_F32
    need = pa.pa_paged_attention_workspace_size(t.S, t.T, t.Hq, t.D, t.max_query_len,
                                                t.max_seq_len, t.P, kv_split_tokens, dt)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=DEV)
    out = pa.pa_paged_attention_varlen(d.q, d.k_pool, d.v_pool, d.block_tables, d.seq_lens,
                                       d.qsl, t.max_query_len, t.max_seq_len, scale=t.scale,
                                       kv_split_tokens=kv_split_tokens, workspace=ws)
    torch.cuda.synchronize()
    return out, int(ws[:4].view(torch.int32).item())


def test_shared_prefix_read_once_matches_private_copies():
    """Prefix caching (Helios blog, "Prefix caching"): sequences that share
    prefix pages attend to them as if each had its own copy. The shared
    prefix is read once per group of sharing rows (group rows in the plan),
    so the shared tick and the private-copy tick sum the prefix in different
    partitions: both are checked against the oracle, and against each other
    at the same tolerance."""
    t = W.make_config(5, poison=True)
    d = DevTick(t).write()
    say("shared prefix: grouped rows")
    a, rows = _attend_with_plan(d)
    n_dec = int((t.query_lens == 1).sum())
    assert rows > n_dec, (rows, n_dec)  # the 32 sharers were grouped
    ref = oracle_tick(t)
    check_attention(a, ref, t.dtype, "shared prefix, grouped")
    # give every sharing sequence its own copy of the prefix pages
    bt = t.block_tables.copy()
    kp, vp = d.k_pool, d.v_pool
    extra = []
    nxt = t.num_pages
    for s in range(32):
        for b in range(len(t.shared_pages)):
            extra.append(int(bt[s, b]))
            bt[s, b] = nxt
            nxt += 1
    idx = torch.tensor(extra, device=DEV, dtype=torch.long)
    kp2 = torch.cat([kp, kp[idx]])
    vp2 = torch.cat([vp, vp[idx]])
    say("shared prefix vs private copies")
    b_out = pa.pa_paged_attention_varlen(d.q, kp2, vp2, i32(bt), d.seq_lens, d.qsl,
                                         t.max_query_len, t.max_seq_len, scale=t.scale)
    torch.cuda.synchronize()
    check_attention(b_out, ref, t.dtype, "private copies")
    diff = (host_f32(a).astype(np.float64) - host_f32(b_out).astype(np.float64))
    assert np.abs(diff).max() <= BF16_MAX_ABS and np.abs(diff).mean() <= BF16_MEAN_ABS


# (Hq, Hkv, D, P, sharers, prefix pages, own keys after the prefix: low, high)
GROUP_CASES = [
    (32, 8, 128, 256, 10, 2, 1, 300),    # G = 4: groups of 4, 4 and a lone sharer
    (16, 16, 128, 16, 20, 5, 1, 40),     # G = 1: groups of 16 and 3 (one-key suffixes)
    (32, 4, 64, 16, 7, 3, 16, 64),       # G = 8: groups of 2 (and a lone sharer), D = 64
    (16, 8, 64, 256, 6, 1, 1, 256),      # G = 2: one group of 5 (up to 8 per group)
    (32, 8, 128, 16, 40, 64, 1, 2000),   # a 1024-key prefix over several chunks, 40 sharers
    (16, 8, 128, 16, 6, 16, 1, 40),      # a prefix of exactly 16 pages
    (32, 8, 128, 16, 9, 17, 1, 300),     # 17 prefix pages (the last one compared in memory)
]


@pytest.mark.parametrize("case", range(len(GROUP_CASES)))
def test_grouped_prefix_rows(case):
    """Decode rows sharing prefix pages, grouped (group rows read the prefix
    once for up to 16 / G sharers, whose own rows start after it; the merge
    sums both) against the oracle, beside rows that share nothing; and the
    same tick with a fixed split, which never groups."""
    Hq, Hkv, D, P, m, pp, lo, hi = GROUP_CASES[case]
    rng = np.random.default_rng(700 + case)
    own = [int(x) for x in rng.integers(lo, hi + 1, size=m)]
    sl = [pp * P + x for x in own] + [int(x) for x in rng.integers(20, 3000, size=5)]
    t = W.build_tick(rng, name="grouped", dtype=W.BF16, Hq=Hq, Hkv=Hkv, D=D, P=P,
                     seq_lens=sl, query_lens=[1] * len(sl), theta=1e4, poison=True,
                     shared_prefix_pages=pp, shared_prefix_seqs=range(m))
    say("grouped prefix rows", GROUP_CASES[case])
    d = DevTick(t).write()
    out, rows = _attend_with_plan(d)
    assert rows > len(sl), (rows, len(sl))
    ref = oracle_tick(t)
    check_attention(out, ref, t.dtype, "grouped")
    fixed, rows_fixed = _attend_with_plan(d, 512)
    assert rows_fixed == len(sl)
    check_attention(fixed, ref, t.dtype, "fixed split")


def test_grouped_prefix_tree():
    """Sharers whose page tables leave the leader's at different pages (a
    prefix tree; the pages after the split hold copies of the leader's, under
    other page ids): rows of one common-prefix length form their own groups,
    and every row still matches the oracle."""
    rng = np.random.default_rng(731)
    P, pp = 16, 6
    own = [int(x) for x in rng.integers(1, 200, size=12)]
    sl = [pp * P + x for x in own] + [int(x) for x in rng.integers(20, 900, size=3)]
    t = W.build_tick(rng, name="tree", dtype=W.BF16, Hq=32, Hkv=8, D=128, P=P,
                     seq_lens=sl, query_lens=[1] * len(sl), theta=1e4, poison=True,
                     pool_factor=2.0, shared_prefix_pages=pp, shared_prefix_seqs=range(12))
    spare = sorted(set(range(t.num_pages)) - set(t.block_tables[t.block_tables >= 0].tolist()))
    bt = t.block_tables.copy()
    kp, vp = t.k_pool.copy(), t.v_pool.copy()
    # sequences 3..6 leave at page 4, 7..9 at page 2; 1, 2, 10, 11 keep all 6
    for seqs, cut in ((range(3, 7), 4), (range(7, 10), 2)):
        for s in seqs:
            for j in range(cut, pp):
                new = spare.pop()
                kp[new] = kp[bt[s, j]]
                vp[new] = vp[bt[s, j]]
                bt[s, j] = new
    t = W.Tick(**{**t.__dict__, "block_tables": bt, "k_pool": kp, "v_pool": vp})
    say("grouped prefix tree")
    d = DevTick(t).write()
    out, rows = _attend_with_plan(d)
    # G = 4: groups of at most 4 rows: {1, 2, 10, 11}, {3..6}, {7, 8, 9}
    assert rows == len(sl) + 3, (rows, len(sl))
    check_attention(out, oracle_tick(t), t.dtype, "prefix tree")


def _subset_tick(t, seqs):
    """The same sequences as their own packed tick (rows copied, pools shared)."""
    u = W.Tick(**{**t.__dict__})
    seqs = list(seqs)
    u.seq_lens = t.seq_lens[seqs]
    u.query_lens = t.query_lens[seqs]
    u.block_tables = t.block_tables[seqs]
    u.qsl = np.zeros(len(seqs) + 1, np.int32)
    u.qsl[1:] = np.cumsum(u.query_lens)
    rows = np.concatenate([np.arange(t.qsl[s], t.qsl[s + 1]) for s in seqs])
    u.q = t.q[rows]
    u.positions = t.positions[rows]
    u.k = t.k[rows] if t.k is not None else None
    u.v = t.v[rows] if t.v is not None else None
    return u, rows


@pytest.mark.parametrize("split", [512, 0])
def test_mixed_tick_equals_separate_calls_and_any_order(split):
    """A row's result does not depend on the other rows of the tick or their
    order: bitwise with a fixed partition size; with the automatic size (chosen
    from the whole tick) the partitions, hence the rounding, may differ, so the
    rows agree to the bf16 parity tolerance."""
    t = W.make_config(4, poison=True)
    say(f"mixed tick vs separate, split {split}")
    d = DevTick(t).write()
    whole = d.attend(kv_split_tokens=split)
    torch.cuda.synchronize()
    whole_h = host_storage(whole, t.dtype)
    # decode rows alone and chunk rows alone, on the pools the full tick wrote
    for seqs in (range(48), range(48, 51), [50, 3, 48, 7, 49, 0]):
        u, rows = _subset_tick(t, seqs)
        q = storage_tensor(host_storage(d.q, t.dtype)[rows], t.dtype)
        out = pa.pa_paged_attention_varlen(q, d.k_pool, d.v_pool, i32(u.block_tables),
                                           i32(u.seq_lens), i32(u.qsl), u.max_query_len,
                                           t.max_seq_len, scale=t.scale, kv_split_tokens=split)
        torch.cuda.synchronize()
        if split:
            assert np.array_equal(host_storage(out, t.dtype), whole_h[rows]), list(seqs)[:4]
        else:
            diff = np.abs(host_f32(out) - host_f32(whole)[rows])
            assert diff.max() <= BF16_MAX_ABS, (list(seqs)[:4], float(diff.max()))


@pytest.mark.parametrize("dtype,D,G", [(W.F32, 16, 2), (W.BF16, 128, 4), (W.BF16, 64, 8),
                                       (W.F32, 64, 1)])
def test_one_hot_position_probe_exact(dtype, D, G):
    """Each row's weight is exactly 1 on one key: the output must be that key's
    V row exactly, which names the (page, row) the kernel read."""
    Hkv = 2
    t, targets = _pins.one_hot_tick(90 + D, dtype=dtype, Hq=Hkv * G, Hkv=Hkv, D=D, P=16,
                                    seq_lens=(9, 14, 6) if D == 16 else (40, 14, 63),
                                    query_lens=(1, 3, 1) if D == 16 else (1, 5, 7))
    say("one-hot probe", dtype, D, G)
    d = DevTick(t)
    out = d.attend()
    torch.cuda.synchronize()
    got = host_f32(out)
    for s, i, j in targets:
        page, row = int(t.block_tables[s][j // t.P]), j % t.P
        r = got[t.qsl[s] + i]
        assert np.all(r[:, 0] == page) and np.all(r[:, 2] == row), (s, i, j, r[:, :3])
        assert np.all(r[:, 1] == j)


def test_sequences_with_no_rows_and_host_bounds_larger_than_needed():
    t = _small(8, seq_lens=(50, 20, 300, 9), query_lens=(1, 0, 40, 0))
    say("empty sequences")
    d = DevTick(t).write()
    out = d.attend(max_query_len=t.max_query_len + 100, max_seq_len=t.max_seq_len + 1000)
    torch.cuda.synchronize()
    check_attention(out, oracle_tick(t), t.dtype, "empty-seqs")


def test_profile_hook_records_kernels():
    t = W.make_config(4, poison=False)
    d = DevTick(t).write()
    torch.cuda.synchronize()
    pa.pa_profile_start(64)
    d.attend()
    rec = pa.pa_profile_stop()
    names = [n for n, _ in rec]
    # a tick that may hold prefill chunks runs decode and prefill in one grid
    assert "plan" in names and "tick_attention" in names
    assert all(ms > 0 for _, ms in rec)
    pa.pa_profile_reset()


def _bits(x):
    return x.view(torch.int16 if x.element_size() == 2 else torch.int32).cpu().numpy()


def _many_seqs_tick(seed, S):
    """S short sequences, mostly decode rows, some chunks of up to 7 tokens and
    some with no rows this tick (runs of equal query_start_loc entries)."""
    rng = np.random.default_rng(seed)
    sl = rng.integers(1, 200, size=S)
    ql = np.ones(S, np.int64)
    ql[::50] = np.minimum(sl[::50], 7)
    ql[3::17] = 0
    return W.build_tick(rng, name=f"many{S}", dtype=W.BF16, Hq=4, Hkv=2, D=64, P=16,
                        seq_lens=list(sl), query_lens=list(ql), theta=1e4, poison=True)


@pytest.mark.parametrize("which", ["cfg4", "cfg3", "cfg5", "small0", "small_f32", "split512",
                                   "many100", "many1100", "many4500", "norope"])
def test_tick_forward_equals_the_three_calls_bitwise(which):
    """pa_tick_forward (slot mapping, page write and plan in one launch) ==
    the three calls in order; the many-sequence ticks take the token search
    over more than 64 and more than 4096 sequences and the plan past its
    cached sequence shapes."""
    if which.startswith("cfg"):
        t = W.make_config(int(which[3:]), poison=True)
    elif which == "small_f32":   # the per-token path: no plan
        t = _small(120, *SMALL_CASES[10])
    elif which.startswith("many"):
        t = _many_seqs_tick(122, int(which[4:]))
    elif which == "norope":  # no cos/sin table: K and V stored as given
        t = _small(123, *SMALL_CASES[1], theta=None)
    else:
        t = _small(121, *SMALL_CASES[0])
    assert not t.new_in_pool
    split = 512 if which == "split512" else 0
    say("tick forward", which)
    a = DevTick(t).write()
    ref = a.attend(split)
    b = DevTick(t)
    table = b.oracle_table()
    slots = torch.full((t.T,), -7, dtype=torch.int32, device=DEV)
    out = pa.pa_tick_forward(b.q, b.k, b.v, b.positions, b.block_tables, b.seq_lens, b.qsl,
                             table, b.k_pool, b.v_pool, t.max_query_len, t.max_seq_len,
                             scale=t.scale, kv_split_tokens=split, slot_mapping=slots)
    torch.cuda.synchronize()
    for name, x, y in (("out", ref, out), ("slots", a.slots, slots),
                       ("k_pool", a.k_pool, b.k_pool), ("v_pool", a.v_pool, b.v_pool)):
        assert np.array_equal(_bits(x), _bits(y)), f"{which}: {name} differs"
    # and the write side equals the oracle's bit for bit (same cos/sin table)
    res = oracle.run_tick(t.dtype, t.q, t.k, t.v, t.positions, t.block_tables, t.qsl,
                          t.seq_lens, t.k_pool, t.v_pool,
                          oracle.rope_table(t.max_pos, t.D, t.theta) if t.theta else None,
                          t.scale)
    for name, x in (("slots", slots), ("k_pool", b.k_pool), ("v_pool", b.v_pool)):
        want = res[name]
        got = _bits(x).reshape(want.shape)
        assert np.array_equal(got, want.view(got.dtype)), f"{which}: {name} != oracle"
    # q and k: the fused bf16 tick rotates them where it reads them and leaves
    # the inputs as they are; a float32 tick rotates them in place, as the
    # three calls do
    for name, x, given, rotated in (("q", b.q, t.q, res["q"]), ("k", b.k, t.k, res["k"])):
        want = given if t.dtype == W.BF16 else rotated
        got = _bits(x).reshape(want.shape)
        assert np.array_equal(got, want.view(got.dtype)), f"{which}: {name}"
    if which.startswith("many"):  # these sizes are not among the parity cases above
        check_attention(out, oracle_tick(t), t.dtype, which)


@pytest.mark.parametrize("D,G,split,chunks", [(128, 4, 0, False), (128, 4, 16, False),
                                              (64, 8, 48, False), (128, 1, 0, True),
                                              (64, 2, 32, True)])
def test_decode_walk_many_short_rows(D, G, split, chunks):
    """Decode rows of 1..70 keys on 16-token pages: every decode wave's chunk
    holds many ranges of one to five 16-key buffers (odd and even counts, so
    the buffer that holds the next range's first keys alternates, and ragged
    ends), with automatic and fixed partitions; with `chunks`, two prefill
    chunks share the tick (the fused kernel's decode workers)."""
    rng = np.random.default_rng(130 + D + G + split)
    S = 300
    sl = [int(x) for x in rng.integers(1, 71, size=S)]
    ql = [1] * S
    if chunks:
        sl += [90, 200]
        ql += [40, 64]
    t = W.build_tick(rng, name="short-rows", dtype=W.BF16, Hq=2 * G, Hkv=2, D=D, P=16,
                     seq_lens=sl, query_lens=ql, theta=1e4, poison=True)
    say("short rows", D, G, split, chunks)
    _, out = run_gpu_tick(t, kv_split_tokens=split)
    check_attention(out, oracle_tick(t), t.dtype, f"short-rows D{D} G{G} split{split}")


def test_side_stream_with_binding_allocated_buffers():
    """The binding allocates the workspace, out and the slots on the stream the
    kernels run on: work queued meanwhile on the current stream, allocating
    and filling fresh memory, cannot take those bytes while the tick runs."""
    t = W.make_config(4, poison=True)
    ref_d = DevTick(t).write()
    ref = ref_d.attend()
    torch.cuda.synchronize()
    d = DevTick(t)
    table = d.oracle_table()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    say("side stream tick")
    out = pa.pa_tick_forward(d.q, d.k, d.v, d.positions, d.block_tables, d.seq_lens, d.qsl,
                             table, d.k_pool, d.v_pool, t.max_query_len, t.max_seq_len,
                             scale=t.scale, stream=side)
    for _ in range(8):
        junk = torch.empty(64 << 20, dtype=torch.uint8, device=DEV)
        junk.fill_(0xFF)
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
