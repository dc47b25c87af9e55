"""Pins for page indexing, the page write and the gather."""

import os

import numpy as np

import oracle
from _brute import brute_gather

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_pool_size_worked_example_from_the_pages():
    # llm-serving-engine README, "KV cache memory layout": [22, 2, 256, 16, 4, 64] fp32 = 184.5 MB.
    with open(os.path.join(GOLDEN, "kv_storage_size.txt")) as f:
        row = [line for line in f if line.strip() and not line.startswith("#")][0].split()
    layers, blocks, bs, hkv, hd, eb = map(int, row[:6])
    printed_mb = float(row[6])
    nbytes = oracle.pool_bytes(layers, blocks, bs, hkv, hd, eb)
    assert nbytes == 184_549_376
    assert round(nbytes / 1e6, 1) == printed_mb


def _labelled_pool(num_pages, P, Hkv, D):
    """Every element encodes (page, row, head, dim) exactly in float32."""
    pg, row, h, d = np.meshgrid(np.arange(num_pages), np.arange(P), np.arange(Hkv),
                                np.arange(D), indexing="ij")
    return (pg * 100000 + row * 100 + h * 10 + d % 10).astype(np.float32)


def test_gather_matches_brute_force_codes():
    rng = np.random.default_rng(6)
    P, Hkv, D = 4, 2, 3
    pool = _labelled_pool(12, P, Hkv, D)
    table = rng.permutation(12)[:5]
    for n in (1, 3, 4, 5, 17, 20):
        got = oracle.gather_sequence(pool, table, n)
        ref = np.array(brute_gather(pool.tolist(), list(table), n, P), dtype=np.float32)
        assert np.array_equal(got, ref)
        # the decoded (page, row) of key j is (table[j // P], j % P)
        for j in range(n):
            code = int(got[j, 0, 0])
            assert code // 100000 == table[j // P] and (code // 100) % 1000 == j % P


def test_slot_mapping_brute_force():
    rng = np.random.default_rng(7)
    P = 16
    bt = np.stack([rng.permutation(64)[:8] for _ in range(3)]).astype(np.int32)
    qsl = np.array([0, 1, 6, 9])
    positions = np.array([100, 20, 21, 22, 23, 24, 0, 1, 2])
    slots = oracle.slot_mapping(bt, qsl, positions, P)
    seq_of = [0, 1, 1, 1, 1, 1, 2, 2, 2]
    for t, s in enumerate(seq_of):
        p = positions[t]
        assert slots[t] == bt[s][p // P] * P + p % P


def test_write_cache_touches_only_its_slots_and_skips_negative():
    rng = np.random.default_rng(8)
    P, Hkv, D = 4, 2, 8
    kp = rng.standard_normal((6, P, Hkv, D)).astype(np.float32)
    vp = rng.standard_normal((6, P, Hkv, D)).astype(np.float32)
    k = rng.standard_normal((3, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((3, Hkv, D)).astype(np.float32)
    slots = np.array([5, -1, 22])
    k2, v2 = oracle.write_cache(kp, vp, slots, k, v)
    assert np.array_equal(k2[1, 1], k[0]) and np.array_equal(v2[5, 2], v[2])
    mask = np.ones((6, P), bool)
    mask[1, 1] = mask[5, 2] = False
    assert np.array_equal(k2[mask], kp[mask]) and np.array_equal(v2[mask], vp[mask])
    # inputs untouched
    assert not np.array_equal(k2, kp)


def test_write_cache_keeps_bits_of_bf16_rows():
    rng = np.random.default_rng(9)
    kp = rng.integers(0, 65535, size=(2, 4, 1, 8)).astype(np.uint16)
    vp = kp.copy()
    k = rng.integers(0, 65535, size=(1, 1, 8)).astype(np.uint16)
    k2, v2 = oracle.write_cache(kp, vp, [6], k, k)
    assert np.array_equal(k2[1, 2], k[0]) and k2.dtype == np.uint16
