"""pa_sample_tokens on the GPU against the sampling oracle, token for token.

Every token is an integer decision, so the bar is equality. Both sides take
the decision on the same integer weights; the one rounding step that can
differ is the float64 exp of a logit (each side's library exp is within an
ulp), which changes a token only when a uniform lands within a few parts in
2**32 of a boundary between tokens, so equality is expected throughout.
"""

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings as hsettings, strategies as st

from oracle import sampling as osm
import paged_kv_cache_page_amd as pa
from _gpu import DEV, say

pytestmark = pytest.mark.gpu

QWEN_VOCAB = 151936


def settings(rng, R, V):
    T = rng.choice([0.0, 0.2, 0.7, 1.0, 1.5, 2.0], R).astype(np.float32)
    k = rng.choice([0, 1, 2, 5, 50, 1000, V, V + 7, -1], R).astype(np.int32)
    p = rng.choice([1.0, 0.95, 0.9, 0.5, 0.01, 1e-7], R).astype(np.float32)
    u = rng.random(R, dtype=np.float32)
    return T, k, p, u


def run(logits, T, k, p, u):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    out = pa.pa_sample_tokens(t(logits), t(T), t(k), t(p), t(u))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(logits, T, k, p, u, where):
    say("sample", where, logits.shape)
    got = run(logits, T, k, p, u)
    want = osm.sample_rows(logits, T, k, p, u)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(where, int(r), float(T[r]), int(k[r]), float(p[r]), float(u[r]),
                            int(got[r]), int(want[r])) for r in bad[:5]]
    return got


@pytest.mark.parametrize("seed", [0, 1])
def test_qwen_vocab_mixed_settings(seed):
    rng = np.random.default_rng(100 + seed)
    R, V = 48, QWEN_VOCAB
    logits = (rng.standard_normal((R, V)) * 4).astype(np.float32)
    T, k, p, u = settings(rng, R, V)
    check(logits, T, k, p, u, f"qwen seed {seed}")


@pytest.mark.parametrize("V", [1, 2, 3, 1023, 1024, 1025, 3001])
def test_small_and_ragged_vocab(V):
    rng = np.random.default_rng(V)
    R = 24
    logits = (rng.standard_normal((R, V)) * 2).astype(np.float32)
    T, k, p, u = settings(rng, R, V)
    check(logits, T, k, p, u, f"V={V}")


@pytest.mark.parametrize("V", [300, 3000, 5000])   # a one-wave list, a workgroup list, or none
def test_ties_signed_zeros_and_minus_inf(V):
    rng = np.random.default_rng(7)
    R = 40
    logits = (np.round(rng.standard_normal((R, V)) * 2) / 4).astype(np.float32)  # wide tie groups
    logits[:, ::7] = -np.inf
    logits[::3, 5] = 0.0
    logits[::3, 6] = -0.0
    logits[1, :] = 0.0                                 # a whole row of one value
    logits[2, :] = -np.inf
    logits[2, V - 7] = 1.0                             # a single finite logit
    T = np.full(R, 1.0, np.float32)
    T[::5] = 0.5
    k = rng.choice([0, 3, 10, 100, 777], R).astype(np.int32)   # cuts through tie groups
    p = rng.choice([1.0, 0.3, 0.6, 0.99], R).astype(np.float32)
    u = rng.random(R, dtype=np.float32)
    u[0], u[3] = 0.0, np.float32(np.nextafter(np.float32(1), np.float32(0)))
    got = check(logits, T, k, p, u, "ties")
    assert got[2] == V - 7


def test_batched_equals_per_row_and_repeats():
    rng = np.random.default_rng(9)
    R, V = 16, 32000
    logits = (rng.standard_normal((R, V)) * 3).astype(np.float32)
    T, k, p, u = settings(rng, R, V)
    batched = run(logits, T, k, p, u)
    for r in range(R):
        one = run(logits[r:r + 1], T[r:r + 1], k[r:r + 1], p[r:r + 1], u[r:r + 1])
        assert one[0] == batched[r], r
    assert np.array_equal(run(logits, T, k, p, u), batched)


def test_rows_sharing_settings_sample_their_own_distribution():
    # 4096 rows of the same logits, one temperature and top-p, uniforms on a grid:
    # the token counts follow the kept probabilities (inverse transform)
    rng = np.random.default_rng(11)
    V, R = 64, 4096
    row = (rng.standard_normal(V) * 1.5).astype(np.float32)
    logits = np.tile(row, (R, 1))
    T = np.full(R, 0.8, np.float32)
    k = np.zeros(R, np.int32)
    p = np.full(R, 0.9, np.float32)
    u = ((np.arange(R) + 0.5) / R).astype(np.float32)
    got = check(logits, T, k, p, u, "shared settings")
    kept = osm.kept_tokens(row, 0.8, 0, 0.9)
    w = osm.weights(row, 0.8)[kept].astype(np.float64)
    freq = np.bincount(got, minlength=V)[kept] / R
    assert np.abs(freq - w / w.sum()).max() <= 2.0 / R


@pytest.mark.parametrize("sigma,T,where", [
    (4.0, 0.2, "short list"),
    (2.0, 0.2, "list of 1025-4096 tokens, radix descent over the list"),
    (1.0, 1.0, "slices overflow, radix descent over the row"),
])
def test_each_draw_path(sigma, T, where):
    # 24576 tokens = 8 slices of 3072; the logit spread against the temperature
    # sets how many tokens pass the weight screen, and so which path a row takes
    rng = np.random.default_rng(int(sigma * 100))
    R, V = 24, 24576
    logits = (rng.standard_normal((R, V)) * sigma).astype(np.float32)
    Tr = np.full(R, T, np.float32)
    k = rng.choice([0, 0, 40, 900, 3000], R).astype(np.int32)
    p = rng.choice([1.0, 0.95, 0.6, 0.2], R).astype(np.float32)
    u = rng.random(R, dtype=np.float32)
    check(logits, Tr, k, p, u, where)


def test_long_merged_list_without_slice_overflow():
    # 8 slices of 3072 tokens; each slice lists about 800 tokens near the row
    # maximum (below its 1024-token capacity), so no slice overflows, while the
    # merged list (about 6400 tokens) exceeds the draw kernel's 4096-token LDS
    # list: the row path, reached without an overflowing slice
    rng = np.random.default_rng(13)
    R, V = 12, 24576
    logits = np.full((R, V), -200.0, np.float32) + rng.standard_normal((R, V)).astype(np.float32)
    for r in range(R):
        for sl in range(V // 3072):
            idx = sl * 3072 + rng.choice(3072, 800, replace=False)
            logits[r, idx] = rng.standard_normal(800).astype(np.float32)
    T = np.full(R, 1.0, np.float32)
    k = rng.choice([0, 0, 5000, 6000, 100], R).astype(np.int32)
    p = rng.choice([1.0, 0.99, 0.9, 0.5], R).astype(np.float32)
    u = rng.random(R, dtype=np.float32)
    check(logits, T, k, p, u, "long merged list")


def test_list_lengths_around_the_one_wave_limit():
    # 8 slices of 3072 tokens; row r lists exactly n[r] tokens (values N(0, 1),
    # spread over every slice so that no slice overflows), the rest sit 200
    # below and weigh 0. Lists of up to 512 tokens are ranked by one wave,
    # longer ones by the whole workgroup: both sides of that limit, and the
    # ends of a wave's lanes (63, 64, 65 tokens)
    rng = np.random.default_rng(17)
    n = np.array([8, 9, 63, 64, 65, 200, 511, 512, 513, 777, 1024, 1025, 2000] * 2)
    R, V = n.size, 24576
    logits = np.full((R, V), -200.0, np.float32) + rng.standard_normal((R, V)).astype(np.float32)
    for r in range(R):
        per = np.full(8, n[r] // 8) + (np.arange(8) < n[r] % 8)
        idx = np.concatenate([sl * 3072 + rng.choice(3072, c, replace=False)
                              for sl, c in enumerate(per)])
        logits[r, idx] = rng.standard_normal(idx.size).astype(np.float32)
        if r >= R // 2:
            logits[r, idx[::3]] = logits[r, idx[0]]   # ties across the listed tokens
    T = np.full(R, 1.0, np.float32)
    T[1::4] = 0.5
    k = rng.choice([0, 0, 5, 50, 500], R).astype(np.int32)
    k[2] = n[2] - 1
    k[3] = n[3]
    p = rng.choice([1.0, 0.95, 0.5, 0.01], R).astype(np.float32)
    u = rng.random(R, dtype=np.float32)
    u[0] = 0.0
    u[1] = np.float32(np.nextafter(np.float32(1), np.float32(0)))
    check(logits, T, k, p, u, "list lengths")


@st.composite
def random_rows(draw):
    # up to 6 rows of up to 7000 tokens: every draw path (one-wave and
    # workgroup lists, overflowing slices), spreads from flat to peaked, ties
    R = draw(st.integers(1, 6))
    V = draw(st.integers(1, 7000))
    spread = draw(st.sampled_from([0.25, 1.0, 4.0, 16.0]))
    ties = draw(st.booleans())
    rng = np.random.default_rng(draw(st.integers(0, 2**31 - 1)))
    logits = (rng.standard_normal((R, V)) * spread).astype(np.float32)
    if ties:
        logits = np.round(logits).astype(np.float32)
    T = rng.choice([0.0, 0.1, 0.2, 0.7, 1.0, 2.0], R).astype(np.float32)
    k = np.where(rng.random(R) < 0.5, 0, rng.integers(1, V + 3, R)).astype(np.int32)
    p = rng.choice([1.0, 0.95, 0.5, 0.1, 1e-6], R).astype(np.float32)
    u = rng.random(R, dtype=np.float32)
    return logits, T, k, p, u


@hsettings(max_examples=30, deadline=None, derandomize=True, database=None,
           suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(random_rows())
def test_random_rows_match_the_oracle(case):
    logits, T, k, p, u = case
    check(logits, T, k, p, u, f"random rows {logits.shape}")
