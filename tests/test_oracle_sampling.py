"""Pins of the sampling oracle (oracle/sampling.py) to things other than itself:
numpy's argmax for greedy rows, a hand-worked top-p example, the sampled
frequencies over a fine grid of uniforms against probabilities computed by
brute force with Python floats and sorted(), exact identities of the
temperature, and the ends of the uniform range. Planted mistakes (tie order,
top-p and top-k off by one, temperature or max shift dropped, drawing in
ranking order) are each caught by at least one pin."""

import math

import numpy as np
import pytest

from oracle import sampling as osm


def brute_probs(x, T, k, p):
    """Kept set and renormalised probabilities, by brute force in Python floats."""
    V = len(x)
    order = sorted(range(V), key=lambda i: (-float(x[i]), i))
    if 0 < k < V:
        order = order[:k]
    m = max(float(v) for v in x)
    w = {i: math.exp((float(x[i]) - m) / T) for i in order}
    if p < 1:
        tot = sum(w.values())
        keep, run = [], 0.0
        for i in order:
            keep.append(i)
            run += w[i]
            if run >= p * tot * (1 - 1e-12):
                break
        order = keep
    tot = sum(w[i] for i in order)
    return {i: w[i] / tot for i in order}


def test_greedy_is_numpy_argmax():
    rng = np.random.default_rng(0)
    for _ in range(50):
        x = np.round(rng.standard_normal(rng.integers(1, 300)) * 2) / 2   # many ties
        x = x.astype(np.float32)
        for T, k in ((0.0, 0), (-1.0, 50), (0.7, 1)):
            for u in (0.0, 0.5, 0.999):
                assert osm.sample_row(x, T, k, 0.9, u) == int(np.argmax(x))


def test_signed_zero_ties_by_index():
    assert list(osm.ranking(np.array([0.0, -0.0], np.float32))) == [0, 1]
    assert list(osm.ranking(np.array([-0.0, 0.0], np.float32))) == [0, 1]


def test_top_p_worked_example():
    # probabilities 0.5, 0.3, 0.15, 0.05 (in shuffled positions)
    probs = {2: 0.5, 0: 0.3, 3: 0.15, 1: 0.05}
    x = np.array([math.log(probs[i]) for i in range(4)], np.float32)
    grid = [(i + 0.5) / 400 for i in range(400)]
    seen = lambda p: {osm.sample_row(x, 1.0, 0, p, u) for u in grid}
    assert seen(0.75) == {2, 0}            # 0.5 + 0.3 reaches 0.75
    assert seen(0.85) == {2, 0, 3}         # needs the third most probable
    assert seen(1.0) == {0, 1, 2, 3}
    assert seen(0.4) == {2}                # the top token alone reaches 0.4
    assert seen(1e-9) == {2}
    # top-k first, then top-p inside what top-k kept
    assert {osm.sample_row(x, 1.0, 2, 1.0, u) for u in grid} == {2, 0}
    assert {osm.sample_row(x, 1.0, 3, 0.9, u) for u in grid} == {2, 0, 3}


@pytest.mark.parametrize("T,k,p", [(1.0, 0, 1.0), (0.5, 0, 1.0), (2.0, 0, 1.0), (1.0, 3, 1.0),
                                   (0.8, 0, 0.7), (1.3, 5, 0.9), (0.2, 0, 0.95)])
def test_frequencies_match_brute_force_probabilities(T, k, p):
    rng = np.random.default_rng(int(T * 10) + k)
    x = rng.standard_normal(7).astype(np.float32)
    M = 20000
    counts = {}
    for i in range(M):
        t = osm.sample_row(x, T, k, p, (i + 0.5) / M)
        counts[t] = counts.get(t, 0) + 1
    ref = brute_probs(x, T, k, p)
    assert set(counts) == set(ref)
    for t, pr in ref.items():
        assert abs(counts[t] / M - pr) <= 2.0 / M + 1e-6, (t, counts[t] / M, pr)


def test_temperature_divides_the_logit_gap():
    rng = np.random.default_rng(3)
    for _ in range(40):
        x = rng.standard_normal(50).astype(np.float32)
        u = float(rng.random())
        # (2x - 2m) / 2 == (x - m) exactly in binary, so the draws agree exactly
        assert osm.sample_row(2 * x, 2.0, 0, 1.0, u) == osm.sample_row(x, 1.0, 0, 1.0, u)
        top2 = np.sort(x)[-2:]
        if top2[1] - top2[0] >= 0.05:     # exp(-50) * 2**32 < 1: only the top token weighs
            assert osm.sample_row(x, 1e-3, 0, 1.0, u) == int(np.argmax(x))


def test_uniform_ends_pick_first_and_last_kept_index():
    x = np.array([0.1, 2.0, -np.inf, 1.5, 1.9, -3.0], np.float32)
    kept = sorted(int(i) for i in osm.kept_tokens(x, 1.0, 3, 1.0))
    assert kept == [1, 3, 4]
    assert osm.sample_row(x, 1.0, 3, 1.0, 0.0) == 1
    assert osm.sample_row(x, 1.0, 3, 1.0, np.nextafter(np.float32(1), np.float32(0))) == 4
    # a -inf logit is never drawn
    draws = {osm.sample_row(x, 1.0, 0, 1.0, (i + 0.5) / 1000) for i in range(1000)}
    assert 2 not in draws and draws <= {0, 1, 3, 4, 5}


def test_weights_are_exact_integers():
    x = np.array([1.0, 0.0, -1.0], np.float32)
    w = osm.weights(x, 1.0)
    assert int(w[0]) == 2 ** 32
    assert int(w[1]) == math.floor(math.exp(-1.0) * 2 ** 32)
    assert int(w[2]) == math.floor(math.exp(-2.0) * 2 ** 32)


# ------------------------------------------- planted mistakes must be caught
PINS = [test_greedy_is_numpy_argmax, test_signed_zero_ties_by_index, test_top_p_worked_example,
        lambda: test_frequencies_match_brute_force_probabilities(0.8, 0, 0.7),
        lambda: test_frequencies_match_brute_force_probabilities(1.3, 5, 0.9),
        lambda: test_frequencies_match_brute_force_probabilities(2.0, 0, 1.0),
        test_temperature_divides_the_logit_gap, test_uniform_ends_pick_first_and_last_kept_index,
        test_weights_are_exact_integers]


def _caught():
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            return True
    return False


def _ties_high_index_first(x):
    x = np.asarray(x, dtype=np.float64) + 0.0
    return np.lexsort((-np.arange(x.size), -x))


def _top_p_one_too_many(x, temperature, top_k, top_p):
    order = osm.ranking(x)
    if 0 < top_k < order.size:
        order = order[:top_k]
    if top_p < 1.0:
        w = osm.weights(x, temperature)[order]
        need = max(math.ceil(float(np.float32(top_p)) * float(int(w.sum()))), 1)
        cum = np.cumsum(w.astype(object))
        t = next(i for i, c in enumerate(cum) if c >= need)
        order = order[:t + 2]
    return order


def _top_k_plus_one(x, temperature, top_k, top_p):
    return _orig["kept_tokens"](x, temperature, top_k + 1 if top_k > 0 else top_k, top_p)


def _no_temperature(x, temperature):
    return _orig["weights"](x, 1.0)


def _no_max_shift(x, temperature):
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        w = np.floor(np.exp(x / np.float64(temperature)) * osm.TWO32)
        return np.nan_to_num(w, posinf=2.0 ** 63).astype(np.uint64)


def _draw_in_ranking_order(x, temperature, top_k, top_p, u):
    x = np.asarray(x, dtype=np.float32)
    if not temperature > 0 or top_k == 1:
        return int(osm.ranking(x)[0])
    kept = osm.kept_tokens(x, temperature, top_k, top_p)
    w = osm.weights(x, temperature)
    S = int(w[kept].sum())
    target, run = int(math.floor(float(np.float32(u)) * S)), 0
    for i in kept:
        run += int(w[i])
        if run > target:
            return int(i)


_orig = {"ranking": osm.ranking, "kept_tokens": osm.kept_tokens, "weights": osm.weights,
         "sample_row": osm.sample_row}


@pytest.mark.parametrize("name,fn", [
    ("ranking", _ties_high_index_first), ("kept_tokens", _top_p_one_too_many),
    ("kept_tokens", _top_k_plus_one), ("weights", _no_temperature), ("weights", _no_max_shift),
    ("sample_row", _draw_in_ranking_order)])
def test_planted_mistakes_are_caught(monkeypatch, name, fn):
    monkeypatch.setattr(osm, name, fn)
    assert _caught(), f"a mistake in {name} ({fn.__name__}) passes every pin"
