"""Plant plausible mistakes in (copies of) the oracle, on the CPU, and check that
at least one pin catches each: evidence that the pins are not blind to the
errors they are meant to rule out."""

import numpy as np
import pytest

import oracle
import oracle.attention as oatt
import oracle.rope as orope
import _pins
import test_oracle_rope as rope_pins


def _attend_factory(group_of=None, mask=None, use_scale=True, subtract_max=True,
                    values_from_keys=False):
    def attend(q, K, V, scale):
        q = np.asarray(q, np.float64)
        K = np.asarray(K, np.float64)
        V = np.asarray(V, np.float64)
        L, Hq, D = q.shape
        n, Hkv, _ = K.shape
        if L == 0:
            return np.zeros((0, Hq, D))
        rows = np.arange(L)[:, None]
        keys = np.arange(n)[None, :]
        visible = mask(rows, keys, n, L) if mask else keys <= (n - L + rows)
        out = np.empty((L, Hq, D))
        for h in range(Hq):
            g = group_of(h, Hq, Hkv) if group_of else h // (Hq // Hkv)
            s = q[:, h] @ K[:, g].T * (scale if use_scale else 1.0)
            s = np.where(visible, s, -np.inf)
            top = s.max(axis=1, keepdims=True) if subtract_max else 0.0
            with np.errstate(over="ignore", invalid="ignore"):
                w = np.exp(s - top)
                w = w / w.sum(axis=1, keepdims=True)
            out[:, h] = w @ (K[:, g] if values_from_keys else V[:, g])
        return out
    return attend


ATTEND_MUTANTS = {
    "interleaved_gqa": _attend_factory(group_of=lambda h, Hq, Hkv: h % Hkv),
    "top_left_causal": _attend_factory(mask=lambda r, k, n, L: k <= r),
    "diagonal_excluded": _attend_factory(mask=lambda r, k, n, L: k < n - L + r),
    "no_causal_mask": _attend_factory(mask=lambda r, k, n, L: np.ones_like(k + r, bool)),
    "dropped_scale": _attend_factory(use_scale=False),
    "no_max_subtraction": _attend_factory(subtract_max=False),
    "values_from_keys": _attend_factory(values_from_keys=True),
}


def _gather_reversed_pages(pool, row, n):
    P = pool.shape[1]
    nb = (n + P - 1) // P
    pages = np.asarray(row[:nb])[::-1]
    return pool[pages].reshape((nb * P,) + pool.shape[2:])[:n]


def _gather_row_major_slot_error(pool, row, n):
    # reads slot j from page table entry j % nb (a transposed index)
    P = pool.shape[1]
    nb = (n + P - 1) // P
    out = np.empty((n,) + pool.shape[2:], pool.dtype)
    for j in range(n):
        out[j] = pool[row[j % nb], j // nb if j // nb < P else P - 1]
    return out


GATHER_MUTANTS = {"reversed_pages": _gather_reversed_pages,
                  "transposed_slot_index": _gather_row_major_slot_error}


def _failing_pins():
    failed = []
    for pin in _pins.ALL_PINS:
        try:
            pin(oracle.paged_attention_varlen)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(ATTEND_MUTANTS))
def test_attention_mutant_is_caught(monkeypatch, name):
    monkeypatch.setattr(oatt, "attend_sequence", ATTEND_MUTANTS[name])
    assert _failing_pins(), f"no pin caught mutant {name}"


@pytest.mark.parametrize("name", sorted(GATHER_MUTANTS))
def test_gather_mutant_is_caught(monkeypatch, name):
    monkeypatch.setattr(oatt, "gather_sequence", GATHER_MUTANTS[name])
    assert _failing_pins(), f"no pin caught mutant {name}"


def _rope_pins_fail():
    tests = [rope_pins.test_inv_freq_closed_form, rope_pins.test_unit_vector_closed_form_half_split_pairs,
             rope_pins.test_position_zero_is_identity_bitwise, rope_pins.test_pair_norms_preserved,
             rope_pins.test_relative_position_property,
             rope_pins.test_rotation_matches_scalar_brute_force_bitwise]
    failed = []
    for t in tests:
        try:
            t()
        except AssertionError:
            failed.append(t.__name__)
    return failed


def _rotate_sign_flip(x, positions, table):
    x = np.asarray(x, np.float32)
    half = x.shape[-1] // 2
    c = table[np.asarray(positions), :half][:, None, :]
    s = table[np.asarray(positions), half:][:, None, :]
    y = np.empty_like(x)
    y[..., :half] = x[..., :half] * c + x[..., half:] * s
    y[..., half:] = x[..., half:] * c - x[..., :half] * s
    return y


def _rotate_interleaved(x, positions, table):
    x = np.asarray(x, np.float32)
    half = x.shape[-1] // 2
    c = table[np.asarray(positions), :half][:, None, :]
    s = table[np.asarray(positions), half:][:, None, :]
    x1, x2 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x1 * c - x2 * s
    y[..., 1::2] = x2 * c + x1 * s
    return y


def _rotate_fused(x, positions, table):
    # float64 arithmetic rounded once at the end: a fused-multiply-add-like mistake
    x = np.asarray(x, np.float64)
    half = x.shape[-1] // 2
    c = table[np.asarray(positions), :half][:, None, :].astype(np.float64)
    s = table[np.asarray(positions), half:][:, None, :].astype(np.float64)
    y = np.empty_like(x)
    y[..., :half] = x[..., :half] * c - x[..., half:] * s
    y[..., half:] = x[..., half:] * c + x[..., :half] * s
    return y.astype(np.float32)


def _inv_freq_wrong_exponent(D, theta):
    i = np.arange(D // 2, dtype=np.float64)
    return np.power(np.float64(theta), -i / np.float64(D))


@pytest.mark.parametrize("name,attr,fn", [
    ("sign_flip", "rope_rotate", _rotate_sign_flip),
    ("interleaved_pairs", "rope_rotate", _rotate_interleaved),
    ("fused_rounding", "rope_rotate", _rotate_fused),
    ("exponent_i_over_D", "rope_inv_freq", _inv_freq_wrong_exponent),
])
def test_rope_mutant_is_caught(monkeypatch, name, attr, fn):
    monkeypatch.setattr(orope, attr, fn)
    # the pins call through the package namespace
    monkeypatch.setattr(oracle, attr, fn)
    assert _rope_pins_fail(), f"no pin caught rope mutant {name}"
