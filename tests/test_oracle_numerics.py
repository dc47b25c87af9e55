"""Pins for the oracle's storage conversions (bf16 <-> float32)."""

import math

import numpy as np
import pytest
import torch

import oracle
from _brute import f32


def _nearest_bf16_brute(x):
    """Nearest bf16 to float32 x by trying both candidates around it (float64
    distances), ties to the even mantissa. Returns uint16 bits."""
    u = int(np.float32(x).view(np.uint32))
    lo_bits = u >> 16
    cands = [lo_bits, lo_bits + 1]
    def val(b):
        return float(np.uint32(b << 16).view(np.float32))
    best = None
    for b in cands:
        v = val(b)
        dist = abs(v - float(x)) if math.isfinite(v) else math.inf
        if best is None or dist < best[1] or (dist == best[1] and b % 2 == 0):
            best = (b, dist)
    return best[0]


def test_bf16_widen_all_patterns_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = oracle.bf16_bits_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    same = (mine.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()


def test_bf16_round_brute_force_nearest_even():
    rng = np.random.default_rng(0)
    xs = np.concatenate([
        rng.standard_normal(2000).astype(np.float32),
        (rng.standard_normal(500) * 1e30).astype(np.float32),
        (rng.standard_normal(500) * 1e-30).astype(np.float32),
        # exact halfway points between neighbouring bf16 values, odd and even kept halves
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x3F80FFFF, 0x3F807FFF, 0x00008000,
                  0x00018000], dtype=np.uint32).view(np.float32),
    ])
    mine = oracle.f32_to_bf16_bits(xs)
    for x, b in zip(xs, mine):
        assert int(b) == _nearest_bf16_brute(x), hex(int(np.float32(x).view(np.uint32)))


def test_bf16_round_matches_torch_and_specials():
    rng = np.random.default_rng(1)
    xs = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(3.0),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 3.4028235e38], dtype=np.float32),
    ])
    mine = oracle.f32_to_bf16_bits(xs)
    ref = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    nan_bits = oracle.f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(oracle.bf16_bits_to_f32(nan_bits))[0]


def test_f32_helper_rounds():
    assert f32(1.0 + 2.0 ** -30) == 1.0
    assert f32(1.0 + 2.0 ** -23) == 1.0 + 2.0 ** -23
