"""Rotary position embedding for the new Q and K of a tick (test infrastructure only).

The pages apply RoPE to Q and K after projection and before attention (Helios
blog, "torch.sdpa and Flash Attention") and build it from cached sin/cos tables
(llm-serving-engine README, component table row "RoPE from scratch"). They give
no formula, so the oracle takes the plainest reading that fits the
Hugging Face Llama/Qwen3 weights those engines load:

* pairs are (i, i + D/2) for i in [0, D/2) (the "rotate half" split);
* pair i turns by the angle ``p * theta**(-2 i / D)`` at absolute position p;
* no frequency scaling.

The cos/sin table is built in float64 and rounded once to float32; the
rotation itself runs in float32 with each product and each sum rounded on its
own (numpy float32 elementwise arithmetic never fuses a multiply into an add).
"""

import numpy as np


def rope_inv_freq(D, theta):
    """Inverse frequencies ``theta**(-2i/D)`` for i in [0, D/2), float64."""
    if D % 2:
        raise ValueError("head_dim must be even for RoPE")
    i = np.arange(D // 2, dtype=np.float64)
    return np.power(np.float64(theta), -(2.0 * i) / np.float64(D))


def rope_table(max_pos, D, theta):
    """cos/sin table, float32 ``[max_pos, D]``: columns [0, D/2) hold
    cos(p * inv_freq_i), columns [D/2, D) hold sin(p * inv_freq_i).

    The angle and both trigonometric values are float64; each entry is rounded
    to float32 once.
    """
    inv = rope_inv_freq(D, theta)
    pos = np.arange(max_pos, dtype=np.float64)
    ang = pos[:, None] * inv[None, :]
    table = np.empty((max_pos, D), dtype=np.float32)
    table[:, : D // 2] = np.cos(ang).astype(np.float32)
    table[:, D // 2 :] = np.sin(ang).astype(np.float32)
    return table


def rope_rotate(x, positions, table):
    """Rotate float32 ``x[T, H, D]`` of tokens at ``positions[T]``.

    ``y[i]      = x[i] * cos - x[i + D/2] * sin``
    ``y[i+D/2]  = x[i + D/2] * cos + x[i] * sin``
    all in float32, one rounding per product and per sum.
    """
    x = np.asarray(x, dtype=np.float32)
    T, H, D = x.shape
    half = D // 2
    positions = np.asarray(positions, dtype=np.int64)
    cos = table[positions, :half][:, None, :]   # [T, 1, D/2] float32
    sin = table[positions, half:][:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    a = x1 * cos          # float32 products, each rounded
    b = x2 * sin
    c = x2 * cos
    d = x1 * sin
    y = np.empty_like(x)
    y[..., :half] = a - b  # float32 difference, rounded
    y[..., half:] = c + d
    return y
