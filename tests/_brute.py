"""Brute-force scalar references for tiny inputs, used to pin the oracle.

Pure-Python loops over Python floats (float64), no numpy linear algebra and no
code shared with ``oracle/``: each quantity is computed from its definition one
term at a time, so a transposed operand, a wrong index or a dropped term in the
vectorised oracle shows up as a mismatch.
"""

import math
import struct


def f32(x):
    """Round a Python float to the nearest float32 (IEEE, ties to even)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def brute_attention(q, K, V, scale, group_of=None):
    """q: list[L][Hq][D]; K, V: list[n][Hkv][D] (floats). Row i sees keys 0..n-L+i.

    ``group_of(h, Hq, Hkv)`` picks the KV head of query head h (default:
    contiguous groups).
    """
    L, Hq, D = len(q), len(q[0]), len(q[0][0])
    n, Hkv = len(K), len(K[0])
    if group_of is None:
        group_of = lambda h, Hq, Hkv: h // (Hq // Hkv)
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(L)]
    for i in range(L):
        last = n - L + i
        for h in range(Hq):
            g = group_of(h, Hq, Hkv)
            scores = []
            for j in range(last + 1):
                acc = 0.0
                for d in range(D):
                    acc += q[i][h][d] * K[j][g][d]
                scores.append(acc * scale)
            top = max(scores)
            weights = [math.exp(s - top) for s in scores]
            total = math.fsum(weights)
            for d in range(D):
                out[i][h][d] = math.fsum(weights[j] * V[j][g][d] for j in range(last + 1)) / total
    return out


def brute_gather(pool, table_row, n, P):
    """``pool[page][row][head][d]`` nested lists -> the n rows of one sequence."""
    rows = []
    for j in range(n):
        page = table_row[j // P]
        rows.append(pool[page][j % P])
    return rows


def brute_rope_row(x, pos, theta):
    """Rotate one head vector (list of D floats) with float32 rounding after every
    operation, angles from float64 cos/sin rounded to float32."""
    D = len(x)
    half = D // 2
    y = [0.0] * D
    for i in range(half):
        inv = theta ** (-(2.0 * i) / D)
        c = f32(math.cos(pos * inv))
        s = f32(math.sin(pos * inv))
        x1, x2 = f32(x[i]), f32(x[i + half])
        y[i] = f32(f32(x1 * c) - f32(x2 * s))
        y[i + half] = f32(f32(x2 * c) + f32(x1 * s))
    return y
