"""Reference token sampling over a tick's logits rows (test infrastructure only).

What the pages state: the sampler offers greedy, temperature, top-k and top-p
sampling (llm-serving-engine README, component table row "Token sampling");
temperature runs from 0 to 2 and top-p lies in (0, 1] (Helios README, the
request fields); greedy rows are sampled together, and so are rows that share
one temperature and top-p (Helios blog, "Continuous batching"), and batched
sampling must equal sampling each row on its own (mini-vLLM page, "Test
suites").

Readings where the pages leave a choice (the same in the library):

* ``temperature <= 0`` (and ``top_k == 1``) is greedy: the largest logit, the
  lowest index among equal ones.
* Tokens are ranked by logit, larger first, equal logits by index, lower
  first (``-0.0`` ranks with ``+0.0``). Top-k keeps the first k of this
  ranking (``k <= 0`` or ``k >= V``: all). Top-p then keeps the shortest
  leading part of what top-k kept whose probability reaches p (``p >= 1``:
  all of it; ``p <= 0``: the first token).
* Probabilities are ``exp((logit - max) / temperature)``, in float64, held as
  integers: ``floor(w * 2**32)``, so the most probable token weighs exactly
  ``2**32``. Every sum, the top-p target ``ceil(p * S)`` and the sampling
  target ``floor(u * S)`` are then exact (S < 2**53 for V <= 2**21), and the
  only rounding is the float64 exp of each logit. A token whose probability
  is below 2**-32 of the top token's is never drawn.
* The random number is the caller's: one uniform ``u`` in [0, 1) per row. The
  token drawn is the first, in index order, among the kept tokens, at which
  the running weight passes ``floor(u * S)``, S the kept tokens' total weight
  (inverse transform sampling; any fixed order samples the same distribution,
  and index order needs no sort).
"""

import math

import numpy as np

TWO32 = 2.0 ** 32


def ranking(x):
    """Token indices by logit, larger first, ties by lower index."""
    x = np.asarray(x, dtype=np.float64) + 0.0          # -0.0 -> +0.0
    return np.lexsort((np.arange(x.size), -x))


def weights(x, temperature):
    """Integer weights floor(exp((x - max) / T) * 2**32), float64 arithmetic."""
    x = np.asarray(x, dtype=np.float64)
    m = x[ranking(x)[0]]
    w = np.exp((x - m) / np.float64(temperature))
    return np.floor(w * TWO32).astype(np.uint64)


def kept_tokens(x, temperature, top_k, top_p):
    """Indices kept by top-k then top-p, in ranking order."""
    order = ranking(x)
    V = order.size
    if 0 < top_k < V:
        order = order[:top_k]
    if top_p < 1.0:
        w = weights(x, temperature)[order]
        need = max(math.ceil(float(np.float64(np.float32(top_p)) * float(int(w.sum())))), 1)
        cum = np.cumsum(w.astype(object))
        t = next(i for i, c in enumerate(cum) if c >= need)
        order = order[:t + 1]
    return order


def sample_row(x, temperature, top_k, top_p, u):
    """One row: the sampled token index."""
    x = np.asarray(x, dtype=np.float32)
    order = ranking(x)
    if not temperature > 0 or top_k == 1:
        return int(order[0])
    keep = np.zeros(x.size, dtype=bool)
    keep[kept_tokens(x, temperature, top_k, top_p)] = True
    w = np.where(keep, weights(x, temperature), np.uint64(0))
    S = int(w.sum())
    target = min(int(math.floor(float(np.float32(u)) * float(S))), S - 1)
    run = 0
    for i in np.flatnonzero(w):
        run += int(w[i])
        if run > target:
            return int(i)
    raise AssertionError("unreachable: the kept weights sum to S > target")


def sample_rows(logits, temperature, top_k, top_p, uniforms):
    """Every row of ``logits`` [R, V] with its own settings; int32 [R]."""
    logits = np.asarray(logits, dtype=np.float32)
    return np.array([sample_row(logits[r], float(temperature[r]), int(top_k[r]),
                                float(top_p[r]), float(uniforms[r]))
                     for r in range(logits.shape[0])], dtype=np.int32)
