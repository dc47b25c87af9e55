"""Seeded synthetic inputs for one packed tick (shared by the tests, the bench
and the oracle's checks).

This module draws inputs only: sequence lengths, page tables built from a
shuffled free list, positions, and N(0, 1) values laid into the pages. It holds
none of the method's arithmetic: no RoPE, no slot mapping of the tick's new
tokens, no attention. bf16 values are produced by torch's float32 -> bfloat16
conversion (round to nearest even) and handed out as raw uint16 bits.

Workload shapes follow the models the pages serve: TinyLlama-1.1B (32 query / 4
KV heads, head_dim 64, 16-token pages; llm-serving-engine README, rows "GQA" and
"KV cache memory layout") and Qwen3-4B (32 query / 8 KV heads, head_dim 128,
256-token pages; Helios blog, "Paged attention").
"""

from dataclasses import dataclass, field
import math

import numpy as np
import torch

F32 = "f32"
BF16 = "bf16"
BF16_NAN_BITS = np.uint16(0x7FC0)


def to_storage(x, dtype):
    """float32 array -> stored representation (float32, or bf16 bits via torch RNE)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F32:
        return x
    t = torch.from_numpy(x).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def nan_fill(shape, dtype):
    if dtype == F32:
        return np.full(shape, np.nan, dtype=np.float32)
    return np.full(shape, BF16_NAN_BITS, dtype=np.uint16)


@dataclass
class Tick:
    """One packed continuous-batching tick of one attention layer.

    Rows of sequence s are ``q[qsl[s]:qsl[s+1]]``; it has ``seq_lens[s]`` keys
    once this tick's tokens are stored (``new_in_pool`` False: the tick's own
    K/V in ``k``/``v`` still have to be written; True: they are already in the
    pool and ``k``/``v`` are None).
    """
    name: str
    dtype: str
    Hq: int
    Hkv: int
    D: int
    P: int
    num_pages: int
    theta: object            # float or None (no RoPE)
    scale: float
    seq_lens: np.ndarray     # int32 [S]
    query_lens: np.ndarray   # int32 [S]
    qsl: np.ndarray          # int32 [S+1]
    positions: np.ndarray    # int32 [T]
    block_tables: np.ndarray  # int32 [S, max_blocks], unused entries -1
    k_pool: np.ndarray       # [num_pages, P, Hkv, D] storage
    v_pool: np.ndarray
    q: np.ndarray            # [T, Hq, D] storage
    k: object                # [T, Hkv, D] storage or None
    v: object
    new_in_pool: bool = False
    shared_pages: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    seed: int = 0

    @property
    def S(self):
        return int(self.seq_lens.shape[0])

    @property
    def T(self):
        return int(self.qsl[-1])

    @property
    def max_blocks(self):
        return int(self.block_tables.shape[1])

    @property
    def max_query_len(self):
        return int(self.query_lens.max()) if self.S else 0

    @property
    def max_seq_len(self):
        return int(self.seq_lens.max()) if self.S else 0

    @property
    def max_pos(self):
        """Rows a RoPE table needs: one past the largest position."""
        return max(self.max_seq_len, 1)


def build_tick(rng, *, name, dtype, Hq, Hkv, D, P, seq_lens, query_lens, theta,
               pool_pages=None, pool_factor=1.25, shared_prefix_pages=0,
               shared_prefix_seqs=(), poison=True, new_in_pool=False, max_blocks=None,
               seed=0):
    """Draw a tick.

    * Pages come from a free list shuffled with ``rng``; pages of a shared prefix
      are taken first and put at the start of every sharing sequence's table.
    * Keys already cached (positions below ``seq_len - query_len``, or all of them
      when ``new_in_pool``) are N(0, 1); every other slot of the pool is NaN when
      ``poison`` (so a read of it shows up), else N(0, 1) too.
    * New Q/K/V rows are N(0, 1).
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    query_lens = np.asarray(query_lens, dtype=np.int32)
    S = int(seq_lens.shape[0])
    if np.any(query_lens > seq_lens):
        raise ValueError("query_len must not exceed seq_len")
    blocks = [(int(n) + P - 1) // P for n in seq_lens]
    shared = set(int(s) for s in shared_prefix_seqs)
    needed = shared_prefix_pages if shared else 0
    for s in range(S):
        needed += blocks[s] - (shared_prefix_pages if s in shared else 0)
    num_pages = int(pool_pages) if pool_pages is not None else int(math.ceil(pool_factor * needed))
    if num_pages < needed:
        raise ValueError("pool too small")
    free = list(rng.permutation(num_pages).astype(np.int32))
    mb = max_blocks if max_blocks is not None else max(blocks + [1])
    bt = np.full((S, mb), -1, dtype=np.int32)
    prefix = [free.pop() for _ in range(shared_prefix_pages)] if shared else []
    for s in range(S):
        own = list(prefix) if s in shared else []
        while len(own) < blocks[s]:
            own.append(free.pop())
        bt[s, : blocks[s]] = own

    qsl = np.zeros(S + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(query_lens)
    T = int(qsl[-1])
    positions = np.empty(T, dtype=np.int32)
    for s in range(S):
        L, n = int(query_lens[s]), int(seq_lens[s])
        positions[qsl[s]: qsl[s + 1]] = np.arange(n - L, n, dtype=np.int32)

    shape = (num_pages, P, Hkv, D)
    if poison:
        k_pool = nan_fill(shape, dtype)
        v_pool = nan_fill(shape, dtype)
    else:
        k_pool = to_storage(rng.standard_normal(shape, dtype=np.float32), dtype)
        v_pool = to_storage(rng.standard_normal(shape, dtype=np.float32), dtype)

    def fill(pool, s, first, count):
        """Write ``count`` cached rows starting at logical row ``first`` of
        sequence s, one page at a time."""
        vals = to_storage(rng.standard_normal((count, Hkv, D), dtype=np.float32), dtype)
        done = 0
        while done < count:
            j = first + done
            page = int(bt[s, j // P])
            row = j % P
            take = min(P - row, count - done)
            pool[page, row: row + take] = vals[done: done + take]
            done += take

    prefix_tokens = shared_prefix_pages * P
    prefix_done = False
    for s in range(S):
        L, n = int(query_lens[s]), int(seq_lens[s])
        cached = n if new_in_pool else n - L
        first = 0
        if s in shared:
            if cached < prefix_tokens:
                raise ValueError("a shared prefix must be fully cached")
            if not prefix_done:
                fill(k_pool, s, 0, prefix_tokens)
                fill(v_pool, s, 0, prefix_tokens)
                prefix_done = True
            first = prefix_tokens
        if cached > first:
            fill(k_pool, s, first, cached - first)
            fill(v_pool, s, first, cached - first)

    q = to_storage(rng.standard_normal((T, Hq, D), dtype=np.float32), dtype)
    if new_in_pool:
        k = v = None
    else:
        k = to_storage(rng.standard_normal((T, Hkv, D), dtype=np.float32), dtype)
        v = to_storage(rng.standard_normal((T, Hkv, D), dtype=np.float32), dtype)
    shared_pages = np.asarray(prefix, dtype=np.int32)
    return Tick(name=name, dtype=dtype, Hq=Hq, Hkv=Hkv, D=D, P=P, num_pages=num_pages,
                theta=theta, scale=1.0 / math.sqrt(D), seq_lens=seq_lens,
                query_lens=query_lens, qsl=qsl, positions=positions, block_tables=bt,
                k_pool=k_pool, v_pool=v_pool, q=q, k=k, v=v, new_in_pool=new_in_pool,
                shared_pages=shared_pages, seed=seed)


CONFIG_NAMES = {
    1: "tiny-decode-fp32",
    2: "tinyllama-decode-bf16",
    3: "qwen3-4b-decode-bf16",
    4: "qwen3-4b-packed-mixed-bf16",
    5: "qwen3-4b-prefix-shared-longctx-bf16",
}


def make_config(cfg, poison=True, seed=None):
    """The five seeded workloads (seed ``1000 + cfg`` unless given).

    1. fp32 decode, contexts {5, 17, 33, 64}, 4/2 heads, D 16, 16-token pages,
       32-page pool, attention only (the tick's K/V are already stored).
    2. bf16 TinyLlama decode: 8 sequences, contexts U[32, 512], 32/4 heads,
       D 64, 16-token pages, RoPE theta 1e4.
    3. bf16 Qwen3-4B decode: 64 sequences, contexts U[256, 4096], 32/8 heads,
       D 128, 256-token pages, RoPE theta 1e6.
    4. bf16 Qwen3-4B packed mixed tick: 48 decode rows (contexts U[256, 4096])
       then chunks of 512, 512 and 1024 tokens, each after k in {0..3} cached
       256-token pages.
    5. bf16 Qwen3-4B prefix-shared long-context decode: 32 sequences of
       2048 + U[64, 1024] keys whose first 8 pages are one shared prefix, plus
       4 sequences of 32768 keys.
    """
    seed = 1000 + cfg if seed is None else seed
    rng = np.random.default_rng(seed)
    name = CONFIG_NAMES[cfg]
    if cfg == 1:
        return build_tick(rng, name=name, dtype=F32, Hq=4, Hkv=2, D=16, P=16,
                          seq_lens=[5, 17, 33, 64], query_lens=[1, 1, 1, 1], theta=None,
                          pool_pages=32, max_blocks=4, poison=poison, new_in_pool=True,
                          seed=seed)
    if cfg == 2:
        n = rng.integers(32, 512, size=8, endpoint=True)
        return build_tick(rng, name=name, dtype=BF16, Hq=32, Hkv=4, D=64, P=16,
                          seq_lens=n, query_lens=np.ones(8, np.int32), theta=1e4,
                          poison=poison, seed=seed)
    if cfg == 3:
        n = rng.integers(256, 4096, size=64, endpoint=True)
        return build_tick(rng, name=name, dtype=BF16, Hq=32, Hkv=8, D=128, P=256,
                          seq_lens=n, query_lens=np.ones(64, np.int32), theta=1e6,
                          poison=poison, max_blocks=16, seed=seed)
    if cfg == 4:
        dec = rng.integers(256, 4096, size=48, endpoint=True)
        chunk_L = np.array([512, 512, 1024])
        prior = rng.integers(0, 3, size=3, endpoint=True)
        n = np.concatenate([dec, 256 * prior + chunk_L])
        L = np.concatenate([np.ones(48, np.int64), chunk_L])
        return build_tick(rng, name=name, dtype=BF16, Hq=32, Hkv=8, D=128, P=256,
                          seq_lens=n, query_lens=L, theta=1e6, poison=poison,
                          max_blocks=16, seed=seed)
    if cfg == 5:
        suffix = rng.integers(64, 1024, size=32, endpoint=True)
        n = np.concatenate([2048 + suffix, np.full(4, 32768)])
        return build_tick(rng, name=name, dtype=BF16, Hq=32, Hkv=8, D=128, P=256,
                          seq_lens=n, query_lens=np.ones(36, np.int32), theta=1e6,
                          shared_prefix_pages=8, shared_prefix_seqs=range(32),
                          poison=poison, max_blocks=128, seed=seed)
    raise ValueError(f"unknown config {cfg}")


def permute_pages(tick, rng):
    """Relabel physical pages: the same tick with every page moved to a new id
    and every page table rewritten to match (inputs only, no arithmetic)."""
    perm = rng.permutation(tick.num_pages).astype(np.int32)   # old id -> new id
    k_pool = np.empty_like(tick.k_pool)
    v_pool = np.empty_like(tick.v_pool)
    k_pool[perm] = tick.k_pool
    v_pool[perm] = tick.v_pool
    bt = np.where(tick.block_tables >= 0, perm[np.maximum(tick.block_tables, 0)], -1)
    out = Tick(**{**tick.__dict__})
    out.k_pool, out.v_pool, out.block_tables = k_pool, v_pool, bt.astype(np.int32)
    out.shared_pages = perm[tick.shared_pages] if tick.shared_pages.size else tick.shared_pages
    return out
