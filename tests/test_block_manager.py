"""The paged block manager, host only.

* The oracle (``oracle/blocks.py``) is pinned to things other than itself:
  the published FNV-1a test vectors, hand-worked scenarios of what the pages
  state (shared prefixes share physical pages, a partial block is never
  cached, leaf-first eviction, the reservation keeps decode going, a page is
  freed on its last release), and, after every step of seeded random traces,
  invariants checked by brute force over its whole state (reference counts
  equal the holders, the free list holds exactly the unheld pages, only
  cached complete blocks with the right tokens are shared, the restored chain
  is the longest cached prefix).
* The library (``pa_bm_*`` in libpa.so) equals the oracle step by step on the
  same traces: every return value, error, block table, count and reference
  count.
* Planted mistakes in the oracle (a FIFO free list, restoring the last
  token's block, most-recently-used or parent-first eviction, restored pages
  left unreferenced, partial blocks published) are each caught by a pin that
  involves the oracle alone.
"""

import random

import pytest

import paged_kv_cache_page_amd as pa
from oracle import blocks as ob


# ----------------------------------------------------------------- adapters
class Lib:
    """pa.BlockManager with the oracle's exceptions (NoPages, ValueError)."""

    def __init__(self, n, p):
        self.m = pa.BlockManager(n, p)
        self.N, self.P = n, p

    def _call(self, fn, *a):
        try:
            return fn(*a)
        except pa.PaError as e:
            if e.status == pa.PA_ERR_NO_PAGES:
                raise ob.NoPages() from None
            raise ValueError(str(e)) from None

    def admit(self, req, prompt, max_new):
        return self._call(self.m.admit, req, prompt, max_new)

    def append(self, req, n):
        return self._call(self.m.append, req, n)

    def finish(self, req, publish=True):
        return self._call(self.m.finish, req, publish)

    def evict(self, pages):
        return self._call(self.m.evict, pages)

    def block_table(self, req):
        return [int(x) for x in self._call(self.m.block_table, req)]

    def stats(self):
        return self.m.stats()

    def refcount(self, page):
        return self._call(self.m.refcount, page)


class Ora:
    """The oracle with unknown requests reported as ValueError."""

    def __init__(self, n, p):
        self.m = ob.BlockManager(n, p)
        self.N, self.P = n, p

    def _call(self, fn, *a):
        try:
            return fn(*a)
        except KeyError:
            raise ValueError("unknown request") from None

    def admit(self, req, prompt, max_new):
        return self.m.admit(req, prompt, max_new)

    def append(self, req, n):
        return self._call(self.m.append, req, n)

    def finish(self, req, publish=True):
        return self._call(self.m.finish, req, publish)

    def evict(self, pages):
        return self.m.evict(pages)

    def block_table(self, req):
        return self._call(self.m.block_table, req)

    def stats(self):
        return self.m.stats()

    def refcount(self, page):
        if not 0 <= page < self.N:
            raise ValueError("page out of range")
        return self.m.refcount[page]


IMPLS = [pytest.param(Ora, id="oracle"), pytest.param(Lib, id="library")]


# ------------------------------------------------------- pins of the oracle
def test_fnv1a_published_vectors():
    # FNV-1a 64-bit test vectors published with the algorithm (Fowler, Noll, Vo)
    assert ob.fnv1a(b"") == 0xCBF29CE484222325
    assert ob.fnv1a(b"a") == 0xAF63DC4C8601EC8C
    assert ob.fnv1a(b"foobar") == 0x85944171F73967E8


def test_block_hash_is_chained():
    a, b = [1, 2, 3, 4], [5, 6, 7, 8]
    h1 = ob.block_hash(0, a)
    assert ob.block_hash(h1, b) != ob.block_hash(0, b)      # the parent enters the hash
    assert ob.block_hash(0, a) != ob.block_hash(0, [2, 1, 3, 4])  # token order matters
    # byte layout: parent as 8 little-endian bytes, then 4 bytes per token
    raw = (0).to_bytes(8, "little") + b"".join(t.to_bytes(4, "little") for t in a)
    assert h1 == ob.fnv1a(raw)


def check_oracle_state(m):
    """Brute-force invariants over the whole oracle state."""
    N, P = m.N, m.P
    holders = [0] * N
    for r in m.reqs.values():
        assert len(r["pages"]) == -(-r["tokens"] // P)           # a table covers its tokens
        assert len(r["pages"]) <= r["reserve"]
        assert len(set(r["pages"])) == len(r["pages"])
        for p in r["pages"]:
            holders[p] += 1
    entry_pages = {}
    for h, e in m.cache.items():
        assert e["page"] not in entry_pages                       # one page per cached block
        entry_pages[e["page"]] = h
        holders[e["page"]] += 1
        assert h == ob.block_hash(e["parent"], e["tokens"]) and len(e["tokens"]) == P
        assert e["parent"] == 0 or e["parent"] in m.cache         # a chain has no gaps
        assert e["children"] == sum(1 for f in m.cache.values() if f["parent"] == h)
    assert m.refcount == holders                                  # refcount conservation
    assert sorted(m.free) == [p for p in range(N) if holders[p] == 0]
    assert len(set(m.free)) == len(m.free)
    assert m.reserved == sum(r["reserve"] - len(r["pages"]) for r in m.reqs.values())
    assert m.available() >= 0                                     # reservations stay backed
    # a page held by two requests is a cached complete block, and each holder's
    # prompt up to and including that block is the block's whole cached prefix
    prefix = {h: cached_prefix(m, h) for h in m.cache}
    for r in m.reqs.values():
        for b, p in enumerate(r["pages"]):
            if holders[p] > 1 and p in entry_pages:
                assert tuple(r["prompt"][:(b + 1) * P]) == prefix[entry_pages[p]]
    for p in range(N):
        if sum(p in r["pages"] for r in m.reqs.values()) > 1:
            assert p in entry_pages


def cached_prefix(m, h):
    toks = []
    while h:
        e = m.cache[h]
        toks = e["tokens"] + toks
        h = e["parent"]
    return tuple(toks)


def longest_cached_prefix(m, prompt):
    """Brute force: the most prompt tokens, a whole number of pages before the
    last prompt token, whose token sequence some cached chain spells."""
    spelled = {cached_prefix(m, h) for h in m.cache}
    best = 0
    for k in range(1, (len(prompt) - 1) // m.P + 1):
        if tuple(prompt[:k * m.P]) in spelled:
            best = k * m.P
    return best


# --------------------------------------------------- hand-worked scenarios
@pytest.mark.parametrize("impl", IMPLS)
def test_shared_prefix_shares_physical_pages(impl):
    m = impl(16, 4)
    a = list(range(1, 11))                       # 10 tokens: blocks [1..4] [5..8], partial [9, 10]
    assert m.admit(1, a, 2) == 0         # 12 tokens -> 3 pages reserved
    assert m.stats() == (16, 3, 0)
    m.append(1, 10)
    assert m.block_table(1) == [0, 1, 2]         # page 0 is handed out first
    m.finish(1)
    assert m.stats() == (14, 0, 2)               # blocks 0 and 1 cached, the partial block freed
    assert [m.refcount(p) for p in range(3)] == [1, 1, 0]
    b = list(range(1, 9)) + [20, 21, 22]
    assert m.admit(2, b, 1) == 8                 # both complete blocks restored
    assert m.block_table(2) == [0, 1]
    assert [m.refcount(p) for p in range(2)] == [2, 2]
    m.append(2, 3)
    assert m.block_table(2) == [0, 1, 2]         # the freed page is on top of the stack
    c = list(range(1, 5)) + [9, 9, 9, 9, 9]
    assert m.admit(3, c, 0) == 4                 # the chain stops at the first differing block
    assert m.block_table(3) == [0]
    assert m.refcount(0) == 3


@pytest.mark.parametrize("impl", IMPLS)
def test_partial_and_last_blocks(impl):
    m = impl(16, 4)
    m.admit(1, [7] * 6, 0)
    m.append(1, 6)
    m.finish(1)
    assert m.stats()[2] == 1                     # only the complete block, never the partial one
    assert m.admit(2, [7] * 6, 0) == 4
    # a prompt of exactly the cached blocks restores all but the block of its last token
    m.admit(3, [7] * 4, 4)
    m.append(3, 8)
    m.finish(3)
    m.finish(2)
    assert m.admit(4, [7] * 4, 0) == 0
    assert m.admit(5, [7] * 5, 0) == 4
    # an unpublished request caches nothing
    m2 = impl(8, 4)
    m2.admit(1, [3] * 8, 0)
    m2.append(1, 8)
    m2.finish(1, publish=False)
    assert m2.stats() == (8, 0, 0)


@pytest.mark.parametrize("impl", IMPLS)
def test_only_written_prompt_blocks_are_published(impl):
    m = impl(8, 4)
    m.admit(1, list(range(12)), 0)
    m.append(1, 5)                               # one complete block written, the rest not
    m.finish(1)
    assert m.stats()[2] == 1
    assert m.admit(2, list(range(12)), 0) == 4


@pytest.mark.parametrize("impl", IMPLS)
def test_leaf_first_lru_eviction(impl):
    m = impl(8, 2)
    m.admit(1, [1, 2, 3, 4, 9], 0)               # chain x: [1,2] -> [3,4]
    m.append(1, 5)
    m.finish(1)                                  # pages 0, 1 cached (page 2 freed)
    m.admit(2, [5, 6, 9], 0)                     # chain y: [5,6]
    m.append(2, 3)
    assert m.block_table(2) == [2, 3]
    m.finish(2)                                  # page 2 cached, page 3 freed
    assert m.stats() == (5, 0, 3)
    # leaves are [3,4] (older) and [5,6]; [1,2] is a parent and stays
    assert m.evict(1) == 1
    assert [m.refcount(p) for p in range(3)] == [1, 0, 1]
    # now [1,2] is an unused leaf older than [5,6]
    assert m.evict(1) == 1
    assert [m.refcount(p) for p in range(3)] == [0, 0, 1]
    assert m.evict(5) == 1 and m.stats() == (8, 0, 0)


@pytest.mark.parametrize("impl", IMPLS)
def test_eviction_never_takes_a_held_block_and_restores_refresh_lru(impl):
    m = impl(8, 2)
    for req, prompt in ((1, [1, 2, 9]), (2, [3, 4, 9]), (3, [5, 6, 9])):
        m.admit(req, prompt, 0)
        m.append(req, 3)
        m.finish(req)
    assert m.stats()[2] == 3                     # pages 0, 1, 2 cached in that order
    assert m.admit(4, [1, 2, 7], 0) == 2         # restores [1,2]: held and most recently used
    assert m.evict(1) == 1 and m.refcount(1) == 0   # [3,4] is now the least recently used
    assert m.evict(8) == 1 and m.refcount(2) == 0   # [5,6]; [1,2] is held by request 4
    assert m.refcount(0) == 2 and m.stats()[2] == 1


@pytest.mark.parametrize("impl", IMPLS)
def test_reservation_keeps_decode_going(impl):
    m = impl(4, 4)
    m.admit(1, [1, 2, 3, 4], 8)                  # 12 tokens: 3 pages reserved
    with pytest.raises(ob.NoPages):
        m.admit(2, [5, 6, 7, 8], 4)              # 2 pages wanted, 1 left unreserved
    assert m.stats() == (4, 3, 0)
    m.admit(3, [5], 3)                           # 1 page fits
    for _ in range(12):
        m.append(1, 1)                           # every decode token finds its page
    assert len(m.block_table(1)) == 3
    with pytest.raises(ValueError):
        m.append(1, 1)                           # past the admitted maximum
    with pytest.raises(ob.NoPages):
        m.admit(4, [1], 16)                      # more pages than the pool has


@pytest.mark.parametrize("impl", IMPLS)
def test_failed_admission_evicts_but_keeps_its_restored_blocks(impl):
    m = impl(4, 2)
    m.admit(1, [1, 2, 3, 4, 5], 0)
    m.append(1, 5)
    m.finish(1)                                  # [1,2] -> [3,4] cached on pages 0, 1
    m.admit(2, [8], 3)                           # 2 pages reserved; 2 free, 0 unreserved
    with pytest.raises(ob.NoPages):
        m.admit(3, [1, 2, 3, 4, 5, 6, 7], 2)     # restores 2 blocks, wants 3 more pages
    # its restored blocks were held during eviction, so nothing was evictable
    assert m.stats() == (2, 2, 2)
    assert [m.refcount(p) for p in range(4)] == [1, 1, 0, 0]
    with pytest.raises(ob.NoPages):
        m.admit(4, [9] * 5, 0)                   # wants 3 pages: evicts both cached blocks, still short
    assert m.stats() == (4, 2, 0)


@pytest.mark.parametrize("impl", IMPLS)
def test_release_on_last_reference(impl):
    m = impl(4, 2)
    m.admit(1, [1, 2, 3], 0)
    m.append(1, 3)
    m.finish(1)
    m.admit(2, [1, 2, 5], 0)
    m.admit(3, [1, 2, 6], 0)
    assert m.refcount(0) == 3
    m.evict(4)                                   # held: not evicted
    assert m.refcount(0) == 3
    m.finish(2, publish=False)
    m.finish(3, publish=False)
    assert m.refcount(0) == 1                    # the cache is the last holder
    assert m.evict(1) == 1 and m.refcount(0) == 0 and m.stats() == (4, 0, 0)


@pytest.mark.parametrize("impl", IMPLS)
def test_bad_calls(impl):
    m = impl(4, 4)
    m.admit(1, [1, 2], 2)
    with pytest.raises(ValueError):
        m.admit(1, [1], 0)                       # already admitted
    with pytest.raises(ValueError):
        m.admit(2, [], 0)                        # empty prompt
    with pytest.raises(ValueError):
        m.append(9, 1)
    with pytest.raises(ValueError):
        m.finish(9)
    with pytest.raises(ValueError):
        m.block_table(9)
    with pytest.raises(ValueError):
        m.refcount(4)
    assert m.stats() == (4, 1, 0)


def test_library_argument_checks():
    with pytest.raises(pa.PaError):
        pa.BlockManager(0, 4)
    with pytest.raises(pa.PaError):
        pa.BlockManager(4, 0)
    m = pa.BlockManager(8, 2)
    m.admit(1, [1, 2, 3], 3)
    m.append(1, 6)
    import ctypes
    import numpy as np
    out = np.zeros(2, dtype=np.int32)
    n = ctypes.c_int32(0)
    st = pa.lib().pa_bm_block_table(m._h, 1, out.ctypes.data_as(ctypes.c_void_p), 2,
                                    ctypes.byref(n))
    assert st == 1                               # a table of 3 pages does not fit 2 entries
    assert pa.lib().pa_bm_evict(m._h, -1, ctypes.byref(n)) == 1
    assert pa.lib().pa_bm_admit(m._h, 2, None, 1, 0, ctypes.byref(n)) == 1
    m.close()


# ------------------------------------------------------- seeded random traces
def run_trace(seed, N, P, steps, with_lib=True):
    rng = random.Random(seed)
    docs = [[rng.randrange(1, 50) for _ in range(6 * P)] for _ in range(3)]
    ora = Ora(N, P)
    lib = Lib(N, P) if with_lib else Ora(N, P)
    live, next_id = [], 0
    for _ in range(steps):
        op = rng.random()
        if op < 0.35 or not live:
            d = rng.choice(docs)
            prompt = d[:rng.randrange(0, len(d) + 1)] + [rng.randrange(1, 50)
                                                        for _ in range(rng.randrange(0, 2 * P))]
            if not prompt:
                prompt = [rng.randrange(1, 50)]
            max_new = rng.randrange(0, 3 * P)
            expect = longest_cached_prefix(ora.m, prompt)
            res = []
            for m in (ora, lib):
                try:
                    res.append(m.admit(next_id, prompt, max_new))
                except ob.NoPages:
                    res.append("no pages")
            assert res[0] == res[1], (seed, res)
            if res[0] != "no pages":
                assert res[0] == expect                  # longest-chain restore
                live.append(next_id)
            next_id += 1
        elif op < 0.75:
            req = rng.choice(live)
            r = ora.m.reqs[req]
            room = r["reserve"] * P - r["tokens"]
            if r["tokens"] < len(r["prompt"]):
                n = len(r["prompt"]) - r["tokens"]       # the prefill of the uncached rest
                if rng.random() < 0.3:
                    n = rng.randrange(0, n + 1)          # a prefill chunk
            else:
                n = rng.randrange(0, min(room, P) + 1)   # decode tokens
            if rng.random() < 0.05:
                n = room + 1                             # past the maximum: refused by both
            res = []
            for m in (ora, lib):
                try:
                    m.append(req, n)
                    res.append("ok")
                except ValueError:
                    res.append("refused")
            assert res[0] == res[1] == ("refused" if n > room else "ok")
        elif op < 0.93:
            req = live.pop(rng.randrange(len(live)))
            publish = rng.random() < 0.8
            ora.finish(req, publish)
            lib.finish(req, publish)
        else:
            k = rng.randrange(0, 4)
            assert ora.evict(k) == lib.evict(k)
        check_oracle_state(ora.m)
        assert ora.stats() == lib.stats()
        for req in live:
            assert ora.block_table(req) == lib.block_table(req)
        assert [ora.refcount(p) for p in range(N)] == [lib.refcount(p) for p in range(N)]
    return ora


@pytest.mark.parametrize("seed,N,P", [(0, 8, 1), (1, 12, 2), (2, 24, 4), (3, 64, 4),
                                      (4, 40, 8), (5, 16, 16), (6, 200, 4), (7, 6, 3)])
def test_library_equals_oracle_on_random_traces(seed, N, P):
    ora = run_trace(seed, N, P, 300)
    # the traces exercise restores, evictions and refusals
    assert ora.m.next_seq > 0



# ------------------------------------------- planted mistakes must be caught
def _oracle_pins():
    """The pins that involve the oracle alone (no library)."""
    return [lambda: test_shared_prefix_shares_physical_pages(Ora),
            lambda: test_partial_and_last_blocks(Ora),
            lambda: test_only_written_prompt_blocks_are_published(Ora),
            lambda: test_leaf_first_lru_eviction(Ora),
            lambda: test_eviction_never_takes_a_held_block_and_restores_refresh_lru(Ora),
            lambda: test_reservation_keeps_decode_going(Ora),
            lambda: test_failed_admission_evicts_but_keeps_its_restored_blocks(Ora),
            lambda: test_release_on_last_reference(Ora),
            lambda: run_trace(2, 24, 4, 200, with_lib=False),
            lambda: run_trace(7, 6, 3, 200, with_lib=False)]


def _caught():
    for pin in _oracle_pins():
        try:
            pin()
        except (AssertionError, ValueError, KeyError, IndexError, ob.NoPages):
            return True
    return False


def _fifo_take(self):
    p = self.free.pop(0)
    self.refcount[p] = 1
    return p


def _match_includes_last_token(self, prompt):
    pages, hashes, key = [], [], 0
    for b in range(len(prompt) // self.P):
        blk = list(prompt[b * self.P:(b + 1) * self.P])
        h = ob.block_hash(key, blk)
        e = self.cache.get(h)
        if e is None or e["parent"] != key or e["tokens"] != blk:
            break
        pages.append(e["page"])
        hashes.append(h)
        key = h
    return pages, hashes


def _evict_most_recent(self):
    cands = [(-e["last_use"], -e["seq"], h) for h, e in self.cache.items()
             if e["children"] == 0 and self.refcount[e["page"]] == 1]
    if not cands:
        return False
    h = min(cands)[2]
    e = self.cache.pop(h)
    if e["parent"] in self.cache:
        self.cache[e["parent"]]["children"] -= 1
    self._drop(e["page"])
    return True


def _evict_ignoring_children(self):
    cands = [(e["last_use"], e["seq"], h) for h, e in self.cache.items()
             if self.refcount[e["page"]] == 1]
    if not cands:
        return False
    h = min(cands)[2]
    e = self.cache.pop(h)
    self._drop(e["page"])
    return True


_orig_admit = ob.BlockManager.admit


def _admit_without_restore_refs(self, req, prompt, max_new_tokens):
    n = _orig_admit(self, req, prompt, max_new_tokens)
    for p in self.reqs[req]["pages"]:
        self.refcount[p] -= 1          # restored pages left unreferenced
    return n


def _publish_partial_blocks(self, req, publish=True):
    r = self.reqs[req]
    r["prompt"] = r["prompt"] + [0] * (-len(r["prompt"]) % self.P)   # the partial block, padded
    r["tokens"] += -r["tokens"] % self.P                             # counted as written
    return _orig_finish(self, req, publish)


_orig_finish = ob.BlockManager.finish


@pytest.mark.parametrize("name,fn", [
    ("_take", _fifo_take), ("_match", _match_includes_last_token),
    ("_evict_one", _evict_most_recent), ("_evict_one", _evict_ignoring_children),
    ("admit", _admit_without_restore_refs), ("finish", _publish_partial_blocks)])
def test_planted_mistakes_are_caught(monkeypatch, name, fn):
    monkeypatch.setattr(ob.BlockManager, name, fn)
    assert _caught(), f"a mistake in {name} ({fn.__name__}) passes every oracle pin"
