"""Reference paged block manager (test infrastructure only).

What the pages state, and this module follows step by step:

* A fixed pool of P-token pages; new tokens take pages from the free page
  list, and any free page fits any request (Helios blog, "Paged attention";
  llm-serving-engine README, row "Physical Block Manager").
* Each request owns a page table of its pages (Helios blog, "Paged
  attention"). Admission reserves the request's maximum length, rounded up to
  whole pages, so that decode has space (Helios blog, "Paged attention";
  Helios README, "Paged attention").
* A page goes back to the pool when its last holder, a request or the prefix
  cache, releases it (Helios blog, "Paged attention"; Helios README, "Paged
  attention").
* Complete P-token prompt blocks are hashed in order, each together with the
  previous block's hash. An arriving request restores the longest matching
  chain of pages and prefills only the unmatched later blocks. Partial last
  blocks are not stored, and requests sharing a prefix share the same
  physical pages (Helios blog, "Prefix caching"; Helios README, "Loading").
* Eviction frees unused blocks first and prefers unused leaf blocks over the
  parents that later blocks still depend on (Helios blog, "Prefix caching";
  Helios README, "Loading"; llm-serving-engine README, row "Prefix / Prompt
  Caching": LRU leaf eviction with ref-counted pinning).

Readings where the pages leave a choice (the same in the library):

* The free list is a stack. Pages N-1 .. 0 are pushed at creation, so page 0 is
  handed out first; a released page is pushed on top.
* A block's hash is FNV-1a (64-bit, as published by Fowler, Noll and Vo) over
  its parent's hash (8 bytes, little-endian) followed by its tokens (4 bytes
  each, little-endian). The first block's parent hash is 0. A cache entry also
  keeps its tokens and parent hash, and a lookup matches only when both agree.
* A restored chain stops short of the last prompt token: only complete blocks
  before it are restored, so the caller always computes that token (its
  attention output gives the first new token).
* "Least recently used" runs on a logical clock that advances by one per
  admission and per finish. Ties go by insertion order. Only a finished
  request's fully written prompt blocks are published; a block already cached
  keeps its page and is marked used.
* Time-based expiry (the pages' sliding TTL) is left to the caller; eviction
  here happens only when pages are short or asked for.
"""

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


def fnv1a(data, h=FNV_OFFSET):
    """FNV-1a over a bytes object."""
    for b in data:
        h ^= b
        h = (h * FNV_PRIME) & MASK64
    return h


def block_hash(parent, tokens):
    """Chained hash of one complete block after the block of hash ``parent``."""
    data = int(parent).to_bytes(8, "little")
    for t in tokens:
        data += (int(t) & 0xFFFFFFFF).to_bytes(4, "little")
    return fnv1a(data)


class NoPages(Exception):
    """Not enough free pages for an admission's reservation."""


class BlockManager:
    def __init__(self, num_pages, page_size):
        assert num_pages >= 1 and page_size >= 1
        self.N, self.P = num_pages, page_size
        self.refcount = [0] * num_pages
        self.free = list(range(num_pages - 1, -1, -1))  # a stack: the last item goes first
        self.reserved = 0
        self.reqs = {}   # id -> dict(pages, prompt, tokens, reserve)
        self.cache = {}  # hash -> dict(page, parent, tokens, children, last_use, seq)
        self.clock = 0
        self.next_seq = 0

    # -- pages --------------------------------------------------------------
    def available(self):
        return len(self.free) - self.reserved

    def _take(self):
        p = self.free.pop()
        self.refcount[p] = 1
        return p

    def _drop(self, p):
        self.refcount[p] -= 1
        if self.refcount[p] == 0:
            self.free.append(p)

    # -- prefix cache -------------------------------------------------------
    def _evict_one(self):
        """Evict the least recently used cached block that no cached block
        depends on and that only the cache holds; False if there is none."""
        cands = [(e["last_use"], e["seq"], h) for h, e in self.cache.items()
                 if e["children"] == 0 and self.refcount[e["page"]] == 1]
        if not cands:
            return False
        _, _, h = min(cands)
        e = self.cache.pop(h)
        if e["parent"] != 0 and e["parent"] in self.cache:
            self.cache[e["parent"]]["children"] -= 1
        self._drop(e["page"])
        return True

    def _match(self, prompt):
        """Pages and hashes of the longest cached chain of complete prompt blocks."""
        pages, hashes, key = [], [], 0
        for b in range((len(prompt) - 1) // self.P):
            blk = list(prompt[b * self.P:(b + 1) * self.P])
            h = block_hash(key, blk)
            e = self.cache.get(h)
            if e is None or e["parent"] != key or e["tokens"] != blk:
                break
            pages.append(e["page"])
            hashes.append(h)
            key = h
        return pages, hashes

    # -- requests -----------------------------------------------------------
    def admit(self, req, prompt, max_new_tokens):
        prompt = [int(t) for t in prompt]
        if req in self.reqs or len(prompt) < 1 or max_new_tokens < 0:
            raise ValueError("bad admission")
        need = -(-(len(prompt) + max_new_tokens) // self.P)
        if need > self.N:
            raise NoPages()
        pages, hashes = self._match(prompt)
        for p in pages:  # held before any eviction, so eviction cannot take them
            self.refcount[p] += 1
        priv = need - len(pages)
        while self.available() < priv and self._evict_one():
            pass
        if self.available() < priv:
            for p in pages:
                self._drop(p)
            raise NoPages()
        for h in hashes:
            self.cache[h]["last_use"] = self.clock
        self.reqs[req] = dict(pages=list(pages), prompt=prompt, tokens=len(pages) * self.P,
                              reserve=need)
        self.reserved += priv
        self.clock += 1
        return len(pages) * self.P

    def append(self, req, n_tokens):
        r = self.reqs[req]
        total = r["tokens"] + n_tokens
        if n_tokens < 0 or total > r["reserve"] * self.P:
            raise ValueError("beyond the admitted maximum")
        while len(r["pages"]) * self.P < total:
            r["pages"].append(self._take())
            self.reserved -= 1
        r["tokens"] = total

    def finish(self, req, publish=True):
        r = self.reqs.pop(req)
        if publish:
            full = min(len(r["prompt"]), r["tokens"]) // self.P
            key = 0
            for b in range(full):
                blk = r["prompt"][b * self.P:(b + 1) * self.P]
                h = block_hash(key, blk)
                e = self.cache.get(h)
                if e is not None:
                    if e["parent"] != key or e["tokens"] != blk:
                        break
                    e["last_use"] = self.clock
                else:
                    page = r["pages"][b]
                    self.cache[h] = dict(page=page, parent=key, tokens=list(blk), children=0,
                                         last_use=self.clock, seq=self.next_seq)
                    self.next_seq += 1
                    self.refcount[page] += 1
                    if key != 0:
                        self.cache[key]["children"] += 1
                key = h
        for p in r["pages"]:
            self._drop(p)
        self.reserved -= r["reserve"] - len(r["pages"])
        self.clock += 1

    def evict(self, pages):
        freed = 0
        while freed < pages:
            before = len(self.free)
            if not self._evict_one():
                break
            freed += len(self.free) - before
        return freed

    def block_table(self, req):
        return list(self.reqs[req]["pages"])

    def stats(self):
        return len(self.free), self.reserved, len(self.cache)
