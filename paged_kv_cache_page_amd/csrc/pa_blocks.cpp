// Host-side paged block manager (include/pa_blocks.h): pages of the shared KV
// pool, per-request page tables with reservations, and the prefix cache of
// complete blocks (Helios blog, "Paged attention" and "Prefix caching"; Helios
// README, "Paged attention" and "Loading"; llm-serving-engine README, rows
// "Physical Block Manager" and "Prefix / Prompt Caching").
//
// Policies, fixed so that a run is reproducible:
//   free list     a stack; pages N-1 .. 0 pushed at creation (page 0 on top),
//                 a released page pushed on top, a taken page popped from it;
//   block hash    FNV-1a (64-bit) over the parent block's hash (8 bytes,
//                 little-endian) and the block's tokens (4 bytes each,
//                 little-endian); the first block's parent hash is 0. A cached
//                 entry also keeps its tokens and parent hash, and a lookup
//                 matches only when both agree, so a hash collision never
//                 restores the wrong pages;
//   restoring     at most the complete blocks before the last prompt token, so
//                 that the caller always computes at least that token;
//   eviction      among cached blocks no other cached block has as parent and
//                 whose page only the cache holds, the least recently used
//                 (logical clock: one tick per admit and per finish), ties by
//                 insertion order;
//   publishing    a finished request's fully written prompt blocks, in order,
//                 while the chain matches; a block already cached (the same
//                 tokens after the same parent) keeps its page and is marked
//                 used; the chain stops at the first hash that is cached with
//                 other contents.
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pa_blocks.h"

#define PA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

uint64_t fnv1a_bytes(uint64_t h, uint64_t v, int nbytes) {
  for (int i = 0; i < nbytes; ++i) {
    h ^= (v >> (8 * i)) & 0xFFu;
    h *= 0x100000001b3ull;
  }
  return h;
}

// Hash of the block tokens[0 .. P) following the block of hash `parent`.
uint64_t chain_hash(uint64_t parent, const int32_t* tokens, int P) {
  uint64_t h = 0xcbf29ce484222325ull;
  h = fnv1a_bytes(h, parent, 8);
  for (int i = 0; i < P; ++i) h = fnv1a_bytes(h, (uint32_t)tokens[i], 4);
  return h;
}

struct CacheEntry {
  int32_t page;
  uint64_t parent;             // hash of the previous block (0: the first block)
  std::vector<int32_t> tokens;
  int32_t children = 0;        // cached blocks whose parent this is
  int64_t last_use = 0;
  int64_t seq = 0;             // insertion order
};

struct Request {
  std::vector<int32_t> pages;  // page table: logical block i -> page
  std::vector<int32_t> prompt;
  int64_t tokens = 0;          // tokens written to the pages
  int32_t reserve = 0;         // pages reserved for the admitted maximum
};

}  // namespace

struct pa_block_manager {
  int32_t N, P;
  std::vector<int32_t> refcount;
  std::vector<int32_t> free_list;  // a stack: back() is taken next
  int64_t reserved = 0;            // pages reserved, not yet taken
  std::unordered_map<int64_t, Request> reqs;
  std::unordered_map<uint64_t, CacheEntry> cache;
  int64_t clock = 0, next_seq = 0;

  int64_t available() const { return (int64_t)free_list.size() - reserved; }

  int32_t take_page() {
    const int32_t p = free_list.back();
    free_list.pop_back();
    refcount[p] = 1;
    return p;
  }

  void drop_ref(int32_t p) {
    if (--refcount[p] == 0) free_list.push_back(p);
  }

  // Evict the least recently used unused leaf; false if there is none.
  bool evict_one() {
    const CacheEntry* best = nullptr;
    uint64_t best_key = 0;
    for (const auto& kv : cache) {
      const CacheEntry& e = kv.second;
      if (e.children != 0 || refcount[e.page] != 1) continue;
      if (!best || e.last_use < best->last_use ||
          (e.last_use == best->last_use && e.seq < best->seq)) {
        best = &e;
        best_key = kv.first;
      }
    }
    if (!best) return false;
    const int32_t page = best->page;
    const uint64_t parent = best->parent;
    cache.erase(best_key);
    if (parent != 0) {
      auto it = cache.find(parent);
      if (it != cache.end()) --it->second.children;
    }
    drop_ref(page);
    return true;
  }
};

PA_EXPORT pa_status_t pa_bm_create(int32_t num_pages, int32_t page_size,
                                   pa_block_manager** out) {
  if (!out || num_pages < 1 || page_size < 1) return PA_ERR_INVALID_ARG;
  pa_block_manager* bm = new (std::nothrow) pa_block_manager();
  if (!bm) return PA_ERR_INVALID_ARG;
  bm->N = num_pages;
  bm->P = page_size;
  bm->refcount.assign((size_t)num_pages, 0);
  bm->free_list.reserve((size_t)num_pages);
  for (int32_t p = num_pages - 1; p >= 0; --p) bm->free_list.push_back(p);
  *out = bm;
  return PA_OK;
}

PA_EXPORT void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

PA_EXPORT pa_status_t pa_bm_admit(pa_block_manager* bm, int64_t req, const int32_t* prompt,
                                  int32_t n_prompt, int32_t max_new_tokens,
                                  int32_t* cached_tokens) {
  if (!bm || !prompt || !cached_tokens || n_prompt < 1 || max_new_tokens < 0 ||
      bm->reqs.count(req))
    return PA_ERR_INVALID_ARG;
  const int64_t total = (int64_t)n_prompt + max_new_tokens;
  const int64_t need = (total + bm->P - 1) / bm->P;
  if (need > bm->N) return PA_ERR_NO_PAGES;
  // longest cached chain of complete prompt blocks, short of the last prompt
  // token (which the caller computes to get the next token); its pages are held
  // first, so that eviction below cannot take them
  std::vector<int32_t> matched;
  uint64_t key = 0;
  for (int32_t b = 0; b < (n_prompt - 1) / bm->P; ++b) {
    const int32_t* blk = prompt + (size_t)b * bm->P;
    const uint64_t k = chain_hash(key, blk, bm->P);
    auto it = bm->cache.find(k);
    if (it == bm->cache.end() || it->second.parent != key ||
        !std::equal(blk, blk + bm->P, it->second.tokens.begin()))
      break;
    matched.push_back(it->second.page);
    ++bm->refcount[it->second.page];
    key = k;
  }
  const int64_t priv = need - (int64_t)matched.size();
  while (bm->available() < priv && bm->evict_one()) {
  }
  if (bm->available() < priv) {
    for (int32_t p : matched) bm->drop_ref(p);
    return PA_ERR_NO_PAGES;
  }
  // the restored entries were just used
  key = 0;
  for (size_t b = 0; b < matched.size(); ++b) {
    const uint64_t k = chain_hash(key, prompt + b * bm->P, bm->P);
    bm->cache[k].last_use = bm->clock;
    key = k;
  }
  Request r;
  r.pages = matched;
  r.prompt.assign(prompt, prompt + n_prompt);
  r.tokens = (int64_t)matched.size() * bm->P;
  r.reserve = (int32_t)need;
  bm->reserved += priv;
  bm->reqs.emplace(req, std::move(r));
  ++bm->clock;
  *cached_tokens = (int32_t)(matched.size() * bm->P);
  return PA_OK;
}

PA_EXPORT pa_status_t pa_bm_append(pa_block_manager* bm, int64_t req, int32_t n_tokens) {
  if (!bm || n_tokens < 0) return PA_ERR_INVALID_ARG;
  auto it = bm->reqs.find(req);
  if (it == bm->reqs.end()) return PA_ERR_INVALID_ARG;
  Request& r = it->second;
  const int64_t tokens = r.tokens + n_tokens;
  if (tokens > (int64_t)r.reserve * bm->P) return PA_ERR_INVALID_ARG;
  // the reservation guarantees these pages: available() >= 0 at all times
  while ((int64_t)r.pages.size() * bm->P < tokens) {
    r.pages.push_back(bm->take_page());
    --bm->reserved;
  }
  r.tokens = tokens;
  return PA_OK;
}

PA_EXPORT pa_status_t pa_bm_finish(pa_block_manager* bm, int64_t req, int32_t publish) {
  if (!bm) return PA_ERR_INVALID_ARG;
  auto it = bm->reqs.find(req);
  if (it == bm->reqs.end()) return PA_ERR_INVALID_ARG;
  Request& r = it->second;
  if (publish) {
    const int64_t full = std::min<int64_t>((int64_t)r.prompt.size(), r.tokens) / bm->P;
    uint64_t key = 0;
    for (int64_t b = 0; b < full; ++b) {
      const int32_t* blk = r.prompt.data() + (size_t)b * bm->P;
      const uint64_t k = chain_hash(key, blk, bm->P);
      auto e = bm->cache.find(k);
      if (e != bm->cache.end()) {
        if (e->second.parent != key || !std::equal(blk, blk + bm->P, e->second.tokens.begin()))
          break;  // a different block under the same hash: the chain stops
        e->second.last_use = bm->clock;
      } else {
        CacheEntry ne;
        ne.page = r.pages[(size_t)b];
        ne.parent = key;
        ne.tokens.assign(blk, blk + bm->P);
        ne.last_use = bm->clock;
        ne.seq = bm->next_seq++;
        ++bm->refcount[ne.page];
        if (key != 0) ++bm->cache[key].children;
        bm->cache.emplace(k, std::move(ne));
      }
      key = k;
    }
  }
  for (int32_t p : r.pages) bm->drop_ref(p);
  bm->reserved -= (int64_t)r.reserve - (int64_t)r.pages.size();
  bm->reqs.erase(it);
  ++bm->clock;
  return PA_OK;
}

PA_EXPORT pa_status_t pa_bm_evict(pa_block_manager* bm, int32_t pages, int32_t* freed) {
  if (!bm || !freed || pages < 0) return PA_ERR_INVALID_ARG;
  int32_t n = 0;
  while (n < pages) {
    const size_t before = bm->free_list.size();
    if (!bm->evict_one()) break;
    n += (int32_t)(bm->free_list.size() - before);
  }
  *freed = n;
  return PA_OK;
}

PA_EXPORT pa_status_t pa_bm_block_table(const pa_block_manager* bm, int64_t req, int32_t* out,
                                        int32_t capacity, int32_t* n) {
  if (!bm || !n || capacity < 0 || (capacity > 0 && !out)) return PA_ERR_INVALID_ARG;
  auto it = bm->reqs.find(req);
  if (it == bm->reqs.end()) return PA_ERR_INVALID_ARG;
  const std::vector<int32_t>& pages = it->second.pages;
  if ((int64_t)pages.size() > capacity) return PA_ERR_INVALID_ARG;
  std::copy(pages.begin(), pages.end(), out);
  *n = (int32_t)pages.size();
  return PA_OK;
}

PA_EXPORT pa_status_t pa_bm_stats(const pa_block_manager* bm, int32_t* free_pages,
                                  int32_t* reserved_pages, int32_t* cached_blocks) {
  if (!bm || !free_pages || !reserved_pages || !cached_blocks) return PA_ERR_INVALID_ARG;
  *free_pages = (int32_t)bm->free_list.size();
  *reserved_pages = (int32_t)bm->reserved;
  *cached_blocks = (int32_t)bm->cache.size();
  return PA_OK;
}

PA_EXPORT pa_status_t pa_bm_refcount(const pa_block_manager* bm, int32_t page,
                                     int32_t* refcount) {
  if (!bm || !refcount || page < 0 || page >= bm->N) return PA_ERR_INVALID_ARG;
  *refcount = bm->refcount[(size_t)page];
  return PA_OK;
}
