/*
 * pa_blocks.h -- host-side paged block manager: the pages of the shared KV
 * pool, each request's page table, and the prefix cache of complete blocks.
 * It produces the block_tables the attention entry points of pa.h consume.
 *
 * What it follows (Helios blog, "Paged attention" and "Prefix caching";
 * Helios README, "Paged attention" and "Loading"; llm-serving-engine README,
 * table rows "Physical Block Manager" and "Prefix / Prompt Caching"):
 *   - a fixed pool of P-token pages; new tokens take pages from the free list
 *     and any free page fits any request;
 *   - admission reserves the request's maximum length (prompt + new tokens),
 *     rounded up to whole pages, so that its decode never runs out of pages;
 *   - a page returns to the free list when its last holder -- a request or the
 *     prefix cache -- releases it;
 *   - complete P-token prompt blocks are hashed in order, each hash chained
 *     with the previous block's; an arriving request restores the longest
 *     cached chain (sharing those physical pages) and prefills only the rest;
 *     a partial last block is never cached;
 *   - when pages are short, unused cached blocks are evicted leaf first
 *     (never a block that a later cached block depends on), least recently
 *     used first.
 *
 * Host memory only; nothing here touches the GPU. One manager is not safe for
 * concurrent use from several threads. Every function returns PA_OK or an
 * error code. On error nothing changes, except that a pa_bm_admit which ends
 * in PA_ERR_NO_PAGES may already have evicted unused cached blocks.
 */
#ifndef PA_BLOCKS_H
#define PA_BLOCKS_H

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/* A manager of num_pages pages of page_size tokens (both >= 1). *out owns the
 * manager until pa_bm_destroy. Pages start free; page 0 is handed out first. */
pa_status_t pa_bm_create(int32_t num_pages, int32_t page_size, pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* bm);

/* Admit request `req` (any id not currently admitted) with prompt tokens
 * prompt[0 .. n_prompt) (n_prompt >= 1) and up to max_new_tokens (>= 0) new
 * tokens. Restores the longest chain of cached complete prompt blocks that
 * end before the last prompt token (so at least that token is left to compute)
 * into its page table (shared pages) and reserves the pages of the rest of
 * n_prompt + max_new_tokens tokens; evicts unused cached blocks if the free
 * pages, less the reservations, fall short. *cached_tokens = the prompt tokens
 * already in the restored pages (a multiple of page_size). PA_ERR_NO_PAGES if
 * the pages cannot be found even after evicting every unused cached block. */
pa_status_t pa_bm_admit(pa_block_manager* bm, int64_t req, const int32_t* prompt,
                        int32_t n_prompt, int32_t max_new_tokens, int32_t* cached_tokens);

/* Record n_tokens (>= 0) more tokens of request req written to its pages
 * (prompt tokens past the cached ones, then generated ones); takes pages from
 * the free list as its table needs them. The total may not exceed the
 * admitted maximum (PA_ERR_INVALID_ARG). */
pa_status_t pa_bm_append(pa_block_manager* bm, int64_t req, int32_t n_tokens);

/* Request req is done. With publish != 0 its complete prompt blocks (those
 * fully written) enter the prefix cache, which then holds a reference to their
 * pages; blocks already cached are kept as they are. The request's references
 * and its unused reservation are released. */
pa_status_t pa_bm_finish(pa_block_manager* bm, int64_t req, int32_t publish);

/* Evict unused cached blocks (leaf first, least recently used first) until
 * `pages` pages were freed or none is left; *freed = the pages freed. */
pa_status_t pa_bm_evict(pa_block_manager* bm, int32_t pages, int32_t* freed);

/* The page table of request req: out[0 .. *n) = its pages in order (logical
 * block i at out[i]), at most capacity entries written; *n = the table's
 * length (a longer table than capacity is PA_ERR_INVALID_ARG). */
pa_status_t pa_bm_block_table(const pa_block_manager* bm, int64_t req, int32_t* out,
                              int32_t capacity, int32_t* n);

/* Counts: free pages, pages reserved but not yet taken, cached blocks. */
pa_status_t pa_bm_stats(const pa_block_manager* bm, int32_t* free_pages, int32_t* reserved_pages,
                        int32_t* cached_blocks);

/* Holders of one page (requests plus the prefix cache). */
pa_status_t pa_bm_refcount(const pa_block_manager* bm, int32_t page, int32_t* refcount);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCKS_H */
