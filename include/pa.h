/*
 * pa.h -- C ABI of the paged-attention tick library (libpa.so), gfx950 (MI355X).
 *
 * One packed continuous-batching tick of one attention layer: decode tokens
 * (one query row per sequence) and chunked-prefill slices (several rows per
 * sequence) share one forward, each with its own positions and page table
 * into a shared pool of fixed-size KV pages (Helios blog "I built an Inference
 * Engine that beats vLLM", sections "Prefill vs Decode", "Continuous batching"
 * and "Paged attention"; Helios README, section "Continuous batching").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument is DEVICE memory owned by the caller, unless the
 *   comment says otherwise. The library allocates no memory, frees nothing
 *   and never synchronises: it checks its host scalars, enqueues kernels on
 *   `stream` (a hipStream_t; NULL = the default stream) and returns.
 * - Return value: PA_OK, or an error code. A PA_ERR_INVALID_ARG or
 *   PA_ERR_UNSUPPORTED return enqueues nothing. Nothing aborts, throws or
 *   prints. PA_ERR_HIP means a HIP launch failed after checks passed.
 * - Device metadata (page tables, lengths, slots) is NOT read by the host,
 *   unless validation is on (pa_set_validation). Out-of-range values there
 *   cannot make a kernel read or write outside the buffers described here
 *   (indices are clamped or the row is skipped), but the results for such
 *   rows are unspecified.
 * - Layouts are dense row-major, innermost dimension last:
 *     q, out   [T, Hq, D]             new query rows of the tick, packed
 *     k, v     [T, Hkv, D]            new key/value rows of the tick, packed
 *     k_pool,
 *     v_pool   [num_pages, P, Hkv, D] one layer's K (resp. V) page pool
 *   (pool order follows the per-layer slice of [layers, 2, blocks,
 *   block_size, kv_heads, head_dim] on the llm-serving-engine README, row
 *   "KV Cache" and section "KV cache memory layout").
 * - dtype PA_F32 = float32 storage, PA_BF16 = bfloat16 storage; all
 *   arithmetic accumulates in float32.
 * - Supported shapes: D in {16, 64, 128} for PA_F32, {64, 128} for PA_BF16;
 *   Hq / Hkv in {1, 2, 4, 8}; P (page size) a power of two >= 16. Others:
 *   PA_ERR_UNSUPPORTED.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,         /* a host scalar or pointer is invalid */
  PA_ERR_UNSUPPORTED = 2,         /* dtype / head_dim / group / page size has no kernel */
  PA_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below the size query's answer */
  PA_ERR_HIP = 4,                 /* a HIP call failed */
  PA_ERR_NO_PAGES = 5             /* the block manager has too few free pages (pa_blocks.h) */
} pa_status_t;

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype_t;

/* Version of this ABI; bumped on any signature or semantic change. */
int32_t pa_abi_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* pa_status_string(pa_status_t status);

/*
 * pa_set_validation -- opt-in checking of the device metadata, process-wide
 * (off by default; on = any nonzero value). A failing request is reported by
 * name, the way the pages' engines report a failed request with its id
 * (Helios README, "Diagnostics and logs").
 *
 * While on, pa_compute_slot_mapping, pa_rope_and_cache_write,
 * pa_paged_attention_varlen and pa_tick_forward first synchronise `stream`
 * and copy their metadata to the host (query_start_loc, seq_lens, the
 * block tables, positions or slot_mapping: a few KB per call, and the
 * copy waits for the work already queued on the stream), then check every
 * precondition the kernels otherwise take on trust, and return
 * PA_ERR_INVALID_ARG with nothing enqueued if one fails:
 *   - query_start_loc starts at 0, never decreases and ends at T;
 *   - for every sequence with rows: L <= seq_len <= max_seq_len,
 *     L <= max_query_len, ceil(seq_len / P) <= max_blocks_per_seq, and those
 *     first block-table entries are page ids in [0, num_pages);
 *   - pa_tick_forward: row i of a sequence with L rows and n keys is at
 *     position n - L + i (this tick's tokens are the sequence's last keys),
 *     inside the cos/sin table when one is given, and the page it is written
 *     to is used by no other sequence of the tick (shared pages are full and
 *     read-only: Helios blog, "Prefix caching");
 *   - pa_rope_and_cache_write: no two rows write the same pool slot.
 * Validation copies and checks on the host; the calls are otherwise unchanged
 * (same kernels, same results). Not meant for the timed serving loop.
 */
void pa_set_validation(int32_t on);

/*
 * pa_validation_message -- why the last call on the calling thread failed
 * validation, naming the sequence, row or token ("" when the last checked
 * call passed or validation is off). Points to thread-local storage that the
 * next call on the same thread overwrites.
 */
const char* pa_validation_message(void);

/*
 * pa_rope_cos_sin_table -- build the cached cos/sin table for RoPE
 * (llm-serving-engine README, row "RoPE from scratch": rotary embeddings from
 * cached sin/cos tables; Helios blog, "torch.sdpa and Flash Attention": RoPE
 * on Q and K after projection).
 *
 *   cos_sin  [max_pos, head_dim] float32, written: column i < D/2 holds
 *            cos(p * theta^(-2i/D)), column D/2 + i holds the sine; the angle
 *            and both functions are evaluated in float64 and rounded once.
 *   max_pos >= 1, head_dim even and >= 2, theta > 0.
 * Built once per model (it depends on no tick data).
 */
pa_status_t pa_rope_cos_sin_table(float* cos_sin, int32_t max_pos, int32_t head_dim,
                                  double theta, void* stream);

/*
 * pa_compute_slot_mapping -- slot of every new token of a packed tick.
 * A token at absolute position p of sequence s goes to slot
 * block_tables[s][p / P] * P + p % P of the pool (Helios blog, "Paged
 * attention": new tokens take pages from the free list and are written into
 * the request's pages; mini-vLLM page, "Paged KV-cache": the block table maps
 * positions to blocks).
 *
 *   block_tables     [S, max_blocks_per_seq] int32, physical page ids
 *   query_start_loc  [S + 1] int32, non-decreasing, [0] = 0, [S] = T;
 *                    rows of sequence s are query_start_loc[s] .. [s+1]-1
 *   positions        [T] int32 absolute positions
 *   slot_mapping     [T] int32, written; -1 where the position or page id is
 *                    out of range (such a row is then skipped by the writer)
 */
pa_status_t pa_compute_slot_mapping(const int32_t* block_tables, const int32_t* query_start_loc,
                                    const int32_t* positions, int32_t* slot_mapping,
                                    int32_t S, int32_t T, int32_t max_blocks_per_seq,
                                    int32_t page_size, int32_t num_pages, void* stream);

/*
 * pa_rope_and_cache_write -- RoPE on the tick's new Q and K (in place), then
 * the new K and V rows into their page slots, all before any attention read
 * (llm-serving-engine README, "_step_prefill": write K/V at the chunk's
 * start slot; Helios README, "Paged attention": decode writes directly into
 * the shared KV pool).
 *
 *   q         [T, Hq, D]  rotated in place; may be NULL (no query rotation)
 *   k         [T, Hkv, D] rotated in place, then stored
 *   v         [T, Hkv, D] stored as is (bit copy)
 *   positions [T] int32   absolute positions (rows into cos_sin)
 *   slot_mapping [T] int32 slot per token; a slot < 0 or >= num_pages * P
 *             skips the pool write of that row (padding rows)
 *   cos_sin   [max_pos, D] float32 from pa_rope_cos_sin_table, or NULL for
 *             no RoPE (then q and k are left unchanged and k is stored as is)
 *   k_pool, v_pool [num_pages, P, Hkv, D], written at the mapped slots only
 *
 * head_dim: a multiple of 16, at most 2048 (else PA_ERR_UNSUPPORTED).
 * Rotation: for pair (i, i + D/2), x1' = x1*c - x2*s and x2' = x2*c + x1*s in
 * float32 with each product and sum rounded separately (no fused
 * multiply-add), then rounded to nearest-even into the storage dtype. A
 * position outside [0, max_pos) leaves that row unrotated.
 * Preconditions (not checked): no two rows map to the same slot.
 */
pa_status_t pa_rope_and_cache_write(void* q, void* k, const void* v,
                                    const int32_t* positions, const int32_t* slot_mapping,
                                    const float* cos_sin, void* k_pool, void* v_pool,
                                    int32_t T, int32_t Hq, int32_t Hkv, int32_t head_dim,
                                    int32_t page_size, int32_t num_pages, int32_t max_pos,
                                    pa_dtype_t dtype, void* stream);

/*
 * pa_paged_attention_workspace_size -- bytes of device scratch that
 * pa_paged_attention_varlen needs for these host scalars (split-KV partial
 * results). May be 0. kv_split_tokens as passed to the attention call.
 */
size_t pa_paged_attention_workspace_size(int32_t S, int32_t T, int32_t Hq, int32_t head_dim,
                                         int32_t max_query_len, int32_t max_seq_len,
                                         int32_t page_size, int32_t kv_split_tokens,
                                         pa_dtype_t dtype);

/*
 * pa_paged_attention_varlen -- attention of one packed tick through the page
 * tables, without gathering K/V into padded dense tensors (Helios README,
 * "Paged attention"; mini-vLLM page, "Paged KV-cache").
 *
 *   q                [T, Hq, D] query rows (already rotated)
 *   k_pool, v_pool   [num_pages, P, Hkv, D] (this tick's K/V already written)
 *   block_tables     [S, max_blocks_per_seq] int32 physical page ids
 *   seq_lens         [S] int32: keys of sequence s, this tick's rows included
 *   query_start_loc  [S + 1] int32: rows of sequence s are qsl[s] .. qsl[s+1]-1
 *   out              [T, Hq, D] written, dtype of q; must not alias q or pools
 *
 * Row i (0-based) of a sequence with L rows and n keys attends keys
 * 0 .. n - L + i: a decode row (L = 1) sees all n keys, a prefill chunk sees
 * every earlier key and itself causally (llm-serving-engine README,
 * "_step_prefill": rectangular causal mask). Query head h reads KV head
 * h / (Hq / Hkv) (grouped-query attention: Helios blog, "torch.sdpa and Flash
 * Attention"). Weights are softmax(scale * q.k) (same section; scale is
 * normally 1/sqrt(D)); sums accumulate in float32 and the output is rounded
 * to nearest-even into the storage dtype.
 *
 * Host scalars: max_query_len >= every L and max_seq_len >= every n (they
 * size the grids; rows beyond them are not computed). S < 2^29 (else
 * PA_ERR_INVALID_ARG). Sequences with L = 0 produce nothing. kv_split_tokens: keys per split-KV partition of a decode
 * row (0 = library default; otherwise a multiple of 16 in [16, 65536]).
 * workspace: device scratch of at least
 * pa_paged_attention_workspace_size(...) bytes (NULL allowed when that is 0);
 * its contents on entry do not matter.
 * Preconditions (not checked): L <= n; the first ceil(n / P) entries of each
 * block-table row are valid page ids; pages shared by several sequences are
 * read-only during the call.
 * Caching: decode rows stream their K/V past the caches (each row's keys are
 * read once), except rows whose first page is also another decode row's
 * first page (a prefix shared through the page tables: Helios blog, "Prefix
 * caching"), whose keys are loaded into the caches for the other sharers.
 * This changes no result.
 * Shared prefixes read once (bf16, kv_split_tokens = 0, S <= 64): decode
 * rows whose page tables start with the same pages as the lowest-indexed
 * decode row holding that first page (their common leading pages, short of
 * the page with a row's last key) are gathered, up to 16 / (Hq / Hkv) rows
 * at a time, and each such group reads those pages once for all its rows;
 * each row's remaining keys are its own split-KV partitions, and the merge
 * sums both (same section: a cached prefix is not recomputed, and here not
 * re-read either). Results are those of the split-KV merge over a different
 * cut of the key axis: equal within rounding, not bit for bit, to the
 * ungrouped call. When the partial results of the groups would not fit the
 * workspace the call does not group.
 */
pa_status_t pa_paged_attention_varlen(const void* q, const void* k_pool, const void* v_pool,
                                      const int32_t* block_tables, const int32_t* seq_lens,
                                      const int32_t* query_start_loc, void* out,
                                      int32_t S, int32_t T, int32_t Hq, int32_t Hkv,
                                      int32_t head_dim, int32_t page_size, int32_t num_pages,
                                      int32_t max_blocks_per_seq, int32_t max_query_len,
                                      int32_t max_seq_len, float scale, int32_t kv_split_tokens,
                                      pa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * pa_tick_forward -- one layer's whole tick in one call: the results of
 *   pa_compute_slot_mapping(block_tables, query_start_loc, positions,
 *                           slot_mapping, ...),
 *   pa_rope_and_cache_write(q, k, v, positions, slot_mapping, cos_sin,
 *                           k_pool, v_pool, ...),
 *   pa_paged_attention_varlen(q, k_pool, v_pool, block_tables, seq_lens,
 *                             query_start_loc, out, ...)
 * in that order, with the same arguments, layouts and preconditions (q must
 * not be NULL; slot_mapping [T] int32 is written): out, slot_mapping, k_pool
 * and v_pool bit for bit. The tick's new K/V are stored before any attention
 * read that needs them (Helios blog, "Continuous batching": all the tick's
 * rows, prefill and decode, go through one forward). Every check of the three
 * calls is made before anything is enqueued.
 *
 * q and k are inputs here, not results. bf16 ticks leave them unchanged:
 * one launch before the attention holds the slot mapping, the page writes
 * (each token's K rotated into its slot, q and k left as given), the rotation
 * of the decode rows' queries into their rows of `out` (where the decode
 * kernel reads them before it writes the results there) and the attention
 * call's planning (which reads only query_start_loc and seq_lens); the
 * attention kernels rotate each prefill row's query where they read it, with
 * the page writer's arithmetic. For that rotation row i of a sequence with
 * L rows and n keys is taken to be at position n - L + i: the tick's rows are
 * the sequence's last keys (pa_set_validation checks it); with other positions
 * the prefill rows' results are unspecified. float32 ticks run the three
 * calls' kernels (the page write then rotates q and k in place), with the
 * slot mapping, page write and planning in one launch.
 */
pa_status_t pa_tick_forward(void* q, void* k, const void* v, const int32_t* positions,
                            const int32_t* block_tables, const int32_t* seq_lens,
                            const int32_t* query_start_loc, const float* cos_sin, void* k_pool,
                            void* v_pool, void* out, int32_t* slot_mapping, int32_t S, int32_t T,
                            int32_t Hq, int32_t Hkv, int32_t head_dim, int32_t page_size,
                            int32_t num_pages, int32_t max_blocks_per_seq,
                            int32_t max_query_len, int32_t max_seq_len, int32_t max_pos,
                            float scale, int32_t kv_split_tokens, pa_dtype_t dtype,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_tick_forward_noalloc -- pa_tick_forward for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc. Same arguments as pa_tick_forward without
 * the workspace, same results bit for bit (the same kernels).
 *
 * Scratch: one fixed array of 64 MiB of device memory that the library holds
 * on every GPU it runs on until the process ends; its address on a GPU is
 * looked up at the first call there. A tick whose workspace
 * (pa_paged_attention_workspace_size with the same arguments) exceeds
 * 64 MiB returns PA_ERR_WORKSPACE_TOO_SMALL with nothing enqueued, and
 * pa_validation_message() then gives the bytes it needs. Every other check is
 * pa_tick_forward's, and all of them run before any HIP call.
 * The call allocates and frees nothing (no hipMalloc, no hipFree, no
 * allocating library routine). All calls on one GPU share its array; each
 * call writes every part of it that it reads, so nothing needs clearing, but
 * calls that overlap in time on one GPU (two streams, or two host threads)
 * race and give unspecified results. Calls on one stream are ordered and safe.
 */
pa_status_t pa_tick_forward_noalloc(void* q, void* k, const void* v, const int32_t* positions,
                                    const int32_t* block_tables, const int32_t* seq_lens,
                                    const int32_t* query_start_loc, const float* cos_sin,
                                    void* k_pool, void* v_pool, void* out,
                                    int32_t* slot_mapping, int32_t S, int32_t T, int32_t Hq,
                                    int32_t Hkv, int32_t head_dim, int32_t page_size,
                                    int32_t num_pages, int32_t max_blocks_per_seq,
                                    int32_t max_query_len, int32_t max_seq_len, int32_t max_pos,
                                    float scale, int32_t kv_split_tokens, pa_dtype_t dtype,
                                    void* stream);

/*
 * Kernel timing for benchmarks (not part of the tick). While on, every kernel
 * the library enqueues is bracketed by two hipEvents recorded on the same
 * stream, for up to `capacity` launches. pa_profile_stop waits for the last
 * event and turns recording off; pa_profile_get returns launch i's kernel
 * name (copied into name[0 .. name_len-1], NUL-terminated) and duration in
 * milliseconds. Host-side state; not thread-safe; events are created by
 * pa_profile_start and destroyed by the next start or by pa_profile_reset.
 */
pa_status_t pa_profile_start(int32_t capacity);
pa_status_t pa_profile_stop(int32_t* num_records);
pa_status_t pa_profile_get(int32_t index, char* name, int32_t name_len, float* milliseconds);
pa_status_t pa_profile_reset(void);

/*
 * Measurement helpers (not part of a tick).
 *
 * pa_probe_stream_read -- read `bytes` of device memory at `buf` once, as a
 * plain stream of non-temporal 16-byte loads over the whole GPU, and write one 32-bit word
 * per thread to `sink` (pa_probe_sink_words() words of device memory): the
 * practical read bandwidth of this GPU, against which the HBM-bound kernels'
 * achieved bandwidth is read. bytes > 0 and a multiple of 16, buf 16-byte
 * aligned, sink 4-byte aligned, else PA_ERR_INVALID_ARG. Asynchronous on
 * `stream`; recorded by the profile hook under "stream_read".
 */
size_t pa_probe_sink_words(void);
pa_status_t pa_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
