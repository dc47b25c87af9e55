// Host-side launch interface between the C ABI (pa_api.hip) and the kernel
// translation units. Nothing here is exported from libpa.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/pa.h"

namespace pa {

// Arguments of the attention kernels. All pointers are device memory.
struct AttnArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* qsl;
  void* out;
  float* ws;           // split-KV partials: o [part_slots*Hq*D], then (m, l) pairs
  int* plan;           // work lists written by the plan (see pa_plan.h)
  int32_t cap_dec, cap_pf;  // capacities of the decode chunk and prefill item lists
  int32_t S, T, Hq, Hkv, D, P, num_pages, max_blocks;
  int32_t p_shift;      // log2(P); P is a power of two
  int32_t max_query_len, max_seq_len;
  int32_t part_tokens;  // keys per split-KV partition (at most); 0 = chosen by the plan kernel
  int32_t part_min, part_max;  // bounds of a chosen partition size (multiples of 16)
  int32_t max_parts;    // partitions a row may need (ceil(max_seq_len / smallest size))
  int32_t part_slots;   // split-KV partial slots (each holds all Hq heads of one partition)
  int32_t dec_grid;     // workgroups of the decode kernel (a multiple of 8)
  float scale_log2e;    // scale * log2(e): weights are exp2(s * scale_log2e - m)
  // Key-range pieces of long prefill items (automatic partitions only):
  float* pf_ws;         // partials: o [pf_slots][kPrefillRows][D], then (m, l) [pf_slots][kPrefillRows]
  int32_t pf_slots;     // partial slots (0 = never split)
  int32_t pf_workers;   // workgroups of the kernel that runs the prefill items
  // The fused tick (bf16): q is the unrotated input. The prefill items rotate
  // each query row where they read it (row i of a chunk of L rows over n keys
  // at position n - L + i); the decode kernel reads a decode row's query,
  // rotated by the page-write launch, from the row's output row. 0 / null
  // otherwise.
  int32_t fused;
  const float* cos_sin;       // [max_pos, D] or null (no RoPE)
  int32_t max_pos;
  // Decode rows sharing a prefix may be grouped (the bf16 matrix-core decode
  // walks group rows; the other decode paths do not): 1 / 0.
  int32_t group_rows;
};

// Plan layout, in ints from the start of the workspace:
//   header [32]: [0] decode rows R, [1] prefill entries (per KV head), [2]
//     chunk keys C, [3] chunks, [4] row alignment A, [5] cut prefill items,
//     [6] chunks taken one per decode wave n_s, [7] claimed items (chunks
//     past n_s x Hkv), [8] prefill queues found empty (counted by the
//     tick kernel's claims), [9..31] unused
//   prefill queue cursors: Hq counters, one per 128-byte line (Hq >= Hkv
//     bounds the KV heads, which the workspace query does not see): the
//     queue of KV head h at kPlanLine * (1 + h); then the counter of the
//     claimed decode chunks on line 1 + Hq. All zeroed by the plan kernel,
//     advanced with device-scope atomics
//   decode rows: plan_rows(S) x (sequence, key offset, keys, token); row i's
//     keys occupy [offset, offset + round_up(keys, A)) of the concatenated key
//     axis and are the sequence's keys [kstart, kstart + keys). A group row
//     (kRowGroup) is the shared prefix of m sharing rows, which follow it in
//     the list: its sequence is one whose page table holds the prefix, its
//     token field is m, and each of its partitions writes one partial per
//     member (partition p of the group row at the member's slot base + p)
//   partitions per decode row: plan_rows(S) ints (0 for a group row, which
//     the merge skips; a member counts the group row's partitions too)
//   first partial slot per decode row: plan_rows(S) ints (rows of one
//     partition own none)
//   first key per decode row (kstart): plan_rows(S) ints
//   first partition index per decode row: plan_rows(S) ints (a member's own
//     partitions follow its group row's)
//   first decode row of each chunk: cap_dec ints
//   prefill entries (16-byte aligned): cap_pf x (sequence, row tile,
//     piece j | pieces J << 16, first partial slot), in decreasing cost order;
//     an item (sequence, row tile) of J > 1 pieces owns the partial slots
//     [slot, slot + J * Hkv): KV head h, piece j at slot + h * J + j
//   the entries' sequence shapes: cap_pf x (first query row q0, query length
//     L, keys n clamped as the kernels clamp them, 0), read beside the entry
//     so that a prefill item does not wait for a second load to learn them
//   cut prefill items: cap_pf x (sequence, row tile, J, slot), merged by the
//     prefill merge kernel after the tick
// Bits of a decode row's sequence index in the plan's row list. kRowShared:
// the row's keys are read by other rows too (a prefix shared through the
// page tables), so they are loaded into the caches, where the sharers find
// them; the other rows' keys are read once and are loaded as a stream.
// kRowGroup: a group row (above). The host bounds S below both bits.
constexpr int kRowShared = 1 << 30;
constexpr int kRowGroup = 1 << 29;
constexpr int kPlanLine = 32;  // ints per 128-byte cache line
// Rows of the decode row list: the decode rows, and at most one group row
// per two of them.
__host__ __device__ inline long plan_rows(long S) { return S + S / 2 + 1; }
// Partial slots per decode row reserved for group members (bf16, automatic
// partitions).
constexpr long kGroupSlotsPerRow = 4;
struct PlanOffsets {
  size_t rows, nparts, pbase, kstart, part0, first_row, pf, pf_shape, merge, total;
};
__host__ __device__ inline PlanOffsets plan_offsets(long S, long Hq, long cap_dec, long cap_pf) {
  PlanOffsets o;
  const size_t R = (size_t)plan_rows(S);
  o.rows = (size_t)kPlanLine * (2 + (size_t)Hq);
  o.nparts = o.rows + 4 * R;
  o.pbase = o.nparts + R;
  o.kstart = o.pbase + R;
  o.part0 = o.kstart + R;
  o.first_row = o.part0 + R;
  o.pf = (o.first_row + (size_t)cap_dec + 3) / 4 * 4;
  o.pf_shape = o.pf + 4 * (size_t)cap_pf;
  o.merge = o.pf_shape + 4 * (size_t)cap_pf;
  o.total = o.merge + 4 * (size_t)cap_pf;
  return o;
}
__host__ __device__ inline int plan_pf_cursor(int h) { return kPlanLine * (1 + h); }
__host__ __device__ inline int plan_pf_dry() { return 8; }
__host__ __device__ inline int plan_dec_cursor(int Hq) { return kPlanLine * (1 + Hq); }

// Query rows per prefill workgroup; a tile holds kPrefillRows / G tokens.
constexpr int kPrefillRows = 128;
// Keys per prefill K/V tile (the unit in which prefill items are cut into pieces).
constexpr int kPrefillTileKeys = 64;
// Partial slots of prefill pieces (per call; the plan kernel lengthens the
// pieces until they fit) and the shortest piece, in tiles.
constexpr int kPrefillSlots = 512;
constexpr int kMinPieceTiles = 4;
// Decode keys a decode wave streams (one KV head, K and V) in the time a
// prefill workgroup takes for one K/V tile of its item, both sharing the GPU:
// about 0.1 us per key against 3 us per tile on MI355X at head_dim 128.
constexpr int kDecodeKeysPerTile = 32;

// Workgroups of `func` (launched with `threads` threads) that the current
// device holds at once: compute units x resident workgroups per unit. Cached
// per (device, kernel). Used to size persistent grids.
int persistent_grid(const void* func, int threads);
// Compute units of the current device (cached).
int cu_count();

// Kernel timing hook (pa_api.hip): called around every launch.
void profile_before(const char* name, hipStream_t stream);
void profile_after(hipStream_t stream);

// K0 / a1 / K1 (pa_rope_cache.hip). K1 takes head dims up to kRopeMaxHeadDim
// (the vectors of a half row fit one workgroup).
constexpr int kRopeMaxHeadDim = 2048;
hipError_t launch_rope_table(float* out, int max_pos, int D, double theta, hipStream_t s);
hipError_t launch_slot_mapping(const int32_t* bt, const int32_t* qsl, const int32_t* pos,
                               int32_t* slots, int S, int T, int max_blocks, int P,
                               int num_pages, hipStream_t s);
hipError_t launch_rope_cache_write(pa_dtype_t dt, void* q, void* k, const void* v,
                                   const int32_t* pos, const int32_t* slots, const float* cs,
                                   void* k_pool, void* v_pool, int T, int Hq, int Hkv, int D,
                                   int P, int num_pages, int max_pos, hipStream_t s);

// Work lists (pa_plan.hip). TM = tokens per prefill tile.
hipError_t launch_plan(const AttnArgs& a, int* plan, int cap_dec, int cap_pf, int TM,
                       hipStream_t s);

// a1 + K1 for every token of the tick and, when plan_args is given, the plan
// of that attention call, in one launch (pa_rope_cache.hip). Same results as
// launch_slot_mapping, launch_rope_cache_write and launch_plan.
hipError_t launch_tick_prep(pa_dtype_t dt, void* q, void* k, const void* v, const int32_t* pos,
                            const int32_t* bt, const int32_t* qsl, int32_t* slots,
                            const float* cs, void* k_pool, void* v_pool, int S, int T, int Hq,
                            int Hkv, int D, int P, int num_pages, int max_blocks, int max_pos,
                            const AttnArgs* plan_args, int cap_dec, int cap_pf, int TM,
                            bool fused, hipStream_t s);

// K2 + K3 (pa_decode.hip). token_mode = false: one row per decode sequence
// (query length 1; other sequences skipped). token_mode = true: one row per
// query token of every sequence (the VALU path for prefill rows).
bool decode_supported(pa_dtype_t dt, int D, int G);
// Workgroups of the persistent decode grid (resident count, a multiple of 8),
// and the largest of them over the supported groups G.
int decode_grid(pa_dtype_t dt, int D, int G);
int decode_grid_max(pa_dtype_t dt, int D);
hipError_t launch_decode(pa_dtype_t dt, const AttnArgs& a, bool token_mode, hipStream_t s);
hipError_t launch_split_reduce(pa_dtype_t dt, const AttnArgs& a, bool token_mode,
                               hipStream_t s);

// Fused tick (pa_tick.hip): decode rows and prefill chunks (K4 on MFMA) in
// one persistent grid; tick_grid = its workgroup count.
bool tick_supported(pa_dtype_t dt, int D);
int tick_grid(pa_dtype_t dt, int D, int G);
hipError_t launch_tick(pa_dtype_t dt, const AttnArgs& a, hipStream_t s);
// After the tick (pa_tick.hip): merge of the decode rows' split-KV partitions
// and of the pieces of cut prefill items, in one launch.
hipError_t launch_tick_reduce(const AttnArgs& a, hipStream_t s);

}  // namespace pa
