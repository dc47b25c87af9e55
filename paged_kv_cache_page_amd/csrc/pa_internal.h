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
  float* ws;           // split-KV partials: o [rows*max_parts*Hq*D], then (m, l) pairs
  int* plan;           // work lists written by the plan kernel (see pa_plan.hip)
  int32_t cap_dec, cap_pf;  // capacities of the decode chunk and prefill item lists
  int32_t S, T, Hq, Hkv, D, P, num_pages, max_blocks;
  int32_t p_shift;      // log2(P); P is a power of two
  int32_t max_query_len, max_seq_len;
  int32_t part_tokens;  // keys per split-KV partition (at most); 0 = chosen by the plan kernel
  int32_t part_min, part_max;  // bounds of a chosen partition size (multiples of 16)
  int32_t max_parts;    // partitions a row may need (ceil(max_seq_len / smallest size))
  int32_t dec_grid;     // workgroups of the decode kernel (a multiple of 8)
  float scale_log2e;    // scale * log2(e): weights are exp2(s * scale_log2e - m)
};

// Plan layout, in ints from the start of the workspace:
//   header [kPlanHeaderInts]: [0] decode rows R, [1] prefill items (per KV
//     head), [2] chunk keys C, [3] chunks, [4] row alignment A, [5..7]
//     unused, [8 + h] cursor of the tick kernel's prefill queue of KV head h
//     (zeroed)
//   decode rows: S x (sequence, key offset, keys, token); row i's keys occupy
//     [offset, offset + round_up(keys, A)) of the concatenated key axis
//   partitions per sequence: S ints (0 = no decode row)
//   first decode row of each chunk: cap_dec ints
//   prefill items: cap_pf x (sequence, row tile)
constexpr int kPlanHeaderInts = 16;
constexpr int kPlanCursors = 8;
struct PlanOffsets {
  size_t rows, nparts, first_row, pf, total;
};
__host__ __device__ inline PlanOffsets plan_offsets(long S, long cap_dec, long cap_pf) {
  PlanOffsets o;
  o.rows = kPlanHeaderInts;
  o.nparts = o.rows + 4 * (size_t)S;
  o.first_row = o.nparts + (size_t)S;
  o.pf = o.first_row + (size_t)cap_dec;
  o.total = o.pf + 2 * (size_t)cap_pf;
  return o;
}
// Query rows per prefill workgroup; a tile holds kPrefillRows / G tokens.
constexpr int kPrefillRows = 64;

// Workgroups of `func` (launched with `threads` threads) that the current
// device holds at once: compute units x resident workgroups per unit. Cached
// per (device, kernel). Used to size persistent grids.
int persistent_grid(const void* func, int threads);
// Compute units of the current device (cached).
int cu_count();

// Kernel timing hook (pa_api.hip): called around every launch.
void profile_before(const char* name, hipStream_t stream);
void profile_after(hipStream_t stream);

// K0 / a1 / K1 (pa_rope_cache.hip)
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

// K2 + K3 (pa_decode.hip). token_mode = false: one row per decode sequence
// (query length 1; other sequences skipped). token_mode = true: one row per
// query token of every sequence (the VALU path for prefill rows).
bool decode_supported(pa_dtype_t dt, int D, int G);
// Workgroups of the persistent decode grid (resident count, a multiple of 8).
int decode_grid(pa_dtype_t dt, int D, int G);
hipError_t launch_decode(pa_dtype_t dt, const AttnArgs& a, bool token_mode, hipStream_t s);
hipError_t launch_split_reduce(pa_dtype_t dt, const AttnArgs& a, bool token_mode,
                               hipStream_t s);

// Fused tick (pa_tick.hip): decode rows and prefill chunks in one grid.
bool tick_supported(pa_dtype_t dt, int D);
hipError_t launch_tick(pa_dtype_t dt, const AttnArgs& a, hipStream_t s);

// K4 (pa_prefill.hip): MFMA prefill-chunk attention for sequences with L > 1.
bool prefill_mfma_supported(pa_dtype_t dt, int D, int G);
hipError_t launch_prefill_mfma(pa_dtype_t dt, const AttnArgs& a, hipStream_t s);

}  // namespace pa
