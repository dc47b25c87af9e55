// Work planning for one packed tick, on the device.
//
// The host knows only upper bounds (max_query_len, max_seq_len); the lengths of
// the tick's sequences live in device memory. Instead of launching a grid over
// every (sequence, tile) pair and letting most workgroups exit, one small
// workgroup reads query_start_loc and seq_lens once and writes two compact
// lists into the workspace:
//   decode rows   every row with query length 1, laid end to end on one key
//                 axis (each row padded to a multiple of A keys), cut into
//                 equal chunks of C keys, one per decode wave: every wave gets
//                 the same work however the lengths are spread (split-KV for
//                 long rows, several short rows per chunk); with a fixed
//                 partition size A = C = that size, so a chunk never spans
//                 two rows and a row's partitions depend on the row alone;
//   prefill entries (sequence, row tile, piece) for every sequence with query
//                 length > 1, ordered by decreasing number of key tiles, so that
//                 the longest start first (longest-processing-time-first
//                 scheduling). With automatic partitions an item whose key
//                 tiles exceed Tp is cut into ceil(tiles / Tp) pieces of equal
//                 tile counts, each run by its own workgroup (their partials
//                 are merged by a small kernel after the tick, from a list of
//                 the cut items the plan also writes): Tp is the tick's mean
//                 tile count per prefill workgroup (at least kMinPieceTiles),
//                 doubled until the pieces' partials fit the slots, so that no
//                 single item outlasts the rest of the prefill work.
// The persistent attention kernels then walk these lists.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kCostBins = 2048;
constexpr int kCachedSeqs = 4096;  // sequence shapes kept in LDS between the passes

constexpr int kPlanWaves = kPlanThreads / 64;

// Exclusive scan of one int per thread over the workgroup (a shuffle scan in
// each wave, then the wave totals through LDS); returns the thread's offset
// and writes the workgroup total to *total (uniform).
__device__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  if (lane == 63) s_wave[w] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kPlanWaves; ++i) {
    const int x = s_wave[i];
    before += i < w ? x : 0;
    all += x;
  }
  __syncthreads();  // s_wave is free again
  *total = all;
  return before + incl - v;
}

// Sum of one 64-bit value per thread over the workgroup (uniform result).
__device__ long long block_sum(long long v, long long* s_wave) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) s_wave[threadIdx.x >> 6] = v;
  __syncthreads();
  long long all = 0;
#pragma unroll
  for (int i = 0; i < kPlanWaves; ++i) all += s_wave[i];
  __syncthreads();
  return all;
}

struct SeqShape {
  int L, n, q0;
};

__device__ __forceinline__ SeqShape seq_shape(const AttnArgs& a, int s) {
  SeqShape r;
  const int q0 = a.qsl[s];
  r.q0 = q0;
  r.L = a.qsl[s + 1] - q0;
  int n = a.seq_lens[s];
  n = min(n, a.max_blocks * a.P);
  r.n = min(n, a.max_seq_len);  // the attention kernels clamp the same way
  if (q0 < 0 || q0 + r.L > a.T || r.L < 0) r.L = 0;  // malformed rows are skipped
  return r;
}

// Key tiles of row tile mt (the keys its last row sees, in kPrefillTileKeys
// units), capped at kCostBins - 1: the plan cuts and orders items by this.
__device__ __forceinline__ int item_tiles(const SeqShape& sh, int mt, int TM) {
  const int i1 = min(sh.L, (mt + 1) * TM);
  const int keys = sh.n - sh.L + i1;
  const int c = (keys + kPrefillTileKeys - 1) / kPrefillTileKeys;
  return c < 0 ? 0 : (c >= kCostBins ? kCostBins - 1 : c);
}

// Pieces of an item of t tiles for piece length Tp (1 = not cut).
__device__ __forceinline__ int item_pieces(int t, int Tp) { return t > Tp ? (t + Tp - 1) / Tp : 1; }

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(AttnArgs a, int* plan, int cap_dec,
                                                            int cap_pf, int TM) {
  __shared__ int s_buf[kPlanWaves];
  __shared__ long long s_keys[kPlanWaves];
  __shared__ int s_hist[kCostBins];
  __shared__ int s_cur[kCostBins];
  __shared__ int s_tp, s_slot_next, s_merge_next, s_maxt;
  __shared__ long long s_tiles[kPlanWaves];
  __shared__ int s_L[kCachedSeqs], s_n[kCachedSeqs], s_q0[kCachedSeqs];
  const int tid = threadIdx.x;
  const PlanOffsets po = plan_offsets(a.S, a.Hq, cap_dec, cap_pf);
  int4* dec_rows = reinterpret_cast<int4*>(plan + po.rows);
  int* nparts_of = plan + po.nparts;
  int* first_row = plan + po.first_row;
  int4* pf_items = reinterpret_cast<int4*>(plan + po.pf);
  int4* merge_items = reinterpret_cast<int4*>(plan + po.merge);
  // fixed partitions: rows padded to whole partitions; otherwise to 16 keys
  const int A = a.part_tokens > 0 ? a.part_tokens : 16;
  auto shape = [&](int s) {
    return s < kCachedSeqs ? SeqShape{s_L[s], s_n[s], s_q0[s]} : seq_shape(a, s);
  };

  for (int i = tid; i < kCostBins; i += kPlanThreads) s_hist[i] = 0;
  if (tid == 0) s_maxt = 0;
  __syncthreads();

  // ---- pass 1: shapes, padded decode keys, prefill cost histogram ----
  long long my_keys = 0;
  for (int s = tid; s < a.S; s += kPlanThreads) {
    const SeqShape sh = seq_shape(a, s);
    if (s < kCachedSeqs) {
      s_L[s] = sh.L;
      s_n[s] = sh.n;
      s_q0[s] = sh.q0;
    }
    if (sh.L == 1 && sh.n >= 1) my_keys += (sh.n + A - 1) / A * A;
  }
  const long long total_keys = block_sum(my_keys, s_keys);  // length of the key axis
  // prefill items' key tiles: one wave per sequence, lanes over its row tiles
  const int lane = tid & 63, wid = tid >> 6;
  long long my_tiles = 0;
  for (int s = wid; s < a.S; s += kPlanWaves) {
    const SeqShape sh = shape(s);
    if (sh.L > 1 && sh.n >= sh.L) {
      const int ntiles = (sh.L + TM - 1) / TM;
      for (int mt = lane; mt < ntiles; mt += 64) {
        const int t = item_tiles(sh, mt, TM);
        atomicAdd(&s_hist[t], 1);
        atomicMax(&s_maxt, t);
        my_tiles += t;
      }
    }
  }
  const long long item_tiles_all = block_sum(my_tiles, s_tiles);  // per KV head

  // ---- piece length Tp (wave 0): the mean tile count per prefill workgroup,
  // doubled until the cut items' partials (J slots per item and KV head) fit ----
  if (wid == 0) {
    int Tp = 0x3FFFFFFF;  // never cut
    if (a.pf_slots > 0 && a.part_tokens == 0 && item_tiles_all > 0) {
      const long long w = a.pf_workers > 0 ? a.pf_workers : 1;
      long long t0 = (item_tiles_all * a.Hkv + w - 1) / w;
      Tp = (int)(t0 < kMinPieceTiles ? kMinPieceTiles : (t0 > kCostBins ? kCostBins : t0));
      for (int tries = 0;; ++tries) {
        long long need = 0;
        for (int b = lane; b <= s_maxt; b += 64) {  // bins past the longest item are empty
          const int J = item_pieces(b, Tp);
          if (J > 1) need += (long long)s_hist[b] * J;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) need += __shfl_xor(need, off);
        if (need * a.Hkv <= a.pf_slots) break;
        if (tries >= 12) {
          Tp = 0x3FFFFFFF;
          break;
        }
        Tp *= 2;
      }
    }
    if (lane == 0) {
      s_tp = Tp;
      s_slot_next = 0;
      s_merge_next = 0;
    }
  }
  __syncthreads();
  const int Tp = s_tp;

  // ---- chunk size ----
  int C = a.part_tokens;
  if (C <= 0) {
    // one chunk per decode wave of the least-served KV head
    const long long waves = (long long)a.dec_grid * 4 / a.Hkv;
    long long c = (total_keys + waves - 1) / waves;
    c = (c + 15) / 16 * 16;
    C = (int)(c < a.part_min ? a.part_min : (c > a.part_max ? a.part_max : c));
  }
  const long long chunks = (total_keys + C - 1) / C;

  // ---- pass 2: decode rows, their offsets on the key axis, chunk starts ----
  int row_base = 0, off_base = 0;
  for (int c0 = 0; c0 < a.S; c0 += kPlanThreads) {
    const int s = c0 + tid;
    SeqShape sh{0, 0, 0};
    int is_dec = 0, pad = 0;
    if (s < a.S) {
      sh = shape(s);
      if (sh.L == 1 && sh.n >= 1) {
        is_dec = 1;
        pad = (sh.n + A - 1) / A * A;
      }
    }
    int nrows, npad;
    const int ri = row_base + block_exclusive_scan(is_dec, s_buf, &nrows);
    const int off = off_base + block_exclusive_scan(pad, s_buf, &npad);
    if (s < a.S) {
      int np = 0;
      if (is_dec) {
        const int j0 = off / C, j1 = (off + pad - 1) / C;
        np = j1 - j0 + 1;
        dec_rows[ri] = make_int4(s, off, sh.n, sh.q0);
        // chunks whose first key falls in this row start here
        for (int j = (off + C - 1) / C; j <= j1; ++j)
          if (j < cap_dec) first_row[j] = ri;
      }
      nparts_of[s] = np;
    }
    row_base += nrows;
    off_base += npad;
  }

  // ---- entries per cost bin: piece j of an item of t tiles cut into J has
  // (j + 1) t / J - j t / J tiles ----
  for (int i = tid; i < kCostBins; i += kPlanThreads) s_hist[i] = 0;
  __syncthreads();
  for (int s = wid; s < a.S; s += kPlanWaves) {
    const SeqShape sh = shape(s);
    if (sh.L > 1 && sh.n >= sh.L) {
      const int ntiles = (sh.L + TM - 1) / TM;
      for (int mt = lane; mt < ntiles; mt += 64) {
        const int t = item_tiles(sh, mt, TM), J = item_pieces(t, Tp);
        for (int j = 0; j < J; ++j) atomicAdd(&s_hist[(j + 1) * t / J - j * t / J], 1);
      }
    }
  }
  __syncthreads();

  // ---- bin offsets in decreasing cost: bin b starts after all bins > b ----
  int pf_total = 0;
  // (kCostBins = 2 * kPlanThreads: each thread owns bins 2t and 2t+1 of the
  // reversed order)
  {
    const int r0 = 2 * tid, r1 = 2 * tid + 1;  // positions in decreasing-cost order
    const int b0 = kCostBins - 1 - r0, b1 = kCostBins - 1 - r1;
    const int h0 = s_hist[b0], h1 = s_hist[b1];
    const int off = block_exclusive_scan(h0 + h1, s_buf, &pf_total);
    s_cur[b0] = off;
    s_cur[b1] = off + h0;
  }
  __syncthreads();

  // ---- pass 3: scatter the prefill entries into their bins (wave per
  // sequence); a cut item takes J * Hkv partial slots ----
  for (int s = wid; s < a.S; s += kPlanWaves) {
    const SeqShape sh = shape(s);
    if (sh.L > 1 && sh.n >= sh.L) {
      const int ntiles = (sh.L + TM - 1) / TM;
      for (int mt = lane; mt < ntiles; mt += 64) {
        const int t = item_tiles(sh, mt, TM), J = item_pieces(t, Tp);
        int slot = 0;
        if (J > 1) {
          slot = atomicAdd(&s_slot_next, J * a.Hkv);
          const int m = atomicAdd(&s_merge_next, 1);
          if (m < cap_pf) merge_items[m] = make_int4(s, mt, J, slot);
        }
        for (int j = 0; j < J; ++j) {
          const int idx = atomicAdd(&s_cur[(j + 1) * t / J - j * t / J], 1);
          if (idx < cap_pf) pf_items[idx] = make_int4(s, mt, j | (J << 16), slot);
        }
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    plan[0] = row_base;
    plan[1] = min(pf_total, cap_pf);
    plan[2] = C;
    plan[3] = (int)(chunks < cap_dec ? chunks : cap_dec);
    plan[4] = A;
    plan[5] = min(s_merge_next, cap_pf);
    for (int i = 6; i < kPlanLine; ++i) plan[i] = 0;
  }
  for (int h = tid; h < a.Hkv; h += kPlanThreads) {
    plan[plan_pf_cursor(h)] = 0;
  }
}

}  // namespace

hipError_t launch_plan(const AttnArgs& a, int* plan, int cap_dec, int cap_pf, int TM,
                       hipStream_t s) {
  profile_before("plan", s);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a, plan, cap_dec, cap_pf,
                     TM);
  profile_after(s);
  return hipGetLastError();
}

}  // namespace pa
