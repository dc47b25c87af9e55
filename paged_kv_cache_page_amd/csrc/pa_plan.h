// The tick's work plan, computed on the device by one wave: shared by the
// plan kernel and the page-write kernel that also plans (the tick's forward).
//
// The host knows only upper bounds (max_query_len, max_seq_len); the lengths of
// the tick's sequences live in device memory. Instead of launching a grid over
// every (sequence, tile) pair and letting most workgroups exit, a single wave
// reads query_start_loc and seq_lens and writes compact lists into the
// workspace (one wave: wave-level scans and reductions, no workgroup
// barriers; a 1024-thread version spent most of its time in them):
//   decode rows   every row with query length 1, laid end to end on one key
//                 axis (each row padded to a multiple of A keys), cut into
//                 equal chunks of C keys, one per decode wave: every wave gets
//                 the same work however the lengths are spread (split-KV for
//                 long rows, several short rows per chunk); chunks past one
//                 per wave (a fixed partition size, or chunks capped at the
//                 largest partition) are claimed from a counter. With a fixed
//                 partition size A = C = that size, so a chunk never spans
//                 two rows and a row's partitions depend on the row alone.
//                 A row of several partitions owns that many consecutive
//                 split-KV partial slots. A row whose first page is also
//                 another decode row's first page (a shared prefix, found
//                 with a hash of the rows' first page ids) is marked so that
//                 the decode kernels load its keys through the caches;
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
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// The plan is one wave: its lanes' LDS traffic is ordered by waiting for the
// wave's own LDS operations (no workgroup barrier, which would also wait for
// the workgroup's other waves).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

constexpr int kCostBins = 2048;     // key tiles of a prefill item, capped

// Bin of a page id in the hash of the decode rows' first pages (multiplicative
// hashing, top bits). Two rows in one bin count as sharing: a collision only
// makes a row's loads cached instead of streamed.
__device__ __forceinline__ int page_hash(int pg) {
  static_assert(kCostBins == 2048, "11-bit hash");
  return (int)(((uint32_t)pg * 2654435761u) >> 21);
}

// Inclusive prefix sum over the wave with DPP lane moves (no LDS round
// trips): shifts by 1, 2, 4, 8 within each 16-lane row, then lane 15 of a row
// added to the next row (row_bcast:15, rows 1 and 3) and lane 31 to the upper
// half (row_bcast:31, rows 2 and 3). Lanes a move does not reach read 0.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp0(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp0<0x111, 0xF>(v);  // row_shr:1
  v += dpp0<0x112, 0xF>(v);  // row_shr:2
  v += dpp0<0x114, 0xF>(v);  // row_shr:4
  v += dpp0<0x118, 0xF>(v);  // row_shr:8
  v += dpp0<0x142, 0xA>(v);  // row_bcast:15
  v += dpp0<0x143, 0xC>(v);  // row_bcast:31
  return v;
}

// Exclusive prefix sum over the wave; *total = the wave's sum (uniform).
__device__ __forceinline__ int wave_excl_scan(int v, int* total) {
  const int incl = wave_incl_scan(v);
  *total = __builtin_amdgcn_readlane(incl, 63);
  return incl - v;
}

__device__ __forceinline__ long long wave_sum(long long v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ int wave_sum32(int v) {
  return __builtin_amdgcn_readlane(wave_incl_scan(v), 63);
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off));
  return v;
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

__device__ __forceinline__ bool is_prefill(const SeqShape& sh) { return sh.L > 1 && sh.n >= sh.L; }

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

// Calls f(s, shape, mt) for every prefill item (sequence s, row tile mt of TM
// tokens), one item per lane: the sequences are taken 64 at a time, their
// tile counts scanned over the wave, and then each lane of an item finds its
// sequence by a binary search over the lanes' first item indices (shuffles,
// no LDS), so a wave pass covers up to 64 items of any sequences. Lanes past
// the last item of a pass get no call.
template <typename Shape, typename F>
__device__ __forceinline__ void for_prefill_items(int S, int TM, Shape&& shape, F&& f) {
  const int lane = threadIdx.x & 63;
  for (int c0 = 0; c0 < S; c0 += 64) {
    const int s = c0 + lane;
    SeqShape sh{0, 0, 0};
    if (s < S) sh = shape(s);
    const int nt = (s < S && is_prefill(sh)) ? (sh.L + TM - 1) / TM : 0;
    int total;
    const int first = wave_excl_scan(nt, &total);  // first item of the lane's sequence
    for (int b0 = 0; b0 < total; b0 += 64) {
      const int item = b0 + lane;
      // the last lane whose sequence starts at or before this item (it holds
      // tiles: a lane without tiles shares its first index with the next lane)
      int k = 0;
#pragma unroll
      for (int step = 32; step >= 1; step >>= 1)
        if (k + step < 64 && __shfl(first, k + step) <= item) k += step;
      const SeqShape u{__shfl(sh.L, k), __shfl(sh.n, k), __shfl(sh.q0, k)};
      const int mt = item - __shfl(first, k);
      if (item < total) f(c0 + k, u, mt);
    }
  }
}

// Sequence shapes cached in LDS between the passes: NC sequences (the rest
// are read again from memory), and the per-bin counts, then bin offsets.
template <int NC>
struct alignas(16) PlanLds {
  int hist[kCostBins];
  int L[NC], n[NC], q0[NC];
  int slot_next, merge_next;
};

// The plan, run by one wave (lanes 0..63 of the calling workgroup; no other
// wave of the workgroup may take part or wait on it).
template <int NC>
__device__ void plan_wave(const AttnArgs& a, int* plan, int cap_dec, int cap_pf, int TM,
                          PlanLds<NC>& sm) {
  int* s_hist = sm.hist;
  int* s_cur = sm.hist;  // bin offsets replace the counts in place
  int* s_L = sm.L;
  int* s_n = sm.n;
  int* s_q0 = sm.q0;
  int& s_slot_next = sm.slot_next;
  int& s_merge_next = sm.merge_next;
  constexpr int kCachedSeqs = NC;
  const int lane = threadIdx.x & 63;
  const PlanOffsets po = plan_offsets(a.S, a.Hq, cap_dec, cap_pf);
  int4* dec_rows = reinterpret_cast<int4*>(plan + po.rows);
  int* nparts_of = plan + po.nparts;
  int* pbase_of = plan + po.pbase;
  int* first_row = plan + po.first_row;
  int4* pf_items = reinterpret_cast<int4*>(plan + po.pf);
  int4* pf_shapes = reinterpret_cast<int4*>(plan + po.pf_shape);
  int4* merge_items = reinterpret_cast<int4*>(plan + po.merge);
  // fixed partitions: rows padded to whole partitions; otherwise to 16 keys
  const int A = a.part_tokens > 0 ? a.part_tokens : 16;
  auto shape = [&](int s) {
    return s < kCachedSeqs ? SeqShape{s_L[s], s_n[s], s_q0[s]} : seq_shape(a, s);
  };

  for (int i = lane; i < kCostBins / 4; i += 64)
    reinterpret_cast<int4*>(s_hist)[i] = make_int4(0, 0, 0, 0);
  if (lane == 0) {
    s_slot_next = 0;
    s_merge_next = 0;
  }

  // ---- pass 1: shapes, padded decode keys (the key axis fits an int: the
  // caller's bounds are checked on the host), and the decode rows' first
  // pages counted in a hash of page ids (the bins array, not yet in use) ----
  int my_keys = 0;
  for (int s = lane; s < a.S; s += 64) {
    // (the first block-table entry is read for every row, so that its load
    // goes out with the shape's instead of after them)
    const int fp = a.block_tables[(size_t)s * a.max_blocks];
    const SeqShape sh = seq_shape(a, s);
    if (s < kCachedSeqs) {
      s_L[s] = sh.L;
      s_n[s] = sh.n;
      s_q0[s] = sh.q0;
    }
    if (sh.L == 1 && sh.n >= 1) {
      my_keys += (sh.n + A - 1) / A * A;
      atomicAdd(&s_hist[page_hash(fp)], 1);
    }
  }
  const int total_keys = wave_sum32(my_keys);  // length of the decode key axis
  wave_lds_sync();

  // ---- chunk size of the decode key axis: one chunk per decode wave of the
  // least-served KV head; chunks past that count (from a fixed partition size,
  // or chunks capped at the largest partition) are claimed from a counter ----
  // (32-bit unsigned divisions: the 64-bit ones are long software routines)
  const unsigned waves = (unsigned)max(1, a.dec_grid * 4 / a.Hkv);
  const unsigned tk = (unsigned)total_keys;
  const unsigned dec_share = (tk + waves - 1u) / waves;  // keys per decode wave (no overflow)
  int C = a.part_tokens;
  if (C <= 0) {
    const unsigned c = (dec_share + 15u) / 16u * 16u;
    C = (int)(c < (unsigned)a.part_min ? (unsigned)a.part_min
                                       : (c > (unsigned)a.part_max ? (unsigned)a.part_max : c));
  }
  int chunks = (int)((tk + (unsigned)C - 1u) / (unsigned)C);
  if (chunks > cap_dec) chunks = cap_dec;  // (never: the workspace query bounds the chunks)
  const int n_static = chunks < (int)waves ? chunks : (int)waves;

  // ---- pass 2: decode rows, their offsets on the key axis, chunk starts,
  // partial slots (rows of more than one partition) ----
  int row_base = 0, off_base = 0, slot_base = 0;
  for (int c0 = 0; c0 < a.S; c0 += 64) {
    const int s = c0 + lane;
    SeqShape sh{0, 0, 0};
    int is_dec = 0, pad = 0, fp = 0;
    if (s < a.S) {
      fp = a.block_tables[(size_t)s * a.max_blocks];
      sh = shape(s);
      if (sh.L == 1 && sh.n >= 1) {
        is_dec = 1;
        pad = (sh.n + A - 1) / A * A;
      }
    }
    int nrows, npad;
    const int ri = row_base + wave_excl_scan(is_dec, &nrows);
    const int off = off_base + wave_excl_scan(pad, &npad);
    int np = 0, j0 = 0, j1 = -1;
    if (is_dec) {
      j0 = off / C;
      j1 = (off + pad - 1) / C;
      np = j1 - j0 + 1;
    }
    int nslots;
    const int pb = slot_base + wave_excl_scan(np > 1 ? np : 0, &nslots);
    if (is_dec) {
      // the row's first page is read by another decode row too (bit 30 of
      // the sequence index, which the host bounds below 2^30): its keys are
      // loaded into the caches as usual, the others' as a stream
      const int shared = s_hist[page_hash(fp)] > 1 ? kRowShared : 0;
      dec_rows[ri] = make_int4(s | shared, off, sh.n, sh.q0);
      nparts_of[ri] = np;
      pbase_of[ri] = pb;
      // chunks whose first key falls in this row start here
      for (int j = (off + C - 1) / C; j <= j1; ++j)
        if (j < cap_dec) first_row[j] = ri;
    }
    row_base += nrows;
    off_base += npad;
    slot_base += nslots;
  }

  // the bins are free again: zero them for the prefill items' tile counts
  wave_lds_sync();
  for (int i = lane; i < kCostBins / 4; i += 64)
    reinterpret_cast<int4*>(s_hist)[i] = make_int4(0, 0, 0, 0);
  wave_lds_sync();

  // ---- prefill items: key tiles (histogram, sum, max) ----
  long long my_tiles = 0;
  int my_maxt = 0;
  for_prefill_items(a.S, TM, shape, [&](int, const SeqShape& sh, int mt) {
    const int t = item_tiles(sh, mt, TM);
    atomicAdd(&s_hist[t], 1);
    my_tiles += t;
    my_maxt = max(my_maxt, t);
  });
  const long long item_tiles_all = wave_sum(my_tiles);  // per KV head
  const int maxt = wave_max(my_maxt);
  wave_lds_sync();

  // ---- piece length Tp: the mean tile count per prefill workgroup, but no
  // less than the time a decode wave spends on its chunk (items shorter than
  // that finish while the decode rows stream anyway, and cutting them only
  // adds partials), doubled until the cut items' partials (J slots per item
  // and KV head) fit ----
  int Tp = 0x3FFFFFFF;  // never cut
  if (a.pf_slots > 0 && a.part_tokens == 0 && item_tiles_all > 0) {
    const long long w = a.pf_workers > 0 ? a.pf_workers : 1;
    long long t0 = (long long)(((double)item_tiles_all * a.Hkv + (double)(w - 1)) / (double)w);
    if (total_keys > 0)
      t0 = max(t0, (long long)((dec_share + kDecodeKeysPerTile - 1) / kDecodeKeysPerTile));
    Tp = (int)(t0 < kMinPieceTiles ? kMinPieceTiles : (t0 > kCostBins ? kCostBins : t0));
    for (int tries = 0;; ++tries) {
      long long need = 0;
      for (int b = lane; b <= maxt; b += 64) {
        const int J = item_pieces(b, Tp);
        if (J > 1) need += (long long)s_hist[b] * J;
      }
      if (wave_sum(need) * a.Hkv <= a.pf_slots) break;
      if (tries >= 12) {
        Tp = 0x3FFFFFFF;
        break;
      }
      Tp *= 2;
    }
  }

  // ---- entries per cost bin: piece j of an item of t tiles cut into J has
  // (j + 1) t / J - j t / J tiles (when nothing is cut, the item histogram
  // already is that) ----
  if (Tp < maxt) {
    for (int b = lane; b <= maxt; b += 64) s_hist[b] = 0;
    wave_lds_sync();
    for_prefill_items(a.S, TM, shape, [&](int, const SeqShape& sh, int mt) {
      const int t = item_tiles(sh, mt, TM), J = item_pieces(t, Tp);
      for (int j = 0; j < J; ++j) atomicAdd(&s_hist[(j + 1) * t / J - j * t / J], 1);
    });
    wave_lds_sync();
  }

  // ---- bin offsets in decreasing cost: bin b starts after all bins > b
  // (written over the counts: each bin is read, then written, by one lane) ----
  int pf_total = 0;
  for (int r0 = 0; r0 <= maxt; r0 += 64) {
    const int r = r0 + lane, b = maxt - r;  // r-th bin in decreasing cost order
    const int h = r <= maxt ? s_hist[b] : 0;
    int tot;
    const int off = pf_total + wave_excl_scan(h, &tot);
    if (r <= maxt) s_cur[b] = off;
    pf_total += tot;
  }
  wave_lds_sync();

  // ---- scatter the prefill entries into their bins; a cut item takes
  // J * Hkv partial slots ----
  for_prefill_items(a.S, TM, shape, [&](int s, const SeqShape& sh, int mt) {
    const int t = item_tiles(sh, mt, TM), J = item_pieces(t, Tp);
    int slot = 0;
    if (J > 1) {
      slot = atomicAdd(&s_slot_next, J * a.Hkv);
      const int m = atomicAdd(&s_merge_next, 1);
      if (m < cap_pf) merge_items[m] = make_int4(s, mt, J, slot);
    }
    for (int j = 0; j < J; ++j) {
      const int idx = atomicAdd(&s_cur[(j + 1) * t / J - j * t / J], 1);
      if (idx < cap_pf) {
        pf_items[idx] = make_int4(s, mt, j | (J << 16), slot);
        pf_shapes[idx] = make_int4(sh.q0, sh.L, sh.n, 0);
      }
    }
  });
  wave_lds_sync();
  if (lane == 0) {
    plan[0] = row_base;
    plan[1] = min(pf_total, cap_pf);
    plan[2] = C;
    plan[3] = (int)chunks;
    plan[4] = A;
    plan[5] = min(s_merge_next, cap_pf);
    plan[6] = n_static;
    plan[7] = ((int)chunks - n_static) * a.Hkv;
    plan[plan_dec_cursor(a.Hq)] = 0;
  }
  for (int i = 8 + lane; i < kPlanLine; i += 64) plan[i] = 0;
  for (int h = lane; h < a.Hkv; h += 64) plan[plan_pf_cursor(h)] = 0;
}


}  // namespace pa
