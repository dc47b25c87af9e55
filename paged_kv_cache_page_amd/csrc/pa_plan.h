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
// wave's own LDS operations (lgkmcnt 0; the vmcnt and expcnt fields at their
// maxima, so the plan's global stores stay in flight: a workgroup-scope fence
// would wait for them at every step), with compiler barriers on both sides
// and no workgroup barrier (which would also wait for the other waves).
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

constexpr int kCostBins = 2048;     // key tiles of a prefill item, capped
// Leading pages compared when grouping rows by a shared prefix.
constexpr int kGroupMaxPages = 1024;
constexpr int kGroupFirstPages = 16;  // of them, read with the rows' shapes

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

__device__ __forceinline__ int wave_sum32(int v) {
  return __builtin_amdgcn_readlane(wave_incl_scan(v), 63);
}

// Sum over the wave of non-negative per-lane values below 2^48 (uniform):
// the low 24 and the high bits summed apart in 32 bits, each sum below 2^30.
__device__ __forceinline__ long long wave_sum(long long v) {
  const int lo = wave_sum32((int)(v & 0xFFFFFF)), hi = wave_sum32((int)(v >> 24));
  return ((long long)hi << 24) + lo;
}

// Maximum over the wave of non-negative values (uniform): the moves of the
// prefix sum, with max in place of +; lanes a move does not reach read 0.
__device__ __forceinline__ int wave_max(int v) {
  v = max(v, dpp0<0x111, 0xF>(v));
  v = max(v, dpp0<0x112, 0xF>(v));
  v = max(v, dpp0<0x114, 0xF>(v));
  v = max(v, dpp0<0x118, 0xF>(v));
  v = max(v, dpp0<0x142, 0xA>(v));
  v = max(v, dpp0<0x143, 0xC>(v));
  return __builtin_amdgcn_readlane(v, 63);
}

// For each lane with `on`, the mask of the lanes with `on` holding the same
// value v (0 for the others): one round per distinct value, each taking the
// value of the lowest lane still unmatched.
__device__ __forceinline__ unsigned long long wave_match(int v, bool on) {
  unsigned long long todo = __ballot(on), mine = 0;
  while (todo != 0) {
    const int u = __builtin_amdgcn_readlane(v, __ffsll((long long)todo) - 1);
    const unsigned long long m = __ballot(on && v == u);
    if (on && v == u) mine = m;
    todo &= ~m;
  }
  return mine;
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
  int grp[4][64];  // per-lane values of the decode row groups (one wave pass)
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
  int fp0 = 0;  // (at most 64 sequences) the lane's sequence: first page and shape
  SeqShape sh0{0, 0, 0};
  // Rows may be grouped by a shared prefix (below): then the lane's first
  // kGroupFirstPages page ids are read here too, beside the shape's loads
  const int Gq = a.Hq / a.Hkv;
  const int Rmax = Gq > 0 ? 16 / Gq : 0;  // a power of two: G divides 16
  const bool may_group = a.group_rows && a.part_tokens == 0 && a.S <= 64 && Rmax >= 2;
  int bt0[kGroupFirstPages];
#pragma unroll
  for (int j = 0; j < kGroupFirstPages; ++j) bt0[j] = -1;
  for (int s = lane; s < a.S; s += 64) {
    // (the first block-table entry is read for every row, so that its load
    // goes out with the shape's instead of after them)
    const int* bt = a.block_tables + (size_t)s * a.max_blocks;
    const int fp = bt[0];
    if (may_group) {
#pragma unroll
      for (int j = 0; j < kGroupFirstPages; ++j) bt0[j] = j < a.max_blocks ? bt[j] : -1;
    }
    const SeqShape sh = seq_shape(a, s);
    if (s < kCachedSeqs) {
      s_L[s] = sh.L;
      s_n[s] = sh.n;
      s_q0[s] = sh.q0;
    }
    if (s == lane) {
      fp0 = fp;
      sh0 = sh;
    }
    if (sh.L == 1 && sh.n >= 1) {
      my_keys += (sh.n + A - 1) / A * A;
      atomicAdd(&s_hist[page_hash(fp)], 1);
    }
  }
  int total_keys = wave_sum32(my_keys);  // length of the decode key axis
  wave_lds_sync();

  // ---- chunk size of the decode key axis: one chunk per decode wave of the
  // least-served KV head; chunks past that count (from a fixed partition size,
  // or chunks capped at the largest partition) are claimed from a counter ----
  // (32-bit unsigned divisions: the 64-bit ones are long software routines)
  const unsigned waves = (unsigned)max(1, a.dec_grid * 4 / a.Hkv);
  int C = 0, chunks = 0;
  unsigned dec_share = 0;  // keys per decode wave
  auto chunking = [&](int tkeys) {
    const unsigned tk = (unsigned)tkeys;
    dec_share = (tk + waves - 1u) / waves;  // (no overflow)
    C = a.part_tokens;
    if (C <= 0) {
      const unsigned c = (dec_share + 15u) / 16u * 16u;
      C = (int)(c < (unsigned)a.part_min ? (unsigned)a.part_min
                                         : (c > (unsigned)a.part_max ? (unsigned)a.part_max : c));
    }
    chunks = (int)((tk + (unsigned)C - 1u) / (unsigned)C);
    if (chunks > cap_dec) chunks = cap_dec;  // (never: the workspace query bounds the chunks)
  };
  // partitions of the axis range [o, o + len)
  auto parts = [&](int o, int len) { return (o + len - 1) / C - o / C + 1; };
  int* kstart_of = plan + po.kstart;
  int* part0_of = plan + po.part0;
  // chunks whose first key falls in axis range [o, o + len) start in row ri
  auto chunk_starts = [&](int o, int len, int ri) {
    for (int j = (o + C - 1) / C; j <= (o + len - 1) / C; ++j)
      if (j < cap_dec) first_row[j] = ri;
  };

  // ---- decode rows grouped by a shared prefix (bf16 matrix-core decode,
  // automatic partitions, at most 64 sequences: one lane per sequence) ----
  // A decode row whose first page id is another decode row's (the hash bins
  // above, confirmed on the ids) shares a prefix with the one of smallest
  // index among them, its leader: the leading pages on which their page
  // tables agree, but no page holding the row's last key. The rows of one
  // leader and one prefix length are cut, in lane order, into groups of at
  // most 16 / G rows (the columns of one score product). A group of two or
  // more rows reads the prefix once: a group row, laid before its members'
  // rows, whose every partition gives one partial per member; each member's
  // own row then covers its keys after the prefix, and the merge sums both.
  // The leader itself keeps its whole row (loaded through the caches).
  // Layout on the key axis, in lane order of the units: an ungrouped row is
  // one unit; a group (at its first member's lane) is the group row's prefix
  // keys, then each member's keys after the prefix, in lane order. Each lane
  // computes its own row; groups are found with ballots (one round per
  // distinct first page, then per distinct prefix) and their sums pass
  // through LDS (a group's last member holds them).
  bool grouped = false;
  int row_base_g = 0;  // decode rows of the grouped list
  const bool dec0 = lane < a.S && sh0.L == 1 && sh0.n >= 1;
  const bool shared0 = dec0 && s_hist[page_hash(fp0)] > 1;
  if (may_group && __ballot(shared0) != 0) {
    const int s = lane;
    const unsigned long long below = (1ull << s) - 1ull;
    const unsigned long long same_fp = wave_match(fp0, shared0);  // (in every lane: ballots)
    const int lead = shared0 ? __ffsll((long long)same_fp) - 1 : s;
    // leading page ids equal to the leader's: the first kGroupFirstPages
    // from the leader's lane, then eight per round from memory
    const bool follower = shared0 && lead != s;
    const int cap_pages = follower ? min((sh0.n - 1) >> a.p_shift, kGroupMaxPages) : 0;
    int lp_pages = 0;
    bool run = true;
#pragma unroll
    for (int j = 0; j < kGroupFirstPages; ++j) {
      const int vl = __shfl(bt0[j], lead);  // (every lane takes part in the shuffle)
      if (run && j < cap_pages && bt0[j] == vl) ++lp_pages;
      else run = false;
    }
    if (run && cap_pages > kGroupFirstPages) {
      const int* bs = a.block_tables + (size_t)s * a.max_blocks;
      const int* bl = a.block_tables + (size_t)lead * a.max_blocks;
      for (int p0 = kGroupFirstPages; p0 < cap_pages; p0 += 8) {
        int vs[8], vl[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          vs[j] = p0 + j < cap_pages ? bs[p0 + j] : 0;
          vl[j] = p0 + j < cap_pages ? bl[p0 + j] : 1;
        }
        int eq = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (eq == j && vs[j] == vl[j]) ++eq;
        lp_pages += eq;
        if (eq < 8) break;
      }
    }
    // rows of one leader and one prefix length: their rank decides the group
    // (bits: group index 0..4, prefix pages 5..15, leader 16..21)
    const bool cand = lp_pages >= 1;
    const int key = (lead << 16) | (lp_pages << 5);
    const unsigned long long same = wave_match(key, cand);
    const int lg = 31 - __builtin_clz(Rmax);
    const int rank = __popcll(same & below), size = __popcll(same);
    const int sg = rank >> lg;
    const bool member = cand && min(Rmax, size - (sg << lg)) >= 2;
    const unsigned long long gm = wave_match(key | sg, member);  // the group's lanes
    grouped = __ballot(member) != 0;
    if (grouped) {
      int* s_pm = sm.grp[0];    // a member's keys after the prefix (padded)
      int* s_np = sm.grp[1];    // a member's own partitions
      int* s_gk = sm.grp[2];    // (first member) the group's keys after the prefix
      int* s_gs = sm.grp[3];    // (first member) the group's partial slots
      const int first = member ? __ffsll((long long)gm) - 1 : s;
      const bool last = member && (gm >> s) == 1ull;
      const int idx = __popcll(gm & below), gsize = __popcll(gm);
      const int g_lp = lp_pages << a.p_shift;
      const int pm = member ? (sh0.n - g_lp + A - 1) / A * A : 0;
      if (member) s_pm[s] = pm;
      wave_lds_sync();
      int kpre = 0;  // keys of the group's members before this one
      for (unsigned long long m = gm & below; m != 0; m &= m - 1ull)
        kpre += s_pm[__ffsll((long long)m) - 1];
      if (last) s_gk[first] = kpre + pm;
      wave_lds_sync();
      const bool own = dec0 && !member;
      const bool head = member && first == s;
      const int len = own ? (sh0.n + A - 1) / A * A : (head ? g_lp + s_gk[s] : 0);
      const int nemit = own ? 1 : (head ? 1 + gsize : 0);
      int nkeys, nrows;
      const int off = wave_excl_scan(len, &nkeys);
      const int ri = wave_excl_scan(nemit, &nrows);
      chunking(nkeys);
      // (every lane takes part in the shuffles)
      const int off_g = __shfl(off, first), ri_g = __shfl(ri, first);
      const int o_m = off_g + g_lp + kpre;  // a member's own keys on the axis
      const int kg = member ? parts(off_g, g_lp) : 0;  // the group row's partitions
      const int npm = member ? parts(o_m, pm) : 0;
      if (member) s_np[s] = npm;
      wave_lds_sync();
      int npre = 0;  // own partitions of the group's members before this one
      for (unsigned long long m = gm & below; m != 0; m &= m - 1ull)
        npre += s_np[__ffsll((long long)m) - 1];
      if (last) s_gs[first] = (idx + 1) * kg + npre + npm;
      wave_lds_sync();
      const int np_own = own ? parts(off, len) : 0;
      const int slots = own ? (np_own > 1 ? np_own : 0) : (head ? s_gs[s] : 0);
      int nslots;
      const int pb = wave_excl_scan(slots, &nslots);
      const int pb_g = __shfl(pb, first);
      // group only while the partial slots fit the workspace (a member holds
      // its group row's partials and its own)
      if (nslots > a.part_slots) {
        grouped = false;
      } else {
        if (own) {
          dec_rows[ri] = make_int4(s | (shared0 ? kRowShared : 0), off, sh0.n, sh0.q0);
          nparts_of[ri] = np_own;
          pbase_of[ri] = pb;
          kstart_of[ri] = 0;
          part0_of[ri] = 0;
          chunk_starts(off, len, ri);
        }
        if (head) {
          // the group row: the leader's page table holds the prefix
          dec_rows[ri] = make_int4(lead | kRowShared | kRowGroup, off, g_lp, gsize);
          nparts_of[ri] = 0;
          pbase_of[ri] = 0;
          kstart_of[ri] = 0;
          part0_of[ri] = 0;
          chunk_starts(off, g_lp, ri);
        }
        if (member) {
          const int rm = ri_g + 1 + idx;
          dec_rows[rm] = make_int4(s, o_m, sh0.n - g_lp, sh0.q0);
          nparts_of[rm] = kg + npm;
          pbase_of[rm] = pb_g + idx * kg + npre;
          kstart_of[rm] = g_lp;
          part0_of[rm] = kg;
          chunk_starts(o_m, pm, rm);
        }
        row_base_g = nrows;
      }
    }
  }
  if (!grouped) chunking(total_keys);
  const int n_static = chunks < (int)waves ? chunks : (int)waves;

  // ---- pass 2: decode rows, their offsets on the key axis, chunk starts,
  // partial slots (rows of more than one partition) ----
  int row_base = 0, off_base = 0, slot_base = 0;
  if (grouped) {
    row_base = row_base_g;
  } else {
  for (int c0 = 0; c0 < a.S; c0 += 64) {
    const int s = c0 + lane;
    SeqShape sh{0, 0, 0};
    int is_dec = 0, pad = 0, fp = 0;
    if (s < a.S) {
      // (at most 64 sequences: pass 1's loads, still in registers)
      fp = a.S <= 64 ? fp0 : a.block_tables[(size_t)s * a.max_blocks];
      sh = a.S <= 64 ? sh0 : shape(s);
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
      // the sequence index, which the host bounds below 2^29): its keys are
      // loaded into the caches as usual, the others' as a stream
      const int shared = s_hist[page_hash(fp)] > 1 ? kRowShared : 0;
      dec_rows[ri] = make_int4(s | shared, off, sh.n, sh.q0);
      nparts_of[ri] = np;
      pbase_of[ri] = pb;
      kstart_of[ri] = 0;
      part0_of[ri] = 0;
      // chunks whose first key falls in this row start here
      for (int j = (off + C - 1) / C; j <= j1; ++j)
        if (j < cap_dec) first_row[j] = ri;
    }
    row_base += nrows;
    off_base += npad;
    slot_base += nslots;
  }
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
