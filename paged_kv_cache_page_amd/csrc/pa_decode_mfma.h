// bf16 decode work items on matrix cores, the walk of a decode worker over its
// chunks of the decode key axis, and the merge of split-KV partitions. Shared
// by the decode kernels and the fused tick kernel.
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// bf16 decode: resident workgroups per CU. One workgroup per CU keeps the
// waves of a CU the same age: the wave arbiter favours older waves, and with
// several workgroups per CU the younger ones' loads queue behind the older
// ones' and the kernel ends on a tail of late waves.
constexpr int kDecodeWgPerCu = 1;

// Which row a work item serves, and that row's key limit.
struct RowInfo {
  int seq;      // sequence index
  int token;    // row of q / out
  int n_eff;    // keys this row attends: 0 .. n_eff - 1
  bool active;
};

template <bool TOKEN_MODE>
__device__ __forceinline__ RowInfo row_info(const AttnArgs& a, int row) {
  RowInfo r;
  r.active = false;
  int s, L, i;
  if constexpr (TOKEN_MODE) {
    int lo = 0, hi = a.S;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.qsl[mid] <= row) lo = mid; else hi = mid;
    }
    s = lo;
    const int q0 = a.qsl[s];
    L = a.qsl[s + 1] - q0;
    i = row - q0;
    r.token = row;
    if (i < 0 || i >= L) return r;
  } else {
    s = row;
    const int q0 = a.qsl[s];
    L = a.qsl[s + 1] - q0;
    i = 0;
    r.token = q0;
    if (L != 1 || q0 < 0 || q0 >= a.T) return r;
  }
  // Keys beyond the block table or beyond max_seq_len are never read (the
  // caller promised neither happens; this keeps every index in range if not).
  int n = a.seq_lens[s];
  n = min(n, a.max_blocks * a.P);
  n = min(n, a.max_seq_len);
  r.seq = s;
  r.n_eff = n - L + i + 1;
  r.active = r.n_eff > 0;
  return r;
}

// K3: merge of a row's split-KV partitions, m* = max_k m_k,
// o = sum_k 2^(m_k - m*) o_k / sum_k 2^(m_k - m*) l_k. Thread idx =
// kMergeLanes (row, query head, 4 consecutive dims) + lane: the kMergeLanes
// adjacent lanes of a group take every kMergeLanes-th partition (m* taken as
// a running maximum, the sums rescaled when it grows), then combine their
// three values the same way with lane exchanges (xor 1, then xor 2), so that
// a row of many partitions waits for a quarter of the dependent loads.
constexpr int kMergeLanes = 4;

template <typename ET, bool TOKEN_MODE>
__device__ __forceinline__ void split_reduce_task(const AttnArgs& a, long idx) {
  const int D = a.D;
  const int quads = D / 4;
  const int lane_k = (int)(idx % kMergeLanes);
  idx /= kMergeLanes;
  const int d4 = (int)(idx % quads);
  const long rh = idx / quads;
  const int h = (int)(rh % a.Hq);
  const long row = rh / a.Hq;
  if (row >= (TOKEN_MODE ? (long)a.T : plan_rows(a.S))) return;
  int nparts, token;
  size_t slot0;  // partial slot of part 0
  if constexpr (TOKEN_MODE) {
    const RowInfo ri = row_info<true>(a, (int)row);
    if (!ri.active) return;
    nparts = (ri.n_eff + a.part_tokens - 1) / a.part_tokens;
    nparts = min(nparts, a.max_parts);
    token = (int)row;
    slot0 = (size_t)row * a.max_parts;
  } else {
    // row = decode row of the plan. The four loads are independent (entries
    // past the plan's rows hold stale values and are used only once row is
    // known to be a decode row), so they overlap.
    const PlanOffsets po = plan_offsets(a.S, a.Hq, a.cap_dec, a.cap_pf);
    const int n_rows = a.plan[0];
    nparts = a.plan[po.nparts + row];
    token = reinterpret_cast<const int4*>(a.plan + po.rows)[row].w;
    slot0 = (size_t)a.plan[po.pbase + row];
    if (row >= n_rows) return;
  }
  if (nparts <= 1) return;
  const float* ml = a.ws + (size_t)a.part_slots * a.Hq * D;
  const size_t p0 = slot0 * a.Hq + h;  // partial index of part 0
  // one pass with a running max over this lane's partitions: their loads are
  // independent
  float mn = kNegBig, lt = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 2
  for (int k = lane_k; k < nparts; k += kMergeLanes) {
    const size_t pi = p0 + (size_t)k * a.Hq;
    const float2 mlk = *reinterpret_cast<const float2*>(ml + 2 * pi);
    const float4 ok = *reinterpret_cast<const float4*>(a.ws + pi * D + 4 * d4);
    if (mlk.x > mn) {
      const float c = fast_exp2(mn - mlk.x);
      mn = mlk.x;
      lt *= c;
      acc.x *= c;
      acc.y *= c;
      acc.z *= c;
      acc.w *= c;
    }
    const float c = fast_exp2(mlk.x - mn);
    lt = fmaf(mlk.y, c, lt);
    acc.x = fmaf(ok.x, c, acc.x);
    acc.y = fmaf(ok.y, c, acc.y);
    acc.z = fmaf(ok.z, c, acc.z);
    acc.w = fmaf(ok.w, c, acc.w);
  }
  // the group's lanes combined (a lane with no partition holds m = kNegBig,
  // l = 0, o = 0, which the combination weighs with 0 or leaves at 0)
#pragma unroll
  for (int x = 1; x < kMergeLanes; x <<= 1) {
    const float mo = __shfl_xor(mn, x), lo = __shfl_xor(lt, x);
    const float4 ao = make_float4(__shfl_xor(acc.x, x), __shfl_xor(acc.y, x),
                                  __shfl_xor(acc.z, x), __shfl_xor(acc.w, x));
    const float m2 = fmaxf(mn, mo);
    const float ca = fast_exp2(mn - m2), cb = fast_exp2(mo - m2);
    lt = lt * ca + lo * cb;
    acc = make_float4(acc.x * ca + ao.x * cb, acc.y * ca + ao.y * cb, acc.z * ca + ao.z * cb,
                      acc.w * ca + ao.w * cb);
    mn = m2;
  }
  if (lane_k != 0) return;
  const float inv = 1.f / lt;
  const size_t oi = ((size_t)token * a.Hq + h) * D + 4 * d4;
  if constexpr (ET::kBytes == 2) {
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + oi) =
        make_uint2(pack_bf16x2(acc.x * inv, acc.y * inv), pack_bf16x2(acc.z * inv, acc.w * inv));
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + oi) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
}

// One range of a decode row handled by one wave: keys [kbeg, kend) of
// sequence seq for query row token, partition part of the row's nparts (its
// partials at slot pslot + part of the split-KV workspace), KV head kvh.
struct DecSeg {
  int seq, token, pslot, kbeg, kend, part, nparts, kvh;
  int cached = 0;  // the row's keys go through the caches (a shared prefix)
  int group = 0;   // a group row: its members (rows grow + 1 .. grow + group)
  int grow = 0;
};

// Walk of decode wave gw = 4 wg + wave over the chunks of the decode key axis
// the plan kernel cut (see pa_plan.h). Wave gw first takes chunk gw / Hkv
// of KV head gw % Hkv (the four waves of a workgroup serve different heads, so
// every XCD streams several heads' rows at once); chunks past one per wave
// are items t = (chunk, KV head) claimed from one shared counter, t -> head
// t % Hkv, chunk n_static + t / Hkv, until they run out. Each claim is issued one
// chunk ahead, so its atomic returns while the wave streams. next() yields the
// part of every row each chunk covers.
struct DecodeCursor {
  const int4* rows;       // (sequence, offset, keys, token) per decode row
  const int* first_row;   // first row of each chunk
  const int* nparts_of;   // partitions per row
  const int* pbase_of;    // first partial slot per row
  const int* kstart_of;   // first key per row
  const int* part0_of;    // first partition index per row
  int* counter;           // claimed items
  int n_rows, C, n_chunks, n_static, n_items, A, Hkv, kvh, chunk, i;
  int claim;   // item claimed ahead (lane 0)
  bool ended;  // the last range yielded ended its chunk

  __device__ __forceinline__ void claim_next() {
    claim = n_items;
    if (n_items > 0 && (threadIdx.x & 63) == 0)
      claim = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // Move to the claimed item (or past the last chunk when none is left).
  __device__ __forceinline__ void take_claim() {
    const int t = __builtin_amdgcn_readfirstlane(claim);
    if (t < n_items) {
      kvh = t % Hkv;
      chunk = n_static + t / Hkv;
      i = first_row[chunk];
      claim_next();
    } else {
      chunk = n_chunks;
    }
  }

  __device__ __forceinline__ DecodeCursor(const AttnArgs& a, int wg) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const PlanOffsets po = plan_offsets(a.S, a.Hq, a.cap_dec, a.cap_pf);
    rows = reinterpret_cast<const int4*>(a.plan + po.rows);
    first_row = a.plan + po.first_row;
    nparts_of = a.plan + po.nparts;
    pbase_of = a.plan + po.pbase;
    kstart_of = a.plan + po.kstart;
    part0_of = a.plan + po.part0;
    counter = a.plan + plan_dec_cursor(a.Hq);
    n_rows = a.plan[0];
    C = a.plan[2];
    n_chunks = a.plan[3];
    A = a.plan[4];
    n_static = a.plan[6];
    n_items = a.plan[7];
    Hkv = a.Hkv;
    const int gw = wg * 4 + wave;
    kvh = gw % Hkv;
    chunk = gw / Hkv;
    i = 0;
    ended = false;
    claim_next();
    if (chunk < n_static)
      i = first_row[chunk];
    else
      take_claim();
  }

  // (A chunk's end is acted on at the following call, so the claim taken
  // there has had a whole range's time to return.)
  __device__ __forceinline__ bool next(DecSeg& d) {
    for (;;) {
      if (ended) {
        take_claim();
        ended = false;
      }
      if (chunk >= n_chunks) return false;
      const int4 r = rows[i];
      const int np = nparts_of[i], pb = pbase_of[i], k0 = kstart_of[i], p0 = part0_of[i];
      const int off = r.y, n = r.z;  // the row's keys: [k0, k0 + n) of the sequence
      const int pad = (n + A - 1) / A * A;
      const int c0 = chunk * C, c1 = c0 + C;
      d.seq = r.x & (kRowGroup - 1);
      d.cached = (r.x & kRowShared) != 0;
      d.group = (r.x & kRowGroup) ? r.w : 0;
      d.grow = i;
      d.token = r.w;
      d.pslot = pb;
      d.kbeg = max(c0, off) - off + k0;
      d.kend = min(min(c1, off + pad) - off, n) + k0;
      d.part = chunk - off / C + p0;
      d.nparts = np;
      d.kvh = kvh;
      if (off + pad >= c1 || i + 1 >= n_rows)  // the chunk ends in this row
        ended = true;
      else
        ++i;
      if (d.kbeg < d.kend) return true;
    }
  }
};

// seg(seq, token, pslot, kbeg, kend, part, nparts, kvh) for every range of the
// wave's chunks, in order.
template <typename Seg>
__device__ __forceinline__ void decode_walk(const AttnArgs& a, int wg, Seg&& seg) {
  DecodeCursor cur(a, wg);
  DecSeg d;
  while (cur.next(d)) seg(d.seq, d.token, d.pslot, d.kbeg, d.kend, d.part, d.nparts, d.kvh);
}

// ---------------------------------------------------------------------------
// bf16 work item on matrix cores. Per 16-key buffer:
//   S^T[key, head] = K[key, :] . Q[head, :]   v_mfma_f32_16x16x32_bf16, A = K
//   rows in the A layout (lane l: key l % 16, dims 8 (l / 16) + 32 ks ..), B =
//   Q^T (lane l: head l % 16, zero for heads >= G). Lane (r, c) (r = l / 16,
//   c = l % 16) then holds the scores of keys 4r .. 4r + 3 for head c. One
//   running max per head for the whole wave (combined over the four lanes of a
//   head with permlane swaps), so the per-lane sums can be added without
//   rescaling.
//   O^T[dim, head] += V^T[dim, key] . P^T[key, head]   v_mfma_f32_16x16x16_bf16
//   per 16 dims: B = the lane's own bf16 weights (keys 4r .. 4r + 3 of head c:
//   the score layout as it stands), A = V^T, read transposed from LDS with
//   ds_read_b64_tr_b16 (lane (r, c) reads key 4r + c / 4, dims 16 db +
//   4 (c % 4) .. + 3; the instruction exchanges 16-bit elements within each
//   16-lane group so that lane (r, c) receives dim 16 db + c of keys 4r ..
//   4r + 3). The accumulators keep that layout: lane (r, c) holds dims
//   16 db + 4r .. + 3 of head c, final after the last key.
// K and V of a buffer go from HBM straight into the wave's own LDS region
// with global_load_lds_dwordx4 (no registers), two buffers deep: the next
// buffer's loads are in flight while one is computed.
template <int D, int G>
struct MfmaDecodeShape {
  static constexpr int ROWB = D * 2;
  static constexpr int KSTEPS = D / 32;       // k-steps of the score MFMA
  static constexpr int BUF = 16 * ROWB;       // bytes of one 16-key buffer of K (or V)
  static constexpr int NQ = BUF / 1024;       // load instructions per matrix per buffer
  static constexpr int NDMA = 2 * NQ;         // load instructions per buffer (K and V)
  static_assert(D == 64 || D == 128, "bf16 head dims 64 and 128");
  static_assert(G >= 1 && G <= 8, "at most 8 query heads per KV head");
};

// One wave's LDS region: buffers 0 and 1, each K then V.
template <int D>
constexpr int dec_region_bytes() { return 4 * 16 * D * 2; }
template <int D>
constexpr int dec_region_units() { return dec_region_bytes<D>() / 16; }

// K buffer layout, in 16-byte units, of key k, chunk c (8 dims):
//   64 ((D / 64) (k / 8) + c / 8) + 8 (k % 8) + ((c % 8) ^ (k / 2) ^ 4 (k % 2)) % 8
// The operand reads (lane l: key l % 16, chunk 4 ks + l / 16) hit distinct
// banks whether 8 or 16 lanes are served a cycle. A load instruction q fills
// units 64 q .. 64 q + 63 (lane j: unit 64 q + j), so lane j of load q fetches
// the key and chunk that unit holds.
template <int D>
__device__ __forceinline__ int kbuf_unit(int k, int c) {
  return 64 * ((D / 64) * (k >> 3) + (c >> 3)) + 8 * (k & 7) + (((c & 7) ^ (k >> 1) ^ ((k & 1) << 2)) & 7);
}
// V buffer layout: rows of 2 D bytes, the 32-byte blocks of key k's row
// permuted by k % 4 (XOR), so that the transposed reads of four keys' same dims
// hit different banks: unit of key k, chunk c at k (D / 8) + 2 ((c / 2) ^ (k % 4)) + c % 2.

// Where a range's 16-key buffers come from.
struct DecSrc {
  const char* kbase;  // K pool + the KV head's offset within a slot
  const char* vbase;
  int page_raw;       // lane i: block-table entry of the range's i-th page (unchecked)
  int pg0;            // the range's first page
  int kbeg;           // first key (a multiple of 16)
  int nbuf;           // 16-key buffers (>= 1)
  int cached;         // ordinary loads (a shared prefix) instead of streaming ones
};

// Per-lane source offsets of the K and V loads within a 16-key buffer (one
// per load instruction), and the wave's LDS region.
template <int D, int G>
struct DecLane {
  size_t slot_stride;  // bytes between consecutive slots of a page
  uint32_t k_off[MfmaDecodeShape<D, G>::NQ], v_off[MfmaDecodeShape<D, G>::NQ];
  uint32_t lds;        // LDS byte address of the wave's region (wave-uniform)
  char* region;        // the same region as a pointer
};

template <int D, int G>
__device__ __forceinline__ DecLane<D, G> dec_lane(const AttnArgs& a, uint4* region) {
  typedef MfmaDecodeShape<D, G> SH;
  const int j = threadIdx.x & 63;
  DecLane<D, G> l;
  l.slot_stride = (size_t)a.Hkv * SH::ROWB;
#pragma unroll
  for (int q = 0; q < SH::NQ; ++q) {
    // K: the inverse of kbuf_unit for unit 64 q + j
    const int kq = q / (D / 64), cq = q % (D / 64);
    const int k = 8 * kq + (j >> 3);
    const int c = 8 * cq + (((j & 7) ^ (k >> 1) ^ ((k & 1) << 2)) & 7);
    l.k_off[q] = (uint32_t)(k * l.slot_stride) + 16 * c;
    // V: unit 64 q + j of the row-major, block-permuted layout
    const int u = 64 * q + j, key = u / (D / 8), w = u % (D / 8);
    const int cv = 2 * ((w >> 1) ^ (key & 3)) + (w & 1);
    l.v_off[q] = (uint32_t)(key * l.slot_stride) + 16 * cv;
  }
  l.region = reinterpret_cast<char*>(region);
  l.lds = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)l.region);
  return l;
}

template <int D, int G>
__device__ __forceinline__ DecSrc dec_src(const AttnArgs& a, const DecSeg& d, int page_raw) {
  typedef MfmaDecodeShape<D, G> SH;
  DecSrc s;
  s.kbase = (const char*)a.k_pool + (size_t)d.kvh * SH::ROWB;
  s.vbase = (const char*)a.v_pool + (size_t)d.kvh * SH::ROWB;
  s.page_raw = page_raw;
  s.pg0 = d.kbeg >> a.p_shift;
  s.kbeg = d.kbeg;
  s.nbuf = (d.kend - d.kbeg + 15) / 16;
  s.cached = __builtin_amdgcn_readfirstlane(d.cached);
  return s;
}

// (dec_dma16 names M0 in its clobber list, which the compiler reports.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// One 16-byte-per-lane load from global memory (wave-uniform base + per-lane
// 32-bit offset) into LDS (lane j's 16 bytes at byte lds + 16 j; lds in M0).
// Inline assembly, so the compiler's wait insertion does not make later LDS
// reads wait for it: the walk waits for these loads itself (dec_wait). The
// "memory" clobber keeps other memory accesses on their side of it; M0 is
// set right before each compiler use of it and holds nothing across code.
// STREAM marks the load non-temporal (nt): a decode row's K/V rows are read
// once per tick, so the caches need not keep them, and the prefill tiles that
// the fused tick re-reads stay cached instead (measured: decode rows alone
// 88.6 -> 78.6 us, the packed tick's step 132.5 -> 124.3 us, same GPU). Rows
// that share their first pages with other rows (a cached prefix) load them
// without the hint, so that the sharers read them from the caches.
template <bool STREAM>
__device__ __forceinline__ void dec_dma16(const char* base, uint32_t voff, uint32_t lds) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint64_t bs = ((uint64_t)hi << 32) | (uint64_t)lo;
  if constexpr (STREAM)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(voff), "s"(bs),
                 "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(bs),
                 "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N of this wave's vector memory operations are
// outstanding (gfx9 s_waitcnt: vmcnt[3:0] and [15:14]; lgkm and export
// counters left at their maxima), then keep the compiler from moving memory
// accesses across.
template <int N>
__device__ __forceinline__ void dec_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}

// Issue the loads of buffer x of range s (past its end: its last buffer) into
// LDS buffer `buf` of the wave's region. A 16-key buffer never crosses a page
// (kbeg is a multiple of 16, P >= 16).
template <int D, int G>
__device__ __forceinline__ void dec_issue(const AttnArgs& a, const DecSrc& s, int x, int buf,
                                          const DecLane<D, G>& ln) {
  typedef MfmaDecodeShape<D, G> SH;
  const int kb = s.kbeg + 16 * min(x, s.nbuf - 1);
  int page = __builtin_amdgcn_readlane(s.page_raw, (kb >> a.p_shift) - s.pg0);
  page = min(max(page, 0), a.num_pages - 1);
  const int row0 = kb & ((1 << a.p_shift) - 1);
  const size_t step_off = (((size_t)page << a.p_shift) + row0) * ln.slot_stride;
  const uint32_t lk = ln.lds + (uint32_t)(2 * SH::BUF * buf), lv = lk + SH::BUF;
  if (s.cached) {
#pragma unroll
    for (int q = 0; q < SH::NQ; ++q) {
      dec_dma16<false>(s.kbase + step_off, ln.k_off[q], lk + 1024 * q);
      dec_dma16<false>(s.vbase + step_off, ln.v_off[q], lv + 1024 * q);
    }
  } else {
#pragma unroll
    for (int q = 0; q < SH::NQ; ++q) {
      dec_dma16<true>(s.kbase + step_off, ln.k_off[q], lk + 1024 * q);
      dec_dma16<true>(s.vbase + step_off, ln.v_off[q], lv + 1024 * q);
    }
  }
}

template <int D, int G>
__device__ __forceinline__ void mfma_compute(const DecLane<D, G>& ln, int buf,
                                             const uint4 (&qb)[D / 32], float& m_run,
                                             float& l_part, f32x4_t (&oacc)[D / 16], int kb,
                                             int kend, int rrow, float sl2e, float bias) {
  typedef MfmaDecodeShape<D, G> SH;
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
  typedef short v4i16_dec __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  char* kbuf = ln.region + 2 * SH::BUF * buf;
  char* vbuf = kbuf + SH::BUF;
  // Keys past the range end (only in the last buffer; wave-uniform test):
  // their V rows (which may hold anything) are zeroed before the products,
  // and their scores get no weight below.
  if (kb + 16 > kend) {
#pragma unroll
    for (int q = 0; q < SH::NQ; ++q) {
      const int u = 64 * q + lane;
      if (kb + u / (D / 8) >= kend)
        *(lds_u32x4*)(vbuf + 16 * u) = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  uint4 kop[SH::KSTEPS];
  const lds_u32x4* kl = (const lds_u32x4*)kbuf;
#pragma unroll
  for (int ks = 0; ks < SH::KSTEPS; ++ks)
    kop[ks] = __builtin_bit_cast(uint4, kl[kbuf_unit<D>(lane & 15, 4 * ks + (lane >> 4))]);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < SH::KSTEPS; ++ks)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kop[ks]),
                                                  __builtin_bit_cast(bf16x8_t, qb[ks]), acc, 0,
                                                  0, 0);
  // log2-domain scores; bias is -inf in the lanes of heads >= G
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = fmaf(acc[i], sl2e, bias);
  if (kb + 16 > kend) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = kb + 4 * rrow + i < kend ? s[i] : -INFINITY;
  }
  float mb = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  {
    auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(mb), __float_as_uint(mb), false,
                                              false);
    mb = fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
    auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(mb), __float_as_uint(mb), false,
                                              false);
    mb = fmaxf(__uint_as_float(y[0]), __uint_as_float(y[1]));
  }
  // Rescale only when some head's running max grows (rare after the first
  // keys). Lane (r, c) holds head c's accumulators and running max.
  if (__any(mb > m_run)) {
    const float mn = fmaxf(m_run, mb);
    const float corr = fast_exp2(m_run - mn);
    m_run = mn;
    l_part *= corr;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      oacc[db][0] *= corr;
      oacc[db][1] *= corr;
      oacc[db][2] *= corr;
      oacc[db][3] *= corr;
    }
  }
  // weights rounded to bf16 once; the sum uses the same rounded values
  const f32x2_t p01 = {fast_exp2(s[0] - m_run), fast_exp2(s[1] - m_run)};
  const f32x2_t p23 = {fast_exp2(s[2] - m_run), fast_exp2(s[3] - m_run)};
  const uint32_t w01 = __builtin_bit_cast(uint32_t, __builtin_convertvector(p01, bf16x2e_t));
  const uint32_t w23 = __builtin_bit_cast(uint32_t, __builtin_convertvector(p23, bf16x2e_t));
  l_part += (bf16_lo(w01) + bf16_hi(w01)) + (bf16_lo(w23) + bf16_hi(w23));

  const v4i16_dec pop = __builtin_bit_cast(v4i16_dec, make_uint2(w01, w23));
  const int rk = 4 * rrow + ((lane & 15) >> 2);  // key this lane's reads start from
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    const char* src = vbuf + rk * 2 * D + 32 * (db ^ (rk & 3)) + 8 * (lane & 3);
    const v4i16_dec vop = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16_dec*)(src));
    oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, pop, oacc[db], 0, 0, 0);
  }
}

template <int N>
__device__ __forceinline__ float lane_sum_xor(float x) {
  static_assert(N == 16 || N == 32, "xor 16 or 32");
  auto r = N == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                      false, false)
                   : __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                      false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The loads a range needs before its first K/V buffer: the page ids of its
// pages (lane i: the i-th) and the Q^T operand (head col's dims 8 rrow + 32 ks
// ..). Issued for the next range while the current one streams, so a range
// start waits only for its first K/V buffer. The values are used (clamped,
// masked) only in decode_range, so issuing them waits for nothing.
template <int D, int G>
struct DecPre {
  int page_raw;
  int mslot;  // a group row: the first partial slot of this lane's member
  uint4 qb[MfmaDecodeShape<D, G>::KSTEPS];
};

template <int D, int G>
__device__ __forceinline__ DecPre<D, G> decode_prefetch(const AttnArgs& a, const DecSeg& d) {
  typedef MfmaDecodeShape<D, G> SH;
  DecPre<D, G> p;
  const int lane = threadIdx.x & 63;
  const int rrow = lane >> 4, col = lane & 15;
  const int pg0 = d.kbeg >> a.p_shift;
  const int npg = ((d.kend - 1) >> a.p_shift) - pg0 + 1;
  const int* bt_row = a.block_tables + (size_t)d.seq * a.max_blocks;
  p.page_raw = bt_row[min(pg0 + (lane < npg ? lane : 0), a.max_blocks - 1)];
  const size_t row_bytes = (size_t)SH::ROWB;
  // the fused tick's page-write launch left the row's rotated query in its
  // output row (q itself is the unrotated input); that row's result is written
  // only once every range of the row has read it
  const char* qbase = a.fused ? (const char*)a.out : (const char*)a.q;
  // column col of the score product: head col of the row; in a group row,
  // head col % G of member col / G (its own query row)
  int token = d.token, hq = col < G ? col : 0;
  p.mslot = 0;
  if (d.group > 0) {
    const PlanOffsets po = plan_offsets(a.S, a.Hq, a.cap_dec, a.cap_pf);
    const int m = min(d.grow + 1 + min(col / G, d.group - 1), (int)plan_rows(a.S) - 1);
    token = reinterpret_cast<const int4*>(a.plan + po.rows)[m].w;
    p.mslot = a.plan[po.pbase + m];
    hq = col % G;
  }
  token = min(max(token, 0), a.T - 1);
  const char* qrow = qbase + ((size_t)token * a.Hq + (size_t)d.kvh * G) * row_bytes;
#pragma unroll
  for (int ks = 0; ks < SH::KSTEPS; ++ks)
    p.qb[ks] = *reinterpret_cast<const uint4*>(qrow + hq * row_bytes + 16 * rrow + 64 * ks);
  return p;
}

// One decode range on a wave. Buffer 0 of the range has been issued into LDS
// buffer buf0; the two LDS buffers alternate, the loads of the next buffer in
// flight while one computes. The range's last step issues buffer 0 of the
// next range sn, so the stream does not drain between ranges (after the last
// range, sn is the range itself: a re-read of one buffer). Returns the LDS
// buffer that holds it.
template <int D, int G>
__device__ __forceinline__ int decode_range(const AttnArgs& a, int buf0, const DecSeg& d,
                                            const DecPre<D, G>& pre, const DecSrc& s,
                                            const DecSrc& sn, const DecLane<D, G>& ln) {
  typedef MfmaDecodeShape<D, G> SH;
  const int lane = threadIdx.x & 63;
  const int rrow = lane >> 4, col = lane & 15;  // score layout: keys 4 rrow.., head col

  // Q^T operand, zero in the lanes of heads >= G. Its loads (and the page ids)
  // were issued with the previous range: they are waited for here, before the
  // next buffer's loads are issued, so that wait does not include those.
  // (a group row's columns: G per member)
  const int ncol = d.group > 0 ? d.group * G : G;
  uint4 qb[SH::KSTEPS];
#pragma unroll
  for (int ks = 0; ks < SH::KSTEPS; ++ks)
    qb[ks] = col < ncol ? pre.qb[ks] : make_uint4(0u, 0u, 0u, 0u);
  const float bias = col < ncol ? 0.f : -INFINITY;
  __builtin_amdgcn_sched_barrier(0);

  float m_run = kNegBig, l_part = 0.f;
  f32x4_t oacc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const float sl2e = a.scale_log2e;
  const int nb = s.nbuf, kend = d.kend;
  int buf = buf0;
  for (int j = 0; j < nb; ++j) {
    // the next buffer: of this range, or buffer 0 of the next one
    if (j + 1 < nb)
      dec_issue<D, G>(a, s, j + 1, buf ^ 1, ln);
    else
      dec_issue<D, G>(a, sn, 0, buf ^ 1, ln);
    dec_wait<SH::NDMA>();  // buffer j has landed (only the next one's loads remain)
    mfma_compute<D, G>(ln, buf, qb, m_run, l_part, oacc, s.kbeg + 16 * j, kend, rrow, sl2e,
                       bias);
    buf ^= 1;
  }

  // The head's weight sum over its four lanes (one max for the whole wave, so
  // no rescaling); lane (rrow, col) holds the final dims 16 db + 4 rrow .. + 3
  // of head col.
  float l = lane_sum_xor<16>(l_part);
  l = lane_sum_xor<32>(l);
  if (col < ncol) {
    const size_t row_bytes = (size_t)SH::ROWB;
    const int hq = d.kvh * G + (d.group > 0 ? col % G : col);
    if (d.group > 0) {
      // partition part of the group row: a partial of this lane's member
      // (the plan keeps every member's slots inside the workspace)
      if (pre.mslot + d.part >= a.part_slots) return buf;
      const size_t pi = ((size_t)pre.mslot + d.part) * a.Hq + hq;
      float* po = a.ws + pi * D;
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
        *reinterpret_cast<float4*>(po + 16 * db + 4 * rrow) =
            make_float4(oacc[db][0], oacc[db][1], oacc[db][2], oacc[db][3]);
      if (rrow == 0) {
        float* ml = a.ws + (size_t)a.part_slots * a.Hq * D;
        *reinterpret_cast<float2*>(ml + 2 * pi) = make_float2(m_run, l);
      }
    } else if (d.nparts == 1) {
      const float inv = 1.f / l;
      char* orow = (char*)a.out + ((size_t)d.token * a.Hq + hq) * row_bytes;
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
        *reinterpret_cast<uint2*>(orow + 2 * (16 * db + 4 * rrow)) =
            make_uint2(pack_bf16x2(oacc[db][0] * inv, oacc[db][1] * inv),
                       pack_bf16x2(oacc[db][2] * inv, oacc[db][3] * inv));
    } else {
      const size_t pi = ((size_t)d.pslot + d.part) * a.Hq + hq;
      float* po = a.ws + pi * D;
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
        *reinterpret_cast<float4*>(po + 16 * db + 4 * rrow) =
            make_float4(oacc[db][0], oacc[db][1], oacc[db][2], oacc[db][3]);
      if (rrow == 0) {
        float* ml = a.ws + (size_t)a.part_slots * a.Hq * D;
        *reinterpret_cast<float2*>(ml + 2 * pi) = make_float2(m_run, l);
      }
    }
  }
  return buf;
}

// A single range (one wave, one work item). region: the wave's
// dec_region_units<D>() units of LDS.
template <int D, int G>
__device__ __forceinline__ void decode_range_alone(const AttnArgs& a, const DecSeg& d,
                                                   uint4* region) {
  const DecLane<D, G> ln = dec_lane<D, G>(a, region);
  const DecPre<D, G> p = decode_prefetch<D, G>(a, d);
  const DecSrc s = dec_src<D, G>(a, d, p.page_raw);
  dec_issue<D, G>(a, s, 0, 0, ln);
  decode_range<D, G>(a, 0, d, p, s, s, ln);
  dec_wait<0>();  // the trailing re-read has landed before the region is left
}

// The decode ranges of wave gw, streamed back to back: each range's page ids
// and Q are issued while the previous range streams, and its first buffer is
// loaded during the previous range's last step. lds: dec_region_units<D>()
// 16-byte units per wave of the workgroup (wave w uses the w-th region).
template <int D, int G>
__device__ __forceinline__ void decode_chunks_mfma(const AttnArgs& a, int wg, uint4* lds) {
  uint4* region = lds + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * dec_region_units<D>();
  const DecLane<D, G> ln = dec_lane<D, G>(a, region);
  DecodeCursor cur(a, wg);
  DecSeg d;
  if (!cur.next(d)) return;
  DecPre<D, G> p = decode_prefetch<D, G>(a, d);
  DecSrc s = dec_src<D, G>(a, d, p.page_raw);
  dec_issue<D, G>(a, s, 0, 0, ln);
  int buf = 0;  // LDS buffer holding the current range's buffer 0
  for (;;) {
    DecSeg dn;
    const bool more = cur.next(dn);
    if (!more) dn = d;
    const DecPre<D, G> pn = decode_prefetch<D, G>(a, dn);
    const DecSrc sn = dec_src<D, G>(a, dn, pn.page_raw);
    buf = decode_range<D, G>(a, buf, d, p, s, sn, ln);
    if (!more) break;
    d = dn;
    p = pn;
    s = sn;
  }
  dec_wait<0>();  // the trailing re-read has landed before the region is reused
}

}  // namespace pa
