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

// K3 task idx = (row, query head, 4 consecutive dims): merge the row's
// split-KV partitions, m* = max_k m_k,
// o = sum_k 2^(m_k - m*) o_k / sum_k 2^(m_k - m*) l_k (m* taken as a running
// maximum, the sums rescaled when it grows).
template <typename ET, bool TOKEN_MODE>
__device__ __forceinline__ void split_reduce_task(const AttnArgs& a, long idx) {
  const int D = a.D;
  const int quads = D / 4;
  const int d4 = (int)(idx % quads);
  const long rh = idx / quads;
  const int h = (int)(rh % a.Hq);
  const long row = rh / a.Hq;
  if (row >= (TOKEN_MODE ? a.T : a.S)) return;
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
  // one pass with a running max: all partitions' loads are independent
  float mn = kNegBig, lt = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int k = 0; k < nparts; ++k) {
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
      const int np = nparts_of[i], pb = pbase_of[i];
      const int off = r.y, n = r.z;
      const int pad = (n + A - 1) / A * A;
      const int c0 = chunk * C, c1 = c0 + C;
      d.seq = r.x;
      d.token = r.w;
      d.pslot = pb;
      d.kbeg = max(c0, off) - off;
      d.kend = min(min(c1, off + pad) - off, n);
      d.part = chunk - off / C;
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
// bf16 work item with the scores on matrix cores. Per 16-key buffer:
//   S^T[key, head] = K[key, :] . Q[head, :]   v_mfma_f32_16x16x32_bf16, A = K
//   rows in the A layout (lane l: key l % 16, dims 8(l/16) + 32 ks ..; loaded
//   as whole lines and rearranged through LDS, see kbuf_unit), B = Q^T (lane
//   l: head l % 16, zero for heads >= G). Lane (r, c)
//   (r = l / 16, c = l % 16) then holds the scores of keys 4r .. 4r + 3 for
//   head c. One running max per head for the whole wave (combined over the
//   four lanes of a head with permlane swaps), so the per-lane sums and output
//   accumulators of different lanes can be added without rescaling.
//   P.V stays on v_dot2: V row (key) slot * UNROLL + u of the buffer sits in
//   the LPK lanes of `slot`; its weights are the (bf16-packed) scores of lane
//   (slot * UNROLL / 4, head), broadcast along the 16-lane row with DPP
//   row_newbcast.
template <int D, int G>
struct MfmaDecodeShape {
  static constexpr int ROWB = D * 2;
  static constexpr int KSTEPS = D / 32;      // k-steps of the score MFMA
  static constexpr int LPK = ROWB / 16;      // lanes per V row (16 bytes each)
  static constexpr int NSLOT = 64 / LPK;     // V rows per step
  static constexpr int UNROLL = 16 / NSLOT;  // steps per 16-key buffer
  static constexpr int NPAIR = UNROLL / 2;
  static_assert(D == 64 || D == 128, "bf16 head dims 64 and 128");
  static_assert(G >= 1 && G <= 8, "at most 8 query heads per KV head");
};


template <int N>
__device__ __forceinline__ uint32_t row_bcast(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x150 + N, 0xF, 0xF, false);
}

template <int D, int G>
struct MfmaBuf {
  uint4 k[MfmaDecodeShape<D, G>::KSTEPS];
  uint4 v[MfmaDecodeShape<D, G>::UNROLL];
};

// K rows of a 16-key buffer are loaded as whole 128-byte lines (8 lanes per
// line, 8 keys per load instruction): loads laid out for the MFMA A operand
// directly (16 keys x 64 bytes per instruction) streamed at ~4.8 TB/s against
// ~6.3 TB/s for whole lines on MI355X. Load i of a lane holds key
// 8 (i / (D / 64)) + lane / 8, 16-byte chunk 8 (i % (D / 64)) + lane % 8; the
// wave passes the buffer through its own 16-key LDS region to put it in the
// operand layout (mfma_compute). Unit (16 bytes) of key k, chunk c there:
//   64 ((D / 64) (k / 8) + c / 8) + 8 (k % 8) + ((c % 8) ^ (k / 2) ^ 4 (k % 2)) % 8
// Writes cover whole 128-byte runs, and the operand reads (lane l: key l % 16,
// chunk 4 ks + l / 16) hit distinct banks whether 8 or 16 lanes are served a
// cycle.
template <int D>
__device__ __forceinline__ int kbuf_unit(int k, int c) {
  return 64 * ((D / 64) * (k >> 3) + (c >> 3)) + 8 * (k & 7) + (((c & 7) ^ (k >> 1) ^ ((k & 1) << 2)) & 7);
}
// 16-byte units of one wave's K region
template <int D>
constexpr int kbuf_units() { return 16 * D * 2 / 16; }

// Where a range's 16-key buffers come from.
struct DecSrc {
  const char* kbase;  // K pool + the KV head's offset within a slot
  const char* vbase;
  int page_raw;       // lane i: block-table entry of the range's i-th page (unchecked)
  int pg0;            // the range's first page
  int kbeg;           // first key (a multiple of 16)
  int nbuf;           // 16-key buffers (>= 1)
};

// Per-lane offsets of the K and V loads within a 16-key buffer.
struct DecLane {
  size_t slot_stride;  // bytes between consecutive slots of a page
  uint32_t k_off, v_off;
};

template <int D, int G>
__device__ __forceinline__ DecLane dec_lane(const AttnArgs& a) {
  typedef MfmaDecodeShape<D, G> SH;
  const int lane = threadIdx.x & 63;
  const int slot = lane / SH::LPK, sub = lane % SH::LPK;
  DecLane l;
  l.slot_stride = (size_t)a.Hkv * SH::ROWB;
  l.k_off = (uint32_t)((lane >> 3) * l.slot_stride) + 16 * (lane & 7);
  l.v_off = (uint32_t)(slot * SH::UNROLL * l.slot_stride) + 16 * sub;
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
  return s;
}

// Issue the loads of buffer x of range s (past its end: its last buffer). A
// 16-key buffer never crosses a page (kbeg is a multiple of 16, P >= 16).
template <int D, int G>
__device__ __forceinline__ void mfma_load(MfmaBuf<D, G>& b, const AttnArgs& a, const DecSrc& s,
                                          int x, const DecLane& ln) {
  typedef MfmaDecodeShape<D, G> SH;
  const int kb = s.kbeg + 16 * min(x, s.nbuf - 1);
  int page = __builtin_amdgcn_readlane(s.page_raw, (kb >> a.p_shift) - s.pg0);
  page = min(max(page, 0), a.num_pages - 1);
  const int row0 = kb & ((1 << a.p_shift) - 1);
  const size_t step_off = (((size_t)page << a.p_shift) + row0) * ln.slot_stride;
  const char* kp = s.kbase + step_off + ln.k_off;
#pragma unroll
  for (int i = 0; i < SH::KSTEPS; ++i)
    b.k[i] = *reinterpret_cast<const uint4*>(kp + (size_t)(8 * (i / (D / 64))) * ln.slot_stride +
                                             128 * (i % (D / 64)));
  const char* vp = s.vbase + step_off + ln.v_off;
#pragma unroll
  for (int u = 0; u < SH::UNROLL; ++u)
    b.v[u] = *reinterpret_cast<const uint4*>(vp + (size_t)u * ln.slot_stride);
}

__device__ __forceinline__ uint32_t word_of4(const uint4& v, int w) {
  return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
}

template <int D, int G>
__device__ __forceinline__ void mfma_compute(MfmaBuf<D, G>& b, const uint4 (&qb)[D / 32],
                                             float& m_run, float& l_part, float (&o)[G][8],
                                             int kb, int kend, int rrow, int slot, float sl2e,
                                             float bias, uint4* kreg) {
  typedef MfmaDecodeShape<D, G> SH;
  // K through the wave's LDS region into the A-operand layout (lane l: key
  // l % 16, dims 8 (l / 16) + 32 ks ..). Only this wave touches the region and
  // its LDS accesses run in order, so no barrier is needed.
  // (an explicit LDS pointer: through a generic one the compiler could not
  // rule out aliasing with the register buffers and kept them in scratch)
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
  lds_u32x4* kl = (lds_u32x4*)kreg;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < SH::KSTEPS; ++i)
    kl[kbuf_unit<D>(8 * (i / (D / 64)) + (lane >> 3), 8 * (i % (D / 64)) + (lane & 7))] =
        __builtin_bit_cast(u32x4_t, b.k[i]);
  uint4 kop[SH::KSTEPS];
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
  // Keys past the range end (only in the last buffer; wave-uniform test):
  // no weight, and their V rows (which may hold anything) zeroed.
  if (kb + 16 > kend) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = kb + 4 * rrow + i < kend ? s[i] : -INFINITY;
#pragma unroll
    for (int u = 0; u < SH::UNROLL; ++u) {
      const bool ok = kb + slot * SH::UNROLL + u < kend;
      b.v[u] = make_uint4(ok ? b.v[u].x : 0u, ok ? b.v[u].y : 0u, ok ? b.v[u].z : 0u,
                          ok ? b.v[u].w : 0u);
    }
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
  // Rescale only when some head's running max grows (rare after the first keys).
  if (__any(mb > m_run)) {
    const float mn = fmaxf(m_run, mb);
    const float corr = fast_exp2(m_run - mn);
    m_run = mn;
    l_part *= corr;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float ch;
      if constexpr (true) {
        const uint32_t cu = __float_as_uint(corr);
        switch (h) {
          case 0: ch = __uint_as_float(row_bcast<0>(cu)); break;
          case 1: ch = __uint_as_float(row_bcast<1>(cu)); break;
          case 2: ch = __uint_as_float(row_bcast<2>(cu)); break;
          case 3: ch = __uint_as_float(row_bcast<3>(cu)); break;
          case 4: ch = __uint_as_float(row_bcast<4>(cu)); break;
          case 5: ch = __uint_as_float(row_bcast<5>(cu)); break;
          case 6: ch = __uint_as_float(row_bcast<6>(cu)); break;
          default: ch = __uint_as_float(row_bcast<7>(cu)); break;
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) o[h][i] *= ch;
    }
  }
  // weights rounded to bf16 once; the sum uses the same rounded values
  const f32x2_t p01 = {fast_exp2(s[0] - m_run), fast_exp2(s[1] - m_run)};
  const f32x2_t p23 = {fast_exp2(s[2] - m_run), fast_exp2(s[3] - m_run)};
  const uint32_t w01 = __builtin_bit_cast(uint32_t, __builtin_convertvector(p01, bf16x2e_t));
  const uint32_t w23 = __builtin_bit_cast(uint32_t, __builtin_convertvector(p23, bf16x2e_t));
  l_part += (bf16_lo(w01) + bf16_hi(w01)) + (bf16_lo(w23) + bf16_hi(w23));

  // V rows of steps (2j, 2j+1) interleaved per dim for v_dot2
  uint32_t vlo[SH::NPAIR][4], vhi[SH::NPAIR][4];
#pragma unroll
  for (int j = 0; j < SH::NPAIR; ++j)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      vlo[j][w] = __builtin_amdgcn_perm(word_of4(b.v[2 * j + 1], w), word_of4(b.v[2 * j], w),
                                        0x05040100u);
      vhi[j][w] = __builtin_amdgcn_perm(word_of4(b.v[2 * j + 1], w), word_of4(b.v[2 * j], w),
                                        0x07060302u);
    }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    uint32_t b01, b23;
    switch (h) {
      case 0: b01 = row_bcast<0>(w01); b23 = row_bcast<0>(w23); break;
      case 1: b01 = row_bcast<1>(w01); b23 = row_bcast<1>(w23); break;
      case 2: b01 = row_bcast<2>(w01); b23 = row_bcast<2>(w23); break;
      case 3: b01 = row_bcast<3>(w01); b23 = row_bcast<3>(w23); break;
      case 4: b01 = row_bcast<4>(w01); b23 = row_bcast<4>(w23); break;
      case 5: b01 = row_bcast<5>(w01); b23 = row_bcast<5>(w23); break;
      case 6: b01 = row_bcast<6>(w01); b23 = row_bcast<6>(w23); break;
      default: b01 = row_bcast<7>(w01); b23 = row_bcast<7>(w23); break;
    }
    uint32_t pw[SH::NPAIR];
    if constexpr (SH::UNROLL == 4) {
      // keys 4 slot + u: elements (0,1) and (2,3) of the row's score lane
      pw[0] = b01;
      pw[1] = b23;
    } else {
      // keys 2 slot + u: elements (0,1) for even slots, (2,3) for odd ones
      pw[0] = (slot & 1) ? b23 : b01;
    }
#pragma unroll
    for (int j = 0; j < SH::NPAIR; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        o[h][2 * w] = dot2_bf16(pw[j], vlo[j][w], o[h][2 * w]);
        o[h][2 * w + 1] = dot2_bf16(pw[j], vhi[j][w], o[h][2 * w + 1]);
      }
  }
}

template <int N>
__device__ __forceinline__ float lane_sum_xor(float x) {
  if constexpr (N == 16 || N == 32) {
    auto r = N == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                        false, false)
                     : __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                        false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    static_assert(N == 8, "xor 8, 16 or 32");
    const float other = dpp_f<0x128>(x);  // row_ror:8 = lane ^ 8
    return (threadIdx.x & 8) ? other + x : x + other;
  }
}

// The loads a range needs before its first K/V buffer: the page ids of its
// pages (lane i: the i-th) and the Q^T operand (head col's dims 8 rrow + 32 ks
// ..). Issued for the next range while the current one streams, so a range
// start waits only for its first K/V buffer. The values are used (clamped,
// masked) only in decode_range, so issuing them waits for nothing.
template <int D, int G>
struct DecPre {
  int page_raw;
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
  p.page_raw = bt_row[pg0 + (lane < npg ? lane : 0)];
  const size_t row_bytes = (size_t)SH::ROWB;
  const char* qrow = (const char*)a.q + ((size_t)d.token * a.Hq + (size_t)d.kvh * G) * row_bytes;
  const int hq = col < G ? col : 0;
#pragma unroll
  for (int ks = 0; ks < SH::KSTEPS; ++ks)
    p.qb[ks] = *reinterpret_cast<const uint4*>(qrow + hq * row_bytes + 16 * rrow + 64 * ks);
  return p;
}

// One decode range on a wave. b0 holds (its loads issued) buffer 0 of the
// range; the two register buffers alternate, the loads of the next buffer in
// flight while one computes. The range's last step loads buffer 0 of the next
// range sn into the other buffer, so the stream does not drain between
// ranges (after the last range, sn is the range itself: a re-read of one
// buffer). That is b1 when the range has an odd number of buffers: the
// caller then passes the buffers swapped for the next range.
template <int D, int G>
__device__ __forceinline__ void decode_range(const AttnArgs& a, MfmaBuf<D, G>& b0,
                                             MfmaBuf<D, G>& b1, const DecSeg& d,
                                             const DecPre<D, G>& pre, const DecSrc& s,
                                             const DecSrc& sn, const DecLane& ln, uint4* kreg) {
  typedef MfmaDecodeShape<D, G> SH;
  constexpr int LPK = SH::LPK, NSLOT = SH::NSLOT;
  const int lane = threadIdx.x & 63;
  const int rrow = lane >> 4, col = lane & 15;  // score layout: keys 4 rrow.., head col
  const int slot = lane / LPK, sub = lane % LPK;  // V layout

  // Q^T operand, zero in the lanes of heads >= G
  uint4 qb[SH::KSTEPS];
#pragma unroll
  for (int ks = 0; ks < SH::KSTEPS; ++ks)
    qb[ks] = col < G ? pre.qb[ks] : make_uint4(0u, 0u, 0u, 0u);
  const float bias = col < G ? 0.f : -INFINITY;

  float m_run = kNegBig, l_part = 0.f;
  float o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) o[h][i] = 0.f;

  const float sl2e = a.scale_log2e;
  const int nb = s.nbuf, kend = d.kend;
  auto load = [&](MfmaBuf<D, G>& b, int x) {
    if (x < nb)
      mfma_load<D, G>(b, a, s, x, ln);
    else
      mfma_load<D, G>(b, a, sn, x - nb, ln);
  };
  for (int j = 0;; j += 2) {
    load(b1, j + 1);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of this compute
    mfma_compute<D, G>(b0, qb, m_run, l_part, o, s.kbeg + 16 * j, kend, rrow, slot, sl2e, bias,
                       kreg);
    if (j + 1 >= nb) break;
    load(b0, j + 2);
    __builtin_amdgcn_sched_barrier(0);
    mfma_compute<D, G>(b1, qb, m_run, l_part, o, s.kbeg + 16 * (j + 1), kend, rrow, slot, sl2e,
                       bias, kreg);
    if (j + 2 >= nb) break;
  }

  // Sums over the lanes of a head (l) and over the V slots (o): one max for
  // the whole wave, so no rescaling.
  float l = lane_sum_xor<16>(l_part);
  l = lane_sum_xor<32>(l);
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float x = o[h][i];
      if constexpr (LPK <= 8) x = lane_sum_xor<8>(x);
      x = lane_sum_xor<16>(x);
      o[h][i] = lane_sum_xor<32>(x);
    }

  // Slot s writes the heads h with h % NSLOT == s; the head's l and m come
  // from lane col = h of the row.
  const size_t row_bytes = (size_t)SH::ROWB;
  const uint32_t lu = __float_as_uint(l), mu = __float_as_uint(m_run);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    uint32_t lh, mh;
    switch (h) {
      case 0: lh = row_bcast<0>(lu); mh = row_bcast<0>(mu); break;
      case 1: lh = row_bcast<1>(lu); mh = row_bcast<1>(mu); break;
      case 2: lh = row_bcast<2>(lu); mh = row_bcast<2>(mu); break;
      case 3: lh = row_bcast<3>(lu); mh = row_bcast<3>(mu); break;
      case 4: lh = row_bcast<4>(lu); mh = row_bcast<4>(mu); break;
      case 5: lh = row_bcast<5>(lu); mh = row_bcast<5>(mu); break;
      case 6: lh = row_bcast<6>(lu); mh = row_bcast<6>(mu); break;
      default: lh = row_bcast<7>(lu); mh = row_bcast<7>(mu); break;
    }
    if (h % NSLOT != slot) continue;
    const int hq = d.kvh * G + h;
    if (d.nparts == 1) {
      const float inv = 1.f / __uint_as_float(lh);
      uint32_t wv[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) wv[w] = pack_bf16x2(o[h][2 * w] * inv, o[h][2 * w + 1] * inv);
      char* orow = (char*)a.out + ((size_t)d.token * a.Hq + hq) * row_bytes;
      *reinterpret_cast<uint4*>(orow + 16 * sub) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    } else {
      const size_t pi = ((size_t)d.pslot + d.part) * a.Hq + hq;
      float* po = a.ws + pi * D + 8 * sub;
      *reinterpret_cast<float4*>(po) = make_float4(o[h][0], o[h][1], o[h][2], o[h][3]);
      *reinterpret_cast<float4*>(po + 4) = make_float4(o[h][4], o[h][5], o[h][6], o[h][7]);
      if (sub == 0) {
        float* ml = a.ws + (size_t)a.part_slots * a.Hq * D;
        *reinterpret_cast<float2*>(ml + 2 * pi) =
            make_float2(__uint_as_float(mh), __uint_as_float(lh));
      }
    }
  }
}

// A single range (one wave, one work item).
template <int D, int G>
__device__ __forceinline__ void decode_range_alone(const AttnArgs& a, const DecSeg& d,
                                                   uint4* kreg) {
  const DecLane ln = dec_lane<D, G>(a);
  const DecPre<D, G> p = decode_prefetch<D, G>(a, d);
  const DecSrc s = dec_src<D, G>(a, d, p.page_raw);
  MfmaBuf<D, G> b0, b1;
  mfma_load<D, G>(b0, a, s, 0, ln);
  decode_range<D, G>(a, b0, b1, d, p, s, s, ln, kreg);
}

// The decode ranges of wave gw, streamed back to back: each range's page ids
// and Q are issued while the previous range streams, and its first buffer is
// loaded during the previous range's last step. lds: kbuf_units<D>() 16-byte
// units per wave of the workgroup (wave w uses the w-th block).
template <int D, int G>
__device__ __forceinline__ void decode_chunks_mfma(const AttnArgs& a, int wg, uint4* lds) {
  uint4* kreg = lds + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * kbuf_units<D>();
  const DecLane ln = dec_lane<D, G>(a);
  DecodeCursor cur(a, wg);
  DecSeg d;
  if (!cur.next(d)) return;
  DecPre<D, G> p = decode_prefetch<D, G>(a, d);
  DecSrc s = dec_src<D, G>(a, d, p.page_raw);
  MfmaBuf<D, G> b0, b1;
  mfma_load<D, G>(b0, a, s, 0, ln);
  bool flip = false;  // the current range's buffer 0 is in b1
  for (;;) {
    DecSeg dn;
    const bool more = cur.next(dn);
    if (!more) dn = d;
    const DecPre<D, G> pn = decode_prefetch<D, G>(a, dn);
    const DecSrc sn = dec_src<D, G>(a, dn, pn.page_raw);
    if (!flip)
      decode_range<D, G>(a, b0, b1, d, p, s, sn, ln, kreg);
    else
      decode_range<D, G>(a, b1, b0, d, p, s, sn, ln, kreg);
    if (!more) break;
    flip ^= (s.nbuf & 1) != 0;
    d = dn;
    p = pn;
    s = sn;
  }
}

}  // namespace pa
