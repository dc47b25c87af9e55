// K2: paged decode attention with split-KV partitions. K3: merge of the partitions.
//
// Decode is HBM-bound: every key row of a (sequence, KV head) is read once and
// used by all G query heads of its group (grouped-query attention: Helios blog,
// "torch.sdpa and Flash Attention"), about 2*G flops per byte. The kernel is
// written for that bound: 16-byte row loads through the page table, the next
// buffer's loads in flight while the current one computes, and the softmax
// kept online in registers. The float32 path below takes its dot products on
// VALU; the bf16 path (pa_decode_mfma.h) loads K and V straight into the
// wave's LDS buffers and puts the scores and P.V on matrix cores.
//
// Work decomposition. A work item is a key range of one row for one KV head
// and is owned by ONE wave: nothing is shared between waves (the bf16 path's
// LDS buffers are the wave's own) and there is no workgroup barrier, so a wave
// never waits for its neighbours. The range's page ids sit in one VGPR (lane i holds
// the i-th page of the range, at most 64 pages) and each buffer takes its page
// with a lane read into a scalar register.
//
// For the decode rows of a tick the plan kernel lays all rows end to end on
// one key axis and cuts it into equal chunks, one per wave (see
// pa_plan.h): a wave walks the rows its chunk covers, one range per row, so
// every wave gets the same number of keys whatever the spread of lengths
// (decode_walk in pa_decode_mfma.h). The per-token mode (prefill rows without
// a matrix-core kernel, i.e. float32) maps waves to (token, fixed partition,
// KV head) directly.
//
// float32: inside a wave, LPK lanes hold one key row (16 or 32 bytes each), so a wave
// covers 64 / LPK keys per step (its "slots") and UNROLL steps per buffer.
// Each lane keeps its own running (max, sum, output) over the keys of its
// slot; at the end the slots are merged with a register butterfly
// (permlane16/32 swaps, DPP below 16 lanes).
//
// A range's result is either final (the row has one range) or a partial
// (m, l, o) in the workspace, merged by K3:
//   m* = max_k m_k,  o = sum_k 2^(m_k - m*) o_k / sum_k 2^(m_k - m*) l_k.
#include "pa_decode_mfma.h"

namespace pa {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

template <typename ET, int D>
struct DecodeShape {
  static constexpr int EB = ET::kBytes;
  static constexpr int ROWB = D * EB;  // bytes of one head row
  static constexpr int LPK = ROWB / 16 > 16 ? 16 : ROWB / 16;  // lanes per key row
  static constexpr int LANE_BYTES = ROWB / LPK;  // 16 or 32
  static constexpr int LOADS = LANE_BYTES / 16;  // 16-byte loads per lane per row
  static constexpr int WORDS = LANE_BYTES / 4;   // 32-bit words per lane per row
  static constexpr int DPL = D / LPK;            // head dims held by a lane
  static constexpr int EPV = 16 / EB;            // elements per 16-byte vector
  static constexpr int KPW = 64 / LPK;           // keys per wave step (slots)
  // A buffer covers KPI consecutive keys starting at a multiple of KPI; pages
  // hold a power of two >= 16 keys, so a buffer never crosses a page.
  static constexpr int KPI = EB == 2 || KPW > 8 ? 16 : 8;
  static constexpr int UNROLL = KPI / KPW;       // steps per buffer
  static_assert(LANE_BYTES == 16 || LANE_BYTES == 32, "lane row share must be 16 or 32 bytes");
  static_assert(UNROLL >= 1 && KPW * UNROLL == KPI, "a buffer is whole steps");
  static_assert(EB == 4 || UNROLL % 2 == 0, "bf16 P.V pairs the steps of a buffer");
  // Head-dim index of the lane's local dim i (sub = lane % LPK).
  __device__ static int dim_of(int sub, int i) {
    return ((i / EPV) * LPK + sub) * EPV + (i % EPV);
  }
};

// Issue the loads of one buffer: the KPI keys starting at `kb` (wave-uniform,
// a multiple of KPI, inside the partition). The page id comes from lane
// `page index` of the page VGPR, so the address is a scalar base plus the
// lane's fixed 32-bit offset. Slots past the partition end read rows of the
// same page (in bounds; masked in compute_step).
template <typename SH>
__device__ __forceinline__ void load_buf(uint32_t (&kr)[SH::UNROLL][SH::WORDS],
                                         uint32_t (&vr)[SH::UNROLL][SH::WORDS],
                                         const char* kbase, const char* vbase, int page_reg,
                                         int pg0, int p_shift, size_t slot_stride, int kb,
                                         uint32_t lane_off) {
  const int page = __builtin_amdgcn_readlane(page_reg, (kb >> p_shift) - pg0);
  const int row0 = kb & ((1 << p_shift) - 1);
  const size_t step_off = (((size_t)page << p_shift) + row0) * slot_stride;
#pragma unroll
  for (int u = 0; u < SH::UNROLL; ++u) {
    const size_t uoff = step_off + (size_t)u * SH::KPW * slot_stride;  // uniform
    const char* kp = kbase + uoff;
    const char* vp = vbase + uoff;
#pragma unroll
    for (int l = 0; l < SH::LOADS; ++l) {
      const uint4 x = *reinterpret_cast<const uint4*>(kp + lane_off + l * SH::LPK * 16);
      kr[u][4 * l] = x.x; kr[u][4 * l + 1] = x.y; kr[u][4 * l + 2] = x.z; kr[u][4 * l + 3] = x.w;
    }
#pragma unroll
    for (int l = 0; l < SH::LOADS; ++l) {
      const uint4 x = *reinterpret_cast<const uint4*>(vp + lane_off + l * SH::LPK * 16);
      vr[u][4 * l] = x.x; vr[u][4 * l + 1] = x.y; vr[u][4 * l + 2] = x.z; vr[u][4 * l + 3] = x.w;
    }
  }
}

// Scores, online softmax and P.V for one buffer (KPI keys of the wave).
template <typename SH, int G>
__device__ __forceinline__ void compute_buf(const uint32_t (&kr)[SH::UNROLL][SH::WORDS],
                                            uint32_t (&vr)[SH::UNROLL][SH::WORDS],
                                            const uint32_t (&qw)[G][SH::WORDS], float (&m)[G],
                                            float (&lsum)[G], float (&o)[G][SH::DPL], int kb,
                                            int kend, int slot, float sl2e) {
  constexpr int UNROLL = SH::UNROLL, WORDS = SH::WORDS, DPL = SH::DPL;
  bool valid[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) valid[u] = kb + u * SH::KPW + slot < kend;
  // Rows past the end may hold anything (NaN included); zero their V so that
  // a zero weight times them stays zero. Only the last buffer of a partition
  // is partial, and the test is wave-uniform.
  if (kb + SH::KPI > kend) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
#pragma unroll
      for (int w = 0; w < WORDS; ++w) vr[u][w] = valid[u] ? vr[u][w] : 0u;
  }
  float sc[UNROLL][G];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float acc = 0.f;
      if constexpr (SH::EB == 2) {
#pragma unroll
        for (int w = 0; w < WORDS; ++w) acc = dot2_bf16(qw[g][w], kr[u][w], acc);
      } else {
#pragma unroll
        for (int w = 0; w < WORDS; ++w)
          acc = fmaf(__uint_as_float(qw[g][w]), __uint_as_float(kr[u][w]), acc);
      }
      acc = group_sum<SH::LPK>(acc);
      sc[u][g] = valid[u] ? acc * sl2e : -INFINITY;
    }
  }
  // bf16: V rows of steps (2j, 2j+1) interleaved per dim, (v_2j[d], v_2j+1[d]),
  // so that one v_dot2 adds both keys' contributions to one output dim.
  constexpr int NPAIR = SH::EB == 2 ? UNROLL / 2 : 1;
  uint32_t vlo[NPAIR][WORDS], vhi[NPAIR][WORDS];
  if constexpr (SH::EB == 2) {
#pragma unroll
    for (int j = 0; j < NPAIR; ++j)
#pragma unroll
      for (int w = 0; w < WORDS; ++w) {
        vlo[j][w] = __builtin_amdgcn_perm(vr[2 * j + 1][w], vr[2 * j][w], 0x05040100u);
        vhi[j][w] = __builtin_amdgcn_perm(vr[2 * j + 1][w], vr[2 * j][w], 0x07060302u);
      }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float mb = sc[0][g];
#pragma unroll
    for (int u = 1; u < UNROLL; ++u) mb = fmaxf(mb, sc[u][g]);
    // Rescale only when some lane's running max grows (rare after the first keys).
    if (__any(mb > m[g])) {
      const float mn = fmaxf(m[g], mb);
      const float corr = fast_exp2(m[g] - mn);
      m[g] = mn;
      lsum[g] *= corr;
#pragma unroll
      for (int i = 0; i < DPL; ++i) o[g][i] *= corr;
    }
    if constexpr (SH::EB == 2) {
#pragma unroll
      for (int j = 0; j < NPAIR; ++j) {
        // weights rounded to bf16 once; the sum uses the same rounded values
        const f32x2_t pf = {fast_exp2(sc[2 * j][g] - m[g]), fast_exp2(sc[2 * j + 1][g] - m[g])};
        const uint32_t pp = __builtin_bit_cast(uint32_t, __builtin_convertvector(pf, bf16x2e_t));
        lsum[g] += bf16_lo(pp) + bf16_hi(pp);
#pragma unroll
        for (int w = 0; w < WORDS; ++w) {
          o[g][2 * w] = dot2_bf16(pp, vlo[j][w], o[g][2 * w]);
          o[g][2 * w + 1] = dot2_bf16(pp, vhi[j][w], o[g][2 * w + 1]);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const float p = fast_exp2(sc[u][g] - m[g]);
        lsum[g] += p;
#pragma unroll
        for (int w = 0; w < WORDS; ++w) o[g][w] = fmaf(p, __uint_as_float(vr[u][w]), o[g][w]);
      }
    }
  }
}

// The two values of x held by this lane and by lane ^ OFF, in an order that
// is the same on both lanes (lower lane's value first), so that a symmetric
// combination of them gives identical bits on both.
template <int OFF>
__device__ __forceinline__ void lane_pair(float x, float& lo, float& hi) {
  if constexpr (OFF == 16 || OFF == 32) {
    // permlane swaps return (even block's value, odd block's value) on both lanes
    auto r = OFF == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                          false, false)
                       : __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                          false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
  } else {
    float other;
    if constexpr (OFF == 8)
      other = dpp_f<0x128>(x);  // row_ror:8 within a 16-lane row = lane ^ 8
    else
      other = __shfl_xor(x, OFF);
    const bool upper = (threadIdx.x & OFF) != 0;
    lo = upper ? other : x;
    hi = upper ? x : other;
  }
}

// Merge the running (m, l, o) of the slots that differ in lane bit OFF.
template <typename SH, int G, int OFF>
__device__ __forceinline__ void merge_slots(float (&m)[G], float (&lsum)[G],
                                            float (&o)[G][SH::DPL]) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float m0, m1, l0, l1;
    lane_pair<OFF>(m[g], m0, m1);
    lane_pair<OFF>(lsum[g], l0, l1);
    const float mn = fmaxf(m0, m1);
    const float c0 = fast_exp2(m0 - mn);
    const float c1 = fast_exp2(m1 - mn);
    m[g] = mn;
    lsum[g] = l0 * c0 + l1 * c1;
#pragma unroll
    for (int i = 0; i < SH::DPL; ++i) {
      float o0, o1;
      lane_pair<OFF>(o[g][i], o0, o1);
      o[g][i] = o0 * c0 + o1 * c1;
    }
  }
}

// One work item, run by one wave: keys [kbeg, kend) (kbeg a multiple of 16,
// kend > kbeg) of sequence `seq` for query row `token`, one KV head. Range
// `part` of the row's `nparts`; its partials go to slot pslot + part.
template <typename ET, int D, int G, bool TOKEN_MODE>
__device__ __forceinline__ void decode_segment(const AttnArgs& a, int seq, int token, int pslot,
                                               int kbeg, int kend, int part, int nparts,
                                               int kvh) {
  typedef DecodeShape<ET, D> SH;
  constexpr int LPK = SH::LPK, WORDS = SH::WORDS, LOADS = SH::LOADS, DPL = SH::DPL;
  constexpr int KPI = SH::KPI, NSLOT = SH::KPW;

  const int lane = threadIdx.x & 63;
  const int sub = lane % LPK;
  const int slot = lane / LPK;
  const int p_shift = a.p_shift;

  // Page ids of the partition: lane i holds page pg0 + i (a partition spans
  // at most 64 pages: PT <= 63 * P).
  const int pg0 = kbeg >> p_shift;
  const int npg = ((kend - 1) >> p_shift) - pg0 + 1;
  const int* bt_row = a.block_tables + (size_t)seq * a.max_blocks;
  const int page_reg = lane < npg ? clampi(bt_row[pg0 + lane], 0, a.num_pages - 1) : 0;

  // The group's query rows, in the lane's dims.
  const size_t row_bytes = (size_t)D * SH::EB;
  const char* qrow = (const char*)a.q + ((size_t)token * a.Hq + (size_t)kvh * G) * row_bytes;
  uint32_t qw[G][WORDS];
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int l = 0; l < LOADS; ++l) {
      const uint4 x = *reinterpret_cast<const uint4*>(qrow + g * row_bytes + (l * LPK + sub) * 16);
      qw[g][4 * l] = x.x; qw[g][4 * l + 1] = x.y; qw[g][4 * l + 2] = x.z; qw[g][4 * l + 3] = x.w;
    }
  }

  float m[G], lsum[G], o[G][DPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegBig;
    lsum[g] = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[g][i] = 0.f;
  }

  const char* kbase = (const char*)a.k_pool + (size_t)kvh * row_bytes;
  const char* vbase = (const char*)a.v_pool + (size_t)kvh * row_bytes;
  const size_t slot_stride = (size_t)a.Hkv * row_bytes;  // bytes between consecutive slots
  const uint32_t lane_off = (uint32_t)(slot * slot_stride) + sub * 16;
  const float sl2e = a.scale_log2e;

  // Two register buffers alternate: while one computes, the other's loads are
  // in flight. Every iteration issues the same loads, so the compiler waits
  // only for the buffer being consumed; the last one or two buffers are
  // peeled so that no load is issued past the partition.
  uint32_t kA[SH::UNROLL][WORDS], vA[SH::UNROLL][WORDS];
  uint32_t kB[SH::UNROLL][WORDS], vB[SH::UNROLL][WORDS];
  const int nbuf = (kend - kbeg + KPI - 1) / KPI;  // >= 1, wave-uniform
  int kb = kbeg;
  load_buf<SH>(kA, vA, kbase, vbase, page_reg, pg0, p_shift, slot_stride, kb, lane_off);
  int j = 0;
  for (; j + 2 < nbuf; j += 2) {
    load_buf<SH>(kB, vB, kbase, vbase, page_reg, pg0, p_shift, slot_stride, kb + KPI, lane_off);
    __builtin_amdgcn_sched_barrier(0);  // keep the next buffer's loads ahead of this compute
    compute_buf<SH, G>(kA, vA, qw, m, lsum, o, kb, kend, slot, sl2e);
    load_buf<SH>(kA, vA, kbase, vbase, page_reg, pg0, p_shift, slot_stride, kb + 2 * KPI,
                 lane_off);
    __builtin_amdgcn_sched_barrier(0);
    compute_buf<SH, G>(kB, vB, qw, m, lsum, o, kb + KPI, kend, slot, sl2e);
    kb += 2 * KPI;
  }
  if (j + 1 < nbuf) {
    load_buf<SH>(kB, vB, kbase, vbase, page_reg, pg0, p_shift, slot_stride, kb + KPI, lane_off);
    __builtin_amdgcn_sched_barrier(0);
    compute_buf<SH, G>(kA, vA, qw, m, lsum, o, kb, kend, slot, sl2e);
    compute_buf<SH, G>(kB, vB, qw, m, lsum, o, kb + KPI, kend, slot, sl2e);
  } else {
    compute_buf<SH, G>(kA, vA, qw, m, lsum, o, kb, kend, slot, sl2e);
  }

  // Merge the slots (lanes sub, sub + LPK, ...): after the butterfly every
  // slot holds the merged state.
  if constexpr (LPK <= 4) merge_slots<SH, G, 4>(m, lsum, o);
  if constexpr (LPK <= 8) merge_slots<SH, G, 8>(m, lsum, o);
  if constexpr (LPK <= 16) merge_slots<SH, G, 16>(m, lsum, o);
  merge_slots<SH, G, 32>(m, lsum, o);
  static_assert(LPK >= 4, "at most 16 slots");

  // Slot s writes the heads g with g % NSLOT == s.
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (g % NSLOT != slot) continue;
    const int h = kvh * G + g;
    if (nparts == 1) {
      const float inv = 1.f / lsum[g];
      char* orow = (char*)a.out + ((size_t)token * a.Hq + h) * row_bytes;
      if constexpr (SH::EB == 2) {
#pragma unroll
        for (int l = 0; l < LOADS; ++l) {
          uint32_t wv[4];
#pragma unroll
          for (int w = 0; w < 4; ++w)
            wv[w] = pack_bf16x2(o[g][8 * l + 2 * w] * inv, o[g][8 * l + 2 * w + 1] * inv);
          *reinterpret_cast<uint4*>(orow + (l * LPK + sub) * 16) =
              make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
      } else {
#pragma unroll
        for (int l = 0; l < LOADS; ++l)
          *reinterpret_cast<float4*>(orow + (l * LPK + sub) * 16) =
              make_float4(o[g][4 * l] * inv, o[g][4 * l + 1] * inv, o[g][4 * l + 2] * inv,
                          o[g][4 * l + 3] * inv);
      }
    } else {
      const size_t pi = ((size_t)pslot + part) * a.Hq + h;
      float* po = a.ws + pi * D;
#pragma unroll
      for (int i = 0; i < DPL; i += 4)
        *reinterpret_cast<float4*>(po + SH::dim_of(sub, i)) =
            make_float4(o[g][i], o[g][i + 1], o[g][i + 2], o[g][i + 3]);
      if (sub == 0) {
        float* ml = a.ws + (size_t)a.part_slots * a.Hq * D;
        *reinterpret_cast<float2*>(ml + 2 * pi) = make_float2(m[g], lsum[g]);
      }
    }
  }
}

template <typename ET, int D, int G, bool TOKEN_MODE>
__global__ __launch_bounds__(kThreads) void decode_kernel(AttnArgs a) {
  // bf16: each wave's K/V buffers in LDS (see dec_issue)
  __shared__ uint4 s_kreg[ET::kBytes == 2 ? kWaves * dec_region_units<(D >= 64 ? D : 64)>() : 1];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if constexpr (TOKEN_MODE) {
    const long unit = (long)blockIdx.x * kWaves + wave;
    const int kvh = (int)(unit % a.Hkv);
    const long rest = unit / a.Hkv;
    if (rest >= (long)a.T * a.max_parts) return;
    const int row = (int)(rest / a.max_parts), part = (int)(rest % a.max_parts);
    const RowInfo ri = row_info<true>(a, row);
    if (!ri.active) return;
    const int PT = a.part_tokens;
    const int nparts = (ri.n_eff + PT - 1) / PT;
    if (part >= nparts) return;
    const int kbeg = part * PT;
    if constexpr (ET::kBytes == 2)
    {
      const DecSeg d{ri.seq, row, row * a.max_parts, kbeg, min(ri.n_eff, kbeg + PT), part,
                     nparts, kvh};
      decode_range_alone<D, G>(a, d, s_kreg + wave * dec_region_units<D>());
    }
    else
      decode_segment<ET, D, G, true>(a, ri.seq, row, row * a.max_parts, kbeg,
                                     min(ri.n_eff, kbeg + PT), part, nparts, kvh);
  } else {
    if constexpr (ET::kBytes == 2) {
      decode_chunks_mfma<D, G>(a, blockIdx.x, s_kreg);
    } else {
      decode_walk(a, blockIdx.x,
                  [&](int seq, int token, int pslot, int kbeg, int kend, int part, int nparts,
                      int kvh) {
                    decode_segment<ET, D, G, false>(a, seq, token, pslot, kbeg, kend, part, nparts,
                                                    kvh);
                  });
    }
  }
}

// K3: kMergeLanes threads per (row, query head, 4 consecutive dims); the body is
// split_reduce_task (pa_decode_mfma.h), shared with the fused tick's reduce.
template <typename ET, bool TOKEN_MODE>
__global__ __launch_bounds__(256) void split_reduce_kernel(AttnArgs a) {
  split_reduce_task<ET, TOKEN_MODE>(a, (long)blockIdx.x * 256 + threadIdx.x);
}

// ------------------------------------------------------------ dispatch -----
template <typename ET, int D, int G>
static int decode_grid_t() {
  int resident = persistent_grid((const void*)decode_kernel<ET, D, G, false>, kThreads);
  if (ET::kBytes == 2) resident = min(resident, cu_count() * kDecodeWgPerCu);
  return resident > 8 ? resident - resident % 8 : 8;
}

template <typename ET, int D, int G>
static hipError_t launch_decode_t(const AttnArgs& a, bool token_mode, hipStream_t s) {
  if (token_mode) {
    const long units = (long)a.T * a.max_parts * a.Hkv;
    const long blocks = (units + kWaves - 1) / kWaves;
    if (blocks == 0) return hipSuccess;
    profile_before("decode_attention_tokens", s);
    hipLaunchKernelGGL((decode_kernel<ET, D, G, true>), dim3((unsigned)blocks), dim3(kThreads),
                       0, s, a);
    profile_after(s);
    return hipGetLastError();
  }
  if (a.cap_dec == 0) return hipSuccess;
  // a multiple of 8 (so of Hkv): workgroup b keeps KV head b % Hkv
  const int grid = a.dec_grid;
  profile_before("decode_attention", s);
  hipLaunchKernelGGL((decode_kernel<ET, D, G, false>), dim3((unsigned)grid), dim3(kThreads), 0,
                     s, a);
  profile_after(s);
  return hipGetLastError();
}

template <typename ET, int D>
static int decode_grid_d(int G) {
  switch (G) {
    case 1: return decode_grid_t<ET, D, 1>();
    case 2: return decode_grid_t<ET, D, 2>();
    case 4: return decode_grid_t<ET, D, 4>();
    case 8: return decode_grid_t<ET, D, 8>();
  }
  return 8;
}

template <typename ET, int D>
static hipError_t launch_decode_d(const AttnArgs& a, int G, bool tm, hipStream_t s) {
  switch (G) {
    case 1: return launch_decode_t<ET, D, 1>(a, tm, s);
    case 2: return launch_decode_t<ET, D, 2>(a, tm, s);
    case 4: return launch_decode_t<ET, D, 4>(a, tm, s);
    case 8: return launch_decode_t<ET, D, 8>(a, tm, s);
  }
  return hipErrorInvalidValue;
}

bool decode_supported(pa_dtype_t dt, int D, int G) {
  const bool g_ok = G == 1 || G == 2 || G == 4 || G == 8;
  if (dt == PA_F32) return g_ok && (D == 16 || D == 64 || D == 128);
  if (dt == PA_BF16) return g_ok && (D == 64 || D == 128);
  return false;
}

int decode_grid(pa_dtype_t dt, int D, int G) {
  if (dt == PA_F32) {
    switch (D) {
      case 16: return decode_grid_d<F32, 16>(G);
      case 64: return decode_grid_d<F32, 64>(G);
      case 128: return decode_grid_d<F32, 128>(G);
    }
  } else {
    switch (D) {
      case 64: return decode_grid_d<BF16, 64>(G);
      case 128: return decode_grid_d<BF16, 128>(G);
    }
  }
  return 8;
}

int decode_grid_max(pa_dtype_t dt, int D) {
  int g = 8;
  for (int G = 1; G <= 8; G *= 2) g = max(g, decode_grid(dt, D, G));
  return g;
}

hipError_t launch_decode(pa_dtype_t dt, const AttnArgs& a, bool token_mode, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  if (dt == PA_F32) {
    switch (a.D) {
      case 16: return launch_decode_d<F32, 16>(a, G, token_mode, s);
      case 64: return launch_decode_d<F32, 64>(a, G, token_mode, s);
      case 128: return launch_decode_d<F32, 128>(a, G, token_mode, s);
    }
  } else {
    switch (a.D) {
      case 64: return launch_decode_d<BF16, 64>(a, G, token_mode, s);
      case 128: return launch_decode_d<BF16, 128>(a, G, token_mode, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_split_reduce(pa_dtype_t dt, const AttnArgs& a, bool token_mode,
                               hipStream_t s) {
  const long rows = token_mode ? a.T : plan_rows(a.S);
  const long threads = rows * a.Hq * (a.D / 4) * kMergeLanes;
  if (threads == 0 || a.max_parts <= 1) return hipSuccess;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  profile_before(token_mode ? "split_reduce_tokens" : "split_reduce", s);
  if (dt == PA_BF16) {
    if (token_mode)
      hipLaunchKernelGGL((split_reduce_kernel<BF16, true>), dim3(blocks), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((split_reduce_kernel<BF16, false>), dim3(blocks), dim3(256), 0, s, a);
  } else {
    if (token_mode)
      hipLaunchKernelGGL((split_reduce_kernel<F32, true>), dim3(blocks), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((split_reduce_kernel<F32, false>), dim3(blocks), dim3(256), 0, s, a);
  }
  profile_after(s);
  return hipGetLastError();
}

}  // namespace pa
