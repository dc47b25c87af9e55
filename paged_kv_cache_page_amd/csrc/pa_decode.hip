// K2: paged decode attention with split-KV partitions. K3: merge of the partitions.
//
// Decode is HBM-bound: every key row of a (sequence, KV head) is read once and
// used by all G query heads of its group (grouped-query attention: Helios blog,
// "torch.sdpa and Flash Attention"), about 2*G flops per byte. The kernel is
// written for that bound: VALU dot products (no matrix cores), 16-byte row
// loads through the page table, the next step's loads in flight while the
// current step computes, and the softmax kept online in registers.
//
// Work decomposition. A work item is (row, split partition, KV head). For the
// decode rows of a tick the items come from the plan list and a persistent
// grid walks them (item index w -> KV head w % Hkv, so with a grid that is a
// multiple of 8 each workgroup keeps one KV head, and with 8 KV heads each
// XCD serves one head: the slices of a prefix page shared by many sequences
// then stay in that XCD's L2). The per-token mode (prefill rows without a
// matrix-core kernel, i.e. float32) uses a plain grid over (token, partition,
// KV head).
//
// Inside a wave, LPK lanes hold one key row (16 or 32 bytes each), so a wave
// covers 64 / LPK keys per step and UNROLL steps per iteration. Each lane
// keeps its own running (max, sum, output) over the keys of its slot; slots
// are merged with cross-lane shuffles at the end, waves through LDS.
//
// A partition's result is either final (the row has one partition) or a
// partial (m, l, o) in the workspace, merged by K3:
//   m* = max_k m_k,  o = sum_k 2^(m_k - m*) o_k / sum_k 2^(m_k - m*) l_k.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxPartPages = 256;

template <typename ET, int D>
struct DecodeShape {
  static constexpr int EB = ET::kBytes;
  static constexpr int ROWB = D * EB;  // bytes of one head row
  static constexpr int LPK = ROWB >= 256 ? (ROWB / 32 > 16 ? 16 : ROWB / 32) : ROWB / 16;
  static constexpr int LANE_BYTES = ROWB / LPK;  // 16 or 32
  static constexpr int LOADS = LANE_BYTES / 16;  // 16-byte loads per lane per row
  static constexpr int WORDS = LANE_BYTES / 4;   // 32-bit words per lane per row
  static constexpr int DPL = D / LPK;            // head dims held by a lane
  static constexpr int EPV = 16 / EB;            // elements per 16-byte vector
  static constexpr int KPW = 64 / LPK;           // keys per wave step (slots)
  // steps per buffer: a buffer always covers 16 consecutive keys, so with pages
  // of >= 16 keys (a power of two) and 16-aligned starts it never crosses a page
  static constexpr int UNROLL = 16 / KPW;
  static constexpr int KPI = KPW * UNROLL;       // keys per buffer (16)
  static_assert(LANE_BYTES == 16 || LANE_BYTES == 32, "lane row share must be 16 or 32 bytes");
  static_assert(KPI == 16, "a buffer covers 16 keys");
  static_assert(EB == 4 || UNROLL == 2, "bf16 P.V pairs the two steps of a buffer");
  // Head-dim index of the lane's local dim i (sub = lane % LPK).
  __device__ static int dim_of(int sub, int i) {
    return ((i / EPV) * LPK + sub) * EPV + (i % EPV);
  }
};

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
  int n = a.seq_lens[s];
  const int cap = a.max_blocks * a.P;
  n = n < cap ? n : cap;
  r.seq = s;
  r.n_eff = n - L + i + 1;
  r.active = r.n_eff > 0;
  return r;
}

template <typename ET, int D, int G>
struct DecodeSmem {
  int pages[kMaxPartPages];
  float o[kWaves][G][D];
  float m[kWaves][G];
  float l[kWaves][G];
};

// Issue the loads of one buffer: the 16 keys starting at `base` (wave-uniform,
// a multiple of 16), all in one page. The page and the row of `base` are
// wave-uniform, so the address is a scalar base plus a per-lane 32-bit offset
// fixed for the whole item; past the end of the range the buffer re-reads the
// range's first keys (its values are then masked).
template <typename SH>
__device__ __forceinline__ void load_step(uint32_t (&kr)[SH::UNROLL][SH::WORDS],
                                          uint32_t (&vr)[SH::UNROLL][SH::WORDS],
                                          const char* kbase, const char* vbase,
                                          const int* pages, int pg0, int p_shift,
                                          size_t slot_stride, int base, int kbeg, int kend,
                                          uint32_t lane_off) {
  const int bb = base < kend ? base : kbeg;
  const int page = __builtin_amdgcn_readfirstlane(pages[(bb >> p_shift) - pg0]);
  const int row0 = bb & ((1 << p_shift) - 1);
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

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2e_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Scores, online softmax and P.V for one buffer (16 keys of the wave).
template <typename SH, int G>
__device__ __forceinline__ void compute_step(const uint32_t (&kr)[SH::UNROLL][SH::WORDS],
                                             uint32_t (&vr)[SH::UNROLL][SH::WORDS],
                                             const uint32_t (&qw)[G][SH::WORDS], float (&m)[G],
                                             float (&lsum)[G], float (&o)[G][SH::DPL], int base,
                                             int kend, int slot, float sl2e) {
  constexpr int UNROLL = SH::UNROLL, WORDS = SH::WORDS, DPL = SH::DPL;
  bool valid[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) valid[u] = base + u * SH::KPW + slot < kend;
  // Rows past the end may hold anything (NaN included); zero their V so that
  // a zero weight times them stays zero. Only the last buffer of a range is
  // partial, and the test is wave-uniform.
  if (base + SH::KPI > kend) {
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
  // bf16: the two steps' V rows interleaved per dim, (v_u0[d], v_u1[d]), so
  // that one v_dot2 adds both keys' contributions to one output dim.
  uint32_t vlo[SH::EB == 2 ? WORDS : 1], vhi[SH::EB == 2 ? WORDS : 1];
  if constexpr (SH::EB == 2) {
#pragma unroll
    for (int w = 0; w < WORDS; ++w) {
      vlo[w] = __builtin_amdgcn_perm(vr[1][w], vr[0][w], 0x05040100u);
      vhi[w] = __builtin_amdgcn_perm(vr[1][w], vr[0][w], 0x07060302u);
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
      // weights rounded to bf16 once; the sum uses the same rounded values
      const f32x2_t pf = {fast_exp2(sc[0][g] - m[g]), fast_exp2(sc[1][g] - m[g])};
      const uint32_t pp = __builtin_bit_cast(uint32_t, __builtin_convertvector(pf, bf16x2e_t));
      lsum[g] += bf16_lo(pp) + bf16_hi(pp);
#pragma unroll
      for (int w = 0; w < WORDS; ++w) {
        o[g][2 * w] = dot2_bf16(pp, vlo[w], o[g][2 * w]);
        o[g][2 * w + 1] = dot2_bf16(pp, vhi[w], o[g][2 * w + 1]);
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

// One work item: keys [part * PT, min(n_eff, (part + 1) * PT)) of one row, one KV head.
template <typename ET, int D, int G, bool TOKEN_MODE>
__device__ __forceinline__ void decode_item(const AttnArgs& a, DecodeSmem<ET, D, G>& sm, int row,
                                            int part, int kvh) {
  typedef DecodeShape<ET, D> SH;
  constexpr int LPK = SH::LPK, WORDS = SH::WORDS, LOADS = SH::LOADS, DPL = SH::DPL;
  constexpr int KPI = SH::KPI;

  const RowInfo ri = row_info<TOKEN_MODE>(a, row);
  if (!ri.active) return;
  const int PT = a.part_tokens;
  const int kbeg = part * PT;
  if (kbeg >= ri.n_eff) return;
  const int kend = min(ri.n_eff, kbeg + PT);
  const int nparts = (ri.n_eff + PT - 1) / PT;

  const int pg0 = kbeg >> a.p_shift;
  const int npg = ((kend - 1) >> a.p_shift) - pg0 + 1;
  const int* bt_row = a.block_tables + (size_t)ri.seq * a.max_blocks;
  for (int i = threadIdx.x; i < npg; i += kThreads)
    sm.pages[i] = clampi(bt_row[pg0 + i], 0, a.num_pages - 1);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (SGPR)
  const int sub = lane % LPK;
  const int slot = lane / LPK;

  // The group's query rows, in the lane's dims.
  const size_t row_bytes = (size_t)D * SH::EB;
  const char* qrow = (const char*)a.q + ((size_t)ri.token * a.Hq + (size_t)kvh * G) * row_bytes;
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
  __syncthreads();  // pages ready

  const char* kbase = (const char*)a.k_pool + (size_t)kvh * row_bytes;
  const char* vbase = (const char*)a.v_pool + (size_t)kvh * row_bytes;
  const size_t slot_stride = (size_t)a.Hkv * row_bytes;  // bytes between consecutive slots
  const uint32_t lane_off = (uint32_t)(slot * slot_stride) + sub * 16;
  const float sl2e = a.scale_log2e;
  const int p_shift = a.p_shift;
  constexpr int STEP = kWaves * KPI;

  // Two register buffers alternate: while one computes, the other's loads are
  // in flight. The loads are issued unconditionally, so the number of
  // outstanding loads is the same on every path and the compiler waits only
  // for the buffer being consumed.
  uint32_t kA[SH::UNROLL][WORDS], vA[SH::UNROLL][WORDS];
  uint32_t kB[SH::UNROLL][WORDS], vB[SH::UNROLL][WORDS];
  int base = kbeg + wave * KPI;
  const int nsteps = base < kend ? (kend - base + STEP - 1) / STEP : 0;  // wave-uniform
  load_step<SH>(kA, vA, kbase, vbase, sm.pages, pg0, p_shift, slot_stride, base, kbeg, kend,
                lane_off);
  for (int it = 0; it < nsteps; it += 2) {
    load_step<SH>(kB, vB, kbase, vbase, sm.pages, pg0, p_shift, slot_stride, base + STEP, kbeg,
                  kend, lane_off);
    __builtin_amdgcn_sched_barrier(0);  // keep the next buffer's loads ahead of this compute
    compute_step<SH, G>(kA, vA, qw, m, lsum, o, base, kend, slot, sl2e);
    base += STEP;
    load_step<SH>(kA, vA, kbase, vbase, sm.pages, pg0, p_shift, slot_stride, base + STEP, kbeg,
                  kend, lane_off);
    __builtin_amdgcn_sched_barrier(0);
    if (it + 1 < nsteps) compute_step<SH, G>(kB, vB, qw, m, lsum, o, base, kend, slot, sl2e);
    base += STEP;
  }

  // Merge the slots of this wave (lanes sub, sub + LPK, ...).
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float m2 = __shfl_xor(m[g], off);
      const float l2 = __shfl_xor(lsum[g], off);
      const float mn = fmaxf(m[g], m2);
      const float ca = fast_exp2(m[g] - mn);
      const float cb = fast_exp2(m2 - mn);
      m[g] = mn;
      lsum[g] = lsum[g] * ca + l2 * cb;
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        const float o2 = __shfl_xor(o[g][i], off);
        o[g][i] = o[g][i] * ca + o2 * cb;
      }
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int i = 0; i < DPL; ++i) sm.o[wave][g][SH::dim_of(sub, i)] = o[g][i];
      if (sub == 0) {
        sm.m[wave][g] = m[g];
        sm.l[wave][g] = lsum[g];
      }
    }
  }
  __syncthreads();

  // Merge the waves; write the final row or this partition's partial.
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int g = idx / D;
    const int e = idx % D;
    float mn = sm.m[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mn = fmaxf(mn, sm.m[w][g]);
    float lt = 0.f, ot = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float c = fast_exp2(sm.m[w][g] - mn);
      lt = fmaf(sm.l[w][g], c, lt);
      ot = fmaf(sm.o[w][g][e], c, ot);
    }
    const int h = kvh * G + g;
    if (nparts == 1) {
      const float val = ot / lt;
      const size_t oi = ((size_t)ri.token * a.Hq + h) * D + e;
      if constexpr (SH::EB == 2)
        reinterpret_cast<uint16_t*>(a.out)[oi] = (uint16_t)f32_to_bf16(val);
      else
        reinterpret_cast<float*>(a.out)[oi] = val;
    } else {
      const size_t pi = ((size_t)row * a.max_parts + part) * a.Hq + h;
      a.ws[pi * D + e] = ot;
      if (e == 0) {
        float* ml = a.ws + (size_t)(TOKEN_MODE ? a.T : a.S) * a.max_parts * a.Hq * D;
        ml[2 * pi] = mn;
        ml[2 * pi + 1] = lt;
      }
    }
  }
}

template <typename ET, int D, int G, bool TOKEN_MODE>
__global__ __launch_bounds__(kThreads) void decode_kernel(AttnArgs a) {
  __shared__ DecodeSmem<ET, D, G> sm;
  if constexpr (TOKEN_MODE) {
    const int bid = blockIdx.x;
    const int kvh = bid % a.Hkv;
    const int rest = bid / a.Hkv;
    decode_item<ET, D, G, true>(a, sm, rest / a.max_parts, rest % a.max_parts, kvh);
  } else {
    const int* items = a.plan + kPlanHeaderInts;
    const int total = a.plan[0] * a.Hkv;
    for (int w = blockIdx.x; w < total; w += gridDim.x) {
      const int it = w / a.Hkv;
      decode_item<ET, D, G, false>(a, sm, items[2 * it], items[2 * it + 1], w % a.Hkv);
      __syncthreads();  // LDS is reused by the next item
    }
  }
}

template <typename ET, bool TOKEN_MODE>
__global__ __launch_bounds__(kThreads) void split_reduce_kernel(AttnArgs a, int G) {
  const int kvh = blockIdx.x % a.Hkv;
  const int row = blockIdx.x / a.Hkv;
  const RowInfo ri = row_info<TOKEN_MODE>(a, row);
  if (!ri.active) return;
  const int PT = a.part_tokens;
  int nparts = (ri.n_eff + PT - 1) / PT;
  if (nparts <= 1) return;
  nparts = nparts < a.max_parts ? nparts : a.max_parts;
  const int D = a.D;
  const float* ml = a.ws + (size_t)(TOKEN_MODE ? a.T : a.S) * a.max_parts * a.Hq * D;
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int g = idx / D;
    const int e = idx % D;
    const int h = kvh * G + g;
    const size_t p0 = (size_t)row * a.max_parts * a.Hq + h;  // partial index of part 0
    float mn = kNegBig;
    for (int k = 0; k < nparts; ++k) mn = fmaxf(mn, ml[2 * (p0 + (size_t)k * a.Hq)]);
    float lt = 0.f, ot = 0.f;
    for (int k = 0; k < nparts; ++k) {
      const size_t pi = p0 + (size_t)k * a.Hq;
      const float c = fast_exp2(ml[2 * pi] - mn);
      lt = fmaf(ml[2 * pi + 1], c, lt);
      ot = fmaf(a.ws[pi * D + e], c, ot);
    }
    const float val = ot / lt;
    const size_t oi = ((size_t)ri.token * a.Hq + h) * D + e;
    if constexpr (ET::kBytes == 2)
      reinterpret_cast<uint16_t*>(a.out)[oi] = (uint16_t)f32_to_bf16(val);
    else
      reinterpret_cast<float*>(a.out)[oi] = val;
  }
}

// ------------------------------------------------------------ dispatch -----
template <typename ET, int D, int G>
static hipError_t launch_decode_t(const AttnArgs& a, bool token_mode, hipStream_t s) {
  if (token_mode) {
    const long blocks = (long)a.T * a.max_parts * a.Hkv;
    if (blocks == 0) return hipSuccess;
    profile_before("decode_attention_tokens", s);
    hipLaunchKernelGGL((decode_kernel<ET, D, G, true>), dim3((unsigned)blocks), dim3(kThreads),
                       0, s, a);
    profile_after(s);
    return hipGetLastError();
  }
  const long items = (long)a.cap_dec * a.Hkv;
  if (items == 0) return hipSuccess;
  const int resident = persistent_grid((const void*)decode_kernel<ET, D, G, false>, kThreads);
  // a multiple of 8 (and of Hkv when Hkv divides 8) keeps each workgroup on one KV head
  long grid = items < resident ? items : resident;
  if (grid > 8) grid -= grid % 8;
  profile_before("decode_attention", s);
  hipLaunchKernelGGL((decode_kernel<ET, D, G, false>), dim3((unsigned)grid), dim3(kThreads), 0,
                     s, a);
  profile_after(s);
  return hipGetLastError();
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
  const long rows = token_mode ? a.T : a.S;
  const long blocks = rows * a.Hkv;
  if (blocks == 0 || a.max_parts <= 1) return hipSuccess;
  const int G = a.Hq / a.Hkv;
  profile_before(token_mode ? "split_reduce_tokens" : "split_reduce", s);
  if (dt == PA_BF16) {
    if (token_mode)
      hipLaunchKernelGGL((split_reduce_kernel<BF16, true>), dim3((unsigned)blocks),
                         dim3(kThreads), 0, s, a, G);
    else
      hipLaunchKernelGGL((split_reduce_kernel<BF16, false>), dim3((unsigned)blocks),
                         dim3(kThreads), 0, s, a, G);
  } else {
    if (token_mode)
      hipLaunchKernelGGL((split_reduce_kernel<F32, true>), dim3((unsigned)blocks),
                         dim3(kThreads), 0, s, a, G);
    else
      hipLaunchKernelGGL((split_reduce_kernel<F32, false>), dim3((unsigned)blocks),
                         dim3(kThreads), 0, s, a, G);
  }
  profile_after(s);
  return hipGetLastError();
}

}  // namespace pa
