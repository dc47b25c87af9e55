// The fused tick kernel: decode rows and prefill chunks of one packed tick in
// one persistent grid (the packed tick as a single forward: Helios blog,
// "Continuous batching" and "Prefill vs Decode").
//
// Decode streams K/V from HBM on VALU and one MFMA per 16 keys; prefill
// chunks are matrix-core and LDS work. Run one after the other, each leaves
// the other's units idle; in one grid they share every CU. The grid holds two
// workgroups per CU (the prefill item's LDS and registers decide the shape):
//   workgroups [0, dec_grid) are dispatched first, one per CU, and walk the
//     decode chunks (the same per-wave chunks as the decode kernel);
//   the others take prefill items from a queue in decreasing-cost order
//     (longest first), and decode workers join that queue when their chunks
//     are done. Workgroup b serves KV head b % Hkv first (the XCD that runs
//     it, with the grid a multiple of 8), so each XCD's L2 holds the K/V tiles
//     of its own heads, which every row tile of a chunk re-reads; when that
//     head's queue is empty it takes the other heads' items in turn. There is
//     one queue per KV head; its cursor is a counter in the plan workspace,
//     zeroed by the plan kernel and advanced with a device-scope atomic.
// Split-KV partials of decode rows (K3's merge) and the pieces of cut prefill
// items are merged afterwards by one reduce launch.
#include "pa_decode_mfma.h"
#include "pa_prefill_mfma.h"

namespace pa {

namespace {

// Next prefill item of a queue for the whole workgroup: thread 0 claims it
// and, in the same round trip, reads how many queues are known to be empty;
// the others read both from LDS. The one claim that returns n_items exactly
// (the first past the queue's end) adds its queue to that count.
__device__ __forceinline__ int2 pf_take(int* cursor, int* dry, int n_items, int2* s_slot) {
  if (threadIdx.x == 0) {
    const int it = __hip_atomic_fetch_add(cursor, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int d = __hip_atomic_load(dry, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (it == n_items) __hip_atomic_fetch_add(dry, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_slot = make_int2(it, d + (it == n_items ? 1 : 0));
  }
  __syncthreads();
  const int2 r = *s_slot;
  __syncthreads();  // everyone has read the slot before it is written again
  return r;
}

template <int D, int G>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(2))) void tick_kernel(
    AttnArgs a) {
  __shared__ PfSmem<D> sm;
  __shared__ int2 s_next;
  static_assert(kPfThreads == 64 * 4, "decode workers are workgroups of four waves");
  // decode workers keep their K/V buffers in the (not yet used) prefill tile
  // buffers: sm.k and sm.v, which follow each other
  static_assert(offsetof(PfSmem<D>, v) == sizeof(sm.k) &&
                    sizeof(sm.k) + sizeof(sm.v) >= 4 * dec_region_bytes<D>(),
                "decode K/V buffers fit");
  if ((int)blockIdx.x < a.dec_grid)
    decode_chunks_mfma<D, G>(a, blockIdx.x, reinterpret_cast<uint4*>(sm.k));

  const PlanOffsets po = plan_offsets(a.S, a.Hq, a.cap_dec, a.cap_pf);
  const int4* items = reinterpret_cast<const int4*>(a.plan + po.pf);
  const int4* shapes = reinterpret_cast<const int4*>(a.plan + po.pf_shape);
  const int n_items = a.plan[1];
  int* dry = a.plan + plan_pf_dry();
  const int home = blockIdx.x % a.Hkv;
  for (int hh = 0; hh < a.Hkv; ++hh) {
    const int kvh = home + hh < a.Hkv ? home + hh : home + hh - a.Hkv;
    int* cursor = a.plan + plan_pf_cursor(kvh);
    // the entry index (read from LDS) is the same in every lane: reading it
    // from the first lane tells the compiler, so the entry and everything
    // derived from it stay in scalar registers with scalar branches
    int2 c = pf_take(cursor, dry, n_items, &s_next);
    int it = __builtin_amdgcn_readfirstlane(c.x);
    while (it < n_items) {
      // (the next entry is claimed only once this one is done: claimed ahead,
      // the last entries sat with busy workgroups while the decode workers,
      // done with their rows, found the queues empty)
      // Prefill waves issue ahead of the decode waves sharing their CU: a
      // prefill tile stalls the whole workgroup at its barriers when its
      // loads or MFMAs wait, while the decode waves' deep load queues absorb
      // the delay (measured: the fused tick ~13% shorter, decode unchanged).
      __builtin_amdgcn_s_setprio(2);
      prefill_item<D, G>(a, sm, items[it], shapes[it], kvh);
      __builtin_amdgcn_s_setprio(0);
      c = pf_take(cursor, dry, n_items, &s_next);
      it = __builtin_amdgcn_readfirstlane(c.x);
    }
    // every queue is known to be empty: the rest of the walk would only claim
    // past their ends, one round trip each
    if (__builtin_amdgcn_readfirstlane(c.y) >= a.Hkv) break;
  }
}

template <int D, int G>
int tick_grid_t() {
  const int grid = persistent_grid((const void*)tick_kernel<D, G>, kPfThreads);
  return grid > 8 ? grid - grid % 8 : 8;  // workgroup b on XCD b % 8 serves KV head b % Hkv
}

template <int D, int G>
hipError_t launch_tick_t(const AttnArgs& a, hipStream_t s) {
  const int grid = tick_grid_t<D, G>();
  profile_before("tick_attention", s);
  hipLaunchKernelGGL((tick_kernel<D, G>), dim3((unsigned)grid), dim3(kPfThreads), 0, s, a);
  profile_after(s);
  return hipGetLastError();
}

template <int D>
hipError_t launch_tick_d(const AttnArgs& a, int G, hipStream_t s) {
  switch (G) {
    case 1: return launch_tick_t<D, 1>(a, s);
    case 2: return launch_tick_t<D, 2>(a, s);
    case 4: return launch_tick_t<D, 4>(a, s);
    case 8: return launch_tick_t<D, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

// Merge of the pieces of one row of a cut prefill item, 4 dims per thread:
// m* = max_j m_j and o = sum_j 2^(m_j - m*) o_j / sum_j 2^(m_j - m*) l_j,
// rounded to bf16. The J pieces' loads are independent, so they overlap.
__device__ __forceinline__ void prefill_merge_row(const AttnArgs& a, int slot0, int J, int r,
                                                  int d4, uint16_t* orow) {
  const int D = a.D;
  const float* po = a.pf_ws;
  const float* pml = a.pf_ws + (size_t)a.pf_slots * kPrefillRows * D;
  float mx = kNegBig;
  for (int j = 0; j < J; ++j) mx = fmaxf(mx, pml[2 * ((size_t)(slot0 + j) * kPrefillRows + r)]);
  float lt = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < J; ++j) {
    const size_t sr = (size_t)(slot0 + j) * kPrefillRows + r;
    const float2 ml = *reinterpret_cast<const float2*>(pml + 2 * sr);
    const float4 o = *reinterpret_cast<const float4*>(po + sr * D + 4 * d4);
    const float c = fast_exp2(ml.x - mx);
    lt = fmaf(ml.y, c, lt);
    acc.x = fmaf(o.x, c, acc.x);
    acc.y = fmaf(o.y, c, acc.y);
    acc.z = fmaf(o.z, c, acc.z);
    acc.w = fmaf(o.w, c, acc.w);
  }
  const float inv = 1.f / lt;
  *reinterpret_cast<uint2*>(orow + 4 * d4) =
      make_uint2(pack_bf16x2(acc.x * inv, acc.y * inv), pack_bf16x2(acc.z * inv, acc.w * inv));
}

// After the tick: the first dec_blocks workgroups merge the split-KV
// partitions of the decode rows (kMergeLanes threads per row, head and 4
// dims); each
// of the others merges the pieces of a group of rows of one (cut prefill
// item, KV head), one thread per row and 4 dims.
constexpr int kReduceThreads = 256;

__global__ __launch_bounds__(kReduceThreads) void tick_reduce_kernel(AttnArgs a, int dec_blocks) {
  if ((int)blockIdx.x < dec_blocks) {
    split_reduce_task<BF16, false>(a, (long)blockIdx.x * kReduceThreads + threadIdx.x);
    return;
  }
  const int quads = a.D / 4;  // 16 or 32
  const int rows_per_wg = kReduceThreads / quads;
  const int groups = kPrefillRows / rows_per_wg;  // workgroups per (item, KV head)
  const int b = (int)blockIdx.x - dec_blocks;
  const int pair = b / groups, rg = b % groups;  // pair = cut item * Hkv + KV head
  if (pair >= a.plan[5] * a.Hkv) return;
  const int kvh = pair % a.Hkv;
  const int4* cut = reinterpret_cast<const int4*>(
      a.plan + plan_offsets(a.S, a.Hq, a.cap_dec, a.cap_pf).merge);
  const int4 e = cut[pair / a.Hkv];  // (sequence, row tile, pieces J, first slot)
  const int G = a.Hq / a.Hkv, TM = kPrefillRows / G;
  const int q0 = a.qsl[e.x];
  const int L = a.qsl[e.x + 1] - q0;
  const int r = rg * rows_per_wg + (int)threadIdx.x / quads, d4 = (int)threadIdx.x % quads;
  const int tok = e.y * TM + r / G;
  if (tok >= min(L, e.y * TM + TM)) return;
  uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) +
                   ((size_t)(q0 + tok) * a.Hq + kvh * G + r % G) * a.D;
  prefill_merge_row(a, e.w + kvh * e.z, e.z, r, d4, orow);
}

template <int D>
int tick_grid_d(int G) {
  switch (G) {
    case 1: return tick_grid_t<D, 1>();
    case 2: return tick_grid_t<D, 2>();
    case 4: return tick_grid_t<D, 4>();
    case 8: return tick_grid_t<D, 8>();
  }
  return 8;
}

}  // namespace

bool tick_supported(pa_dtype_t dt, int D) { return dt == PA_BF16 && (D == 64 || D == 128); }

int tick_grid(pa_dtype_t dt, int D, int G) {
  if (!tick_supported(dt, D)) return 8;
  return D == 64 ? tick_grid_d<64>(G) : tick_grid_d<128>(G);
}

hipError_t launch_tick_reduce(const AttnArgs& a, hipStream_t s) {
  const long dec_threads =
      a.max_parts > 1 ? plan_rows(a.S) * a.Hq * (a.D / 4) * kMergeLanes : 0;
  const int dec_blocks = (int)((dec_threads + kReduceThreads - 1) / kReduceThreads);
  // cut items use at least 2 Hkv partial slots each: at most pf_slots / 2
  // (item, KV head) pairs, kPrefillRows * (D / 4) threads per pair
  const long merge_threads = (long)(a.pf_slots / 2) * kPrefillRows * (a.D / 4);
  const int blocks = dec_blocks + (int)((merge_threads + kReduceThreads - 1) / kReduceThreads);
  if (blocks == 0) return hipSuccess;
  profile_before("tick_reduce", s);
  hipLaunchKernelGGL(tick_reduce_kernel, dim3(blocks), dim3(kReduceThreads), 0, s, a, dec_blocks);
  profile_after(s);
  return hipGetLastError();
}

hipError_t launch_tick(pa_dtype_t dt, const AttnArgs& a, hipStream_t s) {
  if (!tick_supported(dt, a.D)) return hipErrorInvalidValue;
  const int G = a.Hq / a.Hkv;
  return a.D == 64 ? launch_tick_d<64>(a, G, s) : launch_tick_d<128>(a, G, s);
}

}  // namespace pa
