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
//     are done. Workgroup b serves KV head b % Hkv (the XCD that runs it,
//     with the grid a multiple of 8), so each XCD's L2 holds the K/V tiles of
//     its own heads, which every row tile of a chunk re-reads. There is one
//     queue per KV head; its cursor is a counter in the plan header, zeroed by
//     the plan kernel and advanced with a device-wide atomic.
// Split-KV partials of decode rows are merged afterwards by K3, as with the
// decode kernel.
#include "pa_decode_mfma.h"
#include "pa_prefill_mfma.h"

namespace pa {

namespace {

template <int D, int G>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(2))) void tick_kernel(
    AttnArgs a) {
  __shared__ PfSmem<D> sm;
  __shared__ int s_next;
  static_assert(kPfThreads == 64 * 4, "decode workers are workgroups of four waves");
  if ((int)blockIdx.x < a.dec_grid) decode_chunks_mfma<D, G>(a, blockIdx.x, a.dec_grid);

  const int* items = a.plan + plan_offsets(a.S, a.cap_dec, a.cap_pf).pf;
  const int n_items = a.plan[1];
  const int kvh = blockIdx.x % a.Hkv;
  int* cursor = a.plan + kPlanCursors + kvh;
  for (;;) {
    if (threadIdx.x == 0)
      s_next = __hip_atomic_fetch_add(cursor, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __syncthreads();
    const int it = s_next;
    __syncthreads();  // everyone has read s_next before the next item may overwrite it
    if (it >= n_items) break;
    prefill_item<D, G>(a, sm, items[2 * it], items[2 * it + 1], kvh);
  }
}

template <int D, int G>
hipError_t launch_tick_t(const AttnArgs& a, hipStream_t s) {
  int grid = persistent_grid((const void*)tick_kernel<D, G>, kPfThreads);
  grid = grid > 8 ? grid - grid % 8 : 8;  // workgroup b on XCD b % 8 serves KV head b % Hkv
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

}  // namespace

bool tick_supported(pa_dtype_t dt, int D) { return dt == PA_BF16 && (D == 64 || D == 128); }

hipError_t launch_tick(pa_dtype_t dt, const AttnArgs& a, hipStream_t s) {
  if (!tick_supported(dt, a.D)) return hipErrorInvalidValue;
  const int G = a.Hq / a.Hkv;
  return a.D == 64 ? launch_tick_d<64>(a, G, s) : launch_tick_d<128>(a, G, s);
}

}  // namespace pa
