// K4: prefill-chunk paged attention on bf16 matrix cores (gfx950 MFMA): the
// persistent kernel over the plan's prefill items (the item code is in
// pa_prefill_mfma.h).
#include "pa_prefill_mfma.h"

namespace pa {

namespace {

template <int D, int G>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(2))) void prefill_mfma_kernel(AttnArgs a) {
  __shared__ PfSmem<D> sm;
  const int* items = a.plan + plan_offsets(a.S, a.cap_dec, a.cap_pf).pf;
  const int total = a.plan[1] * a.Hkv;
  const int nwg = gridDim.x;
  // Items are sorted by decreasing cost; rounds alternate direction (snake) so
  // the workgroups that took the longest items take the shortest next.
  for (int r = 0;; ++r) {
    const int w = r * nwg + ((r & 1) ? (nwg - 1 - (int)blockIdx.x) : (int)blockIdx.x);
    if (w >= total) break;
    const int it = w / a.Hkv;
    prefill_item<D, G>(a, sm, items[2 * it], items[2 * it + 1], w % a.Hkv);
  }
}

template <int D, int G>
hipError_t launch_pf(const AttnArgs& a, hipStream_t s) {
  const long items = (long)a.cap_pf * a.Hkv;
  if (items == 0) return hipSuccess;
  const int resident = persistent_grid((const void*)prefill_mfma_kernel<D, G>, kPfThreads);
  const long grid = items < resident ? items : resident;
  profile_before("prefill_attention_mfma", s);
  hipLaunchKernelGGL((prefill_mfma_kernel<D, G>), dim3((unsigned)grid), dim3(kPfThreads), 0, s,
                     a);
  profile_after(s);
  return hipGetLastError();
}

template <int D>
hipError_t launch_pf_d(const AttnArgs& a, int G, hipStream_t s) {
  switch (G) {
    case 1: return launch_pf<D, 1>(a, s);
    case 2: return launch_pf<D, 2>(a, s);
    case 4: return launch_pf<D, 4>(a, s);
    case 8: return launch_pf<D, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool prefill_mfma_supported(pa_dtype_t dt, int D, int /*G*/) {
  return dt == PA_BF16 && (D == 64 || D == 128);
}

hipError_t launch_prefill_mfma(pa_dtype_t dt, const AttnArgs& a, hipStream_t s) {
  if (dt != PA_BF16) return hipErrorInvalidValue;
  const int G = a.Hq / a.Hkv;
  if (a.D == 64) return launch_pf_d<64>(a, G, s);
  if (a.D == 128) return launch_pf_d<128>(a, G, s);
  return hipErrorInvalidValue;
}

}  // namespace pa
