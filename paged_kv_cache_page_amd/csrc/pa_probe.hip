// A plain streaming read of device memory, for measurement: the practical
// ceiling of an HBM-bound kernel on this GPU (what a read-only stream reaches,
// against which the decode kernels' achieved bandwidth is read). Not part of a
// tick.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;  // 16-byte loads in flight per thread

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Every thread reads kProbeUnroll 16-byte vectors per step, grid-stride over
// the buffer, and folds them with XOR; one word per thread goes to the sink so
// the loads cannot be dropped. The loads are non-temporal (a stream read once
// needs no cache lines). One workgroup per compute unit: of the shapes
// measured on MI355X over 2 GiB (1-16 workgroups of 256 or 512 threads per
// unit, 4-16 loads in flight, grid-stride or contiguous per workgroup, with
// and without the non-temporal hint), this one read fastest: 7.1 TB/s,
// against 6.2-6.35 TB/s for the best shapes with ordinary loads.
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(
    const u32x4_t* __restrict__ buf, size_t n16, uint32_t* __restrict__ sink) {
  const size_t tid = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  uint32_t acc = 0;
  size_t i = tid;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4_t v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(buf + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[tid] = acc;
}

}  // namespace

int probe_grid() { return cu_count(); }

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s) {
  profile_before("stream_read", s);
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)probe_grid()), dim3(kProbeThreads), 0, s,
                     (const u32x4_t*)buf, bytes / 16, sink);
  profile_after(s);
  return hipGetLastError();
}

}  // namespace pa

#pragma GCC visibility push(default)
extern "C" {

size_t pa_probe_sink_words(void) { return (size_t)pa::probe_grid() * pa::kProbeThreads; }

pa_status_t pa_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 || ((uintptr_t)buf & 15u) || ((uintptr_t)sink & 3u))
    return PA_ERR_INVALID_ARG;
  return pa::launch_stream_read(buf, bytes, sink, (hipStream_t)stream) == hipSuccess ? PA_OK
                                                                                     : PA_ERR_HIP;
}

}  // extern "C"
#pragma GCC visibility pop
