// Work planning for one packed tick, on the device.
//
// The host knows only upper bounds (max_query_len, max_seq_len); the lengths of
// the tick's sequences live in device memory. Instead of launching a grid over
// every (sequence, tile) pair and letting most workgroups exit, one small
// workgroup reads query_start_loc and seq_lens once and writes two compact
// lists into the workspace:
//   decode items  (sequence, split partition) for every row with query length 1;
//   prefill items (sequence, 128-row tile) for every sequence with query length > 1,
//                 ordered by decreasing number of key tiles, so that the longest
//                 tiles start first (longest-processing-time-first scheduling).
// The persistent attention kernels then walk these lists.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kCostBins = 2048;

// Exclusive scan of one int per thread over the workgroup; returns the
// thread's offset and writes the total to *total (uniform).
__device__ int block_exclusive_scan(int v, int* s_buf, int* total) {
  const int tid = threadIdx.x;
  s_buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const int add = tid >= off ? s_buf[tid - off] : 0;
    __syncthreads();
    s_buf[tid] += add;
    __syncthreads();
  }
  const int incl = s_buf[tid];
  *total = s_buf[kPlanThreads - 1];
  __syncthreads();
  return incl - v;
}

struct SeqShape {
  int L, n;
};

__device__ __forceinline__ SeqShape seq_shape(const AttnArgs& a, int s) {
  SeqShape r;
  const int q0 = a.qsl[s];
  r.L = a.qsl[s + 1] - q0;
  int n = a.seq_lens[s];
  const int cap = a.max_blocks * a.P;
  r.n = n < cap ? n : cap;
  if (q0 < 0 || q0 + r.L > a.T || r.L < 0) r.L = 0;  // malformed rows are skipped
  return r;
}

__device__ __forceinline__ int tile_cost(const SeqShape& sh, int mt, int TM) {
  const int i1 = min(sh.L, (mt + 1) * TM);
  const int keys = sh.n - sh.L + i1;
  int c = (keys + 31) / 32;
  return c < 0 ? 0 : (c >= kCostBins ? kCostBins - 1 : c);
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(AttnArgs a, int* plan, int cap_dec,
                                                            int cap_pf, int TM) {
  __shared__ int s_buf[kPlanThreads];
  __shared__ int s_hist[kCostBins];
  __shared__ int s_cur[kCostBins];
  const int tid = threadIdx.x;
  int* dec_items = plan + kPlanHeaderInts;
  int* pf_items = dec_items + 2 * (size_t)cap_dec;
  const int PT = a.part_tokens;

  for (int i = tid; i < kCostBins; i += kPlanThreads) s_hist[i] = 0;

  // ---- decode items (sequence order) and the prefill cost histogram ----
  int dec_base = 0;
  for (int c0 = 0; c0 < a.S; c0 += kPlanThreads) {
    const int s = c0 + tid;
    int nd = 0;
    SeqShape sh{0, 0};
    if (s < a.S) {
      sh = seq_shape(a, s);
      if (sh.L == 1 && sh.n >= 1) nd = min((sh.n + PT - 1) / PT, a.max_parts);
      if (sh.L > 1 && sh.n >= sh.L) {
        const int ntiles = (sh.L + TM - 1) / TM;
        for (int mt = 0; mt < ntiles; ++mt) atomicAdd(&s_hist[tile_cost(sh, mt, TM)], 1);
      }
    }
    int total;
    const int off = block_exclusive_scan(nd, s_buf, &total);
    for (int p = 0; p < nd; ++p) {
      const int idx = dec_base + off + p;
      if (idx < cap_dec) {
        dec_items[2 * idx] = s;
        dec_items[2 * idx + 1] = p;
      }
    }
    dec_base += total;
  }
  __syncthreads();

  // ---- bin offsets in decreasing cost: bin b starts after all bins > b ----
  int pf_total = 0;
  // (kCostBins = 2 * kPlanThreads: each thread owns bins 2t and 2t+1 of the
  // reversed order)
  {
    const int r0 = 2 * tid, r1 = 2 * tid + 1;  // positions in decreasing-cost order
    const int b0 = kCostBins - 1 - r0, b1 = kCostBins - 1 - r1;
    const int h0 = s_hist[b0], h1 = s_hist[b1];
    const int off = block_exclusive_scan(h0 + h1, s_buf, &pf_total);
    s_cur[b0] = off;
    s_cur[b1] = off + h0;
  }
  __syncthreads();

  // ---- scatter prefill items into their bins ----
  for (int c0 = 0; c0 < a.S; c0 += kPlanThreads) {
    const int s = c0 + tid;
    if (s < a.S) {
      const SeqShape sh = seq_shape(a, s);
      if (sh.L > 1 && sh.n >= sh.L) {
        const int ntiles = (sh.L + TM - 1) / TM;
        for (int mt = ntiles - 1; mt >= 0; --mt) {
          const int idx = atomicAdd(&s_cur[tile_cost(sh, mt, TM)], 1);
          if (idx < cap_pf) {
            pf_items[2 * idx] = s;
            pf_items[2 * idx + 1] = mt;
          }
        }
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    plan[0] = min(dec_base, cap_dec);
    plan[1] = min(pf_total, cap_pf);
    plan[2] = 0;
    plan[3] = 0;
  }
}

}  // namespace

hipError_t launch_plan(const AttnArgs& a, int* plan, int cap_dec, int cap_pf, int TM,
                       hipStream_t s) {
  profile_before("plan", s);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a, plan, cap_dec, cap_pf,
                     TM);
  profile_after(s);
  return hipGetLastError();
}

}  // namespace pa
