// Batched token sampling (include/pa_sample.h): one workgroup of 1024 threads
// per logits row, every row with its own greedy / temperature / top-k / top-p
// settings, in one launch (llm-serving-engine README, row "Token sampling";
// Helios blog, "Continuous batching").
//
// Each token gets a 64-bit sort key: the float's order-preserving bits above
// the inverted index, so keys are distinct and a larger key ranks first (a
// larger logit, or an equal logit at a lower index). The kept set is always
// a leading part of the ranking, i.e. the tokens whose key is at least a
// cutoff; top-k and top-p each find their cutoff by a radix descent over the
// key, 10 bits per pass over the row, with per-bucket counts, integer weights
// (64-bit LDS atomics: exact, so the result does not depend on the order of
// the adds) and the largest key per bucket, stopping as soon as the chosen
// bucket holds a single token. A last pass walks the row in index order, tile
// by tile, with a workgroup prefix sum of the kept weights, and stops at the
// tile where the running weight passes floor(u * S).
//
// Weights are floor(exp((x - max) / T) * 2^32) in float64: the subtraction and
// the division are IEEE operations (this file is built without contraction),
// so the only rounding that can differ from another implementation is exp's.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/pa_sample.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kDigit = 10;
constexpr int kBins = 1 << kDigit;
static_assert(kBins == kThreads, "one histogram bin per thread");
constexpr int32_t kMaxVocab = 1 << 21;  // kept weights sum below 2^53: exact in float64

typedef unsigned long long u64;

struct SampleArgs {
  const float* logits;
  int64_t row_stride;
  const float* temperature;
  const int32_t* top_k;
  const float* top_p;
  const float* uniforms;
  int32_t* out;
  int32_t V;
  int32_t ibits;  // bits of the inverted index under the float bits
};

struct SampleLds {
  unsigned int cnt[kBins];
  u64 mass[kBins];
  u64 maxkey[kBins];
  u64 wave[kWaves];
  u64 sel[4];  // chosen bucket, the target left inside it, its count, its largest key
};

__device__ inline u64 sort_key(float x, int32_t i, int ibits) {
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0u;                     // -0.0 ranks with +0.0
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);    // unsigned order = float order
  const uint32_t inv = ((1u << ibits) - 1u) - (uint32_t)i;
  return ((u64)b << ibits) | (u64)inv;
}

__device__ inline u64 weight(float x, double m, double T) {
  const double w = exp(((double)x - m) / T);
  return (u64)floor(w * 4294967296.0);
}

__device__ inline u64 wave_incl_scan(u64 v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const u64 w = __shfl_up(v, o, 64);
    if (lane >= o) v += w;
  }
  return v;
}

// Inclusive prefix sum over the workgroup in thread order; *total = the sum.
__device__ inline u64 block_incl_scan(u64 v, SampleLds& L, u64* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_incl_scan(v, lane);
  if (lane == 63) L.wave[w] = v;
  __syncthreads();
  u64 before = 0, tot = 0;
#pragma unroll
  for (int j = 0; j < kWaves; ++j) {
    const u64 x = L.wave[j];
    before += (j < w) ? x : 0ull;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return v + before;
}

__device__ inline u64 block_max(u64 v, SampleLds& L) {
#pragma unroll
  for (int o = 32; o; o >>= 1) {
    const u64 w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  if ((threadIdx.x & 63) == 0) L.wave[threadIdx.x >> 6] = v;
  __syncthreads();
  u64 m = 0;
#pragma unroll
  for (int j = 0; j < kWaves; ++j) m = L.wave[j] > m ? L.wave[j] : m;
  __syncthreads();
  return m;
}

// The cutoff C such that the tokens with key >= C (among those with key >=
// floor_key) are the shortest leading part of the ranking that holds `target`
// tokens (BY_WEIGHT false) or reaches weight max(ceil(p * total), 1)
// (BY_WEIGHT true; the total is taken in the first pass).
template <bool BY_WEIGHT>
__device__ u64 select_cutoff(const float* row, const SampleArgs& a, u64 floor_key, double m,
                             double T, float p, u64 target, SampleLds& L) {
  const int t = threadIdx.x;
  const int nbits = 32 + a.ibits;
  u64 prefix = 0, rem = target;
  int done = 0;
  for (;;) {
    const int width = min(kDigit, nbits - done);
    const int shift = nbits - done - width;
    L.cnt[t] = 0u;
    L.mass[t] = 0ull;
    L.maxkey[t] = 0ull;
    if (t == 0) {  // if no bucket is chosen (input outside the contract): stop, keep nothing
      L.sel[0] = 0ull;
      L.sel[1] = 1ull;
      L.sel[2] = 1ull;
      L.sel[3] = ~0ull;
    }
    __syncthreads();
    for (int i = t; i < a.V; i += kThreads) {
      const float x = row[i];
      const u64 k = sort_key(x, i, a.ibits);
      if (k < floor_key) continue;
      if (done > 0 && (k >> (shift + width)) != prefix) continue;
      const int d = (int)((k >> shift) & (u64)((1u << width) - 1u));
      atomicAdd(&L.cnt[d], 1u);
      if (BY_WEIGHT) atomicAdd(&L.mass[d], weight(x, m, T));
      atomicMax(&L.maxkey[d], k);
    }
    __syncthreads();
    const int b = kBins - 1 - t;  // thread t scans bucket b: larger buckets first
    const u64 v = BY_WEIGHT ? L.mass[b] : (u64)L.cnt[b];
    u64 total;
    const u64 cum = block_incl_scan(v, L, &total);
    if (BY_WEIGHT && done == 0) {
      const double need = ceil((double)p * (double)total);
      rem = need >= 1.0 ? (u64)need : 1ull;
    }
    if (cum >= rem && cum - v < rem) {
      L.sel[0] = (u64)b;
      L.sel[1] = rem - (cum - v);
      L.sel[2] = (u64)L.cnt[b];
      L.sel[3] = L.maxkey[b];
    }
    __syncthreads();
    const u64 d = L.sel[0];
    rem = L.sel[1];
    const u64 count = L.sel[2], top_key = L.sel[3];
    __syncthreads();  // everyone has read sel before the next pass resets it
    prefix = (prefix << width) | d;
    done += width;
    if (count == 1ull) return top_key;
    if (done >= nbits) return prefix;
  }
}

__global__ __launch_bounds__(kThreads) void sample_kernel(SampleArgs a) {
  __shared__ SampleLds L;
  const int r = blockIdx.x;
  const float* row = a.logits + (int64_t)r * a.row_stride;
  const int V = a.V;

  u64 best = 0;
  for (int i = threadIdx.x; i < V; i += kThreads) {
    const u64 k = sort_key(row[i], i, a.ibits);
    best = k > best ? k : best;
  }
  best = block_max(best, L);
  int32_t top = (int32_t)(((1u << a.ibits) - 1u) - (uint32_t)(best & ((1ull << a.ibits) - 1ull)));
  if (top < 0 || top >= V) top = 0;

  const float T = a.temperature[r];
  const int32_t k = a.top_k[r];
  const float p = a.top_p[r];
  if (!(T > 0.f) || k == 1) {
    if (threadIdx.x == 0) a.out[r] = top;
    return;
  }
  const double m = (double)row[top];
  const double Td = (double)T;

  u64 cut = 0;
  if (k > 1 && k < V) cut = select_cutoff<false>(row, a, 0ull, m, Td, p, (u64)k, L);
  if (p < 1.f) {
    const u64 c2 = select_cutoff<true>(row, a, cut, m, Td, p, 0ull, L);
    cut = c2 > cut ? c2 : cut;
  }

  u64 s = 0;
  for (int i = threadIdx.x; i < V; i += kThreads) {
    const float x = row[i];
    if (sort_key(x, i, a.ibits) >= cut) s += weight(x, m, Td);
  }
  u64 S;
  (void)block_incl_scan(s, L, &S);
  double tr = floor((double)a.uniforms[r] * (double)S);
  if (!(tr >= 0.0)) tr = 0.0;
  if (S > 0 && tr > (double)(S - 1)) tr = (double)(S - 1);
  const u64 target = (u64)tr;

  int32_t pick = top;
  u64 run = 0;
  if (threadIdx.x == 0) L.sel[0] = (u64)top;
  for (int base = 0; base < V; base += kThreads) {
    const int i = base + (int)threadIdx.x;
    u64 q = 0;
    if (i < V) {
      const float x = row[i];
      if (sort_key(x, i, a.ibits) >= cut) q = weight(x, m, Td);
    }
    u64 tile;
    const u64 inc = block_incl_scan(q, L, &tile);
    if (run + tile > target) {  // the same decision in every thread
      if (run + inc > target && run + inc - q <= target) L.sel[0] = (u64)i;
      __syncthreads();
      pick = (int32_t)L.sel[0];
      break;
    }
    run += tile;
  }
  if (threadIdx.x == 0) a.out[r] = (pick >= 0 && pick < V) ? pick : top;
}

}  // namespace

extern "C" __attribute__((visibility("default"))) pa_status_t pa_sample_tokens(
    const float* logits, int64_t row_stride, int32_t rows, int32_t vocab,
    const float* temperature, const int32_t* top_k, const float* top_p, const float* uniforms,
    int32_t* out_tokens, void* stream) {
  if (rows < 0 || vocab < 1 || row_stride < vocab) return PA_ERR_INVALID_ARG;
  if (vocab > kMaxVocab) return PA_ERR_UNSUPPORTED;
  if (rows == 0) return PA_OK;
  if (!logits || !temperature || !top_k || !top_p || !uniforms || !out_tokens)
    return PA_ERR_INVALID_ARG;
  SampleArgs a;
  a.logits = logits;
  a.row_stride = row_stride;
  a.temperature = temperature;
  a.top_k = top_k;
  a.top_p = top_p;
  a.uniforms = uniforms;
  a.out = out_tokens;
  a.V = vocab;
  int ibits = 1;
  while ((1 << ibits) < vocab) ++ibits;
  a.ibits = ibits;
  hipLaunchKernelGGL(sample_kernel, dim3((unsigned)rows), dim3(kThreads), 0,
                     (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}
