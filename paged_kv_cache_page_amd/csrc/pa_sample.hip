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
// bucket holds a single token. A last pass walks the tokens in index order,
// tile by tile, with a workgroup prefix sum of the kept weights, and stops at
// the tile where the running weight passes floor(u * S).
//
// The row is read once, split over workgroups of 3072 tokens each: each
// finds its slice's largest logit and lists the slice's tokens that pass a
// float32 screen for a positive weight against it; the row's workgroup then
// keeps those that pass against the row's maximum, in LDS, in index order. That list is a leading part of the ranking and holds every
// token of positive weight, so top-k, top-p and the draw run on it alone; a
// row whose list would not fit runs them over the row instead. A list of at
// most 512 tokens (the usual case at low temperatures) is ranked by the row's
// first wave alone, with 8-bit digits, no workgroup barrier and one exp per
// token.
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

constexpr int kPer = 8;      // consecutive tokens per thread in the index-order passes
constexpr int kList = 4096;  // tokens the LDS list holds; a longer list reads the row again
constexpr int kListPer = 4;  // candidates per thread and pass when the draw lays out the list

struct SampleLds {
  float cx[kList];    // listed tokens: logit
  int32_t ci[kList];  // and index, in index order
  unsigned int cnt[kBins];
  u64 mass[kBins];
  u64 maxkey[kBins];
  u64 wave[kWaves];
  u64 wcount[kWaves];      // per wave, read once: its slices' listed tokens,
  u64 wmax[kWaves];        // their largest key
  uint32_t wflag[kWaves];  // and whether one of them overflowed
  u64 sel[4];  // chosen bucket, the target left inside it, its count, its largest key
  uint32_t off[kThreads];  // where each slice's list starts when laid end to end
};

__device__ inline uint32_t order_bits(float x) {
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0u;                     // -0.0 ranks with +0.0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);  // unsigned order = float order
}

__device__ inline u64 sort_key(float x, int32_t i, int ibits) {
  const uint32_t inv = ((1u << ibits) - 1u) - (uint32_t)i;
  return ((u64)order_bits(x) << ibits) | (u64)inv;
}

// The row's largest logit and temperature, in the two precisions the weights use.
struct Scale {
  double m, T;   // float64: the weight's own arithmetic
  float mf, zf;  // float32 screen: a logit more than zf = 22.5 T below mf weighs 0
};

// floor(exp((x - m) / T) * 2^32). The float32 screen is conservative: past it,
// (x - m) / T < -22.5 (1 - 2^-23) < -32 ln 2, so the float64 result is 0 too.
__device__ inline u64 weight(float x, const Scale& c) {
  if (c.mf - x > c.zf) return 0ull;
  const double w = exp(((double)x - c.m) / c.T);
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

// Inclusive prefix sum over a workgroup of W waves in thread order; *total =
// the sum. `wave` is W words of LDS.
template <int W>
__device__ inline u64 group_incl_scan(u64 v, u64* wave, u64* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_incl_scan(v, lane);
  if (lane == 63) wave[w] = v;
  __syncthreads();
  u64 before = 0, tot = 0;
#pragma unroll
  for (int j = 0; j < W; ++j) {
    const u64 x = wave[j];
    before += (j < w) ? x : 0ull;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return v + before;
}

template <int W>
__device__ inline u64 group_max(u64 v, u64* wave) {
#pragma unroll
  for (int o = 32; o; o >>= 1) {
    const u64 x = __shfl_xor(v, o, 64);
    v = x > v ? x : v;
  }
  if ((threadIdx.x & 63) == 0) wave[threadIdx.x >> 6] = v;
  __syncthreads();
  u64 m = 0;
#pragma unroll
  for (int j = 0; j < W; ++j) m = wave[j] > m ? wave[j] : m;
  __syncthreads();
  return m;
}

__device__ inline u64 block_incl_scan(u64 v, SampleLds& L, u64* total) {
  return group_incl_scan<kWaves>(v, L.wave, total);
}

// Index of the token a sort key belongs to, clamped into [lo, hi).
__device__ inline int32_t key_index(u64 key, int ibits, int32_t lo, int32_t hi) {
  const int32_t i = (int32_t)(((1u << ibits) - 1u) - (uint32_t)(key & ((1ull << ibits) - 1ull)));
  return (i >= lo && i < hi) ? i : lo;
}

// Where the tokens of one row come from: the row itself, or the list in LDS
// of its tokens that pass the weight screen. Both are in index order.
struct RowSrc {
  const float* row;
  int n;
  __device__ float x(int j) const { return row[j]; }
  __device__ int idx(int j) const { return j; }
};
struct ListSrc {
  const float* cx;
  const int32_t* ci;
  int n;
  __device__ float x(int j) const { return cx[j]; }
  __device__ int idx(int j) const { return ci[j]; }
};

// The cutoff C such that the tokens with key >= C (among those with key >=
// floor_key) are the shortest leading part of the ranking that holds `target`
// tokens (BY_WEIGHT false) or reaches weight max(ceil(p * total), 1)
// (BY_WEIGHT true; the total is taken in the first pass).
// By weight, tokens of weight 0 are left out: they rank below every token of
// positive weight (the weight does not decrease with the logit), so the
// shortest leading part never ends at one.
template <bool BY_WEIGHT, class Src>
__device__ u64 select_cutoff(const Src& src, int ibits, u64 floor_key, const Scale& c, float p,
                             u64 target, SampleLds& L) {
  const int t = threadIdx.x;
  const int nbits = 32 + ibits;
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
    for (int j = t; j < src.n; j += kThreads) {
      const float x = src.x(j);
      const u64 k = sort_key(x, src.idx(j), ibits);
      if (k < floor_key) continue;
      if (done > 0 && (k >> (shift + width)) != prefix) continue;
      const int d = (int)((k >> shift) & (u64)((1u << width) - 1u));
      if (BY_WEIGHT) {
        const u64 w = weight(x, c);
        if (w == 0ull) continue;
        atomicAdd(&L.mass[d], w);
      }
      atomicAdd(&L.cnt[d], 1u);
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

// Top-k, top-p and the draw over the tokens of `src`, which hold every token
// of positive weight and are a leading part of the ranking. Returns the token.
template <class Src>
__device__ int32_t draw(const Src& src, int ibits, int V, int32_t k, float p, float u,
                        const Scale& c, int32_t top, SampleLds& L) {
  u64 cut = 0;
  if (k > 1 && k < src.n) cut = select_cutoff<false>(src, ibits, 0ull, c, p, (u64)k, L);
  if (p < 1.f) {
    const u64 c2 = select_cutoff<true>(src, ibits, cut, c, p, 0ull, L);
    cut = c2 > cut ? c2 : cut;
  }

  u64 s = 0;
  for (int j = threadIdx.x; j < src.n; j += kThreads) {
    const float x = src.x(j);
    if (sort_key(x, src.idx(j), ibits) >= cut) s += weight(x, c);
  }
  u64 S;
  (void)block_incl_scan(s, L, &S);
  double tr = floor((double)u * (double)S);
  if (!(tr >= 0.0)) tr = 0.0;
  if (S > 0 && tr > (double)(S - 1)) tr = (double)(S - 1);
  const u64 target = (u64)tr;

  // index order, kPer consecutive tokens per thread, one workgroup scan per tile
  int32_t pick = top;
  u64 run = 0;
  if (threadIdx.x == 0) L.sel[0] = (u64)top;
  for (int base = 0; base < src.n; base += kThreads * kPer) {
    const int j0 = base + (int)threadIdx.x * kPer;
    u64 q[kPer];
    u64 qs = 0;
#pragma unroll
    for (int jj = 0; jj < kPer; ++jj) {
      const int j = j0 + jj;
      u64 w = 0;
      if (j < src.n) {
        const float x = src.x(j);
        if (sort_key(x, src.idx(j), ibits) >= cut) w = weight(x, c);
      }
      q[jj] = w;
      qs += w;
    }
    u64 tile;
    const u64 inc = block_incl_scan(qs, L, &tile);
    if (run + tile > target) {  // the same decision in every thread
      if (run + inc > target && run + inc - qs <= target) {
        u64 acc = run + inc - qs;
#pragma unroll
        for (int jj = 0; jj < kPer; ++jj) {
          acc += q[jj];
          if (acc > target) {
            L.sel[0] = (u64)src.idx(j0 + jj);
            break;
          }
        }
      }
      __syncthreads();
      pick = (int32_t)L.sel[0];
      break;
    }
    run += tile;
  }
  return (pick >= 0 && pick < V) ? pick : top;
}

// ---- short lists: one wave, no workgroup barriers ----
// A list of at most kWaveList tokens is ranked by the row's first wave alone
// (the others have left): lane l holds tokens l, l + 64, ... of the list with
// their sort keys and weights in registers (one exp per token), and each
// radix pass needs only the wave's own LDS ordering. The cutoffs and the draw
// are the same functions of the list as above (a shortest leading part, then
// the first token in index order whose running weight passes floor(u * S)),
// so the token is the same; only the digit width and the first pass differ
// (the descent starts below the key bits all candidates share).
constexpr int kWavePer = 8;
constexpr int kWaveList = 64 * kWavePer;
constexpr int kWaveDigit = 8;
constexpr int kWaveBins = 1 << kWaveDigit;
constexpr int kWaveBinsPerLane = kWaveBins / 64;
static_assert(kWaveBins <= kBins, "the wave's bins are the first of the workgroup's");

// The wave's LDS operations complete in order: wait for them, with compiler
// barriers on both sides so that none moves across.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// select_cutoff for one wave over the lanes' registers (n = tokens this lane
// holds).
template <bool BY_WEIGHT>
__device__ u64 wave_select_cutoff(const u64 (&key)[kWavePer], const u64 (&wt)[kWavePer], int n,
                                  int ibits, u64 floor_key, float p, u64 target, SampleLds& L) {
  const int lane = threadIdx.x;
  const int nbits = 32 + ibits;
  // The leading key bits that every candidate shares need no pass (each such
  // pass would choose the one bucket that holds them all, leaving rem as it
  // is): start the descent below them.
  u64 kmin = ~0ull, kmax = 0ull;
#pragma unroll
  for (int j = 0; j < kWavePer; ++j) {
    if (j >= n || key[j] < floor_key || (BY_WEIGHT && wt[j] == 0ull)) continue;
    kmin = key[j] < kmin ? key[j] : kmin;
    kmax = key[j] > kmax ? key[j] : kmax;
  }
#pragma unroll
  for (int o = 32; o; o >>= 1) {
    const u64 a = __shfl_xor(kmin, o, 64), b = __shfl_xor(kmax, o, 64);
    kmin = a < kmin ? a : kmin;
    kmax = b > kmax ? b : kmax;
  }
  if (kmin > kmax) return ~0ull;    // no candidate: keep nothing (as when no bucket is chosen)
  if (kmin == kmax) return kmin;    // one candidate: its own key
  int done = __clzll((long long)(kmin ^ kmax)) - (64 - nbits);
  u64 prefix = done > 0 ? kmin >> (nbits - done) : 0ull, rem = target;
  bool first = true;
  for (;;) {
    const int width = min(kWaveDigit, nbits - done);
    const int shift = nbits - done - width;
    wave_lds_sync();  // the previous pass's reads of the bins are done
#pragma unroll
    for (int i = 0; i < kWaveBinsPerLane; ++i) {
      L.cnt[lane + 64 * i] = 0u;
      L.mass[lane + 64 * i] = 0ull;
      L.maxkey[lane + 64 * i] = 0ull;
    }
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < kWavePer; ++j) {
      if (j >= n) continue;
      const u64 k = key[j];
      if (k < floor_key) continue;
      if (done > 0 && (k >> (shift + width)) != prefix) continue;
      const int d = (int)((k >> shift) & (u64)((1u << width) - 1u));
      if (BY_WEIGHT) {
        if (wt[j] == 0ull) continue;
        atomicAdd(&L.mass[d], wt[j]);
      }
      atomicAdd(&L.cnt[d], 1u);
      atomicMax(&L.maxkey[d], k);
    }
    wave_lds_sync();
    // lane l scans buckets kWaveBins - 1 - (4 l + i): larger buckets first
    u64 v[kWaveBinsPerLane];
    u64 s = 0;
#pragma unroll
    for (int i = 0; i < kWaveBinsPerLane; ++i) {
      const int b = kWaveBins - 1 - (kWaveBinsPerLane * lane + i);
      v[i] = BY_WEIGHT ? L.mass[b] : (u64)L.cnt[b];
      s += v[i];
    }
    const u64 incl = wave_incl_scan(s, lane);
    if (BY_WEIGHT && first) {
      const u64 total = __shfl(incl, 63, 64);
      const double need = ceil((double)p * (double)total);
      rem = need >= 1.0 ? (u64)need : 1ull;
    }
    const u64 before = incl - s;
    const u64 owners = __ballot(incl >= rem && before < rem);
    if (owners == 0ull) return ~0ull;  // no bucket chosen (input outside the contract): keep nothing
    const int owner = __ffsll((long long)owners) - 1;
    // in the owner: its first bucket where the running count or weight reaches
    // rem, and what is left of rem inside it
    u64 cum = before;
    int pick = kWaveBinsPerLane - 1;
    bool got = false;
#pragma unroll
    for (int i = 0; i < kWaveBinsPerLane; ++i) {
      if (!got && cum + v[i] >= rem) {
        pick = i;
        got = true;
      }
      if (!got) cum += v[i];
    }
    const int d = __shfl(kWaveBins - 1 - (kWaveBinsPerLane * lane + pick), owner, 64);
    rem = __shfl(rem - cum, owner, 64);
    const u64 count = (u64)L.cnt[d];
    const u64 top_key = L.maxkey[d];
    prefix = (prefix << width) | (u64)d;
    done += width;
    first = false;
    if (count == 1ull) return top_key;
    if (done >= nbits) return prefix;
  }
}

// draw() for a list of at most kWaveList tokens, by the workgroup's first wave.
// Lane l holds list positions l + 64 j (j < jn = ceil(n / 64)), so a list of
// n tokens costs each lane jn exps; index order is (j, lane).
__device__ int32_t draw_wave(const SampleLds& Lc, int n, int ibits, int V, int32_t k, float p,
                             float u, const Scale& c, int32_t top, SampleLds& L) {
  const int lane = threadIdx.x;
  const int jn = (n + 63) >> 6;                  // uniform
  const int mine = max(0, (n - lane + 63) >> 6);  // positions l + 64 j < n: j < mine
  u64 key[kWavePer], wt[kWavePer];
  int32_t idx[kWavePer];
#pragma unroll
  for (int j = 0; j < kWavePer; ++j) {
    key[j] = 0ull;
    wt[j] = 0ull;
    idx[j] = top;
    if (j < jn) {  // uniform; the last j's positions past n are read clamped and left out by mine
      const int q = min(lane + 64 * j, n - 1);
      const float x = Lc.cx[q];
      idx[j] = Lc.ci[q];
      key[j] = sort_key(x, idx[j], ibits);
      wt[j] = weight(x, c);
    }
  }
  u64 cut = 0;
  if (k > 1 && k < n) cut = wave_select_cutoff<false>(key, wt, mine, ibits, 0ull, p, (u64)k, L);
  if (p < 1.f) {
    const u64 c2 = wave_select_cutoff<true>(key, wt, mine, ibits, cut, p, 0ull, L);
    cut = c2 > cut ? c2 : cut;
  }
  // from here on wt holds the kept weights (0 for the tokens cut)
  u64 s = 0;
#pragma unroll
  for (int j = 0; j < kWavePer; ++j) {
    wt[j] = (j < mine && key[j] >= cut) ? wt[j] : 0ull;
    s += wt[j];
  }
  const u64 S = __shfl(wave_incl_scan(s, lane), 63, 64);
  double tr = floor((double)u * (double)S);
  if (!(tr >= 0.0)) tr = 0.0;
  if (S > 0 && tr > (double)(S - 1)) tr = (double)(S - 1);
  const u64 target = (u64)tr;
  // in index order, one wave scan per j: the first position where the
  // running weight passes target
  int32_t pick = top;
  u64 run = 0;
  bool done = false;
#pragma unroll
  for (int j = 0; j < kWavePer; ++j) {
    if (done || j >= jn) continue;  // uniform
    const u64 incl = wave_incl_scan(wt[j], lane);
    const u64 tot = __shfl(incl, 63, 64);
    if (run + tot > target) {
      const u64 owners = __ballot(run + incl > target && run + incl - wt[j] <= target);
      pick = __shfl(idx[j], __ffsll((long long)owners) - 1, 64);
      done = true;
    } else {
      run += tot;
    }
  }
  return (pick >= 0 && pick < V) ? pick : top;
}

// Slices of a row: ceil(V / kSliceLen) workgroups of kScreenThreads threads per
// row, each thread holding kRegs logits in registers (one read of the row),
// find their slice's largest key and list, in index order, the
// slice's tokens that pass the weight screen against that local maximum (a
// superset of what the row's maximum lets through), up to kSliceCap of them.
constexpr int kScreenThreads = 256;
constexpr int kRegs = 12;
constexpr int kSliceLen = kScreenThreads * kRegs;
constexpr int kSliceCap = 1024;
constexpr int kMaxSlices = (kMaxVocab + kSliceLen - 1) / kSliceLen;
static_assert(kMaxSlices <= kThreads, "one slice per drawing thread");

struct Cand {
  float x;
  int32_t i;
};

struct SampleWs {
  u64* lmax;       // [rows * nsl] each slice's largest key
  int32_t* count;  // [rows * nsl] tokens the slice let through (may exceed kSliceCap)
  Cand* cand;      // [rows * nsl * kSliceCap] those tokens, in index order
  int nsl;         // slices per row
};

__global__ __launch_bounds__(kScreenThreads) void sample_screen_kernel(SampleArgs a, SampleWs w) {
  __shared__ u64 s_wave[kScreenThreads / 64];
  const int r = blockIdx.x / w.nsl, sl = blockIdx.x % w.nsl;
  const int t = threadIdx.x;
  const float* row = a.logits + (int64_t)r * a.row_stride;
  const int lo = sl * kSliceLen, hi = min(a.V, lo + kSliceLen);
  const size_t slot = (size_t)r * w.nsl + sl;

  // token lo + kScreenThreads * j + t in register j of thread t: coalesced loads
  float xs[kRegs];
#pragma unroll
  for (int j = 0; j < kRegs; ++j) {
    const int i = lo + kScreenThreads * j + t;
    xs[j] = (i < hi) ? row[i] : 0.f;
  }
  // The thread's largest key. Its tokens come in increasing index order, so
  // of equal float bits the first one seen has the larger key: compare the
  // 32-bit order-preserving bits alone and form the 64-bit key once.
  uint32_t bb = 0u;
  int bi = -1;
#pragma unroll
  for (int j = 0; j < kRegs; ++j) {
    const int i = lo + kScreenThreads * j + t;
    const uint32_t b = order_bits(xs[j]);
    if (i < hi && (bi < 0 || b > bb)) {
      bb = b;
      bi = i;
    }
  }
  u64 best = bi >= 0 ? ((u64)bb << a.ibits) | (u64)(((1u << a.ibits) - 1u) - (uint32_t)bi) : 0ull;
  best = group_max<kScreenThreads / 64>(best, s_wave);
  if (t == 0) w.lmax[slot] = best;
  const float T = a.temperature[r];
  if (!(T > 0.f) || a.top_k[r] == 1 || hi <= lo) {  // greedy rows need only the maximum
    if (t == 0) w.count[slot] = 0;
    return;
  }
  // the slice's largest logit from its key's float bits (-0.0 comes back as
  // +0.0, which screens the same)
  const uint32_t kb = (uint32_t)(best >> a.ibits);
  const float mf = __uint_as_float((kb & 0x80000000u) ? (kb & 0x7FFFFFFFu) : ~kb);
  const float zf = 22.5f * T;

  // index order is (register, wave, lane): per-(register, wave) counts from
  // ballots, their exclusive offsets, then each lane's place among its wave's
  constexpr int kW = kScreenThreads / 64;
  __shared__ uint32_t s_cnt[kRegs][kW];
  __shared__ uint32_t s_total;
  const int lane = t & 63, wv = t >> 6;
  const u64 below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int j = 0; j < kRegs; ++j) {
    const int i = lo + kScreenThreads * j + t;
    const u64 bal = __ballot((i < hi) && !(mf - xs[j] > zf));
    if (lane == 0) s_cnt[j][wv] = (uint32_t)__popcll(bal);
  }
  __syncthreads();
  static_assert(kRegs * kW <= 64, "one lane per (register, wave) count");
  if (t < 64) {  // exclusive offsets in index order, by the first wave
    uint32_t* cnt = &s_cnt[0][0];
    const uint32_t n = lane < kRegs * kW ? cnt[lane] : 0u;
    uint32_t incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t x = __shfl_up(incl, o, 64);
      if (lane >= o) incl += x;
    }
    if (lane < kRegs * kW) cnt[lane] = incl - n;
    if (lane == 63) s_total = incl;
  }
  __syncthreads();
  Cand* out = w.cand + slot * kSliceCap;
#pragma unroll
  for (int j = 0; j < kRegs; ++j) {
    const int i = lo + kScreenThreads * j + t;
    const bool keep = (i < hi) && !(mf - xs[j] > zf);
    const u64 bal = __ballot(keep);
    if (keep) {
      const uint32_t pos = s_cnt[j][wv] + (uint32_t)__popcll(bal & below);
      if (pos < (uint32_t)kSliceCap) out[pos] = Cand{xs[j], i};
    }
  }
  if (t == 0) w.count[slot] = (int32_t)s_total;
}

// One workgroup per row: the row's largest key from its slices; greedy rows
// end there. Otherwise the slices' tokens that also pass the screen against
// the row's maximum -- exactly the tokens of the row that pass it, in index
// order -- go to the LDS list, and top-k, top-p and the draw run on it. A
// slice that overflowed its capacity, or a list longer than kList, sends the
// row down the path that reads the row itself. A list of at most kWaveList
// tokens is ranked by the first wave alone (draw_wave).
__global__ __launch_bounds__(kThreads) void sample_draw_kernel(SampleArgs a, SampleWs w) {
  __shared__ SampleLds L;
  const int r = blockIdx.x;
  const int t = threadIdx.x;
  const float* row = a.logits + (int64_t)r * a.row_stride;
  const int V = a.V;
  const int nsl = w.nsl;
  const size_t slot0 = (size_t)r * nsl;

  // One read of the slices' maxima and counts (thread t: slice t) and one
  // workgroup reduction: the row's largest key, whether a slice overflowed,
  // and each slice's offset in the lists laid end to end (per-wave words of
  // their own: nothing writes them again).
  const float T = a.temperature[r];
  const int32_t k = a.top_k[r];
  const float p = a.top_p[r];
  const float u = a.uniforms[r];
  const int lane = t & 63, wv = t >> 6;
  u64 best = t < nsl ? w.lmax[slot0 + t] : 0ull;
  const int32_t n_t = t < nsl ? w.count[slot0 + t] : 0;
#pragma unroll
  for (int o = 32; o; o >>= 1) {
    const u64 x = __shfl_xor(best, o, 64);
    best = x > best ? x : best;
  }
  const bool ovf_w = __ballot(n_t > kSliceCap) != 0ull;
  const u64 inc_w = wave_incl_scan((u64)n_t, lane);
  if (lane == 63) {
    L.wcount[wv] = inc_w;
    L.wmax[wv] = best;
    L.wflag[wv] = ovf_w ? 1u : 0u;
  }
  __syncthreads();
  u64 before = 0, n_all = 0;
  bool overflow = false;
#pragma unroll
  for (int j = 0; j < kWaves; ++j) {
    const u64 x = L.wcount[j], m = L.wmax[j];
    before += (j < wv) ? x : 0ull;
    n_all += x;
    best = m > best ? m : best;
    overflow = overflow || L.wflag[j] != 0u;
  }
  const int32_t top = key_index(best, a.ibits, 0, V);
  if (!(T > 0.f) || k == 1) {
    if (t == 0) a.out[r] = top;
    return;
  }
  // the row's largest logit from its key's float bits (-0.0 comes back as
  // +0.0, which weighs and screens the same)
  const uint32_t kb = (uint32_t)(best >> a.ibits);
  Scale c;
  c.mf = __uint_as_float((kb & 0x80000000u) ? (kb & 0x7FFFFFFFu) : ~kb);
  c.m = (double)c.mf;
  c.T = (double)T;
  c.zf = 22.5f * T;

  if (!overflow) {
    // the slices' lists laid end to end: each flat position finds its slice
    // by binary search over the offsets
    const u64 end_t = inc_w + before;
    if (t < nsl) L.off[t] = (uint32_t)(end_t - (u64)n_t);
    __syncthreads();
    // (kListPer consecutive positions per thread: their loads go out together)
    u64 listed = 0;
    for (int base = 0; base < (int)n_all; base += kThreads * kListPer) {
      const int q0 = base + t * kListPer;
      int sl = 0;  // the last slice whose offset is <= q0
      if (q0 < (int)n_all) {
        int hi_s = nsl - 1;
        while (sl < hi_s) {
          const int mid = (sl + hi_s + 1) >> 1;
          if ((int)L.off[mid] <= q0) sl = mid; else hi_s = mid - 1;
        }
      }
      Cand e[kListPer];
#pragma unroll
      for (int i = 0; i < kListPer; ++i) {
        const int q = q0 + i;
        e[i] = Cand{0.f, 0};
        if (q < (int)n_all) {
          while (sl + 1 < nsl && (int)L.off[sl + 1] <= q) ++sl;  // past the slice's end
          e[i] = w.cand[(slot0 + sl) * kSliceCap + (size_t)(q - (int)L.off[sl])];
        }
      }
      bool keep[kListPer];
      uint32_t kc = 0;
#pragma unroll
      for (int i = 0; i < kListPer; ++i) {
        keep[i] = q0 + i < (int)n_all && !(c.mf - e[i].x > c.zf);
        kc += keep[i] ? 1u : 0u;
      }
      u64 tot;
      u64 pos = listed + block_incl_scan((u64)kc, L, &tot) - kc;
#pragma unroll
      for (int i = 0; i < kListPer; ++i) {
        if (keep[i]) {
          if (pos < (u64)kList) {
            L.cx[pos] = e[i].x;
            L.ci[pos] = e[i].i;
          }
          ++pos;
        }
      }
      listed += tot;
    }
    __syncthreads();
    if (listed <= (u64)kWaveList) {
      if (t >= 64) return;  // no workgroup barrier follows
      const int32_t pick = draw_wave(L, (int)listed, a.ibits, V, k, p, u, c, top, L);
      if (t == 0) a.out[r] = pick;
      return;
    }
    if (listed <= (u64)kList) {
      ListSrc src{L.cx, L.ci, (int)listed};
      const int32_t pick = draw(src, a.ibits, V, k, p, u, c, top, L);
      if (t == 0) a.out[r] = pick;
      return;
    }
  }
  RowSrc src{row, V};
  const int32_t pick = draw(src, a.ibits, V, k, p, u, c, top, L);
  if (t == 0) a.out[r] = pick;
}

// Workspace layout: lmax, count, cand, each region 256-byte aligned.
size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
int slices_for(int32_t vocab) { return (vocab + kSliceLen - 1) / kSliceLen; }
size_t ws_lmax_bytes(size_t n) { return align256(n * sizeof(u64)); }
size_t ws_count_bytes(size_t n) { return align256(n * sizeof(int32_t)); }
size_t ws_cand_bytes(size_t n) { return align256(n * kSliceCap * sizeof(Cand)); }

}  // namespace

extern "C" __attribute__((visibility("default"))) size_t pa_sample_workspace_size(int32_t rows,
                                                                                  int32_t vocab) {
  if (rows <= 0 || vocab < 1 || vocab > kMaxVocab) return 0;
  const size_t n = (size_t)rows * slices_for(vocab);
  return ws_lmax_bytes(n) + ws_count_bytes(n) + ws_cand_bytes(n);
}

extern "C" __attribute__((visibility("default"))) pa_status_t pa_sample_tokens(
    const float* logits, int64_t row_stride, int32_t rows, int32_t vocab,
    const float* temperature, const int32_t* top_k, const float* top_p, const float* uniforms,
    int32_t* out_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  if (rows < 0 || vocab < 1 || row_stride < vocab) return PA_ERR_INVALID_ARG;
  if (vocab > kMaxVocab) return PA_ERR_UNSUPPORTED;
  if (rows == 0) return PA_OK;
  if (!logits || !temperature || !top_k || !top_p || !uniforms || !out_tokens || !workspace)
    return PA_ERR_INVALID_ARG;
  if ((int64_t)rows * slices_for(vocab) > (1ll << 30)) return PA_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0u) return PA_ERR_INVALID_ARG;
  if (workspace_bytes < pa_sample_workspace_size(rows, vocab)) return PA_ERR_WORKSPACE_TOO_SMALL;
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
  const int nsl = slices_for(vocab);
  const size_t n = (size_t)rows * nsl;
  char* base = static_cast<char*>(workspace);
  SampleWs w;
  w.lmax = reinterpret_cast<u64*>(base);
  w.count = reinterpret_cast<int32_t*>(base + ws_lmax_bytes(n));
  w.cand = reinterpret_cast<Cand*>(base + ws_lmax_bytes(n) + ws_count_bytes(n));
  w.nsl = nsl;
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(sample_screen_kernel, dim3((unsigned)n), dim3(kScreenThreads), 0, st, a, w);
  if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  hipLaunchKernelGGL(sample_draw_kernel, dim3((unsigned)rows), dim3(kThreads), 0, st, a, w);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}
