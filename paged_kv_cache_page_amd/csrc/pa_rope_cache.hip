// K0: RoPE cos/sin table. a1: slot mapping. K1: RoPE on the new Q/K + page write.
//
// K1 is HBM-bound (about 0.1 flop per byte): one workgroup per new token moves
// its Q/K rows through registers once (read, rotate, write back in place) and
// stores K/V into the token's page slot with 16-byte vector accesses.
//
// This translation unit is compiled with -ffp-contract=off, and K1 also
// disables contraction locally: the rotation must round each product and each
// sum on its own, so the stored K is a fixed function of its inputs.
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_plan.h"

namespace pa {

// ---------------------------------------------------------------- K0 -------
// cos/sin of p * theta^(-2i/D), evaluated in double and rounded once to float.
__global__ __launch_bounds__(256) void rope_table_kernel(float* __restrict__ out, int max_pos,
                                                         int D, double theta) {
  const int half = D / 2;
  const long total = (long)max_pos * half;
  for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (long)gridDim.x * blockDim.x) {
    const int p = (int)(idx / half);
    const int i = (int)(idx % half);
    const double inv = pow(theta, -(2.0 * i) / (double)D);
    const double ang = (double)p * inv;
    out[(size_t)p * D + i] = (float)cos(ang);
    out[(size_t)p * D + half + i] = (float)sin(ang);
  }
}

hipError_t launch_rope_table(float* out, int max_pos, int D, double theta, hipStream_t s) {
  const long total = (long)max_pos * (D / 2);
  long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  profile_before("rope_table", s);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, s, out, max_pos,
                     D, theta);
  profile_after(s);
  return hipGetLastError();
}

// ---------------------------------------------------------------- a1 -------
// Token t belongs to the last sequence s with qsl[s] <= t (empty sequences
// have qsl[s] == qsl[s+1] and are passed over by the search). The workgroup
// first copies query_start_loc into LDS (one round of loads) and searches
// there, instead of a chain of dependent global loads per token.
constexpr int kSlotThreads = 256;
constexpr int kSlotQslLds = 4096;  // sequences searched in LDS; longer lists are read from memory

__global__ __launch_bounds__(kSlotThreads) void slot_mapping_kernel(
    const int32_t* __restrict__ bt, const int32_t* __restrict__ qsl,
    const int32_t* __restrict__ pos, int32_t* __restrict__ slots, int S, int T, int max_blocks,
    int P, int num_pages) {
  __shared__ int s_qsl[kSlotQslLds + 1];
  const bool in_lds = S <= kSlotQslLds;
  if (in_lds)
    for (int i = threadIdx.x; i <= S; i += kSlotThreads) s_qsl[i] = qsl[i];
  const int t = blockIdx.x * kSlotThreads + threadIdx.x;
  const int p = t < T ? pos[t] : -1;  // issued before the barrier: overlaps the copy
  __syncthreads();
  if (t >= T) return;
  int lo = 0, hi = S;  // qsl[lo] <= t < qsl[hi] when the metadata is well formed
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((in_lds ? s_qsl[mid] : qsl[mid]) <= t) lo = mid; else hi = mid;
  }
  int slot = -1;
  if (p >= 0) {
    const int blk = p / P;
    if (blk < max_blocks) {
      const int page = bt[(size_t)lo * max_blocks + blk];
      if (page >= 0 && page < num_pages) slot = page * P + p % P;
    }
  }
  slots[t] = slot;
}

hipError_t launch_slot_mapping(const int32_t* bt, const int32_t* qsl, const int32_t* pos,
                               int32_t* slots, int S, int T, int max_blocks, int P,
                               int num_pages, hipStream_t s) {
  if (T == 0) return hipSuccess;
  profile_before("slot_mapping", s);
  hipLaunchKernelGGL(slot_mapping_kernel, dim3((T + kSlotThreads - 1) / kSlotThreads),
                     dim3(kSlotThreads), 0, s, bt, qsl, pos, slots, S, T, max_blocks, P,
                     num_pages);
  profile_after(s);
  return hipGetLastError();
}

// ---------------------------------------------------------------- K1 -------
// One 16-byte vector of the first half of a head row and the matching vector of
// the second half: VP rotation pairs.
template <typename ET>
struct RotPair;

template <>
struct RotPair<BF16> {
  static constexpr int VP = 8;
  __device__ static void rotate(uint4& a, uint4& b, const float* c, const float* s) {
    rope_bf16x8(a, b, c, s);
  }
};

template <>
struct RotPair<F32> {
  static constexpr int VP = 4;
  __device__ static void rotate(uint4& a, uint4& b, const float* c, const float* s) {
#pragma clang fp contract(off)
    float* x1 = reinterpret_cast<float*>(&a);
    float* x2 = reinterpret_cast<float*>(&b);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p1 = x1[i] * c[i], q1 = x2[i] * s[i];
      const float p2 = x2[i] * c[i], q2 = x1[i] * s[i];
      x1[i] = p1 - q1;
      x2[i] = p2 + q2;
    }
  }
};

constexpr int kRopeThreads = 256;

struct RopeArgs {
  char* q;
  char* k;
  const char* v;
  const int32_t* pos;
  const float* cs;
  char* k_pool;
  char* v_pool;
  int Hq, Hkv, D, P, num_pages, max_pos;
  char* q_out;  // the fused tick: where the decode rows' rotated queries go (their out rows)
};

// K1 for token t, whose page slot is `slot` (stored only when in the pool).
// IN_PLACE: q and k are rotated in place (pa_rope_and_cache_write). Otherwise
// (the fused tick) k is left as it is and its rotated rows go to the pool
// only, and the rotated query rows go to r.q_out's row t when q_to_out (a
// decode row, whose attention reads them there) or nowhere (a prefill row: the
// attention kernel rotates those where it reads them).
template <typename ET, bool IN_PLACE = true>
__device__ __forceinline__ void rope_token(const RopeArgs& r, int t, long slot,
                                           bool q_to_out = false) {
  constexpr int EB = ET::kBytes;
  constexpr int VP = RotPair<ET>::VP;       // elements per 16-byte vector
  const int D = r.D, Hkv = r.Hkv;
  const int half = D / 2;
  const int vec_half = half / VP;           // vectors per half row
  const int vec_row = D / VP;               // vectors per row
  const size_t row_bytes = (size_t)D * EB;
  const int p = r.pos[t];
  const bool rotate = r.cs != nullptr && p >= 0 && p < r.max_pos;
  const bool store = slot >= 0 && slot < (long)r.num_pages * r.P;
  const int nq = r.q && (IN_PLACE || q_to_out) ? r.Hq : 0;
  const int rot_tasks = (nq + Hkv) * vec_half;
  const int tasks = rot_tasks + Hkv * vec_row;
  // The block size is a multiple of vec_half (see the launch), so a
  // thread's rotation tasks all take the same vector c of the half row: its
  // cos/sin values are loaded once.
  const int c = (int)threadIdx.x % vec_half;
  float cv[VP], sv[VP];
  if (rotate) {
    const float4* cp = reinterpret_cast<const float4*>(r.cs + (size_t)p * D + c * VP);
    const float4* sp = reinterpret_cast<const float4*>(r.cs + (size_t)p * D + half + c * VP);
#pragma unroll
    for (int i = 0; i < VP / 4; ++i) {
      const float4 cc = cp[i], ss = sp[i];
      cv[4 * i] = cc.x; cv[4 * i + 1] = cc.y; cv[4 * i + 2] = cc.z; cv[4 * i + 3] = cc.w;
      sv[4 * i] = ss.x; sv[4 * i + 1] = ss.y; sv[4 * i + 2] = ss.z; sv[4 * i + 3] = ss.w;
    }
  }
  for (int task = threadIdx.x; task < tasks; task += blockDim.x) {
    if (task < rot_tasks) {
      const int h = task / vec_half;
      const bool is_k = h >= nq;
      const int kh = h - nq;
      char* row = is_k ? r.k + ((size_t)t * Hkv + kh) * row_bytes
                       : r.q + ((size_t)t * r.Hq + h) * row_bytes;
      uint4* p1 = reinterpret_cast<uint4*>(row + (size_t)c * 16);
      uint4* p2 = reinterpret_cast<uint4*>(row + (size_t)half * EB + (size_t)c * 16);
      uint4 a = *p1, b = *p2;
      if (rotate) RotPair<ET>::rotate(a, b, cv, sv);
      if (IN_PLACE) {
        if (rotate) {
          *p1 = a;
          *p2 = b;
        }
      } else if (!is_k) {
        // (q_to_out) the query row, rotated or as given, in the output row
        char* orow = r.q_out + ((size_t)t * r.Hq + h) * row_bytes;
        *reinterpret_cast<uint4*>(orow + (size_t)c * 16) = a;
        *reinterpret_cast<uint4*>(orow + (size_t)half * EB + (size_t)c * 16) = b;
      }
      if (is_k && store) {
        char* dst = r.k_pool + ((size_t)slot * Hkv + kh) * row_bytes;
        *reinterpret_cast<uint4*>(dst + (size_t)c * 16) = a;
        *reinterpret_cast<uint4*>(dst + (size_t)half * EB + (size_t)c * 16) = b;
      }
    } else if (store) {
      const int j = task - rot_tasks;
      const int h = j / vec_row;
      const int cj = j % vec_row;
      const uint4 x = *reinterpret_cast<const uint4*>(r.v + ((size_t)t * Hkv + h) * row_bytes +
                                                      (size_t)cj * 16);
      *reinterpret_cast<uint4*>(r.v_pool + ((size_t)slot * Hkv + h) * row_bytes +
                                (size_t)cj * 16) = x;
    }
  }
}

template <typename ET>
__global__ __launch_bounds__(kRopeThreads) void rope_cache_write_kernel(
    RopeArgs r, const int32_t* __restrict__ slots) {
  rope_token<ET>(r, blockIdx.x, slots[blockIdx.x]);
}

// Threads of a K1 workgroup: the largest multiple of the vectors per half row
// (D / 16 for bf16, D / 8 for fp32) that fits the block.
int rope_threads(pa_dtype_t dt, int D) {
  const int vec_half = D / 2 / (dt == PA_BF16 ? 8 : 4);
  return kRopeThreads / vec_half * vec_half;
}

hipError_t launch_rope_cache_write(pa_dtype_t dt, void* q, void* k, const void* v,
                                   const int32_t* pos, const int32_t* slots, const float* cs,
                                   void* k_pool, void* v_pool, int T, int Hq, int Hkv, int D,
                                   int P, int num_pages, int max_pos, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const RopeArgs r{(char*)q, (char*)k, (const char*)v, pos, cs, (char*)k_pool, (char*)v_pool,
                   Hq, Hkv, D, P, num_pages, max_pos};
  const int threads = rope_threads(dt, D);
  profile_before("rope_cache_write", s);
  if (dt == PA_BF16)
    hipLaunchKernelGGL(rope_cache_write_kernel<BF16>, dim3(T), dim3(threads), 0, s, r, slots);
  else
    hipLaunchKernelGGL(rope_cache_write_kernel<F32>, dim3(T), dim3(threads), 0, s, r, slots);
  profile_after(s);
  return hipGetLastError();
}

// ------------------------------------------------------- a1 + K1 + plan -----
// The tick's forward before attention, in one launch: workgroup 0's first
// wave computes the attention plan (it reads only query_start_loc and
// seq_lens), every other workgroup takes one token: finds its sequence and
// page slot (a1; the slot is also stored), then rotates and writes it (K1).
// The launch ends when the longer of the two is done, instead of running
// slot mapping, page write and plan one after the other.

// Last sequence s in [0, S) with qsl[s] <= t (0 if none): the same sequence
// as a1's search when query_start_loc is non-decreasing. One wave, all lanes
// together: each round tests 64 evenly spaced entries of the remaining range
// and keeps the stretch between the last entry <= t and the next.
__device__ __forceinline__ int wave_find_seq(const int32_t* __restrict__ qsl, int S, int t) {
  const int lane = (int)threadIdx.x & 63;
  int lo = 0, len = S;
  while (len > 64) {
    const int stride = (len + 63) / 64;
    const bool le = lane * stride < len && qsl[lo + lane * stride] <= t;
    const int c = __popcll(__ballot(le));
    if (c == 0) return lo;
    lo += (c - 1) * stride;
    len = min(stride, len - (c - 1) * stride);
  }
  const bool le = lane < len && qsl[lo + lane] <= t;
  const int c = __popcll(__ballot(le));
  return c == 0 ? lo : lo + c - 1;
}

// Fewer cached sequence shapes than the plan kernel: this LDS is reserved by
// every workgroup of the launch, and the page-write workgroups need all their
// compute unit's slots (8 KiB of cost bins + 12 B per cached sequence).
constexpr int kPrepCachedSeqs = 960;

// FUSED (the bf16 tick): q and k are left as they are. Every token rotates
// its k into the pool only; a token that is a decode row of the plan (query
// length 1, at least one key) also puts its rotated query rows in its output
// row, where the decode kernel reads them (a few hundred KB: one row per
// decode sequence); the prefill chunks' query rows are rotated by the
// attention kernel where it reads them, so the chunks' queries (most of q)
// are read once instead of read, written and read again.
template <typename ET, bool FUSED>
__global__ __launch_bounds__(kRopeThreads) void tick_prep_kernel(
    RopeArgs r, const int32_t* __restrict__ bt, const int32_t* __restrict__ qsl,
    int32_t* __restrict__ slots, int S, int max_blocks, AttnArgs a, int cap_dec, int cap_pf,
    int TM, int plan_blocks) {
  __shared__ PlanLds<kPrepCachedSeqs> sm;
  if ((int)blockIdx.x < plan_blocks) {
    if (threadIdx.x < 64) plan_wave(a, a.plan, cap_dec, cap_pf, TM, sm);
    return;
  }
  const int t = (int)blockIdx.x - plan_blocks;
  const int p = r.pos[t];
  const int seq = wave_find_seq(qsl, S, t);
  int slot = -1;
  if (p >= 0) {
    const int blk = p / r.P;
    if (blk < max_blocks) {
      const int page = bt[(size_t)seq * max_blocks + blk];
      if (page >= 0 && page < r.num_pages) slot = page * r.P + p % r.P;
    }
  }
  if (threadIdx.x == 0) slots[t] = slot;
  if constexpr (FUSED) {
    // (seq is the same in every lane and wave of the workgroup)
    const SeqShape sh = seq_shape(a, seq);
    rope_token<ET, false>(r, t, slot, sh.L == 1 && sh.n >= 1 && sh.q0 == t);
  } else {
    rope_token<ET>(r, t, slot);
  }
}

hipError_t launch_tick_prep(pa_dtype_t dt, void* q, void* k, const void* v, const int32_t* pos,
                            const int32_t* bt, const int32_t* qsl, int32_t* slots,
                            const float* cs, void* k_pool, void* v_pool, int S, int T, int Hq,
                            int Hkv, int D, int P, int num_pages, int max_blocks, int max_pos,
                            const AttnArgs* plan_args, int cap_dec, int cap_pf, int TM,
                            bool fused, hipStream_t s) {
  const int plan_blocks = plan_args ? 1 : 0;
  if (T + plan_blocks == 0) return hipSuccess;
  if (fused && (!plan_args || dt != PA_BF16)) return hipErrorInvalidValue;
  RopeArgs r{(char*)q, (char*)k, (const char*)v, pos, cs, (char*)k_pool, (char*)v_pool,
                   Hq, Hkv, D, P, num_pages, max_pos};
  r.q_out = fused && plan_args ? (char*)plan_args->out : nullptr;
  AttnArgs a{};
  if (plan_args) a = *plan_args;
  const int threads = rope_threads(dt, D);
  const dim3 grid((unsigned)(T + plan_blocks));
  profile_before(fused ? "tick_plan_write" : "tick_prep", s);
  if (fused)
    hipLaunchKernelGGL((tick_prep_kernel<BF16, true>), grid, dim3(threads), 0, s, r, bt, qsl,
                       slots, S, max_blocks, a, cap_dec, cap_pf, TM, plan_blocks);
  else if (dt == PA_BF16)
    hipLaunchKernelGGL((tick_prep_kernel<BF16, false>), grid, dim3(threads), 0, s, r, bt, qsl,
                       slots, S, max_blocks, a, cap_dec, cap_pf, TM, plan_blocks);
  else
    hipLaunchKernelGGL((tick_prep_kernel<F32, false>), grid, dim3(threads), 0, s, r, bt, qsl,
                       slots, S, max_blocks, a, cap_dec, cap_pf, TM, plan_blocks);
  profile_after(s);
  return hipGetLastError();
}

}  // namespace pa
