// The C ABI of libpa (declared in include/pa.h): host-scalar checks, workspace
// sizing, launch dispatch, and the optional kernel-timing hook.
//
// No entry point reads device memory from the host, allocates, frees or
// synchronises (the profiling calls and the opt-in validation mode aside).
// Every host-scalar check happens before the first HIP call, so argument
// errors are reported without touching a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// ------------------------------------------------------------- timing ------
namespace {
struct ProfRec {
  const char* name;
  hipEvent_t start;
  hipEvent_t stop;
};
std::vector<ProfRec> g_recs;
bool g_prof_on = false;
int g_prof_n = 0;
bool g_prof_open = false;  // a profile_before without its profile_after

void destroy_events() {
  for (auto& r : g_recs) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_recs.clear();
  g_prof_n = 0;
}
}  // namespace

void profile_before(const char* name, hipStream_t stream) {
  g_prof_open = false;
  if (!g_prof_on || g_prof_n >= (int)g_recs.size()) return;
  g_recs[g_prof_n].name = name;
  if (hipEventRecord(g_recs[g_prof_n].start, stream) == hipSuccess) g_prof_open = true;
}

void profile_after(hipStream_t stream) {
  if (!g_prof_open) return;
  g_prof_open = false;
  if (hipEventRecord(g_recs[g_prof_n].stop, stream) == hipSuccess) ++g_prof_n;
}

// ------------------------------------------------------- grid sizing -----
namespace {
std::mutex g_grid_mu;
std::map<std::pair<int, const void*>, int> g_grid_cache;
}  // namespace

int cu_count() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  cache[dev] = cus;
  return cus;
}

int persistent_grid(const void* func, int threads) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(g_grid_mu);
  auto key = std::make_pair(dev, func);
  auto it = g_grid_cache.find(key);
  if (it != g_grid_cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, func, threads, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  const int grid = cus * per_cu;
  g_grid_cache[key] = grid;
  return grid;
}

// ------------------------------------------------------------- helpers -----
namespace {

constexpr int kTokenModeSplitTokens = 512;  // partition size of the per-token path
constexpr int kAutoMinSplitTokens = 256;    // smallest partition the plan kernel picks

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_bytes(pa_dtype_t dt) { return dt == PA_BF16 ? 2 : 4; }

bool dtype_ok(int dt) { return dt == PA_F32 || dt == PA_BF16; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

// Largest partition: the decode kernel holds a partition's page ids in one
// VGPR (64 lanes), and a partition of 63 * P keys spans at most 64 pages.
int split_max(int P) {
  const long cap = 63L * P;
  return (int)((cap < 65536 ? cap : 65536) / 16 * 16);
}

int split_min(int P) {
  const int mx = split_max(P);
  return kAutoMinSplitTokens < mx ? kAutoMinSplitTokens : mx;
}

// Keys per split-KV partition for these arguments: the request (capped), or
// 0 = chosen on the device by the plan kernel (per-sequence rows only).
int split_tokens(int requested, int P, bool token_mode) {
  const int mx = split_max(P);
  if (requested > 0) return requested < mx ? requested : mx;
  if (token_mode) return kTokenModeSplitTokens < mx ? kTokenModeSplitTokens : mx;
  return 0;
}

// Whether prefill rows (L > 1) go to the MFMA kernel; otherwise every row of
// the tick takes the per-token VALU path.
bool use_mfma_prefill(pa_dtype_t dt, int D, int max_query_len) {
  return max_query_len <= 1 || tick_supported(dt, D);
}

// Workspace layout: the plan lists (seq mode), padded to 256 bytes, then the
// split-KV partials (o for every (row, partition, head), then (m, l) pairs),
// then, for ticks with prefill chunks and automatic partitions, the prefill
// piece partials and their arrival counters.
struct WsLayout {
  long cap_dec, cap_pf;
  size_t plan_bytes, partial_bytes, pf_bytes;
  long part_slots;
  int max_parts, pf_slots;
  bool token_mode;
};

WsLayout workspace_layout(int S, int T, int Hq, int D, int max_query_len, int max_seq_len, int P,
                          int kv_split, pa_dtype_t dt) {
  WsLayout w;
  w.token_mode = !use_mfma_prefill(dt, D, max_query_len);
  const int pt = split_tokens(kv_split, P, w.token_mode);
  long max_parts;
  if (pt > 0) {
    // fixed partitions of pt keys, aligned to the row start
    max_parts = max_seq_len > 0 ? ((long)max_seq_len + pt - 1) / pt : 1;
  } else {
    // equal chunks of the concatenated key axis, at least split_min keys each:
    // a row may straddle one chunk boundary more than its length needs
    const int c = split_min(P);
    max_parts = max_seq_len > 0 ? ((long)max_seq_len + c - 1) / c + 1 : 1;
  }
  w.max_parts = (int)(max_parts < 1 ? 1 : max_parts);
  w.cap_dec = 0;
  w.cap_pf = 0;
  w.plan_bytes = 0;
  w.pf_slots = 0;
  w.pf_bytes = 0;
  // partial slots: at most max_parts per row (packed by the plan kernel in
  // seq mode: a row has one partition per chunk it overlaps)
  w.part_slots = (long)(w.token_mode ? T : S) * w.max_parts;
  if (!w.token_mode) {
    w.cap_dec = (long)S * w.max_parts;
    if (pt == 0) {
      // Automatic partitions: the plan cuts the decode key axis (at most S rows
      // of round_up(max_seq_len, 16) keys) into chunks of at least one decode
      // wave's share, so there are at most as many chunks as decode waves per
      // KV head (at most dec_grid * 4 * 8 / Hq: a group has at most 8 heads),
      // unless the largest partition caps the chunk, and then at most
      // keys / split_max chunks. A row has one partition per chunk it overlaps,
      // and the rows and chunks tile the same axis, so the rows' partitions
      // number at most rows + chunks.
      const long waves = ((long)decode_grid_max(dt, D) * 4 * 8 + Hq - 1) / Hq;
      const long keys = (long)S * (((long)max_seq_len + 15) / 16 * 16);
      const long by_cap = (keys + split_max(P) - 1) / split_max(P);
      const long chunks = waves > by_cap ? waves : by_cap;
      if (chunks < w.cap_dec) w.cap_dec = chunks;
      // (bf16: room for grouped rows of a shared prefix, whose members also
      // hold partials of their group row's partitions; the plan groups rows
      // only while their partials fit)
      const long group_room = dt == PA_BF16 ? kGroupSlotsPerRow * (long)S : 0;
      if ((long)S + chunks + group_room < w.part_slots)
        w.part_slots = (long)S + chunks + group_room;
    }
    if (max_query_len > 1) {
      // a tile holds at least kPrefillRows / 8 tokens (the largest supported group is 8)
      const int tm = kPrefillRows / 8;
      const long by_seq = (long)S * ((max_query_len + tm - 1) / tm);
      const long by_tok = (long)T / tm + S;
      w.cap_pf = by_seq < by_tok ? by_seq : by_tok;
      if (pt == 0) {
        // automatic partitions: long items may be cut into pieces, at most one
        // extra entry per partial slot
        w.pf_slots = kPrefillSlots;
        w.cap_pf += kPrefillSlots;
        w.pf_bytes = ((size_t)kPrefillSlots * kPrefillRows * ((size_t)D + 2) * sizeof(float) +
                      255) / 256 * 256;
      }
    }
    w.plan_bytes = (plan_offsets(S, Hq, w.cap_dec, w.cap_pf).total * sizeof(int) + 255) / 256 * 256;
  }
  w.partial_bytes = w.max_parts > 1 ? ((size_t)w.part_slots * (size_t)Hq *
                                           ((size_t)D + 2) * sizeof(float) + 255) / 256 * 256
                                    : 0;
  return w;
}

size_t workspace_bytes_for(int S, int T, int Hq, int D, int max_query_len, int max_seq_len,
                           int P, int kv_split, pa_dtype_t dt) {
  const WsLayout w = workspace_layout(S, T, Hq, D, max_query_len, max_seq_len, P, kv_split, dt);
  return w.plan_bytes + w.partial_bytes + w.pf_bytes;
}

pa_status_t from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// ------------------------------------------------------- validation -----
// Opt-in checks of the device metadata (pa_set_validation): the metadata is
// copied to the host on the call's stream (which is synchronised first, so the
// values checked are the ones the kernels would read) and every precondition
// the kernels otherwise take on trust is tested before anything is enqueued.
// A failure returns PA_ERR_INVALID_ARG and leaves its reason, naming the
// sequence or token, in a per-thread message (the pages' engines report a
// failing request by name: Helios README, "Diagnostics and logs").
std::atomic<int> g_validate{0};
thread_local char g_vmsg[256] = "";

pa_status_t vfail(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_vmsg, sizeof g_vmsg, fmt, ap);
  va_end(ap);
  return PA_ERR_INVALID_ARG;
}

bool validating() { return g_validate.load(std::memory_order_relaxed) != 0; }

template <typename T>
pa_status_t fetch(std::vector<T>& h, const T* d, size_t n, hipStream_t s) {
  h.resize(n);
  if (n == 0) return PA_OK;
  return from_hip(hipMemcpyAsync(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost, s));
}

// The sequences' metadata on the host.
struct HostMeta {
  std::vector<int32_t> qsl, seq_lens, bt, pos, slots;
};

// query_start_loc of S sequences over T rows: starts at 0, never decreases,
// ends at T.
pa_status_t check_qsl(const HostMeta& m, int S, int T) {
  if (m.qsl[0] != 0) return vfail("query_start_loc[0] = %d, not 0", m.qsl[0]);
  for (int s = 0; s < S; ++s)
    if (m.qsl[s + 1] < m.qsl[s])
      return vfail("query_start_loc decreases at sequence %d (%d -> %d)", s, m.qsl[s],
                   m.qsl[s + 1]);
  if (m.qsl[S] != T) return vfail("query_start_loc[S] = %d, not T = %d", m.qsl[S], T);
  return PA_OK;
}

// Every sequence with rows: L <= n <= max_seq_len, L <= max_query_len, and the
// first ceil(n / P) entries of its page-table row valid page ids.
pa_status_t check_seqs(const HostMeta& m, int S, int P, int num_pages, int max_blocks,
                       int max_query_len, int max_seq_len) {
  for (int s = 0; s < S; ++s) {
    const int L = m.qsl[s + 1] - m.qsl[s], n = m.seq_lens[s];
    if (n < 0) return vfail("sequence %d: seq_len %d < 0", s, n);
    if (L == 0) continue;
    if (L > n) return vfail("sequence %d: %d query rows > seq_len %d", s, L, n);
    if (n > max_seq_len) return vfail("sequence %d: seq_len %d > max_seq_len %d", s, n, max_seq_len);
    if (L > max_query_len)
      return vfail("sequence %d: %d query rows > max_query_len %d", s, L, max_query_len);
    const long pages = ((long)n + P - 1) / P;
    if (pages > max_blocks)
      return vfail("sequence %d: seq_len %d needs %ld pages > max_blocks_per_seq %d", s, n, pages,
                   max_blocks);
    for (long j = 0; j < pages; ++j) {
      const int pg = m.bt[(size_t)s * max_blocks + j];
      if (pg < 0 || pg >= num_pages)
        return vfail("sequence %d: block_tables[%d][%ld] = %d outside [0, %d)", s, s, j, pg,
                     num_pages);
    }
  }
  return PA_OK;
}

// The rows of a tick: row i of sequence s (L rows, n keys) is the token at
// position n - L + i, its slot is a pool slot, and the page it is written to
// belongs to no other sequence (pages shared between sequences are full and
// read-only: Helios blog, "Prefix caching").
pa_status_t check_tick_rows(const HostMeta& m, int S, int P, int max_blocks, int max_pos,
                            bool rope) {
  std::unordered_map<int, int> owner;  // page -> the one sequence that uses it, or -1
  for (int s = 0; s < S; ++s) {
    if (m.qsl[s + 1] == m.qsl[s]) continue;
    const long pages = ((long)m.seq_lens[s] + P - 1) / P;
    for (long j = 0; j < pages; ++j) {
      const int pg = m.bt[(size_t)s * max_blocks + j];
      auto it = owner.find(pg);
      if (it == owner.end()) owner[pg] = s;
      else if (it->second != s) it->second = -1;
    }
  }
  for (int s = 0; s < S; ++s) {
    const int q0 = m.qsl[s], L = m.qsl[s + 1] - q0, n = m.seq_lens[s];
    for (int i = 0; i < L; ++i) {
      const int t = q0 + i, p = m.pos[t];
      if (p != n - L + i)
        return vfail("token %d (sequence %d, row %d of %d): position %d, not seq_len - L + row "
                     "= %d", t, s, i, L, p, n - L + i);
      if (rope && p >= max_pos)
        return vfail("token %d (sequence %d): position %d outside the cos/sin table (%d rows)",
                     t, s, p, max_pos);
      const int pg = m.bt[(size_t)s * max_blocks + p / P];
      if (owner[pg] != s)
        return vfail("token %d (sequence %d): writes page %d, which another sequence also uses",
                     t, s, pg);
    }
  }
  return PA_OK;
}

// No two rows write the same pool slot.
pa_status_t check_slots_unique(const std::vector<int32_t>& slots, long pool_slots) {
  std::unordered_map<int, int> seen;
  for (size_t t = 0; t < slots.size(); ++t) {
    const int sl = slots[t];
    if (sl < 0 || sl >= pool_slots) continue;  // skipped rows
    auto r = seen.emplace(sl, (int)t);
    if (!r.second) return vfail("tokens %d and %zu write the same slot %d", r.first->second, t, sl);
  }
  return PA_OK;
}

}  // namespace
}  // namespace pa

namespace pa {
namespace {

// ------------------------------------------------ fixed scratch -----
// The scratch of pa_tick_forward_noalloc: one fixed array per GPU, for callers
// that cannot allocate (graph capture, serving loops without hipMalloc). The
// runtime places it in each GPU's memory when the library's code is loaded
// there, and it stays until the process ends. In host code `scratch` names a
// host-side stand-in, not device memory: host code uses only the device
// address looked up below, once per device with that device current.
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr size_t kScratchAlign = 256;
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_of;  // device -> address of its `scratch`

pa_status_t scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_of.find(dev);
  if (it == g_scratch_of.end()) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr ||
        ((uintptr_t)ptr % kScratchAlign) != 0)
      return PA_ERR_HIP;
    it = g_scratch_of.emplace(dev, ptr).first;
  }
  *out = it->second;
  return PA_OK;
}

}  // namespace
}  // namespace pa

using namespace pa;

#pragma GCC visibility push(default)
extern "C" {

int32_t pa_abi_version(void) { return 7; }

void pa_set_validation(int32_t on) { g_validate.store(on ? 1 : 0, std::memory_order_relaxed); }

const char* pa_validation_message(void) { return g_vmsg; }

const char* pa_status_string(pa_status_t status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG: a host argument is invalid";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: no kernel for this dtype/shape";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "PA_ERR_WORKSPACE_TOO_SMALL: workspace below the size query";
    case PA_ERR_HIP: return "PA_ERR_HIP: a HIP call failed";
    case PA_ERR_NO_PAGES: return "PA_ERR_NO_PAGES: too few free pages for the reservation";
  }
  return "PA_ERR_UNKNOWN";
}

pa_status_t pa_rope_cos_sin_table(float* cos_sin, int32_t max_pos, int32_t head_dim,
                                  double theta, void* stream) {
  if (!cos_sin || max_pos < 1 || head_dim < 2 || head_dim % 2 || !(theta > 0.0) ||
      !isfinite(theta))
    return PA_ERR_INVALID_ARG;
  return from_hip(launch_rope_table(cos_sin, max_pos, head_dim, theta, (hipStream_t)stream));
}

namespace {
pa_status_t slot_mapping_check(const int32_t* block_tables, const int32_t* query_start_loc,
                               const int32_t* positions, const int32_t* slot_mapping, int32_t S,
                               int32_t T, int32_t max_blocks_per_seq, int32_t page_size,
                               int32_t num_pages) {
  if (S < 0 || T < 0 || max_blocks_per_seq < 1 || page_size < 1 || num_pages < 1)
    return PA_ERR_INVALID_ARG;
  if ((long)num_pages * page_size > INT32_MAX) return PA_ERR_INVALID_ARG;
  if (T > 0 && (S < 1 || !block_tables || !query_start_loc || !positions || !slot_mapping))
    return PA_ERR_INVALID_ARG;
  return PA_OK;
}

pa_status_t rope_check(const void* q, const void* k, const void* v, const int32_t* positions,
                       const int32_t* slot_mapping, const float* cos_sin, const void* k_pool,
                       const void* v_pool, int32_t T, int32_t Hq, int32_t Hkv, int32_t head_dim,
                       int32_t page_size, int32_t num_pages, int32_t max_pos, pa_dtype_t dtype) {
  if (!dtype_ok(dtype) || T < 0 || Hq < 0 || Hkv < 1 || head_dim < 1 || page_size < 1 ||
      num_pages < 1)
    return PA_ERR_INVALID_ARG;
  if ((long)num_pages * page_size > INT32_MAX) return PA_ERR_INVALID_ARG;
  if (q && Hq < 1) return PA_ERR_INVALID_ARG;
  if (cos_sin && max_pos < 1) return PA_ERR_INVALID_ARG;
  // 16-byte vectors on each half row, at most one workgroup's worth per half row
  if (head_dim % 16 || head_dim > kRopeMaxHeadDim) return PA_ERR_UNSUPPORTED;
  if (T == 0) return PA_OK;
  if (!k || !v || !positions || !slot_mapping || !k_pool || !v_pool) return PA_ERR_INVALID_ARG;
  if ((q && !aligned16(q)) || !aligned16(k) || !aligned16(v) || !aligned16(k_pool) ||
      !aligned16(v_pool) || (cos_sin && !aligned16(cos_sin)))
    return PA_ERR_INVALID_ARG;
  return PA_OK;
}
}  // namespace

pa_status_t pa_compute_slot_mapping(const int32_t* block_tables, const int32_t* query_start_loc,
                                    const int32_t* positions, int32_t* slot_mapping, int32_t S,
                                    int32_t T, int32_t max_blocks_per_seq, int32_t page_size,
                                    int32_t num_pages, void* stream) {
  const pa_status_t st = slot_mapping_check(block_tables, query_start_loc, positions,
                                            slot_mapping, S, T, max_blocks_per_seq, page_size,
                                            num_pages);
  if (st != PA_OK) return st;
  g_vmsg[0] = '\0';
  if (validating() && T > 0) {
    HostMeta m;
    const hipStream_t hs = (hipStream_t)stream;
    if (fetch(m.qsl, query_start_loc, (size_t)S + 1, hs) != PA_OK ||
        hipStreamSynchronize(hs) != hipSuccess)
      return PA_ERR_HIP;
    const pa_status_t vs = check_qsl(m, S, T);
    if (vs != PA_OK) return vs;
  }
  return from_hip(launch_slot_mapping(block_tables, query_start_loc, positions, slot_mapping, S,
                                      T, max_blocks_per_seq, page_size, num_pages,
                                      (hipStream_t)stream));
}

pa_status_t pa_rope_and_cache_write(void* q, void* k, const void* v, const int32_t* positions,
                                    const int32_t* slot_mapping, const float* cos_sin,
                                    void* k_pool, void* v_pool, int32_t T, int32_t Hq,
                                    int32_t Hkv, int32_t head_dim, int32_t page_size,
                                    int32_t num_pages, int32_t max_pos, pa_dtype_t dtype,
                                    void* stream) {
  const pa_status_t st = rope_check(q, k, v, positions, slot_mapping, cos_sin, k_pool, v_pool, T,
                                    Hq, Hkv, head_dim, page_size, num_pages, max_pos, dtype);
  if (st != PA_OK || T == 0) return st;
  g_vmsg[0] = '\0';
  if (validating()) {
    HostMeta m;
    const hipStream_t hs = (hipStream_t)stream;
    if (fetch(m.slots, slot_mapping, (size_t)T, hs) != PA_OK ||
        hipStreamSynchronize(hs) != hipSuccess)
      return PA_ERR_HIP;
    const pa_status_t vs = check_slots_unique(m.slots, (long)num_pages * page_size);
    if (vs != PA_OK) return vs;
  }
  return from_hip(launch_rope_cache_write(dtype, q, k, v, positions, slot_mapping, cos_sin,
                                          k_pool, v_pool, T, Hq, Hkv, head_dim, page_size,
                                          num_pages, max_pos, (hipStream_t)stream));
}

size_t pa_paged_attention_workspace_size(int32_t S, int32_t T, int32_t Hq, int32_t head_dim,
                                         int32_t max_query_len, int32_t max_seq_len,
                                         int32_t page_size, int32_t kv_split_tokens,
                                         pa_dtype_t dtype) {
  if (S < 0 || T < 0 || Hq < 1 || head_dim < 1 || page_size < 1 || max_seq_len < 0 ||
      max_query_len < 0 || !dtype_ok(dtype) || kv_split_tokens < 0)
    return 0;
  return workspace_bytes_for(S, T, Hq, head_dim, max_query_len, max_seq_len, page_size,
                             kv_split_tokens, dtype);
}

namespace {

// One attention call prepared: its checked arguments and workspace layout.
struct AttnCall {
  AttnArgs a;
  WsLayout wl;
  pa_dtype_t dtype;
  int G;
  bool empty;  // nothing to enqueue (no rows)
};

// Every host-side check of pa_paged_attention_varlen, then the kernel
// arguments. Enqueues nothing.
pa_status_t attention_setup(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_tables, const int32_t* seq_lens,
                            const int32_t* query_start_loc, void* out, int32_t S, int32_t T,
                            int32_t Hq, int32_t Hkv, int32_t head_dim, int32_t page_size,
                            int32_t num_pages, int32_t max_blocks_per_seq,
                            int32_t max_query_len, int32_t max_seq_len, float scale,
                            int32_t kv_split_tokens, pa_dtype_t dtype, void* workspace,
                            size_t workspace_bytes, AttnCall& c) {
  c.empty = false;
  c.dtype = dtype;
  if (!dtype_ok(dtype) || S < 0 || S >= kRowGroup || T < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv ||
      head_dim < 1 || page_size < 1 || num_pages < 1 || max_blocks_per_seq < 1 ||
      max_query_len < 0 || max_seq_len < 0 || !isfinite(scale))
    return PA_ERR_INVALID_ARG;
  if (kv_split_tokens != 0 && (kv_split_tokens < 16 || kv_split_tokens > 65536 ||
                               kv_split_tokens % 16))
    return PA_ERR_INVALID_ARG;
  if ((long)num_pages * page_size > INT32_MAX) return PA_ERR_INVALID_ARG;
  const int G = Hq / Hkv;
  if (page_size < 16 || (page_size & (page_size - 1)) || !decode_supported(dtype, head_dim, G))
    return PA_ERR_UNSUPPORTED;  // pages: a power of two of at least 16 tokens
  c.G = G;
  if (T == 0 || S == 0) {
    c.empty = true;
    return PA_OK;
  }
  if (!q || !k_pool || !v_pool || !block_tables || !seq_lens || !query_start_loc || !out)
    return PA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
    return PA_ERR_INVALID_ARG;
  const size_t eb = (size_t)elem_bytes(dtype);
  const size_t qbytes = (size_t)T * Hq * head_dim * eb;
  const size_t pool_bytes = (size_t)num_pages * page_size * Hkv * head_dim * eb;
  if (overlap(out, qbytes, q, qbytes) || overlap(out, qbytes, k_pool, pool_bytes) ||
      overlap(out, qbytes, v_pool, pool_bytes))
    return PA_ERR_INVALID_ARG;
  c.wl = workspace_layout(S, T, Hq, head_dim, max_query_len, max_seq_len, page_size,
                          kv_split_tokens, dtype);
  const size_t need = c.wl.plan_bytes + c.wl.partial_bytes + c.wl.pf_bytes;
  if (need > 0 && (!workspace || workspace_bytes < need)) return PA_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0 && ((uintptr_t)workspace & 255u)) return PA_ERR_INVALID_ARG;
  if (c.wl.cap_dec > INT32_MAX / 2 || c.wl.cap_pf > INT32_MAX / 2 ||
      c.wl.part_slots > INT32_MAX / 2)
    return PA_ERR_INVALID_ARG;
  // decode rows are laid end to end on one int32 key axis (rows padded to at
  // most one partition)
  if (!c.wl.token_mode &&
      (long)S * ((long)max_seq_len + split_tokens(kv_split_tokens, page_size, false) + 16) >
          INT32_MAX)
    return PA_ERR_UNSUPPORTED;

  AttnArgs& a = c.a;
  const WsLayout& wl = c.wl;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.qsl = query_start_loc;
  a.out = out;
  a.plan = (int*)workspace;
  a.ws = (float*)((char*)workspace + wl.plan_bytes);
  a.cap_dec = (int32_t)wl.cap_dec;
  a.cap_pf = (int32_t)wl.cap_pf;
  a.S = S;
  a.T = T;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = head_dim;
  a.P = page_size;
  a.p_shift = 0;
  while ((1 << a.p_shift) < page_size) ++a.p_shift;
  a.num_pages = num_pages;
  a.max_blocks = max_blocks_per_seq;
  a.max_query_len = max_query_len;
  a.max_seq_len = max_seq_len;
  a.part_tokens = split_tokens(kv_split_tokens, page_size, wl.token_mode);
  a.part_min = split_min(page_size);
  a.part_max = split_max(page_size);
  a.max_parts = wl.max_parts;
  a.part_slots = (int32_t)wl.part_slots;
  a.dec_grid = wl.token_mode ? 0 : decode_grid(dtype, head_dim, G);
  a.scale_log2e = scale * kLog2e;
  a.pf_slots = wl.pf_slots;
  a.pf_ws = (float*)((char*)workspace + wl.plan_bytes + wl.partial_bytes);
  a.pf_workers = (!wl.token_mode && wl.cap_pf > 0) ? tick_grid(dtype, head_dim, G) : 1;
  // rows sharing a prefix are grouped on the bf16 matrix-core decode path,
  // with automatic partitions (a fixed partition size keeps a row's
  // partitions a function of the row alone) and a merge launch
  a.group_rows = (dtype == PA_BF16 && !wl.token_mode && a.part_tokens == 0 && a.max_parts > 1 &&
                  decode_supported(dtype, head_dim, G))
                     ? 1
                     : 0;
  // not a fused tick unless pa_tick_forward says so
  a.fused = 0;
  a.cos_sin = nullptr;
  a.max_pos = 0;

  return PA_OK;
}

// The plan kernel of a prepared call (seq mode only), on stream s.
pa_status_t attention_plan(const AttnCall& c, hipStream_t s) {
  if (c.empty || c.wl.token_mode) return PA_OK;
  return launch_plan(c.a, c.a.plan, c.a.cap_dec, c.a.cap_pf, kPrefillRows / c.G, s) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

// The attention kernels of a prepared call after its plan, on stream s.
pa_status_t attention_run(const AttnCall& c, hipStream_t s) {
  if (c.empty) return PA_OK;
  const AttnArgs& a = c.a;
  hipError_t e;
  if (!c.wl.token_mode && a.cap_pf > 0 && tick_supported(c.dtype, a.D)) {
    // a tick that may hold prefill chunks: decode and prefill share one grid
    e = launch_tick(c.dtype, a, s);
    if (e != hipSuccess) return PA_ERR_HIP;
    return launch_tick_reduce(a, s) == hipSuccess ? PA_OK : PA_ERR_HIP;
  }
  e = launch_decode(c.dtype, a, c.wl.token_mode, s);
  if (e != hipSuccess) return PA_ERR_HIP;
  if (a.max_parts > 1) {
    e = launch_split_reduce(c.dtype, a, c.wl.token_mode, s);
    if (e != hipSuccess) return PA_ERR_HIP;
  }
  return PA_OK;
}

// Validation of an attention call's metadata (and, for a tick, of its rows'
// positions and pages); PA_OK when validation is off.
pa_status_t validate_call(const int32_t* block_tables, const int32_t* seq_lens,
                          const int32_t* query_start_loc, const int32_t* positions, int S, int T,
                          int P, int num_pages, int max_blocks, int max_query_len,
                          int max_seq_len, int max_pos, bool rope, hipStream_t s) {
  g_vmsg[0] = '\0';
  if (!validating() || S == 0 || T == 0) return PA_OK;
  HostMeta m;
  if (fetch(m.qsl, query_start_loc, (size_t)S + 1, s) != PA_OK ||
      fetch(m.seq_lens, seq_lens, (size_t)S, s) != PA_OK ||
      fetch(m.bt, block_tables, (size_t)S * max_blocks, s) != PA_OK ||
      (positions && fetch(m.pos, positions, (size_t)T, s) != PA_OK) ||
      hipStreamSynchronize(s) != hipSuccess)
    return PA_ERR_HIP;
  pa_status_t st = check_qsl(m, S, T);
  if (st == PA_OK) st = check_seqs(m, S, P, num_pages, max_blocks, max_query_len, max_seq_len);
  if (st == PA_OK && positions) st = check_tick_rows(m, S, P, max_blocks, max_pos, rope);
  return st;
}

}  // namespace

pa_status_t pa_paged_attention_varlen(const void* q, const void* k_pool, const void* v_pool,
                                      const int32_t* block_tables, const int32_t* seq_lens,
                                      const int32_t* query_start_loc, void* out, int32_t S,
                                      int32_t T, int32_t Hq, int32_t Hkv, int32_t head_dim,
                                      int32_t page_size, int32_t num_pages,
                                      int32_t max_blocks_per_seq, int32_t max_query_len,
                                      int32_t max_seq_len, float scale, int32_t kv_split_tokens,
                                      pa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  AttnCall c;
  pa_status_t st = attention_setup(q, k_pool, v_pool, block_tables, seq_lens, query_start_loc,
                                   out, S, T, Hq, Hkv, head_dim, page_size, num_pages,
                                   max_blocks_per_seq, max_query_len, max_seq_len, scale,
                                   kv_split_tokens, dtype, workspace, workspace_bytes, c);
  if (st != PA_OK || c.empty) return st;
  const hipStream_t s = (hipStream_t)stream;
  st = validate_call(block_tables, seq_lens, query_start_loc, nullptr, S, T, page_size,
                     num_pages, max_blocks_per_seq, max_query_len, max_seq_len, 0, false, s);
  if (st != PA_OK) return st;
  st = attention_plan(c, s);
  return st != PA_OK ? st : attention_run(c, s);
}

namespace {

// pa_tick_forward's checks and, when `enqueue`, its launches.
pa_status_t tick_forward_impl(void* q, void* k, const void* v, const int32_t* positions,
                              const int32_t* block_tables, const int32_t* seq_lens,
                              const int32_t* query_start_loc, const float* cos_sin, void* k_pool,
                              void* v_pool, void* out, int32_t* slot_mapping, int32_t S,
                              int32_t T, int32_t Hq, int32_t Hkv, int32_t head_dim,
                              int32_t page_size, int32_t num_pages, int32_t max_blocks_per_seq,
                              int32_t max_query_len, int32_t max_seq_len, int32_t max_pos,
                              float scale, int32_t kv_split_tokens, pa_dtype_t dtype,
                              void* workspace, size_t workspace_bytes, void* stream,
                              bool enqueue) {
  // every check of the three calls before anything is enqueued
  if (T > 0 && !q) return PA_ERR_INVALID_ARG;
  pa_status_t st = slot_mapping_check(block_tables, query_start_loc, positions, slot_mapping, S,
                                      T, max_blocks_per_seq, page_size, num_pages);
  if (st != PA_OK) return st;
  st = rope_check(q, k, v, positions, slot_mapping, cos_sin, k_pool, v_pool, T, Hq, Hkv,
                  head_dim, page_size, num_pages, max_pos, dtype);
  if (st != PA_OK) return st;
  AttnCall c{};
  st = attention_setup(q, k_pool, v_pool, block_tables, seq_lens, query_start_loc, out, S, T, Hq,
                       Hkv, head_dim, page_size, num_pages, max_blocks_per_seq, max_query_len,
                       max_seq_len, scale, kv_split_tokens, dtype, workspace, workspace_bytes, c);
  if (st != PA_OK || T == 0 || !enqueue) return st;
  st = validate_call(block_tables, seq_lens, query_start_loc, positions, S, T, page_size,
                     num_pages, max_blocks_per_seq, max_query_len, max_seq_len, max_pos,
                     cos_sin != nullptr, (hipStream_t)stream);
  if (st != PA_OK) return st;

  // One launch for the slot mapping, the page write and (seq mode) the plan,
  // which reads only query_start_loc and seq_lens; then the attention kernels.
  // bf16 ticks are fused: the first launch writes every token's rotated K and
  // its V into their slots and each decode row's rotated query into its output
  // row (where the decode kernel reads it), the prefill items rotate their
  // query rows where they read them, and q and k are left as given.
  const bool plan = !c.empty && !c.wl.token_mode;
  const bool fused = plan && dtype == PA_BF16;
  if (fused) {
    c.a.fused = 1;
    c.a.cos_sin = cos_sin;
    c.a.max_pos = max_pos;
  }
  if (launch_tick_prep(dtype, q, k, v, positions, block_tables, query_start_loc, slot_mapping,
                       cos_sin, k_pool, v_pool, S, T, Hq, Hkv, head_dim, page_size, num_pages,
                       max_blocks_per_seq, max_pos, plan ? &c.a : nullptr, c.a.cap_dec,
                       c.a.cap_pf, kPrefillRows / c.G, fused, (hipStream_t)stream) != hipSuccess)
    return PA_ERR_HIP;
  return attention_run(c, (hipStream_t)stream);
}

}  // namespace

pa_status_t pa_tick_forward(void* q, void* k, const void* v, const int32_t* positions,
                            const int32_t* block_tables, const int32_t* seq_lens,
                            const int32_t* query_start_loc, const float* cos_sin, void* k_pool,
                            void* v_pool, void* out, int32_t* slot_mapping, int32_t S, int32_t T,
                            int32_t Hq, int32_t Hkv, int32_t head_dim, int32_t page_size,
                            int32_t num_pages, int32_t max_blocks_per_seq,
                            int32_t max_query_len, int32_t max_seq_len, int32_t max_pos,
                            float scale, int32_t kv_split_tokens, pa_dtype_t dtype,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return tick_forward_impl(q, k, v, positions, block_tables, seq_lens, query_start_loc, cos_sin,
                           k_pool, v_pool, out, slot_mapping, S, T, Hq, Hkv, head_dim, page_size,
                           num_pages, max_blocks_per_seq, max_query_len, max_seq_len, max_pos,
                           scale, kv_split_tokens, dtype, workspace, workspace_bytes, stream,
                           true);
}

pa_status_t pa_tick_forward_noalloc(void* q, void* k, const void* v, const int32_t* positions,
                                    const int32_t* block_tables, const int32_t* seq_lens,
                                    const int32_t* query_start_loc, const float* cos_sin,
                                    void* k_pool, void* v_pool, void* out,
                                    int32_t* slot_mapping, int32_t S, int32_t T, int32_t Hq,
                                    int32_t Hkv, int32_t head_dim, int32_t page_size,
                                    int32_t num_pages, int32_t max_blocks_per_seq,
                                    int32_t max_query_len, int32_t max_seq_len, int32_t max_pos,
                                    float scale, int32_t kv_split_tokens, pa_dtype_t dtype,
                                    void* stream) {
  g_vmsg[0] = '\0';
  // Every check first, with a stand-in scratch address (aligned, never
  // dereferenced): a bad or oversized call returns before any HIP call.
  void* const stand_in = reinterpret_cast<void*>((uintptr_t)kScratchAlign);
  pa_status_t st = tick_forward_impl(q, k, v, positions, block_tables, seq_lens,
                                     query_start_loc, cos_sin, k_pool, v_pool, out, slot_mapping,
                                     S, T, Hq, Hkv, head_dim, page_size, num_pages,
                                     max_blocks_per_seq, max_query_len, max_seq_len, max_pos,
                                     scale, kv_split_tokens, dtype, stand_in, kScratchBytes,
                                     stream, false);
  if (st == PA_ERR_WORKSPACE_TOO_SMALL) {
    const size_t need = workspace_bytes_for(S, T, Hq, head_dim, max_query_len, max_seq_len,
                                            page_size, kv_split_tokens, dtype);
    vfail("the tick needs %zu bytes of scratch; the fixed scratch holds %zu", need,
          kScratchBytes);
    return st;
  }
  if (st != PA_OK || T == 0) return st;
  void* scratch_ptr = nullptr;
  st = scratch_address(&scratch_ptr);
  if (st != PA_OK) return st;
  return tick_forward_impl(q, k, v, positions, block_tables, seq_lens, query_start_loc, cos_sin,
                           k_pool, v_pool, out, slot_mapping, S, T, Hq, Hkv, head_dim, page_size,
                           num_pages, max_blocks_per_seq, max_query_len, max_seq_len, max_pos,
                           scale, kv_split_tokens, dtype, scratch_ptr, kScratchBytes, stream,
                           true);
}

pa_status_t pa_profile_start(int32_t capacity) {
  if (capacity < 1 || capacity > (1 << 20)) return PA_ERR_INVALID_ARG;
  g_prof_on = false;
  destroy_events();
  g_recs.resize(capacity);
  for (int i = 0; i < capacity; ++i) {
    if (hipEventCreate(&g_recs[i].start) != hipSuccess ||
        hipEventCreate(&g_recs[i].stop) != hipSuccess) {
      g_recs.resize(i);
      return PA_ERR_HIP;
    }
    g_recs[i].name = "";
  }
  g_prof_n = 0;
  g_prof_on = true;
  return PA_OK;
}

pa_status_t pa_profile_stop(int32_t* num_records) {
  g_prof_on = false;
  if (num_records) *num_records = g_prof_n;
  if (g_prof_n > 0 && hipEventSynchronize(g_recs[g_prof_n - 1].stop) != hipSuccess)
    return PA_ERR_HIP;
  return PA_OK;
}

pa_status_t pa_profile_get(int32_t index, char* name, int32_t name_len, float* milliseconds) {
  if (index < 0 || index >= g_prof_n) return PA_ERR_INVALID_ARG;
  if (name && name_len > 0) {
    strncpy(name, g_recs[index].name, (size_t)name_len - 1);
    name[name_len - 1] = '\0';
  }
  if (milliseconds) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_recs[index].start, g_recs[index].stop) != hipSuccess)
      return PA_ERR_HIP;
    *milliseconds = ms;
  }
  return PA_OK;
}

pa_status_t pa_profile_reset(void) {
  g_prof_on = false;
  destroy_events();
  return PA_OK;
}

}  // extern "C"
#pragma GCC visibility pop
