// K4 device code: prefill-chunk paged attention on bf16 matrix cores (gfx950
// MFMA). Shared by the prefill kernel and the fused tick kernel.
//
// A chunk of L rows attends every earlier key in full and itself causally
// (llm-serving-engine README, "_step_prefill": write K/V at the chunk start,
// gather the prior K/V, apply the rectangular causal mask). With L rows, G
// query heads per KV head and n keys the work is about 4*D*G*L*n flops over
// 2*D*n*2 bytes of K/V per KV head: a dense contraction, so it runs on MFMA.
//
// Workgroup = 4 waves = 64 query rows of one KV head: row r is token r / G
// of the tile and query head r % G, so each K/V tile is read once for the
// whole GQA group. Each wave owns one 16-row block.
//
// Per 64-key tile (K row-major and V transposed, staged in LDS):
//   S^T[key, row] = K[key, :] . Q[row, :]        v_mfma_f32_16x16x32_bf16, A = K, B = Q^T
//   online softmax on S^T columns (one query row per lane column)
//   O^T[dim, row] += V^T[dim, key] . P^T[key, row]   A = V^T (LDS), B = P^T (registers)
// Computing the transposed products keeps a query row's scores, running max,
// running sum and output column in the same lanes, so no transposes or
// shuffles are needed between the two products: the S^T accumulator of a lane
// (4 keys of each 16-key block, one query row) is exactly the P^T operand the
// second MFMA needs, once the contraction's key order is defined to match.
// The row max and row sum combine the four lanes of a row with gfx950's
// v_permlane16_swap / v_permlane32_swap (VALU, no LDS round trip).
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {



constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * 64;
constexpr int kRowsPerWave = 16;
constexpr int kRowsPerWg = kPfWaves * kRowsPerWave;
static_assert(kRowsPerWg == kPrefillRows, "plan and kernel disagree on the tile height");
constexpr int kBN = 64;                                // keys per tile
constexpr int kKB = kBN / 16;                          // 16-key blocks per tile

__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Max / sum over lanes {l, l^16, l^32, l^48}. Each swap returns, for every
// lane, its own value and its partner's (in some order), so symmetric
// combinations need no selects.
__device__ __forceinline__ float max4rows(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum4rows(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Global -> register staging of one tile: K as 16-byte row chunks, V as pairs
// of keys (so V^T is written two keys per 32-bit LDS word).
template <int D>
struct TileRegs {
  static constexpr int C16 = D / 8;                                    // 16-byte chunks per row
  static constexpr int KCH = kBN * C16 / kPfThreads;                   // K chunks per thread
  static constexpr int VCH = (kBN / 2) * C16 / kPfThreads;             // V pair tasks per thread
  static_assert(KCH * kPfThreads == kBN * C16 && VCH * kPfThreads == (kBN / 2) * C16,
                "tile chunks divide evenly over the threads");
  uint4 k[KCH];
  uint4 va[VCH], vb[VCH];
};

// Component-wise select (a select of whole structs can become a select of
// addresses, which forces the registers into scratch memory).
__device__ __forceinline__ uint4 keep_if(const uint4& v, bool ok) {
  return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int w) {
  return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
}

// Byte offsets of the pages holding the four 16-key blocks of the tile at kb0
// (pages hold a power of two >= 16 keys, so a 16-aligned block never crosses a
// page). Page ids come from the LDS copy of the sequence's page table (the
// first kItemPages entries) or, past it, from global memory.
constexpr int kItemPages = 2048;

struct TilePages {
  size_t off[kKB];
};

__device__ __forceinline__ TilePages tile_pages(const int* s_pt, const int* bt_row, int num_pages,
                                                int p_shift, size_t page_bytes, int kb0,
                                                int kmax) {
  TilePages tp;
#pragma unroll
  for (int q = 0; q < kKB; ++q) {
    const int b = min(kb0 + 16 * q, kmax - 1) >> p_shift;  // wave-uniform
    const int page = b < kItemPages ? s_pt[b] : clampi(bt_row[b], 0, num_pages - 1);
    tp.off[q] = (size_t)page * page_bytes;
  }
  return tp;
}

__device__ __forceinline__ size_t pick(const TilePages& tp, int q) {
  return q == 0 ? tp.off[0] : (q == 1 ? tp.off[1] : (q == 2 ? tp.off[2] : tp.off[3]));
}

// Issue the global loads of one tile. Every lane always issues the same loads
// (keys past kmax re-read key kmax - 1 and are zeroed at the store), so the
// count of outstanding loads never depends on the data.
template <int D>
__device__ __forceinline__ void tile_load(TileRegs<D>& r, const char* kpool, const char* vpool,
                                          const TilePages& tp, int rmask, uint32_t slot_stride,
                                          int kb0, int kmax, int tid) {
  constexpr int C16 = TileRegs<D>::C16;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::KCH; ++i) {
    const int c = tid + i * kPfThreads;
    const int key = c / C16, d8 = c % C16;
    const int j = min(kb0 + key, kmax - 1);
    const uint32_t off = (uint32_t)(j & rmask) * slot_stride + d8 * 16;
    r.k[i] = *reinterpret_cast<const uint4*>(kpool + pick(tp, key >> 4) + off);
  }
#pragma unroll
  for (int i = 0; i < TileRegs<D>::VCH; ++i) {
    const int c = tid + i * kPfThreads;
    const int kp = c % (kBN / 2), d8 = c / (kBN / 2);
    const int ja = min(kb0 + 2 * kp, kmax - 1);
    const int jb = min(kb0 + 2 * kp + 1, kmax - 1);
    const char* base = vpool + pick(tp, kp >> 3);  // keys 2kp and 2kp+1 share a 16-key block
    r.va[i] = *reinterpret_cast<const uint4*>(base + (uint32_t)(ja & rmask) * slot_stride + d8 * 16);
    r.vb[i] = *reinterpret_cast<const uint4*>(base + (uint32_t)(jb & rmask) * slot_stride + d8 * 16);
  }
}

template <int D, int KSTR, int VSTR>
__device__ __forceinline__ void tile_store(const TileRegs<D>& r, uint16_t* s_k, uint16_t* s_vt,
                                           int kb0, int kmax, int tid) {
  constexpr int C16 = TileRegs<D>::C16;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::KCH; ++i) {
    const int c = tid + i * kPfThreads;
    const int key = c / C16, d8 = c % C16;
    *reinterpret_cast<uint4*>(&s_k[key * KSTR + d8 * 8]) = keep_if(r.k[i], kb0 + key < kmax);
  }
  uint32_t* vt = reinterpret_cast<uint32_t*>(s_vt);
#pragma unroll
  for (int i = 0; i < TileRegs<D>::VCH; ++i) {
    const int c = tid + i * kPfThreads;
    const int kp = c % (kBN / 2), d8 = c / (kBN / 2);
    const uint4 xa = keep_if(r.va[i], kb0 + 2 * kp < kmax);
    const uint4 xb = keep_if(r.vb[i], kb0 + 2 * kp + 1 < kmax);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t wa = word_of(xa, w), wb = word_of(xb, w);
      const int d = d8 * 8 + 2 * w;
      vt[(d * VSTR) / 2 + kp] = (wa & 0xFFFFu) | (wb << 16);
      vt[((d + 1) * VSTR) / 2 + kp] = (wa >> 16) | (wb & 0xFFFF0000u);
    }
  }
}

// One 64-key tile: S^T = K Q^T, online softmax per query row, O^T += V^T P^T.
template <int D, int KSTR, int VSTR>
__device__ __forceinline__ void tile_compute(const uint16_t* sk, const uint16_t* svt, int kb0,
                                             const uint4 (&qop)[D / 32], int limit, bool masked,
                                             float sl2e, int col, int grp, float& m_run,
                                             float& l_run, f32x4_t (&acc_o)[D / 16]) {
  constexpr int DSTEPS = D / 32;
  constexpr int DBLK = D / 16;

  // ---- S^T = K Q^T for this wave's 16 rows ----
  f32x4_t st[kKB];
#pragma unroll
  for (int kb = 0; kb < kKB; ++kb) st[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ds = 0; ds < DSTEPS; ++ds) {
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
      const uint4 kop =
          *reinterpret_cast<const uint4*>(&sk[(kb * 16 + col) * KSTR + ds * 32 + grp * 8]);
      st[kb] = mfma16x16x32(kop, qop[ds], st[kb]);
    }
  }

  // ---- online softmax of this lane's query row ----
  // The running max m is in log2 units (score * scale * log2 e); a weight is
  // exp2(s * sl2e - m): one fma and one exp2. Only tiles reaching past some
  // row's last visible key (the diagonal and the ragged end) are masked;
  // `masked` is wave-uniform.
  float sv[4 * kKB];
#pragma unroll
  for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[kb * 4 + i] = st[kb][i];
  if (masked) {
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (kb0 + kb * 16 + grp * 4 + i > limit) sv[kb * 4 + i] = -INFINITY;
  }
  float tmax = sv[0];
#pragma unroll
  for (int k = 1; k < 4 * kKB; ++k) tmax = fmaxf(tmax, sv[k]);
  tmax = max4rows(tmax) * sl2e;
  // rescale only when some row's running max grows (wave-uniform test)
  if (__any(tmax > m_run)) {
    const float mn = fmaxf(m_run, tmax);
    const float corr = fast_exp2(m_run - mn);
    m_run = mn;
    l_run *= corr;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      acc_o[db][0] *= corr;
      acc_o[db][1] *= corr;
      acc_o[db][2] *= corr;
      acc_o[db][3] *= corr;
    }
  }
  const float neg_m = -m_run;
  uint32_t pw[2 * kKB];
#pragma unroll
  for (int k = 0; k < 2 * kKB; ++k) {
    const float p0 = fast_exp2(fmaf(sv[2 * k], sl2e, neg_m));
    const float p1 = fast_exp2(fmaf(sv[2 * k + 1], sl2e, neg_m));
    l_run += p0 + p1;
    const f32x2_t pf = {p0, p1};  // rounded once to bf16 (round to nearest even)
    pw[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pf, bf16x2e_t));
  }

  // ---- O^T += V^T P^T, one 32-key k-step per pair of 16-key blocks ----
#pragma unroll
  for (int ks = 0; ks < kKB / 2; ++ks) {
    const uint4 pop = make_uint4(pw[4 * ks], pw[4 * ks + 1], pw[4 * ks + 2], pw[4 * ks + 3]);
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const int d = db * 16 + col;
      const uint2 lo = *reinterpret_cast<const uint2*>(&svt[d * VSTR + ks * 32 + grp * 4]);
      const uint2 hi = *reinterpret_cast<const uint2*>(&svt[d * VSTR + ks * 32 + 16 + grp * 4]);
      acc_o[db] = mfma16x16x32(make_uint4(lo.x, lo.y, hi.x, hi.y), pop, acc_o[db]);
    }
  }
}

// LDS of one prefill workgroup: double-buffered K (row-major) and V^T tiles
// (the next tile is written while the current one is read) and the
// sequence's page table.
template <int D>
struct PfSmem {
  static constexpr int KSTR = D + 8;    // LDS row stride of K (elements), 16-byte pad
  static constexpr int VSTR = kBN + 4;  // LDS row stride of V^T (elements), 8-byte pad
  __attribute__((aligned(16))) uint16_t k[2][kBN * KSTR];
  __attribute__((aligned(16))) uint16_t vt[2][D * VSTR];
  int pt[kItemPages];
};

// One prefill work item: row tile mt (TM tokens x G query heads = 64 rows) of
// sequence s against KV head kvh, run by the whole workgroup (4 waves).
template <int D, int G>
__device__ __forceinline__ void prefill_item(const AttnArgs& a, PfSmem<D>& sm, int s, int mt,
                                             int kvh) {
  constexpr int TM = kRowsPerWg / G;    // tokens per workgroup
  constexpr int DSTEPS = D / 32;        // k-steps of the QK^T product
  constexpr int DBLK = D / 16;          // 16-dim output blocks
  constexpr int KSTR = PfSmem<D>::KSTR;
  constexpr int VSTR = PfSmem<D>::VSTR;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int col = lane & 15;            // query row within the wave's 16-row block
  const int grp = lane >> 4;            // 0..3
  const size_t row_bytes = (size_t)D * 2;
  const int Hq = a.Hq;
  const float sl2e = a.scale_log2e;
  const size_t slot_stride = (size_t)a.Hkv * row_bytes;
  const uint32_t slot_stride32 = (uint32_t)slot_stride;  // offsets within a page fit 32 bits
  const int p_shift = a.p_shift;
  const int rmask = (1 << p_shift) - 1;
  const size_t page_bytes = slot_stride << p_shift;
  const int q0 = a.qsl[s];
  const int L = a.qsl[s + 1] - q0;
  const int i0 = mt * TM;
  int n = a.seq_lens[s];
  n = min(n, a.max_blocks * a.P);
  if (L <= 1 || i0 >= L || q0 < 0 || q0 + L > a.T || n < L) return;  // uniform per item
  const int i1 = min(L, i0 + TM);
  const int kmax = n - L + i1;          // keys visible to the tile's last row
  const int ntiles = (kmax + kBN - 1) / kBN;
  const int last_key = n - L;           // row i sees keys <= last_key + i
  // the smallest key limit among this wave's rows: tiles ending at or below it
  // need no mask (wave-uniform)
  const int min_limit = last_key + i0 + (wave * kRowsPerWave) / G;

  // Q^T operand: this lane's row, 8 dims per k-step.
  const int rr = wave * kRowsPerWave + col;
  const int tok = i0 + rr / G;
  const int head = kvh * G + rr % G;
  const bool row_ok = tok < i1;
  const int limit = min(last_key + tok, n - 1);
  uint4 qop[DSTEPS];
  {
    const int tq = row_ok ? tok : i1 - 1;  // rows past the chunk read a valid row, zeroed
    const char* qrow = (const char*)a.q + ((size_t)(q0 + tq) * Hq + head) * row_bytes;
#pragma unroll
    for (int ds = 0; ds < DSTEPS; ++ds) {
      const uint4 x = *reinterpret_cast<const uint4*>(qrow + (ds * 32 + grp * 8) * 2);
      qop[ds] = keep_if(x, row_ok);
    }
  }

  f32x4_t acc_o[DBLK];
  float m_run = kNegBig, l_run = 0.f;
#pragma unroll
  for (int db = 0; db < DBLK; ++db) acc_o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int* bt_row = a.block_tables + (size_t)s * a.max_blocks;
  const char* kpool = (const char*)a.k_pool + (size_t)kvh * row_bytes;
  const char* vpool = (const char*)a.v_pool + (size_t)kvh * row_bytes;

  const int npg = min((kmax + (1 << p_shift) - 1) >> p_shift, kItemPages);
  for (int i = tid; i < npg; i += kPfThreads) sm.pt[i] = clampi(bt_row[i], 0, a.num_pages - 1);
  __syncthreads();

  // Two register tiles alternate, each loaded two tiles ahead of its use, so
  // a tile's global loads have two tiles of compute to arrive.
  TileRegs<D> rA, rB;
  {
    const TilePages pA = tile_pages(sm.pt, bt_row, a.num_pages, p_shift, page_bytes, 0, kmax);
    tile_load<D>(rA, kpool, vpool, pA, rmask, slot_stride32, 0, kmax, tid);
    const TilePages pB = tile_pages(sm.pt, bt_row, a.num_pages, p_shift, page_bytes, kBN, kmax);
    tile_load<D>(rB, kpool, vpool, pB, rmask, slot_stride32, kBN, kmax, tid);
  }
  for (int kt = 0; kt < ntiles; kt += 2) {
    tile_store<D, KSTR, VSTR>(rA, sm.k[0], sm.vt[0], kt * kBN, kmax, tid);
    {
      const TilePages p2 =
          tile_pages(sm.pt, bt_row, a.num_pages, p_shift, page_bytes, (kt + 2) * kBN, kmax);
      tile_load<D>(rA, kpool, vpool, p2, rmask, slot_stride32, (kt + 2) * kBN, kmax, tid);
    }
    __syncthreads();
    tile_compute<D, KSTR, VSTR>(sm.k[0], sm.vt[0], kt * kBN, qop, limit,
                                kt * kBN + kBN - 1 > min_limit, sl2e, col, grp, m_run, l_run,
                                acc_o);
    if (kt + 1 >= ntiles) break;
    tile_store<D, KSTR, VSTR>(rB, sm.k[1], sm.vt[1], (kt + 1) * kBN, kmax, tid);
    {
      const TilePages p3 =
          tile_pages(sm.pt, bt_row, a.num_pages, p_shift, page_bytes, (kt + 3) * kBN, kmax);
      tile_load<D>(rB, kpool, vpool, p3, rmask, slot_stride32, (kt + 3) * kBN, kmax, tid);
    }
    __syncthreads();
    tile_compute<D, KSTR, VSTR>(sm.k[1], sm.vt[1], (kt + 1) * kBN, qop, limit,
                                (kt + 1) * kBN + kBN - 1 > min_limit, sl2e, col, grp, m_run,
                                l_run, acc_o);
  }
  __syncthreads();  // the next item's first store reuses buffer 0

  // ---- normalise and store ----
  const float lt = sum4rows(l_run);
  if (row_ok) {
    const float inv = 1.f / lt;
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + ((size_t)(q0 + tok) * Hq + head) * D;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const f32x2_t lo = {acc_o[db][0] * inv, acc_o[db][1] * inv};
      const f32x2_t hi = {acc_o[db][2] * inv, acc_o[db][3] * inv};
      const uint2 wv = make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2e_t)),
                                  __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2e_t)));
      *reinterpret_cast<uint2*>(orow + db * 16 + grp * 4) = wv;
    }
  }
}

}  // namespace pa
