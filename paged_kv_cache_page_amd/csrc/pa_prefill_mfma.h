// K4 device code: prefill-chunk paged attention on bf16 matrix cores (gfx950
// MFMA). Shared by the prefill kernel and the fused tick kernel.
//
// A chunk of L rows attends every earlier key in full and itself causally
// (llm-serving-engine README, "_step_prefill": write K/V at the chunk start,
// gather the prior K/V, apply the rectangular causal mask). With L rows, G
// query heads per KV head and n keys the work is about 4*D*G*L*n flops over
// 2*D*n*2 bytes of K/V per KV head: a dense contraction, so it runs on MFMA.
//
// Work item = 128 query rows of one KV head, run by a workgroup of 4 waves:
// row r is token r / G of the tile and query head r % G, so each K/V tile is
// read once for the whole GQA group. Wave w owns rows 32w .. 32w + 31 as two
// 16-row blocks; every K or V operand it reads from LDS feeds both blocks'
// MFMAs, which halves the LDS bytes per flop against one block per wave.
//
// Per 64-key tile:
//   S^T[key, row] = K[key, :] . Q[row, :]        v_mfma_f32_16x16x32_bf16, A = K (LDS), B = Q^T
//   online softmax on S^T columns (one query row per lane column)
//   O^T[dim, row] += V^T[dim, key] . P^T[key, row]   A = V^T (LDS, transposing read), B = P^T
// Computing the transposed products keeps a query row's scores, running max,
// running sum and output column in the same lanes: a lane's S^T accumulator
// (4 keys of each 16-key block, one query row) is its P^T operand once the
// contraction's key order is defined to match, and the row max combines the
// four lanes of a row with v_permlane16_swap / v_permlane32_swap. The row sum
// is one more product per k-step, of the weights with a block of ones.
//
// K and V tiles go from global memory straight into LDS (global_load_lds,
// 16 bytes per lane, no registers), two stages deep: tile t + 1 is in flight
// while tile t is computed. In LDS a tile is a sequence of 16-byte units; key
// row j, 16-byte chunk c (of CPR = D / 8) sits at unit
//   K: (j / 16) * 16 CPR + c * 16 + j % 16
//   V: (j / 8) * 8 CPR + (c / 2) * 16 + (j % 8) * 2 + c % 2
// so that an MFMA operand read covers whole 256-byte runs (no bank conflict
// whether the LDS serves 8, 16 or 32 lanes a cycle) and its address is a
// per-lane constant plus an offset known at compile time:
//   K (ds_read_b128): lane l reads key 16 kb + l % 16, chunk 4 ds + l / 16,
//     unit 16 CPR kb + 64 ds + l;
//   V (ds_read_b64_tr_b16): lane s of 16-lane group g reads 8 bytes of key
//     32 ks + 16 r + 4 g + s / 4 at dims 16 db + 4 (s % 4).
// ds_read_b64_tr_b16 hands lane i of a 16-lane group element k = the i % 4-th
// 16-bit value at the address of lane 4k + i / 4 of its group, so lane i gets
// the column dim0 + i of keys key0 .. key0 + 3: the transposed operand.
// One load instruction fills 64 consecutive units: 16 keys x 64 bytes (K) or
// 8 keys x 128 bytes (V), all of one 16-key block, hence of one page.
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

// The load helpers below name M0 in their clobber lists (see lds_dma16).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

namespace pa {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * 64;
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerWg = kPfWaves * kRowsPerWave;
static_assert(kRowsPerWg == kPrefillRows, "plan and kernel disagree on the tile height");
constexpr int kBN = 64;         // keys per tile
constexpr int kKB = kBN / 16;   // 16-key blocks per tile
constexpr int kPfStages = 2;    // K/V tiles in LDS: kPfStages - 1 in flight while one computes
static_assert(kKB % 2 == 0, "P.V contracts 32 keys per step");
static_assert(kBN == kPrefillTileKeys, "plan and kernel disagree on the tile length");
// Page ids of an item's sequence kept in LDS; pages past these are read from
// the block table in global memory.
constexpr int kItemPages = 512;

typedef short v4i16_t __attribute__((ext_vector_type(4)));

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

__device__ __forceinline__ uint4 keep_if(const uint4& v, bool ok) {
  return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}

template <int D>
struct PfShape {
  static constexpr int CPR = D / 8;                  // 16-byte chunks per key row
  static constexpr int TILE_BYTES = kBN * D * 2;     // one matrix of one tile
  // global_load_lds instructions per wave per matrix per tile (one writes 1 KB)
  static constexpr int DMA_PER_WAVE = TILE_BYTES / 1024 / kPfWaves;
  static constexpr int DMA_PER_TILE = 2 * DMA_PER_WAVE;  // K and V, per wave
  static_assert(DMA_PER_WAVE >= 1 && DMA_PER_WAVE * kPfWaves * 1024 == TILE_BYTES,
                "a tile is whole DMA instructions per wave");
  static_assert(DMA_PER_TILE * (kPfStages - 2) <= 63, "vmcnt immediate");
};

// LDS of one prefill workgroup: two stages of K and V tiles and the
// sequence's first page ids.
template <int D>
struct PfSmem {
  __attribute__((aligned(1024))) uint16_t k[kPfStages][kBN * D];
  __attribute__((aligned(1024))) uint16_t v[kPfStages][kBN * D];
  int pt[kItemPages];
};

// Wait until at most N of this wave's vector memory operations are
// outstanding (lgkm and export counters left alone). gfx9 s_waitcnt fields:
// vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] in [15:14].
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// wait_vmcnt<tiles * per_tile> for a run-time tiles in [0, kPfStages - 2]
// (the tiles whose loads may stay in flight while one is computed).
template <int PER_TILE, int T = kPfStages - 2>
__device__ __forceinline__ void wait_tiles(int tiles) {
  if constexpr (T == 0) {
    wait_vmcnt<0>();
  } else {
    if (tiles >= T) wait_vmcnt<T * PER_TILE>();
    else wait_tiles<PER_TILE, T - 1>(tiles);
  }
}

// One 16-byte-per-lane load from global memory into LDS: lane j's 16 bytes
// land at LDS byte lds + 16 j (lds wave-uniform, in M0). Written as inline
// assembly so that the compiler's wait insertion does not treat every later
// LDS read as depending on it (it would wait for all such loads, the next
// tile's included); the kernel waits for these loads itself (wait_vmcnt) and
// the "memory" clobber keeps other memory accesses on their side of it.
// M0 is reserved by the compiler, which sets it right before each of its own
// uses and keeps no value in it across other code; hence the clobber.
// The LDS address is wave-uniform by construction; reading it from the first
// lane puts it in a scalar register for the compiler.
__device__ __forceinline__ void lds_dma16(const void* gaddr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gaddr),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Workgroup barrier without the memory fence of __syncthreads(): a
// workgroup-scope release would wait for every outstanding load into LDS,
// including the next tile's, which must stay in flight. Callers wait for the
// global loads they need (wait_vmcnt) first; the wave's own LDS accesses are
// drained here (lgkmcnt 0; vmcnt and expcnt fields at their maxima), and the
// empty asm keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Page of the 16-key block starting at key kb (wave-uniform; a page holds a
// power of two >= 16 keys, so a 16-aligned block never crosses one). Keys
// past kmax stand for key kmax - 1. Page ids come from the LDS copy of the
// sequence's page table or, past it, from the block table.
__device__ __forceinline__ uint32_t block_page(const int* s_pt, const int* bt_row, int num_pages,
                                               int p_shift, int kb, int kmax) {
  const int b = min(kb, kmax - 1) >> p_shift;
  const int pg = b < kItemPages ? s_pt[b] : clampi(bt_row[b], 0, num_pages - 1);
  return (uint32_t)__builtin_amdgcn_readfirstlane(pg);  // uniform: keep it in a scalar register
}

// Loads of a full tile (every key < kmax): the address of instruction q is a
// wave-uniform base (page, key block, chunk group) in SGPRs plus a per-lane
// 32-bit offset that is the same for every tile (lk / lv). The last tile of an
// item, which may reach past kmax, takes tile_dma_partial instead.
__device__ __forceinline__ void lds_dma16_s(const char* sbase, uint32_t voff, uint32_t lds) {
  // the base and the LDS address are wave-uniform by construction; the reads
  // of the first lane put them in scalar registers for the compiler
  // (readfirstlane returns a signed int: each half goes through uint32_t so
  // that the low half is not sign-extended into the high one)
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint64_t bs = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(bs),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

// Per-lane offsets of the full-tile loads within a 16-key block (K) or an
// 8-key group (V): key row and chunk of lane j of an instruction.
__device__ __forceinline__ uint32_t dma_lane_k(int j, size_t slot_stride) {
  return (uint32_t)((j % 16) * slot_stride + 16 * (j / 16));
}
__device__ __forceinline__ uint32_t dma_lane_v(int j, size_t slot_stride) {
  return (uint32_t)(((j % 16) / 2) * slot_stride + 16 * (2 * (j / 16) + j % 2));
}

template <int D>
__device__ __forceinline__ void tile_dma_full(uint32_t sk, uint32_t sv, const char* kpool,
                                              const char* vpool, const int* s_pt,
                                              const int* bt_row, int num_pages, int p_shift,
                                              size_t slot_stride, int kb0, int kmax, int wave,
                                              uint32_t lk, uint32_t lv) {
  typedef PfShape<D> SH;
  constexpr int CPR = SH::CPR;
  static_assert(SH::DMA_PER_WAVE * kPfWaves * 64 == kBN * CPR, "a wave loads 1/4 of a tile");
  static_assert(kBN == 16 * kPfWaves, "wave w loads key block w of the tile");
  // wave w's instructions cover key block w (16 keys, one page) of K and V
  const int kb = kb0 + 16 * wave;
  const uint32_t pg = block_page(s_pt, bt_row, num_pages, p_shift, kb, kmax);
  const size_t row0 = ((size_t)pg << p_shift) + (size_t)(kb & ((1 << p_shift) - 1));
  const char* kblk = kpool + row0 * slot_stride;
  const char* vblk = vpool + row0 * slot_stride;
#pragma unroll
  for (int i = 0; i < SH::DMA_PER_WAVE; ++i) {
    const int q = wave * SH::DMA_PER_WAVE + i;
    // K: chunks 4 (q % (CPR / 4)) .. + 3 of the block's 16 keys
    lds_dma16_s(kblk + 64 * (i % (CPR / 4)), lk, sk + 1024 * q);
    // V: 8-key group q % 2 of the block, chunk pairs 4 (q % (CPR / 8)) .. + 3
    //    (D = 128: CPR / 8 = 2 instructions per 8-key group; D = 64: one)
    const int g8 = (64 * q) / (8 * CPR);
    const int cp = ((64 * q) % (8 * CPR)) / 16;
    lds_dma16_s(vblk + (size_t)(8 * (g8 & 1)) * slot_stride + 32 * cp, lv, sv + 1024 * q);
  }
}

// Loads of a tile that may reach past kmax: every lane computes its own key,
// clamped to kmax - 1, so that no row past the sequence is read (such rows may
// hold anything; their scores are masked and their V rows repeat key kmax - 1
// under a zero weight).
template <int D>
__device__ __forceinline__ void tile_dma_partial(uint32_t sk, uint32_t sv, const char* kpool,
                                                 const char* vpool, const int* s_pt,
                                                 const int* bt_row, int num_pages, int p_shift,
                                                 size_t slot_stride, int kb0, int kmax, int wave,
                                                 int lane) {
  typedef PfShape<D> SH;
  constexpr int CPR = SH::CPR;
  const int rmask = (1 << p_shift) - 1;
#pragma unroll
  for (int i = 0; i < SH::DMA_PER_WAVE; ++i) {
    const int q = wave * SH::DMA_PER_WAVE + i;  // wave-uniform
    const int u = 64 * q + lane;
    {
      const int row = (u / (16 * CPR)) * 16 + u % 16, c = (u % (16 * CPR)) / 16;
      const int key = min(kb0 + row, kmax - 1);
      const uint32_t pg = block_page(s_pt, bt_row, num_pages, p_shift, kb0 + (row & ~15), kmax);
      const size_t off = (((size_t)pg << p_shift) + (size_t)(key & rmask)) * slot_stride + 16 * c;
      lds_dma16(kpool + off, sk + 1024 * q);
    }
    {
      const int row = (u / (8 * CPR)) * 8 + (u % 16) / 2;
      const int c = 2 * ((u % (8 * CPR)) / 16) + u % 2;
      const int key = min(kb0 + row, kmax - 1);
      const uint32_t pg = block_page(s_pt, bt_row, num_pages, p_shift, kb0 + (row & ~15), kmax);
      const size_t off = (((size_t)pg << p_shift) + (size_t)(key & rmask)) * slot_stride + 16 * c;
      lds_dma16(vpool + off, sv + 1024 * q);
    }
  }
}

// One tile of kBN keys for the wave's two 16-row blocks: S^T = K Q^T, online
// softmax per query row, O^T += V^T P^T.
template <int D>
__device__ __forceinline__ void tile_compute(const uint16_t* sk, const uint16_t* sv, int kb0,
                                             const uint4 (&qop)[2][D / 32], const int (&limit)[2],
                                             const bool (&masked)[2], float sl2e, int col,
                                             int grp, float (&m_run)[2], f32x4_t (&l_acc)[2],
                                             f32x4_t (&acc_o)[2][D / 16]) {
  constexpr int DSTEPS = D / 32;
  constexpr int DBLK = D / 16;

  constexpr int CPR = PfShape<D>::CPR;
  // ---- S^T = K Q^T: lane (grp, col) reads key kb*16 + col, chunk 4 ds + grp ----
  const int lane = grp * 16 + col;
  f32x4_t st[2][kKB];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) st[b][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ds = 0; ds < DSTEPS; ++ds) {
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
      const uint4 kop =
          *reinterpret_cast<const uint4*>(sk + 8 * (16 * CPR * kb + 64 * ds + lane));
      st[0][kb] = mfma16x16x32(kop, qop[0][ds], st[0][kb]);
      st[1][kb] = mfma16x16x32(kop, qop[1][ds], st[1][kb]);
    }
  }

  // ---- online softmax of this lane's two query rows ----
  // Scores in log2 units (score * scale * log2 e): a weight is
  // exp2(s * sl2e - m), one fma and one exp2. Only tiles reaching past some
  // row's last visible key are masked (`masked` is wave-uniform per block).
  uint32_t pw[2][2 * kKB];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float sv[4 * kKB];
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[kb * 4 + i] = st[b][kb][i];
    if (masked[b]) {
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kb0 + kb * 16 + grp * 4 + i > limit[b]) sv[kb * 4 + i] = -INFINITY;
    }
    float tmax = sv[0];
#pragma unroll
    for (int k = 1; k < 4 * kKB; ++k) tmax = fmaxf(tmax, sv[k]);
    tmax = max4rows(tmax) * sl2e;
    // Rescale only when some row's max grows by more than 2^8 over the
    // running value (wave-uniform test): until then the weights exp2(s - m)
    // stay below 256, and numerator and sum share the same stale m, so the
    // result is unchanged while most tiles skip the rescaling.
    if (__any(tmax > m_run[b] + 8.f)) {
      const float mn = fmaxf(m_run[b], tmax);
      const float corr = fast_exp2(m_run[b] - mn);
      m_run[b] = mn;
      l_acc[b][0] *= corr;
      l_acc[b][1] *= corr;
      l_acc[b][2] *= corr;
      l_acc[b][3] *= corr;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        acc_o[b][db][0] *= corr;
        acc_o[b][db][1] *= corr;
        acc_o[b][db][2] *= corr;
        acc_o[b][db][3] *= corr;
      }
    }
    const float neg_m = -m_run[b];
#pragma unroll
    for (int k = 0; k < 2 * kKB; ++k) {
      const float p0 = fast_exp2(fmaf(sv[2 * k], sl2e, neg_m));
      const float p1 = fast_exp2(fmaf(sv[2 * k + 1], sl2e, neg_m));
      const f32x2_t pf = {p0, p1};  // rounded once to bf16 (round to nearest even)
      pw[b][k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pf, bf16x2e_t));
    }
  }

  // ---- O^T += V^T P^T, one 32-key k-step per pair of 16-key blocks ----
  // Contraction order of k-step ks in lane group g: elements 0..3 are keys
  // 32 ks + 4 g + 0..3, elements 4..7 keys 32 ks + 16 + 4 g + 0..3 (the keys
  // of the lane's S^T accumulators of blocks 2 ks and 2 ks + 1).
  const int s = col;  // lane index within the 16-lane group
  // this lane's byte offset in the V tile (the rest is known per (ks, r, db))
  const int vlane = 16 * ((grp >> 1) * 8 * CPR + (4 * (grp & 1) + s / 4) * 2 + (s % 4) / 2) +
                    8 * (s % 2);
  // Row sums: the same P^T operands times a 16 x 32 block of ones give, in
  // every output element, the sum of the row's bf16 weights (the values the
  // P.V products use), on the matrix cores instead of 32 VALU adds.
  const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
#pragma unroll
  for (int ks = 0; ks < kKB / 2; ++ks) {
    const uint4 pop0 = make_uint4(pw[0][4 * ks], pw[0][4 * ks + 1], pw[0][4 * ks + 2], pw[0][4 * ks + 3]);
    const uint4 pop1 = make_uint4(pw[1][4 * ks], pw[1][4 * ks + 1], pw[1][4 * ks + 2], pw[1][4 * ks + 3]);
    l_acc[0] = mfma16x16x32(ones, pop0, l_acc[0]);
    l_acc[1] = mfma16x16x32(ones, pop1, l_acc[1]);
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      uint32_t w[4];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        // key 32 ks + 16 r + 4 grp + s / 4, dims 16 db + 4 (s % 4) .. + 3
        const char* p = reinterpret_cast<const char*>(sv) + vlane +
                        16 * ((4 * ks + 2 * r) * 8 * CPR + 16 * db);
        const v4i16_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16_t*)(p));
        const uint2 xw = __builtin_bit_cast(uint2, x);
        w[2 * r] = xw.x;
        w[2 * r + 1] = xw.y;
      }
      const uint4 vop = make_uint4(w[0], w[1], w[2], w[3]);
      acc_o[0][db] = mfma16x16x32(vop, pop0, acc_o[0][db]);
      acc_o[1][db] = mfma16x16x32(vop, pop1, acc_o[1][db]);
    }
  }
}

// One prefill work entry, run by the whole workgroup (4 waves): row tile mt
// (TM tokens x G query heads = 128 rows) of sequence s against KV head kvh,
// over the key tiles of piece j of J. An uncut item (J = 1) writes its rows;
// a piece writes its partial (m, l, o) to slot slot0 + kvh * J + j, and the
// merge kernel combines the pieces after the tick.
template <int D, int G>
__device__ __forceinline__ void prefill_item(const AttnArgs& a, PfSmem<D>& sm, int4 e, int4 shape,
                                             int kvh) {
  // wave-uniform by construction (see the callers); explicit for the compiler
  const int s = __builtin_amdgcn_readfirstlane(e.x), mt = __builtin_amdgcn_readfirstlane(e.y);
  const int ez = __builtin_amdgcn_readfirstlane(e.z), slot0 = __builtin_amdgcn_readfirstlane(e.w);
  const int pj = ez & 0xFFFF, pJ = ez >> 16;
  typedef PfShape<D> SH;
  constexpr int TM = kRowsPerWg / G;    // tokens per item
  constexpr int DSTEPS = D / 32;        // k-steps of the QK^T product
  constexpr int DBLK = D / 16;          // 16-dim output blocks

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int col = lane & 15;            // query row within a 16-row block
  const int grp = lane >> 4;            // 0..3
  const size_t row_bytes = (size_t)D * 2;
  const int Hq = a.Hq;
  const float sl2e = a.scale_log2e;
  const size_t slot_stride = (size_t)a.Hkv * row_bytes;
  const int p_shift = a.p_shift;
  // the sequence's shape as the plan read it (query_start_loc, seq_lens
  // clamped to the page table and max_seq_len)
  const int q0 = __builtin_amdgcn_readfirstlane(shape.x);
  const int L = __builtin_amdgcn_readfirstlane(shape.y);
  const int n = __builtin_amdgcn_readfirstlane(shape.z);
  const int i0 = mt * TM;
  if (L <= 1 || i0 >= L || q0 < 0 || q0 + L > a.T || n < L) return;  // uniform per item
  const int i1 = min(L, i0 + TM);
  const int kmax = n - L + i1;          // keys visible to the tile's last row
  const int ntiles = (kmax + kBN - 1) / kBN;
  const int tb = pj * ntiles / pJ, te = (pj + 1) * ntiles / pJ;  // this piece's tiles
  const int last_key = n - L;           // row i sees keys <= last_key + i

  // The wave's two 16-row blocks: rows 32 wave + 16 b + col. Every global
  // load of the item's set-up goes out before any of them is used: the query
  // rows, their cos/sin rows and the first page ids, so that the set-up waits
  // for one round trip to memory rather than one per step (behind a decode
  // stream sharing the GPU, a round trip takes microseconds).
  uint4 qop[2][DSTEPS];
  int tok[2], head[2], limit[2], min_limit[2];
  bool row_ok[2];
  // the fused tick's q is the unrotated input: the lane's dims grp * 8 + 32 ds
  // (pairs ds, ds + DSTEPS / 2) are rotated at the row's position, exactly as
  // the page writer rotates a stored key. Row i of a chunk of L rows over n
  // keys is the token at position n - L + i (the tick's rows are the
  // sequence's last keys), so the cos/sin loads need no load of the position.
  const bool rope = a.fused && a.cos_sin && a.max_pos > 0;
  float rc[2][DSTEPS / 2][8], rs[2][DSTEPS / 2][8];
  bool rope_ok[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int r0 = wave * kRowsPerWave + 16 * b;
    const int rr = r0 + col;
    tok[b] = i0 + rr / G;
    head[b] = kvh * G + rr % G;
    row_ok[b] = tok[b] < i1;
    limit[b] = min(last_key + tok[b], n - 1);
    // smallest key limit of the block's rows: tiles ending at or below it need no mask
    min_limit[b] = last_key + i0 + r0 / G;
    const int tq = row_ok[b] ? tok[b] : i1 - 1;  // rows past the chunk read a valid row, zeroed
    const char* qrow = (const char*)a.q + ((size_t)(q0 + tq) * Hq + head[b]) * row_bytes;
#pragma unroll
    for (int ds = 0; ds < DSTEPS; ++ds)
      qop[b][ds] = *reinterpret_cast<const uint4*>(qrow + (ds * 32 + grp * 8) * 2);
    const int pos = last_key + tq;
    rope_ok[b] = pos >= 0 && pos < a.max_pos;  // (other rows stay as given)
    if (rope) {
      const int pc = clampi(pos, 0, a.max_pos - 1);
#pragma unroll
      for (int ds = 0; ds < DSTEPS / 2; ++ds)
        rope_load8(a.cos_sin, D, pc, grp * 8 + 32 * ds, rc[b][ds], rs[b][ds]);
    }
  }
  const int* bt_row = a.block_tables + (size_t)s * a.max_blocks;
  const int npg = min((kmax + (1 << p_shift) - 1) >> p_shift, kItemPages);
  const int pg_first = tid < npg ? clampi(bt_row[tid], 0, a.num_pages - 1) : 0;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    if (rope && rope_ok[b]) {
#pragma unroll
      for (int ds = 0; ds < DSTEPS / 2; ++ds)
        rope_bf16x8(qop[b][ds], qop[b][ds + DSTEPS / 2], rc[b][ds], rs[b][ds]);
    }
#pragma unroll
    for (int ds = 0; ds < DSTEPS; ++ds) qop[b][ds] = keep_if(qop[b][ds], row_ok[b]);
  }

  f32x4_t acc_o[2][DBLK];
  float m_run[2] = {kNegBig, kNegBig};
  // row sums on the matrix cores (see tile_compute): every element of a
  // lane's accumulator holds the sum of its query row
  f32x4_t l_acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int db = 0; db < DBLK; ++db) acc_o[b][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const char* kpool = (const char*)a.k_pool + (size_t)kvh * row_bytes;
  const char* vpool = (const char*)a.v_pool + (size_t)kvh * row_bytes;

  // the sequence's page ids into LDS (the first kPfThreads loaded above)
  if (tid < npg) sm.pt[tid] = pg_first;
  for (int i = tid + kPfThreads; i < npg; i += kPfThreads)
    sm.pt[i] = clampi(bt_row[i], 0, a.num_pages - 1);
  __syncthreads();

  // A ring of kPfStages LDS stages: the loads of the next kPfStages - 1 tiles
  // are in flight while tile t computes. Every wave waits for its own loads of
  // tile t (vmcnt: the later tiles' loads are the most recent ones); then one
  // barrier per tile both makes all waves' loads of tile t visible and tells
  // that every wave is done with tile t - 1, whose stage the loads issued
  // right after it refill.
  const uint32_t lk = dma_lane_k(lane, slot_stride), lv = dma_lane_v(lane, slot_stride);
  // LDS byte addresses of the stages (wave-uniform: scalar registers)
  const uint32_t lds_k0 = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(sm.k[0]));
  const uint32_t lds_v0 = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(sm.v[0]));
  constexpr uint32_t kStageBytes = sizeof(sm.k[0]);
  auto issue = [&](int tile, int stage) {
    const int kb0 = tile * kBN;
    const uint32_t sk = lds_k0 + kStageBytes * stage, sv = lds_v0 + kStageBytes * stage;
    if (kb0 + kBN <= kmax)
      tile_dma_full<D>(sk, sv, kpool, vpool, sm.pt, bt_row, a.num_pages, p_shift, slot_stride,
                       kb0, kmax, wave, lk, lv);
    else
      tile_dma_partial<D>(sk, sv, kpool, vpool, sm.pt, bt_row, a.num_pages, p_shift,
                          slot_stride, kb0, kmax, wave, lane);
  };
#pragma unroll
  for (int t = 0; t < kPfStages - 1; ++t)
    if (tb + t < te) issue(tb + t, t);
  int st = 0;  // stage of tile t
  for (int t = tb; t < te; ++t) {
    wait_tiles<SH::DMA_PER_TILE>(min(te - 1 - t, kPfStages - 2));
    lds_barrier();
    const int tn = t + kPfStages - 1;  // tile whose loads start now
    if (tn < te) issue(tn, st == 0 ? kPfStages - 1 : st - 1);  // the stage of tile t - 1
    const int kb0 = t * kBN;
    const bool masked[2] = {kb0 + kBN - 1 > min_limit[0], kb0 + kBN - 1 > min_limit[1]};
    tile_compute<D>(sm.k[st], sm.v[st], kb0, qop, limit, masked, sl2e, col, grp, m_run, l_acc,
                    acc_o);
    st = st + 1 == kPfStages ? 0 : st + 1;
  }
  // every wave is done with the stages (and the page ids) before the next
  // item's loads refill them
  lds_barrier();

  if (pJ > 1) {
    // ---- piece of a cut item: partial (m, l, o) of the 128 rows ----
    const int slot = slot0 + kvh * pJ + pj;
    float* po = a.pf_ws + (size_t)slot * kRowsPerWg * D;
    float* pml = a.pf_ws + (size_t)a.pf_slots * kRowsPerWg * D + 2 * (size_t)slot * kRowsPerWg;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int r = wave * kRowsPerWave + 16 * b + col;
      const float lt = l_acc[b][0];
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
        *reinterpret_cast<float4*>(po + (size_t)r * D + db * 16 + grp * 4) =
            make_float4(acc_o[b][db][0], acc_o[b][db][1], acc_o[b][db][2], acc_o[b][db][3]);
      if (grp == 0) *reinterpret_cast<float2*>(pml + 2 * r) = make_float2(m_run[b], lt);
    }
    return;
  }

  // ---- normalise and store ----
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const float lt = l_acc[b][0];
    if (row_ok[b]) {
      const float inv = 1.f / lt;
      uint16_t* orow =
          reinterpret_cast<uint16_t*>(a.out) + ((size_t)(q0 + tok[b]) * Hq + head[b]) * D;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const f32x2_t lo = {acc_o[b][db][0] * inv, acc_o[b][db][1] * inv};
        const f32x2_t hi = {acc_o[b][db][2] * inv, acc_o[b][db][3] * inv};
        const uint2 wv =
            make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2e_t)),
                       __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2e_t)));
        *reinterpret_cast<uint2*>(orow + db * 16 + grp * 4) = wv;
      }
    }
  }
}

}  // namespace pa

#pragma clang diagnostic pop
