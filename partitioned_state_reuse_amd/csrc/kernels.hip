// HIP kernels for gfx950 (CDNA4): partition attention with state-cache update (optionally
// with the reused states' pre-merge in the same launch), state merge (all planes, selected
// planes plus a partial state, fp8 codes), partition importance, and the local-change
// reduction.
//
// The operation follows "DiTango: Cost-Effective Parallel Diffusion Generation with
// Selective Attention State Reuse" (technical summary, "Methodology §2, State Composition"
// and "§1, Anchor-Guided Selection Planner"): per KV partition an attention state
// (O_p, lse_p) is produced; the states are composed by LSE-weighted combination.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "launch.h"

namespace dit {
namespace {

typedef unsigned short u16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Two floats -> two bfloat16 (round to nearest even), packed low/high in 32 bits.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 r = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// ------------------------------------------------------------------------------------
// Partition attention.
//
// One workgroup = kWaves waves (default 4; 3 workgroups per CU, i.e. 3 waves per SIMD) =
// one (batch, head, partition p, query tile of <= 32 kWaves rows of one query block); a
// wave whose 32 rows all lie past the block end only helps with the tile copies.  Each wave
// owns 32 query rows and keeps them in registers as the B operand of S^T = K Q^T
// (v_mfma_f32_32x32x16_bf16), so that each lane's 16 scores per 32-key block belong to one
// query and the softmax reductions over keys stay inside a lane pair (l, l ^ 32), joined
// with v_permlane32_swap.
//
// K and V tiles of kBlockN keys (default 32) are copied global -> LDS by the DMA path
// (buffer_load_dwordx4 ... lds, no VGPR staging) into a ring of kStages buffers (default 2) so
// that the next tile is in flight while the current one is consumed.  Both tiles stay
// row-major [key][d] with a
// per-row XOR swizzle of the 16-byte chunks, chosen so that the K reads (ds_read_b128, A
// operand of K Q^T) and the V reads are free of bank conflicts.  V^T, the A operand of
// O^T = V^T P^T, is read with the LDS transpose load ds_read_b64_tr_b16: in each group of
// 16 lanes, lane i receives element i % 4 of the 8-byte chunks addressed by lanes
// 4 j + i / 4, so pointing lane s of a group at V[key_(s / 4)][d0 + 4 (s % 4) ..] hands
// every lane four keys of one d.  P^T, the B operand, comes straight from the score
// registers; the key order inside each 16-key MFMA step is permuted identically on both
// operands.
//
// Online softmax in base 2, fp32 state, with a lazy running maximum: the maximum used
// for the exponentials is raised only when a tile's maximum exceeds it by more than
// kRescaleLog2 (then exponentials stay <= 2^kRescaleLog2 and nothing overflows), which
// skips the rescale of the accumulators on almost every tile; the tile's maximum itself is
// only computed when some lane's sum of the tile's exponentials (taken against the current
// maximum) exceeds that bound.  P is rounded to bf16 for
// the product.  The epilogue writes the partition's state into its cache slot (bf16, or
// e4m3 codes plus a per-row scale with FP8) through an LDS staging buffer and, for a
// block's local partition, the partial sums of the local-change norm.
// ------------------------------------------------------------------------------------
constexpr float kRescaleLog2 = 8.0f;
constexpr float kProbSumBound = 256.0f;  // 2^kRescaleLog2

template <int D>
struct TileGeom {
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int RPB = 256 / (2 * D);      // rows per 256 bytes (the 64 banks)
  static constexpr int ROWS_PER_KB = 1024 / (2 * D);
  static constexpr int TILE_ELEMS = kBlockN * D;
  static constexpr int KB_PER_TILE = TILE_ELEMS * 2 / 1024;
  // waves past KB_PER_TILE issue nothing when a tile has fewer 1-KB blocks than waves
  static constexpr int KB_PER_WAVE = (KB_PER_TILE + kWaves - 1) / kWaves;
  // physical chunk = logical chunk ^ swizzle(row)
  static __device__ __forceinline__ int swz_k(int r) { return (r / RPB) % CPR; }
  static __device__ __forceinline__ int swz_v(int r) { return 4 * ((r / RPB) % (CPR / 4)); }
};

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 s16x4_lds;

// Per-lane byte offsets (within a tile of one head) of this lane's share of the DMA copy:
// for each of the wave's 1-KB destination blocks, the lane fills physical chunk
// `lane % CPR` of row `kb * ROWS_PER_KB + lane / CPR`, which holds logical chunk
// `slot ^ swizzle(row)`.  Rows at or past `nvalid` re-read row nvalid - 1 (their scores
// are masked and their V rows meet zero probabilities), so no load leaves the partition.
template <int D, bool IS_V>
__device__ __forceinline__ void dma_offsets(int rowstride, int nvalid, int wave, int lane,
                                            uint32_t (&off)[TileGeom<D>::KB_PER_WAVE]) {
  using G = TileGeom<D>;
#pragma unroll
  for (int t = 0; t < G::KB_PER_WAVE; ++t) {
    const int kb = wave * G::KB_PER_WAVE + t;
    const int row = min(kb, G::KB_PER_TILE - 1) * G::ROWS_PER_KB + lane / G::CPR;
    const int c = (lane % G::CPR) ^ (IS_V ? G::swz_v(row) : G::swz_k(row));
    off[t] = (uint32_t)(min(row, nvalid - 1) * rowstride + c * 8) * 2u;
  }
}

// Issue one wave's share of the DMA copy of a tile (tile base and wave index are uniform).
// Buffer loads against a descriptor over the tile's rows rather than global loads: each
// lane supplies a 32-bit offset instead of a 64-bit address (per tile 4 VALU instructions
// instead of 10, and 155 instead of 167 VGPRs), and an offset past the descriptor's range
// reads zeros instead of faulting.
template <int D>
__device__ __forceinline__ void issue_tile(const u16 *__restrict__ gtile,
                                           const uint32_t (&off)[TileGeom<D>::KB_PER_WAVE],
                                           u16 *lds_tile, int wave, uint32_t tile_bytes) {
#if __HIP_DEVICE_COMPILE__  // the buffer-resource builtins exist in the device pass only
  using G = TileGeom<D>;
  const auto rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)gtile, (short)0, (int)tile_bytes, 0x00020000);
#pragma unroll
  for (int t = 0; t < G::KB_PER_WAVE; ++t) {
    const int kb = wave * G::KB_PER_WAVE + t;
    if (G::KB_PER_TILE % kWaves == 0 || kb < G::KB_PER_TILE)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void *)(lds_tile + kb * 512), 16, off[t], 0, 0, 0);
  }
#endif
}

__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The work of one attention workgroup: workgroup `wg` of the `nwg` that carry attention
// items.
template <int D, bool FP8>
__device__ __forceinline__ void attention_item(
    const u16 *__restrict__ q, const u16 *__restrict__ k, const u16 *__restrict__ v,
    void *__restrict__ cache_o, float *__restrict__ cache_scale, float *__restrict__ cache_lse,
    float *__restrict__ delta_part, const AttnDesc &desc, const float scale_log2, const int nwg, const int wg) {
  using G = TileGeom<D>;
  constexpr int KK = D / 16;        // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;        // 32-row blocks of O^T
  constexpr int MB = kBlockN / 32;  // 32-key blocks of S^T per tile
  constexpr int NC = kBlockN / 16;  // 16-key steps of O^T += V^T P^T per tile
  // Ring of kStages K and V tile buffers; separate variables so that the compiler knows a
  // DMA into one buffer does not alias reads of another (no wait is inserted for it).
  __shared__ __attribute__((aligned(1024))) u16 k_lds0[G::TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) u16 k_lds1[G::TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) u16 k_lds2[kStages > 2 ? G::TILE_ELEMS : 1];
  __shared__ __attribute__((aligned(1024))) u16 v_lds0[G::TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) u16 v_lds1[G::TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) u16 v_lds2[kStages > 2 ? G::TILE_ELEMS : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- work item.  Workgroups are dealt round-robin to the 8 XCDs (workgroup w to XCD
  // w mod 8); remap so that each XCD takes a contiguous range of the items: consecutive items
  // (same K/V partition) run on one XCD and share its L2.
  const int xcd = wg & 7, per = nwg >> 3, rem = nwg & 7;
  const int item = xcd * per + min(xcd, rem) + (wg >> 3);
  const int per_head = desc.items_per_head;
  const int bh = item / per_head;
  int idx = item - bh * per_head;
  const int H = desc.H;
  const int b = bh / H;
  const int head = bh - b * H;
  // partition of the item: the last p < P with item_prefix[p] <= idx (a partition without
  // items has the same prefix as the next one, so that p is the one that holds idx); a
  // binary search keeps the chain of dependent scalar loads short when P is large
  int p = 0;
  {
    int hi = desc.P - 1;
    while (p < hi) {
      const int mid = (p + hi + 1) >> 1;
      if (desc.item_prefix[mid] <= idx) p = mid; else hi = mid - 1;
    }
  }
  idx -= desc.item_prefix[p];
  uint64_t bm = desc.blocks_of_part[p];
  int blk = 0;
  for (;;) {
    if (bm == 0) return;  // inconsistent description; the host never builds one
    blk = __builtin_ctzll(bm);
    const int nt = desc.tile_prefix[blk + 1] - desc.tile_prefix[blk];
    if (idx < nt) break;
    idx -= nt;
    bm &= bm - 1;
  }
  const int tile = idx;
  const int q0 = desc.q_off[blk] + tile * kBlockM;
  const int qn = min(kBlockM, desc.q_off[blk + 1] - q0);
  const int kv0 = desc.kv_off[p];
  const int kvn = desc.kv_off[p + 1] - kv0;
  const int rowstride = H * D;
  const int ntiles = (kvn + kBlockN - 1) / kBlockN;

  const u16 *kbase = k + ((int64_t)b * desc.S_kv + kv0) * rowstride + (int64_t)head * D;
  const u16 *vbase = v + ((int64_t)b * desc.S_kv + kv0) * rowstride + (int64_t)head * D;
  const int64_t tile_step = (int64_t)kBlockN * rowstride;
  // bytes a tile's rows span (the descriptor's range; offsets stay below it)
  const uint32_t tile_bytes = (uint32_t)min((int64_t)kBlockN * rowstride * 2, (int64_t)0x7fffffff);

  // ---- DMA offsets of full tiles; the last tile's clamped ones are made when it is issued
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int last_valid = kvn - (ntiles - 1) * kBlockN;
  uint32_t koff_full[G::KB_PER_WAVE], voff_full[G::KB_PER_WAVE];
  dma_offsets<D, false>(rowstride, kBlockN, wave_u, lane, koff_full);
  dma_offsets<D, true>(rowstride, kBlockN, wave_u, lane, voff_full);
  // The ring stage is a compile-time argument everywhere: k_lds<t % kStages> holds K tile t
  // and v_lds<t % kStages> holds V tile t.
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  auto kbuf = [&](auto st) -> u16 * {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return k_lds0; else if constexpr (S == 1) return k_lds1; else return k_lds2;
  };
  auto vbuf = [&](auto st) -> u16 * {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return v_lds0; else if constexpr (S == 1) return v_lds1; else return v_lds2;
  };
  // Issue the copies of K and V tile t.  The last tile of a partition whose length is not a
  // multiple of kBlockN clamps its rows: its offsets overwrite the full-tile ones once, in a
  // wave-uniform branch (tile t is issued after every earlier tile).
  auto issue_kv = [&](int t, auto par) {
    if (t == ntiles - 1 && last_valid < kBlockN) {
      dma_offsets<D, false>(rowstride, last_valid, wave_u, lane, koff_full);
      dma_offsets<D, true>(rowstride, last_valid, wave_u, lane, voff_full);
    }
    issue_tile<D>(kbase + t * tile_step, koff_full, kbuf(par), wave_u, tile_bytes);
    issue_tile<D>(vbase + t * tile_step, voff_full, vbuf(par), wave_u, tile_bytes);
  };
  // prologue: the first kStages - 1 tiles in flight
  if (ntiles > 0) issue_kv(0, S0{});
  if (kStages > 2 && ntiles > 1) issue_kv(1, S1{});

  // ---- this lane's query row, as the B operand: Q[row][16 kk + 8 hh + 0..7]
  const int qrow = wave * 32 + l32;
  const bool qvalid = qrow < qn;
  const bool active = wave * 32 < qn;  // wave-uniform: some of this wave's rows exist
  bf16x8 qf[KK];
  {
    const u16 *qp = q + ((int64_t)b * desc.S_q + q0 + (qvalid ? qrow : 0)) * rowstride +
                    (int64_t)head * D + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (qvalid) u = *(const uint4 *)(qp + 16 * kk);
      qf[kk] = as_bf16x8(u);
    }
  }

  // ---- per-lane LDS byte offsets of the MFMA operand reads.  The XOR swizzle acts on
  // address bits below the row base, so each k-step (K) or d-block (V) is one XOR away
  // from the lane's base offset: K step kk at k_lane ^ (kk << 5), V d-block db at
  // v_lane ^ (db << 6).
  uint32_t k_lane, v_lane;
  {
    const int x = hh ^ G::swz_k(l32);
    k_lane = (uint32_t)(l32 * D + x * 8) * 2u;
    const int grp = lane >> 4, ls = lane & 15;
    const int vrow = 4 * (grp >> 1) + (ls >> 2);
    const int sv = G::swz_v(vrow);
    const int cidx0 = 2 * (grp & 1) + ((ls & 3) >> 1);
    v_lane = (uint32_t)(vrow * D + (cidx0 ^ sv) * 8 + (ls & 1) * 4) * 2u;
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m = -INFINITY, lsum = 0.f;   // m: running maximum in scaled base-2 units

  // S^T = K Q^T of the K tile in `Kt`: s[mb][r] holds key 32 mb + (r & 3) + 8 (r >> 2) + 4 hh
  // of the tile for query row l32.
  auto qk = [&](const u16 *Kt, f32x16 (&s)[MB]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mb][r] = 0.f;
    if constexpr (MB == 1) {
      // operands read kReadAhead MFMAs ahead; the scheduling barriers keep that distance
      bf16x8 ka[KK];
      auto kread = [&](int kk) {
        ka[kk] = as_bf16x8(*(const uint4 *)((const char *)Kt + (k_lane ^ (uint32_t)(kk << 5))));
      };
#pragma unroll
      for (int kk = 0; kk < kReadAhead && kk < KK; ++kk) kread(kk);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + kReadAhead < KK) kread(kk + kReadAhead);
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], qf[kk], s[0], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const bf16x8 a = as_bf16x8(*(const uint4 *)((const char *)Kt + (k_lane ^ (uint32_t)(kk << 5)) + mb * 64 * D));
          s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[mb], 0, 0, 0);
        }
      }
    }
  };
  // Keys at or past `nvalid` of the tile get score -inf.
  auto mask_tail = [&](f32x16 (&s)[MB], int nvalid) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * mb + (r & 3) + 8 * (r >> 2) + 4 * hh;
        if (key >= nvalid) s[mb][r] = -INFINITY;
      }
  };
  // Maximum of a tile's scores for this lane's query (the lane pair holds all keys of the
  // tile), in scaled base-2 units.
  auto tile_max = [&](const f32x16 (&s)[MB]) {
    float mt = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = (mb == 0 ? 2 : 0); r < 16; ++r) mt = fmaxf(mt, s[mb][r]);
    return pair_max(mt) * scale_log2;
  };
  // Lazy running maximum: raise it (and rescale the accumulators) only when the tile's
  // maximum exceeds it by more than kRescaleLog2 for some lane of the wave.
  // Returns whether the maximum moved (wave-uniform).
  auto rescale = [&](float mt) -> bool {
    if (__ballot(mt > m + kRescaleLog2)) {
      const float mnew = fmaxf(m, mt);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      return true;
    }
    return false;
  };
  // Probabilities of a tile against the current running maximum, packed to bf16 as the B
  // operand of the 16-key PV steps; returns this lane's sum of them (not yet in lsum).
  auto probs = [&](const f32x16 (&s)[MB], bf16x8 (&pb)[NC]) {
    const float negm = -m;
    float ts;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int mb = c >> 1;
      const int base = 8 * (c & 1);
      float e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        e[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][base + j], scale_log2, negm));
        ts = (c == 0 && j == 0) ? e[j] : ts + e[j];
      }
      uint4 pu;
      pu.x = pack_bf16x2(e[0], e[1]);
      pu.y = pack_bf16x2(e[2], e[3]);
      pu.z = pack_bf16x2(e[4], e[5]);
      pu.w = pack_bf16x2(e[6], e[7]);
      pb[c] = as_bf16x8(pu);
    }
    return ts;
  };
  // O^T += V^T P^T over the 16-key steps.  k-index 8 hh + j of step c stands for key
  // 16 c + 4 hh + 8 (j >> 2) + (j & 3) on both operands.
  // MFMA i of the tile takes step c = i / DB and d-block db = i % DB; its V^T operand is
  // read kReadAhead MFMAs ahead.
  auto pv = [&](const u16 *Vt, const bf16x8 (&pb)[NC]) {
    constexpr int NPV = NC * DB;
    bf16x8 va[NPV];
    auto vread = [&](int i) {
      const int c = i / DB, db = i % DB;
      const u16 *vp = (const u16 *)((const char *)Vt + (v_lane ^ (uint32_t)(db << 6)) + 32 * c * D);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_lds *)(vp));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_lds *)(vp + 8 * D));
      const uint2 lo2 = __builtin_bit_cast(uint2, lo);
      const uint2 hi2 = __builtin_bit_cast(uint2, hi);
      va[i] = as_bf16x8(make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
    };
#pragma unroll
    for (int i = 0; i < kReadAhead && i < NPV; ++i) vread(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      if (i + kReadAhead < NPV) vread(i + kReadAhead);
      o[i % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], pb[i / DB], o[i % DB], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Wait until this wave's copy of the oldest tile still in flight has landed (the loads of
  // one tile per wave: vmcnt counts them in issue order), optionally leaving the next
  // tile's loads in flight, then meet the other waves: afterwards the tile is complete in
  // LDS and every wave is done reading the buffer that the next issue overwrites.
  constexpr int kLoadsPerTile = 2 * G::KB_PER_WAVE;
  static_assert(kStages == 2 || G::KB_PER_TILE % kWaves == 0, "every wave must issue the same loads per tile");
  static_assert(kLoadsPerTile < 16, "vmcnt immediate");
  auto wait_tiles = [&](bool next_in_flight) {
    if (kStages > 2 && next_in_flight)
      __builtin_amdgcn_s_waitcnt(0x0F70 | kLoadsPerTile);  // vmcnt(kLoadsPerTile)
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);                  // vmcnt(0)
    // A bare barrier: __syncthreads() (or any release fence covering LDS) would also wait
    // for the tile copy that is meant to stay in flight, since copies into LDS count as LDS
    // writes.  The wait above covers the tile about to be read; this wave's reads of the
    // buffer to be overwritten have completed (their data fed the MFMAs); the memory clobber
    // keeps the compiler from moving LDS accesses across the barrier.
    asm volatile("s_barrier" ::: "memory");
  };

  // Tile kt + kStages - 1 is copied while tile kt is consumed.
  auto step = [&](int kt, auto st) {
    constexpr int S = decltype(st)::value;
    using Sa = std::integral_constant<int, (S + kStages - 1) % kStages>;
    const bool ahead = kt + kStages - 1 < ntiles;
    if (ahead) issue_kv(kt + kStages - 1, Sa{});
    if (active) {
      f32x16 s[MB];
      if constexpr (kSetPrio) __builtin_amdgcn_s_setprio(1);
      qk(kbuf(st), s);
      if constexpr (kSetPrio) __builtin_amdgcn_s_setprio(0);
      if (kt == ntiles - 1 && last_valid < kBlockN) mask_tail(s, last_valid);
      // Exponentials first, against the running maximum as it stands.  Every probability
      // is at most the lane's tile sum, so a sum within 2^kRescaleLog2 on every lane keeps
      // the lazy-maximum bound without computing the tile's maximum.  Otherwise (a sum
      // above the bound, or not finite, as on the first tile) the maximum is checked, the
      // accumulators are rescaled if it moved past the bound, and the tile is redone.
      // When no lane's maximum moved past the bound, every exponential already taken is at
      // most 2^kRescaleLog2 and the tile is kept as it is.
      bf16x8 pb[NC];
      float ts = probs(s, pb);
      if (__ballot(!(ts <= kProbSumBound))) {
        if (rescale(tile_max(s))) ts = probs(s, pb);
      }
      lsum += ts;
      if constexpr (kSetPrio) __builtin_amdgcn_s_setprio(1);
      pv(vbuf(st), pb);
      if constexpr (kSetPrio) __builtin_amdgcn_s_setprio(0);
    }
    wait_tiles(ahead);
  };
  if (ntiles > 0) {
    wait_tiles(kStages > 2 && ntiles > 1);
    int kt = 0;
    if constexpr (kStages > 2) {
      for (; kt + 2 < ntiles; kt += 3) {
        step(kt, S0{});
        step(kt + 1, S1{});
        step(kt + 2, S2{});
      }
      if (kt < ntiles) step(kt, S0{});
      if (kt + 1 < ntiles) step(kt + 1, S1{});
    } else {
      for (; kt + 1 < ntiles; kt += 2) {
        step(kt, S0{});
        step(kt + 1, S1{});
      }
      if (kt < ntiles) step(kt, S0{});
    }
  }

  // ---- epilogue: normalise, write the state into cache slot (p, rows), local change
  const float ltot = pair_sum(lsum);
  const bool empty = !(ltot > 0.f);
  const float inv = empty ? 0.f : 1.f / ltot;
  const float lse_nat = empty ? -INFINITY : (m + __log2f(ltot)) * kLn2;
  const bool is_local = delta_part != nullptr && desc.local_part[blk] == p;
  float dnum = 0.f, dden = 0.f;
  // The wave's rows go out through a staging buffer in LDS: one of the tile buffers, free
  // now (every wave has passed the last tile's barrier and no copy is in flight).  The
  // wave writes its rows there in the MFMA layout (lane (l32, hh) holds d = 32 db + 8 g +
  // 4 hh + 0..3 of row l32), then reads them back row by row so that each row of the slot
  // is written with contiguous 16-byte stores; the local-change sums read the old slot
  // contents the same way.  16-byte chunk c of staged row r sits at chunk c ^ (r % chunks
  // per row), so that the column-wise writes and the row-wise reads are free of bank
  // conflicts.
  static_assert(kWaves <= 4, "one staging buffer per wave");
  // Cache slots are written once per step and read back only by the merge (and, for a local
  // partition, the old slot once by this epilogue): with kNtSlots they are streamed with
  // non-temporal accesses, so that they do not displace the K/V tiles other workgroups still
  // read from L2.
  auto store_slot = [](uint4 *dst, const uint4 &v) {
    if constexpr (kNtSlots)
      __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, (u32x4 *)dst);
    else
      *dst = v;
  };
  auto load_slot = [](const uint4 *src) -> uint4 {
    if constexpr (kNtSlots) {
      const u32x4 u = __builtin_nontemporal_load((const u32x4 *)src);
      return make_uint4(u[0], u[1], u[2], u[3]);
    } else {
      return *src;
    }
  };
  char *stg = (char *)(wave == 0 ? k_lds0 : wave == 1 ? k_lds1 : wave == 2 ? v_lds0 : v_lds1);
  auto slot_of = [&](int r) {  // [P, B, S_q] index of query row r of this tile
    return ((int64_t)p * desc.B + b) * desc.S_q + q0 + r;
  };
  auto lslot_of = [&](int r) {  // [P, B, S_q, H] index
    return slot_of(r) * H + head;
  };
  if constexpr (FP8) {
    // compressed slot: e4m3 codes of O / s with s = max_d |O| / 448 per (row, head); the
    // lane pair holds the row's D values
    constexpr int CPR8 = D / 16;  // 16-byte chunks (16 codes) per row
    float amax = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(o[db][r] * inv));
    amax = pair_max(amax);
    const float sc = amax / 448.f;
    const float inv_s = amax > 0.f ? 448.f / amax : 0.f;
    float *stg_scale = (float *)(stg + 32 * D);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hh;
        float x[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) x[t] = (o[db][4 * g + t] * inv) * inv_s;
        int wq = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
        wq = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], wq, true);
        *(int *)(stg + l32 * D + (((d0 >> 4) ^ (l32 % CPR8)) << 4) + (d0 & 15)) = wq;
      }
    }
    if (hh == 0) stg_scale[l32] = sc;
#pragma unroll
    for (int it = 0; it < 32 * CPR8 / 64; ++it) {
      const int c = it * 64 + lane;
      const int r = c / CPR8, col = c % CPR8;
      const uint4 nw = *(const uint4 *)(stg + r * D + ((col ^ (r % CPR8)) << 4));
      if (wave * 32 + r < qn) {
        uint8_t *dst = (uint8_t *)cache_o + (slot_of(wave * 32 + r) * H + head) * D + col * 16;
        if (is_local) {
          const uint4 od = load_slot((const uint4 *)dst);
          const float old_s = cache_scale[lslot_of(wave * 32 + r)];
          const float new_s = stg_scale[r];
          const uint32_t nn[4] = {nw.x, nw.y, nw.z, nw.w}, oo[4] = {od.x, od.y, od.z, od.w};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const f32x2 nv[2] = {__builtin_amdgcn_cvt_pk_f32_fp8((int)nn[t], false),
                                 __builtin_amdgcn_cvt_pk_f32_fp8((int)nn[t], true)};
            const f32x2 ov[2] = {__builtin_amdgcn_cvt_pk_f32_fp8((int)oo[t], false),
                                 __builtin_amdgcn_cvt_pk_f32_fp8((int)oo[t], true)};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float n0 = nv[e >> 1][e & 1] * new_s;
              const float o0 = ov[e >> 1][e & 1] * old_s;
              dnum += (n0 - o0) * (n0 - o0);
              dden += o0 * o0;
            }
          }
        }
        store_slot((uint4 *)dst, nw);
      }
    }
    // after the old scales have been read above
    if (qvalid && hh == 0) {
      cache_lse[lslot_of(qrow)] = lse_nat;
      cache_scale[lslot_of(qrow)] = sc;
    }
  } else {
    constexpr int CPR = D / 8;  // 16-byte chunks (8 bf16) per row
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hh;
        uint2 nw;
        nw.x = pack_bf16x2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv);
        nw.y = pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
        *(uint2 *)(stg + l32 * (2 * D) + (((d0 >> 3) ^ (l32 % CPR)) << 4) + (d0 & 7) * 2) = nw;
      }
    }
#pragma unroll
    for (int it = 0; it < 32 * CPR / 64; ++it) {
      const int c = it * 64 + lane;
      const int r = c / CPR, col = c % CPR;
      const uint4 nw = *(const uint4 *)(stg + r * (2 * D) + ((col ^ (r % CPR)) << 4));
      if (wave * 32 + r < qn) {
        u16 *dst = (u16 *)cache_o + (slot_of(wave * 32 + r) * H + head) * D + col * 8;
        if (is_local) {
          const uint4 od = load_slot((const uint4 *)dst);
          const uint32_t nn[4] = {nw.x, nw.y, nw.z, nw.w}, oo[4] = {od.x, od.y, od.z, od.w};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float n0 = bf16_bits_to_f32(nn[t] & 0xffffu), n1 = bf16_bits_to_f32(nn[t] >> 16);
            const float o0 = bf16_bits_to_f32(oo[t] & 0xffffu), o1 = bf16_bits_to_f32(oo[t] >> 16);
            dnum += (n0 - o0) * (n0 - o0) + (n1 - o1) * (n1 - o1);
            dden += o0 * o0 + o1 * o1;
          }
        }
        store_slot((uint4 *)dst, nw);
      }
    }
    if (qvalid && hh == 0) cache_lse[lslot_of(qrow)] = lse_nat;
  }
  if (is_local) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      dnum += __shfl_xor(dnum, off);
      dden += __shfl_xor(dden, off);
    }
    float *red = (float *)k_lds0;
    __syncthreads();  // every wave is done with the tiles before the scratch is reused
    if (lane == 0) {
      red[2 * wave] = dnum;
      red[2 * wave + 1] = dden;
    }
    __syncthreads();
    if (tid == 0) {
      float n = 0.f, d = 0.f;
      for (int w = 0; w < kWaves; ++w) {
        n += red[2 * w];
        d += red[2 * w + 1];
      }
      float *dp = delta_part + (((int64_t)b * desc.n_tiles + desc.tile_prefix[blk] + tile) * H + head) * 2;
      dp[0] = n;
      dp[1] = d;
    }
  }
}

template <int D, bool FP8>
__global__ __launch_bounds__(kWaves * 64, kMinBlocks) void partition_attention_kernel(
    const u16 *__restrict__ q, const u16 *__restrict__ k, const u16 *__restrict__ v,
    void *__restrict__ cache_o, float *__restrict__ cache_scale, float *__restrict__ cache_lse,
    float *__restrict__ delta_part, const AttnDesc desc, const float scale_log2) {
  attention_item<D, FP8>(q, k, v, cache_o, cache_scale, cache_lse, delta_part, desc, scale_log2, gridDim.x,
                         blockIdx.x);
}

// Workgroups are dealt round-robin to the 8 XCDs (workgroup w runs on XCD w mod 8), and
// each XCD has its own L2.  Neighbouring merge workgroups share cache lines of the lse (and
// scale) planes; remap so that each XCD takes runs of `chunk` consecutive workgroups (a
// line is fetched into one L2), while the 8 XCDs still stream neighbouring runs at the same
// time.  The ragged tail keeps the identity mapping.
__device__ __forceinline__ int lse_chunked_item(int chunk) {
  const int wg = blockIdx.x, nwg = gridDim.x;
  const int span = 8 * chunk;
  const int base = (wg / span) * span;
  if (chunk <= 1 || base + span > nwg) return wg;
  const int r = wg - base;
  return base + (r & 7) * chunk + (r >> 3);
}

// Workgroups per XCD run of the merge kernels: those covering kMergeChunkRows rows of all
// H heads (RPW row-heads per workgroup).
inline int merge_chunk(int RPW, int H) { return std::max(1, kMergeChunkRows * H / RPW); }

// Placement of merge workgroups over row-heads rh = (b S_q + r) H + h.  Plain (n_qb = 0):
// workgroup w takes RPW consecutive row-heads.  With importance partials, the workgroups of
// each (batch, query block) cover only that block's row-heads, so that the partial sums of a
// workgroup belong to one block: block i has ceil(|i| H / RPW) workgroups per batch,
// wg_prefix counts them.
struct MergeGrid {
  int32_t n_qb;
  int32_t wg_per_batch;
  int32_t q_off[DIT_MAX_BLOCKS + 1];
  int32_t wg_prefix[DIT_MAX_BLOCKS + 1];
};

template <int RPW>
__device__ __forceinline__ void merge_rows(const MergeGrid &g, int w, int S_q, int H, int64_t total_rh,
                                           int64_t &rh0, int64_t &rh_end) {
  if (g.n_qb == 0) {
    rh0 = (int64_t)w * RPW;
    rh_end = total_rh;
    return;
  }
  const int b = w / g.wg_per_batch;
  const int wl = w - b * g.wg_per_batch;
  int lo = 0, hi = g.n_qb - 1;  // last block i with wg_prefix[i] <= wl
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (g.wg_prefix[mid] <= wl) lo = mid; else hi = mid - 1;
  }
  rh0 = ((int64_t)b * S_q + g.q_off[lo]) * H + (int64_t)(wl - g.wg_prefix[lo]) * RPW;
  rh_end = ((int64_t)b * S_q + g.q_off[lo + 1]) * H;
}

// ------------------------------------------------------------------------------------
// State merge: one thread per 8 consecutive d of one (row, head), a workgroup per 16
// consecutive row-heads (4 KB contiguous runs of every partition plane).  The row-head's
// lanes first share out the merge weights (group_merge_weights: each lse value is loaded
// by one lane, not by all of them), then the P bf16 states are streamed with 16-byte
// non-temporal loads (PMAX >= P, unrolled) and combined in fp32; the merged output is
// written with non-temporal stores (it is not re-read by this step).  The cache's lse
// planes are [row][head], like the rows of the output: a workgroup's lse values of one
// plane are one contiguous run.
// ------------------------------------------------------------------------------------
// Merge weights of one row-head, computed by the TPR lanes that share it (one wave holds
// whole groups): lane c loads the lse (and, with SCALED, the scale) of planes c, c + TPR,
// ... only, at index ci of each plane; the maximum and the sum of exponentials are reduced
// over the group with an xor butterfly (every lane ends with the same values, in a fixed
// order); the weights w_p = e^{lse_p - lse} (times s_p) go to wts[0 .. PMAX) in LDS, where
// every lane of the group reads them, and, when `wraw` is given, the weights without the
// scale to wraw.  Planes at or past P, planes outside the mask `pm`, empty states and row-heads
// that are not `valid` (no loads at all) get weight 0.  An extra state (extra_lse non-null,
// its lse at index xi loaded by lane 0) takes part in the merge with its weight in
// wts[PMAX].  Returns the merged lse (-inf when every state is empty).
// Reduction over the TPR lanes of a row-head group (aligned runs of TPR lanes), every lane
// ending with the result in a fixed order.  With kMergeDpp the lanes exchange values through
// DPP moves inside rows of 16 lanes (quad swaps, then the half-row and row mirrors), else
// through xor shuffles (LDS permute).
template <int TPR, typename Op>
__device__ __forceinline__ float group_reduce(float x, Op op) {
  if constexpr (kMergeDpp && TPR <= 16) {
    auto dpp = [](float v, auto ctrl) {
      return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value, 0xF, 0xF, false));
    };
    if constexpr (TPR >= 2) x = op(x, dpp(x, std::integral_constant<int, 0xB1>{}));   // quad_perm [1,0,3,2]
    if constexpr (TPR >= 4) x = op(x, dpp(x, std::integral_constant<int, 0x4E>{}));   // quad_perm [2,3,0,1]
    if constexpr (TPR >= 8) x = op(x, dpp(x, std::integral_constant<int, 0x141>{}));  // row_half_mirror
    if constexpr (TPR >= 16) x = op(x, dpp(x, std::integral_constant<int, 0x140>{})); // row_mirror
    return x;
  } else {
#pragma unroll
    for (int off = TPR / 2; off >= 1; off >>= 1) x = op(x, __shfl_xor(x, off));
    return x;
  }
}

template <int TPR, int PMAX, bool SCALED>
__device__ __forceinline__ float group_merge_weights(const float *__restrict__ cache_lse,
                                                     const float *__restrict__ cache_scale, int64_t ci,
                                                     int64_t plane_lse, int P, int c, bool valid, float *wts,
                                                     float *wraw, uint64_t pm = ~0ull,
                                                     const float *extra_lse = nullptr, int64_t xi = 0) {
  constexpr int NPL = (PMAX + TPR - 1) / TPR;
  float lv[NPL];
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < NPL; ++k) {
    const int p = c + TPR * k;
    lv[k] = (valid && p < P && ((pm >> p) & 1)) ? cache_lse[p * plane_lse + ci] : -INFINITY;
    M = fmaxf(M, lv[k]);
  }
  const float lx = (valid && extra_lse != nullptr && c == 0) ? extra_lse[xi] : -INFINITY;
  M = fmaxf(M, lx);
  M = group_reduce<TPR>(M, [](float a, float b) { return fmaxf(a, b); });
  float sum = (lx > -INFINITY) ? __expf(lx - M) : 0.f;
#pragma unroll
  for (int k = 0; k < NPL; ++k) sum += (lv[k] > -INFINITY) ? __expf(lv[k] - M) : 0.f;
  sum = group_reduce<TPR>(sum, [](float a, float b) { return a + b; });
  const float L = (M > -INFINITY) ? M + __logf(sum) : -INFINITY;
#pragma unroll
  for (int k = 0; k < NPL; ++k) {
    const int p = c + TPR * k;
    if (p < PMAX) {
      float w = (lv[k] > -INFINITY) ? __expf(lv[k] - L) : 0.f;
      if (wraw != nullptr) wraw[p] = w;
      if constexpr (SCALED) w = (lv[k] > -INFINITY) ? w * cache_scale[p * plane_lse + ci] : 0.f;
      wts[p] = w;
    }
  }
  if (extra_lse != nullptr && c == 0) wts[PMAX] = (lx > -INFINITY) ? __expf(lx - L) : 0.f;
  // the group's lanes are in this wave: LDS accesses of one wave complete in order, and
  // the barrier keeps the compiler from moving the readers' loads above these stores
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  return L;
}

// Importance partials of one merge workgroup: thread p < P sums plane p's unscaled weights
// over the workgroup's row-heads in order (rows that are not valid hold 0) and stores the sum
// at imp_part[p * gridDim.x + w], plane-major so that each (block, plane) reduction reads
// one contiguous run.
template <int RPW, int PMAX>
__device__ __forceinline__ void importance_partials(const float (&wraw)[RPW][PMAX], int P, int w,
                                                    float *__restrict__ imp_part) {
  __syncthreads();
  if ((int)threadIdx.x < P) {
    float s = 0.f;
#pragma unroll 4
    for (int j = 0; j < RPW; ++j) s += wraw[j][threadIdx.x];
    imp_part[(int64_t)threadIdx.x * gridDim.x + w] = s;
  }
}

// One thread per 8 consecutive d of a row-head.  IMP: per-block placement and importance
// partials.  lse_rowmajor: the merged lse goes out as [B, S_q, H] (a cache plane) instead of
// [B, H, S_q].
template <int D, int PMAX, bool IMP>
__global__ __launch_bounds__(256) void state_merge_kernel(
    const u16 *__restrict__ cache_o, const float *__restrict__ cache_lse, u16 *__restrict__ out,
    float *__restrict__ lse_out, const int S_q, const int H, const int P, const int64_t total_rh,
    const int64_t plane_o, const int64_t plane_lse, const int chunk, const int lse_rowmajor, const MergeGrid g,
    float *__restrict__ imp_part) {
  constexpr int TPR = D / 8;
  constexpr int RPW = 256 / TPR;
  const int w = lse_chunked_item(chunk);
  int64_t rh0, rh_end;
  merge_rows<RPW>(g, w, S_q, H, total_rh, rh0, rh_end);
  const int64_t rh = rh0 + threadIdx.x / TPR;
  const bool valid = rh < rh_end;
  if (!IMP && !valid) return;
  const int c = threadIdx.x % TPR;

  __shared__ float wts_all[RPW][PMAX];
  float *wts = wts_all[threadIdx.x / TPR];
  const float L = group_merge_weights<TPR, PMAX, false>(cache_lse, nullptr, rh, plane_lse, P, c, valid, wts, nullptr);

  if (valid) {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    const u16 *src = cache_o + rh * D + 8 * c;
    // kMergeBatch planes' loads in flight together; a short last batch re-reads plane P - 1
    // in place of the missing ones (never added)
#pragma unroll
    for (int p0 = 0; p0 < PMAX; p0 += kMergeBatch) {
      if (p0 < P) {
        u32x4 u[kMergeBatch];
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j)
          u[j] = __builtin_nontemporal_load((const u32x4 *)(src + (int64_t)min(p0 + j, P - 1) * plane_o));
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
          if (p0 + j < P) {
            const float wp = wts[p0 + j];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              acc[2 * t] += wp * bf16_bits_to_f32(u[j][t] & 0xffffu);
              acc[2 * t + 1] += wp * bf16_bits_to_f32(u[j][t] >> 16);
            }
          }
        }
      }
    }
    uint4 res;
    res.x = pack_bf16x2(acc[0], acc[1]);
    res.y = pack_bf16x2(acc[2], acc[3]);
    res.z = pack_bf16x2(acc[4], acc[5]);
    res.w = pack_bf16x2(acc[6], acc[7]);
    __builtin_nontemporal_store(u32x4{res.x, res.y, res.z, res.w}, (u32x4 *)(out + rh * D + 8 * c));
    if (c == 0) {
      const int64_t br = rh / H;
      const int h = (int)(rh - br * H);
      const int64_t b = br / S_q;
      const int64_t r = br - b * S_q;
      lse_out[lse_rowmajor ? rh : (b * H + h) * S_q + r] = L;
    }
  }
  if constexpr (IMP) importance_partials<RPW, PMAX>(wts_all, P, w, imp_part);
}

// State merge over the compressed cache: per row-head, plane p holds e4m3 codes and a scale
// s_p; the scale folds into the merge weight, w_p = s_p e^{lse_p - lse}.  One thread per
// kFp8Dpt consecutive d (kFp8Dpt-byte code loads, non-temporal; bf16 output stores).
constexpr int kFp8Dpt = DIT_MERGE_FP8_DPT;
template <int D, int PMAX, bool IMP>
__global__ __launch_bounds__(256) void state_merge_fp8_kernel(
    const uint8_t *__restrict__ cache_q8, const float *__restrict__ cache_scale,
    const float *__restrict__ cache_lse, u16 *__restrict__ out, float *__restrict__ lse_out,
    const int S_q, const int H, const int P, const int64_t total_rh, const int64_t plane_o,
    const int64_t plane_lse, const int chunk, const MergeGrid g, float *__restrict__ imp_part) {
  constexpr int TPR = D / kFp8Dpt;
  constexpr int RPW = 256 / TPR;
  constexpr int NW = kFp8Dpt / 4;  // 32-bit code words per thread and plane
  const int w = lse_chunked_item(chunk);
  int64_t rh0, rh_end;
  merge_rows<RPW>(g, w, S_q, H, total_rh, rh0, rh_end);
  const int64_t rh = rh0 + threadIdx.x / TPR;
  const bool valid = rh < rh_end;
  if (!IMP && !valid) return;
  const int c = threadIdx.x % TPR;

  __shared__ float wts_all[RPW][PMAX];
  __shared__ float wraw_all[IMP ? RPW : 1][IMP ? PMAX : 1];
  float *wts = wts_all[threadIdx.x / TPR];
  const float L = group_merge_weights<TPR, PMAX, true>(cache_lse, cache_scale, rh, plane_lse, P, c, valid, wts,
                                                       IMP ? &wraw_all[threadIdx.x / TPR][0] : nullptr);

  if (valid) {
    float acc[kFp8Dpt];
#pragma unroll
    for (int e = 0; e < kFp8Dpt; ++e) acc[e] = 0.f;
    const uint8_t *src = cache_q8 + rh * D + kFp8Dpt * c;
    // kMergeBatch planes' loads in flight together (as in state_merge_kernel)
#pragma unroll
    for (int p0 = 0; p0 < PMAX; p0 += kMergeBatch) {
      if (p0 < P) {
        uint32_t u[kMergeBatch][NW];
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
          const uint8_t *sp = src + (int64_t)min(p0 + j, P - 1) * plane_o;
          if constexpr (NW >= 4) {
#pragma unroll
            for (int q = 0; q < NW / 4; ++q) {
              const u32x4 v4 = __builtin_nontemporal_load((const u32x4 *)sp + q);
              u[j][4 * q + 0] = v4[0];
              u[j][4 * q + 1] = v4[1];
              u[j][4 * q + 2] = v4[2];
              u[j][4 * q + 3] = v4[3];
            }
          } else {
            const u32x2 v2 = __builtin_nontemporal_load((const u32x2 *)sp);
            u[j][0] = v2[0];
            u[j][1] = v2[1];
          }
        }
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
          if (p0 + j < P) {
            const float wp = wts[p0 + j];
#pragma unroll
            for (int t = 0; t < NW; ++t) {
              const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)u[j][t], false);
              const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)u[j][t], true);
              acc[4 * t + 0] += wp * lo[0];
              acc[4 * t + 1] += wp * lo[1];
              acc[4 * t + 2] += wp * hi[0];
              acc[4 * t + 3] += wp * hi[1];
            }
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kFp8Dpt / 8; ++q)
      __builtin_nontemporal_store(u32x4{pack_bf16x2(acc[8 * q + 0], acc[8 * q + 1]), pack_bf16x2(acc[8 * q + 2], acc[8 * q + 3]),
                                        pack_bf16x2(acc[8 * q + 4], acc[8 * q + 5]), pack_bf16x2(acc[8 * q + 6], acc[8 * q + 7])},
                                  (u32x4 *)(out + rh * D + kFp8Dpt * c + 8 * q));
    if (c == 0) {
      const int64_t br = rh / H;
      const int h = (int)(rh - br * H);
      const int64_t b = br / S_q;
      const int64_t r = br - b * S_q;
      lse_out[(b * H + h) * S_q + r] = L;
    }
  }
  if constexpr (IMP) importance_partials<RPW, PMAX>(wraw_all, P, w, imp_part);
}

// Masked merge of one row-head rh by its TPR lanes (this lane is number c of them): the
// cache planes in pm, in increasing order, plus the extra state when extra_lse is non-null
// (a partial composition made earlier, its lse in the [B, H, S_q] layout of a merged output,
// at index xi, which is also where the merged lse goes).  wts: the group's PMAX + 1 weights
// in LDS.  out / lse_out may be the extra state itself (every lane reads the extra values it
// then overwrites, and no others), so those four pointers are not restrict-qualified.
template <int D, int PMAX>
__device__ __forceinline__ void masked_merge_rowhead(const u16 *__restrict__ cache_o,
                                                     const float *__restrict__ cache_lse,
                                                     const u16 *extra_o, const float *extra_lse, u16 *out,
                                                     float *lse_out, const int64_t rh,
                                                     const int64_t xi, const uint64_t pm, const int P,
                                                     const int64_t plane_o, const int64_t plane_lse, const int c,
                                                     float *wts) {
  constexpr int TPR = D / 8;
  const float L = group_merge_weights<TPR, PMAX, false>(cache_lse, nullptr, rh, plane_lse, P, c, true, wts, nullptr,
                                                        pm, extra_lse, xi);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  auto add = [&](const u16 *src, float w) {
    const u32x4 u = __builtin_nontemporal_load((const u32x4 *)src);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      acc[2 * t] += w * bf16_bits_to_f32(u[t] & 0xffffu);
      acc[2 * t + 1] += w * bf16_bits_to_f32(u[t] >> 16);
    }
  };
  const u16 *src = cache_o + rh * D + 8 * c;
  // the selected planes in increasing order, NB loads in flight at a time; a short last
  // batch re-reads its first plane in place of the missing ones (never added)
  constexpr int NB = PMAX < kMaskedMergeBatch ? PMAX : kMaskedMergeBatch;
  uint64_t rest = pm & (P < 64 ? ((uint64_t)1 << P) - 1 : ~(uint64_t)0);
  while (rest) {
    int pi[NB];
    pi[0] = __builtin_ctzll(rest);
    rest &= rest - 1;
    int n = 1;
#pragma unroll
    for (int j = 1; j < NB; ++j) {
      pi[j] = pi[0];
      if (rest) {
        pi[j] = __builtin_ctzll(rest);
        rest &= rest - 1;
        n = j + 1;
      }
    }
    u32x4 u[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) u[j] = __builtin_nontemporal_load((const u32x4 *)(src + (int64_t)pi[j] * plane_o));
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (j < n) {
        const float w = wts[pi[j]];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          acc[2 * t] += w * bf16_bits_to_f32(u[j][t] & 0xffffu);
          acc[2 * t + 1] += w * bf16_bits_to_f32(u[j][t] >> 16);
        }
      }
    }
  }
  if (extra_lse != nullptr) add(extra_o + rh * D + 8 * c, wts[PMAX]);
  uint4 res;
  res.x = pack_bf16x2(acc[0], acc[1]);
  res.y = pack_bf16x2(acc[2], acc[3]);
  res.z = pack_bf16x2(acc[4], acc[5]);
  res.w = pack_bf16x2(acc[6], acc[7]);
  __builtin_nontemporal_store(u32x4{res.x, res.y, res.z, res.w}, (u32x4 *)(out + rh * D + 8 * c));
  if (c == 0) lse_out[xi] = L;
}

// Block of query row r: the last i with q_off[i] <= r.
__device__ __forceinline__ int block_of_row(const int32_t *q_off, int n_qb, int r) {
  int lo = 0, hi = n_qb - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (q_off[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Masked merge: as state_merge_kernel, but row r of query block i combines only the planes
// selected for block i, plus an optional extra state (a partial composition made earlier,
// its lse in the [B, H, S_q] layout of a merged output).
// Used to pre-merge the reused states on a second stream while the attention kernel
// recomputes the others, and to finish with the fresh states and that partial.
template <int D, int PMAX>
__global__ __launch_bounds__(256) void state_merge_masked_kernel(
    const u16 *__restrict__ cache_o, const float *__restrict__ cache_lse, const u16 *extra_o,
    const float *extra_lse, const MergeSelect sel, u16 *out, float *lse_out, const int S_q, const int H,
    const int P, const int64_t total_rh,
    const int64_t plane_o, const int64_t plane_lse, const int chunk) {
  constexpr int TPR = D / 8;
  constexpr int RPW = 256 / TPR;
  const int64_t rh = (int64_t)lse_chunked_item(chunk) * RPW + threadIdx.x / TPR;
  if (rh >= total_rh) return;
  const int c = threadIdx.x % TPR;
  const int64_t br = rh / H;
  const int h = (int)(rh - br * H);
  const int64_t b = br / S_q;
  const int r = (int)(br - b * S_q);
  const uint64_t pm = sel.plane_mask[block_of_row(sel.q_off, sel.n_qb, r)];
  __shared__ float wts_all[RPW][PMAX + 1];
  masked_merge_rowhead<D, PMAX>(cache_o, cache_lse, extra_o, sel.has_extra ? extra_lse : nullptr, out, lse_out, rh,
                                (b * H + h) * S_q + r, pm, P, plane_o, plane_lse, c, wts_all[threadIdx.x / TPR]);
}

// ------------------------------------------------------------------------------------
// Partition attention with the reuse work in its tail.  The launch carries the attention
// items' workgroups first and then tm.n_tail_wg more; the dispatcher hands workgroups out in
// order, so the extra ones start only once every attention item has started, in the slots
// that attention workgroups leave as the launch drains (the XCDs do not finish together).
// Each extra workgroup claims chunks of row-heads from the counter tm.claim (zero at the
// launch) until none is left, and merges, for every row-head of a chunk, the cache planes
// its query block reuses (tm.reuse_mask) into the partial state pre_o / pre_lse: the
// masked merge, on planes that this launch does not write.  Chunks are claimed in order, so
// the XCDs that run out of attention items first take more of them.
// ------------------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void premerge_chunks(const u16 *__restrict__ cache_o, const float *__restrict__ cache_lse,
                                                const AttnDesc &desc, const TailMerge &tm) {
  constexpr int TPR = D / 8;
  constexpr int RPW = kWaves * 64 / TPR;  // row-heads per pass of the workgroup
  constexpr int PMAX = DIT_MAX_PARTITIONS;
  __shared__ float wts_all[RPW][PMAX + 1];
  __shared__ uint32_t claimed;
  const int S_q = desc.S_q, H = desc.H;
  const int64_t total_rh = (int64_t)desc.B * S_q * H;
  const int64_t plane_o = total_rh * D;
  const int c = threadIdx.x % TPR;
  float *wts = wts_all[threadIdx.x / TPR];
  u16 *pre_o = (u16 *)tm.pre_o;
  for (;;) {
    if (threadIdx.x == 0) claimed = __hip_atomic_fetch_add(tm.claim, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint32_t ch = claimed;
    __syncthreads();  // every thread has read it before the next claim overwrites it
    if (ch >= (uint32_t)tm.n_chunks) return;
    const int64_t rh_first = (int64_t)ch * tm.chunk_passes * RPW + threadIdx.x / TPR;
    for (int j = 0; j < tm.chunk_passes; ++j) {
      const int64_t rh = rh_first + (int64_t)j * RPW;
      if (rh >= total_rh) break;
      const int64_t br = rh / H;
      const int h = (int)(rh - br * H);
      const int64_t b = br / S_q;
      const int r = (int)(br - b * S_q);
      const uint64_t pm = tm.reuse_mask[block_of_row(desc.q_off, desc.n_qb, r)];
      masked_merge_rowhead<D, PMAX>(cache_o, cache_lse, nullptr, nullptr, pre_o, tm.pre_lse, rh,
                                    (b * H + h) * S_q + r, pm, desc.P, plane_o, total_rh, c, wts);
    }
  }
}

template <int D>
__global__ __launch_bounds__(kWaves * 64, kMinBlocks) void partition_attention_premerge_kernel(
    const u16 *__restrict__ q, const u16 *__restrict__ k, const u16 *__restrict__ v, void *__restrict__ cache_o,
    float *__restrict__ cache_lse, float *__restrict__ delta_part, const AttnDesc desc, const float scale_log2,
    const TailMerge tm) {
  if ((int)blockIdx.x >= tm.n_attn_wg) {
    premerge_chunks<D>((const u16 *)cache_o, cache_lse, desc, tm);
    return;
  }
  attention_item<D, false>(q, k, v, cache_o, nullptr, cache_lse, delta_part, desc, scale_log2, tm.n_attn_wg,
                           blockIdx.x);
}

__global__ void clear_claim_kernel(uint32_t *claim) {
  if (threadIdx.x == 0) *claim = 0u;
}

template <int D>
hipError_t merge_masked_dispatch(int P, const void *cache_o, const float *cache_lse, const void *extra_o,
                                 const float *extra_lse, const MergeSelect &sel, void *out, float *lse,
                                 int B, int S_q, int H, hipStream_t stream) {
  const int64_t total_rh = (int64_t)B * S_q * H;
  if (total_rh == 0) return hipSuccess;
  constexpr int RPW = 256 / (D / 8);
  const int64_t nwg = (total_rh + RPW - 1) / RPW;
  const int64_t plane_o = total_rh * D;
  const int64_t plane_lse = total_rh;
  const int chunk = merge_chunk(RPW, H);
  dim3 grid((unsigned)nwg), block(256);
  const u16 *co = (const u16 *)cache_o;
  const u16 *eo = (const u16 *)extra_o;
  u16 *oo = (u16 *)out;
  if (P <= 8)
    hipLaunchKernelGGL((state_merge_masked_kernel<D, 8>), grid, block, 0, stream, co, cache_lse, eo, extra_lse, sel, oo, lse, S_q, H, P, total_rh, plane_o, plane_lse, chunk);
  else if (P <= 16)
    hipLaunchKernelGGL((state_merge_masked_kernel<D, 16>), grid, block, 0, stream, co, cache_lse, eo, extra_lse, sel, oo, lse, S_q, H, P, total_rh, plane_o, plane_lse, chunk);
  else if (P <= 32)
    hipLaunchKernelGGL((state_merge_masked_kernel<D, 32>), grid, block, 0, stream, co, cache_lse, eo, extra_lse, sel, oo, lse, S_q, H, P, total_rh, plane_o, plane_lse, chunk);
  else
    hipLaunchKernelGGL((state_merge_masked_kernel<D, 64>), grid, block, 0, stream, co, cache_lse, eo, extra_lse, sel, oo, lse, S_q, H, P, total_rh, plane_o, plane_lse, chunk);
  return hipGetLastError();
}

// Fixed-order tree reduction of one float per thread over a 256-thread workgroup.
__device__ __forceinline__ float block_sum_256(float x, float *sh) {
  sh[threadIdx.x] = x;
  __syncthreads();
#pragma unroll
  for (int s = 128; s >= 1; s >>= 1) {
    if ((int)threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
    __syncthreads();
  }
  return sh[0];
}

// Importance from the stored lse planes (a second pass, for callers without a workspace):
// one workgroup of 1024 threads per (batch, block i, partition p).  Each thread walks the
// block's row-heads e = (r - q_off[i]) H + h with four independent loads in flight (e,
// e + 1024, e + 2048, e + 3072): cache_lse of the plane is contiguous over e, the merged lse
// [B, H, S_q] is gathered.  A fixed-order tree sums the threads.
constexpr int kImpThreads = 1024;
__device__ __forceinline__ float block_sum_1024(float x, float *sh) {
  sh[threadIdx.x] = x;
  __syncthreads();
#pragma unroll
  for (int s = kImpThreads / 2; s >= 1; s >>= 1) {
    if ((int)threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
    __syncthreads();
  }
  return sh[0];
}

__global__ __launch_bounds__(kImpThreads) void importance_kernel(
    const float *__restrict__ cache_lse, const float *__restrict__ lse, const int S_q, const int H,
    const int P, const int B, const BlockDesc blocks, float *__restrict__ out) {
  __shared__ float sh[kImpThreads];
  const int p = blockIdx.x % P;
  const int i = blockIdx.x / P;
  const int b = blockIdx.y;
  const int r0 = blocks.q_off[i];
  const int nr = blocks.q_off[i + 1] - r0;
  const int64_t n = (int64_t)nr * H;
  const float *cl = cache_lse + (((int64_t)p * B + b) * S_q + r0) * H;
  const float *ml = lse + (int64_t)b * H * S_q + r0;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int64_t e = threadIdx.x; e < n; e += 4 * kImpThreads) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t ee = e + u * kImpThreads;
      if (ee < n) {
        const int r = (int)(ee / H);
        const int h = (int)(ee - (int64_t)r * H);
        const float a = cl[ee];
        const float t = ml[(int64_t)h * S_q + r];
        acc[u] += (a > -INFINITY && t > -INFINITY) ? __expf(a - t) : 0.f;
      }
    }
  }
  const float tot = block_sum_1024((acc[0] + acc[1]) + (acc[2] + acc[3]), sh);
  if (threadIdx.x == 0) out[((int64_t)b * blocks.n_qb + i) * P + p] = n > 0 ? tot / (float)n : 0.f;
}

// Importance from the merge's partials: one workgroup per (batch, block i, partition p) sums
// plane p's partials of block i's merge workgroups (a contiguous run) in a fixed order.
__global__ __launch_bounds__(256) void importance_finalize_kernel(const float *__restrict__ part, const int P,
                                                                  const int H, const int nwg, const MergeGrid g,
                                                                  float *__restrict__ out) {
  __shared__ float sh[256];
  const int p = blockIdx.x % P;
  const int i = blockIdx.x / P;
  const int b = blockIdx.y;
  const int w0 = b * g.wg_per_batch + g.wg_prefix[i];
  const int w1 = b * g.wg_per_batch + g.wg_prefix[i + 1];
  const float *src = part + (int64_t)p * nwg;
  float acc = 0.f;
  for (int w = w0 + (int)threadIdx.x; w < w1; w += 256) acc += src[w];
  const float tot = block_sum_256(acc, sh);
  const int64_t n = (int64_t)(g.q_off[i + 1] - g.q_off[i]) * H;
  if (threadIdx.x == 0) out[((int64_t)b * g.n_qb + i) * P + p] = tot / (float)n;
}

// Local change: one workgroup per (batch, block i) sums the (tile, head) partials.
__global__ __launch_bounds__(256) void delta_finalize_kernel(const float *__restrict__ part,
                                                             const int H, const BlockDesc blocks,
                                                             float *__restrict__ out) {
  __shared__ float sh[256];
  const int i = blockIdx.x;
  const int b = blockIdx.y;
  const int64_t e0 = (int64_t)blocks.tile_prefix[i] * H;
  const int64_t e1 = (int64_t)blocks.tile_prefix[i + 1] * H;
  const float *base = part + (int64_t)b * blocks.n_tiles * H * 2;
  float num = 0.f, den = 0.f;
  for (int64_t e = e0 + threadIdx.x; e < e1; e += 256) {
    num += base[2 * e];
    den += base[2 * e + 1];
  }
  const float tn = block_sum_256(num, sh);
  __syncthreads();
  const float td = block_sum_256(den, sh);
  if (threadIdx.x == 0) out[(int64_t)b * blocks.n_qb + i] = sqrtf(tn) / sqrtf(td);
}

// Placement of a merge launch: plain over all row-heads, or per block when importance
// partials are wanted (imp_blocks non-null).
MergeGrid make_merge_grid(int RPW, const BlockDesc *imp_blocks, int B, int S_q, int H, int64_t &nwg) {
  MergeGrid g;
  memset(&g, 0, sizeof(g));
  const int64_t total_rh = (int64_t)B * S_q * H;
  if (imp_blocks == nullptr) {
    nwg = (total_rh + RPW - 1) / RPW;
    return g;
  }
  g.n_qb = imp_blocks->n_qb;
  for (int i = 0; i <= g.n_qb; ++i) g.q_off[i] = imp_blocks->q_off[i];
  for (int i = 0; i < g.n_qb; ++i) {
    const int64_t n = (int64_t)(g.q_off[i + 1] - g.q_off[i]) * H;
    g.wg_prefix[i + 1] = g.wg_prefix[i] + (int32_t)((n + RPW - 1) / RPW);
  }
  g.wg_per_batch = g.wg_prefix[g.n_qb];
  nwg = (int64_t)B * g.wg_per_batch;
  return g;
}

hipError_t launch_importance_finalize(const float *imp_part, int P, int H, int B, int64_t nwg, const MergeGrid &g,
                                      float *importance_out, hipStream_t stream) {
  dim3 grid((unsigned)(g.n_qb * P), (unsigned)B), block(256);
  hipLaunchKernelGGL(importance_finalize_kernel, grid, block, 0, stream, imp_part, P, H, (int)nwg, g,
                     importance_out);
  return hipGetLastError();
}

template <int D, bool IMP>
hipError_t merge_dispatch(int P, const void *cache_o, const float *cache_lse, void *out, float *lse, int B,
                          int S_q, int H, bool lse_rowmajor, const BlockDesc *imp_blocks, float *imp_part,
                          float *importance_out, hipStream_t stream) {
  const int64_t total_rh = (int64_t)B * S_q * H;
  if (total_rh == 0) return hipSuccess;
  constexpr int RPW = 256 / (D / 8);
  int64_t nwg = 0;
  const MergeGrid g = make_merge_grid(RPW, IMP ? imp_blocks : nullptr, B, S_q, H, nwg);
  const int64_t plane_o = total_rh * D;
  const int64_t plane_lse = total_rh;
  const int chunk = merge_chunk(RPW, H);
  dim3 grid((unsigned)nwg), block(256);
  const u16 *co = (const u16 *)cache_o;
  u16 *oo = (u16 *)out;
  const int rm = lse_rowmajor ? 1 : 0;
  if (P <= 8)
    hipLaunchKernelGGL((state_merge_kernel<D, 8, IMP>), grid, block, 0, stream, co, cache_lse, oo, lse, S_q, H, P, total_rh, plane_o, plane_lse, chunk, rm, g, imp_part);
  else if (P <= 16)
    hipLaunchKernelGGL((state_merge_kernel<D, 16, IMP>), grid, block, 0, stream, co, cache_lse, oo, lse, S_q, H, P, total_rh, plane_o, plane_lse, chunk, rm, g, imp_part);
  else if (P <= 32)
    hipLaunchKernelGGL((state_merge_kernel<D, 32, IMP>), grid, block, 0, stream, co, cache_lse, oo, lse, S_q, H, P, total_rh, plane_o, plane_lse, chunk, rm, g, imp_part);
  else
    hipLaunchKernelGGL((state_merge_kernel<D, 64, IMP>), grid, block, 0, stream, co, cache_lse, oo, lse, S_q, H, P, total_rh, plane_o, plane_lse, chunk, rm, g, imp_part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !IMP) return e;
  return launch_importance_finalize(imp_part, P, H, B, nwg, g, importance_out, stream);
}

template <int D, bool IMP>
hipError_t merge_fp8_dispatch(int P, const void *cache_q8, const float *cache_scale, const float *cache_lse,
                              void *out, float *lse, int B, int S_q, int H, const BlockDesc *imp_blocks,
                              float *imp_part, float *importance_out, hipStream_t stream) {
  const int64_t total_rh = (int64_t)B * S_q * H;
  if (total_rh == 0) return hipSuccess;
  constexpr int RPW = 256 / (D / kFp8Dpt);
  int64_t nwg = 0;
  const MergeGrid g = make_merge_grid(RPW, IMP ? imp_blocks : nullptr, B, S_q, H, nwg);
  const int64_t plane_o = total_rh * D;
  const int64_t plane_lse = total_rh;
  const int chunk = merge_chunk(RPW, H);
  dim3 grid((unsigned)nwg), block(256);
  const uint8_t *cq = (const uint8_t *)cache_q8;
  u16 *oo = (u16 *)out;
  if (P <= 8)
    hipLaunchKernelGGL((state_merge_fp8_kernel<D, 8, IMP>), grid, block, 0, stream, cq, cache_scale, cache_lse, oo, lse, S_q, H, P, total_rh, plane_o, plane_lse, chunk, g, imp_part);
  else if (P <= 16)
    hipLaunchKernelGGL((state_merge_fp8_kernel<D, 16, IMP>), grid, block, 0, stream, cq, cache_scale, cache_lse, oo, lse, S_q, H, P, total_rh, plane_o, plane_lse, chunk, g, imp_part);
  else if (P <= 32)
    hipLaunchKernelGGL((state_merge_fp8_kernel<D, 32, IMP>), grid, block, 0, stream, cq, cache_scale, cache_lse, oo, lse, S_q, H, P, total_rh, plane_o, plane_lse, chunk, g, imp_part);
  else
    hipLaunchKernelGGL((state_merge_fp8_kernel<D, 64, IMP>), grid, block, 0, stream, cq, cache_scale, cache_lse, oo, lse, S_q, H, P, total_rh, plane_o, plane_lse, chunk, g, imp_part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !IMP) return e;
  return launch_importance_finalize(imp_part, P, H, B, nwg, g, importance_out, stream);
}

}  // namespace

int64_t merge_workgroups(int D, bool fp8_cache, const BlockDesc *imp_blocks, int B, int S_q, int H) {
  const int rpw = fp8_cache ? 256 / (D / kFp8Dpt) : 256 / (D / 8);
  int64_t nwg = 0;
  make_merge_grid(rpw, imp_blocks, B, S_q, H, nwg);
  return nwg;
}

hipError_t launch_partition_attention(int D, bool fp8_cache, const void *q, const void *k, const void *v,
                                      void *cache_o, float *cache_scale, float *cache_lse, float *delta_partials,
                                      const AttnDesc &desc, float scale_log2, hipStream_t stream) {
  const int64_t nwg = (int64_t)desc.B * desc.H * desc.items_per_head;
  if (nwg == 0) return hipSuccess;
  (void)hipGetLastError();
  dim3 grid((unsigned)nwg), block(kWaves * 64);
  const u16 *qq = (const u16 *)q, *kk = (const u16 *)k, *vv = (const u16 *)v;
  if (D == 128 && !fp8_cache)
    hipLaunchKernelGGL((partition_attention_kernel<128, false>), grid, block, 0, stream, qq, kk, vv, cache_o, cache_scale,
                       cache_lse, delta_partials, desc, scale_log2);
  else if (D == 128)
    hipLaunchKernelGGL((partition_attention_kernel<128, true>), grid, block, 0, stream, qq, kk, vv, cache_o, cache_scale,
                       cache_lse, delta_partials, desc, scale_log2);
  else if (!fp8_cache)
    hipLaunchKernelGGL((partition_attention_kernel<64, false>), grid, block, 0, stream, qq, kk, vv, cache_o, cache_scale,
                       cache_lse, delta_partials, desc, scale_log2);
  else
    hipLaunchKernelGGL((partition_attention_kernel<64, true>), grid, block, 0, stream, qq, kk, vv, cache_o, cache_scale,
                       cache_lse, delta_partials, desc, scale_log2);
  return hipGetLastError();
}

hipError_t launch_partition_attention_premerge(int D, const void *q, const void *k, const void *v, void *cache_o,
                                               float *cache_lse, float *delta_partials, const AttnDesc &desc,
                                               float scale_log2, const TailMerge &tm, hipStream_t stream) {
  (void)hipGetLastError();
  hipLaunchKernelGGL(clear_claim_kernel, dim3(1), dim3(64), 0, stream, tm.claim);
  const int64_t nwg = (int64_t)tm.n_attn_wg + tm.n_tail_wg;
  if (nwg == 0) return hipGetLastError();
  dim3 grid((unsigned)nwg), block(kWaves * 64);
  const u16 *qq = (const u16 *)q, *kk = (const u16 *)k, *vv = (const u16 *)v;
  if (D == 128)
    hipLaunchKernelGGL((partition_attention_premerge_kernel<128>), grid, block, 0, stream, qq, kk, vv, cache_o,
                       cache_lse, delta_partials, desc, scale_log2, tm);
  else
    hipLaunchKernelGGL((partition_attention_premerge_kernel<64>), grid, block, 0, stream, qq, kk, vv, cache_o,
                       cache_lse, delta_partials, desc, scale_log2, tm);
  return hipGetLastError();
}

hipError_t launch_state_merge_fp8(int D, int P, const void *cache_q8, const float *cache_scale,
                                  const float *cache_lse, void *out, float *lse, int B, int S_q, int H,
                                  const BlockDesc *imp_blocks, float *imp_part, float *importance_out,
                                  hipStream_t stream) {
  (void)hipGetLastError();
  const bool imp = imp_blocks != nullptr;
  if (D == 128)
    return imp ? merge_fp8_dispatch<128, true>(P, cache_q8, cache_scale, cache_lse, out, lse, B, S_q, H, imp_blocks, imp_part, importance_out, stream)
               : merge_fp8_dispatch<128, false>(P, cache_q8, cache_scale, cache_lse, out, lse, B, S_q, H, nullptr, nullptr, nullptr, stream);
  return imp ? merge_fp8_dispatch<64, true>(P, cache_q8, cache_scale, cache_lse, out, lse, B, S_q, H, imp_blocks, imp_part, importance_out, stream)
             : merge_fp8_dispatch<64, false>(P, cache_q8, cache_scale, cache_lse, out, lse, B, S_q, H, nullptr, nullptr, nullptr, stream);
}

hipError_t launch_state_merge(int D, int P, const void *cache_o, const float *cache_lse, void *out,
                              float *lse, int B, int S_q, int H, bool lse_rowmajor, const BlockDesc *imp_blocks,
                              float *imp_part, float *importance_out, hipStream_t stream) {
  (void)hipGetLastError();
  const bool imp = imp_blocks != nullptr;
  if (D == 128)
    return imp ? merge_dispatch<128, true>(P, cache_o, cache_lse, out, lse, B, S_q, H, lse_rowmajor, imp_blocks, imp_part, importance_out, stream)
               : merge_dispatch<128, false>(P, cache_o, cache_lse, out, lse, B, S_q, H, lse_rowmajor, nullptr, nullptr, nullptr, stream);
  return imp ? merge_dispatch<64, true>(P, cache_o, cache_lse, out, lse, B, S_q, H, lse_rowmajor, imp_blocks, imp_part, importance_out, stream)
             : merge_dispatch<64, false>(P, cache_o, cache_lse, out, lse, B, S_q, H, lse_rowmajor, nullptr, nullptr, nullptr, stream);
}

hipError_t launch_state_merge_masked(int D, int P, const void *cache_o, const float *cache_lse,
                                     const void *extra_o, const float *extra_lse, const MergeSelect &sel,
                                     void *out, float *lse, int B, int S_q, int H, hipStream_t stream) {
  (void)hipGetLastError();
  if (D == 128)
    return merge_masked_dispatch<128>(P, cache_o, cache_lse, extra_o, extra_lse, sel, out, lse, B, S_q, H, stream);
  return merge_masked_dispatch<64>(P, cache_o, cache_lse, extra_o, extra_lse, sel, out, lse, B, S_q, H, stream);
}

hipError_t launch_importance(const float *cache_lse, const float *lse, int B, int S_q, int H, int P,
                             const BlockDesc &blocks, float *importance_out, hipStream_t stream) {
  (void)hipGetLastError();
  dim3 grid((unsigned)(blocks.n_qb * P), (unsigned)B), block(kImpThreads);
  hipLaunchKernelGGL(importance_kernel, grid, block, 0, stream, cache_lse, lse, S_q, H, P, B, blocks,
                     importance_out);
  return hipGetLastError();
}

hipError_t launch_delta_finalize(const float *partials, int B, int H, const BlockDesc &blocks,
                                 float *delta_out, hipStream_t stream) {
  (void)hipGetLastError();
  dim3 grid((unsigned)blocks.n_qb, (unsigned)B), block(256);
  hipLaunchKernelGGL(delta_finalize_kernel, grid, block, 0, stream, partials, H, blocks, delta_out);
  return hipGetLastError();
}

// Scratch of the allocation-free entry point.  Each GPU holds its own copy at its own
// address; in host code `scratch` names a host-side stand-in, so kernels get the device
// address from hipGetSymbolAddress instead, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices];
}  // namespace

hipError_t scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace dit
