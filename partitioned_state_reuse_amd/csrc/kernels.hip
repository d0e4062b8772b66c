// HIP kernels for gfx950 (CDNA4): partition attention with state-cache update, state merge,
// partition importance, and the local-change reduction.
//
// The operation follows "DiTango: Cost-Effective Parallel Diffusion Generation with
// Selective Attention State Reuse" (technical summary, "Methodology §2, State Composition"
// and "§1, Anchor-Guided Selection Planner"): per KV partition an attention state
// (O_p, lse_p) is produced; the states are composed by LSE-weighted combination.
#include <math.h>

#include "launch.h"

namespace dit {
namespace {

typedef unsigned short u16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

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
// One workgroup = 4 waves = one (batch, head, partition p, query tile of <= 128 rows of
// one query block).  Each wave owns 32 query rows and keeps them in registers as the B
// operand of S^T = K Q^T (v_mfma_f32_32x32x16_bf16), so that each lane's 16 scores
// belong to one query and the softmax reductions over keys stay mostly inside a lane.
// K tiles of 64 keys are staged in LDS row-major; V tiles are staged transposed (d-major)
// so that V^T is the A operand of O^T = V^T P^T, with P^T taken straight from the score
// registers (the key order inside each 16-key MFMA step is permuted identically on both
// operands).  Online softmax in base 2 with fp32 state; P is rounded to bf16 for the
// product.  The epilogue writes the partition's state into its cache slot and, for a
// block's local partition, the partial sums of the local-change norm.
// ------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void partition_attention_kernel(
    const u16 *__restrict__ q, const u16 *__restrict__ k, const u16 *__restrict__ v,
    u16 *__restrict__ cache_o, float *__restrict__ cache_lse, float *__restrict__ delta_part,
    const AttnDesc desc, const float scale_log2) {
  constexpr int KK = D / 16;       // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;       // 32-row blocks of O^T
  constexpr int KS = D + 8;        // LDS row stride (elements) of the K tile
  constexpr int VS = kBlockN + 4;  // LDS row stride (elements) of the transposed V tile
  __shared__ __attribute__((aligned(16))) u16 Ks[kBlockN * KS];
  __shared__ __attribute__((aligned(16))) u16 Vt[D * VS];
  __shared__ float red[8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- work item.  Workgroups are dealt round-robin to the 8 XCDs; remap so that
  // consecutive items (same K/V partition) run on the same XCD and share its L2.
  const int nwg = gridDim.x;
  const int wg = blockIdx.x;
  const int xcd = wg & 7, per = nwg >> 3, rem = nwg & 7;
  const int item = xcd * per + min(xcd, rem) + (wg >> 3);
  const int per_head = desc.items_per_head;
  const int bh = item / per_head;
  int idx = item - bh * per_head;
  const int H = desc.H;
  const int b = bh / H;
  const int head = bh - b * H;
  int p = 0;
  while (desc.item_prefix[p + 1] <= idx) ++p;
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
  const int64_t rowstride = (int64_t)H * D;

  // ---- this lane's query row, as the B operand: Q[row][16 kk + 8 hh + 0..7]
  const int qrow = wave * 32 + l32;
  const bool qvalid = qrow < qn;
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

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  const u16 *kbase = k + ((int64_t)b * desc.S_kv + kv0) * rowstride + (int64_t)head * D;
  const u16 *vbase = v + ((int64_t)b * desc.S_kv + kv0) * rowstride + (int64_t)head * D;
  const int ntiles = (kvn + kBlockN - 1) / kBlockN;

  for (int kt = 0; kt < ntiles; ++kt) {
    const int key0 = kt * kBlockN;
    const int nvalid = min(kBlockN, kvn - key0);
    // ---- stage K rows [key][d]; rows past the partition end are zero
    {
      constexpr int CPR = D / 8;
      constexpr int RPP = 256 / CPR;
      const int c = tid % CPR;
#pragma unroll
      for (int pass = 0; pass < kBlockN / RPP; ++pass) {
        const int r = tid / CPR + pass * RPP;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (r < nvalid) val = *(const uint4 *)(kbase + (int64_t)(key0 + r) * rowstride + 8 * c);
        *(uint4 *)(Ks + r * KS + 8 * c) = val;
      }
    }
    // ---- stage V transposed [d][key]: each thread loads KPT consecutive keys of one
    // 8-wide d chunk and writes, per d, their KPT values as one LDS store
    {
      constexpr int KPT = D / 32;
      constexpr int KG = kBlockN / KPT;
      const int kg = tid % KG;
      const int dc = tid / KG;
      uint4 val[KPT];
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int key = kg * KPT + j;
        val[j] = make_uint4(0, 0, 0, 0);
        if (key < nvalid) val[j] = *(const uint4 *)(vbase + (int64_t)(key0 + key) * rowstride + 8 * dc);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t w[KPT / 2];
#pragma unroll
        for (int j2 = 0; j2 < KPT / 2; ++j2) {
          const uint32_t a0 = ((const uint32_t *)&val[2 * j2])[e >> 1];
          const uint32_t a1 = ((const uint32_t *)&val[2 * j2 + 1])[e >> 1];
          const uint32_t lo = (e & 1) ? (a0 >> 16) : (a0 & 0xffffu);
          const uint32_t hi = (e & 1) ? (a1 >> 16) : (a1 & 0xffffu);
          w[j2] = lo | (hi << 16);
        }
        u16 *dst = Vt + (8 * dc + e) * VS + kg * KPT;
        if constexpr (KPT == 4) {
          *(uint2 *)dst = make_uint2(w[0], w[1]);
        } else {
          *(uint32_t *)dst = w[0];
        }
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T for keys [32 mb, 32 mb + 32)
    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mb][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8 a = as_bf16x8(*(const uint4 *)(Ks + (32 * mb + l32) * KS + 16 * kk + 8 * hh));
        s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[mb], 0, 0, 0);
      }
    }

    // ---- scale into base 2; mask keys past the partition end.  s[mb][r] holds key
    // 32 mb + (r & 3) + 8 (r >> 2) + 4 hh of the tile for query row l32.
    if (nvalid == kBlockN) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[mb][r] *= scale_log2;
    } else {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * mb + (r & 3) + 8 * (r >> 2) + 4 * hh;
          s[mb][r] = key < nvalid ? s[mb][r] * scale_log2 : -INFINITY;
        }
    }

    // ---- online softmax: the lane pair (l, l ^ 32) holds all 64 keys of one query
    float mt = s[0][0];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[mb][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mnew = fmaxf(m, mt);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    m = mnew;
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(s[mb][r] - mnew);
        s[mb][r] = e;
        lsum += e;
      }

    // ---- O^T += V^T P^T over four 16-key steps.  k-index 8 hh + j of step c stands for
    // key 16 c + 4 hh + 8 (j >> 2) + (j & 3) on both operands.
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int mb = c >> 1;
      const int base = 8 * (c & 1);
      uint4 pu;
      pu.x = pack_bf16x2(s[mb][base + 0], s[mb][base + 1]);
      pu.y = pack_bf16x2(s[mb][base + 2], s[mb][base + 3]);
      pu.z = pack_bf16x2(s[mb][base + 4], s[mb][base + 5]);
      pu.w = pack_bf16x2(s[mb][base + 6], s[mb][base + 7]);
      const bf16x8 pb = as_bf16x8(pu);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u16 *vp = Vt + (32 * db + l32) * VS + 16 * c + 4 * hh;
        const uint2 lo = *(const uint2 *)vp;
        const uint2 hi = *(const uint2 *)(vp + 8);
        const bf16x8 a = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o[db], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- epilogue: normalise, write the state into cache slot (p, rows), local change
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const bool empty = !(ltot > 0.f);
  const float inv = empty ? 0.f : 1.f / ltot;
  const float lse_nat = empty ? -INFINITY : (m + __log2f(ltot)) * kLn2;
  const bool is_local = delta_part != nullptr && desc.local_part[blk] == p;
  float dnum = 0.f, dden = 0.f;
  if (qvalid) {
    u16 *op = cache_o + ((((int64_t)p * desc.B + b) * desc.S_q + q0 + qrow) * H + head) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hh;
        uint2 nw;
        nw.x = pack_bf16x2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv);
        nw.y = pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
        if (is_local) {
          const uint2 od = *(const uint2 *)(op + d0);
          const uint32_t nn[2] = {nw.x, nw.y}, oo[2] = {od.x, od.y};
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const float n0 = bf16_bits_to_f32(nn[t] & 0xffffu), n1 = bf16_bits_to_f32(nn[t] >> 16);
            const float o0 = bf16_bits_to_f32(oo[t] & 0xffffu), o1 = bf16_bits_to_f32(oo[t] >> 16);
            dnum += (n0 - o0) * (n0 - o0) + (n1 - o1) * (n1 - o1);
            dden += o0 * o0 + o1 * o1;
          }
        }
        *(uint2 *)(op + d0) = nw;
      }
    }
    if (hh == 0)
      cache_lse[(((int64_t)p * desc.B + b) * H + head) * desc.S_q + q0 + qrow] = lse_nat;
  }
  if (is_local) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      dnum += __shfl_xor(dnum, off);
      dden += __shfl_xor(dden, off);
    }
    if (lane == 0) {
      red[2 * wave] = dnum;
      red[2 * wave + 1] = dden;
    }
    __syncthreads();
    if (tid == 0) {
      const float n = ((red[0] + red[2]) + red[4]) + red[6];
      const float d = ((red[1] + red[3]) + red[5]) + red[7];
      float *dp = delta_part + (((int64_t)b * desc.n_tiles + desc.tile_prefix[blk] + tile) * H + head) * 2;
      dp[0] = n;
      dp[1] = d;
    }
  }
}

// ------------------------------------------------------------------------------------
// State merge: one thread per 8 consecutive d of one (row, head); all P lse values of the
// row-head are kept in registers (PMAX >= P, unrolled), then the P bf16 states are
// streamed with 16-byte loads and combined in fp32.
// ------------------------------------------------------------------------------------
template <int D, int PMAX>
__global__ __launch_bounds__(256) void state_merge_kernel(
    const u16 *__restrict__ cache_o, const float *__restrict__ cache_lse, u16 *__restrict__ out,
    float *__restrict__ lse_out, const int S_q, const int H, const int P, const int64_t total_rh,
    const int64_t plane_o, const int64_t plane_lse) {
  constexpr int TPR = D / 8;
  constexpr int RPW = 256 / TPR;
  const int64_t rh = (int64_t)blockIdx.x * RPW + threadIdx.x / TPR;
  if (rh >= total_rh) return;
  const int c = threadIdx.x % TPR;
  const int64_t br = rh / H;  // b * S_q + r
  const int h = (int)(rh - br * H);
  const int64_t b = br / S_q;
  const int64_t r = br - b * S_q;
  const int64_t li = (b * H + h) * S_q + r;

  float lv[PMAX];
  float M = -INFINITY;
#pragma unroll
  for (int p = 0; p < PMAX; ++p) {
    lv[p] = (p < P) ? cache_lse[p * plane_lse + li] : -INFINITY;
    M = fmaxf(M, lv[p]);
  }
  const bool any = M > -INFINITY;
  float sum = 0.f;
#pragma unroll
  for (int p = 0; p < PMAX; ++p) sum += (lv[p] > -INFINITY) ? __expf(lv[p] - M) : 0.f;
  const float L = any ? M + __logf(sum) : -INFINITY;

  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  const u16 *src = cache_o + rh * D + 8 * c;
#pragma unroll
  for (int p = 0; p < PMAX; ++p) {
    if (p < P) {
      const float w = (lv[p] > -INFINITY) ? __expf(lv[p] - L) : 0.f;
      const u32x4 u = __builtin_nontemporal_load((const u32x4 *)(src + p * plane_o));
      const uint32_t x[4] = {u[0], u[1], u[2], u[3]};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc[2 * t] += w * bf16_bits_to_f32(x[t] & 0xffffu);
        acc[2 * t + 1] += w * bf16_bits_to_f32(x[t] >> 16);
      }
    }
  }
  uint4 res;
  res.x = pack_bf16x2(acc[0], acc[1]);
  res.y = pack_bf16x2(acc[2], acc[3]);
  res.z = pack_bf16x2(acc[4], acc[5]);
  res.w = pack_bf16x2(acc[6], acc[7]);
  *(uint4 *)(out + rh * D + 8 * c) = res;
  if (c == 0) lse_out[li] = L;
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

// Importance: one workgroup per (batch, block i, partition p).
__global__ __launch_bounds__(256) void importance_kernel(
    const float *__restrict__ cache_lse, const float *__restrict__ lse, const int S_q, const int H,
    const int P, const int B, const BlockDesc blocks, float *__restrict__ out) {
  __shared__ float sh[256];
  const int p = blockIdx.x % P;
  const int i = blockIdx.x / P;
  const int b = blockIdx.y;
  const int r0 = blocks.q_off[i];
  const int nr = blocks.q_off[i + 1] - r0;
  const int64_t n = (int64_t)nr * H;
  const float *cl = cache_lse + ((int64_t)p * B + b) * H * S_q;
  const float *ml = lse + (int64_t)b * H * S_q;
  float acc = 0.f;
  for (int64_t e = threadIdx.x; e < n; e += 256) {
    const int h = (int)(e / nr);
    const int r = r0 + (int)(e - (int64_t)h * nr);
    const float a = cl[(int64_t)h * S_q + r];
    const float t = ml[(int64_t)h * S_q + r];
    acc += (a > -INFINITY && t > -INFINITY) ? __expf(a - t) : 0.f;
  }
  const float tot = block_sum_256(acc, sh);
  if (threadIdx.x == 0) out[((int64_t)b * blocks.n_qb + i) * P + p] = n > 0 ? tot / (float)n : 0.f;
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

template <int D>
hipError_t merge_dispatch(int P, const void *cache_o, const float *cache_lse, void *out, float *lse,
                          int B, int S_q, int H, hipStream_t stream) {
  const int64_t total_rh = (int64_t)B * S_q * H;
  if (total_rh == 0) return hipSuccess;
  constexpr int RPW = 256 / (D / 8);
  const int64_t nwg = (total_rh + RPW - 1) / RPW;
  const int64_t plane_o = total_rh * D;
  const int64_t plane_lse = total_rh;
  dim3 grid((unsigned)nwg), block(256);
  const u16 *co = (const u16 *)cache_o;
  u16 *oo = (u16 *)out;
  if (P <= 8)
    hipLaunchKernelGGL((state_merge_kernel<D, 8>), grid, block, 0, stream, co, cache_lse, oo, lse, S_q, H, P, total_rh, plane_o, plane_lse);
  else if (P <= 16)
    hipLaunchKernelGGL((state_merge_kernel<D, 16>), grid, block, 0, stream, co, cache_lse, oo, lse, S_q, H, P, total_rh, plane_o, plane_lse);
  else if (P <= 32)
    hipLaunchKernelGGL((state_merge_kernel<D, 32>), grid, block, 0, stream, co, cache_lse, oo, lse, S_q, H, P, total_rh, plane_o, plane_lse);
  else
    hipLaunchKernelGGL((state_merge_kernel<D, 64>), grid, block, 0, stream, co, cache_lse, oo, lse, S_q, H, P, total_rh, plane_o, plane_lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_partition_attention(int D, const void *q, const void *k, const void *v,
                                      void *cache_o, float *cache_lse, float *delta_partials,
                                      const AttnDesc &desc, float scale_log2, hipStream_t stream) {
  const int64_t nwg = (int64_t)desc.B * desc.H * desc.items_per_head;
  if (nwg == 0) return hipSuccess;
  (void)hipGetLastError();
  dim3 grid((unsigned)nwg), block(256);
  if (D == 128)
    hipLaunchKernelGGL(partition_attention_kernel<128>, grid, block, 0, stream, (const u16 *)q,
                       (const u16 *)k, (const u16 *)v, (u16 *)cache_o, cache_lse, delta_partials, desc,
                       scale_log2);
  else
    hipLaunchKernelGGL(partition_attention_kernel<64>, grid, block, 0, stream, (const u16 *)q,
                       (const u16 *)k, (const u16 *)v, (u16 *)cache_o, cache_lse, delta_partials, desc,
                       scale_log2);
  return hipGetLastError();
}

hipError_t launch_state_merge(int D, int P, const void *cache_o, const float *cache_lse, void *out,
                              float *lse, int B, int S_q, int H, hipStream_t stream) {
  (void)hipGetLastError();
  if (D == 128) return merge_dispatch<128>(P, cache_o, cache_lse, out, lse, B, S_q, H, stream);
  return merge_dispatch<64>(P, cache_o, cache_lse, out, lse, B, S_q, H, stream);
}

hipError_t launch_importance(const float *cache_lse, const float *lse, int B, int S_q, int H, int P,
                             const BlockDesc &blocks, float *importance_out, hipStream_t stream) {
  (void)hipGetLastError();
  dim3 grid((unsigned)(blocks.n_qb * P), (unsigned)B), block(256);
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

}  // namespace dit
