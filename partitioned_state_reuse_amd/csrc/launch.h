// Internal interface between the C ABI (dit_attn.cpp) and the HIP kernels (kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dit_attn.h"

namespace dit {

// Partition-attention tile shape (build-time parameters).
#ifndef DIT_ATTN_WAVES
#define DIT_ATTN_WAVES 4
#endif
#ifndef DIT_ATTN_BLOCK_N
#define DIT_ATTN_BLOCK_N 32
#endif
#ifndef DIT_ATTN_STAGES
#define DIT_ATTN_STAGES 2
#endif
#ifndef DIT_ATTN_MIN_BLOCKS
#define DIT_ATTN_MIN_BLOCKS 3
#endif
constexpr int kWaves = DIT_ATTN_WAVES;      // waves per attention workgroup
constexpr int kBlockM = 32 * kWaves;        // query rows per attention workgroup (32 per wave)
constexpr int kBlockN = DIT_ATTN_BLOCK_N;   // keys per staged KV tile (32 or 64)
constexpr int kStages = DIT_ATTN_STAGES;    // K/V tile buffers in the LDS ring (2 or 3)
#ifndef DIT_ATTN_READ_AHEAD
#define DIT_ATTN_READ_AHEAD 3
#endif
// MFMAs by which the LDS operand reads run ahead of their use in the attention kernel
constexpr int kReadAhead = DIT_ATTN_READ_AHEAD;
#ifndef DIT_ATTN_NT_SLOTS
#define DIT_ATTN_NT_SLOTS 0
#endif
// cache-slot stores (and old-slot loads) of the attention epilogue non-temporal
constexpr bool kNtSlots = DIT_ATTN_NT_SLOTS != 0;
#ifndef DIT_ATTN_SETPRIO
#define DIT_ATTN_SETPRIO 0
#endif
// raise the wave priority while it issues MFMAs (K Q^T and V^T P^T), lower it for the softmax
constexpr bool kSetPrio = DIT_ATTN_SETPRIO != 0;
#ifndef DIT_MERGE_CHUNK_ROWS
#define DIT_MERGE_CHUNK_ROWS 16
#endif
// query rows (of all heads) whose merge workgroups run on one XCD in a row (0: round-robin)
constexpr int kMergeChunkRows = DIT_MERGE_CHUNK_ROWS;
#ifndef DIT_MERGE_MASKED_BATCH
#define DIT_MERGE_MASKED_BATCH 4
#endif
// selected cache planes whose loads a masked-merge thread keeps in flight together
constexpr int kMaskedMergeBatch = DIT_MERGE_MASKED_BATCH;
#ifndef DIT_MERGE_FP8_DPT
#define DIT_MERGE_FP8_DPT 16
#endif
#ifndef DIT_MERGE_BATCH
#define DIT_MERGE_BATCH 1
#endif
// cache planes whose loads a merge thread (plain and fp8 merge) keeps in flight together
constexpr int kMergeBatch = DIT_MERGE_BATCH;
#ifndef DIT_MERGE_DPP
#define DIT_MERGE_DPP 0
#endif
// merge-weight reductions over a row-head's lanes through DPP moves instead of LDS permutes
constexpr bool kMergeDpp = DIT_MERGE_DPP != 0;
constexpr int kMinBlocks = DIT_ATTN_MIN_BLOCKS;     // attention workgroups resident per CU (register budget)

// Work description of one partition-attention launch, passed by value as a kernel
// argument so that a launch needs no host-to-device copy.
//
// Items are (batch, head, partition p, query block i, query tile t) for every (i, p) whose
// recompute flag is set.  Per (batch, head) the items are ordered by partition, then block,
// then tile, so that consecutive workgroups read the same K/V partition.
struct AttnDesc {
  int32_t B, H, S_q, S_kv, n_qb, P;
  int32_t items_per_head;                        // item_prefix[P]
  int32_t n_tiles;                               // tile_prefix[n_qb]
  int32_t q_off[DIT_MAX_BLOCKS + 1];
  int32_t kv_off[DIT_MAX_PARTITIONS + 1];
  int32_t tile_prefix[DIT_MAX_BLOCKS + 1];       // cumulative query tiles over blocks
  int32_t item_prefix[DIT_MAX_PARTITIONS + 1];   // cumulative items over partitions
  uint64_t blocks_of_part[DIT_MAX_PARTITIONS];   // bit i set: block i recomputes partition p
  int32_t local_part[DIT_MAX_BLOCKS];            // -1: no local-change partials for block i
};

// Query-block offsets and tile prefix for the reductions.
struct BlockDesc {
  int32_t n_qb, n_tiles;
  int32_t q_off[DIT_MAX_BLOCKS + 1];
  int32_t tile_prefix[DIT_MAX_BLOCKS + 1];
};

// fp8_cache: cache_o holds e4m3 codes (1 byte per element) and cache_scale one scale per
// (partition, batch, head, row); otherwise cache_o is bf16 and cache_scale is unused.
hipError_t launch_partition_attention(int D, bool fp8_cache, const void *q, const void *k, const void *v,
                                      void *cache_o, float *cache_scale, float *cache_lse, float *delta_partials,
                                      const AttnDesc &desc, float scale_log2, hipStream_t stream);

// Reuse work carried by a partition-attention launch (bf16 cache): n_tail_wg workgroups
// after the n_attn_wg attention ones merge, for every query row, the cache planes its block
// reuses (bit p of reuse_mask[i]: block i reuses plane p) into the partial state pre_o
// [B, S_q, H, D] bf16, pre_lse [B, H, S_q] f32, claiming chunks of chunk_passes * 256 / (D / 8)
// row-heads (n_chunks of them cover B * S_q * H) from the counter `claim`, which the launch
// clears first.
struct TailMerge {
  void *pre_o;
  float *pre_lse;
  uint32_t *claim;
  int32_t n_attn_wg;
  int32_t n_tail_wg;
  int32_t n_chunks;
  int32_t chunk_passes;
  uint64_t reuse_mask[DIT_MAX_BLOCKS];
};

hipError_t launch_partition_attention_premerge(int D, const void *q, const void *k, const void *v, void *cache_o,
                                               float *cache_lse, float *delta_partials, const AttnDesc &desc,
                                               float scale_log2, const TailMerge &tm, hipStream_t stream);

// Merges.  The cache's lse (and scale) planes are [P, B, S_q, H]; the merged lse goes out as
// [B, H, S_q], or, with lse_rowmajor, as [B, S_q, H] (a cache plane: compose).  With
// imp_blocks non-null the merge also writes importance partials (imp_part: P floats per
// merge workgroup, merge_workgroups(...) of them) and finishes the importance into
// importance_out [B, n_qb, P].
hipError_t launch_state_merge_fp8(int D, int P, const void *cache_q8, const float *cache_scale,
                                  const float *cache_lse, void *out, float *lse, int B, int S_q, int H,
                                  const BlockDesc *imp_blocks, float *imp_part, float *importance_out,
                                  hipStream_t stream);

// Plane selection of a masked merge: row r of block i merges plane p when bit p of
// plane_mask[i] is set, plus the extra state when there is one.
struct MergeSelect {
  int32_t n_qb;
  int32_t has_extra;
  int32_t q_off[DIT_MAX_BLOCKS + 1];
  uint64_t plane_mask[DIT_MAX_BLOCKS];
};

hipError_t launch_state_merge_masked(int D, int P, const void *cache_o, const float *cache_lse,
                                     const void *extra_o, const float *extra_lse, const MergeSelect &sel,
                                     void *out, float *lse, int B, int S_q, int H, hipStream_t stream);

hipError_t launch_state_merge(int D, int P, const void *cache_o, const float *cache_lse,
                              void *out, float *lse, int B, int S_q, int H, bool lse_rowmajor,
                              const BlockDesc *imp_blocks, float *imp_part, float *importance_out,
                              hipStream_t stream);

// Workgroups of a merge launch (with imp_blocks: the per-block placement of the importance
// partials).
int64_t merge_workgroups(int D, bool fp8_cache, const BlockDesc *imp_blocks, int B, int S_q, int H);

hipError_t launch_importance(const float *cache_lse, const float *lse, int B, int S_q, int H,
                             int P, const BlockDesc &blocks, float *importance_out,
                             hipStream_t stream);

hipError_t launch_delta_finalize(const float *partials, int B, int H, const BlockDesc &blocks,
                                 float *delta_out, hipStream_t stream);

// Device scratch of the allocation-free entry point: a file-scope device array of
// kScratchBytes in kernels.hip.  scratch_address gives its address on the current device
// (looked up once per device with hipGetSymbolAddress, then cached).
constexpr size_t kScratchBytes = DIT_SCRATCH_BYTES;
hipError_t scratch_address(void **out);

}  // namespace dit
