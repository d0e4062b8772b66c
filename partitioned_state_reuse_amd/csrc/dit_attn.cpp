// C ABI of the partitioned-attention library: argument validation, work descriptions and
// kernel launches.  See include/dit_attn.h for the contract of every entry point.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <exception>

#include "launch.h"

namespace {

using dit::AttnDesc;
using dit::BlockDesc;

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

int check_dims(int B, int S_q, int S_kv, int H, int D) {
  if (B < 1 || S_q < 0 || S_kv < 0 || H < 1) return DIT_ERR_SHAPE;
  if (D != 64 && D != 128) return DIT_ERR_UNSUPPORTED;
  // element offsets are 64-bit in the kernels; grid sizes and row indices are 32-bit
  if ((int64_t)S_q * H > (int64_t)1 << 31 || (int64_t)S_kv * H > (int64_t)1 << 31)
    return DIT_ERR_SHAPE;
  // a dispatch counts its work-items in 32 bits: the merge kernels run D / 8 threads per
  // row-head of all B batches
  if ((int64_t)B * S_q * H * (D / 8) > (int64_t)UINT32_MAX) return DIT_ERR_SHAPE;
  return DIT_OK;
}

// The attention kernel copies a K/V tile through one buffer resource whose range starts at
// the tile's first row: the bytes it addresses, kBlockN - 1 row strides of H * D bf16 plus
// one row of D bf16, must stay within a 31-bit range.
bool tile_fits_buffer_range(int H, int D) {
  return ((int64_t)(dit::kBlockN - 1) * H * D + D) * 2 <= (int64_t)INT32_MAX;
}

int check_q_offsets(const int32_t *q_offsets, int n_qb, int S_q) {
  if (!q_offsets) return DIT_ERR_NULL;
  if (n_qb < 1 || n_qb > DIT_MAX_BLOCKS) return DIT_ERR_SHAPE;
  if (q_offsets[0] != 0 || q_offsets[n_qb] != S_q) return DIT_ERR_OFFSETS;
  for (int i = 0; i < n_qb; ++i)
    if (q_offsets[i + 1] <= q_offsets[i]) return DIT_ERR_OFFSETS;
  return DIT_OK;
}

int check_kv_offsets(const int32_t *kv_offsets, int P, int S_kv) {
  if (!kv_offsets) return DIT_ERR_NULL;
  if (P < 1 || P > DIT_MAX_PARTITIONS) return DIT_ERR_SHAPE;
  if (kv_offsets[0] != 0 || kv_offsets[P] != S_kv) return DIT_ERR_OFFSETS;
  for (int p = 0; p < P; ++p)
    if (kv_offsets[p + 1] < kv_offsets[p]) return DIT_ERR_OFFSETS;
  return DIT_OK;
}

int num_tiles(int rows) { return (rows + dit::kBlockM - 1) / dit::kBlockM; }

void fill_blocks(BlockDesc &bd, const int32_t *q_offsets, int n_qb) {
  memset(&bd, 0, sizeof(bd));
  bd.n_qb = n_qb;
  bd.tile_prefix[0] = 0;
  for (int i = 0; i <= n_qb; ++i) bd.q_off[i] = q_offsets[i];
  for (int i = 0; i < n_qb; ++i)
    bd.tile_prefix[i + 1] = bd.tile_prefix[i] + num_tiles(q_offsets[i + 1] - q_offsets[i]);
  bd.n_tiles = bd.tile_prefix[n_qb];
}

// Workspace layout: the local-change partial sums of the attention kernel, then (from the
// next 256-byte boundary) the importance partials of the merge.
size_t delta_ws_bytes(int B, int S_q, int H, int n_qb) {
  // upper bound on the tile count of any split into n_qb blocks
  const int64_t tiles = (int64_t)(S_q + dit::kBlockM - 1) / dit::kBlockM + n_qb;
  return (size_t)B * (size_t)tiles * (size_t)H * 2 * sizeof(float);
}

size_t imp_ws_offset(int B, int S_q, int H, int n_qb) { return (delta_ws_bytes(B, S_q, H, n_qb) + 255) & ~(size_t)255; }

// Upper bound on the importance partials of any split into n_qb blocks: every merge variant
// takes at least 16 row-heads per workgroup, and each block adds at most one partly filled
// workgroup.
size_t imp_ws_bound(int B, int S_q, int H, int n_qb, int P) {
  const int64_t wgs = ((int64_t)S_q * H + 15) / 16 + n_qb;
  return (size_t)B * (size_t)wgs * (size_t)P * sizeof(float);
}

// Validate an importance request of a merge and return the partials' address in the workspace.
int check_importance(int D, bool fp8, int B, int S_q, int H, int P, const int32_t *q_offsets, int n_qb,
                     void *workspace, size_t workspace_bytes, BlockDesc &bd, float *&imp_part) {
  int st = check_q_offsets(q_offsets, n_qb, S_q);
  if (st) return st;
  fill_blocks(bd, q_offsets, n_qb);
  const int64_t nwg = dit::merge_workgroups(D, fp8, &bd, B, S_q, H);
  if (nwg * 256 > (int64_t)UINT32_MAX) return DIT_ERR_SHAPE;
  if (!workspace) return DIT_ERR_WORKSPACE;
  const size_t off = imp_ws_offset(B, S_q, H, n_qb);
  if (workspace_bytes < off + (size_t)nwg * (size_t)P * sizeof(float)) return DIT_ERR_WORKSPACE;
  imp_part = (float *)((char *)workspace + off);
  return DIT_OK;
}

// Validate and build the work description of one partition-attention launch.
int build_attn(const void *q, const void *k, const void *v, int B, int S_q, int S_kv, int H, int D,
               const int32_t *q_offsets, int n_qb, const int32_t *kv_offsets, int P,
               const int32_t *local_part, const uint8_t *recompute, const uint8_t *cache_valid,
               const void *cache_o, const float *cache_lse, bool want_delta, const void *workspace,
               size_t workspace_bytes, AttnDesc &desc) {
  if (!q || !recompute || !cache_o || !cache_lse) return DIT_ERR_NULL;
  if (S_kv > 0 && (!k || !v)) return DIT_ERR_NULL;  // no keys: k and v may be NULL
  int st = check_dims(B, S_q, S_kv, H, D);
  if (st) return st;
  if (!tile_fits_buffer_range(H, D)) return DIT_ERR_SHAPE;
  if ((st = check_q_offsets(q_offsets, n_qb, S_q))) return st;
  if ((st = check_kv_offsets(kv_offsets, P, S_kv))) return st;
  for (int e = 0; e < n_qb * P; ++e)
    if (recompute[e] > 1) return DIT_ERR_MASK;
  if (local_part) {
    for (int i = 0; i < n_qb; ++i) {
      if (local_part[i] < 0 || local_part[i] >= P) return DIT_ERR_MASK;
      if (!recompute[i * P + local_part[i]]) return DIT_ERR_MASK;
    }
  }
  if (cache_valid) {
    for (int e = 0; e < n_qb * P; ++e)
      if (!recompute[e] && !cache_valid[e]) return DIT_ERR_CACHE_INVALID;
  }
  if (want_delta) {
    if (!local_part) return DIT_ERR_NULL;
    if (!workspace) return DIT_ERR_WORKSPACE;
    if (workspace_bytes < delta_ws_bytes(B, S_q, H, n_qb)) return DIT_ERR_WORKSPACE;
    if (cache_valid)
      for (int i = 0; i < n_qb; ++i)
        if (!cache_valid[i * P + local_part[i]]) return DIT_ERR_CACHE_INVALID;
  }
  memset(&desc, 0, sizeof(desc));
  desc.B = B;
  desc.H = H;
  desc.S_q = S_q;
  desc.S_kv = S_kv;
  desc.n_qb = n_qb;
  desc.P = P;
  for (int i = 0; i <= n_qb; ++i) desc.q_off[i] = q_offsets[i];
  for (int p = 0; p <= P; ++p) desc.kv_off[p] = kv_offsets[p];
  for (int i = 0; i < n_qb; ++i)
    desc.tile_prefix[i + 1] = desc.tile_prefix[i] + num_tiles(q_offsets[i + 1] - q_offsets[i]);
  desc.n_tiles = desc.tile_prefix[n_qb];
  for (int p = 0; p < P; ++p) {
    uint64_t bm = 0;
    int items = 0;
    for (int i = 0; i < n_qb; ++i)
      if (recompute[i * P + p]) {
        bm |= (uint64_t)1 << i;
        items += desc.tile_prefix[i + 1] - desc.tile_prefix[i];
      }
    desc.blocks_of_part[p] = bm;
    desc.item_prefix[p + 1] = desc.item_prefix[p] + items;
  }
  desc.items_per_head = desc.item_prefix[P];
  // one workgroup of kWaves * 64 threads per (batch, head, item); a dispatch counts its
  // work-items in 32 bits
  if ((int64_t)B * H * desc.items_per_head * (dit::kWaves * 64) > (int64_t)UINT32_MAX) return DIT_ERR_SHAPE;
  for (int i = 0; i < n_qb; ++i) desc.local_part[i] = (want_delta && local_part) ? local_part[i] : -1;
  return DIT_OK;
}

float scale_log2_of(float softmax_scale, int D) {
  const float s = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
  return s * 1.4426950408889634f;
}

// The reuse work of an attention launch (the merge of each block's reused planes into
// pre_o / pre_lse by workgroups dispatched after the attention items): its description, with
// the chunk counter at the start of the workspace's second region.  The workspace must hold
// claim_offset(...) + 4 bytes.
size_t claim_offset(int B, int S_q, int H, int n_qb) { return imp_ws_offset(B, S_q, H, n_qb); }

int make_tail(const AttnDesc &desc, const uint8_t *recompute, int B, int S_q, int H, int D, int n_qb, int P,
              void *pre_o, float *pre_lse, void *workspace, dit::TailMerge &tm) {
  memset(&tm, 0, sizeof(tm));
  tm.pre_o = pre_o;
  tm.pre_lse = pre_lse;
  tm.claim = (uint32_t *)((char *)workspace + claim_offset(B, S_q, H, n_qb));
  for (int i = 0; i < n_qb; ++i)
    for (int p = 0; p < P; ++p)
      if (!recompute[i * P + p]) tm.reuse_mask[i] |= (uint64_t)1 << p;
  // chunks: about 8 per resident workgroup slot of the device, 1 to 16 passes each
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return DIT_ERR_HIP;
  const int64_t slots = std::max<int64_t>(1, (int64_t)cus * dit::kMinBlocks);
  const int64_t rpw = (int64_t)dit::kWaves * 64 / (D / 8);  // row-heads per pass of a tail workgroup
  const int64_t passes = ((int64_t)B * S_q * H + rpw - 1) / rpw;
  const int64_t chunk_passes = std::min<int64_t>(16, std::max<int64_t>(1, passes / (8 * slots)));
  const int64_t n_chunks = (passes + chunk_passes - 1) / chunk_passes;
  const int64_t n_attn = (int64_t)B * H * desc.items_per_head;
  const int64_t n_tail = std::min(n_chunks, slots);
  // every tail workgroup ends with one failed claim: the counter reaches n_chunks + n_tail
  if ((n_attn + n_tail) * (dit::kWaves * 64) > (int64_t)UINT32_MAX || n_chunks + n_tail > (int64_t)UINT32_MAX)
    return DIT_ERR_SHAPE;
  tm.n_attn_wg = (int32_t)n_attn;
  tm.n_tail_wg = (int32_t)n_tail;
  tm.n_chunks = (int32_t)n_chunks;
  tm.chunk_passes = (int32_t)chunk_passes;
  return DIT_OK;
}

// One selective step (dit_attn_partitioned) on a given workspace.  fused_importance: the
// importance comes from the merge's partials (in the workspace); otherwise from a second
// pass over the stored lse planes, which needs no workspace.
int run_partitioned(const void *q, const void *k, const void *v, int B, int S_q, int S_kv, int H, int D,
                    const int32_t *q_offsets, int n_qb, const int32_t *kv_offsets, int P, const int32_t *local_part,
                    const uint8_t *recompute, const uint8_t *cache_valid, void *cache_o, float *cache_lse, void *out,
                    float *lse, float softmax_scale, float *importance_out, float *delta_out, void *workspace,
                    size_t workspace_bytes, bool fused_importance, void *stream) {
  try {
    if (!out || !lse) return DIT_ERR_NULL;
    AttnDesc desc;
    const bool want_delta = delta_out != nullptr;
    int st = build_attn(q, k, v, B, S_q, S_kv, H, D, q_offsets, n_qb, kv_offsets, P, local_part, recompute,
                        cache_valid, cache_o, cache_lse, want_delta, workspace, workspace_bytes, desc);
    if (st) return st;
    BlockDesc bd;
    fill_blocks(bd, q_offsets, n_qb);
    float *imp_part = nullptr;
    const bool fuse = importance_out != nullptr && fused_importance;
    if (fuse &&
        (st = check_importance(D, false, B, S_q, H, P, q_offsets, n_qb, workspace, workspace_bytes, bd, imp_part)))
      return st;
    hipStream_t s = as_stream(stream);
    // A step that reuses some slot and asks for no importance (which the full merge computes)
    // takes the reused states' merge into the attention launch, into out / lse, when the
    // workspace can hold the chunk counter; a masked merge then combines the fresh states with
    // that partial state in place.
    bool any_reuse = false;
    for (int e = 0; e < n_qb * P && !any_reuse; ++e) any_reuse = recompute[e] == 0;
    if (importance_out == nullptr && any_reuse && workspace != nullptr &&
        workspace_bytes >= claim_offset(B, S_q, H, n_qb) + sizeof(uint32_t)) {
      dit::TailMerge tm;
      if ((st = make_tail(desc, recompute, B, S_q, H, D, n_qb, P, out, lse, workspace, tm))) return st;
      if (dit::launch_partition_attention_premerge(D, q, k, v, cache_o, cache_lse,
                                                   want_delta ? (float *)workspace : nullptr, desc,
                                                   scale_log2_of(softmax_scale, D), tm, s) != hipSuccess)
        return DIT_ERR_HIP;
      dit::MergeSelect sel;
      memset(&sel, 0, sizeof(sel));
      sel.n_qb = n_qb;
      sel.has_extra = 1;
      for (int i = 0; i <= n_qb; ++i) sel.q_off[i] = q_offsets[i];
      for (int i = 0; i < n_qb; ++i)
        for (int p = 0; p < P; ++p)
          if (recompute[i * P + p]) sel.plane_mask[i] |= (uint64_t)1 << p;
      if (dit::launch_state_merge_masked(D, P, cache_o, cache_lse, out, lse, sel, out, lse, B, S_q, H, s) !=
          hipSuccess)
        return DIT_ERR_HIP;
    } else {
      if (dit::launch_partition_attention(D, false, q, k, v, cache_o, nullptr, cache_lse,
                                          want_delta ? (float *)workspace : nullptr, desc,
                                          scale_log2_of(softmax_scale, D), s) != hipSuccess)
        return DIT_ERR_HIP;
      if (dit::launch_state_merge(D, P, cache_o, cache_lse, out, lse, B, S_q, H, false, fuse ? &bd : nullptr,
                                  imp_part, importance_out, s) != hipSuccess)
        return DIT_ERR_HIP;
    }
    if (importance_out && !fuse &&
        dit::launch_importance(cache_lse, lse, B, S_q, H, P, bd, importance_out, s) != hipSuccess)
      return DIT_ERR_HIP;
    if (want_delta && dit::launch_delta_finalize((const float *)workspace, B, H, bd, delta_out, s) != hipSuccess)
      return DIT_ERR_HIP;
    return DIT_OK;
  } catch (...) {
    return DIT_ERR_INTERNAL;
  }
}

}  // namespace

extern "C" {

const char *dit_status_string(int status) {
  switch (status) {
    case DIT_OK: return "DIT_OK";
    case DIT_ERR_NULL: return "DIT_ERR_NULL: a required pointer is NULL";
    case DIT_ERR_SHAPE: return "DIT_ERR_SHAPE: a size is out of range";
    case DIT_ERR_OFFSETS: return "DIT_ERR_OFFSETS: offsets are malformed";
    case DIT_ERR_MASK: return "DIT_ERR_MASK: recompute mask or local partition invalid";
    case DIT_ERR_CACHE_INVALID: return "DIT_ERR_CACHE_INVALID: reuse of a never-computed cache slot";
    case DIT_ERR_WORKSPACE: return "DIT_ERR_WORKSPACE: workspace missing or too small";
    case DIT_ERR_UNSUPPORTED: return "DIT_ERR_UNSUPPORTED: unsupported head dim or mode";
    case DIT_ERR_HIP: return "DIT_ERR_HIP: a HIP launch failed";
    case DIT_ERR_INTERNAL: return "DIT_ERR_INTERNAL: internal error";
    default: return "unknown status";
  }
}

size_t dit_attn_workspace_bytes(int B, int S_q, int H, int D, int n_qb, int P) {
  if (check_dims(B, S_q, 0, H, D) != DIT_OK) return 0;
  if (n_qb < 1 || n_qb > DIT_MAX_BLOCKS || P < 1 || P > DIT_MAX_PARTITIONS) return 0;
  return imp_ws_offset(B, S_q, H, n_qb) + imp_ws_bound(B, S_q, H, n_qb, P);
}

int dit_partition_attention(const void *q, const void *k, const void *v, int B, int S_q, int S_kv,
                            int H, int D, const int32_t *q_offsets, int n_qb,
                            const int32_t *kv_offsets, int P, const int32_t *local_part,
                            const uint8_t *recompute, const uint8_t *cache_valid, void *cache_o,
                            float *cache_lse, float softmax_scale, void *workspace,
                            size_t workspace_bytes, void *stream) {
  try {
    AttnDesc desc;
    const bool want_delta = workspace != nullptr;
    int st = build_attn(q, k, v, B, S_q, S_kv, H, D, q_offsets, n_qb, kv_offsets, P, local_part,
                        recompute, cache_valid, cache_o, cache_lse, want_delta, workspace,
                        workspace_bytes, desc);
    if (st) return st;
    if (dit::launch_partition_attention(D, false, q, k, v, cache_o, nullptr, cache_lse,
                                        want_delta ? (float *)workspace : nullptr, desc,
                                        scale_log2_of(softmax_scale, D), as_stream(stream)) != hipSuccess)
      return DIT_ERR_HIP;
    return DIT_OK;
  } catch (...) {
    return DIT_ERR_INTERNAL;
  }
}

int dit_partition_attention_premerge(const void *q, const void *k, const void *v, int B, int S_q, int S_kv, int H,
                                     int D, const int32_t *q_offsets, int n_qb, const int32_t *kv_offsets, int P,
                                     const int32_t *local_part, const uint8_t *recompute, const uint8_t *cache_valid,
                                     void *cache_o, float *cache_lse, float softmax_scale, void *pre_o,
                                     float *pre_lse, void *workspace, size_t workspace_bytes, void *stream) {
  try {
    if (!pre_o || !pre_lse) return DIT_ERR_NULL;
    AttnDesc desc;
    const bool want_delta = local_part != nullptr;
    int st = build_attn(q, k, v, B, S_q, S_kv, H, D, q_offsets, n_qb, kv_offsets, P, local_part, recompute,
                        cache_valid, cache_o, cache_lse, want_delta, workspace, workspace_bytes, desc);
    if (st) return st;
    // the chunk counter sits at the start of the workspace's second region
    if (!workspace) return DIT_ERR_WORKSPACE;
    if (workspace_bytes < claim_offset(B, S_q, H, n_qb) + sizeof(uint32_t)) return DIT_ERR_WORKSPACE;
    dit::TailMerge tm;
    if ((st = make_tail(desc, recompute, B, S_q, H, D, n_qb, P, pre_o, pre_lse, workspace, tm))) return st;
    if (dit::launch_partition_attention_premerge(D, q, k, v, cache_o, cache_lse,
                                                 want_delta ? (float *)workspace : nullptr, desc,
                                                 scale_log2_of(softmax_scale, D), tm, as_stream(stream)) != hipSuccess)
      return DIT_ERR_HIP;
    return DIT_OK;
  } catch (...) {
    return DIT_ERR_INTERNAL;
  }
}

int dit_partition_attention_fp8(const void *q, const void *k, const void *v, int B, int S_q, int S_kv, int H, int D,
                                const int32_t *q_offsets, int n_qb, const int32_t *kv_offsets, int P,
                                const int32_t *local_part, const uint8_t *recompute, const uint8_t *cache_valid,
                                void *cache_q8, float *cache_scale, float *cache_lse, float softmax_scale,
                                void *workspace, size_t workspace_bytes, void *stream) {
  try {
    if (!cache_scale) return DIT_ERR_NULL;
    AttnDesc desc;
    const bool want_delta = workspace != nullptr;
    int st = build_attn(q, k, v, B, S_q, S_kv, H, D, q_offsets, n_qb, kv_offsets, P, local_part, recompute,
                        cache_valid, cache_q8, cache_lse, want_delta, workspace, workspace_bytes, desc);
    if (st) return st;
    if (dit::launch_partition_attention(D, true, q, k, v, cache_q8, cache_scale, cache_lse,
                                        want_delta ? (float *)workspace : nullptr, desc,
                                        scale_log2_of(softmax_scale, D), as_stream(stream)) != hipSuccess)
      return DIT_ERR_HIP;
    return DIT_OK;
  } catch (...) {
    return DIT_ERR_INTERNAL;
  }
}

int dit_state_merge_fp8(const void *cache_q8, const float *cache_scale, const float *cache_lse, int B, int S_q,
                        int H, int D, int P, void *out, float *lse, const int32_t *q_offsets, int n_qb,
                        float *importance_out, void *workspace, size_t workspace_bytes, void *stream) {
  try {
    if (!cache_q8 || !cache_scale || !cache_lse || !out || !lse) return DIT_ERR_NULL;
    int st = check_dims(B, S_q, 0, H, D);
    if (st) return st;
    if (P < 1 || P > DIT_MAX_PARTITIONS) return DIT_ERR_SHAPE;
    BlockDesc bd;
    float *imp_part = nullptr;
    if (importance_out &&
        (st = check_importance(D, true, B, S_q, H, P, q_offsets, n_qb, workspace, workspace_bytes, bd, imp_part)))
      return st;
    if (dit::launch_state_merge_fp8(D, P, cache_q8, cache_scale, cache_lse, out, lse, B, S_q, H,
                                    importance_out ? &bd : nullptr, imp_part, importance_out,
                                    as_stream(stream)) != hipSuccess)
      return DIT_ERR_HIP;
    return DIT_OK;
  } catch (...) {
    return DIT_ERR_INTERNAL;
  }
}

int dit_state_merge(const void *cache_o, const float *cache_lse, int B, int S_q, int H, int D, int P,
                    void *out, float *lse, const int32_t *q_offsets, int n_qb, float *importance_out,
                    void *workspace, size_t workspace_bytes, void *stream) {
  try {
    if (!cache_o || !cache_lse || !out || !lse) return DIT_ERR_NULL;
    int st = check_dims(B, S_q, 0, H, D);
    if (st) return st;
    if (P < 1 || P > DIT_MAX_PARTITIONS) return DIT_ERR_SHAPE;
    BlockDesc bd;
    float *imp_part = nullptr;
    if (importance_out &&
        (st = check_importance(D, false, B, S_q, H, P, q_offsets, n_qb, workspace, workspace_bytes, bd, imp_part)))
      return st;
    if (dit::launch_state_merge(D, P, cache_o, cache_lse, out, lse, B, S_q, H, false,
                                importance_out ? &bd : nullptr, imp_part, importance_out,
                                as_stream(stream)) != hipSuccess)
      return DIT_ERR_HIP;
    return DIT_OK;
  } catch (...) {
    return DIT_ERR_INTERNAL;
  }
}

int dit_state_merge_masked(const void *cache_o, const float *cache_lse, int B, int S_q, int H, int D, int P,
                           const int32_t *q_offsets, int n_qb, const uint8_t *plane_select, const void *extra_o,
                           const float *extra_lse, void *out, float *lse, void *stream) {
  try {
    if (!cache_o || !cache_lse || !out || !lse || !plane_select) return DIT_ERR_NULL;
    if ((extra_o == nullptr) != (extra_lse == nullptr)) return DIT_ERR_NULL;
    int st = check_dims(B, S_q, 0, H, D);
    if (st) return st;
    if (P < 1 || P > DIT_MAX_PARTITIONS) return DIT_ERR_SHAPE;
    if ((st = check_q_offsets(q_offsets, n_qb, S_q))) return st;
    dit::MergeSelect sel;
    memset(&sel, 0, sizeof(sel));
    sel.n_qb = n_qb;
    sel.has_extra = extra_o != nullptr;
    for (int i = 0; i <= n_qb; ++i) sel.q_off[i] = q_offsets[i];
    for (int i = 0; i < n_qb; ++i)
      for (int p = 0; p < P; ++p) {
        if (plane_select[i * P + p] > 1) return DIT_ERR_MASK;
        if (plane_select[i * P + p]) sel.plane_mask[i] |= (uint64_t)1 << p;
      }
    if (dit::launch_state_merge_masked(D, P, cache_o, cache_lse, extra_o, extra_lse, sel, out, lse, B, S_q, H,
                                       as_stream(stream)) != hipSuccess)
      return DIT_ERR_HIP;
    return DIT_OK;
  } catch (...) {
    return DIT_ERR_INTERNAL;
  }
}

int dit_state_compose(const void *cache_o, const float *cache_lse, int P_in, const int32_t *group_offsets, int G,
                      int B, int S_q, int H, int D, void *out_o, float *out_lse, void *stream) {
  try {
    if (!cache_o || !cache_lse || !out_o || !out_lse || !group_offsets) return DIT_ERR_NULL;
    int st = check_dims(B, S_q, 0, H, D);
    if (st) return st;
    if (P_in < 1 || P_in > DIT_MAX_PARTITIONS || G < 1 || G > P_in) return DIT_ERR_SHAPE;
    if (group_offsets[0] != 0 || group_offsets[G] != P_in) return DIT_ERR_OFFSETS;
    for (int g = 0; g < G; ++g)
      if (group_offsets[g + 1] <= group_offsets[g]) return DIT_ERR_OFFSETS;
    const int64_t plane_lse = (int64_t)B * H * S_q;
    const int64_t plane_o = plane_lse * D;
    const uint16_t *in_o = (const uint16_t *)cache_o;
    uint16_t *o = (uint16_t *)out_o;
    for (int g = 0; g < G; ++g) {
      const int a = group_offsets[g];
      if (dit::launch_state_merge(D, group_offsets[g + 1] - a, in_o + a * plane_o, cache_lse + a * plane_lse,
                                  o + g * plane_o, out_lse + g * plane_lse, B, S_q, H, true, nullptr, nullptr,
                                  nullptr, as_stream(stream)) != hipSuccess)
        return DIT_ERR_HIP;
    }
    return DIT_OK;
  } catch (...) {
    return DIT_ERR_INTERNAL;
  }
}

int dit_importance(const float *cache_lse, const float *lse, int B, int S_q, int H, int P,
                   const int32_t *q_offsets, int n_qb, float *importance_out, void *stream) {
  try {
    if (!cache_lse || !lse || !importance_out) return DIT_ERR_NULL;
    int st = check_dims(B, S_q, 0, H, 128);
    if (st) return st;
    if (P < 1 || P > DIT_MAX_PARTITIONS) return DIT_ERR_SHAPE;
    if ((st = check_q_offsets(q_offsets, n_qb, S_q))) return st;
    BlockDesc bd;
    fill_blocks(bd, q_offsets, n_qb);
    if (dit::launch_importance(cache_lse, lse, B, S_q, H, P, bd, importance_out, as_stream(stream)) != hipSuccess)
      return DIT_ERR_HIP;
    return DIT_OK;
  } catch (...) {
    return DIT_ERR_INTERNAL;
  }
}

int dit_local_change_finalize(const void *workspace, size_t workspace_bytes, int B, int S_q, int H,
                              int D, const int32_t *q_offsets, int n_qb, float *delta_out, void *stream) {
  try {
    if (!workspace || !delta_out) return DIT_ERR_NULL;
    int st = check_dims(B, S_q, 0, H, D);
    if (st) return st;
    if ((st = check_q_offsets(q_offsets, n_qb, S_q))) return st;
    if (workspace_bytes < delta_ws_bytes(B, S_q, H, n_qb)) return DIT_ERR_WORKSPACE;
    BlockDesc bd;
    fill_blocks(bd, q_offsets, n_qb);
    if (dit::launch_delta_finalize((const float *)workspace, B, H, bd, delta_out, as_stream(stream)) !=
        hipSuccess)
      return DIT_ERR_HIP;
    return DIT_OK;
  } catch (...) {
    return DIT_ERR_INTERNAL;
  }
}

int dit_attn_partitioned(const void *q, const void *k, const void *v, int B, int S_q, int S_kv, int H,
                         int D, const int32_t *q_offsets, int n_qb, const int32_t *kv_offsets, int P,
                         const int32_t *local_part, const uint8_t *recompute, const uint8_t *cache_valid,
                         void *cache_o, float *cache_lse, void *out, float *lse, float softmax_scale,
                         float *importance_out, float *delta_out, void *workspace, size_t workspace_bytes,
                         void *stream) {
  return run_partitioned(q, k, v, B, S_q, S_kv, H, D, q_offsets, n_qb, kv_offsets, P, local_part, recompute,
                         cache_valid, cache_o, cache_lse, out, lse, softmax_scale, importance_out, delta_out,
                         workspace, workspace_bytes, true, stream);
}

int dit_attn_partitioned_noalloc(const void *q, const void *k, const void *v, int B, int S_q, int S_kv, int H,
                                 int D, const int32_t *q_offsets, int n_qb, const int32_t *kv_offsets, int P,
                                 const int32_t *local_part, const uint8_t *recompute, const uint8_t *cache_valid,
                                 void *cache_o, float *cache_lse, void *out, float *lse, float softmax_scale,
                                 float *importance_out, float *delta_out, void *stream) {
  try {
    // the library's own device scratch stands in for the workspace: the local-change partials
    // (sizes beyond it are rejected by the workspace check, DIT_ERR_WORKSPACE); the importance
    // is taken in a second pass, which needs none
    void *ws = nullptr;
    size_t ws_bytes = 0;
    if (delta_out != nullptr) {
      if (dit::scratch_address(&ws) != hipSuccess) return DIT_ERR_HIP;
      ws_bytes = dit::kScratchBytes;
    }
    return run_partitioned(q, k, v, B, S_q, S_kv, H, D, q_offsets, n_qb, kv_offsets, P, local_part, recompute,
                           cache_valid, cache_o, cache_lse, out, lse, softmax_scale, importance_out, delta_out, ws,
                           ws_bytes, false, stream);
  } catch (...) {
    return DIT_ERR_INTERNAL;
  }
}

}  // extern "C"
