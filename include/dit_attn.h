/*
 * dit_attn.h -- C ABI of the partitioned DiT self-attention library for MI355X (gfx950).
 *
 * The operation (DiTango: Cost-Effective Parallel Diffusion Generation with Selective
 * Attention State Reuse, technical summary, "Methodology"): non-causal self-attention of
 * query tokens over a key/value sequence that is split into P contiguous KV partitions.
 *
 *   - Attention over one partition p gives the attention state (O_p, lse_p) of every query
 *     row and head: s_j = scale * q . k_j over the keys j of p, lse_p = ln sum_j e^{s_j},
 *     O_p = sum_j e^{s_j - lse_p} v_j   ("Methodology §2, State Composition").
 *   - States compose associatively and commutatively by LSE-weighted combination:
 *     lse = ln sum_p e^{lse_p}, O = sum_p e^{lse_p - lse} O_p.  The library caches the
 *     per-partition states, not raw K/V.
 *   - A recompute mask chooses, per query block i and partition p, whether the state of
 *     (i, p) is computed from scratch or taken from the cache filled at an earlier
 *     denoising step ("Methodology §1, Anchor-Guided Selection Planner").
 *   - Anchor steps recompute every partition and refresh the partition importance
 *     w_ip = mean over block i's rows and heads of e^{lse_p - lse}; between anchors the
 *     change of each block's always-recomputed local state,
 *     delta_i = ||O_loc(t) - O_loc(t-1)||_F / ||O_loc(t-1)||_F, stands in for how the other
 *     states evolve ("Methodology §1, Error Modeling, Anchor Steps, Online Prediction").
 *   - A host-side planner turns w and delta into the next step's mask, per group of
 *     adjacent partitions ("Methodology §1, Group-wise Strategy").
 *
 * Conventions shared by every call:
 *   - Device pointers are caller-owned device memory (e.g. allocated by PyTorch); the
 *     library allocates and frees no device or pinned memory and keeps no pointer after a
 *     call returns.  Host pointers are only read during the call.
 *   - Layouts (row-major, bf16 = bfloat16, 2 bytes):
 *       q            [B, S_q, H, D]  bf16      (RoPE already applied)
 *       k, v         [B, S_kv, H, D] bf16
 *       cache_o      [P, B, S_q, H, D] bf16    state cache: output of each partition
 *       cache_lse    [P, B, S_q, H] f32        state cache: natural-log lse of each partition
 *                                              (each plane in the row order of out: a run of
 *                                              row-heads reads one contiguous range)
 *       out          [B, S_q, H, D] bf16       merged output
 *       lse          [B, H, S_q] f32           merged lse
 *     All device buffers must be 16-byte aligned.  The buffers a call may write (the cache,
 *     out, lse, importance_out, delta_out, the workspace) must not overlap one another or
 *     q, k, v (the read-only inputs may overlap each other), except where a call says
 *     otherwise (dit_state_merge_masked may take its extra state in out / lse itself).
 *   - q_offsets [n_qb+1]: query-block offsets, q_offsets[0] = 0, strictly increasing,
 *     q_offsets[n_qb] = S_q.  kv_offsets [P+1]: partition offsets, kv_offsets[0] = 0,
 *     non-decreasing (empty partitions allowed), kv_offsets[P] = S_kv.
 *     1 <= n_qb <= DIT_MAX_BLOCKS, 1 <= P <= DIT_MAX_PARTITIONS.
 *   - recompute [n_qb * P] (row-major, block-major): 1 = compute the state of (i, p) and
 *     write it into the cache slot, 0 = reuse the cached slot.  Any other value is an error.
 *   - D must be 64 or 128.
 *   - Every call validates all arguments on the host before it enqueues anything: on any
 *     error return no buffer is touched and nothing is enqueued.  Calls are asynchronous on
 *     `stream` (a hipStream_t; NULL = the null stream) and never synchronise.  A failed
 *     launch returns DIT_ERR_HIP; faults inside a kernel surface at the caller's next
 *     synchronisation.  There is no global mutable state: calls are reentrant.  No C++
 *     exception crosses the ABI (DIT_ERR_INTERNAL).
 *   - Results are deterministic: every reduction has a fixed order and no floating-point
 *     atomics are used, so repeated calls give bitwise-equal outputs.
 */
#ifndef DIT_ATTN_H
#define DIT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DIT_MAX_BLOCKS 64
#define DIT_MAX_PARTITIONS 64
/* Bytes of the device scratch that dit_attn_partitioned_noalloc uses in place of a
 * workspace (one array per GPU the library runs on, held until the process ends). */
#define DIT_SCRATCH_BYTES (1u << 20)

typedef enum {
  DIT_OK = 0,
  DIT_ERR_NULL = -1,          /* a required pointer is NULL */
  DIT_ERR_SHAPE = -2,         /* B, S_q, S_kv, H, n_qb or P out of range: S_q*H and S_kv*H
                                 at most 2^31, B*S_q*H*D/8 below 2^32; for the attention
                                 calls also B*H*(recomputed 128-row tiles)*256 below 2^32 and
                                 (31*H*D + D)*2 at most 2^31 - 1 bytes (the span of one
                                 32-key K/V tile's rows: H*D up to 34,636,828 at D = 128) */
  DIT_ERR_OFFSETS = -3,       /* q_offsets / kv_offsets / group offsets malformed */
  DIT_ERR_MASK = -4,          /* recompute value not 0/1, local partition not recomputed, bad local_part */
  DIT_ERR_CACHE_INVALID = -5, /* reuse (or delta) of a cache slot that cache_valid marks never computed */
  DIT_ERR_WORKSPACE = -6,     /* workspace NULL or smaller than dit_attn_workspace_bytes() */
  DIT_ERR_UNSUPPORTED = -7,   /* D not in {64, 128}, or a mode the library does not implement */
  DIT_ERR_HIP = -8,           /* a HIP launch failed */
  DIT_ERR_INTERNAL = -9       /* unexpected internal error */
} dit_status;

/* Human-readable name of a status code (static string, never NULL). */
const char *dit_status_string(int status);

/* Bytes of device workspace dit_attn_partitioned needs for these sizes, for any split into
 * n_qb query blocks: the local-change partial sums of the attention kernel, then the
 * importance partials of the merge (P floats per merge workgroup); a reuse step without
 * importance keeps the in-launch pre-merge's chunk counter where the importance partials
 * would go.  The split calls take the same workspace.  Calls in flight at the same time (on
 * different streams) must not share a workspace.  Returns 0 if the sizes are invalid. */
size_t dit_attn_workspace_bytes(int B, int S_q, int H, int D, int n_qb, int P);

/*
 * One selective attention step (partition attention, cache update, merge, and optionally
 * importance and local change).  Equivalent to dit_partition_attention, then
 * dit_state_merge, then dit_importance / dit_local_change_finalize when requested.
 * On a step that reuses some slot and asks for no importance, when a workspace is given,
 * the merge of the reused states runs inside the attention launch, into out / lse (as
 * dit_partition_attention_premerge does), and dit_state_merge_masked then combines the
 * fresh states with that partial state in place: the same result up to the rounding order
 * of the fp32 merge (DiTango, technical summary, "Methodology §2, Pipeline Orchestration").
 *
 *   softmax_scale      > 0, or <= 0 for 1/sqrt(D)
 *   local_part         host [n_qb] or NULL: each block's own partition.  When given, the
 *                      local partition of every block must be recomputed (DIT_ERR_MASK).
 *   cache_valid        host [n_qb * P] or NULL: 1 = slot holds a state from an earlier step.
 *                      When given, reusing a slot marked 0 is DIT_ERR_CACHE_INVALID.
 *   importance_out     device [B, n_qb, P] f32 or NULL: w_ip of this step's states.
 *   delta_out          device [B, n_qb] f32 or NULL: delta_i of the local states against the
 *                      states the local slots held before this call.  Needs local_part and
 *                      a workspace; with cache_valid given the local slots must be valid.
 *   workspace          device, >= dit_attn_workspace_bytes(...) when delta_out or
 *                      importance_out is given, else may be NULL (then the reused states are
 *                      merged after the attention launch).  Contents on entry are ignored.  The importance is computed inside the merge (partial sums
 *                      per merge workgroup, finished in a fixed order).  Calls that share a
 *                      workspace must not run at the same time.
 */
int dit_attn_partitioned(const void *q, const void *k, const void *v,
                         int B, int S_q, int S_kv, int H, int D,
                         const int32_t *q_offsets, int n_qb,
                         const int32_t *kv_offsets, int P,
                         const int32_t *local_part,
                         const uint8_t *recompute,
                         const uint8_t *cache_valid,
                         void *cache_o, float *cache_lse,
                         void *out, float *lse,
                         float softmax_scale,
                         float *importance_out,
                         float *delta_out,
                         void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * dit_attn_partitioned for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, results
 * and errors as dit_attn_partitioned, without the workspace: the local-change partial sums
 * go to a device array inside the library, DIT_SCRATCH_BYTES per GPU (file-scope device
 * memory, held until the process ends; its address is looked up once per device, on the
 * first call that needs it with that device current).  The call allocates nothing: no
 * hipMalloc, hipFree or allocating library routine.
 *   - delta_out given and B * (ceil(S_q / 128) + n_qb) * H * 8 bytes (the local-change
 *     partials) above DIT_SCRATCH_BYTES: DIT_ERR_WORKSPACE (e.g. B = 1, H = 40 allows about
 *     3,270 query tiles of 128 rows plus blocks, S_q up to ~410,000 rows).
 *   - The array holds the local-change partial sums and, when delta_out is given, the chunk
 *     counter of the in-launch merge of the reused states (cleared by the call itself);
 *     without delta_out the reused states are merged after the attention launch.  The
 *     importance, when asked for, is taken in a second pass over the stored lse planes (no
 *     partials kept).  The array keeps the last call's contents; every entry a call reads is
 *     written (or cleared) by the same call.  Calls that overlap on one GPU (on different streams, or from
 *     different threads) share the array and race: serialise them.
 *   - Unlike the other calls this one keeps state across calls (the per-device address).
 */
int dit_attn_partitioned_noalloc(const void *q, const void *k, const void *v,
                                 int B, int S_q, int S_kv, int H, int D,
                                 const int32_t *q_offsets, int n_qb,
                                 const int32_t *kv_offsets, int P,
                                 const int32_t *local_part,
                                 const uint8_t *recompute,
                                 const uint8_t *cache_valid,
                                 void *cache_o, float *cache_lse,
                                 void *out, float *lse,
                                 float softmax_scale,
                                 float *importance_out,
                                 float *delta_out,
                                 void *stream);

/*
 * Partition attention and cache update only: for every (i, p) with recompute = 1, compute
 * the state of block i's query rows over partition p's keys and write it into cache slot
 * (p, rows of i); other slots are untouched.  bf16 MFMA products, fp32 accumulation and
 * softmax.  An empty partition writes O = 0, lse = -inf.
 *   cache_valid        host [n_qb * P] or NULL, as for dit_attn_partitioned: when given, a
 *                      slot that is neither recomputed nor marked valid is
 *                      DIT_ERR_CACHE_INVALID (a merge of the cache after this call would
 *                      read it), and so is a local slot marked invalid when the local-change
 *                      partials are written.
 *   workspace          device or NULL, of workspace_bytes >= dit_attn_workspace_bytes(...).
 *                      When given (with local_part, else DIT_ERR_NULL), the kernel also
 *                      writes, per (query tile, head) of each block's local partition, the
 *                      sums sum (O_new - O_old)^2 and sum O_old^2 over the tile's rows and D,
 *                      where O_old is the slot's content before this call and O_new the value
 *                      written; finish them with dit_local_change_finalize on the same
 *                      workspace.  Calls that share a workspace must not run at the same
 *                      time.
 */
int dit_partition_attention(const void *q, const void *k, const void *v,
                            int B, int S_q, int S_kv, int H, int D,
                            const int32_t *q_offsets, int n_qb,
                            const int32_t *kv_offsets, int P,
                            const int32_t *local_part,
                            const uint8_t *recompute,
                            const uint8_t *cache_valid,
                            void *cache_o, float *cache_lse,
                            float softmax_scale,
                            void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * Partition attention with the reuse work in the same launch: the one-GPU form of filling
 * compute bubbles with reuse operations (DiTango, technical summary, "Methodology §2,
 * Pipeline Orchestration").  Does what dit_partition_attention does, and in addition merges,
 * for every query row r of block i and head h, the cache planes that block i reuses
 * (recompute[i * P + p] = 0) into the partial state
 *   pre_o    device out [B, S_q, H, D] bf16
 *   pre_lse  device out [B, H, S_q] f32
 * by the rule of dit_state_merge (a row whose block reuses no plane gets O = 0,
 * lse = -inf).  The merging workgroups are dispatched after every attention workgroup and
 * run in the slots that the attention work leaves as the launch drains; the planes they
 * read are ones this launch does not write.  Finish the step with dit_state_merge_masked
 * (plane_select = recompute, extra state = pre_o / pre_lse): a two-state final combine.
 *   local_part   host [n_qb] or NULL: when given, the local-change partials are written
 *                as by dit_partition_attention with a workspace (finish them with
 *                dit_local_change_finalize); when NULL they are not.
 *   workspace    device, required, of workspace_bytes >= dit_attn_workspace_bytes(...):
 *                the local-change partials and a chunk counter that the call clears on its
 *                stream before the launch.  Calls that share a workspace must not run at the
 *                same time.
 * pre_o / pre_lse must not overlap the cache, q, k or v.  Errors as for
 * dit_partition_attention (bf16 cache only; DIT_ERR_WORKSPACE without a workspace).
 */
int dit_partition_attention_premerge(const void *q, const void *k, const void *v,
                                     int B, int S_q, int S_kv, int H, int D,
                                     const int32_t *q_offsets, int n_qb,
                                     const int32_t *kv_offsets, int P,
                                     const int32_t *local_part,
                                     const uint8_t *recompute,
                                     const uint8_t *cache_valid,
                                     void *cache_o, float *cache_lse,
                                     float softmax_scale,
                                     void *pre_o, float *pre_lse,
                                     void *workspace, size_t workspace_bytes,
                                     void *stream);

/*
 * State merge: for every query row and head, compose the P cached states (all P slots,
 * as the partition-attention call left them) into out / lse by LSE-weighted combination in
 * fp32; states with lse = -inf carry no weight; if every state is empty, out = 0 and
 * lse = -inf.
 *   importance_out     device [B, n_qb, P] f32 or NULL (anchor steps): the partition
 *                      importance of dit_importance, computed in the same pass from the merge
 *                      weights (per-workgroup partial sums in the workspace, then a
 *                      fixed-order reduction per block and partition).  Needs q_offsets
 *                      [n_qb + 1] and the workspace of dit_attn_workspace_bytes; when
 *                      importance_out is NULL they are ignored and may be NULL.
 */
int dit_state_merge(const void *cache_o, const float *cache_lse,
                    int B, int S_q, int H, int D, int P,
                    void *out, float *lse,
                    const int32_t *q_offsets, int n_qb,
                    float *importance_out,
                    void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * Compressed state cache (the cache compression the pages name as future work: DiTango,
 * technical summary, "Significance and Claims", limitations).  Same operation as
 * dit_partition_attention and dit_state_merge, with each cached O_p slot held as OCP fp8
 * e4m3 codes plus one f32 scale per (partition, batch, head, row):
 *   cache_q8     [P, B, S_q, H, D] u8    code c of element x: the e4m3 value nearest
 *                                        x / s (round to nearest, ties to even)
 *   cache_scale  [P, B, S_q, H] f32      s = max_d |O_p| / 448 over the row-head's D values
 *                                        (0 for an all-zero state: codes 0)
 *   cache_lse    as for the bf16 cache
 * The slot's value is s * e4m3(c); per element it is within max(2^-4 |x|, 2^-10 s) of the
 * fp32 state.  Per row-head and plane the cache holds D + 8 bytes instead of 2 D + 4.
 * The local-change partials of dit_partition_attention_fp8 compare the dequantized new and old slot
 * values.  dit_state_merge_fp8 folds each plane's scale into its merge weight,
 * out = sum_p s_p e^{lse_p - lse} e4m3(c_p), accumulated in fp32, written as bf16; its
 * importance arguments are those of dit_state_merge (the weights without the scales).
 * Argument checks and errors as for the bf16 calls (cache_valid included: reuse of a slot
 * marked never computed is DIT_ERR_CACHE_INVALID); cache_scale must be non-NULL.
 * dit_state_merge_fp8 reads every slot: call it only after a dit_partition_attention_fp8
 * call that was given the validity bitmap and returned DIT_OK.
 */
int dit_partition_attention_fp8(const void *q, const void *k, const void *v,
                                int B, int S_q, int S_kv, int H, int D,
                                const int32_t *q_offsets, int n_qb,
                                const int32_t *kv_offsets, int P,
                                const int32_t *local_part,
                                const uint8_t *recompute,
                                const uint8_t *cache_valid,
                                void *cache_q8, float *cache_scale, float *cache_lse,
                                float softmax_scale,
                                void *workspace, size_t workspace_bytes,
                                void *stream);

int dit_state_merge_fp8(const void *cache_q8, const float *cache_scale, const float *cache_lse,
                        int B, int S_q, int H, int D, int P,
                        void *out, float *lse,
                        const int32_t *q_offsets, int n_qb,
                        float *importance_out,
                        void *workspace, size_t workspace_bytes,
                        void *stream);

/*
 * Masked state merge: like dit_state_merge, but row r of query block i composes only the
 * cache planes p with plane_select[i * P + p] = 1 (host [n_qb * P], values 0/1), plus the
 * extra state (extra_o [B, S_q, H, D] bf16, extra_lse [B, H, S_q] f32) when both pointers
 * are non-NULL.  With nothing selected and no extra state, out = 0 and lse = -inf.
 * This is the one-GPU form of filling compute bubbles with reuse work ("Methodology §2,
 * Pipeline Orchestration"): the reused states can be pre-merged into a partial state on a
 * second stream while dit_partition_attention writes the recomputed slots (disjoint memory),
 * then the fresh states and the partial are merged.  out/lse may be the extra state itself
 * only if they are not also read by another stream at the same time.
 */
int dit_state_merge_masked(const void *cache_o, const float *cache_lse,
                           int B, int S_q, int H, int D, int P,
                           const int32_t *q_offsets, int n_qb,
                           const uint8_t *plane_select,
                           const void *extra_o, const float *extra_lse,
                           void *out, float *lse,
                           void *stream);

/*
 * Dynamic group compose ("Methodology §2, Dynamic Group Compose"): compose the cached
 * states of runs of adjacent partitions into coarser states, with no recomputation.
 * Output plane g is the LSE-weighted combination of input planes
 * group_offsets[g] .. group_offsets[g+1]-1 (same rule as dit_state_merge, fp32 math).
 *   cache_o, cache_lse   device in: [P_in, B, S_q, H, D] bf16, [P_in, B, S_q, H] f32
 *   group_offsets        host [G+1]: 0 = first, strictly increasing, last = P_in
 *   out_o, out_lse       device out: [G, B, S_q, H, D] bf16, [G, B, S_q, H] f32; must not
 *                        overlap the input planes
 * Applying it again to its output coarsens further (composition is associative).  After
 * composing, later steps run with the group offsets as partition offsets and the composed
 * planes as the state cache.
 */
int dit_state_compose(const void *cache_o, const float *cache_lse, int P_in,
                      const int32_t *group_offsets, int G,
                      int B, int S_q, int H, int D,
                      void *out_o, float *out_lse,
                      void *stream);

/*
 * Partition importance from the cached states and the merged lse of this step:
 * importance_out[b, i, p] = mean over rows r of block i and heads h of
 * e^{cache_lse[p, b, r, h] - lse[b, h, r]}  (0 for empty partitions).  A second pass over the
 * stored lse planes; it needs no workspace (dit_state_merge computes the same inside the
 * merge).
 */
int dit_importance(const float *cache_lse, const float *lse,
                   int B, int S_q, int H, int P,
                   const int32_t *q_offsets, int n_qb,
                   float *importance_out,
                   void *stream);

/*
 * Finish the local-change reduction started by dit_partition_attention (the partials in its
 * workspace): delta_out[b, i] = sqrt(sum (O_new - O_old)^2) / sqrt(sum O_old^2) over block
 * i's rows, heads and D (NaN if the old state is all zero).
 */
int dit_local_change_finalize(const void *workspace, size_t workspace_bytes,
                              int B, int S_q, int H, int D,
                              const int32_t *q_offsets, int n_qb,
                              float *delta_out,
                              void *stream);

/* ------------------------------------------------------------------------------------
 * Host-side group planner ("Methodology §1, Anchor-Guided Selection Planner").
 *
 * Groups are runs of adjacent partitions given by group_offsets [G+1] (0 = first, strictly
 * increasing, last = P).  Each block's local group (the group holding local_part[i]) is
 * always recomputed.  Modes:
 *   DIT_PLAN_WDELTA   anchor step when step % anchor_every == 0 (all partitions); otherwise
 *                     the K-1 other groups with the largest predicted reuse error
 *                     e_ig = w_ig * sum_{tau = last_ig+1..step} dhat_i(tau)
 *                     (w_ig = sum of the member partitions' importance at the last anchor;
 *                     last_ig = step of the group's last recompute; dhat_i(tau) = delta_i(tau)
 *                     where observed, else the latest delta observed before tau, else 1.0),
 *                     ties broken by smaller group distance min_{p in g} |p - local_part[i]|,
 *                     then by lower group index.  e is evaluated in double precision.
 *   DIT_PLAN_DISTANCE the K-1 other groups ordered by (distance, index); never an anchor.
 *   DIT_PLAN_ANCHOR   every step is an anchor step.
 * K = recompute_groups (1 <= K <= G).
 * ------------------------------------------------------------------------------------ */
typedef struct dit_planner dit_planner;

enum { DIT_PLAN_WDELTA = 0, DIT_PLAN_DISTANCE = 1, DIT_PLAN_ANCHOR = 2 };

/* Create a planner; *out receives the handle (free with dit_planner_destroy). */
int dit_planner_create(int n_qb, int P, const int32_t *group_offsets, int G,
                       const int32_t *local_part, int anchor_every, int recompute_groups,
                       int mode, dit_planner **out);

/* Decide step `step`: mask_out host [n_qb * P] (1 = recompute); groups_out host
 * [n_qb * G] or NULL receives the chosen groups per block (local group first, then in rank
 * order; unused entries -1).  Records the chosen groups as refreshed at `step`. */
int dit_planner_next(dit_planner *pl, int step, uint8_t *mask_out, int32_t *groups_out);

/* Report step `step`'s measurements: importance host [n_qb * P] f32 or NULL (replaces
 * the group importance; normally given at anchor steps), delta host [n_qb] f32 or NULL
 * (non-finite entries are ignored). */
int dit_planner_observe(dit_planner *pl, int step, const float *importance, const float *delta);

/* Predicted reuse error e_ig (host [n_qb * G] doubles) that dit_planner_next(step) would
 * rank by, for inspection and testing. */
int dit_planner_scores(const dit_planner *pl, int step, double *scores_out);

void dit_planner_destroy(dit_planner *pl);

#ifdef __cplusplus
}
#endif

#endif /* DIT_ATTN_H */
