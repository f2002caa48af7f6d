/*
 * mc2.h -- C ABI of the MI355X (gfx950) compute core of the MC2 fused
 * compute/communication operators: one GPU's share of MatmulReduceScatter,
 * AllGatherMatmul and the MoE AllToAllv+GroupedMatmul dispatch/combine pair.
 *
 * Sources (page title, section):
 *   [RS]  torch_npu.npu_mm_reduce_scatter_base API doc -- "功能说明" (formulas),
 *         "函数原型" (prototype), "参数说明" (arguments), "返回值说明" (return).
 *   [AG]  CANN hccl issue 158 (AllGather vs AllGather+MatMul latency on Atlas A2)
 *         -- the benchmark script's npu_all_gather_base_mm call.
 *   [EP]  "NPU Training Operators - MC2" -- "执行路径" (execution path of
 *         ep_mc2_forward), "迁移检查" (pre-migration checks), "验证项"
 *         (validation table).
 *
 * Conventions shared by every entry point:
 *   - All pointers are device pointers unless stated; the caller owns every
 *     buffer (workspaces included). The library allocates no device memory.
 *   - Every call validates its arguments on the host first. On failure it
 *     returns a nonzero mc2_status and enqueues nothing.
 *   - On success the work is enqueued on `stream` and the call returns at once;
 *     results are ordered on that stream. A launch failure reported by the HIP
 *     runtime returns MC2_ERR_HIP.
 *   - Data-dependent faults (expert ids out of range, inconsistent counts,
 *     indices out of range) never force a host synchronisation: the kernels
 *     OR an MC2_DEVERR_* bit into *dev_err when dev_err is not NULL, and skip
 *     the offending data so that every access stays in bounds.
 *   - Matrices are row-major and densely packed. Base pointers must be 16-byte
 *     aligned. No C++ exception crosses this interface.
 */
#ifndef MC2_H_
#define MC2_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mc2_status {
  MC2_OK = 0,
  MC2_ERR_NULL = 1,        /* a required pointer is NULL                    */
  MC2_ERR_SHAPE = 2,       /* a size or shape constraint is violated        */
  MC2_ERR_DTYPE = 3,       /* a dtype or dtype combination is not allowed   */
  MC2_ERR_UNSUPPORTED = 4, /* valid per the pages but not built here        */
  MC2_ERR_HIP = 5,         /* the HIP runtime reported a launch error       */
  MC2_ERR_WORKSPACE = 6,   /* workspace too small                           */
  MC2_ERR_ALIGN = 7        /* a pointer or row pitch is not 16-byte aligned */
} mc2_status;

typedef enum mc2_dtype {
  MC2_F16 = 0,
  MC2_BF16 = 1,
  MC2_I8 = 2,
  MC2_F32 = 3, /* output only, test extension: the value before the cast  */
  MC2_I32 = 4  /* output only, test extension: the raw int8 accumulator   */
} mc2_dtype;

typedef enum mc2_act { MC2_ACT_NONE = 0, MC2_ACT_SWIGLU = 1 } mc2_act;

/* Bits ORed into *dev_err by the kernels. */
#define MC2_DEVERR_EXPERT_ID 1u /* an expert id outside [0, num_experts)      */
#define MC2_DEVERR_COUNTS 2u    /* recv_counts disagree with send_counts, or   */
                                /* the counted rows exceed a buffer's rows     */
#define MC2_DEVERR_INDEX 4u     /* an unpermute index outside the y buffer     */
#define MC2_DEVERR_TIMEOUT 8u   /* an input ready flag did not arrive within
                                   the spin limit (or, never expected, a
                                   K-split partner's partial within ~1 s)     */

/*
 * mc2_mm_rs_local -- MatmulReduceScatter compute share [RS].
 *
 *   basic:  P = sum_{w < nsim} (x1_w @ x2_w + bias)
 *   quant:  P = sum_{w < nsim} (x1_scale[i] * x2_scale[j]) * (x1_w @ x2_w + bias)
 *
 * and destination chunk c (c < world_size) is rows [c*m/W, (c+1)*m/W) of the
 * (m, n) result `out`. nsim == 1 computes this rank's own partial (the real
 * per-rank share); nsim == world_size sums the W stacked partials on one
 * device (the reduce-scatter arithmetic), accumulating all W*k products in
 * fp32 (or int32) and rounding once to the output dtype.
 *
 *   x1      (nsim, m, k) in_dtype             x2  (nsim, k, n), or (nsim, n, k)
 *                                                 when x2_trans != 0
 *           x2_trans is the page's transposed x2 (x2 may be passed transposed,
 *           the input may not): a Linear weight held (n, k). It is the faster
 *           layout here, since each x2 operand is one 16-byte LDS read instead
 *           of two transposing 8-byte reads.
 *   in_dtype MC2_F16, MC2_BF16 or MC2_I8 (x1 and x2 share it)
 *   bias    NULL or (n): in_dtype for F16/BF16 inputs; BF16 for I8 inputs
 *           (an extension: the page allows only a float bias of the input's
 *           dtype). The literal formula adds it inside every partial.
 *   x1_scale (m) fp32 per token, x2_scale (n) fp32 per channel: required for
 *           I8 unless out_dtype is MC2_I32; must be NULL otherwise.
 *   out_dtype  F16/BF16 inputs: equal to in_dtype, or MC2_F32 (test).
 *              I8 inputs: MC2_BF16 (the page's default), MC2_F16, MC2_F32
 *              (test: the fp32 dequantised value) or MC2_I32 (test: the raw
 *              accumulator; no scales, no bias, nsim == 1).
 *   out     (m, n) out_dtype, written chunk by chunk.
 *
 * Constraints [RS "参数说明"]: m % world_size == 0; 256 <= k < 65535;
 * world_size in {1, 2, 4, 8, 16, 32} (1 is a test extension); 0 <= rank < W;
 * nsim in {1, world_size}, and nsim == 1 for I8. Built restrictions: k % 8 == 0
 * (k % 16 for I8) and n % 8 == 0 (n % 16 for I8) so rows stay 16-byte aligned.
 *
 * Chunk schedule and ready flags: chunks are computed in the order
 * (rank + 1 + i) mod W, i = 0..W-1, so that the chunk this rank keeps comes
 * last. comm_turn is the split granularity [RS "参数说明": comm_turn, of which
 * that version accepts only 0]: 0 (the default) or 1 keeps each chunk whole;
 * S > 1 cuts every chunk of m_c = m/W rows into S pieces of q = m_c / S rows
 * in row order, one more row for each of the first m_c % S pieces, and each
 * piece (segment g = c*S + j) gets its own ready flag; 1 <= S <= m_c, else
 * MC2_ERR_SHAPE. Pieces are computed chunk by chunk in the order above, in
 * row order inside a chunk. With G = W * max(comm_turn, 1) segments: when
 * ready_flags is not NULL, ready_flags and flag_counters point to G uint32,
 * the counters in device memory and zero before the first call (the library
 * leaves them zero after each call), the flags in device or host-pinned
 * memory; the last tile to finish segment g stores ready_flags[g] = epoch
 * with release ordering at system scope once every byte of segment g is
 * visible. epoch must be nonzero and should differ between calls. Both flag
 * pointers NULL disables flags.
 *
 * K split of the last round (stream-K for a thin tail) [RS "参数说明":
 * comm_turn, the split granularity; the split here is of the work, not of
 * the chunks]: with 256 x 256 tiles, a last dispatch round (one tile per CU)
 * that is at most half full would leave CUs idle. With a workspace, each of
 * its tiles runs as two K halves on two workgroups that exchange fp32 (int32)
 * partials: the tile's value is then (sum over the first half of the K loop)
 * + (sum over the second), one addition that gives the same bits whichever
 * workgroup performs it. Without one, such a round runs as 128-row halves.
 * (The split is switched off in this build while a fix of its partial
 * stores awaits its device check: a workspace is accepted and ignored.)
 *   workspace        NULL (no K split) or a 16-byte aligned buffer of
 *                    workspace_bytes; its first 4096 bytes (control words)
 *                    must be zero before the first call, and every call
 *                    leaves them zero. mc2_split_workspace_size() bytes
 *                    suffice for every call on the current device; a smaller
 *                    one disables the split where it does not fit. Calls that
 *                    overlap in time must not share a workspace.
 * int8 results are exact whatever the schedule. Float results do not depend
 * on comm_turn except through which tiles fall into a split last round:
 * there the two fp32 halves add with one extra fp32 rounding. A call with the
 * same arguments always gives the same bits.
 */
int mc2_mm_rs_local(const void* x1, const void* x2, int64_t m, int64_t k, int64_t n,
                    int world_size, int rank, int nsim, int x2_trans, int in_dtype,
                    const void* bias, const float* x1_scale, const float* x2_scale,
                    int out_dtype, void* out, uint32_t* ready_flags,
                    uint32_t* flag_counters, uint32_t epoch, int comm_turn, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of a K-split workspace that covers every call of mc2_mm_rs_local,
 * mc2_ag_mm_local and mc2_ag_mm_local_inflags on the current device: 4096
 * bytes of control words plus two 128 KiB partial slots per pair of
 * workgroups (half the compute units). 32 MiB + 4 KiB on 256 CUs.
 */
size_t mc2_split_workspace_size(void);

/*
 * Policy of the K split, process-wide (tuning and tests):
 *   MC2_SPLIT_PAIR   (default) the first K half to finish waits for its
 *                    partner when the partner is running, and each finalizes
 *                    one 128-row half of the tile (128 KiB moved each way);
 *   MC2_SPLIT_ALONE  the first K half to start never waits: it hands its
 *                    whole 256 KiB partial over and the other finalizes the
 *                    whole tile.
 * Both give bitwise the same results. Returns MC2_ERR_SHAPE for another value.
 */
#define MC2_SPLIT_PAIR 0
#define MC2_SPLIT_ALONE 1
int mc2_set_split_policy(int policy);

/*
 * mc2_ag_mm_local -- AllGatherMatmul compute share [AG]: out = allgather(x1) @ x2
 * (+ bias).
 *
 *   x_gathered (W*m_c, k): the W gathered chunks, chunk c = rows of rank c.
 *   x2 (k, n), or (n, k) when x2_trans != 0; bias NULL or (n); all in_dtype
 *   (MC2_F16 or MC2_BF16). out (W*m_c, n) in_dtype.
 *
 * Chunks are computed in the order (rank + i) mod W, starting with the chunk
 * this rank owns. comm_turn pieces, ready flags and the K-split workspace
 * as for mc2_mm_rs_local (W * max(comm_turn, 1) segments,
 * 0 <= comm_turn <= m_c). Constraints: k >= 1, k % 8 == 0, n % 8 == 0,
 * m_c >= 1, world_size in {1, 2, 4, 8, 16, 32}.
 */
int mc2_ag_mm_local(const void* x_gathered, const void* x2, int64_t m_c, int64_t k,
                    int64_t n, int world_size, int rank, int x2_trans, int in_dtype,
                    const void* bias, void* out, uint32_t* ready_flags,
                    uint32_t* flag_counters, uint32_t epoch, int comm_turn, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/*
 * mc2_ag_mm_local_inflags -- mc2_ag_mm_local whose tiles wait for their input
 * segment: the consumer side of the AllGatherMatmul pipeline [AG, CANN hccl
 * issue 158; MC2 "执行路径": communication and computation of different chunks
 * overlap]. Input arrives at the granularity of the output segments
 * (comm_turn pieces, segment g = c*S + j as for mc2_mm_rs_local). Before a
 * tile reads segment g of gathered chunk c (c != rank: the own chunk is
 * local), one thread polls in_flags[g] until it equals in_epoch, then takes
 * a system-scope acquire fence, so every byte written to that segment before
 * the producer's release of in_flags[g] is visible.
 *
 *   in_flags   W * max(comm_turn, 1) uint32 in memory the GPU can read
 *              (device, or host-pinned);
 *              written by an agent that does not need this kernel to make
 *              progress (a copy engine, a peer, the host): the kernel never
 *              raises them itself, so it cannot deadlock on them.
 *   in_epoch   value that marks chunk c ready (nonzero).
 *   spin_limit polls before a tile gives up (>= 1; a poll sleeps ~64 clocks).
 *              A tile that gives up ORs MC2_DEVERR_TIMEOUT into *dev_err and
 *              computes on the data it finds, so the call always completes and
 *              the ready-flag counters stay consistent; its output is then
 *              undefined.
 *   dev_err    NULL or one int32.
 * Other arguments, results and errors as mc2_ag_mm_local; in_flags NULL is
 * MC2_ERR_NULL, in_epoch == 0 or spin_limit == 0 is MC2_ERR_SHAPE.
 */
int mc2_ag_mm_local_inflags(const void* x_gathered, const void* x2, int64_t m_c, int64_t k,
                            int64_t n, int world_size, int rank, int x2_trans, int in_dtype,
                            const void* bias, void* out, uint32_t* ready_flags,
                            uint32_t* flag_counters, uint32_t epoch, int comm_turn,
                            const uint32_t* in_flags,
                            uint32_t in_epoch, uint32_t spin_limit, int32_t* dev_err,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * MatmulAllReduce local share ["NPU Training Operators - MC2", "底层 API 对照":
 * npu_mm_all_reduce_base fuses the TP matmul with all_reduce; same page,
 * "风险": MC2 may cost precision]. Every rank ends with the full
 *
 *   P = sum_{w < W} (x1_w @ x2_w + bias)        x1 (W, m, k), x2 (W, k, n) or
 *                                               (W, n, k) with x2_trans
 *
 * (m, n) in in_dtype (MC2_F16 or MC2_BF16); no row chunking, so m need not be
 * divisible by W. rounding selects how the W partials are combined:
 *   MC2_AR_ONE_ROUNDING  one fp32 accumulator over all W*k products, rounded
 *                        once (the fused kernel; no workspace);
 *   MC2_AR_RANK_ROUNDED  each rank's partial rounded to in_dtype (what a rank
 *                        sends), the W rounded partials summed exactly in
 *                        rank order and rounded once;
 *   MC2_AR_HOP_ROUNDED   as RANK_ROUNDED, but the running sum rounded to in_dtype
 *                        after every addition (a ring reduction carried out
 *                        in the storage dtype).
 * The last two keep the W partials in `workspace` (caller-owned, 16-byte
 * aligned, >= mc2_mm_ar_workspace_size bytes, no initialisation needed;
 * NULL is MC2_ERR_NULL, smaller is MC2_ERR_WORKSPACE); once the stream has
 * run the call, it holds the rounded partials as (W, m, n) in in_dtype. Constraints: W in
 * {1, 2, 4, 8, 16, 32}; 1 <= k < 65535; k % 8 == 0; n % 8 == 0.
 *
 * mc2_ar_sum_local is the combining step alone: out (elems) = the sum of the
 * W stored partials (W, elems) under MC2_AR_RANK_ROUNDED or
 * MC2_AR_HOP_ROUNDED, summed in fp64 in rank order and rounded to dtype with
 * round-to-nearest-even. Constraints: 1 <= W <= 32; elems % 8 == 0;
 * 16-byte aligned pointers.
 */
#define MC2_AR_ONE_ROUNDING 0
#define MC2_AR_RANK_ROUNDED 1
#define MC2_AR_HOP_ROUNDED 2

size_t mc2_mm_ar_workspace_size(int64_t m, int64_t n, int world_size, int in_dtype, int rounding);

int mc2_mm_ar_local(const void* x1, const void* x2, int64_t m, int64_t k, int64_t n,
                    int world_size, int x2_trans, int in_dtype, const void* bias, int rounding,
                    void* out, void* workspace, size_t ws_bytes, hipStream_t stream);

int mc2_ar_sum_local(const void* partials, int world_size, int64_t elems, int dtype,
                     int rounding, void* out, hipStream_t stream);

/*
 * mc2_moe_histc -- token count per expert [EP "执行路径": torch.histc with
 * bins = num_experts, min = 0, max = num_experts]:
 *   counts[e] = #{ i < n_ids : sel[i] == e },  0 <= e < num_experts.
 * Ids outside [0, num_experts) are not counted and set MC2_DEVERR_EXPERT_ID.
 * sel (n_ids) int32; counts (num_experts) int32, fully overwritten.
 * Constraints: n_ids >= 0, 1 <= num_experts <= 1024.
 */
int mc2_moe_histc(const int32_t* sel, int64_t n_ids, int num_experts, int32_t* counts,
                  int32_t* dev_err, hipStream_t stream);

/* Workspace bytes that mc2_moe_permute needs for T tokens, K slots, E experts. */
size_t mc2_moe_permute_workspace_size(int64_t T, int K, int num_experts);

/*
 * mc2_moe_permute -- stable grouping of the T*K routed slots by expert
 * [EP "执行路径": permute(hidden_states, selected_experts)].
 *
 * Slot s = t*K + k routes token t to expert sel[s]. Slots are sorted by expert,
 * ties kept in slot order. With n_valid slots whose ids lie in [0, E):
 *   sorted_idx[p]      = slot at position p (p < n_valid), -1 for p >= n_valid
 *   unpermute_idx[s]   = position of slot s, -1 if sel[s] is out of range
 *   expert_offsets[e]  = first position of expert e; expert_offsets[E] = n_valid
 *   permuted[p]        = x[sorted_idx[p] / K]  (a byte copy of the row)
 * x (T, H) and permuted (T*K, H) hold 16-bit elements (bf16 or fp16); rows
 * p >= n_valid of permuted are not written. workspace: at least
 * mc2_moe_permute_workspace_size(T, K, E) bytes, 16-byte aligned, contents
 * need not be initialised. Constraints: T >= 1, 1 <= K <= 64,
 * 1 <= E <= 1024, H % 8 == 0, T*K < 2^31.
 */
int mc2_moe_permute(const void* x, int64_t T, int64_t H, const int32_t* sel, int K,
                    int num_experts, void* permuted, int32_t* sorted_idx,
                    int32_t* unpermute_idx, int32_t* expert_offsets, void* workspace,
                    size_t ws_bytes, int32_t* dev_err, hipStream_t stream);

/*
 * mc2_moe_permute_noalloc -- mc2_moe_permute for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). Same arguments, results and errors as
 * mc2_moe_permute, without the workspace: the counting workspace is a
 * library-owned device array of MC2_PERMUTE_SCRATCH_BYTES bytes per device
 * (held until the process ends). The call itself allocates nothing.
 * Returns MC2_ERR_WORKSPACE when mc2_moe_permute_workspace_size(T, K, E)
 * exceeds MC2_PERMUTE_SCRATCH_BYTES, i.e. when E * ceil(T / floor(256 / K))
 * + E exceeds 1048576 four-byte entries (131072 tokens at K = 8 and E = 128
 * fit; the MoE workload's 32768 tokens use an eighth). Every call on one
 * device shares that device's array: calls that overlap on one device
 * (concurrent streams) race and must be ordered by the caller.
 */
#define MC2_PERMUTE_SCRATCH_BYTES ((size_t)4 << 20)

int mc2_moe_permute_noalloc(const void* x, int64_t T, int64_t H, const int32_t* sel, int K,
                            int num_experts, void* permuted, int32_t* sorted_idx,
                            int32_t* unpermute_idx, int32_t* expert_offsets, int32_t* dev_err,
                            hipStream_t stream);

/*
 * mc2_gmm_dispatch -- GroupedMatmul part of the dispatch segment
 * [EP "执行路径": AllToAllv -> GroupedMatmul(fc1), then swiglu].
 *
 * This rank (ep_rank) owns experts [ep_rank*E_l, (ep_rank+1)*E_l) of
 * num_experts; send_counts (num_experts) are the per-expert row counts of the
 * permuted send buffer and recv_counts (world_size_src * E_l, source-rank
 * major) the rows received per (source rank, local expert). With one source
 * rank (world_size_src == 1, the only value built here) the received rows of
 * local expert g are the send buffer's rows of expert ep_rank*E_l + g, and
 * recv_counts must equal those send counts (else MC2_DEVERR_COUNTS and nothing
 * is computed). For each local expert g, on its rows R_g:
 *   act == MC2_ACT_NONE:   h = R_g @ w1[g]                      -> (rows, I2)
 *   act == MC2_ACT_SWIGLU: a = R_g @ w1[g]; h = silu(a[:, :I2/2]) * a[:, I2/2:]
 *                          with silu(g) = g / (1 + exp(-g))       -> (rows, I2/2)
 * accumulated in fp32 and stored as bf16, group after group from row 0 of h_out.
 *
 *   send_buf (send_rows, H) bf16; w1 (E_l, H, I2) bf16 (gate columns [0, I2/2),
 *   up columns [I2/2, I2)); h_out (h_rows, I2 or I2/2) bf16. Counts are read on
 *   the device only. Constraints: H % 8 == 0, I2 % 16 == 0, H >= 1.
 */
int mc2_gmm_dispatch(const void* send_buf, int64_t send_rows, const int32_t* send_counts,
                     const int32_t* recv_counts, int world_size_src, int ep_rank,
                     int num_experts, int local_experts, const void* w1, int64_t H,
                     int64_t I2, int act, void* h_out, int64_t h_rows, int32_t* dev_err,
                     hipStream_t stream);

/*
 * mc2_gmm_combine -- GroupedMatmul part of the combine segment
 * [EP "执行路径": GroupedMatmul(fc2) -> AllToAllv, counts swapped].
 *
 * For each local expert g on its rows of h (group after group from row 0):
 * y = h_g @ w2[g] in fp32, stored as bf16 into combine_buf at the rows the
 * send buffer used for expert ep_rank*E_l + g (with one source rank the
 * return AllToAllv puts the rows back where they were sent from). Other rows
 * of combine_buf are not touched. Count checks as for mc2_gmm_dispatch.
 *
 *   h (h_rows, I) bf16; w2 (E_l, I, H) bf16; combine_buf (combine_rows, H) bf16.
 *   Constraints: I % 8 == 0, H % 8 == 0.
 */
int mc2_gmm_combine(const void* h, int64_t h_rows, const int32_t* recv_counts,
                    const int32_t* send_counts, int world_size_src, int ep_rank,
                    int num_experts, int local_experts, const void* w2, int64_t I,
                    int64_t H, void* combine_buf, int64_t combine_rows, int32_t* dev_err,
                    hipStream_t stream);

/*
 * mc2_moe_unpermute -- weighted return of the routed rows to their tokens
 * [EP "执行路径": unpermute(h, unpermute_indices, probs=routing_weights)]:
 *   out[t] = sum_{k < K} probs[t*K + k] * y_full[unpermute_idx[t*K + k]]
 * accumulated in fp32 in ascending k and stored as bf16. Slots with index -1
 * are skipped; an index >= y_rows is skipped and sets MC2_DEVERR_INDEX.
 *   y_full (y_rows, H) bf16; unpermute_idx (T*K) int32; probs (T*K) fp32;
 *   out (T, H) bf16. Constraints: H % 8 == 0, 1 <= K <= 64.
 */
int mc2_moe_unpermute(const void* y_full, int64_t y_rows, const int32_t* unpermute_idx,
                      const float* probs, int64_t T, int K, int64_t H, void* out,
                      int32_t* dev_err, hipStream_t stream);

/*
 * Backward of the dispatch / combine pair ["NPU Training Operators - MC2",
 * "PR 改动": the two autograd Functions wrap the fused operator in forward
 * and backward; "验证项": fc1 / fc2 gradients are compared with the plain
 * alltoall path]. Gradients of the forward above, on the local rows:
 *
 * mc2_gmm_combine_backward, for each local expert g with rows h_g (of h,
 * group after group from row 0) and output gradient dY_g (the rows of dy_buf
 * that mc2_gmm_combine writes for expert ep_rank*E_l + g):
 *   dA_g  = dY_g @ w2[g]^T                                   (fp32)
 *   act == MC2_ACT_NONE:   dgrad_out rows = dA_g                 (rows, I) bf16
 *   act == MC2_ACT_SWIGLU: with the stored fc1 pre-activation g_saved
 *     (rows, 2I) bf16 = [gate | up], s = 1 / (1 + exp(-gate)):
 *     dgrad_out rows = [dA*up*s*(1 + gate*(1 - s)) | dA*gate*s]  (rows, 2I) bf16
 *   dw2_out[g] = h_g^T @ dY_g                               (E_l, I, H) fp32
 * mc2_gmm_dispatch_backward, with dG_g the rows of dg (group after group
 * from row 0) and R_g this rank's rows of send_buf:
 *   dx_buf rows of expert ep_rank*E_l + g = dG_g @ w1[g]^T  (bf16; other rows
 *   untouched);  dw1_out[g] = R_g^T @ dG_g                   (E_l, H, I2) fp32
 * Buffers: dy_buf (dy_rows, H); h (h_rows, I); g_saved (h_rows, 2I) or NULL
 * with MC2_ACT_NONE; dgrad_out (h_rows, I or 2I); dg (dg_rows, I2); send_buf
 * and dx_buf (send_rows / dx_rows, H); all bf16, rows packed. Weights as in
 * the forward: w2 (E_l, I, H), w1 (E_l, H, I2), bf16. Counts
 * and their checks as for mc2_gmm_dispatch (MC2_DEVERR_COUNTS, nothing
 * computed, on a mismatch or when rows exceed a buffer). An expert with no
 * rows gets a zero weight gradient. A weight gradient over more than L rows
 * of one expert is split into slices of L rows whose partial tiles are summed
 * in slice order (the result does not depend on timing); L is the local rows
 * times the output tiles per expert (256 x 256) over the CUs, rounded down to
 * a multiple of 2048, and at least 4096. workspace:
 * caller-owned, 16-byte aligned, at least
 * mc2_gmm_backward_workspace_size(rows, E_l, M, N) bytes with (rows, M, N) =
 * (h_rows, I, H) for the combine backward and (send_rows, H, I2) for the
 * dispatch backward (tile counters and partial tiles; the weight gradient
 * reads h and the send rows in place); no initialisation needed. Constraints:
 * I, H, I2 multiples of 8.
 */
size_t mc2_gmm_backward_workspace_size(int64_t rows, int local_experts, int64_t M, int64_t N);

int mc2_gmm_combine_backward(const void* dy_buf, int64_t dy_rows, const int32_t* recv_counts,
                             const int32_t* send_counts, int world_size_src, int ep_rank,
                             int num_experts, int local_experts, const void* w2, int64_t I,
                             int64_t H, const void* h, int64_t h_rows, const void* g_saved,
                             int act, void* dgrad_out, float* dw2_out, void* workspace,
                             size_t ws_bytes, int32_t* dev_err, hipStream_t stream);

int mc2_gmm_dispatch_backward(const void* dg, int64_t dg_rows, const int32_t* recv_counts,
                              const int32_t* send_counts, int world_size_src, int ep_rank,
                              int num_experts, int local_experts, const void* w1, int64_t H,
                              int64_t I2, const void* send_buf, int64_t send_rows, void* dx_buf,
                              int64_t dx_rows, float* dw1_out, void* workspace, size_t ws_bytes,
                              int32_t* dev_err, hipStream_t stream);

/* Human-readable name of an mc2_status value (static storage). */
const char* mc2_status_string(int status);

/* Library version string (static storage). */
const char* mc2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MC2_H_ */
