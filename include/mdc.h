/*
 * mdc.h -- C ABI of the MoE dispatch/combine library (libmdc.so) for AMD
 * Instinct MI355X (gfx950).
 *
 * The library implements one GPU's share of expert-parallel MoE dispatch and
 * combine.  The W ranks of the expert-parallel group are *virtual*: their
 * buffers live on the same GPU, so the cross-rank AllToAllV becomes a local
 * permutation.
 *
 * Sources (cited by page title and section):
 *   [TL]  "dispatch_combine_shmem.py" (TileLang-Ascend example): moe_dispatch_kernel
 *         (send loop "AlltoAllDispatch", "SetStatus", "GetCumSum", local data copy,
 *         "UpdateTokenNumsOut") and moe_combine_kernel (weighted sum).
 *   [CV4] "aclnnMoeDistributeCombineV4": Function (formula), Function Prototype
 *         (two-phase API and parameter table), Return Value, Constraints
 *         (shape-variable table, API matching constraints, determinism).
 *   [PTO] "PTO MegaMoE Dispatch + Combine Fusion Example": FrontReorder Stage,
 *         Dispatch Stage, GMM1 / SwiGLU / GMM2 Stages, Combine / Unpermute Stages,
 *         Memory Layout and HCCL Window.
 *
 * Conventions shared by every entry point
 *   - Every tensor argument is a device pointer owned by the caller; the
 *     library never allocates, frees or synchronises.  Work is enqueued on
 *     `stream` (a hipStream_t; NULL = the default stream) and the call returns
 *     at once.  Inputs must stay alive and unmodified until the enqueued work
 *     has run.
 *   - bf16 tensors are arrays of 16-bit bf16 bit patterns; bf16 row tensors
 *     (x, expand_x, shared_expert_x, x_out) must be 16-byte aligned.
 *   - Expert e lives on rank e / L as local expert e % L, L = E / W
 *     ([TL] send loop; [CV4] shape-variable table, localExpertNum).
 *   - A route is (s, t, k): source rank s, token t, top-k slot k.
 *   - Argument errors are reported synchronously by the return value, before
 *     anything is enqueued (codes mirror [CV4] Return Value: null tensor,
 *     malformed arguments, values outside the supported range).  Conditions
 *     found in the data (ids outside [0, E+Z+C), too many rows for the
 *     capacity, a pipeline wait that ran out) are not errors: the device
 *     reports them in the workspace's status block (mdc_device_status).
 *   - Results are bitwise deterministic: no floating-point atomics, fixed
 *     summation order ([CV4] Constraints, deterministic computation).
 *   - Calls that share a workspace must not overlap (use one stream or order
 *     them); otherwise the library keeps no state and is reentrant.
 */
#ifndef MDC_H
#define MDC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MDC_ABI_VERSION 4
#define MDC_MAX_TOPK 16        /* 0 < K <= 16 ([CV4] shape-variable table) */
#define MDC_MAX_LOCAL_EXPERTS 2048
#define MDC_MAX_COMBINE_WORLD 64 /* W limit of mdc_combine (pointer tables travel by value) */

typedef enum {
    MDC_OK = 0,
    MDC_ERR_NULLPTR = 1,     /* a required pointer is NULL (cf. ACLNN_ERR_PARAM_NULLPTR, 161001) */
    MDC_ERR_INVALID = 2,     /* the arguments do not describe a well-formed problem: a misaligned
                                tensor, shape fields inconsistent with each other (E % W != 0,
                                H % 8 != 0, rank outside [0, W), a negative size), unknown flag
                                bits, a nonzero reserved field (cf. ACLNN_ERR_PARAM_INVALID, 161002) */
    MDC_ERR_UNSUPPORTED = 3, /* a well-formed problem outside the range this library supports:
                                K > 16, L > 2048, W > 64 for combine, H > 8192 for the quantised
                                dispatch, FFN widths that are not multiples of its tiles, sizes
                                past the 32-bit index limits (cf. ACLNN_ERR_INNER_TILING_ERROR,
                                561002: shape or parameter value outside the supported range) */
    MDC_ERR_WORKSPACE = 4,   /* workspace smaller than the size query returned */
    MDC_ERR_HIP = 5          /* a HIP kernel launch failed */
} mdc_status;

/* Flags (mdc_shape.flags). */
#define MDC_FLAG_FFN_PIPELINE 0x1u   /* mdc_ffn*: run GMM1, the quantisation of g and GMM2 as one
                                        persistent kernel with ready flags between them
                                        (mdc_dispatch_ffn always does) */
#define MDC_FLAG_SPIN_SHIFT 8        /* bits 8..12: if nonzero, s, the pipeline's bounded waits give
                                        up after 2^s polls instead of 2^24 (a test of the time-out
                                        path forces it with a small s) */
#define MDC_FLAG_SPIN_MASK (0x1Fu << MDC_FLAG_SPIN_SHIFT)

/* Device status block.  The first MDC_STATUS_BYTES bytes of the dispatch and FFN
 * workspaces hold one mdc_device_status, which each call rewrites on its stream
 * ([CV4] Return Value: argument errors are returned by the call; conditions
 * found in the data are not errors, so the device reports them here instead).
 * Read it (e.g. copy the 16 bytes to the host) after the call's work has
 * completed; the next call on the same workspace overwrites it. */
#define MDC_STATUS_BYTES 256
typedef struct {
    int32_t dropped_ids;    /* dispatch: active routes of all W sources whose expert id lies
                               outside [0, E + Z + C) (never sent anywhere, no part in combine) */
    int32_t overflow_rows;  /* dispatch: max(0, R - A): received rows not written for lack of
                               capacity */
    int32_t wait_timeouts;  /* FFN pipeline: tiles whose bounded wait for their input rows ran
                               out (GMM1 tiles waiting for dispatched rows in mdc_dispatch_ffn,
                               GMM2 tiles waiting for quantised g); their y rows are NaN */
    int32_t reserved;
} mdc_device_status;

/* Problem shape.  `rank` is the destination rank for dispatch and the source
 * rank whose tokens are combined for combine. */
typedef struct {
    int32_t world;        /* W >= 1 virtual EP ranks */
    int32_t rank;         /* 0 <= rank < W */
    int32_t bs;           /* BS >= 0 tokens per rank */
    int32_t hidden;       /* H > 0, multiple of 8 (one 16-byte vector = 8 bf16) */
    int32_t topk;         /* K, 1..MDC_MAX_TOPK */
    int32_t num_experts;  /* E > 0, multiple of W; L = E / W <= MDC_MAX_LOCAL_EXPERTS */
    int64_t capacity;     /* A >= 0: rows of expand_x / assist_info per rank.
                             [CV4] shape-variable table asks A >= BS*W*min(L, K). */
    int32_t mask_per_route; /* 0: x_active_mask holds one flag per token ([.][BS]);
                               1: one flag per route ([.][BS][K]) ([CV4] parameter
                               notes: a 2D xActiveMask; a token whose K flags are all
                               false takes no part) */
    int32_t zero_experts;   /* Z >= 0: ids in [E, E+Z) are zero experts ([CV4]
                               zeroExpertNum): never dispatched; output 0 in combine */
    int32_t copy_experts;   /* C >= 0: ids in [E+Z, E+Z+C) are copy experts ([CV4]
                               copyExpertNum): never dispatched; output ori_x[t] in
                               combine.  K <= E + Z + C. */
    int32_t flags;          /* MDC_FLAG_* bits; the others must be 0 */
} mdc_shape;

const char* mdc_status_string(mdc_status status);
int32_t mdc_abi_version(void);

/* ------------------------------------------------------------------------
 * Dispatch ([TL] moe_dispatch_kernel; [PTO] FrontReorder + Dispatch stages)
 *
 * For destination rank d = shape->rank, over all W virtual source ranks:
 *   - a route (s, t, k) is sent iff it is active (its token's flag, or its
 *     own flag with mask_per_route) and e = expert_ids[s][t][k] satisfies
 *     d*L <= e < (d+1)*L.  Ids outside [0, E) (zero/copy experts, invalid
 *     ids) are never sent anywhere.
 *   - the received rows are laid out expert-major in the stable order
 *     (local expert le, source s, token t, slot k): row = base(le, s) +
 *     number of earlier routes (t', k') < (t, k) of source s with the same
 *     expert ([TL] send loop: rank-within-expert counts earlier equal ids;
 *     local data copy walks status rows le*W + src; [PTO] Dispatch Stage:
 *     a local expert's rows ordered by source rank).
 *
 * Outputs
 *   ep_recv_counts    [L*W] int32, inclusive prefix of the per-(le, s) counts
 *                     in (le-major, s-minor) order; the last entry is the total
 *                     R of received routes ([TL] GetCumSum / local data copy:
 *                     receive count = begin + count).
 *   expert_token_nums [L] int64, routes received per local expert
 *                     ([TL] UpdateTokenNumsOut).
 *   expand_x          [A][H] bf16: row i = x[s][t] of the route at row i,
 *                     copied bitwise ([TL] send loop row put).
 *   assist_info       [A][3] int32: row i = (s, t, k) ([TL] triplet written
 *                     after the row; [CV4] assistInfoForCombine).
 *   expanded_row_idx  [W][BS][K] int32, the inverse route index ([PTO]
 *                     Memory Layout: expandedRowIdx, route -> expert-major
 *                     row): for every route sent to d the entry is its row, or
 *                     -1 if that row is >= A.  Entries of routes not sent to d
 *                     are left untouched, so the W dispatches of one step fill
 *                     disjoint parts of one shared table.
 *   expand_scales     [A] fp32 or NULL: row i = expert_scales[s][t][k] of the
 *                     route at row i, the weight that travels with the row
 *                     ([CV4] parameter table: expandScalesOptional, the
 *                     dispatch's expandScales output, 1D of shape (A,) in the
 *                     A2 notes).  Written iff expert_scales is given.
 *   workspace status  the dispatch fills the workspace's mdc_device_status
 *                     (dropped_ids, overflow_rows; wait_timeouts = 0).
 *   Only rows [0, min(R, A)) of expand_x / assist_info / expand_scales are
 *   written; rows with index >= A are dropped while the counts still include
 *   them, so overflow shows as ep_recv_counts[L*W-1] > A (and in
 *   overflow_rows).  Rows past the total are untouched.
 *
 * Inputs
 *   x                 [W][BS][H] bf16, the virtual source ranks' tokens.
 *   expert_ids        [W][BS][K] int32.
 *   x_active_mask     [W][BS] uint8 (nonzero = active), or [W][BS][K] with
 *                     mask_per_route, or NULL (all active); any order of active
 *                     and inactive entries is accepted.
 *   expert_scales     [W][BS][K] fp32, the routes' weights, or NULL (then
 *                     expand_scales must be NULL too, unless BS == 0).
 *
 * The call is split in two stages that may be enqueued separately (same
 * stream, same workspace, in this order); mdc_dispatch enqueues both.
 *   mdc_dispatch_layout  route filter, histogram and stable ranks
 *                        ([PTO] FrontReorder Stage); writes only the workspace.
 *   mdc_dispatch_gather  scan, rows, triplets, inverse index, epRecvCounts,
 *                        expertTokenNums, expandScales and the status block
 *                        ([PTO] Dispatch Stage), from the workspace the
 *                        layout stage filled.
 * The workspace size comes from mdc_dispatch_workspace ([CV4] Function
 * Prototype: the first phase returns the workspace size);
 * mdc_dispatch_workspace_size is the same query under its earlier name.
 * ------------------------------------------------------------------------ */
mdc_status mdc_dispatch_workspace(const mdc_shape* shape, size_t* bytes);
mdc_status mdc_dispatch_workspace_size(const mdc_shape* shape, size_t* bytes);

mdc_status mdc_dispatch_layout(const mdc_shape* shape,
                               const int32_t* expert_ids,
                               const uint8_t* x_active_mask,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

mdc_status mdc_dispatch_gather(const mdc_shape* shape,
                               const void* x,
                               const float* expert_scales,
                               void* expand_x,
                               int32_t* assist_info,
                               int32_t* ep_recv_counts,
                               int64_t* expert_token_nums,
                               int32_t* expanded_row_idx,
                               float* expand_scales,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

mdc_status mdc_dispatch(const mdc_shape* shape,
                        const void* x,
                        const int32_t* expert_ids,
                        const uint8_t* x_active_mask,
                        const float* expert_scales,
                        void* expand_x,
                        int32_t* assist_info,
                        int32_t* ep_recv_counts,
                        int64_t* expert_token_nums,
                        int32_t* expanded_row_idx,
                        float* expand_scales,
                        void* workspace, size_t workspace_bytes,
                        void* stream);

/* ------------------------------------------------------------------------
 * mdc_dispatch without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments and results as
 * mdc_dispatch minus the workspace: the workspace is the library's own
 * static device array of MDC_NOALLOC_SCRATCH_BYTES, one per device, held
 * until the process ends.  Shapes whose mdc_dispatch_workspace exceeds that
 * size return MDC_ERR_UNSUPPORTED (at the share shape the workspace is about
 * 0.54 MB; 8 MiB covers about two million routes).  The call allocates
 * nothing; its first call on a device looks up that device's array.  All
 * calls on one device share its array: calls that overlap on one device
 * (other streams, other threads) race and must be ordered by the caller.
 * The status block lives in that array and is not exposed by this call.
 * ------------------------------------------------------------------------ */
#define MDC_NOALLOC_SCRATCH_BYTES (8u << 20)

mdc_status mdc_dispatch_noalloc(const mdc_shape* shape,
                                const void* x,
                                const int32_t* expert_ids,
                                const uint8_t* x_active_mask,
                                const float* expert_scales,
                                void* expand_x,
                                int32_t* assist_info,
                                int32_t* ep_recv_counts,
                                int64_t* expert_token_nums,
                                int32_t* expanded_row_idx,
                                float* expand_scales,
                                void* stream);

/* ------------------------------------------------------------------------
 * Quantised dispatch ([CV4] parameter notes: commQuantMode 2 = int8
 * quantisation during communication, with per-row dynamic scales; [PTO]
 * FrontReorder Stage: quantised token rows carrying their scale).
 *
 * As mdc_dispatch / mdc_dispatch_gather (same placement, triplets, inverse
 * index, counts, expand_scales and status, same workspace and layout stage),
 * but each received row is the int8 quantisation of its source token's row,
 * decided in fp32: amax = max|x|, codes clamp(rint(x * (127 / amax)), -127,
 * 127), and dynamic_scales[row] = amax / 127 (a zero row gives codes 0 and
 * scale 0).
 *   expand_q        [A][H] int8 (16-byte aligned)
 *   dynamic_scales  [A] fp32
 * H <= 8192 (a whole row is held in one wavefront's registers; larger H
 * returns MDC_ERR_UNSUPPORTED).
 * ------------------------------------------------------------------------ */
mdc_status mdc_dispatch_quant_gather(const mdc_shape* shape,
                                     const void* x,
                                     const float* expert_scales,
                                     int8_t* expand_q,
                                     float* dynamic_scales,
                                     int32_t* assist_info,
                                     int32_t* ep_recv_counts,
                                     int64_t* expert_token_nums,
                                     int32_t* expanded_row_idx,
                                     float* expand_scales,
                                     void* workspace, size_t workspace_bytes,
                                     void* stream);

mdc_status mdc_dispatch_quant(const mdc_shape* shape,
                              const void* x,
                              const int32_t* expert_ids,
                              const uint8_t* x_active_mask,
                              const float* expert_scales,
                              int8_t* expand_q,
                              float* dynamic_scales,
                              int32_t* assist_info,
                              int32_t* ep_recv_counts,
                              int64_t* expert_token_nums,
                              int32_t* expanded_row_idx,
                              float* expand_scales,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

/* ------------------------------------------------------------------------
 * Combine ([CV4] Function formula without TP; [TL] moe_combine_kernel;
 * [PTO] Combine / Unpermute stages)
 *
 * For source rank r = shape->rank and every token t:
 *     xOut[t] = bf16_rne( sum over k = 0..K-1 ascending, route present, of
 *                         ( w[t][k]*y[t][k] + w[t][k]*sharedX[t] ) )
 * with an fp32 accumulator starting at +0.0 and every product and sum
 * rounded to fp32 separately (no fused multiply-add), then rounded to bf16
 * nearest-even ([TL] combine: fp32 accumulate, CAST_RINT).  The shared term
 * is weighted per present route, as the [CV4] formula reads; it is omitted
 * when shared_expert_x is NULL.  For an active route (its token's flag, or
 * its own flag with mask_per_route) with e = expert_ids[t][k]:
 *   - 0 <= e < E: y[t][k] is row expanded_row_idx[t][k] of destination
 *     j = e / L, i.e. expand_x[j]: data returns along the dispatch path
 *     ([CV4] Function note and API matching constraints).  The route is
 *     present iff that row is < min(ep_recv_counts[j][L*W-1], A) and
 *     assist_info[j] at that row holds (r, t, k).  Its weight w[t][k] is
 *     expand_scales[j][row] when the expand_scales table is given (the
 *     dispatch's expandScales, [CV4] expandScalesOptional), else
 *     expert_scales[t][k]; the two are equal when the table comes from the
 *     dispatch of these routes;
 *   - E <= e < E+Z (zero expert): present with y = 0 and w = expert_scales[t][k];
 *   - E+Z <= e < E+Z+C (copy expert): present with y = ori_x[t] and
 *     w = expert_scales[t][k];
 *   - otherwise the route contributes nothing.
 * A token with no present route gives a +0.0 row.
 *
 * Inputs
 *   expand_x          host array of W device pointers: rank j's expert
 *                     outputs, [A][H] bf16 (the expand_x layout of dispatch j).
 *   assist_info       host array of W device pointers: rank j's [A][3] int32.
 *   ep_recv_counts    host array of W device pointers: rank j's [L*W] int32.
 *   expanded_row_idx  [BS][K] int32, rank r's slice of the table the W
 *                     dispatches filled.
 *   expert_ids        [BS][K] int32 of rank r.
 *   expert_scales     [BS][K] fp32 of rank r.
 *   x_active_mask     [BS] uint8 of rank r ([BS][K] with mask_per_route), or
 *                     NULL (all active).
 *   expand_scales     host array of W device pointers to rank j's [A] fp32
 *                     expand_scales, or NULL.
 *   shared_expert_x   [BS][H] bf16, or NULL.
 *   ori_x             [BS][H] bf16, rank r's unprocessed tokens ([CV4]
 *                     oriXOptional); required when copy_experts > 0, else
 *                     may be NULL.
 *   performance_info  [W] int64 or NULL ([CV4] Function: communication
 *                     latency collection; parameter table: performanceInfoOptional,
 *                     per-rank wait for data in microseconds, accumulated by
 *                     every call, cleared by the caller).  With virtual ranks
 *                     the wait for rank j's data is the time from the start
 *                     of the call to the arrival of the last row this call
 *                     reads from rank j (the device's constant-rate real-time
 *                     clock), rounded up to whole microseconds and added to
 *                     performance_info[j]; ranks the call reads nothing from
 *                     get 0.  It needs the workspace; without it the
 *                     workspace may be NULL.
 * Output
 *   x_out             [BS][H] bf16.
 * W must be <= MDC_MAX_COMBINE_WORLD.  mdc_combine_workspace returns the
 * workspace size (mdc_combine_workspace_size is its earlier name).
 * ------------------------------------------------------------------------ */
mdc_status mdc_combine_workspace(const mdc_shape* shape, size_t* bytes);
mdc_status mdc_combine_workspace_size(const mdc_shape* shape, size_t* bytes);

mdc_status mdc_combine(const mdc_shape* shape,
                       const void* const* expand_x,
                       const int32_t* const* assist_info,
                       const int32_t* const* ep_recv_counts,
                       const int32_t* expanded_row_idx,
                       const int32_t* expert_ids,
                       const float* expert_scales,
                       const uint8_t* x_active_mask,
                       const float* const* expand_scales,
                       const void* shared_expert_x,
                       const void* ori_x,
                       int64_t* performance_info,
                       void* x_out,
                       void* workspace, size_t workspace_bytes,
                       void* stream);

/* ------------------------------------------------------------------------
 * Grouped int8 expert FFN ([PTO] GMM1 / SwiGLU / GMM2 stages; Specification:
 * int8 weights with per-channel scales; Tiling Parameters: N is GMM1's output
 * width and GMM2 consumes N/2 after SwiGLU).
 *
 * For every row of expand_x (rows [0, min(sum(expert_token_nums), A)), grouped
 * by local expert in expert-major order as dispatch lays them out), with e the
 * row's local expert:
 *   q1, s1 = per-row int8 quantisation of x: amax = max|x|, codes
 *            clamp(rint(x * (127 / amax)), -127, 127), s1 = amax / 127,
 *            decided in fp32 (a zero row gives codes 0 and s1 = 0)
 *   h      = (q1 . w1[e]^T) * s1 * w1_scale[e][n]      int32 accumulate, n < N
 *   g      = silu(h[:, j]) * h[:, j + N/2], j < N/2, stored as bf16 (RNE)
 *   q2, s2 = per-row int8 quantisation of g, as for x
 *   y      = bf16_rne((q2 . w2[e]^T) * s2 * w2_scale[e][c]),  c < H
 * silu(a) = a / (1 + exp(-a)), evaluated in fp32 with the hardware exp and
 * reciprocal (about 1 ulp each); h and y are dequantised in fp32 and
 * rounded to bf16 nearest-even by the hardware conversion.  Which half goes
 * through silu, the quantiser and the intermediate precisions are this
 * library's readings; the pages name the stages and their order.  The
 * result is bitwise repeatable; against an exact (float64) evaluation of the
 * same formula it differs by the bf16 roundings of g and y and by the int8
 * quantisation of g that follows from them.
 *
 * Inputs (device): expand_x [A][H] bf16, expert_token_nums [L] int64 (from
 *   dispatch), w1 [L][N][H] int8, w1_scale [L][N] fp32, w2 [L][H][N/2] int8,
 *   w2_scale [L][H] fp32.   Output: y [A][H] bf16 (rows past the total are
 *   untouched).  inter_n = N must be a positive multiple of 256, H a
 *   multiple of 128 and N * H < 2^31 (one expert's weight matrix is addressed
 *   with 32-bit offsets); the GEMM tiles, (A / 256 + L + 2) * (N / 256 +
 *   ceil(H / 256)), are counted in 32 bits and must stay below 2^31 (else
 *   MDC_ERR_UNSUPPORTED).  The workspace (size from mdc_ffn_workspace;
 *   mdc_ffn_workspace_size is its earlier name) holds the status block, q1,
 *   s1, g, q2, s2, the m-tile table of the grouped GEMMs and the pipeline's
 *   ready counters.
 *
 * GMM1, the quantisation of g and GMM2 run as three stream-ordered kernels.
 * With MDC_FLAG_FFN_PIPELINE in shape->flags they run instead as one
 * persistent kernel whose GMM2 tiles start as soon as their rows of g are
 * quantised ([PTO] fused pipeline: ready flags between the stages).  Both
 * give bit-identical y.  The pipeline's waits are bounded: a GMM2 tile whose
 * wait runs out writes NaN rows and counts itself in the workspace status
 * block's wait_timeouts (never expected; every kernel still exits).
 * ------------------------------------------------------------------------ */
mdc_status mdc_ffn_workspace(const mdc_shape* shape, int32_t inter_n, size_t* bytes);
mdc_status mdc_ffn_workspace_size(const mdc_shape* shape, int32_t inter_n, size_t* bytes);

mdc_status mdc_ffn(const mdc_shape* shape,
                   int32_t inter_n,
                   const void* expand_x,
                   const int64_t* expert_token_nums,
                   const int8_t* w1,
                   const float* w1_scale,
                   const int8_t* w2,
                   const float* w2_scale,
                   void* y,
                   void* workspace, size_t workspace_bytes,
                   void* stream);

/* mdc_ffn on rows already quantised by mdc_dispatch_quant: expand_q [A][H]
 * int8 and dynamic_scales [A] fp32 take the place of q1 and s1 (the codes
 * equal what mdc_ffn computes from the bf16 rows, so y is the same). */
mdc_status mdc_ffn_quant_input(const mdc_shape* shape,
                               int32_t inter_n,
                               const int8_t* expand_q,
                               const float* dynamic_scales,
                               const int64_t* expert_token_nums,
                               const int8_t* w1,
                               const float* w1_scale,
                               const int8_t* w2,
                               const float* w2_scale,
                               void* y,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/* ------------------------------------------------------------------------
 * Quantised dispatch and grouped FFN as one pipeline ([PTO] Overall
 * Architecture: Dispatch -> GMM1 -> SwiGLU -> GMM2 per local-expert group,
 * joined by ready flags; Dispatch Stage: the destination pulls each expert
 * group's rows and sets the group's GMM1-ready flag; Optimization Notes:
 * expert-level overlap and segmented SwiGLU).
 *
 * Computes exactly what mdc_dispatch_quant_gather followed by
 * mdc_ffn_quant_input computes, with the same arguments (shape->rank is the
 * destination rank): every output of the quantised gather (expand_q,
 * dynamic_scales, assist_info, ep_recv_counts, expert_token_nums, the
 * inverse index, expand_scales, the dispatch status block) and y, bit for
 * bit.  Precondition as for mdc_dispatch_quant_gather: mdc_dispatch_layout
 * ran on dispatch_workspace earlier on the same stream.
 *
 * Three launches: one workgroup scans the layout's group counters once
 * (counts, epRecvCounts, status, the FFN's m-tile plan); one thread per
 * route places the routes sent here (inverse index, triplets, weights);
 * then one persistent kernel whose queue interleaves the dispatch of each
 * 256-row m-tile's rows (read from x through their triplets, quantised per
 * row, written to expand_q) with GMM1 tiles of earlier m-tiles, followed by
 * GMM2 tiles: GMM1 on an m-tile starts once its rows are written, GMM2 once
 * its rows of g are quantised.  Its waits are bounded as for
 * MDC_FLAG_FFN_PIPELINE (the spin field of shape->flags applies; a wait that
 * runs out is counted in the FFN workspace's status block and leaves NaN in
 * the tile's y rows).  The dispatch status block (dropped ids, overflow
 * rows) is in dispatch_workspace as for the gather.
 *
 * Requirements: those of mdc_dispatch_quant_gather (H <= 8192) and of
 * mdc_ffn (inter_n, H multiple of 128, tile counts); dispatch_workspace from
 * mdc_dispatch_workspace, ffn_workspace from mdc_ffn_workspace (the FFN
 * workspace is always required; the weights and y may be NULL only when
 * nothing can be received: BS == 0 or A == 0).
 * ------------------------------------------------------------------------ */
mdc_status mdc_dispatch_ffn(const mdc_shape* shape,
                            int32_t inter_n,
                            const void* x,
                            const float* expert_scales,
                            int8_t* expand_q,
                            float* dynamic_scales,
                            int32_t* assist_info,
                            int32_t* ep_recv_counts,
                            int64_t* expert_token_nums,
                            int32_t* expanded_row_idx,
                            float* expand_scales,
                            const int8_t* w1,
                            const float* w1_scale,
                            const int8_t* w2,
                            const float* w2_scale,
                            void* y,
                            void* dispatch_workspace, size_t dispatch_workspace_bytes,
                            void* ffn_workspace, size_t ffn_workspace_bytes,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MDC_H */
