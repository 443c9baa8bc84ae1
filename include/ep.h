/*
 * ep.h -- C ABI of libep.so: the expert-parallel dispatch/combine core for one
 * GPU's share of the work (one source rank, num_ranks emulated destination
 * ranks whose receive slabs share one HBM allocation), on AMD MI355X (gfx950).
 *
 * Four stages, each a call below:
 *   ep_get_layout  topk_idx -> token counts per rank / node / expert, is_token_in_rank
 *   ep_notify      counts   -> channel prefix matrices, receive prefix sums,
 *                              aligned per-expert receive counts, N_recv
 *   ep_layout_notify         -> both of the above in one launch
 *   ep_dispatch    x rows   -> receive region laid out [dst_rank][channel]
 *   ep_combine     expert outputs in receive layout -> weighted sum in token order
 * and beside them:
 *   ep_dispatch_fp8     dispatch of 1-byte (fp8) rows with their per-token scales
 *   ep_quantize_fp8     bf16 rows -> E4M3 rows and scales for it; ep_dequantize_fp8 back
 *   ep_dispatch_to_fp8  bf16 rows in, fp8 rows and scales out: the two above in one launch
 *   ep_dispatch_cached_to_fp8  the same for cached mode
 *   ep_dispatch_cached  new rows to the rows an earlier dispatch assigned (cached mode)
 *   ep_group_by_expert  receive rows regrouped into per-expert segments for grouped GEMMs
 *   ep_dispatch_grouped dispatch straight into those segments, with no receive rows
 *   ep_workspace_bytes, ep_status_string
 * Every call is stream-ordered and allocates nothing, so a sequence of them can be
 * captured in a HIP graph (ep_notify without its host read-back).
 *
 * Sources (web pages, cited by page title and section/function):
 *   mscclpp src/ext/ep/ht_runtime.cc mirror -- the torch-free host runtime:
 *     getDispatchLayout, internodeNotifyDispatch, internodeDispatch,
 *     internodeCombine, intranodeDispatch, intranodeCombine.  It turned tensor
 *     arguments into raw device pointers plus sizes, outputs into caller-owned
 *     buffers and the torch stream into a plain stream, which this ABI keeps.
 *   "DeepEP+NVSHMEM/DeepEP/internode.cu" notes, section 1 notify_dispatch
 *     (sm0 stage 6: prefix sums and expert alignment; sm1-x: channel counts).
 *   "CUDA与DeepEP" article, sections 2.2 (rank -> node), 3.2 (prefix sums),
 *     4.1 (SrcInfo), 4.2 (combine routing).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked (host).  The caller allocates
 *     and frees every buffer; the library never allocates device memory and
 *     keeps no state between calls.  Calls on different streams with disjoint
 *     buffers may run concurrently.
 *   - Each call only enqueues kernels on `stream` and returns, except
 *     ep_notify when num_recv_tokens_host is non-NULL (it then waits for the
 *     stream).  Outputs are valid in stream order after the call's kernels.
 *   - Shape or pointer errors are reported synchronously, before any launch:
 *     EP_ERR_INVALID_ARG for malformed arguments, EP_ERR_UNSUPPORTED for shapes
 *     beyond this version's limits.  EP_ERR_HIP reports a failed launch.
 *   - Data-dependent problems never trap: the kernels skip the offending item
 *     and OR a bit (EP_DEV_*) into *dev_status when dev_status is non-NULL.
 *     The caller zeroes *dev_status when it wants a fresh reading.
 *   - Row buffers (x, recv_x, y, combined_x, grouped_x) must be 16-byte aligned;
 *     rows move in 16-byte units (bf16 rows of `hidden` elements, or 1-byte
 *     elements where a call says so).
 */
#ifndef EP_H
#define EP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    EP_OK = 0,
    EP_ERR_INVALID_ARG = 1,
    EP_ERR_UNSUPPORTED = 2,
    EP_ERR_HIP = 3
} ep_status_t;

/* Bits OR-ed into *dev_status by the kernels. */
enum {
    EP_DEV_BAD_TOPK_IDX = 1,   /* a topk id outside [-1, num_experts): that slot is treated as masked */
    EP_DEV_RECV_OVERFLOW = 2,  /* a receive row >= recv_capacity: the row is not written, send_slot = -1 */
    EP_DEV_COUNT_MISMATCH = 4, /* counts or prefixes disagree with is_token_in_rank: num_tokens_per_rank /
                                  _per_rdma_rank (notify), gbl_channel_prefix_matrix or
                                  recv_gbl_rank_prefix_sum (dispatch) */
    EP_DEV_BAD_SEND_SLOT = 8,  /* a send_slot entry outside its valid range (combine, cached dispatch):
                                  skipped */
    EP_DEV_STALE_WORKSPACE = 16 /* the workspace does not hold what the call needs: its control words were not
                                  zero on entry (a workspace never zero-filled, or shared by calls that ran at
                                  the same time), or the routing state ep_notify left there does not belong to
                                  this is_token_in_rank.  The call's outputs are then not to be trusted. */
};

/* Which form of the row copy a dispatch takes.  [mscclpp ht_runtime.cc: the dispatch calls take a
 * Config, from which the runtime picks the kernel's form (computeIntranodeChannels chooses between
 * the sender/receiver split and all-sender blocks); here the choice rests on where x is.]
 *   push: token order -- each token's x row is read once, up front, and stored to all its
 *         destinations.  Best when x is only in HBM (it reads x as one stream).
 *   pull: receive order -- each XCD writes one advancing window of the receive region and
 *         re-reads x from its L2.  Best when x was just written (still in the Infinity Cache,
 *         as the layer before dispatch leaves it); slower than push when x is only in HBM.
 *         It applies from 2048 tokens, to rows of 1 KiB to 1 MiB, and not to cached mode;
 *         elsewhere the push form is taken.
 * The outputs are the same, bit for bit, whichever form runs. */
typedef enum {
    EP_FORM_AUTO = 0, /* the library's choice: currently the pull form wherever it applies */
    EP_FORM_PUSH = 1,
    EP_FORM_PULL = 2
} ep_dispatch_form_t;

/* Problem shape (host struct, read during the call only). */
typedef struct {
    int32_t num_tokens;       /* t >= 0 tokens on this rank                                      */
    int32_t hidden;           /* h >= 8, h % 8 == 0 (a bf16 row is a whole number of 16-byte units)*/
    int32_t num_topk;         /* 1 <= k <= 32                                                    */
    int32_t num_experts;      /* E >= 1, E % num_ranks == 0; expert e lives on rank e / (E / R)  */
    int32_t num_ranks;        /* 1 <= R <= 64, and R < 8 or R % 8 == 0 (8 ranks per node)        */
    int32_t num_channels;     /* 1 <= C <= 4096; channel c = tokens [c*ceil(t/C), (c+1)*ceil(t/C)) */
    int32_t my_rank;          /* 0 <= my_rank < R; stored as src_rank in recv_src_info           */
    int32_t expert_alignment; /* >= 1; per-expert receive counts are rounded up to a multiple    */
} ep_shape_t;

/*
 * Stage 1, dispatch layout.  [mscclpp ht_runtime.cc, getDispatchLayout]
 * In:  topk_idx [t][k] int64, -1 = masked slot.
 * Out: num_tokens_per_rank      [R]     int32: tokens with at least one expert on rank r
 *      num_tokens_per_rdma_rank [nodes] int32: tokens with at least one expert on a rank of
 *                                              node n (node = rank / 8, nodes = max(1, R / 8))
 *      num_tokens_per_expert    [E]     int32: valid topk slots naming expert e
 *      is_token_in_rank         [t][R]  uint8 (0/1, row-major)
 * workspace: see ep_workspace_bytes (its control words must be zero before the first
 *            call; every call leaves them zero).
 * dev_status (nullable): EP_DEV_BAD_TOPK_IDX.
 */
ep_status_t ep_get_layout(const ep_shape_t *s, const int64_t *topk_idx, int32_t *num_tokens_per_rank,
                          int32_t *num_tokens_per_rdma_rank, int32_t *num_tokens_per_expert,
                          uint8_t *is_token_in_rank, void *workspace, size_t workspace_bytes, int32_t *dev_status,
                          hipStream_t stream);

/*
 * Stage 1 without a workspace, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation).  Same inputs,
 * outputs and dev_status as ep_get_layout; the tickets and running counts live in a static
 * array of the library (66,080 bytes on each GPU, held until the process ends), which the
 * call clears with a small kernel before the layout kernel.  Allocates nothing.
 * Limits: num_experts <= 16384 (EP_ERR_UNSUPPORTED beyond).  The stream must belong to the
 * current device (EP_ERR_INVALID_ARG otherwise).  Every call on one GPU uses that GPU's
 * single array: calls that overlap in time on one GPU (on different streams) race.
 */
ep_status_t ep_get_layout_noalloc(const ep_shape_t *s, const int64_t *topk_idx, int32_t *num_tokens_per_rank,
                                  int32_t *num_tokens_per_rdma_rank, int32_t *num_tokens_per_expert,
                                  uint8_t *is_token_in_rank, int32_t *dev_status, hipStream_t stream);

/*
 * Stage 2, notify.  [mscclpp ht_runtime.cc, internodeNotifyDispatch; internode.cu notes,
 * notify_dispatch sm1-x stages 1-3 and sm0 stage 6]
 * In:  is_token_in_rank [t][R] uint8 (any non-zero byte counts as 1) and the three count
 *      arrays of stage 1.
 * Out: gbl_channel_prefix_matrix  [R][C]     int32: inclusive prefix over channels of the
 *                                                   tokens of each channel sent to rank r
 *      rdma_channel_prefix_matrix [nodes][C] int32: the same per node
 *      recv_gbl_rank_prefix_sum   [R]        int32: inclusive prefix of num_tokens_per_rank;
 *                                                   slab r of the receive region is rows
 *                                                   [prefix[r-1], prefix[r])
 *      recv_rdma_rank_prefix_sum  [nodes]    int32: inclusive prefix of num_tokens_per_rdma_rank
 *      num_recv_tokens_per_expert [E]        int32: ceil(n_e / expert_alignment) * expert_alignment
 *      num_recv_tokens            [1]        int32: N = total receive rows (device)
 *      num_recv_tokens_host  (host, nullable): when non-NULL the call waits for the stream
 *                                              and stores N there.
 *      workspace: the same workspace as ep_get_layout; notify writes the per-token rank
 *                 masks and per-64-token-chunk row offsets that ep_dispatch reads.
 * dev_status (nullable): EP_DEV_COUNT_MISMATCH.
 */
ep_status_t ep_notify(const ep_shape_t *s, const uint8_t *is_token_in_rank, const int32_t *num_tokens_per_rank,
                      const int32_t *num_tokens_per_rdma_rank, const int32_t *num_tokens_per_expert,
                      int32_t *gbl_channel_prefix_matrix, int32_t *rdma_channel_prefix_matrix,
                      int32_t *recv_gbl_rank_prefix_sum, int32_t *recv_rdma_rank_prefix_sum,
                      int32_t *num_recv_tokens_per_expert, int32_t *num_recv_tokens, int32_t *num_recv_tokens_host,
                      void *workspace, size_t workspace_bytes, int32_t *dev_status, hipStream_t stream);

/*
 * Stages 1+2 in one launch: ep_get_layout then ep_notify, from topk_idx to every output of
 * both, with the same values bit for bit.  [the sources of both stages]  The token masks are
 * built once and each 64-token chunk is counted from them on chip, so is_token_in_rank is
 * written (it is an output) but not read back, and one completion election replaces two.
 * Out: the four outputs of ep_get_layout and the seven of ep_notify (num_recv_tokens_host as
 *      there: non-NULL makes the call wait for the stream).
 * workspace: as for ep_notify (it is left as ep_notify leaves it, for ep_dispatch).
 * dev_status (nullable): EP_DEV_BAD_TOPK_IDX, EP_DEV_STALE_WORKSPACE.
 */
ep_status_t ep_layout_notify(const ep_shape_t *s, const int64_t *topk_idx, int32_t *num_tokens_per_rank,
                             int32_t *num_tokens_per_rdma_rank, int32_t *num_tokens_per_expert,
                             uint8_t *is_token_in_rank, int32_t *gbl_channel_prefix_matrix,
                             int32_t *rdma_channel_prefix_matrix, int32_t *recv_gbl_rank_prefix_sum,
                             int32_t *recv_rdma_rank_prefix_sum, int32_t *num_recv_tokens_per_expert,
                             int32_t *num_recv_tokens, int32_t *num_recv_tokens_host, void *workspace,
                             size_t workspace_bytes, int32_t *dev_status, hipStream_t stream);

/*
 * Stages 3+4, dispatch.  [mscclpp ht_runtime.cc, internodeDispatch / intranodeDispatch (inputs
 * isTokenInRank, gblChannelPrefixMatrix, recvGblRankPrefixSum); CUDA与DeepEP article 4.1 SrcInfo]
 * The receive region is laid out [dst_rank][channel]: slab r holds the tokens sent to r,
 * channel segments in channel order, tokens ascending inside a segment.  Channel c of rank r
 * starts at row  prefix[r-1] + gbl_channel_prefix_matrix[r][c-1]  (0 for r = 0, c = 0), so
 * token t's row on rank r is that start plus #{t' in channel c, t' < t, sent to r}.
 * In:  x [t][h] bf16; topk_idx [t][k] int64; topk_weights [t][k] f32;
 *      is_token_in_rank [t][R] uint8 (any non-zero byte counts as 1),
 *      gbl_channel_prefix_matrix [R][C] and recv_gbl_rank_prefix_sum [R] as ep_notify
 *      computes them from that is_token_in_rank.
 *      workspace (nullable):
 *        NULL   -- the row of every (token, rank) is worked out inside the call from the
 *                  three routing inputs: a chunk of 64 tokens is placed from its channel's
 *                  prefix plus a count over at most half a channel.  Needs ceil(t / C) <= 4096
 *                  (EP_ERR_UNSUPPORTED otherwise: pass the workspace).
 *        non-NULL -- the workspace ep_notify filled for this is_token_in_rank: the per-token
 *                  rank masks and per-chunk row offsets it left there are used instead of
 *                  being worked out again.  The call checks them against is_token_in_rank
 *                  and the prefix matrix and sets EP_DEV_STALE_WORKSPACE when they differ.
 * Out (recv_capacity rows allocated by the caller):
 *      recv_x            [cap][h] bf16: bitwise copy of x[t]
 *      recv_topk_weights [cap][k] f32:  w[t][j] where slot j's expert lives on the
 *                                       receiving rank, else 0
 *      recv_topk_idx     [cap][k] int64 (nullable): the receiver's local expert id
 *                                       e - r*(E/R) for those slots, else -1
 *      recv_src_info     [cap][2] int32: {my_rank, t} (8-byte aligned)
 *      send_slot         [t][R]   int32: the row of (t, r), -1 where t is not sent to r
 * Rows >= recv_capacity (or below 0) are skipped and flagged (EP_DEV_RECV_OVERFLOW); their
 * send_slot is -1.
 * form: an ep_dispatch_form_t (EP_FORM_AUTO when the caller does not know where x is).
 * dev_status (nullable): EP_DEV_RECV_OVERFLOW; EP_DEV_COUNT_MISMATCH when the prefix matrix or
 * the receive prefix sums disagree with is_token_in_rank (rows are then placed by the prefix
 * matrix, unchecked); EP_DEV_STALE_WORKSPACE as above.
 */
ep_status_t ep_dispatch(const ep_shape_t *s, const void *x, const int64_t *topk_idx, const float *topk_weights,
                        const uint8_t *is_token_in_rank, const int32_t *gbl_channel_prefix_matrix,
                        const int32_t *recv_gbl_rank_prefix_sum, const void *workspace, size_t workspace_bytes,
                        int32_t recv_capacity, void *recv_x, float *recv_topk_weights, int64_t *recv_topk_idx,
                        int32_t *recv_src_info, int32_t *send_slot, int32_t form, int32_t *dev_status,
                        hipStream_t stream);

/*
 * Dispatch of fp8 rows.  [mscclpp ht_runtime.cc, internodeDispatch / intranodeDispatch:
 * x_scales with num_scales per token are dispatched beside the rows and returned as
 * recv_x_scales (the FP8 scale buffer); the combine side stays bf16]
 * Same as ep_dispatch, with rows of `hidden` one-byte elements (hidden % 16 == 0) moved
 * bit for bit, plus the token's num_scales float scales (0 <= num_scales <= 1024):
 *   x [t][h] fp8 (any 1-byte format), x_scales [t][num_scales] f32 (nullable if num_scales == 0)
 *   recv_x [cap][h], recv_x_scales [cap][num_scales] (nullable if num_scales == 0)
 * Every other argument and output is as in ep_dispatch.
 */
ep_status_t ep_dispatch_fp8(const ep_shape_t *s, const void *x, const float *x_scales, int32_t num_scales,
                            const int64_t *topk_idx, const float *topk_weights, const uint8_t *is_token_in_rank,
                            const int32_t *gbl_channel_prefix_matrix, const int32_t *recv_gbl_rank_prefix_sum,
                            const void *workspace, size_t workspace_bytes, int32_t recv_capacity, void *recv_x,
                            float *recv_x_scales, float *recv_topk_weights, int64_t *recv_topk_idx,
                            int32_t *recv_src_info, int32_t *send_slot, int32_t form, int32_t *dev_status,
                            hipStream_t stream);

/*
 * fp8 rows and scales for ep_dispatch_fp8, made from bf16 rows.  [mscclpp ht_runtime.cc,
 * intranodeDispatch / internodeDispatch take x with a one-byte element size together with
 * xScales, numScales floats per token; how they are produced is not on the pages -- this is
 * the library's quantiser for that input.]
 * A row of `hidden` channels is cut into num_scales groups of g = hidden / num_scales
 * consecutive channels.  For group q of row t:
 *   a = max(largest |x| of the group, 2^-64)
 *   x_scales[t][q] = a / 448                                  (f32, correctly rounded)
 *   x_fp8[t][i]    = e4m3(clamp(x[t][i] * (448 / a), -448, 448))
 * with 448 / a and the product each rounded to f32, and e4m3() the nearest OCP FP8 E4M3 value
 * (sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities; largest finite 448), ties to
 * the even pattern; the sign bit of x is kept, also for values that round to zero.  Then
 * x ~ value(x_fp8) * x_scales within half an E4M3 step: 2^-4 |x|, or 2^-10 of the scale for the
 * smallest values of a group.
 * In:  x [num_rows][hidden] bf16, finite (the codes and scale of a group holding an infinity or
 *      NaN are not defined).
 * Out: x_fp8 [num_rows][hidden] uint8; x_scales [num_rows][num_scales] f32 (4-byte aligned).
 * Limits: hidden a positive multiple of 16 (EP_ERR_INVALID_ARG otherwise, and when num_scales
 * does not divide hidden); g = 16, 32, 64, 128, 256, 512 or 1024 (EP_ERR_UNSUPPORTED otherwise).
 * x and x_fp8 16-byte aligned.  num_rows == 0 enqueues nothing.  One launch, no workspace.
 */
ep_status_t ep_quantize_fp8(const void *x, int64_t num_rows, int32_t hidden, int32_t num_scales, void *x_fp8,
                            float *x_scales, hipStream_t stream);

/*
 * Dispatch of bf16 rows that arrive as fp8 rows with scales: ep_quantize_fp8 of x followed by
 * ep_dispatch_fp8 of its codes and scales, in one launch and bit for bit the same outputs.
 * [mscclpp ht_runtime.cc, intranodeDispatch / internodeDispatch with xElementSize 1 and xScales:
 * the receive side gets fp8 rows and the FP8 scale buffer; the quantiser as for ep_quantize_fp8]
 * Each token's row is read once (2h bytes), quantised once per group of hidden / num_scales
 * channels, and its h-byte codes and num_scales scales are stored to every destination rank, so
 * neither the fp8 copy of x nor its scales pass through HBM on this rank.
 * In:  x [t][h] bf16 (finite); num_scales as for ep_quantize_fp8 (groups of 16 to 1024 channels);
 *      topk_idx, topk_weights, is_token_in_rank, gbl_channel_prefix_matrix,
 *      recv_gbl_rank_prefix_sum and workspace (nullable) as for ep_dispatch.
 * Out: recv_x [cap][h] uint8 E4M3 codes; recv_x_scales [cap][num_scales] f32; recv_topk_weights,
 *      recv_topk_idx (nullable), recv_src_info and send_slot as for ep_dispatch.
 * The row copy takes the push form (token order; the pull form has no quantising variant).
 * Limits: hidden % 16 == 0 and num_scales dividing it (EP_ERR_INVALID_ARG), groups of
 * 16 << l channels, 0 <= l <= 6 (EP_ERR_UNSUPPORTED); the rest as for ep_dispatch_fp8.
 * dev_status (nullable): as for ep_dispatch.
 */
ep_status_t ep_dispatch_to_fp8(const ep_shape_t *s, const void *x, int32_t num_scales, const int64_t *topk_idx,
                              const float *topk_weights, const uint8_t *is_token_in_rank,
                              const int32_t *gbl_channel_prefix_matrix, const int32_t *recv_gbl_rank_prefix_sum,
                              const void *workspace, size_t workspace_bytes, int32_t recv_capacity, void *recv_x,
                              float *recv_x_scales, float *recv_topk_weights, int64_t *recv_topk_idx,
                              int32_t *recv_src_info, int32_t *send_slot, int32_t *dev_status, hipStream_t stream);

/*
 * The inverse of ep_quantize_fp8, for rows an fp8 dispatch delivered (recv_x, recv_x_scales).
 * [the same reading of the pages' fp8 rows and FP8 scale buffer]
 *   out[t][i] = bf16(value(x_fp8[t][i]) * x_scales[t][i / g])
 * with the product rounded to f32 and then to bf16 (nearest, ties to even).  The patterns 0x7F and
 * 0xFF (E4M3 NaN, which the quantiser never writes) give a bf16 NaN.
 * In:  x_fp8 [num_rows][hidden] uint8, x_scales [num_rows][num_scales] f32.
 * Out: out [num_rows][hidden] bf16.  Limits and alignment as for ep_quantize_fp8 (out in place of x).
 */
ep_status_t ep_dequantize_fp8(const void *x_fp8, const float *x_scales, int64_t num_rows, int32_t hidden,
                              int32_t num_scales, void *out, hipStream_t stream);

/*
 * Cached-mode dispatch.  [mscclpp ht_runtime.cc, internodeDispatch / intranodeDispatch with
 * cachedMode: the layout of an earlier call is reused -- no counting, no notification]
 * Copies row t to recv_x[send_slot[t][r]] for every r with send_slot[t][r] >= 0, where
 * send_slot [t][R] was written by an earlier ep_dispatch / ep_dispatch_fp8 / ep_dispatch_to_fp8
 * for the same routing.  Rows are hidden * elem_bytes bytes (elem_bytes 2 = bf16, 1 = fp8; a multiple
 * of 16); num_scales float scales per token go along when num_scales > 0.  No metadata
 * is written.  Entries outside [-1, recv_capacity) are skipped and flagged
 * (EP_DEV_BAD_SEND_SLOT).  Needs no workspace and no layout/notify call.  form: EP_FORM_AUTO
 * or EP_FORM_PUSH, both the push form; EP_FORM_PULL returns EP_ERR_UNSUPPORTED (cached mode has
 * no pull form).
 */
ep_status_t ep_dispatch_cached(const ep_shape_t *s, const void *x, int32_t elem_bytes, const float *x_scales,
                               int32_t num_scales, const int32_t *send_slot, int32_t recv_capacity, void *recv_x,
                               float *recv_x_scales, int32_t form, int32_t *dev_status, hipStream_t stream);

/*
 * Cached-mode dispatch of bf16 rows that arrive as fp8 rows with scales: ep_quantize_fp8 of x
 * followed by ep_dispatch_cached of its codes and scales (elem_bytes 1), in one launch and bit for
 * bit the same outputs.  [mscclpp ht_runtime.cc, cached mode of intranodeDispatch /
 * internodeDispatch with xScales; the quantiser as for ep_quantize_fp8]
 * Each token's row is read once and quantised once; its codes and scales go to every row
 * send_slot[t][r] >= 0 names (send_slot as an earlier dispatch of the same routing wrote it).
 * In:  x [t][h] bf16 (finite); num_scales as for ep_quantize_fp8; send_slot [t][R].
 * Out: recv_x [cap][h] uint8 E4M3 codes; recv_x_scales [cap][num_scales] f32.  No metadata.
 * Entries outside [-1, recv_capacity) are skipped and flagged (EP_DEV_BAD_SEND_SLOT).  Push form.
 * Limits as for ep_dispatch_to_fp8.
 */
ep_status_t ep_dispatch_cached_to_fp8(const ep_shape_t *s, const void *x, int32_t num_scales, const int32_t *send_slot,
                                     int32_t recv_capacity, void *recv_x, float *recv_x_scales, int32_t *dev_status,
                                     hipStream_t stream);

/*
 * Grouping of the received rows by local expert, the layout grouped expert GEMMs read.
 * [DeepEP internode.cu notes, notify_dispatch sm0 stage 6, and mscclpp ht_runtime.cc,
 * internodeNotifyDispatch: per local expert, the received slot count rounded up to
 * expert_alignment -- the sizes below.  The order inside the segments is this library's
 * reading; the pages do not show one.]
 * Segment e = r*(E/R) + le (slab r of the receive region, local expert le) starts at
 * sum_{e' < e} num_recv_tokens_per_expert[e'] and holds one entry per (row, slot) of slab r
 * with recv_topk_idx[row][slot] == le, rows ascending, then slots; the rest of the segment,
 * up to num_recv_tokens_per_expert[e], is padding.  For the entry at grouped position g:
 *   grouped_x        [cap][h] (elem_bytes 2 = bf16, 1 = fp8; h*elem_bytes % 16 == 0):
 *                    recv_x[row] bit for bit; padding rows are zero
 *   grouped_x_scales [cap][num_scales] f32: the row's scales, padding 0 (nullable if
 *                    num_scales == 0; 0 <= num_scales <= 1024)
 *   grouped_row      [cap] int32: row; padding -1
 *   grouped_weights  [cap] f32 (nullable): recv_topk_weights[row][slot]; padding 0
 *   slot_pos         [num_recv_rows][k] int32 (nullable): g of each placed (row, slot), else -1
 *   num_grouped_rows [1] int32 (device): sum of the segment sizes
 * Positions at or past min(num_grouped_rows, grouped_capacity) are not written.
 * In:  recv_x [num_recv_rows][h], recv_x_scales [num_recv_rows][num_scales],
 *      recv_topk_idx [num_recv_rows][k] and recv_topk_weights (nullable unless
 *      grouped_weights is given and num_recv_rows > 0) as ep_dispatch / ep_dispatch_fp8 wrote them;
 *      recv_gbl_rank_prefix_sum [R] and num_recv_tokens_per_expert [E] as ep_notify wrote
 *      them (slab ends non-decreasing; a negative size counts as 0).
 * Rows at or past the end of the last slab (capacity slack, e.g. num_recv_rows = the
 * allocated capacity when N is not known on the host) are not read; their slot_pos is -1.
 * dev_status (nullable): EP_DEV_RECV_OVERFLOW (an entry past its segment's size or the
 * grouped capacity: skipped, slot_pos -1), EP_DEV_BAD_TOPK_IDX (a local id outside
 * [-1, E/R) in a slab row: skipped).  E/R > 512 or num_recv_rows * k >= 2^31:
 * EP_ERR_UNSUPPORTED.
 * Two launches (positions, then the row copy); no workspace.
 */
ep_status_t ep_group_by_expert(const ep_shape_t *s, const void *recv_x, int32_t elem_bytes,
                               const float *recv_x_scales, int32_t num_scales, const int64_t *recv_topk_idx,
                               const float *recv_topk_weights, const int32_t *recv_gbl_rank_prefix_sum,
                               const int32_t *num_recv_tokens_per_expert, int32_t num_recv_rows,
                               int32_t grouped_capacity, void *grouped_x, float *grouped_x_scales,
                               int32_t *grouped_row, float *grouped_weights, int32_t *slot_pos,
                               int32_t *num_grouped_rows, int32_t *dev_status, hipStream_t stream);

/*
 * Dispatch straight into the grouped layout: the outputs of ep_dispatch (or ep_dispatch_fp8)
 * followed by ep_group_by_expert with num_recv_rows = recv_capacity, without the receive rows.
 * [the pages' dispatch as for ep_dispatch; the grouping as for ep_group_by_expert]
 * Writes recv_topk_weights, recv_topk_idx, recv_src_info and send_slot exactly as ep_dispatch
 * does, and every output of ep_group_by_expert for those rows (recv_topk_idx and slot_pos are
 * required here: the grouping reads the ids, and each token's row is read once from x and
 * stored at the grouped positions slot_pos gives its slots):
 *   grouped_x [grouped_capacity][h] = x[t] of the entry's row (bf16 when elem_bytes == 2,
 *             1-byte elements when elem_bytes == 1); grouped_x_scales = that token's
 *             x_scales (num_scales per token, nullable when 0); padding rows are zero.
 * No recv_x is written or read.  In: x, x_scales, topk_idx, topk_weights, is_token_in_rank,
 * gbl_channel_prefix_matrix and recv_gbl_rank_prefix_sum as for ep_dispatch / ep_dispatch_fp8;
 * num_recv_tokens_per_expert as ep_notify wrote it; the workspace as ep_notify left it (required
 * when t > 0, checked as in ep_dispatch).  Receive rows at or past recv_capacity are dropped as in
 * ep_dispatch (EP_DEV_RECV_OVERFLOW) and not grouped.  The workspace is only read.
 * dev_status (nullable): the flags of both calls.  Limits as for both calls.
 * From 2048 tokens (rows of 1 KiB to 1 MiB, E <= 2048) one launch: a slab's rows follow
 * their tokens, so an entry's place in its segment is the number of entries of its expert
 * in earlier (token, slot) pairs, found in token order with no pass over the receive rows.
 * Otherwise four launches (receive metadata, positions over the receive rows, rows, padding).
 */
ep_status_t ep_dispatch_grouped(const ep_shape_t *s, const void *x, int32_t elem_bytes, const float *x_scales,
                                int32_t num_scales, const int64_t *topk_idx, const float *topk_weights,
                                const uint8_t *is_token_in_rank, const int32_t *gbl_channel_prefix_matrix,
                                const int32_t *recv_gbl_rank_prefix_sum, const int32_t *num_recv_tokens_per_expert,
                                const void *workspace, size_t workspace_bytes, int32_t recv_capacity,
                                float *recv_topk_weights, int64_t *recv_topk_idx, int32_t *recv_src_info,
                                int32_t *send_slot, int32_t grouped_capacity, void *grouped_x,
                                float *grouped_x_scales, int32_t *grouped_row, float *grouped_weights,
                                int32_t *slot_pos, int32_t *num_grouped_rows, int32_t *dev_status,
                                hipStream_t stream);

/*
 * Stage 5, combine.  [mscclpp ht_runtime.cc, internodeCombine / intranodeCombine (bf16 out,
 * combined topk weights); CUDA与DeepEP article 4.2 (rows return to their source token)]
 * For each token t, over ranks r ascending with s = send_slot[t][r] >= 0:
 *     W = sum_j recv_topk_weights[s][j]       (fp32 adds, j ascending, from +0)
 *     acc[i] = fmaf(W, y[s][i], acc[i])       (fp32, from +0)
 *   combined_x[t][i] = acc[i] rounded to bf16 (nearest, ties to even)
 *   combined_topk_weights[t][j] = sum over the same r of recv_topk_weights[s][j] (fp32, r ascending)
 * In:  y [num_recv_rows][h] bf16 (expert outputs in receive layout; y = recv_x for identity
 *      experts); recv_topk_weights [num_recv_rows][k]; send_slot [t][R].
 * Out: combined_x [t][h] bf16; combined_topk_weights [t][k] f32 (nullable).
 * dev_status (nullable): EP_DEV_BAD_SEND_SLOT.
 */
ep_status_t ep_combine(const ep_shape_t *s, const void *y, const float *recv_topk_weights, const int32_t *send_slot,
                       int32_t num_recv_rows, void *combined_x, float *combined_topk_weights, int32_t *dev_status,
                       hipStream_t stream);

/* Bytes of workspace ep_get_layout / ep_notify / ep_dispatch / ep_dispatch_grouped need for
 * this shape (0 if s is invalid).  It holds the completion counters and running counts of
 * layout and notify, and the per-token rank masks and per-chunk row offsets notify leaves for
 * dispatch.  The workspace is device memory, 256-byte aligned, owned by the caller, and
 * must be zero-filled before its first use (hipMemset once at allocation): its completion
 * counters and running counts must start at zero, and every call leaves them at zero
 * again.  Calls that run concurrently must not share a workspace. */
size_t ep_workspace_bytes(const ep_shape_t *s);

/* Static text for a status code. */
const char *ep_status_string(ep_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* EP_H */
