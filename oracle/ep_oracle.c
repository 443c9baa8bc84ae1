/*
 * ep_oracle.c -- plain, slow, single-threaded CPU oracle for the expert-parallel
 * dispatch/combine core (layout, notify, dispatch, combine, the grouping of
 * received rows by local expert, and the E4M3 quantiser that makes the fp8
 * rows and scales the fp8 dispatch carries) on one GPU's share.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  The product path (the HIP library
 * and its Python binding) never links, imports or calls it, and it shares no
 * code, header, table or helper with the HIP sources.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -std=c11 ep_oracle.c -lm
 * (-ffp-contract=off keeps every a*b+c as two roundings unless fmaf() is written.)
 *
 * Sources (web pages; cited by page title and section):
 *   [notes]   "DeepEP+NVSHMEM/DeepEP/internode.cu" notes, section
 *             "1. notify_dispatch(internode.cu)": sm0 stage 6 (reductions and
 *             inclusive prefix sums), sm1-x stages 1-3 (per-channel counting).
 *   [qa]      "【cuda】deepep" Q&A on channels inside SymBuffer.
 *   [mscclpp] mscclpp src/ext/ep/ht_runtime.cc mirror: getDispatchLayout,
 *             internodeNotifyDispatch, internodeDispatch, internodeCombine,
 *             intranodeDispatch, intranodeCombine.
 *   [article] "CUDA与DeepEP：分布式MoE系统中的高效通信机制解析": section 2.2
 *             (rank -> node mapping), 3.2 (expert sums, prefix sums),
 *             4.1 (SrcInfo), 4.2 (combine routing loop).
 *
 * Every function below computes the plain definition with nested loops, in the
 * order the definition states.  Where the pages leave a step open, the reading
 * taken is written next to the code.
 *
 * Status bits returned by every function (0 = clean):
 *   ORC_BAD_TOPK_IDX   1  a topk id outside [-1, E); the slot is treated as masked
 *   ORC_RECV_OVERFLOW  2  a receive row index >= the receive capacity (or a grouped
 *                         entry past its segment or the grouped capacity); skipped
 *   ORC_COUNT_MISMATCH 4  per-rank/per-node counts disagree with is_token_in_rank
 *   ORC_BAD_SEND_SLOT  8  a send_slot outside [-1, rows) in combine or cached dispatch; skipped
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORC_BAD_TOPK_IDX 1
#define ORC_RECV_OVERFLOW 2
#define ORC_COUNT_MISMATCH 4
#define ORC_BAD_SEND_SLOT 8

/* Ranks per node is fixed at 8 ([mscclpp] NUM_MAX_NVL_PEERS; [article] §2.2:
 * node = rank / 8, GPU-in-node = rank % 8).  With fewer than 8 ranks there is
 * one node ([mscclpp] constructor: num_rdma_ranks = max(1, ranks / 8)). */
static int32_t orc_num_nodes(int32_t num_ranks) {
    int32_t n = num_ranks / 8;
    return n > 0 ? n : 1;
}

/* Channel c owns the contiguous token range [c*Tc, min((c+1)*Tc, T)) with
 * Tc = ceil(T / C).  The pages give only "channel = block / 2" ([qa]); the plain
 * reading is balanced contiguous ranges, so a channel can be empty when T < C. */
static int64_t orc_channel_begin(int64_t T, int64_t C, int64_t c) {
    int64_t tc = (T + C - 1) / C;
    int64_t b = c * tc;
    return b < T ? b : T;
}
static int64_t orc_channel_end(int64_t T, int64_t C, int64_t c) {
    return orc_channel_begin(T, C, c + 1);
}

/* a topk id is valid when 0 <= e < E; -1 marks a masked slot. */
static int orc_topk_valid(int64_t e, int32_t E, int *status) {
    if (e == -1) return 0;
    if (e < -1 || e >= E) {
        *status |= ORC_BAD_TOPK_IDX;
        return 0;
    }
    return 1;
}

/* ------------------------------------------------------------------------- */
/* Stage 1: dispatch layout.  [mscclpp] getDispatchLayout takes topk_idx and
 * yields tokens per rank, per RDMA rank (node), per expert and the
 * is_token_in_rank map; the kernel body is not on the pages.  Reading:
 *   is_token_in_rank[t][r] = 1 iff some valid slot j has expert_of_rank == r,
 *     with rank_of(e) = e / (E / R)  (experts are split evenly, E % R == 0);
 *   num_tokens_per_rank[r] = #tokens with is_token_in_rank[t][r];
 *   num_tokens_per_rdma_rank[n] = #tokens with ANY rank of node n
 *     ([notes] sm1-x stage 1 tests the 8 bytes of a node at once, != 0);
 *   num_tokens_per_expert[e] = #valid slots equal to e (counted per slot). */
int oracle_layout(int32_t T, int32_t K, int32_t E, int32_t R, const int64_t *topk_idx,
                  int32_t *num_tokens_per_rank, int32_t *num_tokens_per_rdma_rank,
                  int32_t *num_tokens_per_expert, uint8_t *is_token_in_rank) {
    int status = 0;
    const int32_t nodes = orc_num_nodes(R);
    const int32_t experts_per_rank = E / R;
    for (int32_t r = 0; r < R; ++r) num_tokens_per_rank[r] = 0;
    for (int32_t n = 0; n < nodes; ++n) num_tokens_per_rdma_rank[n] = 0;
    for (int32_t e = 0; e < E; ++e) num_tokens_per_expert[e] = 0;

    for (int64_t t = 0; t < T; ++t) {
        uint8_t *row = is_token_in_rank + t * R;
        for (int32_t r = 0; r < R; ++r) row[r] = 0;
        for (int32_t j = 0; j < K; ++j) {
            int64_t e = topk_idx[t * K + j];
            if (!orc_topk_valid(e, E, &status)) continue;
            num_tokens_per_expert[e] += 1;
            row[e / experts_per_rank] = 1;
        }
        for (int32_t r = 0; r < R; ++r)
            if (row[r]) num_tokens_per_rank[r] += 1;
        for (int32_t n = 0; n < nodes; ++n) {
            int any = 0;
            for (int32_t r = n * 8; r < R && r < (n + 1) * 8; ++r) any |= row[r];
            if (any) num_tokens_per_rdma_rank[n] += 1;
        }
    }
    return status;
}

/* ------------------------------------------------------------------------- */
/* Stage 2: notify.  [notes] sm1-x: per channel, count the tokens sent to each
 * rank and to each node, and store per-channel prefix sums in
 * gbl_channel_prefix_matrix [R][C] and rdma_channel_prefix_matrix [nodes][C].
 * Reading: inclusive prefix over channels (last column = the total), matching
 * the inclusive receive prefix sums of sm0 stage 6.
 * [notes] sm0 stage 6 / [article] §3.2: inclusive prefix sums of received
 * counts, the last value being the total received; per-expert received counts
 * rounded up to expert_alignment.  With one source rank and R emulated
 * destinations the receive prefix runs over destination ranks (nodes). */
int oracle_notify(int32_t T, int32_t E, int32_t R, int32_t C, int32_t expert_alignment,
                  const uint8_t *is_token_in_rank, const int32_t *num_tokens_per_rank,
                  const int32_t *num_tokens_per_rdma_rank, const int32_t *num_tokens_per_expert,
                  int32_t *gbl_channel_prefix_matrix, int32_t *rdma_channel_prefix_matrix,
                  int32_t *recv_gbl_rank_prefix_sum, int32_t *recv_rdma_rank_prefix_sum,
                  int32_t *num_recv_tokens_per_expert, int32_t *num_recv_tokens) {
    int status = 0;
    const int32_t nodes = orc_num_nodes(R);

    for (int32_t r = 0; r < R; ++r) {
        int32_t running = 0;
        for (int32_t c = 0; c < C; ++c) {
            for (int64_t t = orc_channel_begin(T, C, c); t < orc_channel_end(T, C, c); ++t)
                running += is_token_in_rank[t * R + r] != 0;
            gbl_channel_prefix_matrix[(int64_t)r * C + c] = running;
        }
        if (running != num_tokens_per_rank[r]) status |= ORC_COUNT_MISMATCH;
    }
    for (int32_t n = 0; n < nodes; ++n) {
        int32_t running = 0;
        for (int32_t c = 0; c < C; ++c) {
            for (int64_t t = orc_channel_begin(T, C, c); t < orc_channel_end(T, C, c); ++t) {
                int any = 0;
                for (int32_t r = n * 8; r < R && r < (n + 1) * 8; ++r)
                    any |= is_token_in_rank[t * R + r] != 0;
                running += any;
            }
            rdma_channel_prefix_matrix[(int64_t)n * C + c] = running;
        }
        if (running != num_tokens_per_rdma_rank[n]) status |= ORC_COUNT_MISMATCH;
    }

    int32_t sum = 0;
    for (int32_t r = 0; r < R; ++r) {
        sum += num_tokens_per_rank[r];
        recv_gbl_rank_prefix_sum[r] = sum;
    }
    *num_recv_tokens = sum;
    sum = 0;
    for (int32_t n = 0; n < nodes; ++n) {
        sum += num_tokens_per_rdma_rank[n];
        recv_rdma_rank_prefix_sum[n] = sum;
    }
    for (int32_t e = 0; e < E; ++e) {
        int32_t n = num_tokens_per_expert[e];
        num_recv_tokens_per_expert[e] = (n + expert_alignment - 1) / expert_alignment * expert_alignment;
    }
    return status;
}

/* ------------------------------------------------------------------------- */
/* Stages 3+4: dispatch.  The receive region is one allocation laid out
 * [dst_rank][channel]: slab r starts at the exclusive prefix of the receive
 * prefix sum, and inside a slab the channel segments follow in channel order,
 * tokens ascending (a channel's segment for rank r starts at
 * gbl_channel_prefix_matrix[r][c-1]).  So rows are handed out by walking
 * r, then c, then t, with one running row counter.
 * For each (t, r) routed:
 *   recv_x[row]          = x[t]                      (bitwise copy of the bf16 row)
 *   recv_topk_weights[row][j] = w[t][j] if slot j's expert lives on r, else 0
 *   recv_topk_idx[row][j]     = e - r*(E/R) (the receiver's local expert id) if
 *                               slot j's expert lives on r, else -1
 *   recv_src_info[row]   = {my_rank, t}   ([article] §4.1 SrcInfo)
 *   send_slot[t][r]      = row, -1 where token t is not sent to r
 *                          ([mscclpp] the per-(token, rank) gather map the dispatch
 *                          sender fills and combine reads).
 * Rows at or beyond recv_capacity are not written, their send_slot stays -1
 * and ORC_RECV_OVERFLOW is raised.  recv_topk_idx may be NULL.
 * The given prefixes are checked against the walk: a channel segment that does
 * not start where the walk reaches it, a slab that does not end at its receive
 * prefix, or a last column (inclusive, so the slab's whole count) that differs
 * raises ORC_COUNT_MISMATCH; the rows still follow the walk. */
static int orc_dispatch_rows(int32_t T, int64_t row_bytes, int32_t K, int32_t E, int32_t R, int32_t C,
                             int32_t my_rank, int32_t recv_capacity, const uint8_t *x, const float *x_scales,
                             int32_t num_scales, const int64_t *topk_idx, const float *topk_weights,
                             const uint8_t *is_token_in_rank, const int32_t *gbl_channel_prefix_matrix,
                             const int32_t *recv_gbl_rank_prefix_sum, uint8_t *recv_x, float *recv_x_scales,
                             float *recv_topk_weights, int64_t *recv_topk_idx, int32_t *recv_src_info,
                             int32_t *send_slot) {
    int status = 0;
    const int32_t experts_per_rank = E / R;
    for (int64_t i = 0; i < (int64_t)T * R; ++i) send_slot[i] = -1;

    for (int32_t r = 0; r < R; ++r) {
        const int64_t slab_begin = r > 0 ? recv_gbl_rank_prefix_sum[r - 1] : 0;
        int64_t row = slab_begin;
        for (int32_t c = 0; c < C; ++c) {
            const int64_t seg_begin = slab_begin + (c > 0 ? gbl_channel_prefix_matrix[(int64_t)r * C + c - 1] : 0);
            if (row != seg_begin) status |= ORC_COUNT_MISMATCH;
            for (int64_t t = orc_channel_begin(T, C, c); t < orc_channel_end(T, C, c); ++t) {
                if (!is_token_in_rank[t * R + r]) continue;
                if (row >= recv_capacity) {
                    status |= ORC_RECV_OVERFLOW;
                    ++row;
                    continue;
                }
                send_slot[t * R + r] = (int32_t)row;
                memcpy(recv_x + row * row_bytes, x + t * row_bytes, (size_t)row_bytes);
                for (int32_t i = 0; i < num_scales; ++i)
                    recv_x_scales[row * num_scales + i] = x_scales[t * num_scales + i];
                for (int32_t j = 0; j < K; ++j) {
                    int64_t e = topk_idx[t * K + j];
                    int on_r = orc_topk_valid(e, E, &status) && e / experts_per_rank == r;
                    recv_topk_weights[row * K + j] = on_r ? topk_weights[t * K + j] : 0.0f;
                    if (recv_topk_idx) recv_topk_idx[row * K + j] = on_r ? e - (int64_t)r * experts_per_rank : -1;
                }
                recv_src_info[row * 2 + 0] = my_rank;
                recv_src_info[row * 2 + 1] = (int32_t)t;
                ++row;
            }
        }
        if (row != (int64_t)recv_gbl_rank_prefix_sum[r]) status |= ORC_COUNT_MISMATCH;
        /* the last column is inclusive: it holds the slab's whole count */
        if (row != slab_begin + gbl_channel_prefix_matrix[(int64_t)r * C + C - 1]) status |= ORC_COUNT_MISMATCH;
    }
    return status;
}

/* bf16 rows of H elements. */
int oracle_dispatch(int32_t T, int32_t H, int32_t K, int32_t E, int32_t R, int32_t C,
                    int32_t my_rank, int32_t recv_capacity, const uint16_t *x,
                    const int64_t *topk_idx, const float *topk_weights,
                    const uint8_t *is_token_in_rank, const int32_t *gbl_channel_prefix_matrix,
                    const int32_t *recv_gbl_rank_prefix_sum, uint16_t *recv_x,
                    float *recv_topk_weights, int64_t *recv_topk_idx, int32_t *recv_src_info,
                    int32_t *send_slot) {
    return orc_dispatch_rows(T, (int64_t)H * 2, K, E, R, C, my_rank, recv_capacity, (const uint8_t *)x, NULL, 0,
                             topk_idx, topk_weights, is_token_in_rank, gbl_channel_prefix_matrix,
                             recv_gbl_rank_prefix_sum, (uint8_t *)recv_x, NULL, recv_topk_weights, recv_topk_idx,
                             recv_src_info, send_slot);
}

/* fp8 rows: H one-byte elements per token plus num_scales float scales per token,
 * both moved bit for bit ([mscclpp] internodeDispatch / intranodeDispatch take
 * x_scales with num_scales per token and return recv_x_scales; the FP8 scale
 * buffer travels beside the rows).  The combine side stays bf16. */
int oracle_dispatch_fp8(int32_t T, int32_t H, int32_t K, int32_t E, int32_t R, int32_t C, int32_t my_rank,
                        int32_t recv_capacity, const uint8_t *x, const float *x_scales, int32_t num_scales,
                        const int64_t *topk_idx, const float *topk_weights, const uint8_t *is_token_in_rank,
                        const int32_t *gbl_channel_prefix_matrix, const int32_t *recv_gbl_rank_prefix_sum,
                        uint8_t *recv_x, float *recv_x_scales, float *recv_topk_weights, int64_t *recv_topk_idx,
                        int32_t *recv_src_info, int32_t *send_slot) {
    return orc_dispatch_rows(T, (int64_t)H, K, E, R, C, my_rank, recv_capacity, x, x_scales, num_scales, topk_idx,
                             topk_weights, is_token_in_rank, gbl_channel_prefix_matrix, recv_gbl_rank_prefix_sum,
                             recv_x, recv_x_scales, recv_topk_weights, recv_topk_idx, recv_src_info, send_slot);
}

/* Cached mode ([mscclpp] internodeDispatch with cachedMode: the layout of an
 * earlier call is reused, no counting or notification).  Rows (and scales, when
 * num_scales > 0) go where send_slot [t][R] -- recorded by an earlier dispatch
 * with the same routing -- says; no metadata is produced.  Entries outside
 * [-1, recv_capacity) raise ORC_BAD_SEND_SLOT and are skipped. */
int oracle_dispatch_cached(int32_t T, int32_t R, int64_t row_bytes, const uint8_t *x, const float *x_scales,
                           int32_t num_scales, const int32_t *send_slot, int32_t recv_capacity, uint8_t *recv_x,
                           float *recv_x_scales) {
    int status = 0;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t r = 0; r < R; ++r) {
            int64_t s = send_slot[t * R + r];
            if (s == -1) continue;
            if (s < -1 || s >= recv_capacity) {
                status |= ORC_BAD_SEND_SLOT;
                continue;
            }
            memcpy(recv_x + s * row_bytes, x + t * row_bytes, (size_t)row_bytes);
            for (int32_t i = 0; i < num_scales; ++i) recv_x_scales[s * num_scales + i] = x_scales[t * num_scales + i];
        }
    }
    return status;
}

/* ------------------------------------------------------------------------- */
/* bf16 helpers (IEEE binary32 truncated to its upper 16 bits). */
static float orc_bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a binary32 value to the nearest bf16, ties to the even bf16 pattern:
 * compare the 16 dropped bits with the half-way point 0x8000.  NaN stays NaN
 * (quiet bit forced).  Infinities and the largest finite values overflow to
 * infinity as round-to-nearest prescribes. */
static uint16_t orc_f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xffffu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
    return (uint16_t)kept;
}

/* Exposed for the rounding pin (compared against a library conversion). */
void oracle_bf16_round(const float *in, uint16_t *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16_rne(in[i]);
}

/* ------------------------------------------------------------------------- */
/* Stage 5: combine.  [mscclpp] internodeCombine / intranodeCombine return
 * combined_x (bf16) and combined_topk_weights from the received rows and their
 * topk weights; [article] §4.2: each received row goes back to output[src_idx]
 * of its source.  The reduction order is not on the pages.  Reading:
 *   for each token t, over destination ranks r ascending with s = send_slot[t][r] >= 0:
 *     W = sum_j recv_topk_weights[s][j]   (fp32 adds, j ascending, from +0)
 *     acc[i] = fmaf(W, y[s][i], acc[i])   (fp32, acc starting at +0)
 *   combined_x[t][i] = bf16_rne(acc[i]);
 *   combined_topk_weights[t][j] = sum over the same r of recv_topk_weights[s][j]
 *                                 (fp32 adds, r ascending, from +0).
 * A token sent nowhere gets +0 rows and weights.  send_slot entries outside
 * [-1, num_recv) raise ORC_BAD_SEND_SLOT and are skipped.
 * combined_topk_weights may be NULL. */
int oracle_combine(int32_t T, int32_t H, int32_t K, int32_t R, int32_t num_recv, const uint16_t *y,
                   const float *recv_topk_weights, const int32_t *send_slot, uint16_t *combined_x,
                   float *combined_topk_weights, float *acc_scratch /* [H] */) {
    int status = 0;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t i = 0; i < H; ++i) acc_scratch[i] = 0.0f;
        if (combined_topk_weights)
            for (int32_t j = 0; j < K; ++j) combined_topk_weights[t * K + j] = 0.0f;
        for (int32_t r = 0; r < R; ++r) {
            int32_t s = send_slot[t * R + r];
            if (s == -1) continue;
            if (s < -1 || s >= num_recv) {
                status |= ORC_BAD_SEND_SLOT;
                continue;
            }
            float W = 0.0f;
            for (int32_t j = 0; j < K; ++j) W = W + recv_topk_weights[(int64_t)s * K + j];
            const uint16_t *yrow = y + (int64_t)s * H;
            for (int32_t i = 0; i < H; ++i) acc_scratch[i] = fmaf(W, orc_bf16_to_f32(yrow[i]), acc_scratch[i]);
            if (combined_topk_weights)
                for (int32_t j = 0; j < K; ++j)
                    combined_topk_weights[t * K + j] = combined_topk_weights[t * K + j] + recv_topk_weights[(int64_t)s * K + j];
        }
        for (int32_t i = 0; i < H; ++i) combined_x[t * H + i] = orc_f32_to_bf16_rne(acc_scratch[i]);
    }
    return status;
}

/* The same weighted sum evaluated in binary64 without the final rounding:
 * out[t][i] = sum_r (sum_j w[s_r][j]) * y[s_r][i].  Used only to bound the
 * rounding error of the fp32 combine (a pin, not a parity target). */
int oracle_combine_f64(int32_t T, int32_t H, int32_t K, int32_t R, int32_t num_recv, const uint16_t *y,
                       const float *recv_topk_weights, const int32_t *send_slot, double *out) {
    int status = 0;
    for (int64_t t = 0; t < T; ++t) {
        double *o = out + t * H;
        for (int32_t i = 0; i < H; ++i) o[i] = 0.0;
        for (int32_t r = 0; r < R; ++r) {
            int32_t s = send_slot[t * R + r];
            if (s == -1) continue;
            if (s < -1 || s >= num_recv) {
                status |= ORC_BAD_SEND_SLOT;
                continue;
            }
            double W = 0.0;
            for (int32_t j = 0; j < K; ++j) W += (double)recv_topk_weights[(int64_t)s * K + j];
            for (int32_t i = 0; i < H; ++i) o[i] += W * (double)orc_bf16_to_f32(y[(int64_t)s * H + i]);
        }
    }
    return status;
}

/* ------------------------------------------------------------------------- */
/* Grouping of the receive rows by local expert (the step after dispatch that
 * grouped expert GEMMs consume).  The pages give only its sizes: [notes] sm0
 * stage 6 and [mscclpp] internodeNotifyDispatch hand back, per local expert,
 * the received slot count rounded up to expert_alignment.  Reading (the
 * grouping order itself is not on the pages):
 *   a receive row of slab r holds, for slot j, local expert
 *   le = recv_topk_idx[row][j] (-1 = not on r); its global expert is
 *   e = r * (E / R) + le.  Segment e of the grouped region starts at
 *   sum_{e' < e} aligned[e'] and holds, in (row, j) ascending order, one entry
 *   per (row, j) with that expert; positions past the entries up to aligned[e]
 *   are padding (zero row, grouped_row -1, weight 0).
 *   grouped_x[pos] = recv_x[row] (bitwise, with its scales), grouped_row[pos] =
 *   row, grouped_weights[pos] = recv_topk_weights[row][j], slot_pos[row][j] =
 *   pos (-1 for slots with no entry).  *num_grouped_rows = sum_e aligned[e].
 * Rows at or past the end of the last slab (or num_recv_rows) hold no
 * received token -- capacity slack -- so their ids are not read; their
 * slot_pos entries are -1.  A negative segment size counts as 0.  An entry
 * beyond its segment's aligned size or at/after grouped_capacity is skipped
 * with ORC_RECV_OVERFLOW; a local id outside [-1, E/R) in a slab row with
 * ORC_BAD_TOPK_IDX. */
int oracle_group_by_expert(int32_t E, int32_t R, int32_t K, int64_t row_bytes, const uint8_t *recv_x,
                           const float *recv_x_scales, int32_t num_scales, const int64_t *recv_topk_idx,
                           const float *recv_topk_weights, const int32_t *recv_gbl_rank_prefix_sum,
                           const int32_t *aligned_per_expert, int32_t num_recv_rows, int32_t grouped_capacity,
                           uint8_t *grouped_x, float *grouped_x_scales, int32_t *grouped_row,
                           float *grouped_weights, int32_t *slot_pos, int32_t *num_grouped_rows) {
    int status = 0;
    const int32_t er = E / R;
    int64_t last = recv_gbl_rank_prefix_sum[R - 1]; /* end of the last slab */
    if (last > num_recv_rows) last = num_recv_rows;
    for (int64_t i = 0; i < (int64_t)num_recv_rows * K; ++i) {
        slot_pos[i] = -1;
        if (i < last * K && (recv_topk_idx[i] < -1 || recv_topk_idx[i] >= er)) status |= ORC_BAD_TOPK_IDX;
    }
    int64_t offset = 0; /* start of segment e */
    for (int32_t r = 0; r < R; ++r) {
        int64_t lo = (r == 0) ? 0 : recv_gbl_rank_prefix_sum[r - 1]; /* slab r */
        int64_t hi = recv_gbl_rank_prefix_sum[r];
        if (hi > num_recv_rows) hi = num_recv_rows;
        if (lo > hi) lo = hi;
        for (int32_t le = 0; le < er; ++le) {
            const int32_t e = r * er + le;
            const int64_t size = aligned_per_expert[e] > 0 ? aligned_per_expert[e] : 0;
            int64_t used = 0; /* entries placed so far in segment e */
            for (int64_t row = lo; row < hi; ++row) {
                for (int32_t j = 0; j < K; ++j) {
                    if (recv_topk_idx[row * K + j] != le) continue;
                    const int64_t pos = offset + used;
                    if (used >= size || pos >= grouped_capacity) {
                        status |= ORC_RECV_OVERFLOW;
                        continue;
                    }
                    memcpy(grouped_x + pos * row_bytes, recv_x + row * row_bytes, (size_t)row_bytes);
                    for (int32_t i = 0; i < num_scales; ++i)
                        grouped_x_scales[pos * num_scales + i] = recv_x_scales[row * num_scales + i];
                    grouped_row[pos] = (int32_t)row;
                    grouped_weights[pos] = recv_topk_weights[row * K + j];
                    slot_pos[row * K + j] = (int32_t)pos;
                    ++used;
                }
            }
            for (int64_t i = used; i < size; ++i) { /* padding */
                const int64_t pos = offset + i;
                if (pos >= grouped_capacity) break;
                memset(grouped_x + pos * row_bytes, 0, (size_t)row_bytes);
                for (int32_t s = 0; s < num_scales; ++s) grouped_x_scales[pos * num_scales + s] = 0.0f;
                grouped_row[pos] = -1;
                grouped_weights[pos] = 0.0f;
            }
            offset += size;
        }
    }
    *num_grouped_rows = (int32_t)offset;
    return status;
}

/* ------------------------------------------------------------------------- */
/* fp8 rows and their scales.  [mscclpp] intranodeDispatch / internodeDispatch
 * take x with an element size of one byte together with xScales, numScales
 * float scales per token, and return them as recvXScales (the "FP8 scale
 * buffer"); combine stays bf16.  How x and its scales are produced is not on
 * the pages.  Reading (the quantiser this library offers for that input):
 *  - element format: OCP FP8 E4M3.  One sign bit, four exponent bits (bias 7)
 *    and three mantissa bits; a zero exponent field holds the subnormals
 *    m * 2^-9; the patterns S.1111.111 are NaN; there are no infinities; the
 *    largest finite value is 1.75 * 2^8 = 448.
 *  - a row of H channels splits into S = num_scales groups of g = H / S
 *    consecutive channels; group q of row t takes
 *        a = max(max over the group of |x|, 2^-64)       (exact in binary32)
 *        scale[t][q] = a / 448                            (binary32 division)
 *        code[t][i]  = e4m3(clamp(x[t][i] * (448 / a), -448, 448))
 *    with 448 / a and the product each rounded to binary32 and e4m3() the
 *    nearest value, ties to the even code; -0 and negative values that round
 *    to zero keep the sign bit.  The floor 2^-64 keeps 448 / a finite and the
 *    scale a normal binary32 number for an all-zero (or tiny) group.
 *  - dequantisation: out[t][i] = bf16_rne(value(code[t][i]) * scale[t][q]),
 *    the product rounded to binary32.
 * Inputs are finite; a group holding an infinity or NaN is outside the
 * reading (its codes are not defined here). */

/* The value of an E4M3 pattern, straight from the field definition. */
static double orc_e4m3_value(uint8_t c) {
    const int sign = c >> 7, ex = (c >> 3) & 15, man = c & 7;
    if (ex == 15 && man == 7) return NAN;
    double mag = ex == 0 ? ldexp((double)man, -9) : ldexp(1.0 + man / 8.0, ex - 7);
    return sign ? -mag : mag;
}

/* Nearest E4M3 pattern to a finite v with |v| <= 448, ties to the even
 * pattern.  Normal range (|v| >= 2^-6): with |v| = f * 2^E, 1 <= f < 2, the
 * representable neighbours are spaced 2^(E-3) apart, so the mantissa is
 * rint(|v| / 2^(E-3)) in [8, 16]; 16 carries into the next binade.  Below
 * 2^-6 the spacing is the subnormal step 2^-9. */
static uint8_t orc_e4m3_rne(float v) {
    const double mag = fabs((double)v);
    uint8_t code;
    if (mag >= ldexp(1.0, -6)) {
        int e;
        (void)frexp(mag, &e); /* mag = m * 2^e, 0.5 <= m < 1 */
        int E = e - 1;
        double q = rint(ldexp(mag, 3 - E)); /* exact scaling; rint rounds half to even */
        if (q == 16.0) {
            q = 8.0;
            E += 1;
        }
        code = (uint8_t)(((E + 7) << 3) | ((int)q - 8));
    } else {
        code = (uint8_t)rint(ldexp(mag, 9)); /* 0..8; 8 is the smallest normal */
    }
    return signbit(v) ? (uint8_t)(code | 0x80) : code;
}

/* Exposed for the pins (compared with a library conversion and a brute-force
 * nearest-value search). */
void oracle_e4m3_encode(const float *in, uint8_t *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_rne(in[i]);
}
void oracle_e4m3_decode(const uint8_t *in, double *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_value(in[i]);
}

/* Quantise rows [rows][H] bf16 to E4M3 codes [rows][H] and scales
 * [rows][num_scales] as read above.  Returns 0, or -1 when num_scales does not
 * divide H. */
int oracle_quantize_e4m3(int64_t rows, int32_t H, int32_t num_scales, const uint16_t *x, uint8_t *codes,
                         float *scales) {
    if (num_scales <= 0 || H % num_scales != 0) return -1;
    const int32_t g = H / num_scales;
    for (int64_t t = 0; t < rows; ++t) {
        for (int32_t q = 0; q < num_scales; ++q) {
            const uint16_t *xg = x + t * H + (int64_t)q * g;
            float a = 0.0f;
            for (int32_t i = 0; i < g; ++i) {
                const float m = fabsf(orc_bf16_to_f32(xg[i]));
                if (m > a) a = m;
            }
            if (a < 0x1p-64f) a = 0x1p-64f;
            const float inv = 448.0f / a;
            scales[t * num_scales + q] = a / 448.0f;
            for (int32_t i = 0; i < g; ++i) {
                float v = orc_bf16_to_f32(xg[i]) * inv;
                if (v > 448.0f) v = 448.0f;
                if (v < -448.0f) v = -448.0f;
                codes[t * H + (int64_t)q * g + i] = orc_e4m3_rne(v);
            }
        }
    }
    return 0;
}

/* Dequantise codes [rows][H] with scales [rows][num_scales] to bf16 [rows][H]:
 * value(code) * scale rounded to binary32, then to bf16 (nearest, ties to
 * even).  value() is exact in binary32.  Returns 0, or -1 when num_scales
 * does not divide H. */
int oracle_dequantize_e4m3(int64_t rows, int32_t H, int32_t num_scales, const uint8_t *codes, const float *scales,
                           uint16_t *out) {
    if (num_scales <= 0 || H % num_scales != 0) return -1;
    const int32_t g = H / num_scales;
    for (int64_t t = 0; t < rows; ++t)
        for (int32_t i = 0; i < H; ++i) {
            const float v = (float)orc_e4m3_value(codes[t * H + i]);
            out[t * H + i] = orc_f32_to_bf16_rne(v * scales[t * num_scales + i / g]);
        }
    return 0;
}
