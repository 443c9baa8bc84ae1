// ep_notify.hip -- stage 2, notify (gfx950).
//
// Definitions (internode.cu notes, notify_dispatch; mscclpp ht_runtime.cc
// mirror, internodeNotifyDispatch):
//   gbl_channel_prefix_matrix[r][c]  = tokens of channels 0..c sent to rank r
//                                      (prefix over channels, inclusive)
//   rdma_channel_prefix_matrix[n][c] = the same for node n (a token counts once
//                                      per node, when any rank of the node gets it)
//   recv_gbl_rank_prefix_sum[r]      = inclusive prefix of num_tokens_per_rank
//   recv_rdma_rank_prefix_sum[n]     = inclusive prefix of num_tokens_per_rdma_rank
//   num_recv_tokens_per_expert[e]    = per-expert count rounded up to expert_alignment
//   num_recv_tokens                  = last entry of recv_gbl_rank_prefix_sum
// Channel c owns tokens [c*Tc, min((c+1)*Tc, t)), Tc = ceil(t / C).
//
// Design (not the pages' one-SM-per-channel loop): one launch.  The token axis
// is cut into 64-token chunks, one chunk per wave and one token per lane, and
// the chunks into groups of four.
//   Every wave turns its lanes' is_token_in_rank rows into 64-bit rank masks
//   (stored for dispatch); a 64x64 bit transpose across the wave hands lane r
//   the chunk's column for rank r, whose popcount is the (chunk, rank) count.
//   The four waves of a group trade their counts through LDS: each stores its
//   chunk's offset inside the group, and for each channel whose end falls in
//   its chunk the value there (that offset plus the chunk's tokens before the
//   end); the group's last chunk stores the group's totals.  Every value has
//   one writer: no atomics.
//   The last block to finish (the only one, without an election, up to 1024
//   tokens) then scans only the group totals: it brings them into LDS in one
//   round trip (or works in the workspace when they do not fit), each thread
//   scanning a run of groups of one column (rank or node) in registers and one
//   wave per column combining the runs with a shuffle scan, which gives each
//   group's row offset inside each rank's slab.  A chunk's offset (what
//   dispatch needs) is its group's offset plus its offset inside the group; a
//   channel's prefix is the offset of the group holding its end plus the value
//   stored for it.  The receive prefixes over ranks and nodes are one wave scan
//   each.
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kNotifyWaves = 16;
constexpr int kNotifyThreads = kNotifyWaves * kWave;

struct NotifyParams {
    const uint8_t *in_rank;
    const int32_t *per_rank, *per_node, *per_expert;
    int32_t *gbl, *rdma, *recv_gbl, *recv_rdma, *recv_per_expert, *num_recv;
    uint64_t *mask;
    int32_t *rank_off, *rank_base, *node_base, *rank_part, *node_part;
    uint64_t *ticket;  // completion ticket (chunks)
    int32_t *dev_status;
    int64_t T, Tc;
    int R, C, E, nodes, align, load_unit;
    // fused layout + notify: the per-rank / per-node totals are not inputs but come
    // from the scan, and are written to tot_rank / tot_node
    bool fused;
    int32_t *tot_rank, *tot_node;
};

// A chunk's columns: lane r (< R) holds which of the chunk's 64 tokens go to
// rank r, lane n (< nodes) which of them reach node n.
struct ChunkCols {
    uint64_t rank_bits, node_bits;
};

// The chunk's columns from its tokens' rank masks (lane l: token q*64 + l's
// mask, 0 past the last token).  Stores the masks for dispatch and the chunk's
// per-rank and per-node counts into the LDS row s_row (ranks, then nodes).
__device__ ChunkCols chunk_columns(const NotifyParams &p, int64_t q, int lane, uint64_t m, int32_t *s_row) {
    const int64_t tok = q * kChunk + lane;
    const int R = p.R, nodes = p.nodes;
    if (tok < p.T) p.mask[tok] = m;
    ChunkCols cc;
    cc.rank_bits = transpose64(m);
    cc.node_bits = 0;
    for (int n = 0; n < nodes; ++n) {
        const bool any = R < kRanksPerNode ? m != 0 : ((m >> (n * kRanksPerNode)) & 0xffull) != 0;
        const uint64_t b = ballot64(any);
        cc.node_bits = (lane == n) ? b : cc.node_bits;
    }
    if (lane < R) s_row[lane] = __popcll(cc.rank_bits);
    if (lane < nodes) s_row[R + lane] = __popcll(cc.node_bits);
    return cc;
}

// Chunk q, the w-th of the nw chunks of its group (LDS rows s_grp[0..nw) hold
// the group's chunk counts): its offset inside the group (the tokens of the
// group's earlier chunks) goes to rank_off, the value at each channel end that
// falls in [64q, 64q + 64) -- that offset plus the chunk's tokens before the end
// -- to rank_part / node_part, and, from the group's last chunk, the group's
// totals to rank_base / node_base.
__device__ void chunk_offsets(const NotifyParams &p, int64_t q, int lane, const ChunkCols &cc, const int32_t *s_grp,
                              int w, int nw) {
    const int R = p.R, nodes = p.nodes, NC = R + nodes;
    int32_t ro = 0, no = 0;
    for (int j = 0; j < w; ++j) {
        if (lane < R) ro += s_grp[j * NC + lane];
        if (lane < nodes) no += s_grp[j * NC + R + lane];
    }
    if (lane < R) p.rank_off[q * R + lane] = ro;
    const int64_t first = q * kChunk;
    // from the channel before the one holding token `first` (it may end exactly
    // there); a 32-bit division whenever T allows
    const int64_t c_hold = p.T <= INT32_MAX ? (int64_t)((uint32_t)first / (uint32_t)p.Tc) : first / p.Tc;
    for (int64_t c = c_hold > 0 ? c_hold - 1 : 0; c < p.C; ++c) {
        const int64_t end = (c + 1) * p.Tc < p.T ? (c + 1) * p.Tc : p.T;
        if (end >= first + kChunk) break;
        if (end < first) continue;
        const uint64_t below = (1ull << (end - first)) - 1ull;  // end - first in [0, 63]
        if (lane < R) p.rank_part[c * R + lane] = ro + __popcll(cc.rank_bits & below);
        if (lane < nodes) p.node_part[c * nodes + lane] = no + __popcll(cc.node_bits & below);
    }
    if (w == nw - 1) {
        const int64_t g = q / kGroupChunks;
        if (lane < R) p.rank_base[g * R + lane] = ro + __popcll(cc.rank_bits);
        if (lane < nodes) p.node_base[g * nodes + lane] = no + __popcll(cc.node_bits);
    }
}

// One wave scans one column of a [rows][stride] count matrix in place into
// exclusive offsets.  Returns the column's total.
__device__ int32_t scan_column(int32_t *col, int stride, int64_t rows, int lane) {
    const int64_t per = (rows + kWave - 1) / kWave;
    const int64_t b = lane * per;
    const int64_t e = (b + per) < rows ? (b + per) : rows;
    int32_t s = 0;
    for (int64_t row = b; row < e; ++row) s += col[row * stride];
    const int32_t incl = wave_inclusive_scan(s);
    int32_t run = incl - s;
    for (int64_t row = b; row < e; ++row) {
        const int32_t v = col[row * stride];
        col[row * stride] = run;
        run += v;
    }
    return readlane32(incl, kWave - 1);
}

// groups of a column one lane of the last block holds: 1 (up to 64 groups, 16384
// tokens) or 4 (up to 256 groups); larger problems finish in global memory
constexpr int kMaxGroupsPerLane = 4;
// per-expert counts a thread of the last block loads with the others (E <= 4096 in one go)
constexpr int kExpertBatch = 4;
// columns (ranks + nodes <= 72) a wave of the last block takes: ceil(72 / 16)
constexpr int kColBatch = 5;

__device__ __forceinline__ int64_t channel_end(const NotifyParams &p, int64_t c) {
    return (c + 1) * p.Tc < p.T ? (c + 1) * p.Tc : p.T;
}

// Inclusive prefix sums over destination ranks and nodes (two waves), and N.
__device__ void recv_prefixes(const NotifyParams &p, int32_t per_rank, int32_t per_node, int lane, int wave) {
    if (wave == kNotifyWaves - 1) {
        const int32_t incl = wave_inclusive_scan(per_rank);
        if (lane < p.R) p.recv_gbl[lane] = incl;
        if (lane == p.R - 1) p.num_recv[0] = incl;
    } else if (wave == kNotifyWaves - 2) {
        const int32_t incl = wave_inclusive_scan(per_node);
        if (lane < p.nodes) p.recv_rdma[lane] = incl;
    }
}

// Fused layout + notify: the per-rank and per-node totals are the scan's column
// totals (tot[column]); they are written out and the receive prefixes follow them.
__device__ void finish_totals(const NotifyParams &p, const int32_t *tot, int lane, int wave) {
    const int32_t per_rank = lane < p.R ? tot[lane] : 0;
    const int32_t per_node = lane < p.nodes ? tot[p.R + lane] : 0;
    if (wave == kNotifyWaves - 1 && lane < p.R) p.tot_rank[lane] = per_rank;
    if (wave == kNotifyWaves - 2 && lane < p.nodes) p.tot_node[lane] = per_node;
    recv_prefixes(p, per_rank, per_node, lane, wave);
}

// Groups of a column per lane for the last block's column-wise finish (1 or 4),
// or 0 when the problem finishes in global memory instead (more than 256 groups,
// T of 2^20 or more, or more columns than its waves take).
__device__ __forceinline__ int finish_groups_per_lane(const NotifyParams &p) {
    const int64_t G = num_groups(p.T);
    if (p.T >= (1 << 20) || p.R + p.nodes > kColBatch * kNotifyWaves) return 0;
    return G <= kWave ? 1 : G <= kMaxGroupsPerLane * kWave ? kMaxGroupsPerLane : 0;
}

// Last block, up to 64 * PG groups: one wave per column (ranks, then nodes; wave
// w takes columns w, w + 16, ...), no barrier until the totals.  Lane j holds
// groups j*PG .. j*PG + PG - 1 of the column; all of a wave's loads (its columns'
// group totals and the values stored at channel ends j, j + 64, ... -- the first
// 64 in this round trip) are made before any is used.  A column's group offsets
// come from the lane's running sum and a wave scan, go back to the workspace
// (dispatch adds them to its chunks' offsets) and to a row of LDS the wave
// alone uses; lane j then takes channel j: the offset of the group its end falls
// in plus the value stored for the end (an end at t = 64 Q is the column total),
// so each prefix-matrix row goes out in consecutive words.  All indices fit 32
// bits (T < 2^20 here).
template <bool FUSED, int PG, class Mid>
__device__ void finish_by_columns(const NotifyParams &p, int tid, int lane, int wave, Mid mid) {
    __shared__ int32_t s_goff[kNotifyWaves][kMaxGroupsPerLane * kWave];  // a wave's column of group offsets
    __shared__ int32_t s_tot[kMaxRanks + kMaxRanks / kRanksPerNode];
    const int R = p.R, nodes = p.nodes, NC = R + nodes, C = p.C;
    const int T = (int)p.T, Tc = (int)p.Tc;
    const int Q = (T + kChunk - 1) / kChunk, G = (Q + kGroupChunks - 1) / kGroupChunks;
    auto end_of = [&](int c) { return (c + 1) * Tc < T ? (c + 1) * Tc : T; };

    // ---- one round trip of loads for all of the wave's columns (and, for
    // notify, the totals and per-expert counts), issued before any is used
    int32_t gv[kColBatch][PG], cv[kColBatch];
    const bool c_in = lane < C && end_of(lane) < Q * kChunk;  // channel `lane` ends inside a chunk
#pragma unroll
    for (int k = 0; k < kColBatch; ++k) {
        const int col = wave + k * kNotifyWaves;  // the same for the whole wave
        const bool on = col < NC;
        const bool is_rank = col < R;
        const int stride = is_rank ? R : nodes;
        const int32_t *gsrc = (is_rank ? p.rank_base + col : p.node_base + (col - R)) + (ptrdiff_t)lane * PG * stride;
        const int32_t *csrc = (is_rank ? p.rank_part + col : p.node_part + (col - R)) + (ptrdiff_t)lane * stride;
#pragma unroll
        for (int i = 0; i < PG; ++i) gv[k][i] = (on && lane * PG + i < G) ? gsrc[i * stride] : 0;
        cv[k] = (on && c_in) ? *csrc : 0;
    }
    int32_t per_rank = 0, per_node = 0, pe[kExpertBatch];
    if constexpr (!FUSED) {
        per_rank = p.per_rank[lane < R ? lane : 0];
        per_node = p.per_node[lane < nodes ? lane : 0];
#pragma unroll
        for (int k = 0; k < kExpertBatch; ++k) {
            const int e = tid + k * kNotifyThreads;
            pe[k] = p.per_expert[e < p.E ? e : 0];
        }
    }

    // ---- per column: offsets, then the prefix-matrix row
#pragma unroll
    for (int k = 0; k < kColBatch; ++k) {
        const int col = wave + k * kNotifyWaves;
        if (col >= NC) break;  // wave-uniform
        const bool is_rank = col < R;
        const int stride = is_rank ? R : nodes;
        int32_t *gdst = (is_rank ? p.rank_base + col : p.node_base + (col - R)) + (ptrdiff_t)lane * PG * stride;
        int32_t run = 0;
#pragma unroll
        for (int i = 0; i < PG; ++i) run += gv[k][i];
        const int32_t incl = wave_inclusive_scan(run);
        const int32_t total = readlane32(incl, kWave - 1);
        run = incl - run;
#pragma unroll
        for (int i = 0; i < PG; ++i) {
            if (lane * PG + i < G) {
                gdst[i * stride] = run;
                s_goff[wave][lane * PG + i] = run;
            }
            run += gv[k][i];
        }
        if (lane == 0) s_tot[col] = total;
        int32_t *row = is_rank ? p.gbl + col * C : p.rdma + (col - R) * C;
        auto prefix = [&](int c, int32_t at_end) {
            const int qe = end_of(c) / kChunk;
            return qe < Q ? s_goff[wave][qe / kGroupChunks] + at_end : total;
        };
        if (lane < C) row[lane] = prefix(lane, cv[k]);
        const int32_t *csrc = is_rank ? p.rank_part + col : p.node_part + (col - R);
        for (int c = lane + kWave; c < C; c += kWave)
            row[c] = prefix(c, end_of(c) < Q * kChunk ? csrc[c * stride] : 0);
    }
    // the caller's work that waits on its own memory round trip (made beside these
    // loads), after every load above is consumed: a wait for one of them after its
    // stores would wait for those stores too
    mid();
    if constexpr (!FUSED) {  // aligned per-expert counts need nothing from the scan
        per_rank = lane < R ? per_rank : 0;
        per_node = lane < nodes ? per_node : 0;
        auto aligned = [&](int32_t n) { return (int32_t)(((int64_t)n + p.align - 1) / p.align * p.align); };
#pragma unroll
        for (int k = 0; k < kExpertBatch; ++k) {
            const int e = tid + k * kNotifyThreads;
            if (e < p.E) p.recv_per_expert[e] = aligned(pe[k]);
        }
        for (int e = tid + kExpertBatch * kNotifyThreads; e < p.E; e += kNotifyThreads)
            p.recv_per_expert[e] = aligned(p.per_expert[e]);
    }
    __syncthreads();  // s_tot complete

    // receive prefix sums over destination ranks and nodes (inclusive): fused,
    // from the scan's totals; notify, from its inputs, checked against the totals
    if constexpr (FUSED) {
        finish_totals(p, s_tot, lane, wave);
    } else {
        recv_prefixes(p, per_rank, per_node, lane, wave);
        if (wave == kNotifyWaves - 3) {
            const bool bad = (lane < R && s_tot[lane] != per_rank) || (lane < nodes && s_tot[R + lane] != per_node);
            if (ballot64(bad) != 0ull && lane == 0) flag(p.dev_status, EP_DEV_COUNT_MISMATCH);
        }
    }
}

// Last block, large problems: the same steps on the workspace in global memory.
template <class Mid>
__device__ void finish_in_global(const NotifyParams &p, int tid, int lane, int wave, Mid mid) {
    mid();
    __shared__ int32_t s_tot_g[kMaxRanks + kMaxRanks / kRanksPerNode];
    const int R = p.R, nodes = p.nodes, NC = R + nodes;
    const int64_t Q = num_chunks(p.T), G = num_groups(p.T);
    for (int col = wave; col < NC; col += kNotifyWaves) {
        const bool is_rank = col < R;
        int32_t *cp = is_rank ? p.rank_base + col : p.node_base + (col - R);
        const int32_t total = scan_column(cp, is_rank ? R : nodes, G, lane);
        if (lane == 0) s_tot_g[col] = total;
        if (!p.fused) {
            const int32_t want = is_rank ? p.per_rank[col] : p.per_node[col - R];
            if (lane == 0 && total != want) flag(p.dev_status, EP_DEV_COUNT_MISMATCH);
        }
    }
    if (!p.fused) {
        recv_prefixes(p, lane < R ? p.per_rank[lane] : 0, lane < nodes ? p.per_node[lane] : 0, lane, wave);
        for (int e = tid; e < p.E; e += kNotifyThreads) {  // fused, the expert totals' loop writes them
            const int64_t n = p.per_expert[e];
            p.recv_per_expert[e] = (int32_t)((n + p.align - 1) / p.align * p.align);
        }
    }
    __syncthreads();  // the group offsets and totals visible to the whole block
    if (p.fused) finish_totals(p, s_tot_g, lane, wave);
    for (int64_t i = tid; i < (int64_t)NC * p.C; i += kNotifyThreads) {
        const int cc = (int)(i / p.C);
        const int64_t c = i % p.C;
        const int64_t qe = channel_end(p, c) / kChunk;
        const int64_t g = qe / kGroupChunks;
        if (cc < R) {
            p.gbl[cc * (int64_t)p.C + c] = qe < Q ? p.rank_base[g * R + cc] + p.rank_part[c * R + cc] : s_tot_g[cc];
        } else {
            const int n = cc - R;
            p.rdma[n * (int64_t)p.C + c] = qe < Q ? p.node_base[g * nodes + n] + p.node_part[c * nodes + n] : s_tot_g[cc];
        }
    }
}

static_assert(kNotifyWaves % kGroupChunks == 0, "a block holds whole groups of chunks");

__global__ __launch_bounds__(kNotifyThreads) void notify_kernel(NotifyParams p) {
    __shared__ int32_t s_grp[kNotifyWaves * (kMaxRanks + kMaxRanks / kRanksPerNode)];  // [wave][NC] chunk counts
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const int64_t Q = num_chunks(p.T);
    const int NC = p.R + p.nodes;

    // every lane reads the epoch (thread 0 uses it): a load under a branch would be
    // waited for where the branch joins, before this wave issues its own loads
    const uint32_t epoch0 = ticket_epoch(p.ticket);
    // the wave's chunk from its tokens' is_token_in_rank rows, then its offsets
    // inside its group once the group's four waves have counted
    const int64_t q = (int64_t)blockIdx.x * kNotifyWaves + wave;
    ChunkCols cc{0ull, 0ull};
    if (q < Q) {
        const int64_t tok = q * kChunk + lane;
        const uint64_t m = tok < p.T ? load_rank_mask(p.in_rank + tok * p.R, p.R, p.load_unit) : 0ull;
        cc = chunk_columns(p, q, lane, m, s_grp + wave * NC);
    }
    __syncthreads();
    if (q < Q) {
        const int w = wave % kGroupChunks;
        const int64_t left = Q - (q - w);
        chunk_offsets(p, q, lane, cc, s_grp + (wave - w) * NC, w, (int)(left < kGroupChunks ? left : kGroupChunks));
    }

    // a single block (up to 1024 tokens) finishes once its own waves are done:
    // a workgroup barrier (with its workgroup-scope fences) makes their stores
    // visible, and no ticket is taken.  Otherwise the ticket counts chunks, and
    // the block that completes them scans (a ticket that was not zero is flagged,
    // see elect_completing_block).
    if (gridDim.x == 1) {
        __syncthreads();
    } else {
        const int64_t left = Q - (int64_t)blockIdx.x * kNotifyWaves;
        const uint32_t mine = (uint32_t)(left < kNotifyWaves ? left : kNotifyWaves);
        if (!elect_completing_block(p.ticket, epoch0, mine, (uint32_t)Q, p.dev_status)) return;
    }
    const int pg = finish_groups_per_lane(p);
    if (pg == 1)
        finish_by_columns<false, 1>(p, tid, lane, wave, [] {});
    else if (pg == kMaxGroupsPerLane)
        finish_by_columns<false, kMaxGroupsPerLane>(p, tid, lane, wave, [] {});
    else
        finish_in_global(p, tid, lane, wave, [] {});
}

// ---------------------------------------------------------------- layout + notify in one launch
// From topk_idx straight to every output of both stages.  A block takes 256
// tokens (four chunks), four lanes to a token: lane j of a quad reads the token's
// ids j, j+4, ..., so a wave's loads cover 16 consecutive topk rows, and the
// quad ORs its rank bits together (as the layout builds a mask).  Waves 0..3
// then count one chunk each from the masks in LDS (as notify does from
// is_token_in_rank): one pass over the tokens, one election.  Few waves per CU
// keep the LDS histogram's atomics and the loads' address work spread over many
// CUs.  The per-expert counts go through that histogram and the running counts;
// the per-rank and per-node totals are the scan's column totals.  The completing
// block publishes the expert totals and then finishes as notify does, with all
// sixteen waves.
constexpr int kFusedMaxLdsExperts = 8192;  // 32 KiB of LDS histogram; larger E counts in the workspace
constexpr int kFusedChunks = 4;            // chunks per block
constexpr int kFusedTokens = kFusedChunks * kChunk;
static_assert(kFusedTokens * 4 == kNotifyThreads, "four lanes per token");
static_assert(kFusedChunks == kGroupChunks, "a block's chunks are one group");

// OR of a 64-bit value over the four lanes of each quad (two DPP quad permutations).
__device__ __forceinline__ uint64_t quad_or64(uint64_t v) {
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    lo |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, 0xB1, 0xf, 0xf, false);  // quad_perm [1,0,3,2]
    hi |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, 0xB1, 0xf, 0xf, false);
    lo |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, 0x4E, 0xf, 0xf, false);  // quad_perm [2,3,0,1]
    hi |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, 0x4E, 0xf, 0xf, false);
    return ((uint64_t)hi << 32) | lo;
}

struct FusedParams {
    const int64_t *topk_idx;
    int32_t *per_expert;
    uint8_t *in_rank;
    int32_t *acc_expert;  // running per-expert counts [E], zero between calls
    uint64_t *ticket;     // completion ticket (chunks)
    uint32_t *report;     // valid slots the finished blocks report
    int K, store_unit;
};

// SINGLE: a one-block grid (up to 256 tokens), which finishes without an election
// and keeps the per-expert counts in LDS; a compile-time choice, so that neither
// instantiation carries the other's branches between its loads.  KQ: topk slots
// per lane, ceil(topk / 4) rounded up to 2 or 8.
template <bool SINGLE, int KQ>
__global__ __launch_bounds__(kNotifyThreads) void layout_notify_kernel(FusedParams f, NotifyParams p) {
    __shared__ uint64_t s_mask[kFusedTokens];
    __shared__ int32_t s_grp[kFusedChunks * (kMaxRanks + kMaxRanks / kRanksPerNode)];  // [chunk][NC] counts
    __shared__ uint32_t s_slots, s_esum;
    extern __shared__ int32_t s_expert[];  // E entries when E <= kFusedMaxLdsExperts
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const int R = p.R, E = p.E, K = f.K;
    const bool lds_experts = E <= kFusedMaxLdsExperts;
    constexpr bool single = SINGLE;
    const uint32_t epoch0 = SINGLE ? 0u : ticket_epoch(f.ticket);  // every lane, as in notify_kernel
    const int64_t Q = num_chunks(p.T);
    if (tid == 0) {
        s_slots = 0;
        s_esum = 0;
    }
    if (lds_experts)
        for (int e = tid; e < E; e += kNotifyThreads) s_expert[e] = 0;
    __syncthreads();

    // ---- the token's slots part, part + 4, ...: rank bits, valid slots, expert counts
    const int64_t t0 = (int64_t)blockIdx.x * kFusedTokens;
    const int64_t t = t0 + (tid >> 2);
    const int part = tid & 3;
    const int experts_per_rank = E / R;
    uint64_t mask = 0;
    int bad = 0, slots = 0;
    if (t < p.T) {
        const int64_t *row = f.topk_idx + t * K;
        int64_t ev[KQ];  // all of the lane's loads in flight together
#pragma unroll
        for (int u = 0; u < KQ; ++u) ev[u] = part + 4 * u < K ? row[part + 4 * u] : -1;
#pragma unroll
        for (int u = 0; u < KQ; ++u) {
            const int64_t e = ev[u];
            if (e == -1) continue;
            if (e < -1 || e >= E) {
                bad = 1;
                continue;
            }
            ++slots;
            if (lds_experts)
                atomicAdd(&s_expert[(int)e], 1);
            else
                atomicAdd(&f.acc_expert[(int)e], 1);
            mask |= 1ull << ((int)e / experts_per_rank);
        }
    }
    mask = quad_or64(mask);  // every lane of the quad: the token's rank mask
    if (part == 0) s_mask[tid >> 2] = mask;
    if (ballot64(bad != 0) != 0ull && lane == 0) flag(p.dev_status, EP_DEV_BAD_TOPK_IDX);
    const int w_slots = wave_sum(slots);
    if (lane == 0) atomicAdd(&s_slots, (uint32_t)w_slots);
    __syncthreads();

    // ---- the block's chunks (one group), one wave each, from the masks in LDS
    const int64_t q = (int64_t)blockIdx.x * kFusedChunks + wave;
    const bool counts = wave < kFusedChunks && q < Q;
    ChunkCols cc{0ull, 0ull};
    if (counts) cc = chunk_columns(p, q, lane, s_mask[wave * kChunk + lane], s_grp + wave * (R + p.nodes));

    // ---- is_token_in_rank rows of this block: one contiguous range of nt*R bytes
    {
        const int64_t left = p.T - t0;
        const int nt = (int)(left < kFusedTokens ? (left > 0 ? left : 0) : kFusedTokens);
        const int nbytes = nt * R;
        uint8_t *dst = f.in_rank + t0 * R;
        if (f.store_unit == 16) {
            const int upr = R / 16;
            for (int u = tid; u < nbytes / 16; u += kNotifyThreads) {
                const int rw = u / upr, part = u - rw * upr;
                const uint64_t m = s_mask[rw] >> (16 * part);
                uint4 v;
                v.x = spread4((uint32_t)m & 0xfu);
                v.y = spread4((uint32_t)(m >> 4) & 0xfu);
                v.z = spread4((uint32_t)(m >> 8) & 0xfu);
                v.w = spread4((uint32_t)(m >> 12) & 0xfu);
                reinterpret_cast<uint4 *>(dst)[u] = v;
            }
        } else if (f.store_unit == 4) {
            const int upr = R / 4;
            for (int u = tid; u < nbytes / 4; u += kNotifyThreads) {
                const int rw = u / upr, part = u - rw * upr;
                reinterpret_cast<uint32_t *>(dst)[u] = spread4((uint32_t)(s_mask[rw] >> (4 * part)) & 0xfu);
            }
        } else {
            for (int b = tid; b < nbytes; b += kNotifyThreads) {
                const int rw = b / R, r = b - rw * R;
                dst[b] = (uint8_t)((s_mask[rw] >> r) & 1ull);
            }
        }
    }

    // ---- the chunks' offsets inside the group, once all four have counted
    __syncthreads();
    if (counts) {
        const int64_t left = Q - (int64_t)blockIdx.x * kFusedChunks;
        chunk_offsets(p, q, lane, cc, s_grp, wave, (int)(left < kFusedChunks ? left : kFusedChunks));
    }

    // ---- completion: the block that completes the chunks goes on
    if (!single) {
        if (lds_experts)
            for (int e = tid; e < E; e += kNotifyThreads)
                if (s_expert[e] != 0) atomicAdd(&f.acc_expert[e], s_expert[e]);
        if (tid == 0) atomicAdd(&f.report[0], s_slots);
        const int64_t left = Q - (int64_t)blockIdx.x * kFusedChunks;
        const uint32_t mine = (uint32_t)(left < kFusedChunks ? left : kFusedChunks);
        if (!elect_completing_block(f.ticket, epoch0, mine, (uint32_t)Q, p.dev_status)) return;
    } else {
        __syncthreads();
    }
    // The slots the blocks reported and the first per-expert running counts are
    // read now; their values are used only once the finish's loads are in flight
    // (the per-expert totals and their aligned counts, in `mid`) and at the end
    // (the valid-slot check), so all of them share one round trip.  Every block
    // has made its last addition to them before the election, so the elected
    // block reads them (agent-scope loads) and clears them (agent-scope stores)
    // alone.  Every lane makes the loads, at indices clamped into range.
    const bool from_lds = single && lds_experts;
    const uint32_t reported = single ? s_slots : __hip_atomic_load(f.report, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int32_t ev[kExpertBatch];
#pragma unroll
    for (int k = 0; k < kExpertBatch; ++k) {
        const int e = tid + k * kNotifyThreads;
        const int ec = e < E ? e : 0;
        ev[k] = from_lds ? s_expert[ec] : __hip_atomic_load(&f.acc_expert[ec], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    auto mid = [&] {
        auto publish = [&](int e, int32_t v) {
            f.per_expert[e] = v;
            // a count (0 <= v < 2^31) rounded up in 32-bit unsigned arithmetic: the
            // same low 32 bits as in 64-bit
            const uint32_t a = (uint32_t)p.align;
            p.recv_per_expert[e] = (int32_t)(((uint32_t)v + a - 1u) / a * a);
            if (!from_lds) __hip_atomic_store(&f.acc_expert[e], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        };
        uint32_t esum = 0;
#pragma unroll
        for (int k = 0; k < kExpertBatch; ++k) {
            const int e = tid + k * kNotifyThreads;
            if (e < E) {
                publish(e, ev[k]);
                esum += (uint32_t)ev[k];
            }
        }
        for (int e = tid + kExpertBatch * kNotifyThreads; e < E; e += kNotifyThreads) {
            const int32_t v = from_lds ? s_expert[e] : atomicExch(&f.acc_expert[e], 0);
            publish(e, v);
            esum += (uint32_t)v;
        }
        const int w_e = wave_sum((int)esum);
        if (lane == 0) atomicAdd(&s_esum, (uint32_t)w_e);
    };
    const int pg = finish_groups_per_lane(p);
    if (pg == 1)
        finish_by_columns<true, 1>(p, tid, lane, wave, mid);
    else if (pg == kMaxGroupsPerLane)
        finish_by_columns<true, kMaxGroupsPerLane>(p, tid, lane, wave, mid);
    else
        finish_in_global(p, tid, lane, wave, mid);
    // every wave added its expert sum before the finish's first barrier
    if (tid == 0) {
        if (!single) __hip_atomic_store(f.report, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (reported != s_esum) flag(p.dev_status, EP_DEV_STALE_WORKSPACE);
    }
}

}  // namespace

hipError_t launch_layout_notify(const ep_shape_t &s, const int64_t *topk_idx, int32_t *per_rank, int32_t *per_node,
                                int32_t *per_expert, uint8_t *in_rank, int32_t *gbl, int32_t *rdma,
                                int32_t *recv_gbl, int32_t *recv_rdma, int32_t *recv_per_expert, int32_t *num_recv,
                                char *ws, int32_t *dev_status, hipStream_t stream) {
    const Workspace w = workspace_layout(s.num_tokens, s.num_ranks, s.num_experts, s.num_channels, s.num_topk);
    NotifyParams p;
    p.in_rank = in_rank;
    p.per_rank = nullptr;
    p.per_node = nullptr;
    p.per_expert = per_expert;
    p.gbl = gbl;
    p.rdma = rdma;
    p.recv_gbl = recv_gbl;
    p.recv_rdma = recv_rdma;
    p.recv_per_expert = recv_per_expert;
    p.num_recv = num_recv;
    p.mask = reinterpret_cast<uint64_t *>(ws + w.mask);
    p.rank_off = reinterpret_cast<int32_t *>(ws + w.rank_off);
    p.rank_base = reinterpret_cast<int32_t *>(ws + w.rank_base);
    p.node_base = reinterpret_cast<int32_t *>(ws + w.node_base);
    p.rank_part = reinterpret_cast<int32_t *>(ws + w.rank_part);
    p.node_part = reinterpret_cast<int32_t *>(ws + w.node_part);
    p.ticket = nullptr;
    p.dev_status = dev_status;
    p.T = s.num_tokens;
    p.C = s.num_channels;
    p.Tc = (p.T + p.C - 1) / p.C;
    p.R = s.num_ranks;
    p.E = s.num_experts;
    p.nodes = num_nodes(p.R);
    p.align = s.expert_alignment;
    p.load_unit = 1;
    p.fused = true;
    p.tot_rank = per_rank;
    p.tot_node = per_node;
    FusedParams f;
    f.topk_idx = topk_idx;
    f.per_expert = per_expert;
    f.in_rank = in_rank;
    f.acc_expert = reinterpret_cast<int32_t *>(ws + w.acc) + p.R + p.nodes;
    f.ticket = reinterpret_cast<uint64_t *>(reinterpret_cast<uint32_t *>(ws + w.tickets) + kTicketFused);
    f.report = reinterpret_cast<uint32_t *>(ws + w.tickets) + kTicketFused + 2;
    f.K = s.num_topk;
    f.store_unit = 1;
    if (p.R % 16 == 0 && reinterpret_cast<uintptr_t>(in_rank) % 16 == 0)
        f.store_unit = 16;
    else if (p.R % 4 == 0 && reinterpret_cast<uintptr_t>(in_rank) % 4 == 0)
        f.store_unit = 4;
    const int64_t Q = num_chunks(p.T);
    const int64_t blocks = Q > 0 ? (Q + kFusedChunks - 1) / kFusedChunks : 1;
    const size_t lds = p.E <= kFusedMaxLdsExperts ? sizeof(int32_t) * (size_t)p.E : 0;
    static_assert(kMaxTopk == 4 * 8, "KQ = 8 covers every topk");
    const dim3 grid((unsigned)blocks), block(kNotifyThreads);
    if (f.K <= 8) {
        if (blocks == 1)
            hipLaunchKernelGGL((layout_notify_kernel<true, 2>), grid, block, lds, stream, f, p);
        else
            hipLaunchKernelGGL((layout_notify_kernel<false, 2>), grid, block, lds, stream, f, p);
    } else {
        if (blocks == 1)
            hipLaunchKernelGGL((layout_notify_kernel<true, 8>), grid, block, lds, stream, f, p);
        else
            hipLaunchKernelGGL((layout_notify_kernel<false, 8>), grid, block, lds, stream, f, p);
    }
    return hipGetLastError();
}

hipError_t launch_notify(const ep_shape_t &s, const uint8_t *in_rank, const int32_t *per_rank,
                         const int32_t *per_node, const int32_t *per_expert, int32_t *gbl, int32_t *rdma,
                         int32_t *recv_gbl, int32_t *recv_rdma, int32_t *recv_per_expert, int32_t *num_recv,
                         char *ws, int32_t *dev_status, hipStream_t stream) {
    const Workspace w = workspace_layout(s.num_tokens, s.num_ranks, s.num_experts, s.num_channels, s.num_topk);
    NotifyParams p;
    p.in_rank = in_rank;
    p.per_rank = per_rank;
    p.per_node = per_node;
    p.per_expert = per_expert;
    p.gbl = gbl;
    p.rdma = rdma;
    p.recv_gbl = recv_gbl;
    p.recv_rdma = recv_rdma;
    p.recv_per_expert = recv_per_expert;
    p.num_recv = num_recv;
    p.mask = reinterpret_cast<uint64_t *>(ws + w.mask);
    p.rank_off = reinterpret_cast<int32_t *>(ws + w.rank_off);
    p.rank_base = reinterpret_cast<int32_t *>(ws + w.rank_base);
    p.node_base = reinterpret_cast<int32_t *>(ws + w.node_base);
    p.rank_part = reinterpret_cast<int32_t *>(ws + w.rank_part);
    p.node_part = reinterpret_cast<int32_t *>(ws + w.node_part);
    p.ticket = reinterpret_cast<uint64_t *>(reinterpret_cast<uint32_t *>(ws + w.tickets) + kTicketNotify);
    p.dev_status = dev_status;
    p.T = s.num_tokens;
    p.C = s.num_channels;
    p.Tc = (p.T + p.C - 1) / p.C;
    p.R = s.num_ranks;
    p.E = s.num_experts;
    p.nodes = num_nodes(p.R);
    p.align = s.expert_alignment;
    const uintptr_t a = reinterpret_cast<uintptr_t>(in_rank);
    p.load_unit = (p.R % 16 == 0 && a % 16 == 0) ? 16 : (p.R % 8 == 0 && a % 8 == 0) ? 8 : 1;
    p.fused = false;
    p.tot_rank = p.tot_node = nullptr;

    const int64_t Q = num_chunks(p.T);
    // at least one block: the last (only) block also handles t = 0
    const int64_t blocks = Q > 0 ? (Q + kNotifyWaves - 1) / kNotifyWaves : 1;
    hipLaunchKernelGGL(notify_kernel, dim3((unsigned)blocks), dim3(kNotifyThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ep
