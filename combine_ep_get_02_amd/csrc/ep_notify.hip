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
// is cut into 64-token chunks, one chunk per wave and one token per lane.
//   Every wave turns its lanes' is_token_in_rank rows into 64-bit rank masks
//   (stored for dispatch); a 64x64 bit transpose across the wave hands lane r
//   the chunk's column for rank r, whose popcount is the (chunk, rank) count.
//   For each channel whose end falls inside the chunk it also stores the count
//   of the chunk's tokens before that end.  Every value has one writer: no
//   atomics.
//   The last block to finish (the only one, without an election, up to 1024
//   tokens) then scans: it brings the counts, the partials and the per-rank
//   totals into LDS in one round trip (or works in the
//   workspace when they do not fit), one wave per column (rank or node), each
//   lane summing a run of chunks and a wave-wide shuffle scan combining the
//   runs, which turns the counts into exclusive row offsets inside each rank's
//   slab (what dispatch needs).  A channel's prefix is the offset of the chunk
//   holding its end plus the partial count stored for it.  The receive
//   prefixes over ranks and nodes are one wave scan each.
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
    int32_t *rank_off, *node_off, *rank_part, *node_part;
    uint64_t *ticket;  // completion ticket (chunks)
    int32_t *dev_status;
    int64_t T, Tc;
    int R, C, E, nodes, align, load_unit;
    // fused layout + notify: the per-rank / per-node totals are not inputs but come
    // from the scan, and are written to tot_rank / tot_node
    bool fused;
    int32_t *tot_rank, *tot_node;
};

// The chunk's counts from its tokens' rank masks (lane l: token q*64 + l's mask, 0
// past the last token): the masks for dispatch, the (chunk, rank) and (chunk, node)
// counts, and the partial counts at channel ends inside the chunk.
__device__ void count_chunk_masks(const NotifyParams &p, int64_t q, int lane, uint64_t m) {
    const int64_t first = q * kChunk;
    const int64_t tok = first + lane;
    const int R = p.R, nodes = p.nodes;
    if (tok < p.T) p.mask[tok] = m;
    const uint64_t my_bits = transpose64(m);  // lane r: which tokens of the chunk go to rank r
    uint64_t my_node_bits = 0;  // lane n: which tokens of the chunk reach node n
    for (int n = 0; n < nodes; ++n) {
        const bool any = R < kRanksPerNode ? m != 0 : ((m >> (n * kRanksPerNode)) & 0xffull) != 0;
        const uint64_t b = ballot64(any);
        my_node_bits = (lane == n) ? b : my_node_bits;
    }
    if (lane < R) p.rank_off[q * R + lane] = __popcll(my_bits);
    if (lane < nodes) p.node_off[q * nodes + lane] = __popcll(my_node_bits);
    // channels whose end lies strictly inside this chunk (the first channel
    // that can end past `first` from a 32-bit division whenever T allows)
    const int64_t c_first = p.T <= INT32_MAX ? (int64_t)((uint32_t)first / (uint32_t)p.Tc) : first / p.Tc;
    for (int64_t c = c_first; c < p.C; ++c) {
        const int64_t end = (c + 1) * p.Tc < p.T ? (c + 1) * p.Tc : p.T;
        if (end >= first + kChunk) break;
        if (end <= first) continue;
        const uint64_t below = (1ull << (end - first)) - 1ull;
        if (lane < R) p.rank_part[c * R + lane] = __popcll(my_bits & below);
        if (lane < nodes) p.node_part[c * nodes + lane] = __popcll(my_node_bits & below);
    }
}

__device__ void count_chunk(const NotifyParams &p, int64_t q, int lane) {
    const int64_t tok = q * kChunk + lane;
    const uint64_t m = tok < p.T ? load_rank_mask(p.in_rank + tok * p.R, p.R, p.load_unit) : 0ull;
    count_chunk_masks(p, q, lane, m);
}

// One wave scans one column of the [Q][stride] count matrix into exclusive
// offsets, and writes the total into row Q.  Returns the total.
__device__ int32_t scan_column(int32_t *col, int stride, int64_t Q, int lane) {
    const int64_t per = (Q + kWave - 1) / kWave;
    const int64_t b = lane * per;
    const int64_t e = (b + per) < Q ? (b + per) : Q;
    int32_t s = 0;
    for (int64_t row = b; row < e; ++row) s += col[row * stride];
    const int32_t incl = wave_inclusive_scan(s);
    int32_t run = incl - s;
    for (int64_t row = b; row < e; ++row) {
        const int32_t v = col[row * stride];
        col[row * stride] = run;
        run += v;
    }
    const int32_t total = readlane32(incl, kWave - 1);
    if (lane == 0) col[Q * stride] = total;
    return total;
}

// LDS capacity of the last block for the [Q][NC] counts plus the [C][NC]
// partials; larger problems scan in global memory instead.
constexpr int kScanLds = 12288;
// rows of either matrix one thread of the last block holds: within the LDS
// capacity, ceil(Q / (threads / NC)) and ceil(C / (threads / NC)) stay at or
// below 14 for any NC <= 146 (finish_fits_lds checks it all the same)
constexpr int kPasses = 14;
// per-expert counts a thread of the last block loads with the others (E <= 4096 in one go)
constexpr int kExpertBatch = 4;
// columns (ranks + nodes <= 72) a wave scans together: ceil(72 / 16)
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

// Whether the last block finishes in LDS: the [Q + 1][NC] offsets and the
// [C][NC] partials fit, and every thread's share of rows fits its registers.
__device__ __forceinline__ bool finish_fits_lds(const NotifyParams &p) {
    const int64_t NC = p.R + p.nodes, Q = num_chunks(p.T);
    if ((Q + 1) * NC + (int64_t)p.C * NC > kScanLds) return false;
    const int64_t S = kNotifyThreads / NC;
    return (Q + S - 1) / S <= kPasses && ((int64_t)p.C + S - 1) / S <= kPasses && NC <= kColBatch * kNotifyWaves;
}

// Last block, small problems.  Thread (seg, col) of the S = threads / NC
// segments owns rows [seg * L, seg * L + L) of column col of the [Q][NC] count
// matrix (NC = ranks + nodes, L = ceil(Q / S)) and the partial rows seg,
// seg + S, ...: it loads them in one round trip and scans its rows in registers;
// the segment totals are scanned per column in LDS (one wave per column); then
// every thread writes its rows' offsets to the workspace and to LDS, and the
// prefix matrices are read off LDS at the channel ends.  All indices fit 32 bits
// (the LDS bound keeps T below 2^20).
template <bool FUSED, class Mid>
__device__ void finish_in_lds(const NotifyParams &p, int tid, int lane, int wave, Mid mid) {
    __shared__ int32_t s_cnt[kScanLds];        // [Q+1][NC] offsets, then [C][NC] partials behind them
    __shared__ int32_t s_seg[kNotifyThreads];  // [S][NC] segment totals, then their offsets
    __shared__ int32_t s_tot[kMaxRanks + kMaxRanks / kRanksPerNode];
    const int R = p.R, nodes = p.nodes, NC = R + nodes, C = p.C;
    const int T = (int)p.T, Tc = (int)p.Tc;
    const int Q = (T + kChunk - 1) / kChunk;
    int32_t *s_part = s_cnt + (Q + 1) * NC;
    const int S = kNotifyThreads / NC;
    const int L = (Q + S - 1) / S;
    const int seg = tid / NC, col = tid - seg * NC;
    const bool active = seg < S;
    const bool is_rank = col < R;
    const int stride = is_rank ? R : nodes;
    int32_t *off = is_rank ? p.rank_off + col : p.node_off + (col - R);
    const int32_t *part = is_rank ? p.rank_part + col : p.node_part + (col - R);
    const int q0 = seg * L;
    const int rows = active ? (Q - q0 < L ? (Q - q0 > 0 ? Q - q0 : 0) : L) : 0;

    // ---- one round trip of loads, all issued before any is used: the thread's
    // count rows, its partial rows (channels whose end lies inside a chunk; the
    // others have none), and for notify the totals and per-expert counts.  The
    // addresses walk by a fixed step, none computed from a loaded value; loads
    // that only some lanes need are made by all at an index clamped into range,
    // the rest of the lanes dropping the value where it is used (a load under a
    // branch would be waited for where the branch joins).
    int32_t v[kPasses], vp[kPasses], pe[kExpertBatch];
    {
        const int32_t *src = off + (ptrdiff_t)q0 * stride;
        const int32_t *psrc = part + (ptrdiff_t)seg * stride;
        const ptrdiff_t pstep = (ptrdiff_t)S * stride;
#pragma unroll
        for (int k = 0; k < kPasses; ++k) {
            v[k] = k < rows ? *src : 0;
            src += stride;
            const int c = seg + k * S;
            const int end = (c + 1) * Tc < T ? (c + 1) * Tc : T;
            vp[k] = (active && c < C && end % kChunk != 0) ? *psrc : 0;
            psrc += pstep;
        }
    }
    int32_t per_rank = 0, per_node = 0;
    if constexpr (!FUSED) {
        per_rank = p.per_rank[lane < R ? lane : 0];
        per_node = p.per_node[lane < nodes ? lane : 0];
#pragma unroll
        for (int k = 0; k < kExpertBatch; ++k) {
            const int e = tid + k * kNotifyThreads;
            pe[k] = p.per_expert[e < p.E ? e : 0];
        }
    }
    mid();  // the caller's work that waits on its own memory round trip, overlapped with these loads

    // ---- the segment in registers: v[k] becomes row q0 + k's offset inside it
    int32_t run = 0;
#pragma unroll
    for (int k = 0; k < kPasses; ++k) {
        const int32_t x = v[k];
        v[k] = run;
        run += x;
    }
    if (active) s_seg[seg * NC + col] = run;
#pragma unroll
    for (int k = 0; k < kPasses; ++k) {
        const int c = seg + k * S;
        if (active && c < C) s_part[c * NC + col] = vp[k];
    }
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
    __syncthreads();

    // ---- segment offsets, one wave per column (lanes over segments); the
    // column totals go to s_tot
    if (S <= kWave) {
        int32_t x[kColBatch];
#pragma unroll
        for (int k = 0; k < kColBatch; ++k) {
            const int cc = wave + k * kNotifyWaves;
            x[k] = (lane < S && cc < NC) ? s_seg[lane * NC + cc] : 0;
        }
#pragma unroll
        for (int k = 0; k < kColBatch; ++k) {
            const int cc = wave + k * kNotifyWaves;  // the same for the whole wave
            if (cc >= NC) break;
            const int32_t incl = wave_inclusive_scan(x[k]);
            if (lane < S) s_seg[lane * NC + cc] = incl - x[k];
            if (lane == kWave - 1) s_tot[cc] = incl;
        }
    } else {  // NC < 16: up to 8 segments a lane, at most one column a wave
        const int per = (S + kWave - 1) / kWave;
        const int b = lane * per, e = b + per < S ? b + per : S;
        for (int cc = wave; cc < NC; cc += kNotifyWaves) {
            int32_t sum = 0;
            for (int g = b; g < e; ++g) sum += s_seg[g * NC + cc];
            const int32_t incl = wave_inclusive_scan(sum);
            int32_t r2 = incl - sum;
            for (int g = b; g < e; ++g) {
                const int32_t x = s_seg[g * NC + cc];
                s_seg[g * NC + cc] = r2;
                r2 += x;
            }
            if (lane == kWave - 1) s_tot[cc] = incl;
        }
    }
    __syncthreads();

    // ---- every row's offset: to the workspace (dispatch reads it) and to LDS;
    // row Q holds the column totals
    if (active) {
        const int32_t base = s_seg[seg * NC + col];
#pragma unroll
        for (int k = 0; k < kPasses; ++k) {
            if (k < rows) {
                const int32_t o = base + v[k];
                off[(q0 + k) * stride] = o;
                s_cnt[(q0 + k) * NC + col] = o;
            }
        }
        if (seg == 0) {
            off[Q * stride] = s_tot[col];
            s_cnt[Q * NC + col] = s_tot[col];
        }
    }
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
    __syncthreads();

    // ---- the prefix matrices: at channel c's end, the offset of the chunk it
    // ends in plus the chunk's tokens before the end
    if (active) {
        int32_t *dst = is_rank ? p.gbl + col * C : p.rdma + (col - R) * C;
        for (int c = seg; c < C; c += S) {
            const int end = (c + 1) * Tc < T ? (c + 1) * Tc : T;
            dst[c] = s_cnt[(end / kChunk) * NC + col] + s_part[c * NC + col];
        }
    }
}

// Last block, large problems: the same steps on the workspace in global memory.
template <class Mid>
__device__ void finish_in_global(const NotifyParams &p, int tid, int lane, int wave, Mid mid) {
    mid();
    __shared__ int32_t s_tot_g[kMaxRanks + kMaxRanks / kRanksPerNode];
    const int R = p.R, nodes = p.nodes, NC = R + nodes;
    const int64_t Q = num_chunks(p.T);
    for (int col = wave; col < NC; col += kNotifyWaves) {
        const bool is_rank = col < R;
        int32_t *cp = is_rank ? p.rank_off + col : p.node_off + (col - R);
        const int32_t total = scan_column(cp, is_rank ? R : nodes, Q, lane);
        if (p.fused) {
            if (lane == 0) s_tot_g[col] = total;
        } else {
            const int32_t want = is_rank ? p.per_rank[col] : p.per_node[col - R];
            if (lane == 0 && total != want) flag(p.dev_status, EP_DEV_COUNT_MISMATCH);
        }
    }
    if (!p.fused)
        recv_prefixes(p, lane < R ? p.per_rank[lane] : 0, lane < nodes ? p.per_node[lane] : 0, lane, wave);
    if (!p.fused)  // fused, the expert totals' loop writes them
        for (int e = tid; e < p.E; e += kNotifyThreads) {
            const int64_t n = p.per_expert[e];
            p.recv_per_expert[e] = (int32_t)((n + p.align - 1) / p.align * p.align);
        }
    __syncthreads();  // scanned offsets visible to the whole block
    if (p.fused) finish_totals(p, s_tot_g, lane, wave);
    for (int64_t i = tid; i < (int64_t)NC * p.C; i += kNotifyThreads) {
        const int cc = (int)(i / p.C);
        const int64_t c = i % p.C;
        const int64_t end = channel_end(p, c);
        const int64_t qe = end / kChunk;
        const bool inside = (end % kChunk) != 0;
        if (cc < R) {
            p.gbl[cc * (int64_t)p.C + c] = p.rank_off[qe * R + cc] + (inside ? p.rank_part[c * R + cc] : 0);
        } else {
            const int n = cc - R;
            p.rdma[n * (int64_t)p.C + c] = p.node_off[qe * nodes + n] + (inside ? p.node_part[c * nodes + n] : 0);
        }
    }
}

__global__ __launch_bounds__(kNotifyThreads) void notify_kernel(NotifyParams p) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const int64_t Q = num_chunks(p.T);

    const uint32_t epoch0 = (gridDim.x > 1 && tid == 0) ? ticket_epoch(p.ticket) : 0u;
    const int64_t q = (int64_t)blockIdx.x * kNotifyWaves + wave;
    if (q < Q) count_chunk(p, q, lane);

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
    if (finish_fits_lds(p))
        finish_in_lds<false>(p, tid, lane, wave, [] {});
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

__global__ __launch_bounds__(kNotifyThreads) void layout_notify_kernel(FusedParams f, NotifyParams p) {
    __shared__ uint64_t s_mask[kFusedTokens];
    __shared__ uint32_t s_slots, s_esum;
    extern __shared__ int32_t s_expert[];  // E entries when E <= kFusedMaxLdsExperts
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const int R = p.R, E = p.E, K = f.K;
    const bool lds_experts = E <= kFusedMaxLdsExperts;
    const bool single = gridDim.x == 1;
    const uint32_t epoch0 = (!single && tid == 0) ? ticket_epoch(f.ticket) : 0u;
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
        int64_t ev[kMaxTopk / 4];  // all of the lane's loads in flight together
#pragma unroll
        for (int u = 0; u < kMaxTopk / 4; ++u) ev[u] = part + 4 * u < K ? row[part + 4 * u] : -1;
#pragma unroll
        for (int u = 0; u < kMaxTopk / 4; ++u) {
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

    // ---- the block's chunks, one wave each, from the masks in LDS
    if (wave < kFusedChunks) {
        const int64_t q = (int64_t)blockIdx.x * kFusedChunks + wave;
        if (q < Q) count_chunk_masks(p, q, lane, s_mask[wave * kChunk + lane]);
    }

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
            p.recv_per_expert[e] = (int32_t)(((int64_t)v + p.align - 1) / p.align * p.align);
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
    if (finish_fits_lds(p))
        finish_in_lds<true>(p, tid, lane, wave, mid);
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
    p.node_off = reinterpret_cast<int32_t *>(ws + w.node_off);
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
    hipLaunchKernelGGL(layout_notify_kernel, dim3((unsigned)blocks), dim3(kNotifyThreads), lds, stream, f, p);
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
    p.node_off = reinterpret_cast<int32_t *>(ws + w.node_off);
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
