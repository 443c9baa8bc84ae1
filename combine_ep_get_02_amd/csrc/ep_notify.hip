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
};

__device__ void count_chunk(const NotifyParams &p, int64_t q, int lane) {
    const int64_t first = q * kChunk;
    const int64_t tok = first + lane;
    const int R = p.R, nodes = p.nodes;
    uint64_t m = 0;
    if (tok < p.T) {
        m = load_rank_mask(p.in_rank + tok * R, R, p.load_unit);
        p.mask[tok] = m;
    }
    const uint64_t my_bits = transpose64(m);  // lane r: which tokens of the chunk go to rank r
    uint64_t my_node_bits = 0;  // lane n: which tokens of the chunk reach node n
    for (int n = 0; n < nodes; ++n) {
        const bool any = R < kRanksPerNode ? m != 0 : ((m >> (n * kRanksPerNode)) & 0xffull) != 0;
        const uint64_t b = ballot64(any);
        my_node_bits = (lane == n) ? b : my_node_bits;
    }
    if (lane < R) p.rank_off[q * R + lane] = __popcll(my_bits);
    if (lane < nodes) p.node_off[q * nodes + lane] = __popcll(my_node_bits);
    // channels whose end lies strictly inside this chunk
    for (int64_t c = first / p.Tc; c < p.C; ++c) {
        const int64_t end = (c + 1) * p.Tc < p.T ? (c + 1) * p.Tc : p.T;
        if (end >= first + kChunk) break;
        if (end <= first) continue;
        const uint64_t below = (1ull << (end - first)) - 1ull;
        if (lane < R) p.rank_part[c * R + lane] = __popcll(my_bits & below);
        if (lane < nodes) p.node_part[c * nodes + lane] = __popcll(my_node_bits & below);
    }
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
// rows of either matrix one thread loads: ceil(kScanLds / NC / (kNotifyThreads / NC)) for any NC <= 72
constexpr int kPasses = 14;
// per-expert counts a thread of the last block loads with the others (E <= 4096 in one go)
constexpr int kExpertBatch = 4;
// columns (ranks + nodes <= 72) a wave scans together: ceil(72 / 16)
constexpr int kColBatch = 5;

__device__ __forceinline__ int64_t channel_end(const NotifyParams &p, int64_t c) {
    return (c + 1) * p.Tc < p.T ? (c + 1) * p.Tc : p.T;
}

// Last block, small problems: the counts, the partials and the per-rank / per-node
// totals come into LDS in one round trip, are scanned there, and every output is
// written from LDS.
__device__ void finish_in_lds(const NotifyParams &p, int tid, int lane, int wave) {
    __shared__ int32_t s_cnt[kScanLds];  // [Q+1][NC], then [C][NC] partials behind it
    __shared__ int32_t s_tot[kMaxRanks + kMaxRanks / kRanksPerNode];
    // everything below fits kScanLds entries, so 32-bit indices suffice
    const int R = p.R, nodes = p.nodes, NC = R + nodes, C = p.C;
    const int Q = (int)num_chunks(p.T);
    int32_t *s_part = s_cnt + (Q + 1) * NC;
    // fixed (row, column) of this thread: rows advance by RP per pass
    const int RP = kNotifyThreads / NC;
    const int r0 = tid / NC, col = tid - r0 * NC;
    const bool active = r0 < RP;
    const bool is_rank = col < R;

    // ---- one round trip of loads: at most kPasses rows per thread for each
    // matrix (rows <= kScanLds / NC, RP = kNotifyThreads / NC), the per-rank,
    // per-node and first per-expert counts, all issued before any is used
    int32_t vq[kPasses], vc[kPasses], pe[kExpertBatch];
    if (active) {
#pragma unroll
        for (int k = 0; k < kPasses; ++k) {
            const int q = r0 + k * RP;
            vq[k] = q < Q ? (is_rank ? p.rank_off[q * R + col] : p.node_off[q * nodes + (col - R)]) : 0;
            const int c = r0 + k * RP;
            vc[k] = (c < C && (channel_end(p, c) % kChunk) != 0)
                        ? (is_rank ? p.rank_part[c * R + col] : p.node_part[c * nodes + (col - R)])
                        : 0;
        }
    }
    const int32_t per_rank = lane < R ? p.per_rank[lane] : 0;
    const int32_t per_node = lane < nodes ? p.per_node[lane] : 0;
#pragma unroll
    for (int k = 0; k < kExpertBatch; ++k) {
        const int e = tid + k * kNotifyThreads;
        pe[k] = e < p.E ? p.per_expert[e] : 0;
    }
    if (active) {
#pragma unroll
        for (int k = 0; k < kPasses; ++k) {
            const int q = r0 + k * RP;
            if (q < Q) s_cnt[q * NC + col] = vq[k];
            const int c = r0 + k * RP;
            if (c < C) s_part[c * NC + col] = vc[k];
        }
        // rows beyond kPasses passes (none within the LDS size limit)
        for (int q = r0 + kPasses * RP; q < Q; q += RP)
            s_cnt[q * NC + col] = is_rank ? p.rank_off[q * R + col] : p.node_off[q * nodes + (col - R)];
        for (int c = r0 + kPasses * RP; c < C; c += RP)
            s_part[c * NC + col] = (channel_end(p, c) % kChunk) != 0
                                       ? (is_rank ? p.rank_part[c * R + col] : p.node_part[c * nodes + (col - R)])
                                       : 0;
    }
    // aligned per-expert counts need nothing from the scan
    auto aligned = [&](int32_t n) { return (int32_t)(((int64_t)n + p.align - 1) / p.align * p.align); };
#pragma unroll
    for (int k = 0; k < kExpertBatch; ++k) {
        const int e = tid + k * kNotifyThreads;
        if (e < p.E) p.recv_per_expert[e] = aligned(pe[k]);
    }
    for (int e = tid + kExpertBatch * kNotifyThreads; e < p.E; e += kNotifyThreads)
        p.recv_per_expert[e] = aligned(p.per_expert[e]);
    __syncthreads();

    // ---- scans: one wave per column, lanes over runs of chunks; a wave's
    // columns (up to kColBatch) are read together so their LDS loads overlap
    const int per = (Q + kWave - 1) / kWave;
    const int b = lane * per;
    const int e = (b + per) < Q ? (b + per) : Q;
    for (int c0 = wave; c0 < NC; c0 += kNotifyWaves * kColBatch) {
        int32_t sum[kColBatch];
#pragma unroll
        for (int k = 0; k < kColBatch; ++k) {
            const int cc = c0 + k * kNotifyWaves;
            sum[k] = 0;
            if (cc < NC)
                for (int q = b; q < e; ++q) sum[k] += s_cnt[q * NC + cc];
        }
#pragma unroll
        for (int k = 0; k < kColBatch; ++k) {
            const int cc = c0 + k * kNotifyWaves;  // the same for the whole wave
            if (cc >= NC) break;
            const int32_t incl = wave_inclusive_scan(sum[k]);
            int32_t run = incl - sum[k];
            for (int q = b; q < e; ++q) {
                const int32_t v = s_cnt[q * NC + cc];
                s_cnt[q * NC + cc] = run;
                run += v;
            }
            const int32_t total = readlane32(incl, kWave - 1);
            if (lane == 0) {
                s_cnt[Q * NC + cc] = total;
                s_tot[cc] = total;
            }
        }
    }
    // receive prefix sums over destination ranks and nodes (inclusive)
    if (wave == kNotifyWaves - 1) {
        const int32_t incl = wave_inclusive_scan(per_rank);
        if (lane < R) p.recv_gbl[lane] = incl;
        if (lane == R - 1) p.num_recv[0] = incl;
    } else if (wave == kNotifyWaves - 2) {
        const int32_t incl = wave_inclusive_scan(per_node);
        if (lane < nodes) p.recv_rdma[lane] = incl;
    }
    __syncthreads();

    // ---- outputs
    if (wave == kNotifyWaves - 3) {
        const bool bad = (lane < R && s_tot[lane] != per_rank) || (lane < nodes && s_tot[R + lane] != per_node);
        if (ballot64(bad) != 0ull && lane == 0) flag(p.dev_status, EP_DEV_COUNT_MISMATCH);
    }
    if (active) {
        for (int q = r0; q <= Q; q += RP) {
            if (is_rank)
                p.rank_off[q * R + col] = s_cnt[q * NC + col];
            else
                p.node_off[q * nodes + (col - R)] = s_cnt[q * NC + col];
        }
        for (int c = r0; c < C; c += RP) {
            const int qe = (int)(channel_end(p, c) / kChunk);
            const int32_t v = s_cnt[qe * NC + col] + s_part[c * NC + col];
            if (is_rank)
                p.gbl[col * C + c] = v;
            else
                p.rdma[(col - R) * C + c] = v;
        }
    }
}

// Last block, large problems: the same steps on the workspace in global memory.
__device__ void finish_in_global(const NotifyParams &p, int tid, int lane, int wave) {
    const int R = p.R, nodes = p.nodes, NC = R + nodes;
    const int64_t Q = num_chunks(p.T);
    for (int col = wave; col < NC; col += kNotifyWaves) {
        const bool is_rank = col < R;
        int32_t *cp = is_rank ? p.rank_off + col : p.node_off + (col - R);
        const int32_t total = scan_column(cp, is_rank ? R : nodes, Q, lane);
        const int32_t want = is_rank ? p.per_rank[col] : p.per_node[col - R];
        if (lane == 0 && total != want) flag(p.dev_status, EP_DEV_COUNT_MISMATCH);
    }
    if (wave == kNotifyWaves - 1) {
        const int32_t v = lane < R ? p.per_rank[lane] : 0;
        const int32_t incl = wave_inclusive_scan(v);
        if (lane < R) p.recv_gbl[lane] = incl;
        if (lane == R - 1) p.num_recv[0] = incl;
    } else if (wave == kNotifyWaves - 2) {
        const int32_t v = lane < nodes ? p.per_node[lane] : 0;
        const int32_t incl = wave_inclusive_scan(v);
        if (lane < nodes) p.recv_rdma[lane] = incl;
    }
    for (int e = tid; e < p.E; e += kNotifyThreads) {
        const int64_t n = p.per_expert[e];
        p.recv_per_expert[e] = (int32_t)((n + p.align - 1) / p.align * p.align);
    }
    __syncthreads();  // scanned offsets visible to the whole block
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
    const int64_t NC = p.R + p.nodes;
    if ((Q + 1) * NC + (int64_t)p.C * NC <= kScanLds)
        finish_in_lds(p, tid, lane, wave);
    else
        finish_in_global(p, tid, lane, wave);
}

}  // namespace

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

    const int64_t Q = num_chunks(p.T);
    // at least one block: the last (only) block also handles t = 0
    const int64_t blocks = Q > 0 ? (Q + kNotifyWaves - 1) / kNotifyWaves : 1;
    hipLaunchKernelGGL(notify_kernel, dim3((unsigned)blocks), dim3(kNotifyThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ep
