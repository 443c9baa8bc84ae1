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
// Design (not the pages' one-SM-per-channel loop): the token axis is cut into
// 64-token chunks, one chunk per wave and one token per lane.
//   count kernel (grid over chunks): lane j turns its token's is_token_in_rank
//     row into a 64-bit rank mask, stores it for dispatch, and R ballots give
//     every (chunk, rank) count (lane r keeps rank r's ballot).  For each channel
//     whose end falls inside the chunk it also stores the count of the chunk's
//     tokens before that end.  Every value has one writer: no atomics.
//   scan kernel (one workgroup): an LDS-staged two-level scan over the chunks
//     turns the counts into exclusive row offsets inside each rank's slab (what
//     dispatch needs); a channel's prefix is then the offset of the chunk holding
//     its end plus the partial count stored for it.  The receive prefixes over
//     ranks and nodes, the aligned expert counts and N follow.
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kCountWaves = 4;
constexpr int kScanThreads = 1024;

struct NotifyParams {
    const uint8_t *in_rank;
    const int32_t *per_rank, *per_node, *per_expert;
    int32_t *gbl, *rdma, *recv_gbl, *recv_rdma, *recv_per_expert, *num_recv;
    uint64_t *mask;
    int32_t *rank_off, *node_off, *rank_part, *node_part;
    int32_t *dev_status;
    int64_t T, Tc;
    int R, C, E, nodes, align, load_unit;
};

__device__ __forceinline__ uint64_t load_rank_mask(const uint8_t *row, int R, int load_unit) {
    uint64_t m = 0;
    if (load_unit == 16) {
        const uint4 *p = reinterpret_cast<const uint4 *>(row);
        for (int g = 0; g < R / 16; ++g) {
            const uint4 v = p[g];
            const uint64_t bits = nonzero_bytes4(v.x) | (nonzero_bytes4(v.y) << 4) | (nonzero_bytes4(v.z) << 8) |
                                  (nonzero_bytes4(v.w) << 12);
            m |= bits << (16 * g);
        }
    } else if (load_unit == 8) {
        const uint2 *p = reinterpret_cast<const uint2 *>(row);
        for (int g = 0; g < R / 8; ++g) {
            const uint2 v = p[g];
            const uint64_t bits = nonzero_bytes4(v.x) | (nonzero_bytes4(v.y) << 4);
            m |= bits << (8 * g);
        }
    } else {
        for (int r = 0; r < R; ++r) m |= (uint64_t)(row[r] != 0) << r;
    }
    return m;
}

__global__ __launch_bounds__(kCountWaves *kWave) void notify_count_kernel(NotifyParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t q = (int64_t)blockIdx.x * kCountWaves + (threadIdx.x >> 6);
    const int64_t Q = num_chunks(p.T);
    if (q >= Q) return;  // whole wave leaves together
    const int64_t first = q * kChunk;
    const int64_t tok = first + lane;
    const int R = p.R, nodes = p.nodes;

    uint64_t m = 0;
    if (tok < p.T) {
        m = load_rank_mask(p.in_rank + tok * R, R, p.load_unit);
        p.mask[tok] = m;
    }
    uint64_t my_bits = 0;  // lane r: which tokens of the chunk go to rank r
    for (int r = 0; r < R; ++r) {
        const uint64_t b = ballot64((m >> r) & 1ull);
        my_bits = (lane == r) ? b : my_bits;
    }
    uint64_t my_node_bits = 0;  // lane n: which tokens of the chunk reach node n
    for (int n = 0; n < nodes; ++n) {
        const bool any = R < kRanksPerNode ? m != 0 : ((m >> (n * kRanksPerNode)) & 0xffull) != 0;
        const uint64_t b = ballot64(any);
        my_node_bits = (lane == n) ? b : my_node_bits;
    }
    if (lane < R) p.rank_off[q * R + lane] = __popcll(my_bits);
    if (lane < nodes) p.node_off[q * nodes + lane] = __popcll(my_node_bits);

    // channels whose end lies strictly inside this chunk
    if (p.Tc > 0) {
        for (int64_t c = first / p.Tc; c < p.C; ++c) {
            const int64_t end = (c + 1) * p.Tc < p.T ? (c + 1) * p.Tc : p.T;
            if (end >= first + kChunk) break;
            if (end <= first) continue;
            const uint64_t below = (1ull << (end - first)) - 1ull;
            if (lane < R) p.rank_part[c * R + lane] = __popcll(my_bits & below);
            if (lane < nodes) p.node_part[c * nodes + lane] = __popcll(my_node_bits & below);
        }
    }
}

__global__ __launch_bounds__(kScanThreads) void notify_scan_kernel(NotifyParams p) {
    __shared__ int32_t part[kScanThreads];
    const int tid = threadIdx.x;
    const int R = p.R, nodes = p.nodes, NC = R + nodes;
    const int64_t Q = num_chunks(p.T);
    const int G = kScanThreads / NC;
    const int64_t per = (Q + G - 1) / G;
    const int g = tid / NC, col = tid % NC;
    int32_t *colp = col < R ? p.rank_off + col : p.node_off + (col - R);
    const int stride = col < R ? R : nodes;

    // pass 1: each group sums its run of chunks for its column
    if (g < G) {
        int32_t s = 0;
        const int64_t b = g * per, e = (b + per) < Q ? (b + per) : Q;
        for (int64_t row = b; row < e; ++row) s += colp[row * stride];
        part[g * NC + col] = s;
    }
    __syncthreads();
    // pass 2: exclusive scan over groups, one thread per column; row Q = total
    if (tid < NC) {
        int32_t run = 0;
        for (int gg = 0; gg < G; ++gg) {
            const int32_t v = part[gg * NC + tid];
            part[gg * NC + tid] = run;
            run += v;
        }
        int32_t *cp = tid < R ? p.rank_off + tid : p.node_off + (tid - R);
        cp[Q * (tid < R ? R : nodes)] = run;
        const int32_t want = tid < R ? p.per_rank[tid] : p.per_node[tid - R];
        if (run != want) flag(p.dev_status, EP_DEV_COUNT_MISMATCH);
    }
    __syncthreads();
    // pass 3: rewrite each group's run as exclusive offsets
    if (g < G) {
        int32_t run = part[g * NC + col];
        const int64_t b = g * per, e = (b + per) < Q ? (b + per) : Q;
        for (int64_t row = b; row < e; ++row) {
            const int32_t v = colp[row * stride];
            colp[row * stride] = run;
            run += v;
        }
    }
    __syncthreads();

    // channel prefix matrices: offset of the chunk holding the channel's end
    // plus the partial count inside that chunk
    for (int64_t i = tid; i < (int64_t)NC * p.C; i += kScanThreads) {
        const int cc = (int)(i / p.C);
        const int64_t c = i % p.C;
        const int64_t end = (c + 1) * p.Tc < p.T ? (c + 1) * p.Tc : p.T;
        const int64_t qe = end / kChunk;
        const bool inside = (end % kChunk) != 0;
        if (cc < R) {
            p.gbl[cc * (int64_t)p.C + c] = p.rank_off[qe * R + cc] + (inside ? p.rank_part[c * R + cc] : 0);
        } else {
            const int n = cc - R;
            p.rdma[n * (int64_t)p.C + c] = p.node_off[qe * nodes + n] + (inside ? p.node_part[c * nodes + n] : 0);
        }
    }
    // receive prefix sums over destination ranks / nodes (inclusive)
    if (tid == 0) {
        int32_t run = 0;
        for (int r = 0; r < R; ++r) {
            run += p.per_rank[r];
            p.recv_gbl[r] = run;
        }
        p.num_recv[0] = run;
    } else if (tid == kWave) {
        int32_t run = 0;
        for (int n = 0; n < nodes; ++n) {
            run += p.per_node[n];
            p.recv_rdma[n] = run;
        }
    }
    for (int e = tid; e < p.E; e += kScanThreads) {
        const int64_t n = p.per_expert[e];
        p.recv_per_expert[e] = (int32_t)((n + p.align - 1) / p.align * p.align);
    }
}

}  // namespace

hipError_t launch_notify(const ep_shape_t &s, const uint8_t *in_rank, const int32_t *per_rank,
                         const int32_t *per_node, const int32_t *per_expert, int32_t *gbl, int32_t *rdma,
                         int32_t *recv_gbl, int32_t *recv_rdma, int32_t *recv_per_expert, int32_t *num_recv,
                         char *ws, int32_t *dev_status, hipStream_t stream) {
    const Workspace w = workspace_layout(s.num_tokens, s.num_ranks, s.num_channels);
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
    if (Q > 0) {
        const int64_t blocks = (Q + kCountWaves - 1) / kCountWaves;
        hipLaunchKernelGGL(notify_count_kernel, dim3((unsigned)blocks), dim3(kCountWaves * kWave), 0, stream, p);
    }
    hipLaunchKernelGGL(notify_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ep
