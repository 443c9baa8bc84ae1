// ep_layout.hip -- stage 1, dispatch layout (gfx950).
//
// Computes, from topk_idx [t][k] (int64, -1 = masked), the token counts per
// destination rank, per node (rank / 8) and per expert, and the
// is_token_in_rank map.  Definitions: mscclpp ht_runtime.cc mirror,
// getDispatchLayout (inputs and outputs; the kernel body is not on the pages);
// the per-node rule -- a token counts for a node when any of the node's 8
// ranks receives it -- follows the internode.cu notes, notify_dispatch sm1-x
// stage 1, which tests a node's 8 bytes of is_token_in_rank at once.
//
// Design: one thread per token builds the token's 64-bit rank mask (R <= 64,
// so rank r is bit r).  Per-rank and per-node counts come from wave64 ballots
// (lane r keeps the popcount for rank r), experts go to an LDS histogram, and
// each block adds its partial counts to the outputs with one atomic per
// non-zero entry.  Integer atomics commute, so the result is deterministic.
// The block's is_token_in_rank rows are staged as masks in LDS and written
// out as a contiguous byte range with 16/4/1-byte stores.
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kLayoutThreads = 256;
constexpr int kMaxLdsExperts = 8192;  // 32 KiB of LDS histogram; larger E counts in global memory

__global__ void layout_zero_kernel(int32_t *per_rank, int R, int32_t *per_node, int nodes, int32_t *per_expert,
                                   int E) {
    const int n = R + nodes + E;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += blockDim.x * gridDim.x) {
        if (i < R)
            per_rank[i] = 0;
        else if (i < R + nodes)
            per_node[i - R] = 0;
        else
            per_expert[i - R - nodes] = 0;
    }
}

// byte i of the result = bit i of the low 4 bits of `nib`
__device__ __forceinline__ uint32_t spread4(uint32_t nib) {
    return (nib & 1u) | ((nib & 2u) << 7) | ((nib & 4u) << 14) | ((nib & 8u) << 21);
}

__global__ __launch_bounds__(kLayoutThreads) void layout_kernel(const int64_t *__restrict__ topk_idx, int T, int K,
                                                                int E, int R, int nodes, int store_unit,
                                                                int32_t *__restrict__ per_rank,
                                                                int32_t *__restrict__ per_node,
                                                                int32_t *__restrict__ per_expert,
                                                                uint8_t *__restrict__ in_rank,
                                                                int32_t *__restrict__ dev_status) {
    __shared__ int32_t s_rank[kMaxRanks];
    __shared__ int32_t s_node[kMaxRanks / kRanksPerNode];
    __shared__ uint64_t s_mask[kLayoutThreads];
    extern __shared__ int32_t s_expert[];  // E entries when E <= kMaxLdsExperts

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const bool lds_experts = E <= kMaxLdsExperts;
    for (int i = tid; i < R; i += kLayoutThreads) s_rank[i] = 0;
    for (int i = tid; i < nodes; i += kLayoutThreads) s_node[i] = 0;
    if (lds_experts)
        for (int i = tid; i < E; i += kLayoutThreads) s_expert[i] = 0;
    __syncthreads();

    const int64_t t0 = (int64_t)blockIdx.x * kLayoutThreads;
    const int64_t t = t0 + tid;
    const int experts_per_rank = E / R;
    uint64_t mask = 0;
    int bad = 0;
    if (t < T) {
        const int64_t *row = topk_idx + t * K;
        for (int j = 0; j < K; ++j) {
            const int64_t e = row[j];
            if (e == -1) continue;
            if (e < -1 || e >= E) {
                bad = 1;
                continue;
            }
            const int ei = (int)e;
            if (lds_experts)
                atomicAdd(&s_expert[ei], 1);
            else
                atomicAdd(&per_expert[ei], 1);
            mask |= 1ull << (ei / experts_per_rank);
        }
    }
    s_mask[tid] = mask;

    // lane r of each wave collects the wave's count for rank r
    int rank_cnt = 0;
    for (int r = 0; r < R; ++r) {
        const int c = __popcll(ballot64((mask >> r) & 1ull));
        rank_cnt = (lane == r) ? c : rank_cnt;
    }
    if (lane < R && rank_cnt != 0) atomicAdd(&s_rank[lane], rank_cnt);
    int node_cnt = 0;
    for (int n = 0; n < nodes; ++n) {
        const bool any = R < kRanksPerNode ? mask != 0 : ((mask >> (n * kRanksPerNode)) & 0xffull) != 0;
        const int c = __popcll(ballot64(any));
        node_cnt = (lane == n) ? c : node_cnt;
    }
    if (lane < nodes && node_cnt != 0) atomicAdd(&s_node[lane], node_cnt);
    if (ballot64(bad != 0) != 0 && lane == 0) flag(dev_status, EP_DEV_BAD_TOPK_IDX);
    __syncthreads();

    // is_token_in_rank rows of this block: one contiguous range of nt*R bytes
    const int nt = (int)((T - t0) < kLayoutThreads ? (T - t0) : kLayoutThreads);
    const int64_t nbytes = (int64_t)nt * R;
    uint8_t *dst = in_rank + t0 * R;
    if (store_unit == 16) {  // R % 16 == 0, 16-byte aligned
        for (int64_t u = tid; u < nbytes / 16; u += kLayoutThreads) {
            const int64_t b = u * 16;
            const uint64_t m = s_mask[b / R] >> (b % R);
            uint4 v;
            v.x = spread4((uint32_t)m & 0xfu);
            v.y = spread4((uint32_t)(m >> 4) & 0xfu);
            v.z = spread4((uint32_t)(m >> 8) & 0xfu);
            v.w = spread4((uint32_t)(m >> 12) & 0xfu);
            reinterpret_cast<uint4 *>(dst)[u] = v;
        }
    } else if (store_unit == 4) {  // R % 4 == 0, 4-byte aligned
        for (int64_t u = tid; u < nbytes / 4; u += kLayoutThreads) {
            const int64_t b = u * 4;
            reinterpret_cast<uint32_t *>(dst)[u] = spread4((uint32_t)(s_mask[b / R] >> (b % R)) & 0xfu);
        }
    } else {
        for (int64_t b = tid; b < nbytes; b += kLayoutThreads)
            dst[b] = (uint8_t)((s_mask[b / R] >> (b % R)) & 1ull);
    }

    for (int i = tid; i < R; i += kLayoutThreads)
        if (s_rank[i] != 0) atomicAdd(&per_rank[i], s_rank[i]);
    for (int i = tid; i < nodes; i += kLayoutThreads)
        if (s_node[i] != 0) atomicAdd(&per_node[i], s_node[i]);
    if (lds_experts)
        for (int i = tid; i < E; i += kLayoutThreads)
            if (s_expert[i] != 0) atomicAdd(&per_expert[i], s_expert[i]);
}

}  // namespace

hipError_t launch_layout(const ep_shape_t &s, const int64_t *topk_idx, int32_t *per_rank, int32_t *per_node,
                         int32_t *per_expert, uint8_t *in_rank, int32_t *dev_status, hipStream_t stream) {
    const int R = s.num_ranks, E = s.num_experts, nodes = num_nodes(R);
    const int64_t T = s.num_tokens;
    const int nzero = R + nodes + E;
    const int zblocks = (nzero + 255) / 256 < 64 ? (nzero + 255) / 256 : 64;
    hipLaunchKernelGGL(layout_zero_kernel, dim3(zblocks), dim3(256), 0, stream, per_rank, R, per_node, nodes,
                       per_expert, E);
    if (T > 0) {
        int unit = 1;
        if (R % 16 == 0 && reinterpret_cast<uintptr_t>(in_rank) % 16 == 0)
            unit = 16;
        else if (R % 4 == 0 && reinterpret_cast<uintptr_t>(in_rank) % 4 == 0)
            unit = 4;
        const size_t lds = E <= kMaxLdsExperts ? sizeof(int32_t) * (size_t)E : 0;
        const int64_t blocks = (T + kLayoutThreads - 1) / kLayoutThreads;
        hipLaunchKernelGGL(layout_kernel, dim3((unsigned)blocks), dim3(kLayoutThreads), lds, stream, topk_idx,
                           (int)T, s.num_topk, E, R, nodes, unit, per_rank, per_node, per_expert, in_rank,
                           dev_status);
    }
    return hipGetLastError();
}

}  // namespace ep
