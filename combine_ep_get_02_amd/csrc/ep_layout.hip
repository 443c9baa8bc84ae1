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
// Design: one launch.  One thread per token builds the token's 64-bit rank
// mask (R <= 64, so rank r is bit r).  Per-rank counts come from a 64x64 bit
// transpose across the wave (lane r gets the column of rank r and counts it),
// per-node counts from wave64 ballots, experts go to an LDS
// histogram, and each block adds its non-zero partial counts into running
// counters in the workspace.  The block's is_token_in_rank rows are staged as
// masks in LDS and written out as one contiguous byte range with 16/4/1-byte
// stores.  The last block to finish moves the running counters into the
// outputs and zeroes them for the next call, so no separate zero-fill launch
// is needed; a single block (up to 256 tokens) writes its LDS counts out
// directly.  Integer atomics commute: the result is deterministic.
// The completion ticket counts tokens, so a ticket that was not zero shows as
// a count past t and is flagged (see elect_completing_block); beside it every
// block reports its valid slots and (token, rank) / (token, node) pairs, and
// the last block checks that each class of running counts adds up to what was
// reported, so running counts that were not zero are flagged as well.
#include <mutex>

#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kLayoutThreads = 256;
constexpr int kMaxLdsExperts = 8192;  // 32 KiB of LDS histogram; larger E counts in the workspace directly

struct LayoutParams {
    const int64_t *topk_idx;
    int32_t *per_rank, *per_node, *per_expert;
    uint8_t *in_rank;
    int32_t *acc;  // [R + nodes + E] running counts, zero between calls
    uint64_t *ticket;      // completion ticket (tokens)
    uint32_t *report;      // valid slots, (token, rank) and (token, node) pairs the finished blocks report
    int32_t *dev_status;
    int64_t T;
    int K, E, R, nodes, store_unit;
};

__global__ __launch_bounds__(kLayoutThreads) void layout_kernel(LayoutParams p) {
    __shared__ int32_t s_rank[kMaxRanks];
    __shared__ int32_t s_node[kMaxRanks / kRanksPerNode];
    __shared__ uint64_t s_mask[kLayoutThreads];
    __shared__ uint32_t s_chk[3];  // the block's valid slots, (token, rank) and (token, node) pairs
    extern __shared__ int32_t s_expert[];  // E entries when E <= kMaxLdsExperts

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int R = p.R, E = p.E, K = p.K, nodes = p.nodes;
    const bool lds_experts = E <= kMaxLdsExperts;
    const bool single = gridDim.x == 1 && lds_experts;  // one block: no ticket, no running counts
    // every lane reads the epoch (thread 0 uses it): a load under a branch would be
    // waited for where the branch joins, before this wave issues its own loads
    const uint32_t epoch0 = ticket_epoch(p.ticket);
    int32_t *acc_rank = p.acc, *acc_node = p.acc + R, *acc_expert = p.acc + R + nodes;
    for (int i = tid; i < R; i += kLayoutThreads) s_rank[i] = 0;
    for (int i = tid; i < nodes; i += kLayoutThreads) s_node[i] = 0;
    if (tid < 3) s_chk[tid] = 0;
    if (lds_experts)
        for (int i = tid; i < E; i += kLayoutThreads) s_expert[i] = 0;
    __syncthreads();

    const int64_t t0 = (int64_t)blockIdx.x * kLayoutThreads;
    const int64_t t = t0 + tid;
    const int experts_per_rank = E / R;
    uint64_t mask = 0;
    int bad = 0, slots = 0;
    if (t < p.T) {
        const int64_t *row = p.topk_idx + t * K;
        // slots in batches of 8: a batch's loads are all in flight before any is used
        for (int j0 = 0; j0 < K; j0 += 8) {
            int64_t ev[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) ev[u] = j0 + u < K ? row[j0 + u] : -1;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t e = ev[u];
                if (e == -1) continue;
                if (e < -1 || e >= E) {
                    bad = 1;
                    continue;
                }
                const int ei = (int)e;
                ++slots;
                if (lds_experts)
                    atomicAdd(&s_expert[ei], 1);
                else
                    atomicAdd(&acc_expert[ei], 1);
                mask |= 1ull << (ei / experts_per_rank);
            }
        }
    }
    s_mask[tid] = mask;

    // lane r of each wave collects the wave's count for rank r: the bit
    // transpose hands lane r the column "token goes to r" of the wave
    const int rank_cnt = __popcll(transpose64(mask));
    if (lane < R && rank_cnt != 0) atomicAdd(&s_rank[lane], rank_cnt);
    int node_cnt = 0;
    for (int n = 0; n < nodes; ++n) {
        const bool any = R < kRanksPerNode ? mask != 0 : ((mask >> (n * kRanksPerNode)) & 0xffull) != 0;
        const int c = __popcll(ballot64(any));
        node_cnt = (lane == n) ? c : node_cnt;
    }
    if (lane < nodes && node_cnt != 0) atomicAdd(&s_node[lane], node_cnt);
    if (ballot64(bad != 0) != 0ull && lane == 0) flag(p.dev_status, EP_DEV_BAD_TOPK_IDX);
    {
        const int w_slots = wave_sum(slots), w_ranks = wave_sum(__popcll(mask));
        const int w_nodes = wave_sum(lane < nodes ? node_cnt : 0);
        if (lane == 0) {
            atomicAdd(&s_chk[0], (uint32_t)w_slots);
            atomicAdd(&s_chk[1], (uint32_t)w_ranks);
            atomicAdd(&s_chk[2], (uint32_t)w_nodes);
        }
    }
    __syncthreads();

    // is_token_in_rank rows of this block: one contiguous range of nt*R bytes
    const int64_t left = p.T - t0;
    const int nt = (int)(left < kLayoutThreads ? (left > 0 ? left : 0) : kLayoutThreads);
    const int nbytes = nt * R;  // <= 256 * 64
    uint8_t *dst = p.in_rank + t0 * R;
    if (p.store_unit == 16) {  // R % 16 == 0, 16-byte aligned
        const int upr = R / 16;  // 16-byte units per row
        for (int u = tid; u < nbytes / 16; u += kLayoutThreads) {
            const int row = u / upr, part = u - row * upr;
            const uint64_t m = s_mask[row] >> (16 * part);
            uint4 v;
            v.x = spread4((uint32_t)m & 0xfu);
            v.y = spread4((uint32_t)(m >> 4) & 0xfu);
            v.z = spread4((uint32_t)(m >> 8) & 0xfu);
            v.w = spread4((uint32_t)(m >> 12) & 0xfu);
            reinterpret_cast<uint4 *>(dst)[u] = v;
        }
    } else if (p.store_unit == 4) {  // R % 4 == 0, 4-byte aligned
        const int upr = R / 4;
        for (int u = tid; u < nbytes / 4; u += kLayoutThreads) {
            const int row = u / upr, part = u - row * upr;
            reinterpret_cast<uint32_t *>(dst)[u] = spread4((uint32_t)(s_mask[row] >> (4 * part)) & 0xfu);
        }
    } else {
        for (int b = tid; b < nbytes; b += kLayoutThreads) {
            const int row = b / R, r = b - row * R;
            dst[b] = (uint8_t)((s_mask[row] >> r) & 1ull);
        }
    }

    if (single) {
        // a single block (t <= 256): its counts are the totals, and the running
        // counters are not touched
        for (int i = tid; i < R; i += kLayoutThreads) p.per_rank[i] = s_rank[i];
        for (int i = tid; i < nodes; i += kLayoutThreads) p.per_node[i] = s_node[i];
        for (int i = tid; i < E; i += kLayoutThreads) p.per_expert[i] = s_expert[i];
        return;
    }

    // this block's partial counts into the running counters
    for (int i = tid; i < R; i += kLayoutThreads)
        if (s_rank[i] != 0) atomicAdd(&acc_rank[i], s_rank[i]);
    for (int i = tid; i < nodes; i += kLayoutThreads)
        if (s_node[i] != 0) atomicAdd(&acc_node[i], s_node[i]);
    if (lds_experts)
        for (int i = tid; i < E; i += kLayoutThreads)
            if (s_expert[i] != 0) atomicAdd(&acc_expert[i], s_expert[i]);
    // what this block reports beside its ticket (ordered before it by the election's fence)
    if (tid == 0) {
        atomicAdd(&p.report[0], s_chk[0]);
        atomicAdd(&p.report[1], s_chk[1]);
        atomicAdd(&p.report[2], s_chk[2]);
    }

    if (!elect_completing_block(p.ticket, epoch0, (uint32_t)nt, (uint32_t)p.T, p.dev_status)) return;
    // last block: publish the totals and leave the counters at zero, four
    // counters per thread in flight at a time; each class of counts is summed
    // for the check against the blocks' reports
    __shared__ uint32_t s_sum[3];
    if (tid < 3) s_sum[tid] = 0;
    const int n = R + nodes + E;
    uint32_t sum_e = 0, sum_r = 0, sum_n = 0;
    for (int i0 = tid; i0 < n; i0 += 4 * kLayoutThreads) {
        int32_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * kLayoutThreads;
            v[u] = i < n ? atomicExch(&p.acc[i], 0) : 0;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * kLayoutThreads;
            if (i >= n) continue;
            if (i < R) {
                p.per_rank[i] = v[u];
                sum_r += (uint32_t)v[u];
            } else if (i < R + nodes) {
                p.per_node[i - R] = v[u];
                sum_n += (uint32_t)v[u];
            } else {
                p.per_expert[i - R - nodes] = v[u];
                sum_e += (uint32_t)v[u];
            }
        }
    }
    const int w_e = wave_sum((int)sum_e), w_r = wave_sum((int)sum_r), w_n = wave_sum((int)sum_n);
    __syncthreads();  // s_sum cleared before any wave adds to it
    if (lane == 0) {
        atomicAdd(&s_sum[0], (uint32_t)w_e);
        atomicAdd(&s_sum[1], (uint32_t)w_r);
        atomicAdd(&s_sum[2], (uint32_t)w_n);
    }
    __syncthreads();
    if (tid == 0) {
        const uint32_t slots_all = atomicExch(&p.report[0], 0u), ranks_all = atomicExch(&p.report[1], 0u);
        const uint32_t nodes_all = atomicExch(&p.report[2], 0u);
        if (slots_all != s_sum[0] || ranks_all != s_sum[1] || nodes_all != s_sum[2])
            flag(p.dev_status, EP_DEV_STALE_WORKSPACE);
    }
}

// Zeroes n words (the scratch of the allocation-free layout, before each call).
__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t *p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// The allocation-free layout's scratch: the layout part of a workspace (the
// tickets, then the running counts from byte 256) in a static device array, so
// the call needs no workspace.  Each GPU holds its own copy, at its own
// address, until the process ends; calls on one GPU share it.
constexpr size_t kScratchBytes =
    256 + sizeof(int32_t) * (size_t)(kMaxRanks + kMaxRanks / kRanksPerNode + kNoallocMaxExperts);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of this GPU's scratch, looked up once per device (with that
// device current) and kept; the array's name in host code is not that address.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(int device, void **out) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[device] == nullptr) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[device] = ptr;
    }
    *out = g_scratch_ptr[device];
    return hipSuccess;
}

}  // namespace

hipError_t launch_layout_noalloc(const ep_shape_t &s, const int64_t *topk_idx, int32_t *per_rank, int32_t *per_node,
                                 int32_t *per_expert, uint8_t *in_rank, int32_t *dev_status, hipStream_t stream) {
    int device = -1;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return e;
    void *ptr = nullptr;
    e = scratch_address(device, &ptr);
    if (e != hipSuccess) return e;
    // the tickets and the running counts must start at zero: cleared by a kernel
    // (not a memset, so the call can be captured in a graph)
    const Workspace w = workspace_layout(s.num_tokens, s.num_ranks, s.num_experts, s.num_channels, s.num_topk);
    const int words = (int)((w.acc + sizeof(int32_t) * (size_t)(s.num_ranks + num_nodes(s.num_ranks) +
                                                               s.num_experts)) / sizeof(uint32_t));
    hipLaunchKernelGGL(clear_words_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                       static_cast<uint32_t *>(ptr), words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_layout(s, topk_idx, per_rank, per_node, per_expert, in_rank, static_cast<char *>(ptr), dev_status,
                         stream);
}

hipError_t launch_layout(const ep_shape_t &s, const int64_t *topk_idx, int32_t *per_rank, int32_t *per_node,
                         int32_t *per_expert, uint8_t *in_rank, char *ws, int32_t *dev_status, hipStream_t stream) {
    const Workspace w = workspace_layout(s.num_tokens, s.num_ranks, s.num_experts, s.num_channels, s.num_topk);
    LayoutParams p;
    p.topk_idx = topk_idx;
    p.per_rank = per_rank;
    p.per_node = per_node;
    p.per_expert = per_expert;
    p.in_rank = in_rank;
    p.acc = reinterpret_cast<int32_t *>(ws + w.acc);
    p.ticket = reinterpret_cast<uint64_t *>(reinterpret_cast<uint32_t *>(ws + w.tickets) + kTicketLayout);
    p.report = reinterpret_cast<uint32_t *>(ws + w.tickets) + kTicketLayout + 2;
    p.dev_status = dev_status;
    p.T = s.num_tokens;
    p.K = s.num_topk;
    p.E = s.num_experts;
    p.R = s.num_ranks;
    p.nodes = num_nodes(p.R);
    p.store_unit = 1;
    if (p.R % 16 == 0 && reinterpret_cast<uintptr_t>(in_rank) % 16 == 0)
        p.store_unit = 16;
    else if (p.R % 4 == 0 && reinterpret_cast<uintptr_t>(in_rank) % 4 == 0)
        p.store_unit = 4;
    const size_t lds = p.E <= kMaxLdsExperts ? sizeof(int32_t) * (size_t)p.E : 0;
    // one block even for t = 0: the last (only) block publishes the zero counts
    const int64_t blocks = p.T > 0 ? (p.T + kLayoutThreads - 1) / kLayoutThreads : 1;
    hipLaunchKernelGGL(layout_kernel, dim3((unsigned)blocks), dim3(kLayoutThreads), lds, stream, p);
    return hipGetLastError();
}

}  // namespace ep
