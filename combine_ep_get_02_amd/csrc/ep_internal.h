// ep_internal.h -- private to libep.so: workspace layout, kernel launchers and
// the wave64 helpers shared by the four stage kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ep.h"

namespace ep {

constexpr int kWave = 64;             // CDNA wavefront width
constexpr int kRanksPerNode = 8;      // ranks per node (rank -> node is rank / 8)
constexpr int kMaxRanks = 64;         // one rank per lane of a wave
constexpr int kMaxTopk = 32;
constexpr int kMaxChannels = 4096;
constexpr int kChunk = 64;            // tokens per routing chunk (one per lane)

__host__ __device__ inline int num_nodes(int R) { return R / kRanksPerNode > 0 ? R / kRanksPerNode : 1; }
__host__ __device__ inline int64_t num_chunks(int64_t T) { return (T + kChunk - 1) / kChunk; }

// Workspace shared by the four stages.  All offsets 256-byte aligned.
//   tickets   uint32 [64]           completion counters of the multi-block layout and
//                                   notify kernels; zero between calls
//   acc       int32  [R+nodes+E]    layout's running counts; zero between calls
//   mask      uint64 [t]            bit r set when token t goes to rank r (notify -> dispatch)
//   rank_off  int32  [Q+1][R]       per-chunk token counts, scanned in place into
//                                   exclusive offsets inside each rank's slab; row Q
//                                   holds the totals
//   node_off  int32  [Q+1][nodes]   the same per node
//   rank_part int32  [C][R]         tokens of rank r in [64*floor(end_c/64), end_c)
//   node_part int32  [C][nodes]     the same per node
// The tickets and acc must be zero before the first call; every layout/notify call
// leaves them zero again.
struct Workspace {
    size_t tickets, acc, mask, rank_off, node_off, rank_part, node_part, total;
};
constexpr int kTicketLayout = 0;
constexpr int kTicketNotify = 16;  // separate 64-byte lines

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

inline Workspace workspace_layout(int64_t T, int R, int E, int C) {
    Workspace w;
    const int64_t Q = num_chunks(T);
    const int nodes = num_nodes(R);
    size_t off = 0;
    w.tickets = off;   off = align256(off + sizeof(uint32_t) * 64);
    w.acc = off;       off = align256(off + sizeof(int32_t) * (size_t)(R + nodes + E));
    w.mask = off;      off = align256(off + sizeof(uint64_t) * (size_t)(T > 0 ? T : 1));
    w.rank_off = off;  off = align256(off + sizeof(int32_t) * (size_t)(Q + 1) * R);
    w.node_off = off;  off = align256(off + sizeof(int32_t) * (size_t)(Q + 1) * nodes);
    w.rank_part = off; off = align256(off + sizeof(int32_t) * (size_t)C * R);
    w.node_part = off; off = align256(off + sizeof(int32_t) * (size_t)C * nodes);
    w.total = off;
    return w;
}

// ---------------------------------------------------------------- launchers
hipError_t launch_layout(const ep_shape_t &s, const int64_t *topk_idx, int32_t *per_rank, int32_t *per_node,
                         int32_t *per_expert, uint8_t *in_rank, char *ws, int32_t *dev_status, hipStream_t stream);

hipError_t launch_notify(const ep_shape_t &s, const uint8_t *in_rank, const int32_t *per_rank,
                         const int32_t *per_node, const int32_t *per_expert, int32_t *gbl, int32_t *rdma,
                         int32_t *recv_gbl, int32_t *recv_rdma, int32_t *recv_per_expert, int32_t *num_recv,
                         char *ws, int32_t *dev_status, hipStream_t stream);

hipError_t launch_dispatch(const ep_shape_t &s, const uint4 *x, const int64_t *topk_idx, const float *topk_w,
                           const int32_t *recv_gbl, const char *ws, int32_t cap, uint4 *recv_x, float *recv_w,
                           int64_t *recv_idx, int32_t *src_info, int32_t *send_slot, int32_t *dev_status,
                           hipStream_t stream);

hipError_t launch_combine(const ep_shape_t &s, const uint4 *y, const float *recv_w, const int32_t *send_slot,
                          int32_t num_recv_rows, uint4 *combined_x, float *combined_w, int32_t *dev_status,
                          hipStream_t stream);

// ---------------------------------------------------------------- wave64 helpers
__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

// Broadcast lane `src` (wave-uniform) of a 64-bit value to the whole wave.
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int src) {
    uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, src);
    uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), src);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ int readlane32(int v, int src) { return __builtin_amdgcn_readlane(v, src); }

__device__ __forceinline__ float readlanef(float v, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = __lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int u = __shfl_up(v, d, kWave);
        if (lane >= d) v += u;
    }
    return v;
}

// Nonzero-byte test of four packed bytes -> 4 bits (bit i set when byte i != 0).
__device__ __forceinline__ uint32_t nonzero_bytes4(uint32_t w) {
    uint32_t hi = (((w & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w) & 0x80808080u;
    return ((hi >> 7) & 1u) | ((hi >> 14) & 2u) | ((hi >> 21) & 4u) | ((hi >> 28) & 8u);
}

__device__ __forceinline__ void flag(int32_t *dev_status, int bits) {
    if (dev_status != nullptr && bits != 0) atomicOr(dev_status, bits);
}

// Last-block election for a multi-block kernel: every thread has finished its
// global writes; after this returns true in exactly one block (the last to get
// here), that block sees every other block's writes.  The ticket is reset for
// the next call by the elected block.
__device__ __forceinline__ bool elect_last_block(uint32_t *ticket) {
    __shared__ bool last;
    __syncthreads();  // every wave's stores of this block have completed
    if (threadIdx.x == 0) {
        __threadfence();  // one device-scope release for the whole block
        const uint32_t prev = atomicAdd(ticket, 1u);
        last = prev == gridDim.x - 1;
        if (last) {
            atomicExch(ticket, 0u);
            __threadfence();  // acquire: other blocks' writes are visible from here on
        }
    }
    __syncthreads();
    return last;
}

}  // namespace ep
