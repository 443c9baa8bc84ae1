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
constexpr int kMaxScales = 1024;      // per-token scales of fp8 rows
constexpr int kChunk = 64;            // tokens per routing chunk (one per lane)

__host__ __device__ inline int num_nodes(int R) { return R / kRanksPerNode > 0 ? R / kRanksPerNode : 1; }
__host__ __device__ inline int64_t num_chunks(int64_t T) { return (T + kChunk - 1) / kChunk; }
// Chunks per offset group: a chunk's row offset inside a rank's slab is its
// group's offset (rank_base) plus its offset inside the group (rank_off).
constexpr int kGroupChunks = 4;
__host__ __device__ inline int64_t num_groups(int64_t T) { return (num_chunks(T) + kGroupChunks - 1) / kGroupChunks; }

// Workspace shared by the four stages.  All offsets 256-byte aligned.
//   tickets   uint32 [64]           completion counters of the multi-block layout and
//                                   notify kernels (work done so far), layout's followed
//                                   by the counts its finished blocks report (checked by
//                                   the last block); zero between calls
//   acc       int32  [R+nodes+E]    layout's running counts; zero between calls
//   mask      uint64 [t]            bit r set when token t goes to rank r (notify -> dispatch)
//   rank_off  int32  [Q][R]         chunk q's row offset inside its group: tokens of
//                                   rank r in the group's chunks before q
//   rank_base int32  [G][R]         group g's token counts, scanned in place into the
//                                   group's row offset inside each rank's slab
//                                   (G = ceil(Q / kGroupChunks)); chunk q starts at
//                                   rank_base[q / 4][r] + rank_off[q][r]
//   node_base int32  [G][nodes]     the same per node
//   rank_part int32  [C][R]         at channel c's end (when it falls in chunk
//                                   q = end / 64 < Q): rank_off[q][r] plus the tokens
//                                   of rank r in [64*q, end)
//   node_part int32  [C][nodes]     the same per node
// The tickets and acc must be zero before the first call; every layout/notify call
// leaves them zero again.
struct Workspace {
    size_t tickets, acc, mask, rank_off, rank_base, node_base, rank_part, node_part, total;
};
// uint32 word offsets of the tickets (each a 64-bit ticket, see elect_completing_block)
constexpr int kTicketLayout = 0;   // counts tokens; words 2..4: valid slots, (token, rank) and (token, node) pairs
constexpr int kTicketNotify = 16;  // counts chunks (a separate 64-byte line)
constexpr int kTicketFused = 32;   // layout + notify in one launch: counts chunks; word 34: valid slots

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

inline Workspace workspace_layout(int64_t T, int R, int E, int C, int K) {
    Workspace w;
    (void)K;  // no part of the layout depends on k
    const int64_t Q = num_chunks(T), G = num_groups(T);
    const int nodes = num_nodes(R);
    size_t off = 0;
    w.tickets = off;   off = align256(off + sizeof(uint32_t) * 64);
    w.acc = off;       off = align256(off + sizeof(int32_t) * (size_t)(R + nodes + E));
    w.mask = off;      off = align256(off + sizeof(uint64_t) * (size_t)(T > 0 ? T : 1));
    w.rank_off = off;  off = align256(off + sizeof(int32_t) * (size_t)(Q > 0 ? Q : 1) * R);
    w.rank_base = off; off = align256(off + sizeof(int32_t) * (size_t)(G > 0 ? G : 1) * R);
    w.node_base = off; off = align256(off + sizeof(int32_t) * (size_t)(G > 0 ? G : 1) * nodes);
    w.rank_part = off; off = align256(off + sizeof(int32_t) * (size_t)C * R);
    w.node_part = off; off = align256(off + sizeof(int32_t) * (size_t)C * nodes);
    w.total = off;
    return w;
}

// ---------------------------------------------------------------- launchers
hipError_t launch_layout(const ep_shape_t &s, const int64_t *topk_idx, int32_t *per_rank, int32_t *per_node,
                         int32_t *per_expert, uint8_t *in_rank, char *ws, int32_t *dev_status, hipStream_t stream);

// The same on the library's static per-GPU scratch, for callers that cannot
// allocate a workspace (experts up to kNoallocMaxExperts).
constexpr int kNoallocMaxExperts = 16384;
hipError_t launch_layout_noalloc(const ep_shape_t &s, const int64_t *topk_idx, int32_t *per_rank, int32_t *per_node,
                                 int32_t *per_expert, uint8_t *in_rank, int32_t *dev_status, hipStream_t stream);

// Layout and notify in one launch (the outputs of both, and notify's workspace state).
hipError_t launch_layout_notify(const ep_shape_t &s, const int64_t *topk_idx, int32_t *per_rank, int32_t *per_node,
                                int32_t *per_expert, uint8_t *in_rank, int32_t *gbl, int32_t *rdma,
                                int32_t *recv_gbl, int32_t *recv_rdma, int32_t *recv_per_expert, int32_t *num_recv,
                                char *ws, int32_t *dev_status, hipStream_t stream);

hipError_t launch_notify(const ep_shape_t &s, const uint8_t *in_rank, const int32_t *per_rank,
                         const int32_t *per_node, const int32_t *per_expert, int32_t *gbl, int32_t *rdma,
                         int32_t *recv_gbl, int32_t *recv_rdma, int32_t *recv_per_expert, int32_t *num_recv,
                         char *ws, int32_t *dev_status, hipStream_t stream);

// Arguments of one dispatch launch.  Rows are row_units 16-byte units (bf16:
// hidden / 8, fp8: hidden / 16); cached_slot non-null selects cached mode.
struct DispatchArgs {
    const void *x;
    int64_t row_units;
    const float *x_scales;  // [t][num_scales], may be null when num_scales == 0
    int num_scales;
    const int64_t *topk_idx;
    const float *topk_w;
    const uint8_t *in_rank;      // [t][R] is_token_in_rank (not cached mode)
    const int32_t *gbl;          // [R][C] channel prefix matrix (not cached mode)
    const int32_t *recv_gbl;
    const char *ws;              // the workspace notify filled, or null: routing worked out from the above
    const int32_t *cached_slot;  // [t][R] rows of an earlier dispatch (cached mode)
    int32_t cap;
    void *recv_x;
    float *recv_scales;
    float *recv_w;
    int64_t *recv_idx;
    int32_t *src_info;
    int32_t *send_slot;
    int32_t *dev_status;
    int form;          // ep_dispatch_form_t: EP_FORM_PUSH keeps the push form
    bool quantize;     // x is bf16 and every row leaves as E4M3 codes with num_scales scales
                       // (push form; row_units counts the 16-byte units of the fp8 row)
    int quant_log2;    // with quantize: log2 of the lanes (16 channels each) per scale group
};

hipError_t launch_dispatch(const ep_shape_t &s, const DispatchArgs &a, hipStream_t stream);
// Longest channel (tokens) for which dispatch works out its routing without a workspace.
constexpr int64_t kMaxDeriveChannelTokens = 4096;

// Arguments of the grouping by local expert (one launch computing positions,
// one copying rows).  Rows are row_units 16-byte units.
struct GroupArgs {
    const void *recv_x;        // [N][row]; or x [t][row] when topk_idx is given
    bool from_x;               // rows straight from x (through topk_idx, send_slot, slot_pos), not recv_x
    const int64_t *topk_idx;   // [t][k] (from_x)
    const int32_t *send_slot;  // [t][R] (from_x)
    int64_t num_tokens;        // t (from_x)
    int64_t row_units;
    const float *recv_scales;  // [N][num_scales] (or x's [t][num_scales]), null when num_scales == 0
    int num_scales;
    const int64_t *recv_idx;   // [N][k] local expert ids
    const float *recv_w;       // [N][k], may be null
    const int32_t *recv_gbl;   // [R] inclusive slab ends
    const int32_t *aligned;    // [E] segment sizes
    int32_t num_rows;          // N
    int32_t cap;               // grouped rows allocated
    void *grouped_x;
    float *grouped_scales;
    int32_t *grouped_row;      // [cap]
    float *grouped_w;          // [cap], may be null
    int32_t *slot_pos;         // [N][k], may be null (not with from_x)
    int32_t *num_grouped;      // [1]
    int32_t *dev_status;
};
constexpr int kMaxGroupExperts = 512;  // local experts per rank the grouping supports

hipError_t launch_group(const ep_shape_t &s, const GroupArgs &a, hipStream_t stream);

// Outputs of the dispatch straight into the grouped layout, pull form (one
// launch: routing, receive metadata, positions, grouped rows and padding).
struct GroupedPullArgs {
    const int32_t *aligned;  // [E] segment sizes
    int32_t cap;             // grouped rows allocated
    void *grouped_x;
    float *grouped_scales;
    int32_t *grouped_row;    // [cap]
    float *grouped_w;        // [cap], may be null
    int32_t *slot_pos;       // [recv capacity][k]
    int32_t *num_grouped;    // [1]
};
// Whether the dispatch straight into the grouped layout takes that form (from 2048
// tokens, rows of 1 KiB to 1 MiB, at most 2048 experts); it needs the workspace.
bool grouped_pull_applies(const ep_shape_t &s, int64_t row_units);
hipError_t launch_dispatch_grouped_pull(const ep_shape_t &s, const DispatchArgs &a, const GroupedPullArgs &g,
                                        hipStream_t stream);

hipError_t launch_combine(const ep_shape_t &s, const uint4 *y, const float *recv_w, const int32_t *send_slot,
                          int32_t num_recv_rows, uint4 *combined_x, float *combined_w, int32_t *dev_status,
                          hipStream_t stream);

// E4M3 quantiser: channels per lane, and log2 of the lanes per scale group for a row of
// `hidden` channels cut into num_scales groups (-1 unless the group is 16 << l channels,
// 0 <= l <= 6).
constexpr int kQuantChannels = 16;
int quant_lanes_log2(int hidden, int num_scales);
hipError_t launch_quantize(const void *x, int64_t rows, int hidden, int num_scales, void *codes, float *scales,
                           hipStream_t stream);
hipError_t launch_dequantize(const void *codes, const float *scales, int64_t rows, int hidden, int num_scales,
                             void *out, hipStream_t stream);

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

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS):
// shifts by 1, 2, 4, 8 inside each row of 16 lanes (lanes whose source falls
// outside the row read 0), then lane 15 of each row is broadcast into the next
// row (rows 1 and 3) and lane 31 into rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
    return v;
}

// Inclusive prefix sum over the wave of non-negative values below 2^41 (sums of
// a few int32 sizes a lane): the low 16 bits and the rest are scanned as two
// 32-bit DPP scans (each sum stays below 2^31 over 64 lanes) and recombined
// exactly.
__device__ __forceinline__ int64_t wave_inclusive_scan64(int64_t v) {
    const int lo = wave_inclusive_scan((int)(v & 0xffff));
    const int hi = wave_inclusive_scan((int)(v >> 16));
    return ((int64_t)hi << 16) + lo;
}

__device__ __forceinline__ int64_t wave_sum64(int64_t v) {
    const int64_t incl = wave_inclusive_scan64(v);
    const uint32_t lo = (uint32_t)readlane32((int)(uint32_t)incl, kWave - 1);
    const uint32_t hi = (uint32_t)readlane32((int)(uint32_t)(incl >> 32), kWave - 1);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Value of v held by lane (lane ^ S), the whole wave active.  Inside a row of 16
// lanes DPP does it: quad permutations for 1 and 2, and for 4 and 8 a mirror
// (lane ^ 7 in each half row, lane ^ 15 in each row) followed by a second
// permutation.  Across rows, gfx950's v_permlane16_swap run on (v, v) leaves
// rows {0, 0, 2, 2} in its first result and rows {1, 1, 3, 3} in its second.
template <int S>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
    if constexpr (S == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xf, 0xf, false);  // quad_perm [1,0,3,2]
    } else if constexpr (S == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xf, 0xf, false);  // quad_perm [2,3,0,1]
    } else if constexpr (S == 4) {
        const int h = __builtin_amdgcn_mov_dpp((int)v, 0x141, 0xf, 0xf, false);  // row_half_mirror: ^ 7
        return (uint32_t)__builtin_amdgcn_mov_dpp(h, 0x1B, 0xf, 0xf, false);    // quad_perm [3,2,1,0]: ^ 3
    } else if constexpr (S == 8) {
        const int m = __builtin_amdgcn_mov_dpp((int)v, 0x140, 0xf, 0xf, false);  // row_mirror: ^ 15
        return (uint32_t)__builtin_amdgcn_mov_dpp(m, 0x141, 0xf, 0xf, false);   // row_half_mirror: ^ 7
    } else {
        static_assert(S == 16, "lane_xor: 1, 2, 4, 8 or 16");
        const auto sw = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (__lane_id() & 16) ? sw[0] : sw[1];
    }
}

// One butterfly step of the transpose below at distance S < 32: each 32-bit half
// trades its S-wide off-diagonal bit fields with the same half of lane ^ S.
template <int S>
__device__ __forceinline__ uint64_t transpose_step(uint64_t x, uint32_t keep) {
    uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
    const uint32_t ylo = lane_xor<S>(lo), yhi = lane_xor<S>(hi);
    if ((__lane_id() & S) == 0) {
        lo = (lo & keep) | ((ylo & keep) << S);
        hi = (hi & keep) | ((yhi & keep) << S);
    } else {
        lo = (lo & ~keep) | ((ylo & ~keep) >> S);
        hi = (hi & ~keep) | ((yhi & ~keep) >> S);
    }
    return ((uint64_t)hi << 32) | lo;
}

// Transpose of the 64x64 bit matrix whose row t is lane t's 64-bit value:
// lane r receives column r, i.e. bit t of the result is bit r of lane t -- the
// same as 64 ballots of "bit r is set", in six butterfly exchange steps (at
// step s, rows t and t^s swap the s-wide off-diagonal sub-blocks).  The step at
// distance 32 is one v_permlane32_swap of (low half, high half): lanes 0..31
// receive the low halves of lanes 32..63 as their new high halves, and lanes
// 32..63 the high halves of lanes 0..31 as their new low halves.  No LDS
// traffic; the whole wave must be active.
__device__ __forceinline__ uint64_t transpose64(uint64_t x) {
    const auto sw = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)(x >> 32), false, false);
    x = ((uint64_t)sw[1] << 32) | sw[0];
    x = transpose_step<16>(x, 0x0000ffffu);
    x = transpose_step<8>(x, 0x00ff00ffu);
    x = transpose_step<4>(x, 0x0f0f0f0fu);
    x = transpose_step<2>(x, 0x33333333u);
    x = transpose_step<1>(x, 0x55555555u);
    return x;
}

__device__ __forceinline__ uint32_t spread4(uint32_t nib) {
    return (nib & 1u) | ((nib & 2u) << 7) | ((nib & 4u) << 14) | ((nib & 8u) << 21);
}

// Nonzero-byte test of four packed bytes -> 4 bits (bit i set when byte i != 0).
__device__ __forceinline__ uint32_t nonzero_bytes4(uint32_t w) {
    uint32_t hi = (((w & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w) & 0x80808080u;
    return ((hi >> 7) & 1u) | ((hi >> 14) & 2u) | ((hi >> 21) & 4u) | ((hi >> 28) & 8u);
}

// Rank mask of one is_token_in_rank row (R <= 64 bytes, any non-zero byte counts
// as 1): bit r set when byte r is non-zero.  load_unit 16 or 8 reads the row in
// aligned 16- or 8-byte pieces (R a multiple of that and the row aligned to it),
// 1 byte by byte.
__device__ __forceinline__ uint64_t load_rank_mask(const uint8_t *row, int R, int load_unit) {
    uint64_t m = 0;
    // fixed-bound unrolled loops so all of a row's loads are in flight together
    if (load_unit == 16) {
        const uint4 *p = reinterpret_cast<const uint4 *>(row);
        uint4 v[kMaxRanks / 16];
#pragma unroll
        for (int g = 0; g < kMaxRanks / 16; ++g)
            if (g < R / 16) v[g] = p[g];
#pragma unroll
        for (int g = 0; g < kMaxRanks / 16; ++g) {
            if (g < R / 16) {
                const uint64_t bits = nonzero_bytes4(v[g].x) | (nonzero_bytes4(v[g].y) << 4) |
                                      (nonzero_bytes4(v[g].z) << 8) | (nonzero_bytes4(v[g].w) << 12);
                m |= bits << (16 * g);
            }
        }
    } else if (load_unit == 8) {
        const uint2 *p = reinterpret_cast<const uint2 *>(row);
        uint2 v[kMaxRanks / 8];
#pragma unroll
        for (int g = 0; g < kMaxRanks / 8; ++g)
            if (g < R / 8) v[g] = p[g];
#pragma unroll
        for (int g = 0; g < kMaxRanks / 8; ++g) {
            if (g < R / 8) {
                const uint64_t bits = nonzero_bytes4(v[g].x) | (nonzero_bytes4(v[g].y) << 4);
                m |= bits << (8 * g);
            }
        }
    } else {
        for (int r = 0; r < R; ++r) m |= (uint64_t)(row[r] != 0) << r;
    }
    return m;
}

__device__ __forceinline__ void flag(int32_t *dev_status, int bits) {
    if (dev_status != nullptr && bits != 0) atomicOr(dev_status, bits);
}

// Sum over the 64 lanes of a wave (wrapping like the uint32 counters it feeds).
__device__ __forceinline__ int wave_sum(int v) { return readlane32(wave_inclusive_scan(v), kWave - 1); }

// Completion ticket of a multi-block kernel: a 64-bit word in the workspace,
// the count of work units done so far in the low half and an epoch in the high
// half.  Every block reads the epoch when it starts (ticket_epoch) and thread 0
// hands it to elect_completing_block once the block's global writes are done.
__device__ __forceinline__ uint32_t ticket_epoch(const uint64_t *ticket) {
    return (uint32_t)(__hip_atomic_load(ticket, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 32);
}

// Every block adds its units of work (`mine`: tokens, chunks) to the ticket
// with a device-scope release; the block that brings the count to `total` is
// elected, sees every other block's writes from then on, and takes the count
// back to zero while moving the epoch on.  In a clean call no block arrives
// after that.  A ticket whose count was not zero on entry (a workspace never
// cleared, or shared by calls running at the same time) shows as a count past
// `total`, or as a block arriving after the election (the epoch moved since it
// started); such a block flags EP_DEV_STALE_WORKSPACE.  (Thread 0 alone holds
// epoch0; total < 2^32.)
__device__ __forceinline__ bool elect_completing_block(uint64_t *ticket, uint32_t epoch0, uint32_t mine,
                                                       uint32_t total, int32_t *dev_status) {
    __shared__ bool last;
    __syncthreads();  // every wave's stores of this block have completed
    if (threadIdx.x == 0) {
        __threadfence();  // one device-scope release for the whole block
        const uint64_t prev = atomicAdd((unsigned long long *)ticket, (unsigned long long)mine);
        const uint64_t count = (uint32_t)prev, done = count + mine;
        const bool same_epoch = (uint32_t)(prev >> 32) == epoch0;
        last = same_epoch && count <= total && done >= total;
        if (!same_epoch || done > total) flag(dev_status, EP_DEV_STALE_WORKSPACE);
        if (last) {
            // count - done (zero unless blocks arrived after this one), epoch + 1
            atomicAdd((unsigned long long *)ticket, (unsigned long long)((1ull << 32) - done));
            __threadfence();  // acquire: other blocks' writes are visible from here on
        }
    }
    __syncthreads();
    return last;
}

// ---------------------------------------------------------------- E4M3 quantiser
// Shared by ep_quantize_fp8 and the dispatch that quantises on the way (one code path,
// so both give the same codes and scales).  A group of 16 << lanes_log2 channels is
// 1 << lanes_log2 aligned lanes, each owning 16 consecutive channels.
//   a = max(largest |x| of the group, 2^-64); scale = a / 448;
//   code = e4m3(clamp(x * (448 / a), -448, 448)), nearest with ties to even
// (v_cvt_pk_fp8_f32 under the default rounding mode; OCP E4M3, bias 7, largest 448).
typedef unsigned int qvec4 __attribute__((ext_vector_type(4)));
constexpr float kE4m3Max = 448.0f;
constexpr float kE4m3AmaxFloor = 0x1p-64f;  // keeps 448 / a finite and the scale a normal number

__device__ __forceinline__ uint32_t e4m3_pack4(float v0, float v1, float v2, float v3) {
    v0 = __builtin_amdgcn_fmed3f(v0, -kE4m3Max, kE4m3Max);
    v1 = __builtin_amdgcn_fmed3f(v1, -kE4m3Max, kE4m3Max);
    v2 = __builtin_amdgcn_fmed3f(v2, -kE4m3Max, kE4m3Max);
    v3 = __builtin_amdgcn_fmed3f(v3, -kE4m3Max, kE4m3Max);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);  // bytes 0, 1
    w = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, w, true);       // bytes 2, 3
    return (uint32_t)w;
}

// Larger magnitude of each half of two bf16 pairs: for finite values the magnitude's bit
// pattern (sign cleared) orders as its value, so one packed 16-bit integer max serves.
__device__ __forceinline__ uint32_t bf16x2_absmax(uint32_t m, uint32_t w) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    const u16x2 a = __builtin_bit_cast(u16x2, w & 0x7fff7fffu), b = __builtin_bit_cast(u16x2, m);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

// lo / hi: the lane's channels 0-7 / 8-15 as bf16 pairs.  Every lane of the wave must
// call this together (the group's maximum is a butterfly of lane shuffles); lanes that own
// no channels pass zeros and form whole groups of their own.
__device__ __forceinline__ qvec4 e4m3_quantize16(qvec4 lo, qvec4 hi, int lanes_log2, float *scale) {
    uint32_t mm = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) mm = bf16x2_absmax(bf16x2_absmax(mm, lo[k]), hi[k]);
    const uint32_t mb = (mm & 0xffffu) > (mm >> 16) ? (mm & 0xffffu) : (mm >> 16);
    float m = __uint_as_float(mb << 16);
    for (int s = 1; s < (1 << lanes_log2); s <<= 1) m = fmaxf(m, __shfl_xor(m, s));
    m = fmaxf(m, kE4m3AmaxFloor);
    const float inv = kE4m3Max / m;
    *scale = m / kE4m3Max;
    qvec4 c;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        c[k] = e4m3_pack4(__uint_as_float(lo[2 * k] << 16) * inv, __uint_as_float(lo[2 * k] & 0xffff0000u) * inv,
                          __uint_as_float(lo[2 * k + 1] << 16) * inv,
                          __uint_as_float(lo[2 * k + 1] & 0xffff0000u) * inv);
        c[2 + k] = e4m3_pack4(__uint_as_float(hi[2 * k] << 16) * inv, __uint_as_float(hi[2 * k] & 0xffff0000u) * inv,
                              __uint_as_float(hi[2 * k + 1] << 16) * inv,
                              __uint_as_float(hi[2 * k + 1] & 0xffff0000u) * inv);
    }
    return c;
}

}  // namespace ep
