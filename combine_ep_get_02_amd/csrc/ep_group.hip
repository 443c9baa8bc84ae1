// ep_group.hip -- grouping of the receive rows by local expert (gfx950).
//
// Definitions: the pages give only the sizes of the groups -- per local
// expert, the received slot count rounded up to expert_alignment (DeepEP
// internode.cu notes, notify_dispatch sm0 stage 6; mscclpp ht_runtime.cc
// mirror, internodeNotifyDispatch hands them back per local expert).  The
// layout is this library's reading: segment e = r*(E/R) + le (receive slab r,
// local expert le) starts at the sum of the sizes of the segments before it
// and holds one entry per (row, slot) of slab r whose local id is le, rows
// ascending, then slots; the rest of the segment is padding (zero row, row
// -1, weight 0).
//
// Design: two launches.
//  positions: one 1024-thread block per slab walks it in groups of 16 tiles
//   of 64 rows, one tile per wave, one row per lane.  A wave enumerates the
//   distinct local ids present in its tile (the lowest lane still holding an
//   unplaced slot names the next id); for each id a DPP wave scan of the
//   lanes' slot counts ranks every slot inside the tile, stably in (row, slot)
//   order.  The tiles' totals are scanned across the 16 waves in LDS and added
//   to running per-id counts, and a second pass over the same ids writes each
//   slot's position, the grouped row index and the weight.  Padding positions
//   are marked last.
//  copy: one wave per grouped row copies the receive row it names (zeros for
//   padding) with 16-byte non-temporal loads and stores; the grouped rows are
//   written in order, as one contiguous stream.
#include "ep_internal.h"

namespace ep {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGroupWaves = 16;
constexpr int kGroupThreads = kGroupWaves * kWave;

struct PositionParams {
    const int64_t *recv_idx;
    const float *recv_w;
    const int32_t *recv_gbl;
    const int32_t *aligned;
    int32_t *grouped_row;
    float *grouped_w;
    int32_t *slot_pos;
    int32_t *num_grouped;
    int32_t *dev_status;
    int64_t num_rows, cap;
    int R, K, er;
};

__device__ __forceinline__ int64_t wave_inclusive_scan64(int64_t v) {
    const int lane = __lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int64_t o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    return v;
}

// Key of the lowest set slot of `pending` (the slot order is the entry order).
__device__ __forceinline__ int lowest_key(const int (&key)[kMaxTopk], uint32_t pending) {
    int first = -1;
#pragma unroll
    for (int j = kMaxTopk - 1; j >= 0; --j)
        if ((pending >> j) & 1u) first = key[j];
    return first;
}

__device__ __forceinline__ uint32_t slots_with_key(const int (&key)[kMaxTopk], uint32_t pending, int id) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j)
        if (((pending >> j) & 1u) && key[j] == id) m |= 1u << j;
    return m;
}

__global__ __launch_bounds__(kGroupThreads) void group_positions_kernel(PositionParams p) {
    // dynamic LDS: int64 s_off[er] | int32 s_size[er] | int32 s_run[er] | int32 s_tile[16][er]
    extern __shared__ int64_t s_dyn[];
    __shared__ unsigned long long s_base;
    __shared__ int64_t s_wsum[kGroupWaves];
    const int er = p.er, K = p.K;
    int64_t *s_off = s_dyn;
    int32_t *s_size = reinterpret_cast<int32_t *>(s_off + er);
    int32_t *s_run = s_size + er;
    int32_t *s_tile = s_run + er;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const int r = blockIdx.x;

    // ---- where this slab's first segment starts: the sizes of all earlier slabs' segments
    if (tid == 0) s_base = 0;
    __syncthreads();
    int64_t part = 0;
    for (int64_t e = tid; e < (int64_t)r * er; e += kGroupThreads) {
        const int32_t a = p.aligned[e];
        part += a > 0 ? a : 0;
    }
    if (part != 0) atomicAdd(&s_base, (unsigned long long)part);

    // ---- this slab's segment starts and sizes (er <= 512 < 1024 threads: one each)
    int64_t size = 0;
    if (tid < er) {
        const int32_t a = p.aligned[(int64_t)r * er + tid];
        size = a > 0 ? a : 0;
    }
    const int64_t incl = wave_inclusive_scan64(size);
    if (lane == kWave - 1) s_wsum[wave] = incl;
    __syncthreads();
    int64_t start = (int64_t)s_base + incl - size;
    for (int w = 0; w < wave; ++w) start += s_wsum[w];
    if (tid < er) {
        s_off[tid] = start;
        s_size[tid] = (int32_t)(size < INT32_MAX ? size : INT32_MAX);
        s_run[tid] = 0;
    }
    if (r == p.R - 1 && tid == 0) {
        int64_t total = (int64_t)s_base;
        for (int w = 0; w < kGroupWaves; ++w) total += s_wsum[w];
        p.num_grouped[0] = (int32_t)(total < INT32_MAX ? total : INT32_MAX);
    }

    // ---- the slab's rows
    int64_t hi = p.recv_gbl[r];
    hi = hi < p.num_rows ? hi : p.num_rows;
    hi = hi > 0 ? hi : 0;
    int64_t lo = r > 0 ? p.recv_gbl[r - 1] : 0;
    lo = lo < hi ? lo : hi;
    lo = lo > 0 ? lo : 0;
    bool bad = false, over = false;
    int32_t *tile = s_tile + wave * er;
    __syncthreads();

    for (int64_t g0 = lo; g0 < hi; g0 += kGroupThreads) {
        const int64_t row = g0 + tid;  // wave w takes rows g0 + 64w .. g0 + 64w + 63
        const bool in = row < hi;
        int key[kMaxTopk];
        uint32_t valid = 0;  // bit j: slot j holds a local id of this slab
#pragma unroll
        for (int j = 0; j < kMaxTopk; ++j) {
            key[j] = -1;
            if (j < K && in) {
                const int64_t v = p.recv_idx[row * K + j];
                if (v >= 0 && v < er) {
                    key[j] = (int)v;
                    valid |= 1u << j;
                } else if (v != -1) {
                    bad = true;
                }
            }
        }

        // pass 1: the tile's entry count per local id
        for (int i = lane; i < er; i += kWave) tile[i] = 0;
        for (uint32_t pending = valid;;) {
            const uint64_t holders = ballot64(pending != 0u);
            if (holders == 0ull) break;
            const int id = readlane32(lowest_key(key, pending), __builtin_ctzll(holders));
            const uint32_t m = slots_with_key(key, pending, id);
            const int c = wave_inclusive_scan(__popc(m));
            if (lane == kWave - 1) tile[id] = c;
            pending &= ~m;
        }
        __syncthreads();
        // exclusive starts of each wave's entries, per local id, after the earlier groups
        for (int i = tid; i < er; i += kGroupThreads) {
            int32_t run = s_run[i];
            for (int w = 0; w < kGroupWaves; ++w) {
                const int32_t c = s_tile[w * er + i];
                s_tile[w * er + i] = run;
                run += c;
            }
            s_run[i] = run;
        }
        __syncthreads();

        // pass 2: positions
        for (uint32_t pending = valid;;) {
            const uint64_t holders = ballot64(pending != 0u);
            if (holders == 0ull) break;
            const int id = readlane32(lowest_key(key, pending), __builtin_ctzll(holders));
            const uint32_t m = slots_with_key(key, pending, id);
            const int cnt = __popc(m);
            const int64_t first = (int64_t)tile[id] + (wave_inclusive_scan(cnt) - cnt);
            const int64_t seg = s_off[id];
            const int32_t seg_size = s_size[id];
            for (uint32_t mm = m; mm != 0u; mm &= mm - 1u) {
                const int j = __builtin_ctz(mm);
                const int64_t li = first + __popc(m & ((1u << j) - 1u));
                const int64_t pos = seg + li;
                const bool ok = li < seg_size && pos < p.cap;
                if (ok) {
                    p.grouped_row[pos] = (int32_t)row;
                    if (p.grouped_w != nullptr) p.grouped_w[pos] = p.recv_w[row * K + j];
                } else {
                    over = true;
                }
                if (p.slot_pos != nullptr) p.slot_pos[row * K + j] = ok ? (int32_t)pos : -1;
            }
            pending &= ~m;
        }
        if (p.slot_pos != nullptr && in) {
#pragma unroll
            for (int j = 0; j < kMaxTopk; ++j)
                if (j < K && !((valid >> j) & 1u)) p.slot_pos[row * K + j] = -1;
        }
        __syncthreads();  // the tile counts are reused by the next group
    }

    // ---- padding: the positions of each segment past its entries
    for (int i = wave; i < er; i += kGroupWaves) {
        const int64_t seg_size = s_size[i];
        const int64_t used = s_run[i] < seg_size ? s_run[i] : seg_size;
        const int64_t seg = s_off[i];
        for (int64_t q = used + lane; q < seg_size && seg + q < p.cap; q += kWave) {
            p.grouped_row[seg + q] = -1;
            if (p.grouped_w != nullptr) p.grouped_w[seg + q] = 0.0f;
        }
    }

    // ---- rows past the last slab: in no segment
    if (r == p.R - 1) {
        for (int64_t i = hi * K + tid; i < p.num_rows * K; i += kGroupThreads) {
            const int64_t v = p.recv_idx[i];
            if (v < -1 || v >= er) bad = true;
            if (p.slot_pos != nullptr) p.slot_pos[i] = -1;
        }
    }
    if (ballot64(bad) != 0ull && lane == 0) flag(p.dev_status, EP_DEV_BAD_TOPK_IDX);
    if (ballot64(over) != 0ull && lane == 0) flag(p.dev_status, EP_DEV_RECV_OVERFLOW);
}

struct CopyParams {
    const u32x4 *src;
    const float *src_scales;
    const int32_t *grouped_row;
    const int32_t *num_grouped;
    u32x4 *dst;
    float *dst_scales;
    int32_t *dev_status;
    int64_t row_units, num_rows, cap;
    int S, num_scales;
};

template <int VPL, bool EXACT, int WPB>
__global__ __launch_bounds__(WPB *kWave) void group_copy_kernel(CopyParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t w = (int64_t)blockIdx.x * WPB + (threadIdx.x >> 6);
    const int64_t g = w / p.S;
    const int seg = (int)(w - g * p.S);
    int64_t limit = p.num_grouped[0];
    limit = limit < p.cap ? limit : p.cap;
    if (g >= limit) return;  // whole wave
    int row = __builtin_amdgcn_readfirstlane(p.grouped_row[g]);
    if (row < -1 || row >= p.num_rows) {  // not written by the positions pass
        if (lane == 0 && seg == 0) flag(p.dev_status, EP_DEV_BAD_SEND_SLOT);
        row = -1;
    }
    const int64_t c0 = (int64_t)seg * VPL * kWave + lane;
    u32x4 *dst = p.dst + g * p.row_units + c0;
    if (row >= 0) {
        const u32x4 *src = p.src + (int64_t)row * p.row_units + c0;
        u32x4 v[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (EXACT || c0 + i * kWave < p.row_units) v[i] = __builtin_nontemporal_load(src + i * kWave);
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (EXACT || c0 + i * kWave < p.row_units) __builtin_nontemporal_store(v[i], dst + i * kWave);
    } else {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (EXACT || c0 + i * kWave < p.row_units) __builtin_nontemporal_store(z, dst + i * kWave);
    }
    if (seg == 0) {
        for (int i = lane; i < p.num_scales; i += kWave)
            p.dst_scales[g * p.num_scales + i] = row >= 0 ? p.src_scales[(int64_t)row * p.num_scales + i] : 0.0f;
    }
}

template <int VPL, bool EXACT, int WPB>
hipError_t run_copy(CopyParams p, hipStream_t stream) {
    p.S = (int)((p.row_units + VPL * kWave - 1) / (VPL * kWave));
    const int64_t blocks = (p.cap * p.S + WPB - 1) / WPB;
    hipLaunchKernelGGL((group_copy_kernel<VPL, EXACT, WPB>), dim3((unsigned)blocks), dim3(WPB * kWave), 0, stream,
                       p);
    return hipGetLastError();
}

hipError_t run_copy_tiled(const CopyParams &p, int vpl, int wpb, hipStream_t stream) {
    const bool exact = p.row_units % (vpl * kWave) == 0;
#define EP_GROUP_CASE(V, W) \
    if (vpl == V && wpb == W) return exact ? run_copy<V, true, W>(p, stream) : run_copy<V, false, W>(p, stream);
    EP_GROUP_CASE(1, 8)
    EP_GROUP_CASE(2, 8)
    EP_GROUP_CASE(4, 8)
    EP_GROUP_CASE(7, 4)
    EP_GROUP_CASE(7, 8)
    EP_GROUP_CASE(14, 4)
    EP_GROUP_CASE(14, 8)
#undef EP_GROUP_CASE
    return hipErrorInvalidValue;
}

// One wave per whole row at the 7168-element widths, 1 KiB segments otherwise.
void copy_tiling(int64_t row_units, int *vpl, int *wpb) {
    *wpb = 8;
    if (row_units == 14 * kWave)
        *vpl = 14;
    else if (row_units == 7 * kWave)
        *vpl = 7;
    else
        *vpl = 1;
}

}  // namespace

size_t group_lds_bytes(int er) { return (size_t)er * (sizeof(int64_t) + 2 * sizeof(int32_t) + kGroupWaves * sizeof(int32_t)); }

hipError_t launch_group(const ep_shape_t &s, const GroupArgs &a, hipStream_t stream) {
    PositionParams q;
    q.recv_idx = a.recv_idx;
    q.recv_w = a.recv_w;
    q.recv_gbl = a.recv_gbl;
    q.aligned = a.aligned;
    q.grouped_row = a.grouped_row;
    q.grouped_w = a.grouped_w;
    q.slot_pos = a.slot_pos;
    q.num_grouped = a.num_grouped;
    q.dev_status = a.dev_status;
    q.num_rows = a.num_rows;
    q.cap = a.cap;
    q.R = s.num_ranks;
    q.K = s.num_topk;
    q.er = s.num_experts / s.num_ranks;
    hipLaunchKernelGGL(group_positions_kernel, dim3((unsigned)q.R), dim3(kGroupThreads), group_lds_bytes(q.er), stream,
                       q);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.cap == 0) return err;

    CopyParams c;
    c.src = reinterpret_cast<const u32x4 *>(a.recv_x);
    c.src_scales = a.recv_scales;
    c.grouped_row = a.grouped_row;
    c.num_grouped = a.num_grouped;
    c.dst = reinterpret_cast<u32x4 *>(a.grouped_x);
    c.dst_scales = a.grouped_scales;
    c.dev_status = a.dev_status;
    c.row_units = a.row_units;
    c.num_rows = a.num_rows;
    c.cap = a.cap;
    c.num_scales = a.num_scales;
    c.S = 1;
    int vpl, wpb;
    copy_tiling(c.row_units, &vpl, &wpb);
    return run_copy_tiled(c, vpl, wpb, stream);
}

}  // namespace ep
