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
//  positions: one 512-thread block per group of 512 rows of a slab (one
//   tile of 64 rows per wave, one row per lane); a block first counts, per
//   local id, the entries in the slab's rows before its group.  A wave enumerates the
//   distinct local ids present in its tile (the lowest lane still holding an
//   unranked slot names the next id); for each id a DPP wave scan of the
//   lanes' slot counts gives every slot of that id its rank inside the tile,
//   stably in (row, slot) order, kept in a register per slot.  The tiles'
//   totals are scanned across the block's waves in LDS and added to running per-id
//   counts; then each slot's position is its segment start + its wave's start
//   + its rank, and the grouped row index and weight are written there.
//   Padding positions are marked last.  The kernel is instantiated for up to
//   8, 16 or 32 slots per row so the per-slot loops are no longer than k.
//  copy: one wave per grouped row copies the receive row it names (zeros for
//   padding) with 16-byte non-temporal loads and stores; the grouped rows are
//   written in order, as one contiguous stream.
// Straight from x (ep_dispatch_grouped below 2048 tokens, after its metadata
// launch): the same positions launch, then each token's row pushed to its
// positions (group_push_kernel) and the padding zeroed after it
// (group_pad_kernel).  From 2048 tokens the whole call is one launch in
// ep_dispatch.hip, which finds the same positions in token order.
#include "ep_internal.h"

namespace ep {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGroupWaves = 8;
constexpr int kGroupThreads = kGroupWaves * kWave;
static_assert(kMaxGroupExperts <= kGroupThreads, "one thread per local expert of a slab");

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

// Key of the lowest set slot of `pending` (the slot order is the entry order).
template <int KB>
__device__ __forceinline__ int lowest_key(const int (&key)[KB], uint32_t pending) {
    int first = -1;
#pragma unroll
    for (int j = KB - 1; j >= 0; --j)
        if ((pending >> j) & 1u) first = key[j];
    return first;
}

// Clamped bounds of slab r: rows [lo, hi) with 0 <= lo <= hi <= num_rows.
__device__ __forceinline__ void slab_bounds(const int32_t *recv_gbl, int r, int64_t num_rows, int64_t *lo,
                                            int64_t *hi) {
    int64_t h = recv_gbl[r];
    h = h < num_rows ? h : num_rows;
    h = h > 0 ? h : 0;
    int64_t l = r > 0 ? recv_gbl[r - 1] : 0;
    l = l < h ? l : h;
    *lo = l > 0 ? l : 0;
    *hi = h;
}

// KB: slots per row the kernel is built for (k <= KB).  One block per group of
// up to 512 rows of one slab (at least one block per slab, so that empty
// slabs still get their padding).
template <int KB>
__global__ __launch_bounds__(kGroupThreads) void group_positions_kernel(PositionParams p) {
    // dynamic LDS: int64 s_off[er] | int32 s_size[er] | int32 s_run[er] | int32 s_tile[waves][er]
    extern __shared__ int64_t s_dyn[];
    __shared__ int64_t s_wsum[kGroupWaves], s_wbase[kGroupWaves], s_wall[kGroupWaves];
    const int er = p.er, K = p.K, R = p.R;
    int64_t *s_off = s_dyn;
    int32_t *s_size = reinterpret_cast<int32_t *>(s_off + er);
    int32_t *s_run = s_size + er;
    int32_t *s_tile = s_run + er;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;

    // ---- which slab and which group of it: lane l of every wave counts slab l's
    // groups (every lane loads, at a rank clamped into range: a load under a branch
    // would be waited for where the branch joins)
    int groups = 0;
    {
        int64_t l0, h0;
        slab_bounds(p.recv_gbl, lane < R ? lane : R - 1, p.num_rows, &l0, &h0);
        const int64_t n = h0 - l0;
        groups = lane < R ? (n > 0 ? (int)((n + kGroupThreads - 1) / kGroupThreads) : 1) : 0;
    }
    const int ends = wave_inclusive_scan(groups);  // lane l: groups of slabs 0..l
    const int total_groups = readlane32(ends, kWave - 1);
    const int b = blockIdx.x;
    if (b >= total_groups) return;  // the same decision in every wave of the block
    const int r = __popcll(ballot64(lane < R && ends <= b));
    const int group = b - (r > 0 ? readlane32(ends, r - 1) : 0);
    const bool last_group = group == readlane32(groups, r) - 1;
    int64_t lo, hi;
    slab_bounds(p.recv_gbl, r, p.num_rows, &lo, &hi);
    const int64_t g0 = lo + (int64_t)group * kGroupThreads;  // this block's rows: [g0, min(g0 + 512, hi))

    // ---- this group's rows (one tile of 64 rows per wave, one row per lane): ids and
    // weights, loaded first, together with the segment sizes below
    bool bad = false, over = false;
    const int64_t row = g0 + tid;
    const bool in = row < hi;
    const bool in_any = g0 < hi;  // the same for the whole block
    int key[KB];
    int rank[KB];        // rank of the slot among the tile's entries of its id
    float wt[KB];        // the slot's weight (fetched with the ids when KB <= 16)
    uint32_t valid = 0;  // bit j: slot j holds a local id of this slab
    const bool want_w = p.grouped_w != nullptr;
    // the row's ids (and weights, and token) loaded by every lane at once, at a row
    // and slot clamped into range, before any is used
    int64_t vid[KB];
    if (in_any) {  // block-uniform: rows exist
        const int64_t lrow = in ? row : 0;
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            const int jj = j < K ? j : K - 1;
            vid[j] = p.recv_idx[lrow * K + jj];
            if (KB <= 16 && want_w) wt[j] = p.recv_w[lrow * K + jj];
        }
    }
    // this slab's segment sizes (er <= kMaxGroupExperts <= threads: one each) and
    // the first pass of the sums below, loaded at once at clamped indices
    const int64_t n_before = (int64_t)r * er, n_all = (int64_t)R * er;
    const int32_t size_ld = p.aligned[(int64_t)r * er + (tid < er ? tid : 0)];
    const int32_t before_ld = p.aligned[tid < n_before ? tid : 0];
    const int32_t all_ld = p.aligned[tid < n_all ? tid : 0];
    const int32_t size_raw = tid < er ? size_ld : 0;

    // ---- segment starts: the sizes of all segments of earlier slabs (a block sum),
    // then a scan over this slab's
    int64_t part = tid < n_before && before_ld > 0 ? before_ld : 0, all = 0;
    for (int64_t e = tid + kGroupThreads; e < n_before; e += kGroupThreads) {
        const int32_t a = p.aligned[e];
        part += a > 0 ? a : 0;
    }
    if (b == 0) {  // one block reports the total
        all = tid < n_all && all_ld > 0 ? all_ld : 0;
        for (int64_t e = tid + kGroupThreads; e < n_all; e += kGroupThreads) {
            const int32_t a = p.aligned[e];
            all += a > 0 ? a : 0;
        }
    }
    part = wave_sum64(part);
    all = wave_sum64(all);
    if (lane == 0) {
        s_wbase[wave] = part;
        s_wall[wave] = all;
    }

    // ---- entries of each local id in the slab's rows before this group: each wave
    // counts tiles of 64 of those rows into its own row of the tile table with LDS
    // atomics (only lanes of the same wave can meet on an address), then the rows
    // are added up; TU tiles per pass, their ids all loaded before any is counted
    int32_t *tile = s_tile + wave * er;
    for (int i = lane; i < er; i += kWave) tile[i] = 0;
    constexpr int TU = KB <= 8 ? 4 : 1;
    for (int64_t t0 = lo + (int64_t)wave * kWave; t0 < g0; t0 += (int64_t)TU * kGroupThreads) {
        int pkey[TU][KB];
#pragma unroll
        for (int u = 0; u < TU; ++u) {
            const int64_t prow = t0 + (int64_t)u * kGroupThreads + lane;
#pragma unroll
            for (int j = 0; j < KB; ++j) {
                pkey[u][j] = -1;
                if (j < K && prow < g0) {
                    const int64_t v = p.recv_idx[prow * K + j];
                    if (v >= 0 && v < er) pkey[u][j] = (int)v;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < TU; ++u)
#pragma unroll
            for (int j = 0; j < KB; ++j)
                if (pkey[u][j] >= 0) atomicAdd(&tile[pkey[u][j]], 1);
    }
#pragma unroll
    for (int j = 0; j < KB; ++j) {
        key[j] = -1;
        rank[j] = 0;
        if (!(KB <= 16 && want_w) || !(j < K && in)) wt[j] = 0.0f;
        if (j < K && in) {
            const int64_t v = vid[j];
            if (v >= 0 && v < er) {
                key[j] = (int)v;
                valid |= 1u << j;
            } else if (v != -1) {
                bad = true;
            }
        }
    }

    const int64_t size = size_raw > 0 ? size_raw : 0;
    const int64_t incl = wave_inclusive_scan64(size);
    if (lane == kWave - 1) s_wsum[wave] = incl;
    __syncthreads();
    int64_t base = 0, total_all = 0, start = incl - size;
    for (int w = 0; w < kGroupWaves; ++w) {
        base += s_wbase[w];
        total_all += s_wall[w];
        if (w < wave) start += s_wsum[w];
    }
    start += base;
    if (tid < er) {
        s_off[tid] = start;
        s_size[tid] = (int32_t)(size < INT32_MAX ? size : INT32_MAX);
    }
    for (int i = tid; i < er; i += kGroupThreads) {
        int32_t run = 0;
        for (int w = 0; w < kGroupWaves; ++w) run += s_tile[w * er + i];
        s_run[i] = run;
    }
    if (b == 0 && tid == 0) p.num_grouped[0] = (int32_t)(total_all < INT32_MAX ? total_all : INT32_MAX);

    __syncthreads();  // s_off, s_size and the earlier rows' counts are complete

    // ranks inside the tile and the tile's entry count per local id
    for (int i = lane; i < er; i += kWave) tile[i] = 0;
    for (uint32_t pending = valid;;) {
        const uint64_t holders = ballot64(pending != 0u);
        if (holders == 0ull) break;
        const int id = readlane32(lowest_key<KB>(key, pending), __builtin_ctzll(holders));
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < KB; ++j)
            if (((pending >> j) & 1u) && key[j] == id) m |= 1u << j;
        const int cnt = __popc(m);
        const int incl_c = wave_inclusive_scan(cnt);
        const int before = incl_c - cnt;
#pragma unroll
        for (int j = 0; j < KB; ++j)
            if ((m >> j) & 1u) rank[j] = before + __popc(m & ((1u << j) - 1u));
        if (lane == kWave - 1) tile[id] = incl_c;
        pending &= ~m;
    }
    __syncthreads();
    // exclusive start of each wave's entries per local id, after the slab's earlier rows
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

    // positions: segment start + the wave's start + the rank in the tile
    if (in) {
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            if (j >= K) continue;
            int32_t at = -1;
            if ((valid >> j) & 1u) {
                const int id = key[j];
                const int64_t li = (int64_t)tile[id] + rank[j];
                const int64_t pos = s_off[id] + li;
                if (li < s_size[id] && pos < p.cap) {
                    p.grouped_row[pos] = (int32_t)row;
                    if (want_w) p.grouped_w[pos] = KB <= 16 ? wt[j] : p.recv_w[row * K + j];
                    at = (int32_t)pos;
                } else {
                    over = true;
                }
            }
            if (p.slot_pos != nullptr) p.slot_pos[row * K + j] = at;
        }
    }

    // ---- padding, by the slab's last group once every entry is counted
    if (last_group) {
        for (int i = wave; i < er; i += kGroupWaves) {
            const int64_t seg_size = s_size[i];
            const int64_t used = s_run[i] < seg_size ? s_run[i] : seg_size;
            const int64_t seg = s_off[i];
            for (int64_t q = used + lane; q < seg_size && seg + q < p.cap; q += kWave) {
                p.grouped_row[seg + q] = -1;
                if (want_w) p.grouped_w[seg + q] = 0.0f;
            }
        }
    }

    // ---- rows past the last slab hold no received token (capacity slack): their ids
    // are not read, their slots are in no segment (the last block)
    if (b == total_groups - 1 && p.slot_pos != nullptr) {
        for (int64_t i = hi * K + tid; i < p.num_rows * K; i += kGroupThreads) p.slot_pos[i] = -1;
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
    const int64_t srow = row;
    const int64_t c0 = (int64_t)seg * VPL * kWave + lane;
    u32x4 *dst = p.dst + g * p.row_units + c0;
    if (row >= 0) {
        const u32x4 *src = p.src + srow * p.row_units + c0;
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
        for (int i0 = 0; i0 < p.num_scales; i0 += kWave) {  // wave-uniform, per-lane predicate
            const int i = i0 + lane;
            const float sc = (i < p.num_scales && row >= 0) ? p.src_scales[srow * p.num_scales + i] : 0.0f;
            if (i < p.num_scales) p.dst_scales[g * p.num_scales + i] = sc;
        }
    }
}

// ---- straight from x (dispatch into the grouped layout): each token's row is
// read once and stored to every grouped position of its slots, found through
// send_slot (the receive row on the slot's rank) and slot_pos (the row's entry);
// then the padding rows are zeroed.
struct PushParams {
    const u32x4 *x;
    const float *x_scales;
    const int64_t *topk_idx;
    const int32_t *send_slot;
    const int32_t *slot_pos;
    const int32_t *num_grouped;
    u32x4 *dst;
    float *dst_scales;
    int64_t T, row_units, num_rows, cap;
    int R, K, E, er, S, num_scales;
};

template <int VPL, bool EXACT, int WPB>
__global__ __launch_bounds__(WPB *kWave) void group_push_kernel(PushParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t w = (int64_t)blockIdx.x * WPB + (threadIdx.x >> 6);
    if (w >= p.T * p.S) return;  // whole wave
    const int64_t t = w / p.S;
    const int seg = (int)(w - t * p.S);
    // the x segment first, consumed last
    const int64_t c0 = (int64_t)seg * VPL * kWave + lane;
    const u32x4 *src = p.x + t * p.row_units + c0;
    u32x4 v[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        if (EXACT || c0 + i * kWave < p.row_units) v[i] = __builtin_nontemporal_load(src + i * kWave);
    // lane j < k: the grouped position of slot j, or -1 (masked, dropped, or past the
    // written grouped rows)
    int64_t limit = p.num_grouped[0];
    limit = limit < p.cap ? limit : p.cap;
    int pos = -1;
    if (lane < p.K) {
        const int64_t e = p.topk_idx[t * p.K + lane];
        if (e >= 0 && e < p.E) {
            const int s = p.send_slot[t * p.R + (int)(e / p.er)];
            if (s >= 0 && s < p.num_rows) pos = p.slot_pos[(int64_t)s * p.K + lane];
        }
        if (pos >= limit) pos = -1;
    }
    const uint64_t dests = ballot64(pos >= 0);
    for (uint64_t dd = dests; dd != 0ull; dd &= dd - 1ull) {
        const int64_t g = readlane32(pos, __builtin_ctzll(dd));
        u32x4 *dst = p.dst + g * p.row_units + c0;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (EXACT || c0 + i * kWave < p.row_units) __builtin_nontemporal_store(v[i], dst + i * kWave);
        if (seg == 0) {  // a wave-uniform loop with a per-lane predicate
            for (int i0 = 0; i0 < p.num_scales; i0 += kWave) {
                const int i = i0 + lane;
                const float sc = i < p.num_scales ? p.x_scales[t * p.num_scales + i] : 0.0f;
                if (i < p.num_scales) p.dst_scales[g * p.num_scales + i] = sc;
            }
        }
    }
}

// Padding rows (grouped_row -1) of the written grouped rows: zero rows and scales.
__global__ __launch_bounds__(256) void group_pad_kernel(const int32_t *grouped_row, const int32_t *num_grouped,
                                                        u32x4 *dst, float *dst_scales, int64_t row_units,
                                                        int64_t cap, int num_scales) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    int64_t limit = num_grouped[0];
    limit = limit < cap ? limit : cap;
    if (g >= limit || grouped_row[g] != -1) return;  // whole wave
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t u = lane; u < row_units; u += kWave) __builtin_nontemporal_store(z, dst + g * row_units + u);
    for (int i0 = 0; i0 < num_scales; i0 += kWave)  // wave-uniform, per-lane predicate
        if (i0 + lane < num_scales) dst_scales[g * num_scales + i0 + lane] = 0.0f;
}

template <int VPL, bool EXACT, int WPB>
hipError_t run_push(PushParams p, hipStream_t stream) {
    p.S = (int)((p.row_units + VPL * kWave - 1) / (VPL * kWave));
    const int64_t blocks = (p.T * p.S + WPB - 1) / WPB;
    hipLaunchKernelGGL((group_push_kernel<VPL, EXACT, WPB>), dim3((unsigned)blocks), dim3(WPB * kWave), 0, stream,
                       p);
    return hipGetLastError();
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

// Measured on MI355X (prefill, skew, large workloads): 2 KiB segments, 8
// waves per block, ahead of whole-row waves and of 1 KiB segments.
void copy_tiling(int64_t row_units, int *vpl, int *wpb) {
    (void)row_units;
    *vpl = 2;
    *wpb = 8;
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
    const size_t lds = group_lds_bytes(q.er);
    // enough blocks for every slab's groups of 512 rows, at least one per slab
    const dim3 grid((unsigned)((q.num_rows + kGroupThreads - 1) / kGroupThreads + q.R));
    if (q.K <= 8)
        hipLaunchKernelGGL(group_positions_kernel<8>, grid, dim3(kGroupThreads), lds, stream, q);
    else if (q.K <= 16)
        hipLaunchKernelGGL(group_positions_kernel<16>, grid, dim3(kGroupThreads), lds, stream, q);
    else
        hipLaunchKernelGGL(group_positions_kernel<32>, grid, dim3(kGroupThreads), lds, stream, q);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.cap == 0) return err;

    if (a.from_x) {  // rows straight from x
        if (a.num_tokens > 0) {
            PushParams u;
            u.x = reinterpret_cast<const u32x4 *>(a.recv_x);
            u.x_scales = a.recv_scales;
            u.topk_idx = a.topk_idx;
            u.send_slot = a.send_slot;
            u.slot_pos = a.slot_pos;
            u.num_grouped = a.num_grouped;
            u.dst = reinterpret_cast<u32x4 *>(a.grouped_x);
            u.dst_scales = a.grouped_scales;
            u.T = a.num_tokens;
            u.row_units = a.row_units;
            u.num_rows = a.num_rows;
            u.cap = a.cap;
            u.R = s.num_ranks;
            u.K = s.num_topk;
            u.E = s.num_experts;
            u.er = s.num_experts / s.num_ranks;
            u.num_scales = a.num_scales;
            u.S = 1;
            // the push tiling of the receive dispatch: 7 KiB segments, 4 waves per block
            // for 7168-element bf16 rows, 1 KiB segments otherwise
            if (a.row_units % (7 * kWave) == 0)
                err = run_push<7, true, 4>(u, stream);
            else if (a.row_units % kWave == 0)
                err = run_push<1, true, 8>(u, stream);
            else
                err = run_push<1, false, 8>(u, stream);
            if (err != hipSuccess) return err;
        }
        hipLaunchKernelGGL(group_pad_kernel, dim3((unsigned)((a.cap + 3) / 4)), dim3(256), 0, stream, a.grouped_row,
                           a.num_grouped, reinterpret_cast<u32x4 *>(a.grouped_x), a.grouped_scales, a.row_units, a.cap,
                           a.num_scales);
        return hipGetLastError();
    }

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
