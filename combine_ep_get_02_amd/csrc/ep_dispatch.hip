// ep_dispatch.hip -- stages 3+4, dispatch: row assignment and packing (gfx950).
//
// Definitions (mscclpp ht_runtime.cc mirror, internodeDispatch /
// intranodeDispatch; CUDA与DeepEP article 4.1, SrcInfo): the receive region
// holds every destination rank's slab in one allocation, laid out
// [dst_rank][channel]; inside a slab the channel segments follow in channel
// order with tokens ascending.  Because channels are contiguous ascending token
// ranges, token t's row on rank r is
//     slab_begin(r) + #{t' < t : t' goes to r},   slab_begin(r) = recv_gbl[r-1].
// For each routed (t, r): recv_x[row] = x[t] (bitwise), the topk weights and
// local expert ids of the slots whose expert lives on r (0 / -1 elsewhere),
// src_info[row] = {my_rank, t}, send_slot[t][r] = row.
//
// Design (the pages' sender/forwarder rings are transport machinery and are not
// reproduced): one wave per (token, row segment of VPL*1 KiB).  The wave first
// issues the 16-byte loads of its x segment (one read of x per token overall),
// then resolves the token's rows while they are in flight: notify left each
// token's 64-bit rank mask and, per 64-token chunk, the exclusive row offset
// inside every slab; the wave loads its chunk's 64 masks (one per lane) and for
// each destination r a ballot over "lane's token goes to r", masked to the
// lanes before this token, gives the in-chunk rank -- rows come out in the
// canonical order without a serial scan, and lane r ends up holding the row
// for rank r.  The segment is then stored to every destination with 16-byte
// non-temporal stores.  The tiling (whole rows per wave with the block's waves
// sweeping the destinations together, or row segments with consecutive waves
// writing consecutive pieces of the same rows) is picked per row width and
// token count from measurements.
#include "ep_internal.h"

namespace ep {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct DispatchParams {
    const u32x4 *x;
    const float *x_scales;
    const int64_t *topk_idx;
    const float *topk_w;
    const int32_t *recv_gbl;
    const uint64_t *mask;
    const int32_t *rank_off;
    const int32_t *cached_slot;
    u32x4 *recv_x;
    float *recv_scales;
    float *recv_w;
    int64_t *recv_idx;
    int32_t *src_info;
    int32_t *send_slot;
    int32_t *dev_status;
    int64_t T;
    int64_t row_units;  // 16-byte units per row
    int R, K, E, experts_per_rank, my_rank, cap, S, num_scales;
};

// GRAN > 0: the block's waves sweep the destination ranks in order and meet at
// a barrier every GRAN ranks, so the blocks' concurrent stores gather in a few
// slabs instead of spreading over all of them.  GRAN == 0: free-running waves.
// CACHED: the rows come from send_slot of an earlier dispatch with the same
// routing (p.cached_slot); no routing, metadata or send_slot output.
template <int VPL, bool EXACT, int WPB, int GRAN, bool CACHED>
__global__ __launch_bounds__(WPB *kWave) void dispatch_kernel(DispatchParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t w0 = (int64_t)blockIdx.x * WPB + (threadIdx.x >> 6);
    const bool live = w0 < p.T * p.S;
    if (GRAN == 0 && !live) return;  // whole wave leaves together
    // with barriers every wave stays to the end; idle ones work on token 0 and store nothing
    const int64_t w = live ? w0 : 0;
    const int64_t t = w / p.S;
    const int seg = (int)(w - t * p.S);
    const int R = p.R;

    // ---- the x segment: issued first, consumed last
    const int64_t c0 = (int64_t)seg * VPL * kWave + lane;
    const u32x4 *src = p.x + t * p.row_units + c0;
    u32x4 v[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        if (EXACT || c0 + i * kWave < p.row_units) v[i] = __builtin_nontemporal_load(src + i * kWave);

    int slot = -1;
    int64_t e = -1;
    float wt = 0.0f;
    if (CACHED) {
        // ---- rows recorded by an earlier dispatch
        bool bad = false;
        if (live && lane < R) {
            slot = p.cached_slot[t * R + lane];
            if (slot < -1 || slot >= p.cap) {
                bad = true;
                slot = -1;
            }
        }
        if (ballot64(bad) != 0ull && lane == 0 && seg == 0) flag(p.dev_status, EP_DEV_BAD_SEND_SLOT);
    } else {
        // ---- routing state: chunk masks, slab bases, this token's topk slots
        const int64_t q = t / kChunk;
        const int my = (int)(t - q * kChunk);
        const int64_t tok = q * kChunk + lane;
        const uint64_t m = tok < p.T ? p.mask[tok] : 0ull;
        int base = 0;
        if (lane < R) base = (lane > 0 ? p.recv_gbl[lane - 1] : 0) + p.rank_off[q * R + lane];
        if (live && seg == 0 && lane < p.K) {
            e = p.topk_idx[t * p.K + lane];
            wt = p.topk_w[t * p.K + lane];
        }

        // ---- row assignment (a3): lane r gets the row for rank r
        const uint64_t mine = readlane64(m, my);
        const uint64_t before = (1ull << my) - 1ull;
        for (uint64_t mm = mine; mm != 0ull; mm &= mm - 1ull) {
            const int r = __builtin_ctzll(mm);
            const uint64_t b = ballot64((m >> r) & 1ull);
            if (lane == r) slot = base + __popcll(b & before);
        }
        const bool over = slot >= p.cap;
        if (over) slot = -1;
        if (live && seg == 0 && ballot64(over) != 0ull && lane == 0) flag(p.dev_status, EP_DEV_RECV_OVERFLOW);
    }
    if (!live) slot = -1;
    const uint64_t dests = ballot64(slot >= 0);

    // ---- per-token scales (fp8 rows) travel beside the rows
    if (live && seg == 0 && p.num_scales > 0) {
        for (int i0 = 0; i0 < p.num_scales; i0 += kWave) {
            const int i = i0 + lane;
            const float sc = i < p.num_scales ? p.x_scales[t * p.num_scales + i] : 0.0f;
            for (uint64_t dd = dests; dd != 0ull; dd &= dd - 1ull) {
                const int64_t s = readlane32(slot, __builtin_ctzll(dd));
                if (i < p.num_scales) p.recv_scales[s * p.num_scales + i] = sc;
            }
        }
    }

    if (!CACHED && live && seg == 0) {
        if (lane < R) p.send_slot[t * R + lane] = slot;
        // ---- metadata (a4): weights / local ids of the slots living on each destination
        const int erank = (e >= 0 && e < p.E) ? (int)e / p.experts_per_rank : -1;
        for (uint64_t dd = dests; dd != 0ull; dd &= dd - 1ull) {
            const int r = __builtin_ctzll(dd);
            const int64_t s = readlane32(slot, r);
            if (lane < p.K) {
                const bool on = erank == r;
                p.recv_w[s * p.K + lane] = on ? wt : 0.0f;
                if (p.recv_idx != nullptr) p.recv_idx[s * p.K + lane] = on ? e - (int64_t)r * p.experts_per_rank : -1;
            }
            if (lane == 0) reinterpret_cast<int2 *>(p.src_info)[s] = make_int2(p.my_rank, (int)t);
        }
    }

    // ---- row copy (a4): the segment to every destination, ranks ascending
    auto store_to = [&](uint64_t dd) {
        for (; dd != 0ull; dd &= dd - 1ull) {
            const int r = __builtin_ctzll(dd);
            const int64_t s = readlane32(slot, r);
            u32x4 *dst = p.recv_x + s * p.row_units + c0;
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                if (EXACT || c0 + i * kWave < p.row_units) __builtin_nontemporal_store(v[i], dst + i * kWave);
        }
    };
    if (GRAN == 0) {
        store_to(dests);
    } else {
        for (int r0 = 0; r0 < R; r0 += GRAN) {
            const uint64_t window = (GRAN >= kWave ? ~0ull : ((1ull << GRAN) - 1ull)) << r0;
            store_to(dests & window);
            __syncthreads();
        }
    }
}

template <int VPL, bool EXACT, int WPB, int GRAN>
hipError_t run(DispatchParams p, hipStream_t stream) {
    p.S = (int)((p.row_units + VPL * kWave - 1) / (VPL * kWave));
    const int64_t waves = p.T * p.S;
    const int64_t blocks = (waves + WPB - 1) / WPB;
    if (p.cached_slot != nullptr)
        hipLaunchKernelGGL((dispatch_kernel<VPL, EXACT, WPB, GRAN, true>), dim3((unsigned)blocks), dim3(WPB * kWave),
                           0, stream, p);
    else
        hipLaunchKernelGGL((dispatch_kernel<VPL, EXACT, WPB, GRAN, false>), dim3((unsigned)blocks),
                           dim3(WPB * kWave), 0, stream, p);
    return hipGetLastError();
}

// Tiling: 16-byte units per lane per segment (VPL), waves per block (WPB) and
// the rank-sweep barrier granularity (GRAN, 0 = none).  Only the tilings below
// are instantiated; dispatch_tiling picks one per row width.
hipError_t run_tiled(const DispatchParams &p, int vpl, int wpb, int gran, hipStream_t stream) {
    const bool exact = p.row_units % (vpl * kWave) == 0;
#define EP_DISPATCH_CASE(V, W, G) \
    if (vpl == V && wpb == W && gran == G) return exact ? run<V, true, W, G>(p, stream) : run<V, false, W, G>(p, stream);
    EP_DISPATCH_CASE(1, 4, 0)
    EP_DISPATCH_CASE(1, 8, 0)
    EP_DISPATCH_CASE(1, 8, 1)
    EP_DISPATCH_CASE(1, 8, 4)
    EP_DISPATCH_CASE(2, 4, 0)
    EP_DISPATCH_CASE(2, 8, 0)
    EP_DISPATCH_CASE(2, 8, 1)
    EP_DISPATCH_CASE(4, 4, 0)
    EP_DISPATCH_CASE(7, 4, 0)
    EP_DISPATCH_CASE(7, 8, 0)
    EP_DISPATCH_CASE(7, 16, 4)
    EP_DISPATCH_CASE(8, 4, 0)
    EP_DISPATCH_CASE(8, 8, 1)
    EP_DISPATCH_CASE(14, 4, 0)
    EP_DISPATCH_CASE(14, 4, 1)
    EP_DISPATCH_CASE(14, 8, 0)
    EP_DISPATCH_CASE(14, 8, 1)
    EP_DISPATCH_CASE(14, 8, 4)
    EP_DISPATCH_CASE(14, 16, 1)
    EP_DISPATCH_CASE(14, 16, 4)
#undef EP_DISPATCH_CASE
    return hipErrorInvalidValue;
}

// Measured on MI355X (rows of 7168 bf16 or fp8 elements at 128..4096 tokens,
// and the skew / large workloads).  Whole rows per wave with the rank sweep
// (16 waves per block, a barrier every 4 ranks) win once there are enough
// tokens to give every compute unit a block; below that the rows are split so
// more waves share the copy.  Other widths: 1 KiB segments, 8 waves per block.
void dispatch_tiling(int64_t row_units, int64_t num_tokens, int *vpl, int *wpb, int *gran) {
    *vpl = 1;
    *wpb = 8;
    *gran = 0;
    if (row_units == 14 * kWave) {  // 7168 bf16
        if (num_tokens >= 2048) {
            *vpl = 14;
            *wpb = 16;
            *gran = 4;
        } else {
            *vpl = 7;
            *wpb = 4;
        }
    } else if (row_units == 7 * kWave) {  // 7168 fp8 (or 3584 bf16)
        if (num_tokens >= 4096) {
            *vpl = 7;
            *wpb = 16;
            *gran = 4;
        } else {
            *vpl = 4;
            *wpb = 4;
        }
    }
}

}  // namespace

hipError_t launch_dispatch(const ep_shape_t &s, const DispatchArgs &a, hipStream_t stream) {
    if (s.num_tokens == 0) return hipSuccess;
    DispatchParams p;
    p.x = reinterpret_cast<const u32x4 *>(a.x);
    p.x_scales = a.x_scales;
    p.topk_idx = a.topk_idx;
    p.topk_w = a.topk_w;
    p.recv_gbl = a.recv_gbl;
    p.mask = nullptr;
    p.rank_off = nullptr;
    if (a.ws != nullptr) {
        const Workspace w = workspace_layout(s.num_tokens, s.num_ranks, s.num_experts, s.num_channels);
        p.mask = reinterpret_cast<const uint64_t *>(a.ws + w.mask);
        p.rank_off = reinterpret_cast<const int32_t *>(a.ws + w.rank_off);
    }
    p.cached_slot = a.cached_slot;
    p.recv_x = reinterpret_cast<u32x4 *>(a.recv_x);
    p.recv_scales = a.recv_scales;
    p.recv_w = a.recv_w;
    p.recv_idx = a.recv_idx;
    p.src_info = a.src_info;
    p.send_slot = a.send_slot;
    p.dev_status = a.dev_status;
    p.T = s.num_tokens;
    p.row_units = a.row_units;
    p.R = s.num_ranks;
    p.K = s.num_topk;
    p.E = s.num_experts;
    p.experts_per_rank = s.num_experts / s.num_ranks;
    p.my_rank = s.my_rank;
    p.cap = a.cap;
    p.num_scales = a.num_scales;
    p.S = 1;
    int vpl, wpb, gran;
    dispatch_tiling(p.row_units, p.T, &vpl, &wpb, &gran);
    return run_tiled(p, vpl, wpb, gran, stream);
}

}  // namespace ep
