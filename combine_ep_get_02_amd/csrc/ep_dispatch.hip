// ep_dispatch.hip -- stages 3+4, dispatch: row assignment and packing (gfx950).
//
// Definitions (mscclpp ht_runtime.cc mirror, internodeDispatch /
// intranodeDispatch; CUDA与DeepEP article 4.1, SrcInfo): the receive region
// holds every destination rank's slab in one allocation, laid out
// [dst_rank][channel]; inside a slab the channel segments follow in channel
// order with tokens ascending.  Because channels are contiguous ascending token
// ranges, token t of channel c has, on rank r, the row
//     slab_begin(r) + gbl[r][c-1] + #{t' in channel c, t' < t : t' goes to r}
// (slab_begin(r) = recv_gbl[r-1]), which with a consistent prefix matrix is
//     slab_begin(r) + #{t' < t : t' goes to r}.
// For each routed (t, r): recv_x[row] = x[t] (bitwise), the topk weights and
// local expert ids of the slots whose expert lives on r (0 / -1 elsewhere),
// src_info[row] = {my_rank, t}, send_slot[t][r] = row.
//
// Design (the pages' sender/forwarder rings are transport machinery and are not
// reproduced).  Every row's position is known without a serial scan once each
// 64-token chunk has its tokens' 64-bit rank masks and its row offset inside
// every slab.  Those come either from the workspace notify filled (checked here
// against is_token_in_rank and the channel prefix matrix), or, without a
// workspace, straight from the routing inputs: the masks from is_token_in_rank
// rows, the offset from the prefix matrix entry of the chunk's channel plus the
// tokens between the channel's edge and the chunk, counted with the same bit
// transpose.  Two forms:
//  - pull (from 2048 tokens, rows of 1 KiB to 1 MiB): the rows are produced in
//    receive order.  Each XCD takes groups of 128 tokens in turn; a wave finds
//    the group's rows per rank with a 64x64 bit transpose of the masks and a
//    wave scan, and the XCD's waves write the group's output as one advancing
//    window of small tasks, reading x from the XCD's L2 (dispatch_pull_kernel);
//  - push (fewer tokens, other widths, cached mode): one wave per (token, row
//    segment) loads its x segment once and stores it to every destination
//    (dispatch_kernel).  For each destination r a ballot over the chunk's
//    masks, masked to the lanes before the token, gives the in-chunk rank, so
//    lane r ends up holding the row for rank r.
// All row traffic uses 16-byte accesses with non-temporal stores.  The form
// and tiling are picked per row width and token count from measurements.
#include "ep_internal.h"

namespace ep {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct DispatchParams {
    const u32x4 *x;
    const float *x_scales;
    const int64_t *topk_idx;
    const float *topk_w;
    const uint8_t *in_rank;  // [t][R] is_token_in_rank
    const int32_t *gbl;      // [R][C] channel prefix matrix (inclusive)
    const int32_t *recv_gbl;
    const uint64_t *mask;    // workspace: per-token rank masks, or null (derive)
    const int32_t *rank_off;  // workspace: per-chunk row offsets inside each chunk's group, or null (derive)
    const int32_t *rank_base; // workspace: per-group row offsets inside each slab (a chunk starts at the sum)
    const int32_t *cached_slot;
    u32x4 *recv_x;
    float *recv_scales;
    float *recv_w;
    int64_t *recv_idx;
    int32_t *src_info;
    int32_t *send_slot;
    int32_t *dev_status;
    int64_t T;
    int64_t Tc;         // tokens per channel, ceil(t / C)
    int64_t row_units;  // 16-byte units per row
    int R, K, E, C, experts_per_rank, my_rank, cap, S, num_scales;
    int in_unit;        // load unit of an is_token_in_rank row (16, 8 or 1 bytes)
    int quant_log2;     // quantising dispatch: log2 of the lanes per scale group
    bool derive;        // routing from is_token_in_rank and the prefix matrix (no workspace)
};

// ---------------------------------------------------------------- routing
// Rank mask of token tok (0 past the last token): from its is_token_in_rank row
// when deriving, else from the workspace.
__device__ __forceinline__ uint64_t token_mask(const DispatchParams &p, int64_t tok, bool derive) {
    if (tok >= p.T) return 0ull;
    return derive ? load_rank_mask(p.in_rank + tok * p.R, p.R, p.in_unit) : p.mask[tok];
}

// Lane r < R: the tokens of [x, y) sent to rank r (0 on the other lanes), 64
// tokens a step: lane l loads token s + l's row, the bit transpose hands lane r
// the step's column for rank r.
__device__ int count_tokens(const DispatchParams &p, int64_t x, int64_t y, int lane) {
    int n = 0;
    for (int64_t s = x; s < y; s += kChunk) {
        const int64_t tok = s + lane;
        const uint64_t m = tok < y ? load_rank_mask(p.in_rank + tok * p.R, p.R, p.in_unit) : 0ull;
        n += __popcll(transpose64(m));
    }
    return n;
}

// Tokens of a group's columns (lane r: bit l of col[c] = token c*64 + l goes to
// rank r) at offsets below d, 0 <= d <= 64*CPG.
template <int CPG>
__device__ __forceinline__ int count_below(const uint64_t (&col)[CPG], int64_t d) {
    int n = 0;
#pragma unroll
    for (int c = 0; c < CPG; ++c) {
        const int64_t k = d - c * kChunk;
        const uint64_t m = k >= kChunk ? ~0ull : (k <= 0 ? 0ull : (1ull << k) - 1ull);
        n += __popcll(col[c] & m);
    }
    return n;
}

// Lane r < R: #{t < a : token t goes to rank r}, the offset inside slab r of a
// group of CPG chunks starting at token a (a multiple of 64) with columns col.
// Channel c holding a covers [b, e); the prefix matrix gives the count before b
// (entry c-1) and before e (entry c), so the offset is entry c-1 plus the tokens
// of [b, a), or entry c minus those of [a, e).  The side with fewer tokens beyond
// the group's own is counted (at most half a channel); other = true takes the
// other side instead (a second reading of the same offset, for the checks).
// The part of derive_offset that needs no columns: the prefix entry and the
// tokens counted outside the group; derive_offset = this plus derive_inner.
template <int CPG>
__device__ int derive_outer(const DispatchParams &p, int64_t a, int lane) {
    constexpr int64_t GT = CPG * kChunk;
    const int64_t c = a / p.Tc;
    const int64_t b = c * p.Tc;
    const int64_t e = b + p.Tc < p.T ? b + p.Tc : p.T;
    const int64_t back = a - b;
    const int64_t fwd = e > a + GT ? e - (a + GT) : 0;
    int v = 0;
    if (fwd <= back) {
        if (lane < p.R) v = p.gbl[(int64_t)lane * p.C + c];
        if (fwd > 0) v -= count_tokens(p, a + GT, e, lane);
    } else {
        if (lane < p.R && c > 0) v = p.gbl[(int64_t)lane * p.C + c - 1];
        v += count_tokens(p, b, a, lane);
    }
    return v;
}
template <int CPG>
__device__ int derive_inner(const DispatchParams &p, int64_t a, const uint64_t (&col)[CPG]) {
    constexpr int64_t GT = CPG * kChunk;
    const int64_t c = a / p.Tc;
    const int64_t b = c * p.Tc;
    const int64_t e = b + p.Tc < p.T ? b + p.Tc : p.T;
    const int64_t fwd = e > a + GT ? e - (a + GT) : 0;
    return fwd <= a - b ? -count_below(col, (e < a + GT ? e : a + GT) - a) : 0;
}

template <int CPG>
__device__ int derive_offset(const DispatchParams &p, int64_t a, const uint64_t (&col)[CPG], int lane,
                             bool other = false) {
    constexpr int64_t GT = CPG * kChunk;
    const int64_t c = a / p.Tc;
    const int64_t b = c * p.Tc;
    const int64_t e = b + p.Tc < p.T ? b + p.Tc : p.T;
    const int64_t back = a - b;
    const int64_t fwd = e > a + GT ? e - (a + GT) : 0;
    int v = 0;
    if ((fwd <= back) != other) {
        if (lane < p.R) v = p.gbl[(int64_t)lane * p.C + c];
        v -= count_below(col, (e < a + GT ? e : a + GT) - a);
        if (fwd > 0) v -= count_tokens(p, a + GT, e, lane);
    } else {
        if (lane < p.R && c > 0) v = p.gbl[(int64_t)lane * p.C + c - 1];
        v += count_tokens(p, b, a, lane);
    }
    return v;
}

// The routing inputs checked against a group's columns by one wave per group
// (lane r: off0 = the group's offset inside slab r, alt = the same offset read a
// second, independent way, slab0 = the slab start).  True when one disagrees:
//  - off0 != alt;
//  - a channel start in [a, a + GT] before the last token not at off0 plus the
//    group's tokens before it (prefix entry c-1);
//  - in the group holding the last token: a channel total from the last token's
//    channel on, or a slab size, not the group's offset plus its tokens.
// Over all groups this checks every entry the rows depend on.
template <int CPG>
__device__ bool anchors_disagree(const DispatchParams &p, int64_t a, const uint64_t (&col)[CPG], int off0, int alt,
                                 int slab0, int lane) {
    constexpr int64_t GT = CPG * kChunk;
    const bool rk = lane < p.R;
    bool bad = rk && off0 != alt;
    for (int64_t c = (a + p.Tc - 1) / p.Tc; c * p.Tc < p.T && c * p.Tc <= a + GT; ++c) {
        const int want = (rk && c > 0) ? p.gbl[(int64_t)lane * p.C + c - 1] : 0;
        bad |= rk && off0 + count_below(col, c * p.Tc - a) != want;
    }
    if (a + GT >= p.T) {
        const int total = off0 + count_below(col, GT);
        bad |= rk && p.recv_gbl[rk ? lane : 0] - slab0 != total;
        for (int64_t c = (p.T - 1) / p.Tc; c < p.C; ++c) bad |= rk && p.gbl[(int64_t)lane * p.C + c] != total;
    }
    return ballot64(bad) != 0ull;
}

// Per-token scales (fp8 rows) travel beside the rows: lane r holds the row of
// destination r (or -1), `dests` has bit r set for every routed destination.
__device__ __forceinline__ void copy_scales(const DispatchParams &p, int64_t t, int slot, uint64_t dests, int lane) {
    if (p.num_scales <= 0) return;
    for (int i0 = 0; i0 < p.num_scales; i0 += kWave) {
        const int i = i0 + lane;
        const float sc = i < p.num_scales ? p.x_scales[t * p.num_scales + i] : 0.0f;
        for (uint64_t dd = dests; dd != 0ull; dd &= dd - 1ull) {
            const int64_t s = readlane32(slot, __builtin_ctzll(dd));
            if (i < p.num_scales) p.recv_scales[s * p.num_scales + i] = sc;
        }
    }
}

// send_slot of token t and the metadata (a4) of its rows: weights / local ids
// of the topk slots living on each destination (lane j < k holds slot j's
// expert id e and weight wt) and {my_rank, t} as the row's source.  With
// slot_pos (dispatch straight into the grouped layout), lane j's grouped
// position `pos` (or -1) goes to the row of slot j's rank, -1 to the others.
__device__ __forceinline__ void token_metadata(const DispatchParams &p, int64_t t, int slot, uint64_t dests,
                                               int64_t e, float wt, int lane, int32_t *slot_pos = nullptr,
                                               int pos = -1) {
    if (lane < p.R) p.send_slot[t * p.R + lane] = slot;
    const int erank = (e >= 0 && e < p.E) ? (int)e / p.experts_per_rank : -1;
    for (uint64_t dd = dests; dd != 0ull; dd &= dd - 1ull) {
        const int r = __builtin_ctzll(dd);
        const int64_t s = readlane32(slot, r);
        if (lane < p.K) {
            const bool on = erank == r;
            p.recv_w[s * p.K + lane] = on ? wt : 0.0f;
            if (p.recv_idx != nullptr) p.recv_idx[s * p.K + lane] = on ? e - (int64_t)r * p.experts_per_rank : -1;
            if (slot_pos != nullptr) slot_pos[s * p.K + lane] = on ? pos : -1;
        }
        if (lane == 0) reinterpret_cast<int2 *>(p.src_info)[s] = make_int2(p.my_rank, (int)t);
    }
}

// GRAN > 0: the block's waves sweep the destination ranks in order and meet at
// a barrier every GRAN ranks, so the blocks' concurrent stores gather in a few
// slabs instead of spreading over all of them.  GRAN == 0: free-running waves.
// CACHED: the rows come from send_slot of an earlier dispatch with the same
// routing (p.cached_slot); no routing, metadata or send_slot output.
// QUANT: x is bf16 and each row leaves as E4M3 codes plus its scales (the
// quantiser of ep_quantize_fp8, run once per token segment before the stores).
// Units are then those of the fp8 row: lane i of slice j owns 16 channels, two
// 16-byte loads of x and one 16-byte store per destination; a scale group is
// 1 << quant_log2 aligned lanes, and its first lane stores the group's scale.
template <int VPL, bool EXACT, int WPB, int GRAN, bool CACHED, bool QUANT = false>
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
    u32x4 v[VPL > 0 ? VPL : 1];  // VPL == 0: metadata only, no row
    u32x4 vh[QUANT ? VPL : 1];   // QUANT: channels 8-15 of the lane's 16 (v holds 0-7)
    if constexpr (QUANT) {
        const u32x4 *src = p.x + 2 * (t * p.row_units + c0);  // two bf16 units per fp8 unit
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            if (EXACT || c0 + i * kWave < p.row_units) {
                v[i] = __builtin_nontemporal_load(src + 2 * i * kWave);
                vh[i] = __builtin_nontemporal_load(src + 2 * i * kWave + 1);
            } else {
                v[i] = vh[i] = zero;  // past the row: whole groups of zeros, never stored
            }
        }
    } else {
        const u32x4 *src = p.x + t * p.row_units + c0;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (EXACT || c0 + i * kWave < p.row_units) v[i] = __builtin_nontemporal_load(src + i * kWave);
    }

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
        const int64_t a = q * kChunk;
        const uint64_t m = token_mask(p, a + lane, p.derive);
        const int slab0 = (lane < R && lane > 0) ? p.recv_gbl[lane - 1] : 0;
        int off = 0;  // lane r: the chunk's offset inside slab r
        uint64_t colq[1] = {0ull};
        if (p.derive) {
            colq[0] = transpose64(m);
            off = derive_offset<1>(p, a, colq, lane);
        } else if (lane < R) {
            off = p.rank_base[(q / kGroupChunks) * R + lane] + p.rank_off[q * R + lane];
        }
        const int base = lane < R ? slab0 + off : 0;
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
        const bool routed = lane < R && ((mine >> lane) & 1ull);
        const bool over = routed && (slot < 0 || slot >= p.cap);  // a negative row only from bad prefixes
        if (over) slot = -1;
        if (live && seg == 0) {
            if (ballot64(over) != 0ull && lane == 0) flag(p.dev_status, EP_DEV_RECV_OVERFLOW);
            // the workspace's mask must be this token's is_token_in_rank row
            if (!p.derive) {
                const bool want = lane < R && p.in_rank[t * R + lane] != 0;
                if (ballot64(want != routed) != 0ull && lane == 0) flag(p.dev_status, EP_DEV_STALE_WORKSPACE);
            }
            // the first token's wave checks the chunk against the prefix matrix
            if (my == 0) {
                if (!p.derive) colq[0] = transpose64(m);
                const int alt = derive_offset<1>(p, a, colq, lane, p.derive);
                if (anchors_disagree<1>(p, a, colq, off, alt, slab0, lane) && lane == 0)
                    flag(p.dev_status, EP_DEV_COUNT_MISMATCH);
            }
        }
    }
    if (!live) slot = -1;
    const uint64_t dests = ballot64(slot >= 0);

    if (!QUANT && live && seg == 0) copy_scales(p, t, slot, dests, lane);
    if (!CACHED && live && seg == 0) token_metadata(p, t, slot, dests, e, wt, lane);

    if (VPL == 0) return;  // metadata only
    // ---- QUANT: the segment's codes (in v) and its groups' scales, once for every destination
    float qs[QUANT ? VPL : 1];
    if constexpr (QUANT) {
#pragma unroll
        for (int i = 0; i < VPL; ++i) v[i] = e4m3_quantize16(v[i], vh[i], p.quant_log2, &qs[i]);
    }
    const bool qlead = QUANT && (lane & ((1 << p.quant_log2) - 1)) == 0;
    // ---- row copy (a4): the segment to every destination, ranks ascending
    auto store_to = [&](uint64_t dd) {
        for (; dd != 0ull; dd &= dd - 1ull) {
            const int r = __builtin_ctzll(dd);
            const int64_t s = readlane32(slot, r);
            u32x4 *dst = p.recv_x + s * p.row_units + c0;
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                if (EXACT || c0 + i * kWave < p.row_units) __builtin_nontemporal_store(v[i], dst + i * kWave);
            if constexpr (QUANT) {
                float *ds = p.recv_scales + s * p.num_scales;
#pragma unroll
                for (int i = 0; i < VPL; ++i)
                    if (qlead && (EXACT || c0 + i * kWave < p.row_units)) ds[(c0 + i * kWave) >> p.quant_log2] = qs[i];
            }
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

// Position of the n-th (from 0) set bit of x, for n < popcount(x): a binary
// search on the popcounts of halves.  With wave-uniform arguments it runs on
// the scalar unit and leaves no vector register behind.
// (Integer steps only: a bool here would be widened through a vector register.)
__device__ __forceinline__ int nth_set_bit(uint64_t x, int n) {
    int pos = 0;
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) {
        const int c = __popcll(x & ((1ull << w) - 1ull));
        const int take = (int)((uint32_t)(c - 1 - n) >> 31);  // 1 when n >= c
        n -= take * c;
        x >>= take * w;
        pos += take * w;
    }
    return pos;
}

// XCDs of the MI355X.  Consecutive workgroup ids are placed round-robin over
// them, and each XCD has its own L2, so blocks with the same id modulo 8 share
// one L2.  A different placement changes only the speed, never the result.
constexpr int kXcds = 8;
constexpr int64_t kMaxPullRowUnits = 1 << 16;  // 1 MiB rows

// Pull form (many tokens): the rows are produced in receive order instead of
// token order.  Tokens are taken in groups of CPG 64-token chunks; XCD j owns
// groups j, j+8, ...  A group's rows for rank r are contiguous in slab r
// (`rank_off` gives where they start and how many there are), so the group's
// output is R runs of rows, ranks ascending.  The XCD's waves cut it into
// tasks of U 1 KiB pieces (a piece is 64 lanes x 16 bytes) and take task k,
// k+W, k+2W, ... (W = the XCD's wave count): at any moment the XCD writes one
// narrow, advancing window, like a fill.  Every task reads its token's x with
// ordinary loads; a token has ~R*(1-(1-1/R)^k) rows, and all but the first
// read hit the group's x in the XCD's L2.  Before its tasks, each group's GT
// token tasks (send_slot, metadata, scales) go to GT of the XCD's waves, a
// different set for each group.  Without a workspace (DERIVE) the group's
// columns come from is_token_in_rank rows: waves 0..CPG-1 of each block build
// one chunk's columns each and wave CPG the part of the group's offsets that
// lies outside it (prefix entry and count to the channel edge); one barrier,
// and every wave of the block reads them from LDS (double-buffered by group).
template <int CPG, int U, bool EXACT, int WPB, bool DERIVE>
__global__ __launch_bounds__(WPB *kWave) void dispatch_pull_kernel(DispatchParams p) {
    constexpr int GT = CPG * kChunk;  // tokens per group
    __shared__ uint64_t s_col[2][CPG][kWave];
    __shared__ int s_outer[2][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int xcd = (int)(blockIdx.x % kXcds);
    const int wib = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // wave in block
    const int64_t G = (num_chunks(p.T) + CPG - 1) / CPG;
    const int W = (int)(gridDim.x / kXcds) * WPB;  // waves per XCD; the grid is a multiple of kXcds
    // wave index inside the XCD, made visibly wave-uniform so that the piece
    // arithmetic below stays on the scalar unit
    const int wx = (int)(blockIdx.x / kXcds) * WPB + wib;
    const int R = p.R;
    int par = 0;
    const int TPR = (int)((p.row_units + U * kWave - 1) / (U * kWave));  // tasks per row

    for (int64_t g = xcd; g < G; g += kXcds) {
        const int64_t q0 = g * CPG;  // first chunk of the group
        // The group's GT token tasks (send_slot, metadata, scales) go to waves
        // kt = 0..GT-1, counted from an offset that moves on by GT every group so
        // that they spread evenly over the XCD's waves.  A wave's first token's
        // ids, weights and chunk offsets are loaded here, together with the
        // group's masks, so its token task does not wait on memory later.
        const int rot = (int)(((g / kXcds) * GT) % W);
        const int kt = wx >= rot ? wx - rot : wx - rot + W;
        const int64_t a = q0 * kChunk;  // the group's first token
        const int64_t t1 = a + kt;
        const bool tok1 = kt < GT && t1 < p.T;
        int64_t e1 = -1;
        float w1 = 0.0f;
        bool in1 = false;  // the first token's is_token_in_rank byte (lane r), checked against the workspace
        if (tok1) {
            if (lane < p.K) {
                e1 = p.topk_idx[t1 * p.K + lane];
                w1 = p.topk_w[t1 * p.K + lane];
            }
            if (!DERIVE && lane < R) in1 = p.in_rank[t1 * R + lane] != 0;
        }
        const int slab0 = (lane < R && lane > 0) ? p.recv_gbl[lane - 1] : 0;
        int off0 = 0;  // lane r: the group's offset inside slab r
        if (!DERIVE && lane < R) off0 = p.rank_base[(q0 / kGroupChunks) * R + lane] + p.rank_off[q0 * R + lane];
        // lane r: bit l of col[c] set when token (q0 + c)*64 + l goes to rank r
        uint64_t col[CPG];
        int n = 0;
        if (DERIVE) {
            // waves 0..CPG-1 build one chunk's columns each, wave CPG the part of
            // the offset outside the group; the block's waves read both from LDS
            if (wib < CPG) s_col[par][wib][lane] = transpose64(token_mask(p, a + wib * kChunk + lane, true));
            if (wib == CPG) s_outer[par][lane] = derive_outer<CPG>(p, a, lane);
            __syncthreads();
#pragma unroll
            for (int c = 0; c < CPG; ++c) col[c] = s_col[par][c][lane];
            off0 = s_outer[par][lane] + derive_inner<CPG>(p, a, col);
            par ^= 1;
        } else {
#pragma unroll
            for (int c = 0; c < CPG; ++c) col[c] = transpose64(token_mask(p, a + c * kChunk + lane, DERIVE));
        }
#pragma unroll
        for (int c = 0; c < CPG; ++c) n += __popcll(col[c]);  // 0 on lanes >= R
        // the group's rows on rank r: [s0, s0 + n) in slab r, run r of the
        // group's output starting at pex; chunk c's rows start at cb[c]
        const int s0 = lane < R ? slab0 + off0 : 0;
        int cb[CPG];
        {
            int run = s0;
#pragma unroll
            for (int c = 0; c < CPG; ++c) {
                cb[c] = run;
                run += __popcll(col[c]);
            }
        }
        const int incl = wave_inclusive_scan(n);
        const int pex = lane < R ? incl - n : INT32_MAX;
        const int rows = readlane32(incl, kWave - 1);
        // one wave per group checks the offsets against the prefix matrix: the
        // derived offset against the other side of its channel, the workspace's
        // against the derived one
        if (kt == 0) {
            const int alt = derive_offset<CPG>(p, a, col, lane, DERIVE);
            if (anchors_disagree<CPG>(p, a, col, off0, alt, slab0, lane) && lane == 0)
                flag(p.dev_status, EP_DEV_COUNT_MISMATCH);
        }

        // ---- token tasks: send_slot, metadata, scales (more than one per wave
        // only when the XCD has fewer than GT waves)
        for (int k = kt; k < GT; k += W) {
            const int64_t t = a + k;
            if (t >= p.T) break;  // wave-uniform; later k are larger
            const int c = k / kChunk, l = k - c * kChunk;
            uint64_t cc = col[0];
            int base = cb[0];
#pragma unroll
            for (int c2 = 1; c2 < CPG; ++c2) {
                if (c == c2) {
                    cc = col[c2];
                    base = cb[c2];
                }
            }
            int64_t e = e1;
            float wt = w1;
            bool in = in1;
            if (k != kt) {
                e = -1;
                wt = 0.0f;
                if (lane < p.K) {
                    e = p.topk_idx[t * p.K + lane];
                    wt = p.topk_w[t * p.K + lane];
                }
                if (!DERIVE && lane < R) in = p.in_rank[t * R + lane] != 0;
            }
            const bool routed = lane < R && ((cc >> l) & 1ull);
            // the workspace's mask must be this token's is_token_in_rank row
            if (!DERIVE && ballot64(in != routed) != 0ull && lane == 0) flag(p.dev_status, EP_DEV_STALE_WORKSPACE);
            int slot = -1;
            if (routed) slot = base + __popcll(cc & ((1ull << l) - 1ull));
            const bool over = routed && (slot < 0 || slot >= p.cap);  // a negative row only from bad prefixes
            if (over) slot = -1;
            if (ballot64(over) != 0ull && lane == 0) flag(p.dev_status, EP_DEV_RECV_OVERFLOW);
            const uint64_t dests = ballot64(slot >= 0);
            copy_scales(p, t, slot, dests, lane);
            token_metadata(p, t, slot, dests, e, wt, lane);
        }

        // ---- the group's rows in receive order.  A task is U consecutive
        // pieces of one row (TPR tasks per row); the XCD's waves take tasks
        // wx, wx+W, ... so its concurrent stores cover W*U KiB of consecutive
        // output.  The routing is resolved once per task, and the task's row and
        // part advance by a fixed step instead of a division per task.
        // (rows * TPR < 2^31: at most 64*CPG*R rows, and the pull form is used
        // for rows of at most kMaxPullRowUnits units.)
        const int tasks = rows * TPR;
        // The wave's tasks are k = wx + n*W, n = 0, 1, ...  They are routed 64 at
        // a time, lane i taking task n = base + i on the vector unit: the row of
        // the group's output and the part of it (rr, part), the rank (a binary
        // search over the run starts), the row in the slab and the token (the
        // o-th set bit of the rank's column).  The task loop then reads them
        // back with two readlanes, so each task costs the scalar unit little
        // more than its address arithmetic.
        for (int base = 0; wx + base * W < tasks; base += kWave) {
            int rt_row, rt_pack;  // lane i: task base + i: slab row; token | part << 8 | ok << 30
            {
                const int n = base + lane;
                const int kk = wx + n * W;
                const bool valid = kk < tasks;
                const int k = valid ? kk : wx + base * W;
                const int rr = k / TPR, part = k - rr * TPR;
                int r = 0;
#pragma unroll
                for (int step = 32; step >= 1; step >>= 1) {
                    const int cand = r + step;
                    if (__shfl(pex, cand, kWave) <= rr) r = cand;
                }
                const int o = rr - __shfl(pex, r, kWave);
                const int row = __shfl(s0, r, kWave) + o;
                uint64_t cc = 0;
                int c = 0, oc = o;
#pragma unroll
                for (int c2 = 0; c2 < CPG; ++c2) {
                    const uint32_t lo = __shfl((unsigned)(uint32_t)col[c2], r, kWave);
                    const uint32_t hi = __shfl((unsigned)(uint32_t)(col[c2] >> 32), r, kWave);
                    const uint64_t cq = ((uint64_t)hi << 32) | lo;
                    if (c2 == 0) {
                        cc = cq;
                    } else {
                        const int pc = __popcll(cc);
                        if (c == c2 - 1 && oc >= pc) {
                            oc -= pc;
                            c = c2;
                            cc = cq;
                        }
                    }
                }
                // o < the run's length by construction; checked, so that a bad
                // offset can only drop the row, never pick a token past t
                const bool found = (unsigned)oc < __popcll(cc);
                const int tok = found ? c * kChunk + nth_set_bit(cc, oc) : 0;
                const bool ok = valid && found && row >= 0 && row < p.cap;  // rows past the capacity: dropped
                rt_row = ok ? row : 0;
                rt_pack = tok | (part << 8) | ((int)ok << 30);
            }
            const int nb = (tasks - wx - base * W + W - 1) / W;  // tasks of this batch
            const int nbatch = nb < kWave ? nb : kWave;
            for (int j = 0; j < nbatch; ++j) {
                // the task's U loads are issued, then its U stores; lanes past a
                // ragged row end still load (from a valid place) so that no branch
                // sits between the loads, and only their stores are skipped.
                // Addresses are a wave-uniform base plus the fixed per-lane offset.
                // (Two tasks per pass measured slower.)
                const int pk = readlane32(rt_pack, j);
                const int row = readlane32(rt_row, j);
                const bool ok = (pk >> 30) != 0;
                const int64_t t = q0 * kChunk + (pk & 0xff);
                const int64_t first = (int64_t)((pk >> 8) & 0x3fffff) * U * kWave;
                const int lim = (int)(p.row_units - first);
                const u32x4 *src = p.x + t * p.row_units + first;
                u32x4 *dst = p.recv_x + (int64_t)row * p.row_units + first;
                u32x4 v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int cu = u * kWave + lane;
                    v[u] = src[(EXACT || cu < lim) ? cu : lim - 1];
                }
                // keeps the compiler from moving a load into its store's branch (a
                // load there would be waited for before the next one is issued)
                asm volatile("" ::: "memory");
                if (ok) {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int cu = u * kWave + lane;
                        if (EXACT || cu < lim) __builtin_nontemporal_store(v[u], dst + cu);
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------- straight into the grouped layout
// Dispatch straight into the grouped layout of ep_group.hip, pull form (from
// 2048 tokens), in one launch.  A slab's rows follow their tokens, so in
// (token, slot) order an entry's place inside its expert's segment is the
// number of entries of that expert in earlier (token, slot) pairs: no pass in
// receive order is needed.  Tokens go in groups of kGpTokens (two chunks); XCD
// j owns groups j, j+8, ... as in the receive dispatch's pull form.  Every
// block keeps per expert the received entries of all tokens before its current
// group (counted by itself from topk_idx: the groups before its first, then
// the seven groups between two of its own, their ids loaded at a group's start
// and counted before its copies, or after them with more than 8 slots a token),
// and ranks the current group's entries stably
// per expert: a wave finds the lanes sharing its id with one ballot per id bit,
// the waves' counts go to a byte table (expert x wave) and each entry adds
// those of the waves before it.  The group's counts are scanned over the
// experts (by every wave at once up to 512 experts, so that only two barriers
// sit in the ranking).  With the segment starts that gives every entry's
// position.  Loads whose values are used after a group's copies would wait for
// all of the wave's stores (one counter covers both), so everything the next
// group needs from memory is loaded at the start of a group and resolved
// before its copies.
// Then, per group: its token tasks (send_slot, receive metadata, slot_pos,
// grouped_row and weights) spread over the XCD's waves; its grouped rows in
// position order (runs expert by expert) as tasks of U 1 KiB pieces over the
// XCD's waves, x read again from the XCD's L2; its scales.  After the last
// group the padding rows, over the whole grid.  Receive rows at or past the
// capacity are the last rows of their slabs, so per rank a token index bounds
// the received tokens; it is found once, and only when rows are dropped.  The
// routing inputs are checked against the workspace as in the receive dispatch,
// once per group, by XCD 0's waves before their first group.
constexpr int kGpTokens = 2 * kChunk;     // tokens per group
constexpr int kGpWaves = 16;              // waves per block
constexpr int kGpThreads = kGpWaves * kWave;
constexpr int kGpBlocksPerXcd = 32;       // one block per CU
constexpr int kGpMaxExperts = 2048;
constexpr int kGpMaxEntries = kGpTokens * kMaxTopk;
constexpr int kGpNoLimit = INT32_MAX;     // token threshold of a rank with no dropped row
constexpr int kGpWaveScanExperts = 512;   // up to this many, every wave scans the group's counts

struct GroupedOut {
    const int32_t *aligned;  // [E] segment sizes (a negative size counts as 0)
    u32x4 *dst;              // [gcap][row]
    float *dst_scales;       // [gcap][num_scales]
    int32_t *grouped_row;    // [gcap]
    float *grouped_w;        // [gcap], or null
    int32_t *slot_pos;       // [cap][k]
    int32_t *num_grouped;    // [1]
    int64_t gcap;
};

// Raw ids of entries tid + n * kGpThreads of the tokens from a, loaded at
// clamped places (no branch around the loads, and nothing uses them yet: a use
// would wait for the wave's earlier stores too); gp_keys makes them keys.
template <int NE>
__device__ __forceinline__ void gp_load_ids(const DispatchParams &p, int64_t a, int tid, int64_t (&raw)[NE]) {
    const int n_ent = kGpTokens * p.K;
    const int64_t e0 = a * p.K, e_end = p.T * p.K;
#pragma unroll
    for (int n = 0; n < NE; ++n) {
        const int i = tid + n * kGpThreads;
        raw[n] = p.topk_idx[i < n_ent && e0 + i < e_end ? e0 + i : 0];
    }
}

// Whether entry (token t, expert id v or -1) has a receive row: t is before its
// rank's threshold when rows are dropped.
__device__ __forceinline__ bool gp_received(const DispatchParams &p, int v, int64_t t, bool drops,
                                            const int *s_thr) {
    if (v < 0) return false;
    return !drops || t < s_thr[v / p.experts_per_rank];
}

// The keys of the group of tokens from a: the expert id of each entry with a
// receive row, else -1 (past the last token, an id naming no expert, a dropped
// row).
template <int NE>
__device__ __forceinline__ void gp_keys(const DispatchParams &p, int64_t a, int tid, const int64_t (&raw)[NE],
                                        bool drops, const int *s_thr, int (&key)[NE]) {
    const int n_ent = kGpTokens * p.K;
    const int64_t e0 = a * p.K, e_end = p.T * p.K;
#pragma unroll
    for (int n = 0; n < NE; ++n) {
        const int i = tid + n * kGpThreads;
        const bool in = i < n_ent && e0 + i < e_end && raw[n] >= 0 && raw[n] < p.E;
        const int v = in ? (int)raw[n] : -1;
        key[n] = gp_received(p, v, a + i / p.K, drops, s_thr) ? v : -1;
    }
}

// The received entries of tokens [t0, t1) added to cnt per expert (LDS atomics).
__device__ void gp_count(const DispatchParams &p, int64_t t0, int64_t t1, int tid, bool drops, const int *s_thr,
                         int *cnt) {
    constexpr int B = 4;
    const int64_t i0 = t0 * p.K, i1 = t1 * p.K;
    for (int64_t i = i0 + tid; i < i1; i += (int64_t)B * kGpThreads) {
        int64_t v[B];
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const int64_t at = i + (int64_t)u * kGpThreads;
            v[u] = p.topk_idx[at < i1 ? at : i0];
        }
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const int64_t at = i + (int64_t)u * kGpThreads;
            const int id = v[u] >= 0 && v[u] < p.E ? (int)v[u] : -1;
            if (at < i1 && gp_received(p, id, at / p.K, drops, s_thr)) atomicAdd(&cnt[id], 1);
        }
    }
}

// First token of rank r (wave-uniform) whose receive row is at or past the
// capacity, or kGpNoLimit: the chunk is found from the workspace's offsets
// (groups of four chunks, then the chunk), the token from the chunk's masks.
__device__ int gp_rank_threshold(const DispatchParams &p, int r, int lane) {
    const int slab0 = r > 0 ? p.recv_gbl[r - 1] : 0;
    const int m = p.cap - slab0;  // receive rows of rank r below the capacity
    if (m >= p.recv_gbl[r] - slab0) return kGpNoLimit;
    if (m <= 0) return 0;
    const int64_t Q = num_chunks(p.T), G4 = num_groups(p.T);
    int64_t g4 = 0;  // the last group of chunks whose rows start at or before row m
    for (int64_t b = 0; b < G4; b += kWave) {
        const int64_t gi = b + lane;
        const int v = p.rank_base[(gi < G4 ? gi : G4 - 1) * p.R + r];
        const uint64_t le = ballot64(gi < G4 && v <= m);
        if (le != 0ull) g4 = b + 63 - __builtin_clzll(le);
        if (le != ~0ull) break;
    }
    const int64_t q = g4 * kGroupChunks + lane;
    const bool qin = lane < kGroupChunks && q < Q;
    const int off = p.rank_base[g4 * p.R + r] + p.rank_off[(qin ? q : g4 * kGroupChunks) * p.R + r];
    const uint64_t lq = ballot64(qin && off <= m);
    const int ql = lq != 0ull ? 63 - __builtin_clzll(lq) : 0;
    const int64_t qs = g4 * kGroupChunks + ql;
    const int k = m - readlane32(off, ql);
    const int64_t tok = qs * kChunk + lane;
    const uint64_t mk = p.mask[tok < p.T ? tok : p.T - 1];
    const uint64_t col = ballot64(tok < p.T && ((mk >> r) & 1ull));
    if (k < 0 || k >= (int)__popcll(col)) {  // only with a workspace that disagrees with itself
        const int64_t end = (qs + 1) * kChunk;
        return (int)(end < p.T ? end : p.T);
    }
    return (int)(qs * kChunk + nth_set_bit(col, k));
}

// Sum of the bytes of v below byte w (w wave-uniform), and of all 16.
__device__ __forceinline__ int bytes_below(u32x4 v, int w) {
    int s = 0;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int nb = w - 4 * d;
        const uint32_t keep = nb >= 4 ? 0xffffffffu : nb <= 0 ? 0u : (1u << (8 * nb)) - 1u;
        s = (int)__builtin_amdgcn_sad_u8(v[d] & keep, 0u, (uint32_t)s);
    }
    return s;
}
__device__ __forceinline__ int bytes_sum(u32x4 v) {
    uint32_t s = 0;
#pragma unroll
    for (int d = 0; d < 4; ++d) s = __builtin_amdgcn_sad_u8(v[d], 0u, s);
    return (int)s;
}

// Exclusive scan of v[0..E) into out over the block (ept consecutive entries a
// thread); returns the total.  Ends with a barrier.
__device__ __forceinline__ int gp_block_scan(const int *v, int *out, int E, int tid, int *s_w32) {
    const int lane = tid & (kWave - 1), wave = tid >> 6;
    const int ept = (E + kGpThreads - 1) / kGpThreads;
    const int e_lo = tid * ept;
    int run = 0;
    for (int i = 0; i < ept; ++i)
        if (e_lo + i < E) run += v[e_lo + i];
    const int incl = wave_inclusive_scan(run);
    if (lane == kWave - 1) s_w32[wave] = incl;
    __syncthreads();
    int before = incl - run, total = 0;
    for (int w = 0; w < kGpWaves; ++w) {
        if (w < wave) before += s_w32[w];
        total += s_w32[w];
    }
    for (int i = 0; i < ept; ++i) {
        if (e_lo + i < E) {
            const int c = v[e_lo + i];
            out[e_lo + i] = before;
            before += c;
        }
    }
    __syncthreads();
    return total;
}

// The group's counts per expert (earlier passes' in s_run plus the byte table's
// rows) into s_run, and their exclusive scan over the experts into s_pre; the
// byte table cleared for the next pass.  Returns the group's total.  Ends with a
// barrier.
__device__ __forceinline__ int gp_counts_scan(u32x4 *s_cnt, int *s_run, int *s_pre, bool add_run, int E, int tid,
                                              int *s_w32) {
    const int lane = tid & (kWave - 1), wave = tid >> 6;
    const int ept = (E + kGpThreads - 1) / kGpThreads;
    const int e_lo = tid * ept;
    int run = 0;
    for (int i = 0; i < ept; ++i) {
        if (e_lo + i < E) {
            const int c = (add_run ? s_run[e_lo + i] : 0) + bytes_sum(s_cnt[e_lo + i]);
            s_run[e_lo + i] = c;
            run += c;
        }
    }
    const int incl = wave_inclusive_scan(run);
    if (lane == kWave - 1) s_w32[wave] = incl;
    __syncthreads();
    for (int e = tid; e < E; e += kGpThreads) s_cnt[e] = u32x4{0u, 0u, 0u, 0u};
    int before = incl - run, total = 0;
    for (int w = 0; w < kGpWaves; ++w) {
        if (w < wave) before += s_w32[w];
        total += s_w32[w];
    }
    for (int i = 0; i < ept; ++i) {
        if (e_lo + i < E) {
            s_pre[e_lo + i] = before;
            before += s_run[e_lo + i];
        }
    }
    __syncthreads();
    return total;
}

// The ids of the NB groups of tokens from t0 (entry tid of each), as expert ids
// or -1, to be counted into s_base (only with one entry a thread).
template <int NB>
__device__ __forceinline__ void gp_load_groups(const DispatchParams &p, int64_t t0, int64_t t1, int tid,
                                               int (&ids)[NB]) {
    const int n_ent = kGpTokens * p.K;
    const int64_t e0 = t0 * p.K, e_end = (t1 < p.T ? t1 : p.T) * p.K;
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const int64_t at = e0 + (int64_t)u * n_ent + tid;
        const bool in = tid < n_ent && at < e_end;
        const int64_t v = p.topk_idx[in ? at : 0];
        ids[u] = in && v >= 0 && v < p.E ? (int)v : -1;
    }
}
template <int NB>
__device__ __forceinline__ void gp_count_groups(const DispatchParams &p, int64_t t0, int tid, const int (&ids)[NB],
                                                bool drops, const int *s_thr, int *cnt) {
    const int n_ent = kGpTokens * p.K;
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const int64_t at = t0 * p.K + (int64_t)u * n_ent + tid;
        if (gp_received(p, ids[u], at / p.K, drops, s_thr)) atomicAdd(&cnt[ids[u]], 1);
    }
}

template <int U, bool EXACT, int NE>
__global__ __launch_bounds__(kGpThreads) void dispatch_grouped_pull_kernel(DispatchParams p, GroupedOut o) {
    constexpr int NT = kGpThreads;
    constexpr int NB = NE == 1 ? kXcds - 1 : 1;  // groups between two of an XCD's (counted from registers)
    __shared__ int s_seg[kGpMaxExperts];    // segment start (clamped to INT32_MAX)
    __shared__ int s_size[kGpMaxExperts];   // segment size
    __shared__ int s_base[kGpMaxExperts];   // received entries in the tokens before the current group
    __shared__ int s_run[kGpMaxExperts];    // the current group's received entries
    __shared__ int s_pre[kGpMaxExperts];    // where the expert's run starts in the group's output
    __shared__ u32x4 s_cnt[kGpMaxExperts];  // byte w: entries of wave w in the current pass
    __shared__ int2 s_list[kGpMaxEntries];  // the group's output: {token in group, position}
    __shared__ int s_epos[kGpMaxEntries];   // each entry's position, or -1
    __shared__ int s_thr[kWave];            // per rank: first token with no receive row
    __shared__ int64_t s_w64[kGpWaves];
    __shared__ int s_w32[kGpWaves];
    uint8_t *s_cnt8 = reinterpret_cast<uint8_t *>(s_cnt);
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const int xcd = (int)(blockIdx.x % kXcds);
    const int W = (int)(gridDim.x / kXcds) * kGpWaves;  // waves per XCD; the grid is a multiple of 8
    const int wx = (int)(blockIdx.x / kXcds) * kGpWaves + __builtin_amdgcn_readfirstlane(wave);
    const int K = p.K, E = p.E, R = p.R;
    const int n_ent = kGpTokens * K;
    const int64_t G = (p.T + kGpTokens - 1) / kGpTokens;
    const int TPR = (int)((p.row_units + U * kWave - 1) / (U * kWave));  // tasks per row
    const int nbits = E > 1 ? 32 - __builtin_clz((unsigned)(E - 1)) : 0;
    const uint64_t lt = (1ull << lane) - 1ull;
    const int rl = lane < R ? lane : R - 1;
    const int slab0 = (lane < R && lane > 0) ? p.recv_gbl[rl - 1 > 0 ? rl - 1 : 0] : 0;  // lane r: slab r's start

    // ---- loads first: the first group's ids and routing, the segment sizes, the
    // ids of the groups before it
    int64_t raw[NE];
    gp_load_ids<NE>(p, (int64_t)(xcd < G ? xcd : 0) * kGpTokens, tid, raw);
    const int ept = (E + NT - 1) / NT;
    const int e_lo = tid * ept;
    int al[2] = {0, 0};  // ept <= 2
#pragma unroll
    for (int i = 0; i < 2; ++i)
        if (i < ept) al[i] = o.aligned[e_lo + i < E ? e_lo + i : 0];
    const int64_t g_first = xcd < G ? xcd : G;
    int pc[NB];
    if (NE == 1) gp_load_groups<NB>(p, 0, g_first * kGpTokens, tid, pc);
    const int n_recv_all = p.recv_gbl[R - 1];

    // ---- segment sizes and starts: a block scan over the experts
    int64_t run = 0;
    for (int i = 0; i < ept; ++i) {
        if (e_lo + i < E) {
            const int sz = al[i] > 0 ? al[i] : 0;
            s_size[e_lo + i] = sz;
            run += sz;
        }
    }
    const int64_t incl = wave_inclusive_scan64(run);
    if (lane == kWave - 1) s_w64[wave] = incl;
    for (int e = tid; e < E; e += NT) {
        s_base[e] = 0;
        s_cnt[e] = u32x4{0u, 0u, 0u, 0u};
    }
    // rows are dropped only when the capacity is below the receive total
    const bool drops = n_recv_all > p.cap;
    for (int r = wave; r < R; r += kGpWaves) {
        const int thr = drops ? gp_rank_threshold(p, r, lane) : kGpNoLimit;
        if (lane == 0) s_thr[r] = thr;
    }
    // slot_pos of the rows past the last slab (capacity slack): in no segment
    {
        int64_t hi = n_recv_all < p.cap ? n_recv_all : p.cap;
        hi = hi > 0 ? hi : 0;
        const int64_t gt = (int64_t)blockIdx.x * NT + tid, GT = (int64_t)gridDim.x * NT;
        for (int64_t i = hi * K + gt; i < (int64_t)p.cap * K; i += GT) o.slot_pos[i] = -1;
    }
    __syncthreads();
    int64_t before = incl - run, total = 0;
    for (int w = 0; w < kGpWaves; ++w) {
        if (w < wave) before += s_w64[w];
        total += s_w64[w];
    }
    for (int i = 0; i < ept; ++i) {
        if (e_lo + i < E) {
            s_seg[e_lo + i] = (int)(before < INT32_MAX ? before : INT32_MAX);
            before += s_size[e_lo + i];
        }
    }
    const int64_t limit = total < o.gcap ? total : o.gcap;
    if (blockIdx.x == 0 && tid == 0) o.num_grouped[0] = (int32_t)(total < INT32_MAX ? total : INT32_MAX);
    // the entries of the tokens before this XCD's first group
    if (NE == 1)
        gp_count_groups<NB>(p, 0, tid, pc, drops, s_thr, s_base);
    else
        gp_count(p, 0, g_first * kGpTokens < p.T ? g_first * kGpTokens : p.T, tid, drops, s_thr, s_base);
    __syncthreads();

    // ---- the routing inputs checked against the workspace, one group a wave of
    // XCD 0 (whose blocks have no tokens to count before their first group)
    if (xcd == 0) {
        for (int64_t g = wx; g < G; g += W) {
            const int64_t a = g * kGpTokens, q0 = g * 2;
            uint64_t col[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) col[c] = transpose64(token_mask(p, a + c * kChunk + lane, false));
            const int off = p.rank_base[(q0 / kGroupChunks) * R + rl] + p.rank_off[q0 * R + rl];
            const int alt = derive_offset<2>(p, a, col, lane, false);
            if (anchors_disagree<2>(p, a, col, off, alt, slab0, lane) && lane == 0)
                flag(p.dev_status, EP_DEV_COUNT_MISMATCH);
        }
    }

    // the first group's keys (the next group's are made during each group, before
    // its copies, from ids loaded at its start)
    int key_c[NE];
    gp_keys<NE>(p, (int64_t)xcd * kGpTokens, tid, raw, drops, s_thr, key_c);

    for (int64_t g = xcd; g < G; g += kXcds) {
        const int64_t a = g * kGpTokens;  // the group's first token
        const bool next = g + kXcds < G;
        int key[NE], rank[NE];
#pragma unroll
        for (int n = 0; n < NE; ++n) {
            key[n] = key_c[n];
            rank[n] = 0;
        }
        // ---- loads issued now and used after the positions, by when this wave's
        // stores of the last group have long completed (a load used right away
        // would wait for them): the next group's ids, and the ids of the groups up
        // to it
        gp_load_ids<NE>(p, (next ? g + kXcds : g) * kGpTokens, tid, raw);
        // (with several entries a thread the ids become keys at once, which keeps
        // registers free for the ranking but waits for the last group's stores)
        if (NE > 1 && next) gp_keys<NE>(p, (g + kXcds) * kGpTokens, tid, raw, drops, s_thr, key_c);
        int ob[NB];
        if (NE == 1) gp_load_groups<NB>(p, a + kGpTokens, a + (int64_t)kXcds * kGpTokens, tid, ob);

        // ---- stable ranks of the group's entries per expert, pass by pass
        int total_g = 0;
        if (NE == 1 && E <= kGpWaveScanExperts) {
            // one pass, few experts: after the byte table is complete every wave
            // works out the group's counts and their exclusive scan over the experts
            // (lane l: experts l, l + 64, ...) and writes the starts, the same values
            // from every wave, so no barrier sits between them and their use
            const int kk = key[0];
            uint64_t peers = ballot64(kk >= 0);
            for (int b = 0; b < nbits; ++b) {
                const bool bit = ((kk >> b) & 1) != 0;
                const uint64_t B = ballot64(bit);
                peers &= bit ? B : ~B;
            }
            const int inw = __popcll(peers & lt);
            if (kk >= 0 && inw == 0) s_cnt8[kk * 16 + wave] = (uint8_t)__popcll(peers);
            __syncthreads();
            for (int e0 = 0; e0 < E; e0 += kWave) {
                const int e = e0 + lane;
                const int c = e < E ? bytes_sum(s_cnt[e]) : 0;
                const int inc = wave_inclusive_scan(c);
                if (e < E) {
                    s_pre[e] = total_g + inc - c;
                    if (wave == 0) s_run[e] = c;
                }
                total_g += readlane32(inc, kWave - 1);
            }
            if (kk >= 0) rank[0] = bytes_below(s_cnt[kk], wave) + inw;
        } else {
#pragma unroll
            for (int n = 0; n < NE; ++n) {
                const int kk = key[n];
                uint64_t peers = ballot64(kk >= 0);
                for (int b = 0; b < nbits; ++b) {
                    const bool bit = ((kk >> b) & 1) != 0;
                    const uint64_t B = ballot64(bit);
                    peers &= bit ? B : ~B;
                }
                const int inw = __popcll(peers & lt);
                if (kk >= 0 && inw == 0) s_cnt8[kk * 16 + wave] = (uint8_t)__popcll(peers);
                __syncthreads();
                if (kk >= 0) rank[n] = (n > 0 ? s_run[kk] : 0) + bytes_below(s_cnt[kk], wave) + inw;
                if (n > 0) __syncthreads();  // s_run is read before it moves on
                if (n + 1 < NE) {
                    for (int e = tid; e < E; e += NT) s_run[e] = (n > 0 ? s_run[e] : 0) + bytes_sum(s_cnt[e]);
                    __syncthreads();
                    for (int e = tid; e < E; e += NT) s_cnt[e] = u32x4{0u, 0u, 0u, 0u};
                    __syncthreads();
                } else {
                    total_g = gp_counts_scan(s_cnt, s_run, s_pre, n > 0, E, tid, s_w32);
                }
            }
        }

        // ---- positions: segment start + entries before the group + rank
        bool over = false;
#pragma unroll
        for (int n = 0; n < NE; ++n) {
            const int i = tid + n * NT;
            if (i < n_ent) {
                const int kk = key[n];
                int at = -1;
                if (kk >= 0) {
                    const int64_t li = (int64_t)s_base[kk] + rank[n];
                    const int64_t pos = (int64_t)s_seg[kk] + li;
                    const bool placed = li < s_size[kk] && pos < limit;
                    if (placed) at = (int)pos;
                    over |= !placed;
                    s_list[s_pre[kk] + rank[n]] = make_int2(placed ? i / K : -1, at);
                }
                s_epos[i] = at;
            }
        }
        if (ballot64(over) != 0ull && lane == 0) flag(p.dev_status, EP_DEV_RECV_OVERFLOW);
        __syncthreads();
        if (NE == 1 && E <= kGpWaveScanExperts)  // every wave is past its last read of the table
            for (int e = tid; e < E; e += NT) s_cnt[e] = u32x4{0u, 0u, 0u, 0u};
        // ---- the next group's keys, from the loads above
        if (NE == 1 && next) gp_keys<NE>(p, (g + kXcds) * kGpTokens, tid, raw, drops, s_thr, key_c);
        // ---- entries before this XCD's next group: this group's, then the groups
        // up to it (s_base is next read after the group's last barrier)
        for (int e = tid; e < E; e += NT)
            if (s_run[e] != 0) atomicAdd(&s_base[e], s_run[e]);
        if (NE == 1) gp_count_groups<NB>(p, a + kGpTokens, tid, ob, drops, s_thr, s_base);

        // ---- token tasks: send_slot, receive metadata, slot_pos, grouped_row and
        // weights (more than one per wave only when the XCD has fewer waves than
        // the group has tokens)
        const int rot = (int)(((g / kXcds) * kGpTokens) % W);
        const int kt = wx >= rot ? wx - rot : wx - rot + W;
        for (int k = kt; k < kGpTokens; k += W) {
            const int64_t t = a + k;
            if (t >= p.T) break;  // wave-uniform; later k are larger
            // the token's chunk: lane r holds rank r's column and where the chunk's
            // rows start in slab r (the group's offset plus the first chunk's rows)
            const int c = k / kChunk, l = k - c * kChunk;
            const uint64_t m0 = token_mask(p, a + lane, false);
            const uint64_t m1 = token_mask(p, a + kChunk + lane, false);
            const int off0 = p.rank_base[((g * 2) / kGroupChunks) * R + rl] + p.rank_off[(g * 2) * R + rl];
            const int jl = lane < K ? lane : K - 1;
            const int64_t e_ld = p.topk_idx[t * K + jl];
            const float w_ld = p.topk_w[t * K + jl];
            const bool in = p.in_rank[t * R + rl] != 0;
            const int pos_ld = s_epos[k * K + jl];
            const int64_t e = lane < K ? e_ld : -1;
            const float wt = lane < K ? w_ld : 0.0f;
            const int pos = lane < K ? pos_ld : -1;
            const uint64_t c0 = transpose64(m0);
            const uint64_t cc = c == 0 ? c0 : transpose64(m1);
            const int base = (lane < R ? slab0 + off0 : 0) + (c == 0 ? 0 : (int)__popcll(c0));
            const bool routed = lane < R && ((cc >> l) & 1ull);
            // the workspace's mask must be this token's is_token_in_rank row
            if (ballot64((lane < R && in) != routed) != 0ull && lane == 0) flag(p.dev_status, EP_DEV_STALE_WORKSPACE);
            int slot = routed ? base + __popcll(cc & ((1ull << l) - 1ull)) : -1;
            const bool drop = routed && (slot < 0 || slot >= p.cap);  // a negative row only from bad prefixes
            if (drop) slot = -1;
            if (ballot64(drop) != 0ull && lane == 0) flag(p.dev_status, EP_DEV_RECV_OVERFLOW);
            const uint64_t dests = ballot64(slot >= 0);
            token_metadata(p, t, slot, dests, e, wt, lane, o.slot_pos, pos);
            // a placed entry's row: the receive row of its rank
            const int er = (e >= 0 && e < E) ? (int)e / p.experts_per_rank : 0;
            const int srow = __shfl(slot, er, kWave);
            if (pos >= 0) {
                o.grouped_row[pos] = srow;
                if (o.grouped_w != nullptr) o.grouped_w[pos] = wt;
            }
        }

        // ---- the group's grouped rows in position order: task k is piece-run
        // (k % TPR) of output entry (k / TPR); the wave's tasks k = wx + n*W are
        // resolved 64 at a time, lane i taking n = base + i, and read back with
        // two readlanes each
        const int tasks = total_g * TPR;
        for (int base = 0; wx + base * W < tasks; base += kWave) {
            int rt_pos, rt_pack;  // lane i: the task's position; token in group | part << 8 | ok << 30
            {
                const int kk = wx + (base + lane) * W;
                const bool valid = kk < tasks;
                const int k = valid ? kk : 0;
                const int ent = k / TPR, part = k - ent * TPR;
                const int2 le = s_list[ent];
                const bool ok = valid && le.x >= 0;
                rt_pos = ok ? le.y : 0;
                rt_pack = (ok ? le.x : 0) | (part << 8) | ((int)ok << 30);
            }
            const int nb = (tasks - wx - base * W + W - 1) / W;  // tasks of this batch
            const int nbatch = nb < kWave ? nb : kWave;
            for (int j = 0; j < nbatch; ++j) {
                // U loads, then U stores; lanes past a ragged row end load from a
                // valid place and skip their store
                const int pk = readlane32(rt_pack, j);
                const int64_t at = readlane32(rt_pos, j);
                const bool ok = (pk >> 30) != 0;
                const int64_t t = a + (pk & 0xff);
                const int part = (pk >> 8) & 0x3fffff;
                const int64_t first = (int64_t)part * U * kWave;
                const int lim = (int)(p.row_units - first);
                const u32x4 *src = p.x + t * p.row_units + first;
                u32x4 *dst = o.dst + at * p.row_units + first;
                u32x4 v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int cu = u * kWave + lane;
                    v[u] = src[(EXACT || cu < lim) ? cu : lim - 1];
                }
                asm volatile("" ::: "memory");
                if (ok) {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int cu = u * kWave + lane;
                        if (EXACT || cu < lim) __builtin_nontemporal_store(v[u], dst + cu);
                    }
                }
            }
        }
        // ---- the scales: output entry e = wx, wx + W, ..., lanes over the token's
        // scales (a wave-uniform loop with a per-lane predicate)
        if (p.num_scales > 0) {
            for (int e = wx; e < total_g; e += W) {
                const int2 le = s_list[e];
                const int tl = __builtin_amdgcn_readfirstlane(le.x);
                const int64_t at = __builtin_amdgcn_readfirstlane(le.y);
                if (tl < 0) continue;  // wave-uniform
                const int64_t t = a + tl;
                for (int i0 = 0; i0 < p.num_scales; i0 += kWave) {
                    const int i = i0 + lane;
                    const float sc = i < p.num_scales ? p.x_scales[t * p.num_scales + i] : 0.0f;
                    if (i < p.num_scales) o.dst_scales[at * p.num_scales + i] = sc;
                }
            }
        }
        if (NE != 1) {
            const int64_t t1 = a + (int64_t)kXcds * kGpTokens;
            gp_count(p, a + kGpTokens, t1 < p.T ? t1 : p.T, tid, drops, s_thr, s_base);
        }
        __syncthreads();  // every wave is done with the group's tables before they are rebuilt
    }

    // ---- padding: positions [start + placed, start + size) of every segment below
    // the limit (every block holds the same counts now), over the grid's waves
    for (int e = tid; e < E; e += NT) {
        const int64_t st = s_seg[e], sz = s_size[e];
        const int64_t used = s_base[e] < sz ? s_base[e] : sz;
        const int64_t end = st + sz < limit ? st + sz : limit;
        const int64_t n = end - (st + used);
        s_run[e] = n > 0 ? (int)n : 0;
    }
    __syncthreads();
    const int P = gp_block_scan(s_run, s_pre, E, tid, s_w32);
    const int64_t gw = (int64_t)blockIdx.x * kGpWaves + wave, GW = (int64_t)gridDim.x * kGpWaves;
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t b0 = gw * kWave; b0 < P; b0 += GW * kWave) {
        // lane i: padding row b0 + i -- its expert (the last with s_pre <= it) and position
        const int64_t k = b0 + lane;
        int lo = 0, hi = E - 1;
        while (lo < hi) {  // per-lane binary search; at most 11 steps
            const int mid = (lo + hi + 1) >> 1;
            if (s_pre[mid] <= k) lo = mid; else hi = mid - 1;
        }
        const int64_t st = s_seg[lo], sz = s_size[lo];
        const int64_t used = s_base[lo] < sz ? s_base[lo] : sz;
        const int pos = (int)(st + used + (k - s_pre[lo]));
        if (k < P) {
            o.grouped_row[pos] = -1;
            if (o.grouped_w != nullptr) o.grouped_w[pos] = 0.0f;
        }
        const int64_t nb = P - b0 < kWave ? P - b0 : kWave;
        for (int j = 0; j < nb; ++j) {
            const int64_t at = readlane32(pos, j);
            u32x4 *d = o.dst + at * p.row_units;
            for (int64_t u = lane; u < p.row_units; u += kWave) __builtin_nontemporal_store(z, d + u);
            for (int i0 = 0; i0 < p.num_scales; i0 += kWave)  // wave-uniform, per-lane predicate
                if (i0 + lane < p.num_scales) o.dst_scales[at * p.num_scales + i0 + lane] = 0.0f;
        }
    }
}

template <int CPG, int U, bool EXACT, int WPB>
hipError_t run_pull(DispatchParams p, int blocks_per_xcd, hipStream_t stream) {
    const dim3 grid((unsigned)(kXcds * blocks_per_xcd)), block(WPB * kWave);
    if (p.derive)
        hipLaunchKernelGGL((dispatch_pull_kernel<CPG, U, EXACT, WPB, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((dispatch_pull_kernel<CPG, U, EXACT, WPB, false>), grid, block, 0, stream, p);
    return hipGetLastError();
}

template <int VPL, bool EXACT, int WPB, int GRAN, bool QUANT = false>
hipError_t run(DispatchParams p, hipStream_t stream) {
    p.S = (int)((p.row_units + VPL * kWave - 1) / (VPL * kWave));
    const int64_t waves = p.T * p.S;
    const int64_t blocks = (waves + WPB - 1) / WPB;
    if constexpr (QUANT) {
        if (p.cached_slot != nullptr)
            hipLaunchKernelGGL((dispatch_kernel<VPL, EXACT, WPB, GRAN, true, true>), dim3((unsigned)blocks),
                               dim3(WPB * kWave), 0, stream, p);
        else
            hipLaunchKernelGGL((dispatch_kernel<VPL, EXACT, WPB, GRAN, false, true>), dim3((unsigned)blocks),
                               dim3(WPB * kWave), 0, stream, p);
    } else if (p.cached_slot != nullptr)
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

// Push-form tiling (cached mode at any size, and fewer than 2048 tokens
// otherwise).  Measured on MI355X (rows of 7168 bf16 or fp8 elements at
// 128..4096 tokens, and the skew / large workloads).  Whole rows per wave with the rank sweep
// (16 waves per block, a barrier every 4 ranks) win once there are enough
// tokens to give every compute unit a block; below that the rows are split so
// more waves share the copy.  Other widths: 1 KiB segments, 8 waves per block.
// Pull-form tiling: chunks per token group (cpg), pieces per task (u), waves
// per block (wpb) and blocks per XCD (bpx); cpg == 0 selects the push form.
struct PullTiling {
    int cpg, u, wpb, bpx;
};

hipError_t run_pull_tiled(const DispatchParams &p, const PullTiling &t, hipStream_t stream) {
    const bool exact = p.row_units % ((int64_t)t.u * kWave) == 0;
#define EP_PULL_CASE(C, U, W) \
    if (t.cpg == C && t.u == U && t.wpb == W) \
        return exact ? run_pull<C, U, true, W>(p, t.bpx, stream) : run_pull<C, U, false, W>(p, t.bpx, stream);
    EP_PULL_CASE(2, 1, 8)
    EP_PULL_CASE(2, 2, 8)
    EP_PULL_CASE(2, 4, 8)
    EP_PULL_CASE(2, 8, 8)
#undef EP_PULL_CASE
    return hipErrorInvalidValue;
}

// Measured on MI355X (7168-element bf16 and fp8 rows at 1024..4096 tokens, and
// 4096-element rows at 16384 tokens): from 2048 tokens (16 groups of 128, two
// per XCD) the pull form is 9-20% faster than the push form; below that, and
// for rows under 1 KiB, the push form is kept.  Groups of 128 tokens (1.8 MiB of
// 7168-element bf16 rows) sit well inside an XCD's 4 MiB L2.  Tasks: one piece
// for rows of 14 KiB and more (two tasks per pass, or more pieces per task,
// measured slower); two pieces for rows of 7 to 14 KiB (as fast as one piece
// with x in cache, and 12-15% faster than one piece when x has to come from
// memory); the whole row (4 or 8 pieces) for shorter rows.  64 blocks of 8
// waves per XCD: 16 waves per CU.
PullTiling pull_tiling(int64_t row_units, int64_t num_tokens) {
    if (row_units < kWave || row_units > kMaxPullRowUnits || num_tokens < 2048) return PullTiling{0, 0, 0, 0};
    const int u = row_units >= 14 * kWave ? 1 : row_units >= 7 * kWave ? 2 : row_units > 4 * kWave ? 8 : 4;
    return PullTiling{2, u, 8, 64};
}

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

// The quantising dispatch (push form; also its cached mode).  For 7168 channels from 4096 tokens whole rows
// per wave, 4 free-running waves per block: 56.8 us at prefill, against 59.3-60.6 with
// the rank sweep of the fp8 rows (16 waves, a barrier every 4 ranks), 57.0-57.5 with 8
// or 16 free-running waves, 58.0-61.8 with the row split over 2, 4 or 7 waves (one run).
// Its cached mode, which has no routing to do before its stores, takes the rank sweep:
// 52.5-53.4 us against 56.7-58.4 free-running (53.8-54.5 with a barrier every rank).
// Below 4096 tokens 4096-channel segments; other widths 1024-channel segments, 8 waves.
hipError_t run_quant_tiled(const DispatchParams &p, hipStream_t stream) {
    if (p.row_units == 7 * kWave && p.T >= 4096)
        return p.cached_slot != nullptr ? run<7, true, 16, 4, true>(p, stream) : run<7, true, 4, 0, true>(p, stream);
    if (p.row_units == 7 * kWave) return run<4, false, 4, 0, true>(p, stream);
    return p.row_units % kWave == 0 ? run<1, true, 8, 0, true>(p, stream) : run<1, false, 8, 0, true>(p, stream);
}

template <int U, bool EXACT, int NE>
hipError_t run_grouped_pull(const DispatchParams &p, const GroupedOut &o, hipStream_t stream) {
    hipLaunchKernelGGL((dispatch_grouped_pull_kernel<U, EXACT, NE>), dim3((unsigned)(kXcds * kGpBlocksPerXcd)),
                       dim3(kGpThreads), 0, stream, p, o);
    return hipGetLastError();
}

// Pieces per task as for the receive dispatch's pull form: 1 for rows of 14 KiB
// and more, 2 from 7 KiB, else 4 (2 with more than 8 slots a token), so that
// the 1024-thread blocks keep to 128 registers with nothing spilled.
template <int NE>
hipError_t run_grouped_pull_tiled(const DispatchParams &p, const GroupedOut &o, hipStream_t stream) {
    const int64_t ru = p.row_units;
    const int u = ru >= 14 * kWave ? 1 : ru >= 7 * kWave || NE > 1 ? 2 : 4;
    const bool exact = ru % (u * kWave) == 0;
#define EP_GP_CASE(UU) \
    if (u == UU) return exact ? run_grouped_pull<UU, true, NE>(p, o, stream) : run_grouped_pull<UU, false, NE>(p, o, stream);
    EP_GP_CASE(1)
    EP_GP_CASE(2)
    if constexpr (NE == 1) {
        EP_GP_CASE(4)
    }
#undef EP_GP_CASE
    return hipErrorInvalidValue;
}

DispatchParams make_params(const ep_shape_t &s, const DispatchArgs &a) {
    DispatchParams p;
    p.x = reinterpret_cast<const u32x4 *>(a.x);
    p.x_scales = a.x_scales;
    p.topk_idx = a.topk_idx;
    p.topk_w = a.topk_w;
    p.in_rank = a.in_rank;
    p.gbl = a.gbl;
    p.recv_gbl = a.recv_gbl;
    p.mask = nullptr;
    p.rank_off = p.rank_base = nullptr;
    p.derive = a.ws == nullptr;
    if (a.ws != nullptr) {
        const Workspace w = workspace_layout(s.num_tokens, s.num_ranks, s.num_experts, s.num_channels, s.num_topk);
        p.mask = reinterpret_cast<const uint64_t *>(a.ws + w.mask);
        p.rank_off = reinterpret_cast<const int32_t *>(a.ws + w.rank_off);
        p.rank_base = reinterpret_cast<const int32_t *>(a.ws + w.rank_base);
    }
    p.C = s.num_channels;
    p.Tc = ((int64_t)s.num_tokens + p.C - 1) / p.C;
    {
        const uintptr_t ia = reinterpret_cast<uintptr_t>(a.in_rank);
        const int R = s.num_ranks;
        p.in_unit = (R % 16 == 0 && ia % 16 == 0) ? 16 : (R % 8 == 0 && ia % 8 == 0) ? 8 : 1;
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
    p.quant_log2 = a.quantize ? a.quant_log2 : 0;
    p.S = 1;
    return p;
}

}  // namespace

// Metadata only (no receive rows): send_slot, weights, local ids, src_info,
// one wave per token.
hipError_t run_meta(DispatchParams p, hipStream_t stream) {
    p.S = 1;
    const int64_t blocks = (p.T + 7) / 8;
    hipLaunchKernelGGL((dispatch_kernel<0, true, 8, 0, false>), dim3((unsigned)blocks), dim3(8 * kWave), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_dispatch(const ep_shape_t &s, const DispatchArgs &a, hipStream_t stream) {
    if (s.num_tokens == 0) return hipSuccess;
    DispatchParams p = make_params(s, a);
    if (p.recv_x == nullptr && p.cached_slot == nullptr) {
        p.num_scales = 0;  // no rows, so no scales beside them
        return run_meta(p, stream);
    }
    if (a.quantize) return run_quant_tiled(p, stream);
    // cached mode always takes the push form
    if (a.form != EP_FORM_PUSH && p.cached_slot == nullptr) {
        const PullTiling pt = pull_tiling(p.row_units, p.T);
        if (pt.cpg > 0) return run_pull_tiled(p, pt, stream);
    }
    int vpl, wpb, gran;
    dispatch_tiling(p.row_units, p.T, &vpl, &wpb, &gran);
    return run_tiled(p, vpl, wpb, gran, stream);
}

bool grouped_pull_applies(const ep_shape_t &s, int64_t row_units) {
    return s.num_tokens >= 2048 && row_units >= kWave && row_units <= kMaxPullRowUnits &&
           s.num_experts <= kGpMaxExperts && s.num_topk <= kMaxTopk;
}

hipError_t launch_dispatch_grouped_pull(const ep_shape_t &s, const DispatchArgs &a, const GroupedPullArgs &g,
                                        hipStream_t stream) {
    if (s.num_tokens == 0) return hipSuccess;
    if (a.ws == nullptr || !grouped_pull_applies(s, a.row_units)) return hipErrorInvalidValue;
    const DispatchParams p = make_params(s, a);
    GroupedOut o;
    o.aligned = g.aligned;
    o.dst = reinterpret_cast<u32x4 *>(g.grouped_x);
    o.dst_scales = g.grouped_scales;
    o.grouped_row = g.grouped_row;
    o.grouped_w = g.grouped_w;
    o.slot_pos = g.slot_pos;
    o.num_grouped = g.num_grouped;
    o.gcap = g.cap;
    return s.num_topk <= 8 ? run_grouped_pull_tiled<1>(p, o, stream) : run_grouped_pull_tiled<4>(p, o, stream);
}

}  // namespace ep
