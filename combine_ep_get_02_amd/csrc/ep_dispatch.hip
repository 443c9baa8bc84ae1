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
    int32_t *tok_pos;
    int32_t *dev_status;
    int64_t T;
    int64_t Tc;         // tokens per channel, ceil(t / C)
    int64_t row_units;  // 16-byte units per row
    int R, K, E, C, experts_per_rank, my_rank, cap, S, num_scales;
    int in_unit;        // load unit of an is_token_in_rank row (16, 8 or 1 bytes)
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
// expert id e and weight wt) and {my_rank, t} as the row's source.  tok_pos
// (the grouped dispatch only) is cleared to -1 for the grouping to fill in.
__device__ __forceinline__ void token_metadata(const DispatchParams &p, int64_t t, int slot, uint64_t dests,
                                               int64_t e, float wt, int lane) {
    if (lane < p.R) p.send_slot[t * p.R + lane] = slot;
    if (p.tok_pos != nullptr && lane < p.K) p.tok_pos[t * p.K + lane] = -1;
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
    u32x4 v[VPL > 0 ? VPL : 1];  // VPL == 0: metadata only, no row
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

    if (live && seg == 0) copy_scales(p, t, slot, dests, lane);
    if (!CACHED && live && seg == 0) token_metadata(p, t, slot, dests, e, wt, lane);

    if (VPL == 0) return;  // metadata only
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
                const bool found = oc < __popcll(cc);
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

template <int CPG, int U, bool EXACT, int WPB>
hipError_t run_pull(DispatchParams p, int blocks_per_xcd, hipStream_t stream) {
    const dim3 grid((unsigned)(kXcds * blocks_per_xcd)), block(WPB * kWave);
    if (p.derive)
        hipLaunchKernelGGL((dispatch_pull_kernel<CPG, U, EXACT, WPB, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((dispatch_pull_kernel<CPG, U, EXACT, WPB, false>), grid, block, 0, stream, p);
    return hipGetLastError();
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
    p.tok_pos = a.tok_pos;
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
    if (p.recv_x == nullptr && p.cached_slot == nullptr) {
        p.num_scales = 0;  // no rows, so no scales beside them
        return run_meta(p, stream);
    }
    // cached mode always takes the push form
    if (a.form != EP_FORM_PUSH && p.cached_slot == nullptr) {
        const PullTiling pt = pull_tiling(p.row_units, p.T);
        if (pt.cpg > 0) return run_pull_tiled(p, pt, stream);
    }
    int vpl, wpb, gran;
    dispatch_tiling(p.row_units, p.T, &vpl, &wpb, &gran);
    return run_tiled(p, vpl, wpb, gran, stream);
}

}  // namespace ep
