// ep_combine.hip -- stage 5, combine (gfx950).
//
// Definitions (mscclpp ht_runtime.cc mirror, internodeCombine /
// intranodeCombine: bf16 combined rows plus combined topk weights; CUDA与DeepEP
// article 4.2: every received row returns to its source token).  The order of
// the reduction is not on the pages; it is fixed here as
//   for r ascending with s = send_slot[t][r] >= 0:
//     W = sum_j recv_topk_weights[s][j]      (fp32 adds, j ascending, from +0)
//     acc[i] = fmaf(W, y[s][i], acc[i])      (fp32, from +0)
//   combined_x[t][i] = bf16 round-to-nearest-even of acc[i]
//   combined_topk_weights[t][j] = sum over the same r of recv_topk_weights[s][j]
//
// Design: a token-parallel gather driven by send_slot, the map dispatch
// recorded; one wave per (token, row segment of VPL*1 KiB).  Lane r reads
// send_slot[t][r], so the wave knows every contributing row at once and starts
// loading the first two rows' segments.  Lane r loads its row's weights in one
// batch and adds them in j order (W); the first segment's wave also adds the
// rows' weights column by column in rank order (the combined weights).  The
// row segments stream in pairs with 16-byte non-temporal loads and are folded
// in ascending rank order into per-lane fp32 accumulators with v_fma_f32; the
// wave ends with one bf16 store per element.  HBM traffic: the ~8 rows read per
// token plus the one row written.
// For wide rows and many tokens the outputs go out in bursts instead: a block
// of 16 waves takes 8 consecutive tokens (their segments in turn), keeps the
// bf16 results in LDS, and after its last gather writes the 8 rows as one
// contiguous run.  Every result is computed the same way in both kernels.
#include <mutex>

#include "ep_internal.h"

namespace ep {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));


struct CombineParams {
    const u32x4 *y;
    const float *recv_w;
    const int32_t *send_slot;
    u32x4 *out;
    float *out_w;
    int32_t *dev_status;
    int64_t T;
    int64_t row_units;
    int R, K, nrows, S;
};

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// fp32 -> bf16, round to nearest, ties to even (adding 0x7fff plus the kept
// LSB carries into the kept half exactly when the dropped half exceeds the
// midpoint, or equals it with an odd kept half); NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int VPL, bool EXACT>
__device__ __forceinline__ void load_seg(u32x4 (&v)[VPL], const u32x4 *src, int64_t c0, int64_t units) {
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        if (EXACT || c0 + i * kWave < units) v[i] = __builtin_nontemporal_load(src + i * kWave);
}

template <int VPL, bool EXACT>
__device__ __forceinline__ void fma_seg(float (&acc)[VPL][8], const u32x4 (&v)[VPL], float w, int64_t c0,
                                        int64_t units) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        if (EXACT || c0 + i * kWave < units) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                acc[i][2 * k] = __builtin_fmaf(w, bf16_lo(v[i][k]), acc[i][2 * k]);
                acc[i][2 * k + 1] = __builtin_fmaf(w, bf16_hi(v[i][k]), acc[i][2 * k + 1]);
            }
        }
    }
}

// One wave's task: token t, row segment seg.  Returns the segment's bf16
// results (packed in pairs) in o; the segment-0 wave also flags bad slots and
// writes the combined weights.
template <int VPL, bool EXACT>
__device__ __forceinline__ void combine_task(const CombineParams &p, int64_t t, int seg, int lane, u32x4 (&o)[VPL]) {
    const int K = p.K;
    const int64_t U = p.row_units;
    const int64_t c0 = (int64_t)seg * VPL * kWave + lane;

    int slot = -1;
    bool bad = false;
    if (lane < p.R) {
        slot = p.send_slot[t * p.R + lane];
        if (slot < -1 || slot >= p.nrows) {
            bad = true;
            slot = -1;
        }
    }
    uint64_t ee = ballot64(slot >= 0);  // contributing ranks not yet loaded

    // rows in pairs, ranks ascending: the first pair is in flight while the
    // weights are summed
    u32x4 a[VPL], b[VPL];
    int ra = -1, rb = -1;
    auto fetch = [&](u32x4(&v)[VPL], int &rk) {
        if (ee != 0ull) {
            rk = __builtin_ctzll(ee);
            ee &= ee - 1ull;
            const int64_t s = readlane32(slot, rk);
            load_seg<VPL, EXACT>(v, p.y + s * U + c0, c0, U);
        } else {
            rk = -1;
        }
    };
    const uint64_t dests = ee;
    fetch(a, ra);
    fetch(b, rb);

    // lane r: W of its row, the row's weights added in j order (batches of 8
    // loads in flight together)
    float W = 0.0f;
    float wv[8];
    for (int j0 = 0; j0 < K; j0 += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) wv[u] = (slot >= 0 && j0 + u < K) ? p.recv_w[(int64_t)slot * K + j0 + u] : 0.0f;
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (j0 + u < K) W = W + wv[u];
    }
    if (seg == 0) {
        if (ballot64(bad) != 0ull && lane == 0) flag(p.dev_status, EP_DEV_BAD_SEND_SLOT);
        if (p.out_w != nullptr) {
            // combined weight j: the rows' weight j added in rank order (lane j)
            float cw = 0.0f;
            for (int j0 = 0; j0 < K; j0 += 8) {
                if (K > 8) {  // wv holds the last batch of the W loop: reload this one
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        wv[u] = (slot >= 0 && j0 + u < K) ? p.recv_w[(int64_t)slot * K + j0 + u] : 0.0f;
                }
                for (uint64_t dd = dests; dd != 0ull; dd &= dd - 1ull) {
                    const int r = __builtin_ctzll(dd);
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const float x = readlanef(wv[u], r);
                        if (lane == j0 + u) cw = cw + x;
                    }
                }
            }
            if (lane < K) p.out_w[t * K + lane] = cw;
        }
    }

    float acc[VPL][8];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[i][k] = 0.0f;
    while (ra >= 0) {
        fma_seg<VPL, EXACT>(acc, a, readlanef(W, ra), c0, U);
        if (rb >= 0) fma_seg<VPL, EXACT>(acc, b, readlanef(W, rb), c0, U);
        fetch(a, ra);
        fetch(b, rb);
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) o[i][k] = to_bf16(acc[i][2 * k]) | (to_bf16(acc[i][2 * k + 1]) << 16);
}

// One wave per (token, row segment); each wave stores its segment.
template <int VPL, bool EXACT, int WPB>
__global__ __launch_bounds__(WPB *kWave) void combine_kernel(CombineParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t w = (int64_t)blockIdx.x * WPB + (threadIdx.x >> 6);
    if (w >= p.T * p.S) return;  // whole wave leaves together
    const int64_t t = w / p.S;
    const int seg = (int)(w - t * p.S);
    const int64_t U = p.row_units;
    const int64_t c0 = (int64_t)seg * VPL * kWave + lane;
    u32x4 o[VPL];
    combine_task<VPL, EXACT>(p, t, seg, lane, o);
    u32x4 *dst = p.out + t * U + c0;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        if (EXACT || c0 + i * kWave < U) __builtin_nontemporal_store(o[i], dst + i * kWave);
}

// TB consecutive tokens per block of WPB waves: the waves take the tokens'
// segments in turn and keep the results in LDS (TB rows), then the block
// writes the TB rows as one contiguous run.
template <int VPL, bool EXACT, int TB, int WPB>
__global__ __launch_bounds__(WPB *kWave) void combine_staged_kernel(CombineParams p) {
    extern __shared__ u32x4 s_rows[];  // [TB][row_units]
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * TB;
    const int64_t U = p.row_units;
    const int tasks = TB * p.S;
    for (int k = wave; k < tasks; k += WPB) {
        const int tl = k / p.S;
        const int seg = k - tl * p.S;
        if (t0 + tl >= p.T) break;  // the wave's later tasks are later tokens
        u32x4 o[VPL];
        combine_task<VPL, EXACT>(p, t0 + tl, seg, lane, o);
        const int64_t c0 = (int64_t)seg * VPL * kWave + lane;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (EXACT || c0 + i * kWave < U) s_rows[tl * U + c0 + i * kWave] = o[i];
    }
    __syncthreads();
    const int64_t rows = p.T - t0 < TB ? p.T - t0 : TB;
    u32x4 *dst = p.out + t0 * U;
    for (int64_t i = threadIdx.x; i < rows * U; i += WPB * kWave) __builtin_nontemporal_store(s_rows[i], dst + i);
}

template <int VPL, bool EXACT, int WPB>
hipError_t run(CombineParams p, hipStream_t stream) {
    p.S = (int)((p.row_units + VPL * kWave - 1) / (VPL * kWave));
    const int64_t waves = p.T * p.S;
    const int64_t blocks = (waves + WPB - 1) / WPB;
    hipLaunchKernelGGL((combine_kernel<VPL, EXACT, WPB>), dim3((unsigned)blocks), dim3(WPB * kWave), 0, stream, p);
    return hipGetLastError();
}

// Staged form: 2 KiB segments, 8 tokens per block of 16 waves (fewer tokens when
// 8 rows would not fit kStagedLds bytes of LDS).
constexpr int kStagedWaves = 16;
constexpr size_t kStagedLds = 112 * 1024;

template <bool EXACT, int TB>
hipError_t run_staged_tb(CombineParams p, hipStream_t stream) {
    p.S = (int)((p.row_units + 2 * kWave - 1) / (2 * kWave));
    const size_t lds = (size_t)TB * p.row_units * sizeof(u32x4);
    static std::once_flag once;  // the kernel's dynamic LDS limit, raised once per process
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
        attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&combine_staged_kernel<2, EXACT, TB, kStagedWaves>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)kStagedLds);
    });
    if (attr != hipSuccess) return attr;
    const int64_t blocks = (p.T + TB - 1) / TB;
    hipLaunchKernelGGL((combine_staged_kernel<2, EXACT, TB, kStagedWaves>), dim3((unsigned)blocks),
                       dim3(kStagedWaves * kWave), lds, stream, p);
    return hipGetLastError();
}

// Tokens per block of the staged form for these rows (0: the rows are too wide).
int staged_tokens(int64_t row_units) {
    const int64_t fit = (int64_t)(kStagedLds / (sizeof(u32x4) * (size_t)row_units));
    return fit >= 8 ? 8 : fit >= 4 ? 4 : fit >= 2 ? 2 : 0;
}

hipError_t run_staged(const CombineParams &p, int tb, hipStream_t stream) {
    const bool exact = p.row_units % (2 * kWave) == 0;
    if (tb == 8) return exact ? run_staged_tb<true, 8>(p, stream) : run_staged_tb<false, 8>(p, stream);
    if (tb == 4) return exact ? run_staged_tb<true, 4>(p, stream) : run_staged_tb<false, 4>(p, stream);
    return exact ? run_staged_tb<true, 2>(p, stream) : run_staged_tb<false, 2>(p, stream);
}

hipError_t run_tiled(const CombineParams &p, int vpl, int wpb, hipStream_t stream) {
    const bool exact = p.row_units % (vpl * kWave) == 0;
#define EP_COMBINE_CASE(V, W) \
    if (vpl == V && wpb == W) return exact ? run<V, true, W>(p, stream) : run<V, false, W>(p, stream);
    EP_COMBINE_CASE(1, 4)
    EP_COMBINE_CASE(2, 4)
    EP_COMBINE_CASE(2, 8)
    EP_COMBINE_CASE(4, 4)
    EP_COMBINE_CASE(7, 4)
    EP_COMBINE_CASE(8, 4)
#undef EP_COMBINE_CASE
    return hipErrorInvalidValue;
}

// Measured on MI355X (prefill, skew and large workloads, and 512..2048-token
// cuts of prefill): rows of 14 KiB and more in 2 KiB segments, 8 waves per
// block from 4096 tokens and 4 below; narrower rows in 1 KiB segments, 4 waves
// per block.
void combine_tiling(int64_t row_units, int64_t num_tokens, int *vpl, int *wpb) {
    if (row_units >= 14 * kWave) {
        *vpl = 2;
        *wpb = num_tokens >= 4096 ? 8 : 4;
    } else {
        *vpl = 1;
        *wpb = 4;
    }
}

}  // namespace

hipError_t launch_combine(const ep_shape_t &s, const uint4 *y, const float *recv_w, const int32_t *send_slot,
                          int32_t num_recv_rows, uint4 *combined_x, float *combined_w, int32_t *dev_status,
                          hipStream_t stream) {
    if (s.num_tokens == 0) return hipSuccess;
    CombineParams p;
    p.y = reinterpret_cast<const u32x4 *>(y);
    p.recv_w = recv_w;
    p.send_slot = send_slot;
    p.out = reinterpret_cast<u32x4 *>(combined_x);
    p.out_w = combined_w;
    p.dev_status = dev_status;
    p.T = s.num_tokens;
    p.row_units = s.hidden / 8;
    p.R = s.num_ranks;
    p.K = s.num_topk;
    p.nrows = num_recv_rows;
    p.S = 1;
    // rows of 14 KiB and more from 4096 tokens: the staged form (prefill 87 -> 82.5 us,
    // skew 75.5 -> 72.3; 4 KiB rows at 16384 tokens were slower staged, 142 against 138)
    const int tb = staged_tokens(p.row_units);
    if (p.row_units >= 14 * kWave && p.T >= 4096 && tb > 0) return run_staged(p, tb, stream);
    int vpl, wpb;
    combine_tiling(p.row_units, p.T, &vpl, &wpb);
    return run_tiled(p, vpl, wpb, stream);
}

}  // namespace ep
