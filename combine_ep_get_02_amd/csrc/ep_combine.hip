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

template <int VPL, bool EXACT, int WPB>
__global__ __launch_bounds__(WPB *kWave) void combine_kernel(CombineParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t w = (int64_t)blockIdx.x * WPB + (threadIdx.x >> 6);
    if (w >= p.T * p.S) return;  // whole wave leaves together
    const int64_t t = w / p.S;
    const int seg = (int)(w - t * p.S);
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

    u32x4 *dst = p.out + t * U + c0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        if (EXACT || c0 + i * kWave < U) {
            u32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = to_bf16(acc[i][2 * k]) | (to_bf16(acc[i][2 * k + 1]) << 16);
            __builtin_nontemporal_store(o, dst + i * kWave);
        }
    }
}

template <int VPL, bool EXACT, int WPB>
hipError_t run(CombineParams p, hipStream_t stream) {
    p.S = (int)((p.row_units + VPL * kWave - 1) / (VPL * kWave));
    const int64_t waves = p.T * p.S;
    const int64_t blocks = (waves + WPB - 1) / WPB;
    hipLaunchKernelGGL((combine_kernel<VPL, EXACT, WPB>), dim3((unsigned)blocks), dim3(WPB * kWave), 0, stream, p);
    return hipGetLastError();
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
    int vpl, wpb;
    combine_tiling(p.row_units, p.T, &vpl, &wpb);
    return run_tiled(p, vpl, wpb, stream);
}

}  // namespace ep
