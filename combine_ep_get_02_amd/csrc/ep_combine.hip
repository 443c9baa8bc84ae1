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
// Design: one wave per (token, row segment); a token-parallel gather driven by
// send_slot, the map dispatch recorded.  Lane r reads send_slot[t][r] and sums
// its row's weights, so the wave knows every contribution's row and weight at
// once; the segment of each contributing row is then streamed in with 16-byte
// non-temporal loads (8 bf16 per lane per load) and folded into per-lane fp32
// accumulators with v_fma_f32 in ascending rank order.  One bf16 store per
// element leaves the wave.  HBM traffic is the ~8 rows read per token plus the
// one row written.
#include "ep_internal.h"

namespace ep {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCombineWaves = 4;

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
__global__ __launch_bounds__(kCombineWaves *kWave) void combine_kernel(CombineParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t w = (int64_t)blockIdx.x * kCombineWaves + (threadIdx.x >> 6);
    if (w >= p.T * p.S) return;  // whole wave leaves together
    const int64_t t = w / p.S;
    const int seg = (int)(w - t * p.S);

    int slot = -1;
    bool bad = false;
    if (lane < p.R) {
        slot = p.send_slot[t * p.R + lane];
        if (slot < -1 || slot >= p.nrows) {
            bad = true;
            slot = -1;
        }
    }
    const uint64_t dests = ballot64(slot >= 0);
    float W = 0.0f;
    if (slot >= 0) {
        const float *wr = p.recv_w + (int64_t)slot * p.K;
        for (int j = 0; j < p.K; ++j) W = W + wr[j];
    }
    if (seg == 0) {
        if (ballot64(bad) != 0ull && lane == 0) flag(p.dev_status, EP_DEV_BAD_SEND_SLOT);
        if (p.out_w != nullptr) {
            float cw = 0.0f;
            for (uint64_t dd = dests; dd != 0ull; dd &= dd - 1ull) {
                const int64_t s = readlane32(slot, __builtin_ctzll(dd));
                if (lane < p.K) cw = cw + p.recv_w[s * p.K + lane];
            }
            if (lane < p.K) p.out_w[t * p.K + lane] = cw;
        }
    }

    const int64_t c0 = (int64_t)seg * VPL * kWave + lane;
    float acc[VPL][8];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[i][k] = 0.0f;

    for (uint64_t dd = dests; dd != 0ull; dd &= dd - 1ull) {
        const int r = __builtin_ctzll(dd);
        const int64_t s = readlane32(slot, r);
        const float wr = readlanef(W, r);
        const u32x4 *src = p.y + s * p.row_units + c0;
        u32x4 v[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (EXACT || c0 + i * kWave < p.row_units) v[i] = __builtin_nontemporal_load(src + i * kWave);
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            if (EXACT || c0 + i * kWave < p.row_units) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    acc[i][2 * k] = __builtin_fmaf(wr, bf16_lo(v[i][k]), acc[i][2 * k]);
                    acc[i][2 * k + 1] = __builtin_fmaf(wr, bf16_hi(v[i][k]), acc[i][2 * k + 1]);
                }
            }
        }
    }

    u32x4 *dst = p.out + t * p.row_units + c0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        if (EXACT || c0 + i * kWave < p.row_units) {
            u32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = to_bf16(acc[i][2 * k]) | (to_bf16(acc[i][2 * k + 1]) << 16);
            __builtin_nontemporal_store(o, dst + i * kWave);
        }
    }
}

template <int VPL, bool EXACT>
hipError_t run(const CombineParams &p, hipStream_t stream) {
    const int64_t waves = p.T * p.S;
    const int64_t blocks = (waves + kCombineWaves - 1) / kCombineWaves;
    hipLaunchKernelGGL((combine_kernel<VPL, EXACT>), dim3((unsigned)blocks), dim3(kCombineWaves * kWave), 0, stream,
                       p);
    return hipGetLastError();
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
    const int64_t U = p.row_units;
    if (U % (7 * kWave) == 0) {
        p.S = (int)(U / (7 * kWave));
        return run<7, true>(p, stream);
    }
    if (U % (8 * kWave) == 0) {
        p.S = (int)(U / (8 * kWave));
        return run<8, true>(p, stream);
    }
    if (U % (4 * kWave) == 0) {
        p.S = (int)(U / (4 * kWave));
        return run<4, true>(p, stream);
    }
    if (U % kWave == 0) {
        p.S = (int)(U / kWave);
        return run<1, true>(p, stream);
    }
    p.S = (int)((U + 4 * kWave - 1) / (4 * kWave));
    return run<4, false>(p, stream);
}

}  // namespace ep
