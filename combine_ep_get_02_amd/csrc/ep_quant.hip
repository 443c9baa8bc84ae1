// ep_quant.hip -- bf16 rows to OCP FP8 E4M3 codes with per-group float scales,
// the fp8 rows and scales that ep_dispatch_fp8 carries, and back to bf16.
//
// [mscclpp ht_runtime.cc, intranodeDispatch / internodeDispatch: x with an
// element size of one byte travels with xScales, numScales floats per token,
// returned as the receive side's FP8 scale buffer; the pages do not say how x
// and its scales are made.]  This library's quantiser: a row of H channels is
// cut into S groups of g = H / S consecutive channels; group q of row t takes
//   a = max(max |x| over the group, 2^-64)
//   scale[t][q] = a / 448                                (binary32, correctly rounded)
//   code[t][i]  = e4m3(clamp(x[t][i] * (448 / a), -448, 448))
// where 448 / a and the product are binary32 roundings and e4m3() is the nearest
// E4M3 value, ties to even (one sign bit, four exponent bits with bias 7, three
// mantissa bits, no infinities, 448 the largest finite value).  Dequantisation is
// bf16_rne(value(code) * scale) with the product rounded to binary32.
//
// Both kernels stream 1024 channels of the flattened [rows][H] array per wave.  In
// the quantiser each lane owns 16 consecutive channels (32 bytes of bf16, 16 bytes
// of codes); groups of g channels are g / 16 aligned lanes, so a group's largest
// magnitude is a butterfly of lane maxima inside the wave, and a group never
// straddles two waves (g divides 1024).  The dequantiser gives each lane two
// 8-channel chunks 512 channels apart, so that every access instruction covers one
// contiguous span.  HBM bytes per row: 2H read + H + 4S written (quantise), H + 4S
// read + 2H written (dequantise).
//
// The conversions are gfx950's own: v_cvt_pk_fp8_f32 (nearest-even under the
// default rounding mode; its input is clamped to +-448 first, so no input is out
// of range) and v_cvt_pk_f32_fp8 (exact).  fp32 division is the compiler's
// correctly rounded sequence, once per group.  The per-lane quantisation step
// (e4m3_quantize16, ep_internal.h) is the one the dispatch that quantises on the
// way runs too.
#include "ep_internal.h"

namespace ep {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kQuantWaves = 4;          // waves per block
constexpr int64_t kQuantMaxBlocks = 1 << 16;

struct QuantParams {
    const u32x4 *x;      // bf16 [units][2]: unit u = channels 16u .. 16u+15 of the flattened rows
    u32x4 *codes;        // [units]
    float *scales;       // [units >> lanes_log2]
    int64_t units;       // rows * H / 16
    int lanes_log2;      // log2(g / 16): lanes per group
};

struct DequantParams {
    const u32x4 *codes;  // [units]
    const float *scales; // [units >> lanes_log2]
    u32x4 *out;          // bf16 [2 * units]: unit q = channels 8q .. 8q+7
    int64_t units;
    int lanes_log2;
};

// fp32 -> bf16, nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(kQuantWaves *kWave) void quantize_e4m3_kernel(QuantParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nwaves = (int64_t)gridDim.x * kQuantWaves;
    const int lead_mask = (1 << p.lanes_log2) - 1;
    for (int64_t w = (int64_t)blockIdx.x * kQuantWaves + (threadIdx.x >> 6); w * kWave < p.units; w += nwaves) {
        const int64_t u = w * kWave + lane;
        const bool on = u < p.units;  // a wave's idle tail lanes form whole groups of their own
        u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (on) {
            a = p.x[2 * u];
            b = p.x[2 * u + 1];
        }
        float scale;
        const u32x4 c = e4m3_quantize16(a, b, p.lanes_log2, &scale);
        if (on) {
            p.codes[u] = c;
            if ((lane & lead_mask) == 0) p.scales[u >> p.lanes_log2] = scale;
        }
    }
}

// A wave takes 1024 channels (64 units of codes); lane L decodes the 8-byte code chunks L and
// L + 64 of them into the bf16 units L and L + 64, so each load and each store instruction of the
// wave covers one contiguous span (512 bytes of codes, 1 KiB of bf16).  With two 16-byte halves
// per lane instead, each store instruction wrote every other 16 bytes of 2 KiB: 123-125 us for
// 31,430 rows of 7168 with 505 MB written for 450 (lines written in two pieces), against 107.9-108.3
// here (one run).
__global__ __launch_bounds__(kQuantWaves *kWave) void dequantize_e4m3_kernel(DequantParams p) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nwaves = (int64_t)gridDim.x * kQuantWaves;
    const u32x2 *codes8 = reinterpret_cast<const u32x2 *>(p.codes);
    const int64_t chunks = 2 * p.units;  // 8-byte code chunks = bf16 output units
    const int glog = p.lanes_log2 + 1;   // log2 of the chunks per scale group
    for (int64_t w = (int64_t)blockIdx.x * kQuantWaves + (threadIdx.x >> 6); w * kWave < p.units; w += nwaves) {
        u32x2 c[2];
        float s[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t q = (2 * w + h) * kWave + lane;
            if (q < chunks) {
                c[h] = __builtin_nontemporal_load(codes8 + q);
                s[h] = p.scales[q >> glog];
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t q = (2 * w + h) * kWave + lane;
            if (q >= chunks) continue;
            u32x4 o;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[h][k], false);  // bytes 0, 1
                const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[h][k], true);   // bytes 2, 3
                o[2 * k] = to_bf16(lo.x * s[h]) | (to_bf16(lo.y * s[h]) << 16);
                o[2 * k + 1] = to_bf16(hi.x * s[h]) | (to_bf16(hi.y * s[h]) << 16);
            }
            __builtin_nontemporal_store(o, p.out + q);
        }
    }
}

int blocks_for(int64_t units) {
    const int64_t waves = (units + kWave - 1) / kWave;
    const int64_t blocks = (waves + kQuantWaves - 1) / kQuantWaves;
    return (int)(blocks < kQuantMaxBlocks ? blocks : kQuantMaxBlocks);
}

}  // namespace

int quant_lanes_log2(int hidden, int num_scales) {
    if (num_scales < 1 || hidden % num_scales != 0) return -1;
    const int g = hidden / num_scales;
    for (int l = 0; l <= 6; ++l)
        if (g == kQuantChannels << l) return l;
    return -1;
}

hipError_t launch_quantize(const void *x, int64_t rows, int hidden, int num_scales, void *codes, float *scales,
                           hipStream_t stream) {
    QuantParams p;
    p.x = static_cast<const u32x4 *>(x);
    p.codes = static_cast<u32x4 *>(codes);
    p.scales = scales;
    p.units = rows * (hidden / kQuantChannels);
    p.lanes_log2 = quant_lanes_log2(hidden, num_scales);
    if (p.units == 0) return hipSuccess;
    hipLaunchKernelGGL(quantize_e4m3_kernel, dim3((unsigned)blocks_for(p.units)), dim3(kQuantWaves * kWave), 0,
                       stream, p);
    return hipGetLastError();
}

hipError_t launch_dequantize(const void *codes, const float *scales, int64_t rows, int hidden, int num_scales,
                             void *out, hipStream_t stream) {
    DequantParams p;
    p.codes = static_cast<const u32x4 *>(codes);
    p.scales = scales;
    p.out = static_cast<u32x4 *>(out);
    p.units = rows * (hidden / kQuantChannels);
    p.lanes_log2 = quant_lanes_log2(hidden, num_scales);
    if (p.units == 0) return hipSuccess;
    hipLaunchKernelGGL(dequantize_e4m3_kernel, dim3((unsigned)blocks_for(p.units)), dim3(kQuantWaves * kWave), 0,
                       stream, p);
    return hipGetLastError();
}

}  // namespace ep
