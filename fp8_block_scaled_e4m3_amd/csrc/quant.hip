// quant.hip -- activation quantisers: bf16 / fp32 activations -> e4m3 codes plus the scales
// the GEMM routes consume, in the layouts they consume them (the step before the GEMM: page
// "Flydsl Fp8 Blockscale Gemm", Procedure step 6, and page "aiter PR #6370", Integration).
//
//  * route BS: per 1x128 group of a row, scale = amax / 448 in fp32 (1 for an all-zero group),
//    written K-block-major a_scale[kb*M + m]; codes = e4m3(x / scale) with the division
//    correctly rounded in fp32.
//  * route MX: per 1x32 group, the smallest integer e with amax <= 448 * 2^e (clamped to
//    [-127, 127], 0 for an all-zero group) as the ue8m0 byte e + 127 in a row-major
//    [M, K/32] array (fp8mx_pack_a_scale packs it); codes = e4m3(x * 2^-e), exact scaling.
//  * e4m3 encoding: nearest value, ties to the even mantissa, saturating at +-448; a NaN
//    element stays NaN (code 0x7F with its sign) and is left out of its group's amax. An
//    infinite element makes its group's scale infinite: the group's finite elements encode as
//    zero and the infinite one's code is unspecified.
//
// Memory-bound: every element is read once (2 or 4 bytes) and written once (1 byte). Lanes
// share a group: 16 lanes hold the 128 values of a BS group, 4 lanes the 32 of an MX group,
// each lane 8 consecutive values (one 16-byte load of bf16, two of fp32), so a wave reads
// whole contiguous row segments and writes 8 contiguous code bytes per lane. The group's amax
// is a butterfly max over its lanes.
#include "device.hpp"
#include "launch.hpp"

namespace fp8bs {

namespace {

// e4m3 code of q: round to nearest even on the e4m3 grid, saturating at +-448.
__device__ __forceinline__ uint32_t e4m3_code(float q)
{
    const uint32_t sign = (__float_as_uint(q) >> 31) << 7;
    const float a = fabsf(q);
    if (a != a)
        return sign | 0x7Fu;
    if (a >= 448.0f)
        return sign | 0x7Eu;
    if (a < 0.015625f)  // below the smallest normal 2^-6: multiples of 2^-9 (8 is 2^-6, code 0x08)
        return sign | (uint32_t)__builtin_rintf(a * 512.0f);
    const int E = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;  // -6 .. 8
    int m = (int)__builtin_rintf(ldexpf(a, 3 - E));                // 8 .. 16, exact scaling
    int e = E;
    if (m == 16) {
        m = 8;
        e += 1;
    }
    return sign | ((uint32_t)(e + 7) << 3) | (uint32_t)(m - 8);
}

// 8 consecutive inputs of one lane as fp32 (exact for bf16).
template <int IN_BF16>
__device__ __forceinline__ void load8(const void* x, size_t idx, float (&v)[8])
{
    if constexpr (IN_BF16) {
        const uint4 w = *(const uint4*)((const uint16_t*)x + idx);
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(u[i] << 16);
            v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    } else {
        const float4 a = *(const float4*)((const float*)x + idx);
        const float4 b = *(const float4*)((const float*)x + idx + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

__device__ __forceinline__ uint2 pack8(const uint32_t (&c)[8])
{
    return uint2{c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24), c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
}

__device__ __forceinline__ float amax8(const float (&v)[8])
{
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        m = fmaxf(m, fabsf(v[i]));  // fmaxf drops NaN
    return m;
}

// Route BS: unit u = (kb, m) with kb = u / M (so the four units of a wave share kb and write
// four consecutive scales), 16 lanes per unit.
template <int IN_BF16>
__global__ void __launch_bounds__(256) quantize_bs_kernel(const void* __restrict__ x, uint8_t* __restrict__ codes,
                                                          float* __restrict__ a_scale, int M, int K)
{
    const int lane = threadIdx.x & 63;
    const int sub = lane & 15;
    const long long units = (long long)M * (K >> 7);
    const long long waves = (long long)gridDim.x * (blockDim.x >> 6);
    for (long long u0 = ((long long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * 4; u0 < units;
         u0 += waves * 4) {
        const long long u = u0 + (lane >> 4);
        const bool live = u < units;
        const long long uu = live ? u : units - 1;  // idle lanes redo the last unit, store nothing
        const int kb = (int)(uu / M);
        const int m = (int)(uu - (long long)kb * M);
        const size_t idx = (size_t)m * K + (size_t)kb * 128 + 8 * sub;
        float v[8];
        load8<IN_BF16>(x, idx, v);
        float amax = amax8(v);
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1)
            amax = fmaxf(amax, __shfl_xor(amax, o, 16));
        const float s = amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f);
        uint32_t c[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)  // a NaN element keeps its own sign
            c[i] = e4m3_code(v[i] != v[i] ? v[i] : __fdiv_rn(v[i], s));
        if (live) {
            *(uint2*)(codes + idx) = pack8(c);
            if (sub == 0)
                a_scale[(size_t)kb * M + m] = s;
        }
    }
}

// Route MX: unit u = (m, g) row-major over [M, K/32], 4 lanes per unit, 16 units per wave.
template <int IN_BF16>
__global__ void __launch_bounds__(256) quantize_mx_kernel(const void* __restrict__ x, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ e8m0, int M, int K)
{
    const int lane = threadIdx.x & 63;
    const int sub = lane & 3;
    const int G = K >> 5;
    const long long units = (long long)M * G;
    const long long waves = (long long)gridDim.x * (blockDim.x >> 6);
    for (long long u0 = ((long long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * 16; u0 < units;
         u0 += waves * 16) {
        const long long u = u0 + (lane >> 2);
        const bool live = u < units;
        const long long uu = live ? u : units - 1;
        const int m = (int)(uu / G);
        const int g = (int)(uu - (long long)m * G);
        const size_t idx = (size_t)m * K + (size_t)g * 32 + 8 * sub;
        float v[8];
        load8<IN_BF16>(x, idx, v);
        float amax = amax8(v);
        amax = fmaxf(amax, __shfl_xor(amax, 1, 4));
        amax = fmaxf(amax, __shfl_xor(amax, 2, 4));
        // smallest e with amax <= 448 * 2^e = 1.75 * 2^(e+8): with amax in [2^(x-1), 2^x),
        // e = x - 9 when amax <= 1.75 * 2^(x-1), else x - 8. fp32 subnormals clamp to -127.
        int e = 0;
        if (amax > 0.0f) {
            const int field = (int)((__float_as_uint(amax) >> 23) & 0xffu);
            if (field == 0) {
                e = -127;
            } else {
                const int xexp = field - 126;
                e = amax <= ldexpf(1.75f, xexp - 1) ? xexp - 9 : xexp - 8;
                e = min(max(e, -127), 127);
            }
        }
        uint32_t c[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            c[i] = e4m3_code(v[i] != v[i] ? v[i] : ldexpf(v[i], -e));
        if (live) {
            *(uint2*)(codes + idx) = pack8(c);
            if (sub == 0)
                e8m0[uu] = (uint8_t)(e + 127);
        }
    }
}

int quant_grid(long long units_per_wave_step, long long units)
{
    const long long waves = (units + units_per_wave_step - 1) / units_per_wave_step;
    const long long blocks = (waves + 3) / 4;
    const long long cap = (long long)device_cus() * 8;
    return (int)(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
}

}  // namespace

hipError_t launch_quantize(int route, const void* x, int in_bf16, void* codes, void* scales, int M, int K,
                           hipStream_t stream)
{
    if (M == 0)
        return hipSuccess;
    if (route == kRouteBS) {
        const int grid = quant_grid(4, (long long)M * (K >> 7));
        if (in_bf16)
            hipLaunchKernelGGL(quantize_bs_kernel<1>, dim3(grid), dim3(256), 0, stream, x, (uint8_t*)codes,
                               (float*)scales, M, K);
        else
            hipLaunchKernelGGL(quantize_bs_kernel<0>, dim3(grid), dim3(256), 0, stream, x, (uint8_t*)codes,
                               (float*)scales, M, K);
    } else {
        const int grid = quant_grid(16, (long long)M * (K >> 5));
        if (in_bf16)
            hipLaunchKernelGGL(quantize_mx_kernel<1>, dim3(grid), dim3(256), 0, stream, x, (uint8_t*)codes,
                               (uint8_t*)scales, M, K);
        else
            hipLaunchKernelGGL(quantize_mx_kernel<0>, dim3(grid), dim3(256), 0, stream, x, (uint8_t*)codes,
                               (uint8_t*)scales, M, K);
    }
    return hipGetLastError();
}

}  // namespace fp8bs
