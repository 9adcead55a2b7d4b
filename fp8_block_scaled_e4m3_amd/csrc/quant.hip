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
//  * e4m3 encoding: nearest value, ties to the even mantissa (a scaled finite input is at most
//    448 * (1 + 2^-23) in magnitude, which rounds to +-448, so saturation never arises); a NaN
//    element stays NaN (code 0x7F with its sign) and is left out of its group's amax. An
//    infinite element makes its group's scale infinite: the group's finite elements encode as
//    zero and the infinite one's code is unspecified.
//
// Memory-bound: every element is read once (2 or 4 bytes) and written once (1 byte). Each lane
// holds 16 consecutive values (two 16-byte loads of bf16, four of fp32) and writes their 16
// codes with one 16-byte store; 8 lanes hold the 128 values of a BS group, 2 lanes the 32 of an
// MX group, and the group's amax is a butterfly max over its lanes.
//
// Per-element arithmetic is kept to a few instructions so that HBM, not the ALU, bounds the
// pass:
//  * The BS quotient RN32(x / s), where every group of the wave has s >= 2^-90 (all but the
//    tiniest groups): Markstein's correction of a product (P. Markstein, IBM J. Res. Dev. 34(1),
//    1990), y = RN32(1 / s), q0 = RN32(x * y), q = RN32(q0 + (x - q0 * s) * y) with the residual
//    from one fused multiply-add; correctly rounded because y is and the residual is exact for
//    these magnitudes (quotients below 2^-11 may differ in their last bits but encode as zero
//    either way). Checked on the host for every bf16 (x, amax) pair with such a scale and on
//    10^8 random fp32 pairs (tests/quant_division_check.c).
//  * Otherwise RN32(x * y) evaluated in fp64 with y = RN64(1 / s), one fp64 division per lane
//    and group. This is exact: the fp64 product is within 2^-52 (relative) of x / s, while
//    x / s (24-bit numerator, 24-bit divisor) is never an fp32 rounding midpoint and stays at
//    least 2^-49 (relative) away from every midpoint, so both round to the same fp32 value.
//    (Also checked on the device for every finite bf16 x against every scale of a positive
//    finite bf16 amax, and on 2^34 random fp32 pairs: no difference to __fdiv_rn.)
//  * The e4m3 rounding is the hardware conversion v_cvt_pk_fp8_f32 (OCP e4m3 on this GPU, round
//    to nearest even). It equals the rounding stated above for every finite fp32 input below
//    464 in magnitude (checked on the device for all 2^32 fp32 bit patterns); scaled finite
//    inputs never exceed 448 * (1 + 2^-23). Its NaN code does not carry the input's sign, so
//    each code's sign bit is replaced by its input's (a no-op for every non-NaN input).
#include "device.hpp"
#include "launch.hpp"

namespace fp8bs {

namespace {

constexpr int kQuantThreads = 256;

// 16 consecutive inputs of one lane as fp32 (exact for bf16) plus the sign bit of each in
// position 8i+7 of sign[i/4] (the layout of the packed codes).
template <int IN_BF16>
__device__ __forceinline__ void load16(const void* x, size_t idx, float (&v)[16], uint32_t (&sign)[4])
{
    if constexpr (IN_BF16) {
        const uint4 a = *(const uint4*)((const uint16_t*)x + idx);
        const uint4 b = *(const uint4*)((const uint16_t*)x + idx + 8);
        const uint32_t u[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = __uint_as_float(u[i] << 16);
            v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
        // byte 1 and byte 3 of each word carry the two values' sign bits in their bit 7
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sign[i] = __builtin_amdgcn_perm(u[2 * i + 1], u[2 * i], 0x07050301u) & 0x80808080u;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 f = *(const float4*)((const float*)x + idx + 4 * i);
            v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
            sign[i] = (__float_as_uint(f.x) >> 31 << 7) | (__float_as_uint(f.y) >> 31 << 15) |
                      (__float_as_uint(f.z) >> 31 << 23) | (__float_as_uint(f.w) >> 31 << 31);
        }
    }
}

__device__ __forceinline__ float amax16(const float (&v)[16])
{
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        m = fmaxf(m, fabsf(v[i]));  // fmaxf drops NaN
    return m;
}

// e4m3 codes of q[0..15] (the hardware rounding), sign bits taken from the inputs.
__device__ __forceinline__ uint4 codes16(const float (&q)[16], const uint32_t (&sign)[4])
{
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int d = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * i], q[4 * i + 1], 0, false);
        d = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * i + 2], q[4 * i + 3], d, true);
        w[i] = ((uint32_t)d & 0x7f7f7f7fu) | sign[i];
    }
    return uint4{w[0], w[1], w[2], w[3]};
}

// Route BS. Block b covers rows [64 * (b % MB), +64) of K block kb = b / MB (MB = ceil(M / 64));
// each wave takes 8 rows per pass (8 lanes per row), two passes.
template <int IN_BF16>
__global__ void __launch_bounds__(kQuantThreads) quantize_bs_kernel(const void* __restrict__ x,
                                                                    uint8_t* __restrict__ codes,
                                                                    float* __restrict__ a_scale, int M, int K, int MB)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = lane & 7;
    const int b = blockIdx.x;
    const int kb = b / MB, mb = b - kb * MB;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const int m = 64 * mb + 32 * pass + 8 * wave + (lane >> 3);
        const bool live = m < M;
        const int mm = live ? m : M - 1;  // lanes past M redo row M-1 and store nothing
        const size_t idx = (size_t)mm * K + (size_t)kb * 128 + 16 * sub;
        float v[16];
        uint32_t sign[4];
        load16<IN_BF16>(x, idx, v, sign);
        float amax = amax16(v);
        amax = fmaxf(amax, __shfl_xor(amax, 1, 8));
        amax = fmaxf(amax, __shfl_xor(amax, 2, 8));
        amax = fmaxf(amax, __shfl_xor(amax, 4, 8));
        const float s = amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f);
        float q[16];
        if (__all(s >= 0x1p-90f && s <= 0x1.fffffep+127f)) {
            // every group of the wave has a finite scale of at least 2^-90: the correction step
            // (the fp64 product costs about three times the vector-ALU time, which shows on
            // short rows: 16384 x 768 bf16, 6.02 against 6.42 us)
            const float y = __frcp_rn(s);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float q0 = __fmul_rn(v[i], y);
                q[i] = fmaf(fmaf(-q0, s, v[i]), y, q0);
            }
        } else {
            const double y = 1.0 / (double)s;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                q[i] = (float)((double)v[i] * y);
        }
        const uint4 c = codes16(q, sign);
        if (live) {
            *(uint4*)(codes + idx) = c;
            if (sub == 0)
                a_scale[(size_t)kb * M + m] = s;
        }
    }
}

// Route MX. The [M, K/32] groups are contiguous 32-element runs of x (K % 32 == 0), so group u
// starts at element 32u and its byte is e8m0[u]: 2 lanes per group, 32 groups per wave and pass,
// four passes per block.
template <int IN_BF16>
__global__ void __launch_bounds__(kQuantThreads) quantize_mx_kernel(const void* __restrict__ x,
                                                                    uint8_t* __restrict__ codes,
                                                                    uint8_t* __restrict__ e8m0, long long groups)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = lane & 1;
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
        const long long u = ((long long)blockIdx.x * 4 + pass) * 128 + 32 * wave + (lane >> 1);
        const bool live = u < groups;
        const long long uu = live ? u : groups - 1;
        const size_t idx = (size_t)uu * 32 + 16 * sub;
        float v[16];
        uint32_t sign[4];
        load16<IN_BF16>(x, idx, v, sign);
        float amax = amax16(v);
        amax = fmaxf(amax, __shfl_xor(amax, 1, 2));
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
        float q[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
            q[i] = ldexpf(v[i], -e);  // exact (results below 2^-126 encode as zero either way)
        const uint4 c = codes16(q, sign);
        if (live) {
            *(uint4*)(codes + idx) = c;
            if (sub == 0)
                e8m0[uu] = (uint8_t)(e + 127);
        }
    }
}

}  // namespace

hipError_t launch_quantize(int route, const void* x, int in_bf16, void* codes, void* scales, int M, int K,
                           hipStream_t stream)
{
    if (M == 0)
        return hipSuccess;
    if (route == kRouteBS) {
        const int MB = (M + 63) / 64;
        const int grid = MB * (K >> 7);  // M * K < 2^31, so this fits
        if (in_bf16)
            return launch_kernel(quantize_bs_kernel<1>, dim3(grid), dim3(kQuantThreads), stream, x, (uint8_t*)codes,
                                 (float*)scales, M, K, MB);
        return launch_kernel(quantize_bs_kernel<0>, dim3(grid), dim3(kQuantThreads), stream, x, (uint8_t*)codes,
                             (float*)scales, M, K, MB);
    }
    const long long groups = (long long)M * (K >> 5);
    const int grid = (int)((groups + 511) / 512);
    if (in_bf16)
        return launch_kernel(quantize_mx_kernel<1>, dim3(grid), dim3(kQuantThreads), stream, x, (uint8_t*)codes,
                             (uint8_t*)scales, groups);
    return launch_kernel(quantize_mx_kernel<0>, dim3(grid), dim3(kQuantThreads), stream, x, (uint8_t*)codes,
                         (uint8_t*)scales, groups);
}

}  // namespace fp8bs
