// decode.hip -- the small-M ("decode") regime: M <= 64 rows of activations against a weight
// matrix streamed once from HBM (page "Flydsl Fp8 Blockscale Gemm", When to use: the decode
// variants; page "aiter PR #6370", Not included: a separate GEMV-style kernel for M <= 32).
//
// With so few rows the GEMM is bound by reading B (N*K bytes) and a 128-row output tile would
// leave most of every matrix instruction idle, so the work is cut the other way: a workgroup
// of 8 waves owns one 16-row sub-tile of the prepared weights (16 output columns), the 8 waves
// split the K blocks between them, and each wave loads its fragments straight from global
// memory into registers (no LDS staging: every weight byte is used once). Each wave keeps an
// M x 16 partial sum (per K block: one matrix instruction per 16 activation rows, then the
// route's scaling); the 8 partials are added through LDS in a fixed order, so results are
// deterministic run to run. Routes:
//  * BS: unscaled instruction + promote acc += p * (a_s[kb, m] * b_s[n/128, kb]);
//  * MX: scaled instruction, activation exponents read row-major from a_e8m0 [M, K/32], weight
//    exponents from the packed buffer of fp8mx_prep_weights;
//  * PT: in-place accumulation, a_s[m] * b_s[n] applied once at the end.
#include "device.hpp"
#include "launch.hpp"

namespace fp8bs {

namespace {

constexpr int kDecodeWaves = 8;

// Lane l = i + 16q reads bytes [16q, 16q+16) and [64+16q, 64+16q+16) of the 128-byte K block of
// row `row` (the fragment layout of the 16x16x128 instruction).
__device__ __forceinline__ v8i load_frag(const uint8_t* base, size_t row, int K, int kb, int q)
{
    const uint8_t* p = base + row * (size_t)K + (size_t)kb * 128 + 16 * q;
    const v4i lo = *(const v4i*)p;
    const v4i hi = *(const v4i*)(p + 64);
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

template <int ROUTE, int SI>
__global__ void __launch_bounds__(kDecodeWaves * 64)
decode_kernel(const uint8_t* __restrict__ A, const void* __restrict__ a_scale, const uint8_t* __restrict__ B,
              const void* __restrict__ b_scale, uint16_t* __restrict__ C, int M, int N, int K)
{
    __shared__ v4f red[kDecodeWaves][SI][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15, q = lane >> 4;
    const int jt = blockIdx.x;  // 16-row sub-tile of the prepared weights
    const int KB = K >> 7;
    const int kb0 = (wave * KB) / kDecodeWaves, kb1 = ((wave + 1) * KB) / kDecodeWaves;
    const size_t brow = (size_t)jt * 16 + i;
    int arow[SI];
#pragma unroll
    for (int si = 0; si < SI; ++si)
        arow[si] = min(16 * si + i, M - 1);  // rows past M repeat row M-1 and are not stored

    v4f acc[SI];
#pragma unroll
    for (int si = 0; si < SI; ++si)
        acc[si] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll 2
    for (int kb = kb0; kb < kb1; ++kb) {
        const v8i bf = load_frag(B, brow, K, kb, q);
        if constexpr (ROUTE == kRouteBS) {
            const int nb = jt >> 3;  // the sub-tile's 16 weight rows lie in 128-row block jt / 8
            const float sb = ((const float*)b_scale)[(size_t)nb * KB + kb];
#pragma unroll
            for (int si = 0; si < SI; ++si) {
                const v8i af = load_frag(A, arow[si], K, kb, q);
                const float sa = ((const float*)a_scale)[(size_t)kb * M + arow[si]];
                const v4f p = mfma_f8(bf, af, v4f{0.f, 0.f, 0.f, 0.f});
                acc[si] += p * (sa * sb);
            }
        } else if constexpr (ROUTE == kRoutePT) {
#pragma unroll
            for (int si = 0; si < SI; ++si)
                acc[si] = mfma_f8(bf, load_frag(A, arow[si], K, kb, q), acc[si]);
        } else {
            // weight exponents: packed dword (kb * N/64 + window) * 64 + lane, byte = sub-tile
            // index inside the 64-row window; activation exponent of (row i, K group q)
            const uint32_t wd = ((const uint32_t*)b_scale)[((size_t)kb * (N >> 6) + (jt >> 2)) * 64 + lane];
            const int sbyte = (int)((wd >> (8 * (jt & 3))) & 0xffu);
            const int G = K >> 5;
#pragma unroll
            for (int si = 0; si < SI; ++si) {
                const v8i af = load_frag(A, arow[si], K, kb, q);
                const int sabyte = ((const uint8_t*)a_scale)[(size_t)arow[si] * G + 4 * kb + q];
                acc[si] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af, acc[si], kFmtE4M3, kFmtE4M3, 0,
                                                                          sbyte, 0, sabyte);
            }
        }
    }

#pragma unroll
    for (int si = 0; si < SI; ++si)
        red[wave][si][lane] = acc[si];
    __syncthreads();
    if (wave < SI) {
        const int si = wave;
        v4f s = red[0][si][lane];
#pragma unroll
        for (int w = 1; w < kDecodeWaves; ++w)
            s += red[w][si][lane];
        const int m = 16 * si + i;
        // result register r of lane group q is prepared row 16*(jt%4) + 4q + r of the 64-row
        // window, i.e. output column 64*(jt/4) + 32*((jt%4)/2) + 8q + 4*(jt%2) + r
        const int n = 64 * (jt >> 2) + 32 * ((jt & 3) >> 1) + 8 * q + 4 * (jt & 1);
        if constexpr (ROUTE == kRoutePT) {
            const float sa = ((const float*)a_scale)[min(m, M - 1)];
            const v4f sb = *(const v4f*)((const float*)b_scale + n);
            s = s * (sb * sa);
        }
        if (m < M) {
            v2i packed;
            packed.x = (int)pack_bf16x2(s.x, s.y);
            packed.y = (int)pack_bf16x2(s.z, s.w);
            *(v2i*)(C + (size_t)m * N + n) = packed;
        }
    }
}

template <int ROUTE>
hipError_t launch_route(int si, const GemmArgs& a)
{
    const dim3 grid(a.N / 16), block(kDecodeWaves * 64);
    const uint8_t* A = (const uint8_t*)a.A;
    const uint8_t* B = (const uint8_t*)a.B;
    uint16_t* C = (uint16_t*)a.C;
    switch (si) {
    case 1:
        hipLaunchKernelGGL((decode_kernel<ROUTE, 1>), grid, block, 0, a.stream, A, a.a_scale, B, a.b_scale, C, a.M,
                           a.N, a.K);
        break;
    case 2:
        hipLaunchKernelGGL((decode_kernel<ROUTE, 2>), grid, block, 0, a.stream, A, a.a_scale, B, a.b_scale, C, a.M,
                           a.N, a.K);
        break;
    case 3:
        hipLaunchKernelGGL((decode_kernel<ROUTE, 3>), grid, block, 0, a.stream, A, a.a_scale, B, a.b_scale, C, a.M,
                           a.N, a.K);
        break;
    default:
        hipLaunchKernelGGL((decode_kernel<ROUTE, 4>), grid, block, 0, a.stream, A, a.a_scale, B, a.b_scale, C, a.M,
                           a.N, a.K);
        break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(int route, const GemmArgs& a)
{
    if (a.M <= 0 || a.M > kDecodeMaxRows || a.N % 64 != 0 || a.K % 128 != 0)
        return hipErrorInvalidValue;
    const int si = (a.M + 15) / 16;
    if (route == kRouteBS)
        return launch_route<kRouteBS>(si, a);
    if (route == kRoutePT)
        return launch_route<kRoutePT>(si, a);
    return launch_route<kRouteMX>(si, a);
}

}  // namespace fp8bs
