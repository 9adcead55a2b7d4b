// decode.hip -- the small-M ("decode") regime: few rows of activations against a weight
// matrix streamed once from HBM (page "Flydsl Fp8 Blockscale Gemm", When to use: the decode
// variants; page "aiter PR #6370", Not included: a separate GEMV-style kernel for M <= 32).
//
// With so few rows the GEMM is bound by reading B (N*K bytes) and a 128-row output tile would
// leave most of every matrix instruction idle, so the work is cut the other way: a workgroup
// owns one 16-row sub-tile of the prepared weights (16 output columns) and one chunk of up to
// 64 activation rows (grid y; more rows take more chunks, each re-reading the weights, mostly
// from L2), its waves split the K blocks between them, and each wave keeps a rows x 16 partial
// sum (per K block: one matrix instruction per 16 activation rows, then the route's scaling);
// the partials are added through LDS in a fixed order, so results are deterministic run to
// run and do not depend on the chunking. Two variants:
//  * direct: each wave loads its fragments straight from global memory into registers (16
//    bytes per lane, 64 contiguous bytes of each of 16 rows per instruction). Cheapest when
//    the activations are few (M <= 4) and a wave owns one or two K blocks.
//  * LDS-staged: each wave copies its K block's activation rows, weight rows and scales into a
//    double-buffered LDS region of its own with direct-to-LDS loads of whole 128-byte row
//    segments (8 rows per instruction, 16-byte chunks XOR-swizzled by (row >> 1) & 7), the next
//    block's copy in flight while the current one is computed; fragments are then read from
//    LDS. Every workgroup re-reads all M x K activation bytes (L2 hits), and whole-line loads
//    move them about twice as fast as the direct variant's half-line ones (measured: M = 64
//    against 2048 x 7168 weights 17.8 -> 7.3 us). No wave reads another wave's buffer, so
//    only the wave's own vmcnt is waited for.
// Routes:
//  * BS: unscaled instruction + promote acc += p * (a_s[kb, m] * b_s[n/128, kb]);
//  * MX: scaled instruction, activation exponents read row-major from a_e8m0 [M, K/32] (or,
//    kRouteMXPacked, as the packed dwords of fp8mx_pack_a_scale, the sub-tile picked by op_sel),
//    weight exponents from the packed buffer of fp8mx_prep_weights;
//  * PT: in-place accumulation, a_s[m] * b_s[n] applied once at the end.
#include "device.hpp"
#include "launch.hpp"

namespace fp8bs {

namespace {

constexpr int kDecodeWaves = 8;

constexpr bool is_mx(int route) { return route == kRouteMX || route == kRouteMXPacked; }

// Scaled instruction with the activation exponent taken from byte `sel` of a packed dword (the
// byte select must be a compile-time constant; sel is one after unrolling).
template <int SEL>
__device__ __forceinline__ v4f mfma_packed_sel(const v8i& b, const v8i& a, const v4f& c, int sb, int sa_dword)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, kFmtE4M3, kFmtE4M3, 0, sb, SEL, sa_dword);
}
__device__ __forceinline__ v4f mfma_packed(int sel, const v8i& b, const v8i& a, const v4f& c, int sb, int sa_dword)
{
    switch (sel & 3) {
    case 0:
        return mfma_packed_sel<0>(b, a, c, sb, sa_dword);
    case 1:
        return mfma_packed_sel<1>(b, a, c, sb, sa_dword);
    case 2:
        return mfma_packed_sel<2>(b, a, c, sb, sa_dword);
    default:
        return mfma_packed_sel<3>(b, a, c, sb, sa_dword);
    }
}

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
decode_direct_kernel(const uint8_t* __restrict__ A, const void* __restrict__ a_scale, const uint8_t* __restrict__ B,
              const void* __restrict__ b_scale, uint16_t* __restrict__ C, int M, int N, int K)
{
    __shared__ v4f red[kDecodeWaves][SI][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15, q = lane >> 4;
    const int jt = blockIdx.x;  // 16-row sub-tile of the prepared weights
    const int m0 = blockIdx.y * kDecodeMaxRows;  // first activation row of the chunk
    const int KB = K >> 7;
    const int kb0 = (wave * KB) / kDecodeWaves, kb1 = ((wave + 1) * KB) / kDecodeWaves;
    const size_t brow = (size_t)jt * 16 + i;
    int arow[SI];
#pragma unroll
    for (int si = 0; si < SI; ++si)
        arow[si] = min(m0 + 16 * si + i, M - 1);  // rows past M repeat row M-1 and are not stored

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
            // packed activation exponents: dword (kb * M/64 + chunk) * 64 + lane, byte = sub-tile
            uint32_t ad = 0;
            if constexpr (ROUTE == kRouteMXPacked)
                ad = ((const uint32_t*)a_scale)[((size_t)kb * (M >> 6) + blockIdx.y) * 64 + lane];
#pragma unroll
            for (int si = 0; si < SI; ++si) {
                const v8i af = load_frag(A, arow[si], K, kb, q);
                if constexpr (ROUTE == kRouteMXPacked) {
                    acc[si] = mfma_packed(si, bf, af, acc[si], sbyte, (int)ad);
                } else {
                    const int sabyte = ((const uint8_t*)a_scale)[(size_t)arow[si] * G + 4 * kb + q];
                    acc[si] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af, acc[si], kFmtE4M3, kFmtE4M3,
                                                                              0, sbyte, 0, sabyte);
                }
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
        const int m = m0 + 16 * si + i;
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

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ v4i dbuf_desc(const void* base)
{
    const uint64_t a = (uint64_t)base;
    return v4i{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), 0x7FFFFFFF, 0x00020000};
}

template <int BYTES>
__device__ __forceinline__ void dma(const v4i& rs, uint32_t dst, int voff, int soff)
{
    if constexpr (BYTES == 16)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     :
                     : "s"(dst), "v"(voff), "s"(rs), "s"(soff)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                     :
                     : "s"(dst), "v"(voff), "s"(rs), "s"(soff)
                     : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ uint32_t swz(uint32_t row) { return (row >> 1) & 7u; }

// Per-wave LDS buffer of one K block: [A: 16*SI rows x 128 B][B: 16*JT rows x 128 B][scales
// 512 B]; JT = 16-row weight sub-tiles per workgroup
template <int ROUTE, int SI, int JT>
struct DBuf {
    static constexpr int kA = 16 * SI * 128;
    static constexpr int kB = 16 * JT * 128;
    static constexpr int kS = ROUTE == kRoutePT ? 0 : 512;  // a_s / a_e8m0 in [0, 256), b_s in [256, 512)
    static constexpr int kBytes = kA + kB + kS;
    static constexpr int kLoads = 2 * SI + 2 * JT + (ROUTE == kRoutePT ? 0 : 2);
};

// LDS: two buffers per wave
template <int SI, int JT>
constexpr int waves_for() { return SI == 4 ? 7 : kDecodeWaves; }

template <int ROUTE, int SI, int JT>
__global__ void __launch_bounds__((waves_for<SI, JT>() * 64))
decode_lds_kernel(const uint8_t* __restrict__ A, const void* __restrict__ a_scale, const uint8_t* __restrict__ B,
              const void* __restrict__ b_scale, uint16_t* __restrict__ C, int M, int N, int K)
{
    static_assert(JT == 1 || (JT == 2 && SI <= 2), "two weight sub-tiles per workgroup up to 32 rows");
    using D = DBuf<ROUTE, SI, JT>;
    constexpr int NW = waves_for<SI, JT>();
    static_assert(2 * NW * D::kBytes <= 160 * 1024, "LDS");
    static_assert(NW * SI * JT * 64 * 16 <= 2 * NW * D::kBytes, "reduction fits the operand buffers");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * NW * D::kBytes];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15, q = lane >> 4;
    const int jt = blockIdx.x * JT;  // first 16-row sub-tile of the prepared weights
    const int m0 = blockIdx.y * kDecodeMaxRows;  // first activation row of the chunk
    const int KB = K >> 7;
    const int kb0 = (wave * KB) / NW, kb1 = ((wave + 1) * KB) / NW;
    const v4i rsA = dbuf_desc(A), rsB = dbuf_desc(B), rsSA = dbuf_desc(a_scale), rsSB = dbuf_desc(b_scale);
    uint8_t* mybuf = lds + wave * 2 * D::kBytes;

    // DMA lane offsets (without the K block term): A group g covers rows m0+8g .. m0+8g+7
    // (clamped to M-1), B group g rows 8g..8g+7 of the sub-tiles; lane l -> row l/8, physical
    // chunk l%8 holding logical chunk (l%8) ^ swz(row)
    const int r8 = lane >> 3, c8 = lane & 7;
    int voffA[2 * SI];
#pragma unroll
    for (int g = 0; g < 2 * SI; ++g) {
        const int row = 8 * g + r8;
        voffA[g] = min(m0 + row, M - 1) * K + ((c8 ^ (int)swz(row)) << 4);
    }
    int voffB[2 * JT];
#pragma unroll
    for (int g = 0; g < 2 * JT; ++g) {
        const int row = 8 * g + r8;
        voffB[g] = (jt * 16 + row) * K + ((c8 ^ (int)swz(row)) << 4);
    }
    // scales: BS a_s[kb*M + m] (lane = row m - m0), b_s[nb*KB + kb]; MX a_e8m0 dword of row m
    // at K block kb, packed weight dword ((kb*N/64 + window)*64 + lane)
    int voffSA = 0, voffSB = 0;
    if constexpr (ROUTE == kRouteBS) {
        voffSA = min(m0 + lane, M - 1) * 4;
        voffSB = (jt >> 3) * KB * 4;
    } else if constexpr (ROUTE == kRouteMX) {
        voffSA = min(m0 + lane, M - 1) * (K >> 5);
        voffSB = ((jt >> 2) * 64 + lane) * 4;
    } else if constexpr (ROUTE == kRouteMXPacked) {  // packed dword (kb*M/64 + chunk)*64 + lane
        voffSA = ((int)blockIdx.y * 64 + lane) * 4;
        voffSB = ((jt >> 2) * 64 + lane) * 4;
    }

    auto issue = [&](int kb, int b) {
        uint8_t* base = mybuf + b * D::kBytes;
        const uint32_t sb = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(lds_u8*)base);
        const int koff = __builtin_amdgcn_readfirstlane(kb * 128);
#pragma unroll
        for (int g = 0; g < 2 * SI; ++g)
            dma<16>(rsA, sb + g * 1024, voffA[g], koff);
#pragma unroll
        for (int g = 0; g < 2 * JT; ++g)
            dma<16>(rsB, sb + D::kA + g * 1024, voffB[g], koff);
        if constexpr (ROUTE == kRouteBS) {
            dma<4>(rsSA, sb + D::kA + D::kB, voffSA, __builtin_amdgcn_readfirstlane(kb * M * 4));
            dma<4>(rsSB, sb + D::kA + D::kB + 256, voffSB, __builtin_amdgcn_readfirstlane(kb * 4));
        } else if constexpr (is_mx(ROUTE)) {
            const int soff_a = ROUTE == kRouteMX ? kb * 4 : kb * (M >> 6) * 256;
            dma<4>(rsSA, sb + D::kA + D::kB, voffSA, __builtin_amdgcn_readfirstlane(soff_a));
            dma<4>(rsSB, sb + D::kA + D::kB + 256, voffSB, __builtin_amdgcn_readfirstlane(kb * (N >> 6) * 256));
        }
    };
    const uint32_t c_lo = ((q ^ swz(i)) << 4) + i * 128u;
    const uint32_t c_hi = (((q + 4u) ^ swz(i)) << 4) + i * 128u;
    auto frag = [&](const uint8_t* base) -> v8i {
        const v4i lo = *(const v4i*)(base + c_lo);
        const v4i hi = *(const v4i*)(base + c_hi);
        return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    };

    v4f acc[JT][SI];
#pragma unroll
    for (int t = 0; t < JT; ++t)
#pragma unroll
        for (int si = 0; si < SI; ++si)
            acc[t][si] = v4f{0.f, 0.f, 0.f, 0.f};

    if (kb0 < kb1)
        issue(kb0, 0);
    for (int kb = kb0; kb < kb1; ++kb) {
        const int b = (kb - kb0) & 1;
        if (kb + 1 < kb1) {
            issue(kb + 1, b ^ 1);
            wait_vm<D::kLoads>();
        } else {
            wait_vm<0>();
        }
        asm volatile("" ::: "memory");  // the buffer's reads stay below the wait
        const uint8_t* base = mybuf + b * D::kBytes;
        v8i af[SI];
#pragma unroll
        for (int si = 0; si < SI; ++si)
            af[si] = frag(base + si * 16 * 128);
        // the JT sub-tiles share their 128-row weight-scale block and 64-row exponent window
#pragma unroll
        for (int t = 0; t < JT; ++t) {
            const v8i bf = frag(base + D::kA + t * 16 * 128);
            if constexpr (ROUTE == kRouteBS) {
                const float sb = *(const float*)(base + D::kA + D::kB + 256);
#pragma unroll
                for (int si = 0; si < SI; ++si) {
                    const float sa = ((const float*)(base + D::kA + D::kB))[16 * si + i];  // row m0+16si+i, clamped
                    const v4f p = mfma_f8(bf, af[si], v4f{0.f, 0.f, 0.f, 0.f});
                    acc[t][si] += p * (sa * sb);
                }
            } else if constexpr (ROUTE == kRoutePT) {
#pragma unroll
                for (int si = 0; si < SI; ++si)
                    acc[t][si] = mfma_f8(bf, af[si], acc[t][si]);
            } else {
                const uint32_t wd = ((const uint32_t*)(base + D::kA + D::kB + 256))[lane];
                const int sbyte = (int)((wd >> (8 * ((jt + t) & 3))) & 0xffu);
                const uint32_t apk = ((const uint32_t*)(base + D::kA + D::kB))[lane];  // packed: this lane's dword
#pragma unroll
                for (int si = 0; si < SI; ++si) {
                    if constexpr (ROUTE == kRouteMXPacked) {
                        acc[t][si] = mfma_packed(si, bf, af[si], acc[t][si], sbyte, (int)apk);
                    } else {
                        const uint32_t ad = ((const uint32_t*)(base + D::kA + D::kB))[16 * si + i];
                        const int sabyte = (int)((ad >> (8 * q)) & 0xffu);
                        acc[t][si] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            bf, af[si], acc[t][si], kFmtE4M3, kFmtE4M3, 0, sbyte, 0, sabyte);
                    }
                }
            }
        }
        // every read of this buffer is done before the next iteration's loads refill it
        __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));
    }

    __syncthreads();  // reduction storage reuses the operand buffers
    v4f* red = (v4f*)lds;  // [wave][t][si][64]
#pragma unroll
    for (int t = 0; t < JT; ++t)
#pragma unroll
        for (int si = 0; si < SI; ++si)
            red[((wave * JT + t) * SI + si) * 64 + lane] = acc[t][si];
    __syncthreads();
    if (wave < SI) {
        // sub-tiles jt and jt+1 (jt even) hold output columns n..n+3 and n+4..n+7
        const int si = wave;
        const int m = m0 + 16 * si + i;
        const int n = 64 * (jt >> 2) + 32 * ((jt & 3) >> 1) + 8 * q + 4 * (jt & 1);
        v4f s[JT];
#pragma unroll
        for (int t = 0; t < JT; ++t) {
            s[t] = red[(t * SI + si) * 64 + lane];
#pragma unroll
            for (int w = 1; w < NW; ++w)
                s[t] += red[((w * JT + t) * SI + si) * 64 + lane];
            if constexpr (ROUTE == kRoutePT) {
                const float sa = ((const float*)a_scale)[min(m, M - 1)];
                const v4f sbv = *(const v4f*)((const float*)b_scale + n + 4 * t);
                s[t] = s[t] * (sbv * sa);
            }
        }
        if (m < M) {
            if constexpr (JT == 2) {
                v4i packed;
                packed.x = (int)pack_bf16x2(s[0].x, s[0].y);
                packed.y = (int)pack_bf16x2(s[0].z, s[0].w);
                packed.z = (int)pack_bf16x2(s[1].x, s[1].y);
                packed.w = (int)pack_bf16x2(s[1].z, s[1].w);
                *(v4i*)(C + (size_t)m * N + n) = packed;
            } else {
                v2i packed;
                packed.x = (int)pack_bf16x2(s[0].x, s[0].y);
                packed.y = (int)pack_bf16x2(s[0].z, s[0].w);
                *(v2i*)(C + (size_t)m * N + n) = packed;
            }
        }
    }
}

template <int ROUTE, int SI>
hipError_t launch_one(int variant, const GemmArgs& a)
{
    const int chunks = (a.M + kDecodeMaxRows - 1) / kDecodeMaxRows;
    const uint8_t* A = (const uint8_t*)a.A;
    const uint8_t* B = (const uint8_t*)a.B;
    uint16_t* C = (uint16_t*)a.C;
    if (variant == kDecodeLdsPair) {
        if constexpr (SI <= 2)
            return launch_kernel(decode_lds_kernel<ROUTE, SI, 2>, dim3(a.N / 32, chunks), dim3(waves_for<SI, 2>() * 64),
                                 a.stream, A, a.a_scale, B, a.b_scale, C, a.M, a.N, a.K);
        else
            return hipErrorInvalidValue;
    }
    if (variant == kDecodeLds)
        return launch_kernel(decode_lds_kernel<ROUTE, SI, 1>, dim3(a.N / 16, chunks), dim3(waves_for<SI, 1>() * 64),
                             a.stream, A, a.a_scale, B, a.b_scale, C, a.M, a.N, a.K);
    return launch_kernel(decode_direct_kernel<ROUTE, SI>, dim3(a.N / 16, chunks), dim3(kDecodeWaves * 64), a.stream,
                         A, a.a_scale, B, a.b_scale, C, a.M, a.N, a.K);
}

template <int ROUTE>
hipError_t launch_route(int si, int variant, const GemmArgs& a)
{
    switch (si) {
    case 1:
        return launch_one<ROUTE, 1>(variant, a);
    case 2:
        return launch_one<ROUTE, 2>(variant, a);
    case 3:
        return launch_one<ROUTE, 3>(variant, a);
    default:
        return launch_one<ROUTE, 4>(variant, a);
    }
}

}  // namespace

hipError_t launch_decode(int route, const GemmArgs& a, int variant)
{
    if (a.M <= 0 || (a.M + kDecodeMaxRows - 1) / kDecodeMaxRows > kDecodeMaxChunks || a.N % 64 != 0 ||
        a.K % 128 != 0)
        return hipErrorInvalidValue;
    if (variant == kDecodeLdsPair && (min(a.M, kDecodeMaxRows) > 32 || a.N % 32 != 0))
        return hipErrorInvalidValue;
    if (variant == kDecodeAuto) {
        // the LDS-staged variant unless the activations are few and every wave owns at most two
        // K blocks (there the extra LDS round trip is not repaid: 1 x 65536 x 1536 direct 16.3
        // us, staged 18.1; 64 x 2048 x 7168 direct 17.8, staged 7.3)
        const int blocks_per_wave = ((a.K >> 7) + kDecodeWaves - 1) / kDecodeWaves;
        variant = (a.M > 4 || blocks_per_wave >= 3) ? kDecodeLds : kDecodeDirect;
        // 17 to 32 rows: two weight sub-tiles per workgroup halve the activation re-reads (7168 x
        // 7168 weights, M = 32: 10.0 against 11.8 us; 16384 x 4096: 13.3 against 16.1), while
        // the grid keeps 192 workgroups (4096 x 4096: 5.2 against 4.6; 2048 x 7168: 6.1 against
        // 5.1) and K <= 7168 (28672 x 8192, already near HBM speed: 50.3 against 43.0); with at
        // most 16 rows they lose
        const int rows = min(a.M, kDecodeMaxRows);
        const int chunks = (a.M + kDecodeMaxRows - 1) / kDecodeMaxRows;
        if (variant == kDecodeLds && rows > 16 && rows <= 32 && a.N % 32 == 0 && (a.N / 32) * chunks >= 192 &&
            a.K <= 7168)
            variant = kDecodeLdsPair;
    }
    const int si = (min(a.M, kDecodeMaxRows) + 15) / 16;
    if (route == kRouteBS)
        return launch_route<kRouteBS>(si, variant, a);
    if (route == kRoutePT)
        return launch_route<kRoutePT>(si, variant, a);
    if (route == kRouteMXPacked)
        return launch_route<kRouteMXPacked>(si, variant, a);
    return launch_route<kRouteMX>(si, variant, a);
}

}  // namespace fp8bs
