// mx_gemm.hip -- route MX: fp8 e4m3 GEMM with 1x32 ue8m0 scales on both operands, applied by
// the scaled matrix-core instruction (page "aiter PR #6370", "Why it is faster"): one
// v_mfma_scale_f32_16x16x128_f8f6f4 consumes a whole 128-wide K step with its four 32-wide
// groups already scaled by powers of two, so there is a single fp32 accumulator and no
// software promote.
//
// Scale feed: both scale operands arrive packed K-block-major, four bytes to a dword (the
// packing is done once by fp8mx_pack_a_scale / fp8mx_prep_weights). For one 128-wide K step
// and one 64-row group, lane i + 16g of a wave reads dword ((kstep * R/64 + group) * 64 + lane),
// whose byte t is the exponent of row 16t + i over K group g -- one coalesced 256-byte load
// per wave, and the four 16-row sub-tiles of the group pick their byte with op_sel at no
// VALU cost (same page, second bullet).
#include "device.hpp"
#include "launch.hpp"

#include <utility>

namespace fp8bs {

template <int I, int J>
__device__ __forceinline__ v4f mfma_mx(const v8i& w, const v8i& x, const v4f& c, int ws, int xs) {
    // weights first (swap-AB): op_sel of the weight scale selects sub-tile J's byte, op_sel of
    // the activation scale selects sub-tile I's byte.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, x, c, kFmtE4M3, kFmtE4M3, J, ws, I, xs);
}

template <int SI, int SJ, int I = 0, int J = 0>
__device__ __forceinline__ void mx_block(v4f (&acc)[SI][SJ], const v8i (&af)[SI], const v8i (&bf)[SJ],
                                         int sa, int sb) {
    if constexpr (I < SI) {
        if constexpr (J < SJ) {
            acc[I][J] = mfma_mx<I, J>(bf[J], af[I], acc[I][J], sb, sa);
            mx_block<SI, SJ, I, J + 1>(acc, af, bf, sa, sb);
        } else {
            mx_block<SI, SJ, I + 1, 0>(acc, af, bf, sa, sb);
        }
    }
}

template <int BM, int BN, int WM, int WN>
struct MxTile {
    static constexpr int kThreads = WM * WN * 64;
    static constexpr int TM = BM / WM;
    static constexpr int TN = BN / WN;
    static constexpr int SI = TM / 16;
    static constexpr int SJ = TN / 16;
    static constexpr int kChunksA = BM * 8 / kThreads;
    static constexpr int kChunksB = BN * 8 / kThreads;
    static constexpr int kStageBytes = (BM + BN) * 128;
    static constexpr int kLdsBytes = 2 * kStageBytes;
    static_assert(TM == 64 && TN == 64, "one packed 64-row scale group per wave and operand");
    static_assert((BM * 8) % kThreads == 0 && (BN * 8) % kThreads == 0, "even chunk split");
};

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(WM * WN * 64)
mx_gemm_kernel(const uint8_t* __restrict__ A, const uint32_t* __restrict__ a_packed,
               const uint8_t* __restrict__ B, const uint32_t* __restrict__ b_packed,
               uint16_t* __restrict__ C, int M, int N, int K, int tiles_n)
{
    using T = MxTile<BM, BN, WM, WN>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WM;
    const int wn = wave / WM;
    const int tm = blockIdx.x / tiles_n;
    const int tn = blockIdx.x % tiles_n;
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int KS = K >> 7;
    const int groups_m = M >> 6;
    const int groups_n = N >> 6;

    v4i ga[T::kChunksA];
    v4i gb[T::kChunksB];
    auto gload = [&](int ks) {
        const size_t kofs = (size_t)ks * 128;
#pragma unroll
        for (int c = 0; c < T::kChunksA; ++c) {
            const int id = c * T::kThreads + tid;
            const int row = id >> 3, ch = id & 7;
            const int m = min(m0 + row, M - 1);  // rows past M are read but never stored
            ga[c] = *(const v4i*)(A + (size_t)m * K + kofs + ch * 16);
        }
#pragma unroll
        for (int c = 0; c < T::kChunksB; ++c) {
            const int id = c * T::kThreads + tid;
            const int row = id >> 3, ch = id & 7;
            gb[c] = *(const v4i*)(B + (size_t)(n0 + row) * K + kofs + ch * 16);
        }
    };
    auto lstore = [&](int stage) {
        uint8_t* sA = smem + stage * T::kStageBytes;
        uint8_t* sB = sA + BM * 128;
#pragma unroll
        for (int c = 0; c < T::kChunksA; ++c) {
            const int id = c * T::kThreads + tid;
            *(v4i*)(sA + lds_tile_offset(id >> 3, id & 7)) = ga[c];
        }
#pragma unroll
        for (int c = 0; c < T::kChunksB; ++c) {
            const int id = c * T::kThreads + tid;
            *(v4i*)(sB + lds_tile_offset(id >> 3, id & 7)) = gb[c];
        }
    };

    const int mg = min((m0 + wm * T::TM) >> 6, groups_m - 1);
    const int ng = (n0 + wn * T::TN) >> 6;
    int sa_next, sb_next;
    auto sload = [&](int ks) {
        sa_next = (int)a_packed[((size_t)ks * groups_m + mg) * 64 + lane];
        sb_next = (int)b_packed[((size_t)ks * groups_n + ng) * 64 + lane];
    };

    v4f acc[T::SI][T::SJ];
#pragma unroll
    for (int i = 0; i < T::SI; ++i)
#pragma unroll
        for (int j = 0; j < T::SJ; ++j)
            acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int frag_chunk = lane >> 4;
    const int frag_row = lane & 15;

    sload(0);
    gload(0);
    lstore(0);
    __syncthreads();

    for (int ks = 0; ks < KS; ++ks) {
        const int stage = ks & 1;
        const int sa = sa_next, sb = sb_next;
        if (ks + 1 < KS) {
            sload(ks + 1);
            gload(ks + 1);
        }
        const uint8_t* sA = smem + stage * T::kStageBytes;
        const uint8_t* sB = sA + BM * 128;
        v8i af[T::SI];
        v8i bf[T::SJ];
#pragma unroll
        for (int i = 0; i < T::SI; ++i) {
            const int r = wm * T::TM + 16 * i + frag_row;
            const v4i lo = *(const v4i*)(sA + lds_tile_offset(r, frag_chunk));
            const v4i hi = *(const v4i*)(sA + lds_tile_offset(r, frag_chunk + 4));
            af[i] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        }
#pragma unroll
        for (int j = 0; j < T::SJ; ++j) {
            const int r = wn * T::TN + 16 * j + frag_row;
            const v4i lo = *(const v4i*)(sB + lds_tile_offset(r, frag_chunk));
            const v4i hi = *(const v4i*)(sB + lds_tile_offset(r, frag_chunk + 4));
            bf[j] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        }
        mx_block<T::SI, T::SJ>(acc, af, bf, sa, sb);

        if (ks + 1 < KS)
            lstore(stage ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < T::SI; ++i) {
        const int m = m0 + wm * T::TM + 16 * i + frag_row;
        if (m >= M)
            continue;
        uint16_t* crow = C + (size_t)m * N + n0 + wn * T::TN + 4 * (lane >> 4);
#pragma unroll
        for (int j = 0; j < T::SJ; ++j) {
            const v4f v = acc[i][j];
            v2i packed;
            packed.x = (int)pack_bf16x2(v.x, v.y);
            packed.y = (int)pack_bf16x2(v.z, v.w);
            *(v2i*)(crow + 16 * j) = packed;
        }
    }
}

template <int BM, int BN, int WM, int WN>
static hipError_t launch_mx_tile(const MxArgs& a)
{
    using T = MxTile<BM, BN, WM, WN>;
    auto kern = mx_gemm_kernel<BM, BN, WM, WN>;
    static bool attr_done = false;
    if (!attr_done) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           T::kLdsBytes);
        if (e != hipSuccess)
            return e;
        attr_done = true;
    }
    const int tiles_m = (a.M + BM - 1) / BM;
    const int tiles_n = a.N / BN;
    hipLaunchKernelGGL(kern, dim3(tiles_m * tiles_n), dim3(T::kThreads), T::kLdsBytes, a.stream,
                       (const uint8_t*)a.A, (const uint32_t*)a.a_packed, (const uint8_t*)a.B,
                       (const uint32_t*)a.b_packed, (uint16_t*)a.C, a.M, a.N, a.K, tiles_n);
    return hipGetLastError();
}

hipError_t launch_mx(const MxArgs& a)
{
    if (a.N % 128 == 0)
        return launch_mx_tile<128, 128, 2, 2>(a);
    return launch_mx_tile<128, 64, 2, 1>(a);
}

}  // namespace fp8bs
