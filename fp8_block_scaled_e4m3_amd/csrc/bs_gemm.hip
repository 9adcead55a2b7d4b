// bs_gemm.hip -- route BS: fp8 e4m3 GEMM with fp32 per-1x128 activation scales and fp32
// per-128x128 weight scales, software-promoted after an unscaled matrix-core product.
//
// Method (page "Flydsl Fp8 Blockscale Gemm", Mechanism A): the fp32 block scales cannot be
// expressed by the matrix core's power-of-two scale operands, so each 128-wide K block is
// multiplied unscaled into a fresh fp32 partial, which is then multiplied by
// a_s[m,kb] * b_s[n/128,kb] and added to a running fp32 accumulator ("promote"), once per
// K block. With the 16x16x128 instruction one K block of one 16x16 output tile is exactly
// one instruction, so the partial is four registers that die right after their promote.
//
// Work decomposition: a workgroup owns a BM x BN tile of C and walks K in 128-wide blocks.
// Per block, the A rows [BM x 128] and B rows [BN x 128] are staged global -> registers ->
// LDS (double-buffered, one barrier per block); each wave reads its operand fragments from
// LDS and runs (TM/16) x (TN/16) instructions with the weights as the first operand, so
// every lane owns four consecutive columns of one output row.
#include "device.hpp"
#include "launch.hpp"

namespace fp8bs {

template <int BM, int BN, int WM, int WN>
struct BsTile {
    static constexpr int kThreads = WM * WN * 64;
    static constexpr int TM = BM / WM;  // rows of C per wave
    static constexpr int TN = BN / WN;  // columns of C per wave
    static constexpr int SI = TM / 16;  // 16-row sub-tiles per wave
    static constexpr int SJ = TN / 16;  // 16-column sub-tiles per wave
    static constexpr int kChunksA = BM * 8 / kThreads;  // 16-byte chunks per thread per block
    static constexpr int kChunksB = BN * 8 / kThreads;
    static constexpr int kStageBytes = (BM + BN) * 128;
    static constexpr int kLdsBytes = 2 * kStageBytes;
    static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "tile must split into 16x16 sub-tiles");
    static_assert((BM * 8) % kThreads == 0 && (BN * 8) % kThreads == 0, "even chunk split");
    static_assert(TN <= 128 && 128 % TN == 0, "a wave's columns must sit in one 128-row weight-scale block");
};

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(WM * WN * 64)
bs_gemm_kernel(const uint8_t* __restrict__ A, const float* __restrict__ a_scale,
               const uint8_t* __restrict__ B, const float* __restrict__ b_scale,
               uint16_t* __restrict__ C, int M, int N, int K, int tiles_n)
{
    using T = BsTile<BM, BN, WM, WN>;
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
    const int KB = K >> 7;

    // ---- global -> register staging of one K block --------------------------------------
    v4i ga[T::kChunksA];
    v4i gb[T::kChunksB];
    auto gload = [&](int kb) {
        const size_t kofs = (size_t)kb * 128;
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

    // ---- per-lane scale bookkeeping ----------------------------------------------------
    // With the weights as first operand, lane l's results of sub-tile (i, j) all belong to
    // output row 16*i + l%16 of the wave's rows, so one activation scale per sub-tile row.
    int srow[T::SI];
#pragma unroll
    for (int i = 0; i < T::SI; ++i)
        srow[i] = min(m0 + wm * T::TM + 16 * i + (lane & 15), M - 1);
    const float* bsc_row = b_scale + (size_t)((n0 + wn * T::TN) >> 7) * KB;
    float sa_next[T::SI];
    float sb_next;
    auto sload = [&](int kb) {
#pragma unroll
        for (int i = 0; i < T::SI; ++i)
            sa_next[i] = a_scale[(size_t)kb * M + srow[i]];
        sb_next = bsc_row[kb];
    };

    v4f acc[T::SI][T::SJ];
#pragma unroll
    for (int i = 0; i < T::SI; ++i)
#pragma unroll
        for (int j = 0; j < T::SJ; ++j)
            acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int frag_chunk = lane >> 4;  // this lane's operand bytes: chunks q and q + 4
    const int frag_row = lane & 15;

    sload(0);
    gload(0);
    lstore(0);
    __syncthreads();

    for (int kb = 0; kb < KB; ++kb) {
        const int stage = kb & 1;
        float sa[T::SI];
#pragma unroll
        for (int i = 0; i < T::SI; ++i)
            sa[i] = sa_next[i];
        const float sb = sb_next;
        if (kb + 1 < KB) {
            sload(kb + 1);
            gload(kb + 1);
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
#pragma unroll
        for (int i = 0; i < T::SI; ++i) {
            const float s = sa[i] * sb;
#pragma unroll
            for (int j = 0; j < T::SJ; ++j) {
                const v4f p = mfma_f8(bf[j], af[i], v4f{0.f, 0.f, 0.f, 0.f});
                acc[i][j] += p * s;
            }
        }

        if (kb + 1 < KB)
            lstore(stage ^ 1);
        __syncthreads();
    }

    // ---- epilogue: fp32 -> bf16 (nearest even), 8 contiguous bytes per lane per sub-tile ----
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
static hipError_t launch_bs_tile(const BsArgs& a)
{
    using T = BsTile<BM, BN, WM, WN>;
    auto kern = bs_gemm_kernel<BM, BN, WM, WN>;
    static bool attr_done = false;  // benign race: the attribute call is idempotent
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
                       (const uint8_t*)a.A, a.a_scale, (const uint8_t*)a.B, a.b_scale,
                       (uint16_t*)a.C, a.M, a.N, a.K, tiles_n);
    return hipGetLastError();
}

hipError_t launch_bs(const BsArgs& a)
{
    return launch_bs_tile<128, 128, 2, 2>(a);
}

}  // namespace fp8bs
