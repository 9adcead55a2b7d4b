// probe.hip -- diagnostic: matrix-core throughput on the caller's own fp8 operand bytes.
//
// The gfx950 matrix core slows down when the operand bits change from one instruction to the
// next (measured: ~97% of the nominal rate on constant operands, ~45% on random or quantised
// operand bytes). This kernel measures that data-dependent ceiling directly: every wave loads
// four activation and four weight fragments from A and the prepared B (the same per-lane
// layout the GEMM uses), then runs back-to-back v_mfma_f32_16x16x128_f8f6f4 on them with no
// memory traffic, in the GEMM's issue order (one operand changes per instruction). It is the
// "identical MFMA work, nothing else" instrument of page "Flydsl Fp8 Blockscale Gemm",
// Bottleneck diagnosis (points 2 and 4).
#include "device.hpp"
#include "launch.hpp"

namespace fp8bs {

constexpr int kProbeThreads = 512;  // 8 waves, 2 per SIMD, like the GEMM's large tiles

__global__ void __launch_bounds__(kProbeThreads)
mfma_ceiling_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, int M, int N, int K,
                    int iters, float* __restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
    const int KB = K >> 7;
    const int q = lane >> 4;
    auto frag = [&](const uint8_t* base, int rows, int row, int kb) -> v8i {
        const uint8_t* p = base + (size_t)(row % rows) * K + (size_t)kb * 128;
        const v4i lo = *(const v4i*)(p + 16 * q);
        const v4i hi = *(const v4i*)(p + 64 + 16 * q);
        return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    };
    v8i a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = frag(A, M, wave * 64 + 16 * i + (lane & 15), (wave + i) % KB);
        b[i] = frag(B, N, wave * 64 + 16 * i + (lane & 15), (wave + i) % KB);
    }
    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i][j] = mfma_f8(b[j], a[i], acc[i][j]);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            s += acc[i][j].x + acc[i][j].y + acc[i][j].z + acc[i][j].w;
    if (lane == 0)
        sink[wave] = s;
}

hipError_t launch_mfma_ceiling(const void* A, const void* B_prep, int M, int N, int K, int iters, float* sink,
                               int sink_len, long long* flops, hipStream_t stream)
{
    const int waves_per_wg = kProbeThreads / 64;
    int wgs = device_cus();
    if (wgs * waves_per_wg > sink_len)
        wgs = sink_len / waves_per_wg;
    if (wgs < 1)
        return hipErrorInvalidValue;
    if (flops)
        *flops = (long long)wgs * waves_per_wg * iters * 16 * (2LL * 16 * 16 * 128);
    return launch_kernel(mfma_ceiling_kernel, dim3(wgs), dim3(kProbeThreads), stream, (const uint8_t*)A,
                         (const uint8_t*)B_prep, M, N, K, iters, sink);
}

}  // namespace fp8bs
