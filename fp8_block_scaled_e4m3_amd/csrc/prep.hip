// prep.hip -- one-time weight and scale preparation (untimed set-up work; page "Flydsl Fp8
// Blockscale Gemm", Procedure steps 2 and 6, and page "aiter PR #6370", Integration).
#include "device.hpp"
#include "launch.hpp"

namespace fp8bs {

// Pack ue8m0 exponents e8m0[rows, K/32] (row-major) into the K-block-major, four-per-dword
// layout the scaled instruction reads: dword d = (kstep * rows/64 + group) * 64 + lane with
// lane = 16g + i holds, in byte t, the exponent of (prepared) row 64*group + 16t + i over K
// group 4*kstep + g. For weights (permute = 1) the prepared row order is that of the prepared
// weight buffer, so byte t of lane i scales weight row 64*group + weight_row_perm(16t + i).
__global__ void pack_scales_kernel(const uint8_t* __restrict__ e8m0, uint32_t* __restrict__ packed,
                                   int rows, int K, int permute)
{
    const int groups = rows >> 6;
    const int gk = K >> 5;
    const size_t total = (size_t)(K >> 7) * groups * 64;
    const size_t d = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (d >= total)
        return;
    const int lane = (int)(d & 63);
    const int group = (int)((d >> 6) % groups);
    const int kstep = (int)((d >> 6) / groups);
    const int g = lane >> 4, i = lane & 15;
    uint32_t word = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int local = 16 * t + i;
        const int row = group * 64 + (permute ? weight_row_perm(local) : local);
        word |= (uint32_t)e8m0[(size_t)row * gk + kstep * 4 + g] << (8 * t);
    }
    packed[d] = word;
}

hipError_t launch_pack_scales(const void* e8m0, void* packed, int rows, int K, int permute, hipStream_t stream)
{
    const size_t total = (size_t)(K >> 7) * (rows >> 6) * 64;
    if (total == 0)
        return hipSuccess;
    const int threads = 256;
    const unsigned blocks = (unsigned)((total + threads - 1) / threads);
    return launch_kernel(pack_scales_kernel, dim3(blocks), dim3(threads), stream, (const uint8_t*)e8m0,
                         (uint32_t*)packed, rows, K, permute);
}

// Prepared weights: B [N, K] with the rows of every 64-row window reordered by
// weight_row_perm, so that a wave multiplying the window's four 16-row sub-tiles (weights as
// the first matrix operand) receives, in each lane, eight consecutive output columns for each
// pair of sub-tiles -- one 16-byte, 64-byte-per-row-coalesced C store per pair. One thread
// copies one 16-byte chunk.
__global__ void prep_weights_kernel(const uint8_t* __restrict__ B, uint8_t* __restrict__ B_prep, int N, int K)
{
    const int chunks_per_row = K >> 4;
    const size_t total = (size_t)N * chunks_per_row;
    const size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= total)
        return;
    const int row = (int)(c / chunks_per_row);
    const int ch = (int)(c - (size_t)row * chunks_per_row);
    const int src = (row & ~63) + weight_row_perm(row & 63);
    *(v4i*)(B_prep + (size_t)row * K + ch * 16) = *(const v4i*)(B + (size_t)src * K + ch * 16);
}

hipError_t launch_prep_weights(const void* B, void* B_prep, int N, int K, hipStream_t stream)
{
    const size_t total = (size_t)N * (size_t)(K >> 4);
    if (total == 0)
        return hipSuccess;
    const int threads = 256;
    const unsigned blocks = (unsigned)((total + threads - 1) / threads);
    return launch_kernel(prep_weights_kernel, dim3(blocks), dim3(threads), stream, (const uint8_t*)B,
                         (uint8_t*)B_prep, N, K);
}

}  // namespace fp8bs
