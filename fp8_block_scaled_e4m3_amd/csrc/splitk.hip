// splitk.hip -- the second pass of the split-K GEMM: C = bf16(sum over the K ranges of their fp32
// sums), the ranges added in order (0, then 1, ...) so the result is the same run to run.
//
// Split K is for shapes whose output tiles are too few to occupy the CUs while K is deep (page
// "Flydsl Fp8 Blockscale Gemm", Bottleneck diagnosis: a grid of too few workgroups is bound by
// each tile's K loop): the tile GEMM runs splits x tiles work units, each over K/splits, and
// writes fp32 partial tiles; this pass reads splits x 4 bytes and writes 2 bytes per element,
// bound by memory bandwidth.
#include "device.hpp"
#include "launch.hpp"

#include <mutex>

namespace fp8bs {

// Scratch for the split-K partial tiles of fp8bs_gemm_splitk_noalloc, for callers that cannot
// allocate: one copy per GPU, held until the process ends. Host code never uses this name as an
// address (on the host it is a stand-in, not device memory): splitk_scratch() looks up the
// device address once per device and every launch takes that pointer.
static __device__ __align__(256) uint8_t scratch[kSplitkScratchBytes];

void* splitk_scratch()
{
    static std::once_flag once[kMaxDevices];
    static void* ptr[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::call_once(once[dev], [dev] {  // with device `dev` current
        void* p = nullptr;
        ptr[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess ? p : nullptr;
    });
    return ptr[dev];
}

namespace {

constexpr int kReduceThreads = 256;

// one thread: 8 consecutive columns of one row (two 16-byte reads per range, one 16-byte store)
__global__ void __launch_bounds__(kReduceThreads)
splitk_reduce_kernel(const float* __restrict__ partial, int splits, uint16_t* __restrict__ C, int M, int N)
{
    const size_t groups_per_row = (size_t)(N >> 3);
    const size_t g = (size_t)blockIdx.x * kReduceThreads + threadIdx.x;
    if (g >= (size_t)M * groups_per_row)
        return;
    const size_t m = g / groups_per_row;
    const size_t off = m * (size_t)N + (g - m * groups_per_row) * 8;
    const size_t plane = (size_t)M * (size_t)N;
    v4f lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < splits; ++s) {
        const float* p = partial + (size_t)s * plane + off;
        const v4f a = *(const v4f*)p;
        const v4f b = *(const v4f*)(p + 4);
        lo.x += a.x;
        lo.y += a.y;
        lo.z += a.z;
        lo.w += a.w;
        hi.x += b.x;
        hi.y += b.y;
        hi.z += b.z;
        hi.w += b.w;
    }
    v4i packed;
    packed.x = (int)pack_bf16x2(lo.x, lo.y);
    packed.y = (int)pack_bf16x2(lo.z, lo.w);
    packed.z = (int)pack_bf16x2(hi.x, hi.y);
    packed.w = (int)pack_bf16x2(hi.z, hi.w);
    *(v4i*)(C + off) = packed;
}

}  // namespace

hipError_t launch_splitk_reduce(const float* partial, int splits, void* C, int M, int N, hipStream_t stream)
{
    if (M <= 0 || N % 8 != 0 || splits < 1)
        return hipErrorInvalidValue;
    const size_t groups = (size_t)M * (size_t)(N >> 3);
    const unsigned blocks = (unsigned)((groups + kReduceThreads - 1) / kReduceThreads);
    return launch_kernel(splitk_reduce_kernel, dim3(blocks), dim3(kReduceThreads), stream, partial, splits,
                         (uint16_t*)C, M, N);
}

}  // namespace fp8bs
