// api.hip -- the C ABI of libfp8bs (declared in include/fp8bs.h): argument validation on the
// host, then an asynchronous launch on the caller's stream. Nothing here allocates memory or
// synchronises the host.
#include "fp8bs.h"
#include "launch.hpp"

#include <stdint.h>

namespace {

constexpr int kVersion = 10000;  // 1.0.0

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? FP8BS_OK : FP8BS_E_HIP; }

// Shape rules of route BS: K in whole 128-wide blocks, N in whole 128-row weight blocks.
int check_bs_shape(int M, int N, int K)
{
    if (M < 0 || N < 128 || K < 128 || N % 128 != 0 || K % 128 != 0)
        return FP8BS_E_SHAPE;
    return FP8BS_OK;
}

// Shape rules of route MX (page "aiter PR #6370", Constraints): M and N in whole 64-row packed
// scale groups, K in whole 128-wide steps and at least two of them.
int check_mx_shape(int M, int N, int K)
{
    if (M < 0 || M % 64 != 0 || N < 64 || N % 64 != 0 || K < 256 || K % 128 != 0)
        return FP8BS_E_SHAPE;
    return FP8BS_OK;
}

}  // namespace

extern "C" {

int fp8bs_version(void) { return kVersion; }

const char* fp8bs_strerror(int status)
{
    switch (status) {
    case FP8BS_OK: return "ok";
    case FP8BS_E_NULL: return "a required pointer is NULL";
    case FP8BS_E_SHAPE: return "M, N or K violates the route's shape constraints";
    case FP8BS_E_ALIGN: return "a pointer is not suitably aligned (16 bytes for tensors, 4 for fp32 scales)";
    case FP8BS_E_CONFIG: return "invalid kernel configuration for this shape";
    case FP8BS_E_HIP: return "the HIP runtime reported an error while enqueueing work";
    default: return "unknown status";
    }
}

size_t fp8bs_prep_weight_bytes(int N, int K)
{
    if (N <= 0 || K <= 0)
        return 0;
    return (size_t)N * (size_t)K;
}

int fp8bs_prep_weights(const void* B, void* B_prep, int N, int K, hipStream_t stream)
{
    if (!B || !B_prep)
        return FP8BS_E_NULL;
    if (N < 64 || N % 64 != 0 || K < 128 || K % 128 != 0)
        return FP8BS_E_SHAPE;
    if (!aligned(B, 16) || !aligned(B_prep, 16))
        return FP8BS_E_ALIGN;
    return hip_status(fp8bs::launch_prep_weights(B, B_prep, N, K, stream));
}

int fp8bs_gemm(const void* A, const float* a_scale, const void* B_prep, const float* b_scale,
               void* C, int M, int N, int K, hipStream_t stream)
{
    int st = check_bs_shape(M, N, K);
    if (st != FP8BS_OK)
        return st;
    if (M == 0)
        return FP8BS_OK;
    if (!A || !a_scale || !B_prep || !b_scale || !C)
        return FP8BS_E_NULL;
    if (!aligned(A, 16) || !aligned(B_prep, 16) || !aligned(C, 16) || !aligned(a_scale, 4) ||
        !aligned(b_scale, 4))
        return FP8BS_E_ALIGN;
    fp8bs::BsArgs args{A, a_scale, B_prep, b_scale, C, M, N, K, stream};
    return hip_status(fp8bs::launch_bs(args));
}

size_t fp8mx_packed_scale_bytes(int rows, int K)
{
    if (rows <= 0 || K <= 0)
        return 0;
    return (size_t)rows * (size_t)(K / 32);
}

int fp8mx_pack_a_scale(const void* a_e8m0, void* a_scale_packed, int M, int K, hipStream_t stream)
{
    if (M < 0 || M % 64 != 0 || K < 256 || K % 128 != 0)
        return FP8BS_E_SHAPE;
    if (M == 0)
        return FP8BS_OK;
    if (!a_e8m0 || !a_scale_packed)
        return FP8BS_E_NULL;
    if (!aligned(a_scale_packed, 16))
        return FP8BS_E_ALIGN;
    return hip_status(fp8bs::launch_pack_scales(a_e8m0, a_scale_packed, M, K, stream));
}

int fp8mx_prep_weights(const void* B, const void* b_e8m0, void* B_prep, void* b_scale_packed,
                       int N, int K, hipStream_t stream)
{
    if (N < 64 || N % 64 != 0 || K < 256 || K % 128 != 0)
        return FP8BS_E_SHAPE;
    if (!B || !b_e8m0 || !B_prep || !b_scale_packed)
        return FP8BS_E_NULL;
    if (!aligned(B, 16) || !aligned(B_prep, 16) || !aligned(b_scale_packed, 16))
        return FP8BS_E_ALIGN;
    hipError_t e = fp8bs::launch_prep_weights(B, B_prep, N, K, stream);
    if (e != hipSuccess)
        return FP8BS_E_HIP;
    return hip_status(fp8bs::launch_pack_scales(b_e8m0, b_scale_packed, N, K, stream));
}

int fp8mx_gemm(const void* A, const void* a_scale_packed, const void* B_prep,
               const void* b_scale_packed, void* C, int M, int N, int K, hipStream_t stream)
{
    int st = check_mx_shape(M, N, K);
    if (st != FP8BS_OK)
        return st;
    if (M == 0)
        return FP8BS_OK;
    if (!A || !a_scale_packed || !B_prep || !b_scale_packed || !C)
        return FP8BS_E_NULL;
    if (!aligned(A, 16) || !aligned(B_prep, 16) || !aligned(C, 16) ||
        !aligned(a_scale_packed, 16) || !aligned(b_scale_packed, 16))
        return FP8BS_E_ALIGN;
    fp8bs::MxArgs args{A, a_scale_packed, B_prep, b_scale_packed, C, M, N, K, stream};
    return hip_status(fp8bs::launch_mx(args));
}

}  // extern "C"
