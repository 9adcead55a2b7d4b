// launch.hpp -- host-side launchers of libfp8bs (internal; the public ABI is include/fp8bs.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

struct BsArgs {
    const void* A;
    const float* a_scale;  // [K/128, M]
    const void* B;         // prepared weights
    const float* b_scale;  // [N/128, K/128]
    void* C;
    int M, N, K;
    hipStream_t stream;
};

struct MxArgs {
    const void* A;
    const void* a_packed;
    const void* B;         // prepared weights
    const void* b_packed;
    void* C;
    int M, N, K;
    hipStream_t stream;
};

hipError_t launch_bs(const BsArgs& a);
hipError_t launch_mx(const MxArgs& a);
hipError_t launch_prep_weights(const void* B, void* B_prep, int N, int K, hipStream_t stream);
hipError_t launch_pack_scales(const void* e8m0, void* packed, int rows, int K, hipStream_t stream);

}  // namespace fp8bs
