// launch.hpp -- host-side launchers of libfp8bs (internal; the public ABI is include/fp8bs.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

namespace fp8bs {

// Per-device host caches hold this many devices.
constexpr int kMaxDevices = 64;

// Enqueue kernel<<<grid, block, 0, stream>>>(args...) and return the status of this launch
// alone (hipLaunchKernel's own return value): an error that earlier, unrelated work left
// pending in the runtime is neither reported as this launch's failure nor cleared.
template <typename... P, typename... A>
inline hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream, A... args)
{
    static_assert(sizeof...(P) == sizeof...(A), "one argument per kernel parameter");
    std::tuple<P...> values{static_cast<P>(args)...};
    void* ptrs[sizeof...(P) > 0 ? sizeof...(P) : 1];
    std::apply([&](auto&... v) {
        int i = 0;
        ((ptrs[i++] = (void*)&v), ...);
    }, values);
    return hipLaunchKernel((const void*)kernel, grid, block, ptrs, 0, stream);
}

enum { kRouteBS = 0, kRouteMX = 1, kRoutePT = 2 };
// Small-M kernel only: route MX with the packed activation scales of fp8mx_pack_a_scale (M % 64
// == 0) instead of the row-major a_e8m0 bytes.
constexpr int kRouteMXPacked = 3;

struct GemmArgs {
    const void* A;        // [M, K] e4m3
    const void* a_scale;  // BS: fp32 [K/128, M]; MX: packed ue8m0 dwords
    const void* B;        // prepared weights
    const void* b_scale;  // BS: fp32 [N/128, K/128]; MX: packed ue8m0 dwords
    void* C;              // [M, N] bf16
    int M, N, K;
    hipStream_t stream;
};

// One instantiated kernel shape: BM x BN output tile, WM x WN waves, STAGES LDS buffers.
struct VariantInfo {
    int block_m, block_n, waves_m, waves_n, stages, pingpong;
};

struct GemmConfig {
    int variant;     // index into the instantiated shapes (variant_info)
    int group_m;     // tile rows walked together by consecutive tiles
    int xcd_remap;   // give each XCD a contiguous range of the tile order
    int persistent;  // 1: one workgroup per CU slot looping over tiles; 0: one per tile
    int c_store;     // C store cache policy: 0 write-back, 1 write-through, 2 write-through non-temporal
};

const VariantInfo* variant_info(int v);
int device_cus();
bool variant_supports(int route, int v);
hipError_t launch_gemm(int route, const GemmArgs& a, const GemmConfig& c);
// Split K (route BS): the tile GEMM writes fp32 sums of each of `splits` equal K ranges to
// partial[splits][M][N] (K/128 % splits == 0; variants with split_supported()), then
// launch_splitk_reduce adds them in range order and rounds to bf16 C.
bool split_supported(int variant);
hipError_t launch_gemm_split(const GemmArgs& a, const GemmConfig& c, int splits, float* partial);
hipError_t launch_splitk_reduce(const float* partial, int splits, void* C, int M, int N, hipStream_t stream);
// The library's static split-K scratch on the current device (kSplitkScratchBytes, 256-byte
// aligned): its device address, looked up once per device; nullptr if the lookup failed.
constexpr size_t kSplitkScratchBytes = (size_t)32 << 20;
void* splitk_scratch();
hipError_t launch_mfma_ceiling(const void* A, const void* B_prep, int M, int N, int K, int iters, float* sink,
                               int sink_len, long long* flops, hipStream_t stream);
// Loop skeleton probe (probe.hip): `parts` a mask of the kLp* parts, one of the instantiated
// combinations; out: bytes for the stored tiles (parts with kLpStores), rotated over whole slots.
bool loop_probe_parts_ok(int parts);
size_t loop_probe_out_bytes(int parts);
hipError_t launch_loop_probe(int parts, const void* A, const void* B_prep, size_t a_bytes, int steps, void* out,
                             size_t out_bytes, float* sink, int sink_len, long long* flops, hipStream_t stream);
hipError_t launch_prep_weights(const void* B, void* B_prep, int N, int K, hipStream_t stream);
hipError_t launch_pack_scales(const void* e8m0, void* packed, int rows, int K, int permute, hipStream_t stream);
// Small-M kernel (decode.hip): M >= 1 in chunks of kDecodeMaxRows rows (at most kDecodeMaxChunks
// chunks: the grid's y extent), N % 64 == 0, K % 128 == 0. Route BS
// takes a_scale [K/128, M] fp32 as the main kernel does; route MX takes the activation
// exponents row-major, a_e8m0 [M, K/32] (kRouteMXPacked: packed as for the main kernel);
// route PT a_scale [M], b_scale [N]. Variant: kDecodeAuto (chosen by shape), kDecodeDirect
// (fragments loaded straight into registers), kDecodeLds (operands staged through LDS by
// direct-to-LDS loads) or kDecodeLdsPair (the same with two 16-row weight sub-tiles per
// workgroup; min(M, 64) <= 32 and N % 32 == 0); results agree bit for bit up to 48 rows.
constexpr int kDecodeMaxRows = 64;
constexpr int kDecodeMaxChunks = 65535;
constexpr int kDecodeAuto = 1, kDecodeDirect = 2, kDecodeLds = 3, kDecodeLdsPair = 4;
hipError_t launch_decode(int route, const GemmArgs& a, int variant);

// Activation quantiser of route kRouteBS (scales: fp32 [K/128, M]) or kRouteMX (scales: ue8m0
// bytes [M, K/32]); x is bf16 (in_bf16 = 1) or fp32 [M, K].
hipError_t launch_quantize(int route, const void* x, int in_bf16, void* codes, void* scales, int M, int K,
                           hipStream_t stream);

}  // namespace fp8bs
