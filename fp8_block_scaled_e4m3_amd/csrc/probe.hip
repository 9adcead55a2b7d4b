// probe.hip -- diagnostics: matrix-core throughput on the caller's own fp8 operand bytes, and
// a skeleton of the GEMM mainloop that adds its ingredients one at a time.
//
// The gfx950 matrix core slows down when the operand bits change from one instruction to the
// next (measured: ~97% of the nominal rate on constant operands, ~75% in this kernel on the
// narrow-N workload's quantised bytes). This kernel measures that data-dependent ceiling
// directly: every wave loads
// four activation and four weight fragments from A and the prepared B (the same per-lane
// layout the GEMM uses), then runs back-to-back v_mfma_f32_16x16x128_f8f6f4 on them with no
// memory traffic, in the GEMM's issue order (one operand changes per instruction). It is the
// "identical MFMA work, nothing else" instrument of page "Flydsl Fp8 Blockscale Gemm",
// Bottleneck diagnosis (points 2 and 4).
#include "device.hpp"
#include "launch.hpp"

#include <algorithm>

namespace fp8bs {

constexpr int kProbeThreads = 512;  // 8 waves, 2 per SIMD, like the GEMM's large tiles

// the promote of the loop skeleton: the GEMM's (one fused multiply-add per component)
__device__ __forceinline__ void promote_probe(v4f& acc, const v4f& p, float s)
{
    acc.x = __builtin_fmaf(p.x, s, acc.x);
    acc.y = __builtin_fmaf(p.y, s, acc.y);
    acc.z = __builtin_fmaf(p.z, s, acc.z);
    acc.w = __builtin_fmaf(p.w, s, acc.w);
}

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

// ---- loop skeleton ------------------------------------------------------------------------
// The GEMM mainloop with its parts switched on one at a time, on the caller's own operand bytes,
// to see what each costs the matrix core (page "Flydsl Fp8 Blockscale Gemm", Bottleneck
// diagnosis: phase decomposition with identical matrix work). One workgroup per CU, eight
// computing waves (two per SIMD); each step every wave runs the (TM/16) x 4 matrix instructions
// of a TM x 64 x 128 block. Parts (bit mask):
//   kLpReads    each step reads all of the wave's operand fragments from LDS (two 16-byte reads
//               per fragment, the GEMM's swizzle), each as soon as its register falls free;
//               without it the operands stay in registers;
//   kLpLoads    48 KB (TM = 64) or 64 KB (TM = 128) per step go global -> LDS with buffer_load
//               ... lds into a separate LDS region, issued by four extra loader waves (TM = 64)
//               or by the computing waves, one per few matrix instructions (TM = 128), plus one
//               workgroup barrier per step after the loads of the previous step have landed;
//   kLpPromote  route BS's promote: a fresh partial per instruction and 4 fused multiply-adds two
//               instructions later;
//   kLpStores   every 6 steps (one K-light tile) each computing wave stores its TM x 64 block as
//               bf16-sized data, one 16-byte store per lane and sub-tile pair, at the step end;
//   kLpBig      TM = 128 instead of 64.
// The results are not a GEMM: the LDS-DMA region is never read and the stored values are
// whatever the accumulators hold. Only the launch time matters.
enum { kLpReads = 1, kLpLoads = 2, kLpPromote = 4, kLpStores = 8, kLpBig = 16 };
constexpr int kLpStepsPerTile = 6;

template <int PARTS>
__global__ void __launch_bounds__(((PARTS & kLpLoads) && !(PARTS & kLpBig) ? 12 : 8) * 64)
loop_probe_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, int window, int steps,
                  uint8_t* __restrict__ out, int out_slots, float* __restrict__ sink)
{
    constexpr bool kReads = PARTS & kLpReads, kLoads = PARTS & kLpLoads, kPromote = PARTS & kLpPromote;
    constexpr bool kStores = PARTS & kLpStores, kBig = PARTS & kLpBig;
    constexpr int TM = kBig ? 128 : 64, SI = TM / 16, SJ = 4;
    constexpr bool kLoaderWaves = kLoads && !kBig;
    constexpr int kWaves = kLoaderWaves ? 12 : 8;
    constexpr int kStepBytes = kBig ? 64 * 1024 : 48 * 1024;  // global -> LDS bytes per step
    __shared__ __attribute__((aligned(1024))) uint8_t frag_lds[64 * 1024];
    __shared__ __attribute__((aligned(1024))) uint8_t dma_lds[64 * 1024];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // fragment region: 32 KB of A's bytes, then 32 KB of the prepared weights
    for (int i = tid; i < 64 * 1024 / 16; i += kWaves * 64) {
        const uint8_t* src = i < 2048 ? A + (size_t)i * 16 : B + (size_t)(i - 2048) * 16;
        *(v4i*)(frag_lds + (size_t)i * 16) = *(const v4i*)src;
    }
    __syncthreads();
    const uint64_t abase = (uint64_t)A;
    const v4i rs = v4i{(int)(uint32_t)abase, (int)((uint32_t)(abase >> 32) & 0xffffu), 0x7FFFFFFF, 0x00020000};
    const uint32_t dma_base = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)dma_lds);
    // step s reads A's bytes [off(s), off(s) + kStepBytes): a window of 16 steps per workgroup
    auto src_off = [&](int s) {
        return __builtin_amdgcn_readfirstlane((int)(((uint32_t)blockIdx.x * 16u + (uint32_t)(s & 15)) * kStepBytes %
                                                    (uint32_t)window));
    };
    auto dma = [&](uint32_t lds_off, int voff, int soff) {
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     :
                     : "s"(dma_base + lds_off), "v"(voff), "s"(rs), "s"(soff)
                     : "memory", "m0");
    };
    if (kLoaderWaves && wave >= 8) {
        // loader wave lw: 12 loads of 1 KB per step, then wait for its previous step's loads
        const int lw = wave - 8;
        for (int s = 0; s < steps; ++s) {
            const int soff = src_off(s);
#pragma unroll
            for (int g = 0; g < 12; ++g)
                dma((uint32_t)((lw * 12 + g) * 1024), (lw * 12 + g) * 1024 + lane * 16, soff);
            __builtin_amdgcn_s_waitcnt((12 & 15) | ((12 >> 4) << 14) | (7 << 4));  // vmcnt <= 12
            __builtin_amdgcn_s_barrier();
        }
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }
    const uint32_t frow = lane & 15, q = lane >> 4;
    const uint32_t c_lo = ((q ^ ((frow >> 1) & 7)) << 4) + frow * 128u;
    const uint32_t c_hi = (((q + 4) ^ ((frow >> 1) & 7)) << 4) + frow * 128u;
    auto frag = [&](uint32_t off) -> v8i {
        const v4i lo = *(const v4i*)(frag_lds + ((off + c_lo) & 0xffffu));
        const v4i hi = *(const v4i*)(frag_lds + ((off + c_hi) & 0xffffu));
        return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    };
    v8i a[SI], b[SJ];
#pragma unroll
    for (int i = 0; i < SI; ++i)
        a[i] = frag((uint32_t)((wave & 3) * 8192 + i * 2048));
#pragma unroll
    for (int j = 0; j < SJ; ++j)
        b[j] = frag((uint32_t)(32768 + wave * 2048 + j * 2048));
    v4f acc[SI][SJ];
#pragma unroll
    for (int i = 0; i < SI; ++i)
#pragma unroll
        for (int j = 0; j < SJ; ++j)
            acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    v4f p[3] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
    const float sc = 1.0f + (float)lane * 1e-3f;
    constexpr int kMathLoads = kStepBytes / 1024 / 8;          // TM = 128: loads per wave per step
    constexpr int kSpacing = (SI * SJ) / (kMathLoads ? kMathLoads : 1);
    constexpr int kEarlyLoads = (SJ + kSpacing - 1) / kSpacing;  // of them issued before the barrier
    for (int s = 0; s < steps; ++s) {
        const uint32_t sh = (uint32_t)(s & 7) * 4096u;
        const int soff = src_off(s);
#pragma unroll
        for (int i = 0; i < SI; ++i) {
#pragma unroll
            for (int j = 0; j < SJ; ++j) {
                const int t = i * SJ + j;
                if constexpr (kPromote) {
                    p[t % 3] = mfma_f8(b[j], a[i], v4f{0.f, 0.f, 0.f, 0.f});
                    if (t >= 2)
                        promote_probe(acc[(t - 2) / SJ][(t - 2) % SJ], p[(t - 2) % 3], sc);
                } else {
                    acc[i][j] = mfma_f8(b[j], a[i], acc[i][j]);
                }
                if constexpr (kLoads && kBig) {
                    if (t % kSpacing == 0 && t / kSpacing < kMathLoads)
                        dma((uint32_t)((wave * kMathLoads + t / kSpacing) * 1024),
                            (wave * kMathLoads + t / kSpacing) * 1024 + lane * 16, soff);
                }
                if (kReads && i == SI - 1)
                    b[j] = frag(32768u + sh + (uint32_t)j * 2048u);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (kReads)
                a[i] = frag(sh + (uint32_t)i * 2048u);
            else
                asm volatile("" : "+v"(a[i]));
            if (kLoads && i == 0) {
                if constexpr (kBig)  // the previous step's loads (and any stores before them) are done
                    __builtin_amdgcn_s_waitcnt((kEarlyLoads & 15) | ((kEarlyLoads >> 4) << 14) | (7 << 4));
                __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));  // lgkmcnt(0)
                __builtin_amdgcn_s_barrier();
            }
        }
        if constexpr (!kReads) {
#pragma unroll
            for (int j = 0; j < SJ; ++j)
                asm volatile("" : "+v"(b[j]));
        }
        if constexpr (kPromote) {
            constexpr int n = SI * SJ;
            promote_probe(acc[(n - 2) / SJ][(n - 2) % SJ], p[(n - 2) % 3], sc);
            promote_probe(acc[(n - 1) / SJ][(n - 1) % SJ], p[(n - 1) % 3], sc);
        }
        if constexpr (kStores) {
            if (s % kLpStepsPerTile == kLpStepsPerTile - 1) {
                constexpr int kPerWave = SI * (SJ / 2) * 1024;  // bytes per wave and tile
                const int slot = (s / kLpStepsPerTile) % out_slots;
                uint8_t* base = out + ((size_t)slot * gridDim.x + blockIdx.x) * (8 * kPerWave) + (size_t)wave * kPerWave;
#pragma unroll
                for (int si = 0; si < SI; ++si)
#pragma unroll
                    for (int sj = 0; sj < SJ; sj += 2) {
                        v4i v;
                        v.x = (int)pack_bf16x2(acc[si][sj].x, acc[si][sj].y);
                        v.y = (int)pack_bf16x2(acc[si][sj].z, acc[si][sj].w);
                        v.z = (int)pack_bf16x2(acc[si][sj + 1].x, acc[si][sj + 1].y);
                        v.w = (int)pack_bf16x2(acc[si][sj + 1].z, acc[si][sj + 1].w);
                        *(v4i*)(base + ((si * (SJ / 2) + sj / 2) * 64 + lane) * 16) = v;
                    }
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < SI; ++i)
#pragma unroll
        for (int j = 0; j < SJ; ++j)
            t += acc[i][j].x + acc[i][j].y + acc[i][j].z + acc[i][j].w;
    if (lane == 0)
        sink[blockIdx.x * 8 + wave] = t;
}

bool loop_probe_parts_ok(int parts)
{
    switch (parts) {
    case 0: case 1: case 3: case 7: case 15: case 5:
    case 16 | 1: case 16 | 3: case 16 | 7: case 16 | 15:
        return true;
    default:
        return false;
    }
}

size_t loop_probe_out_bytes(int parts)
{
    if (!(parts & kLpStores))
        return 0;
    return (size_t)device_cus() * 8 * ((parts & kLpBig) ? 16 : 8) * 1024;  // one slot of tiles
}

template <int PARTS>
static hipError_t launch_lp(const void* A, const void* B, int window, int steps, void* out, int slots, float* sink,
                            hipStream_t stream)
{
    constexpr int threads = ((PARTS & kLpLoads) && !(PARTS & kLpBig) ? 12 : 8) * 64;
    return launch_kernel(loop_probe_kernel<PARTS>, dim3(device_cus()), dim3(threads), stream, (const uint8_t*)A,
                         (const uint8_t*)B, window, steps, (uint8_t*)out, slots, sink);
}

hipError_t launch_loop_probe(int parts, const void* A, const void* B_prep, size_t a_bytes, int steps, void* out,
                             size_t out_bytes, float* sink, int sink_len, long long* flops, hipStream_t stream)
{
    const int wgs = device_cus();
    if (!loop_probe_parts_ok(parts) || sink_len < wgs * 8 || steps < 1)
        return hipErrorInvalidValue;
    const size_t step_bytes = (parts & kLpBig) ? 64 * 1024 : 48 * 1024;
    // the DMA window: whole steps of A's bytes, at most 1 GiB
    const size_t window = std::min<size_t>(a_bytes / step_bytes * step_bytes, (size_t)1 << 30);
    if (window < step_bytes)
        return hipErrorInvalidValue;
    const size_t slot_bytes = loop_probe_out_bytes(parts);
    const int slots = slot_bytes ? (int)std::min<size_t>(out_bytes / slot_bytes, 64) : 1;
    if (slot_bytes && slots < 1)
        return hipErrorInvalidValue;
    if (flops)
        *flops = (long long)wgs * 8 * steps * ((parts & kLpBig) ? 32 : 16) * (2LL * 16 * 16 * 128);
    switch (parts) {
    case 0: return launch_lp<0>(A, B_prep, (int)window, steps, out, slots, sink, stream);
    case 1: return launch_lp<1>(A, B_prep, (int)window, steps, out, slots, sink, stream);
    case 3: return launch_lp<3>(A, B_prep, (int)window, steps, out, slots, sink, stream);
    case 5: return launch_lp<5>(A, B_prep, (int)window, steps, out, slots, sink, stream);
    case 7: return launch_lp<7>(A, B_prep, (int)window, steps, out, slots, sink, stream);
    case 15: return launch_lp<15>(A, B_prep, (int)window, steps, out, slots, sink, stream);
    case 17: return launch_lp<17>(A, B_prep, (int)window, steps, out, slots, sink, stream);
    case 19: return launch_lp<19>(A, B_prep, (int)window, steps, out, slots, sink, stream);
    case 23: return launch_lp<23>(A, B_prep, (int)window, steps, out, slots, sink, stream);
    case 31: return launch_lp<31>(A, B_prep, (int)window, steps, out, slots, sink, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace fp8bs
