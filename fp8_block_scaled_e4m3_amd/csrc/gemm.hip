// gemm.hip -- the two GEMM routes of libfp8bs on one gfx950 mainloop.
//
// Route BS (page "Flydsl Fp8 Blockscale Gemm", Mechanism A): fp32 block scales cannot be
// expressed by the matrix core's power-of-two scale operands, so each 128-wide K block of a
// 16x16 output tile is one UNSCALED v_mfma_f32_16x16x128_f8f6f4 into a fresh fp32 partial
// (four VGPRs), then "promoted": acc += partial * (a_s[m,kb] * b_s[n/128,kb]). The promote
// is 4 fp32 FMAs per instruction, issued two matrix instructions after the one it reads, so
// the vector ALU works while the matrix core runs and neither waits on the other.
//
// Route MX (page "aiter PR #6370", "Why it is faster"): the 1x32 ue8m0 scales ride in the
// scale operands of v_mfma_scale_f32_16x16x128_f8f6f4, accumulating straight into acc.
//
// Work decomposition (shared by both routes):
//  * Persistent workgroups: one per CU slot, each walking a list of BM x BN output tiles. The
//    (tile, 128-wide K block) pairs of a workgroup form one stream of steps; the operands of
//    step s + STAGES - 1 are requested while step s computes, across tile boundaries, so a new
//    tile starts on data that is already in LDS and a finished tile's C stores drain while
//    the next tile computes.
//  * Operands move global -> LDS with buffer_load_dwordx4 ... lds (no staging registers; the
//    K advance is a scalar offset) into a ring of STAGES LDS buffers. The block scales of the
//    step travel in the same buffer (buffer_load_dword ... lds), so every wave issues the same
//    number of loads per step and a single vmcnt wait covers them. The loads go out one per
//    matrix instruction: issued back to back they stall the issuing wave in the texture path
//    for several hundred cycles each step.
//  * Each wave computes a TM x TN sub-tile with the weights as the first matrix operand
//    (swap-AB), so every lane owns four consecutive columns of one output row and stores
//    8 contiguous bytes (page "aiter PR #6370", "Why it is faster", first bullet). Of the two
//    operands the one with fewer fragments per wave is held in registers for the whole step
//    and the other streams through a two-deep register ring; one barrier per step, after the
//    step's last matrix instruction, after which the wave reads the next step's first
//    fragments while its last instructions and promotes still run.
//  * Schedules (config field `pingpong`): 0, every wave loads and computes; 1, ping-pong (the
//    two halves of the workgroup alternate memory and matrix phases); 2, warp-specialised:
//    WM x WN math waves that only read LDS and run matrix instructions, plus four loader waves
//    (one per SIMD) that only issue the global -> LDS loads, so the load-issue stalls of the
//    texture path never hold up a wave that has matrix work to issue. With 64 x 64 per wave
//    the math waves of schedule 2 hold all eight fragments of a step in registers: the barrier
//    sits after the step's first row of instructions, and each fragment of the next step is
//    read as soon as its register falls free, a row or more ahead of its use. Every LDS address
//    is then a per-lane base plus an immediate offset, which leaves the vector ALU to the
//    promote (each vector instruction taken out of the loop shortened it measurably).
//  * Tiles are handed out so that the workgroups running at the same time on one XCD (each
//    XCD has its own L2) work on neighbouring tiles (page "Flydsl Fp8 Blockscale Gemm",
//    Mechanism B: XCD-aware rasterisation).
//
// LDS layout of one stage: [A: BM rows x 128 B][B: BN rows x 128 B][A scales][B scales]. The
// 16-byte chunks of a row r are XOR-swizzled with ((r >> 1) & 7): the sixteen lanes that read
// the same chunk of sixteen consecutive rows fall on sixteen distinct 16-byte bank groups.
#include "device.hpp"
#include "launch.hpp"

#include <mutex>
#include <type_traits>
#include <utility>

namespace fp8bs {

__device__ __forceinline__ uint32_t swz(uint32_t row) { return (row >> 1) & 7u; }

// The kernel's lambdas are always inlined: a lambda left as a call keeps its captures in
// scratch memory (the optimiser's inlining budget runs out on the larger tiles otherwise).
#define FP8BS_INLINE __attribute__((always_inline))

// The software promote acc + p * s, one fused multiply-add per component (one rounding), spelled
// out so that every schedule rounds the same way whatever the optimiser hoists or shares.
__device__ __forceinline__ void promote_fma(v4f& acc, const v4f& p, float s)
{
    acc.x = __builtin_fmaf(p.x, s, acc.x);
    acc.y = __builtin_fmaf(p.y, s, acc.y);
    acc.z = __builtin_fmaf(p.z, s, acc.z);
    acc.w = __builtin_fmaf(p.w, s, acc.w);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kLdsCapacity = 160 * 1024;

template <int ROUTE, int BM, int BN, int WM, int WN, int STAGES, int PP>
struct Tile {
    // PP == 2 (warp-specialised): WM x WN math waves plus four loader waves (one per SIMD:
    // waves w, w+4, w+8 share a SIMD)
    static constexpr int kMathWaves = WM * WN;
    static constexpr int kWaves = PP >= 2 ? kMathWaves + 4 : kMathWaves;
    static constexpr int kLoaders = PP >= 2 ? 4 : kWaves;  // waves that issue the loads
    static constexpr int kThreads = kWaves * 64;
    static constexpr int TM = BM / WM;
    static constexpr int TN = BN / WN;
    static constexpr int SI = TM / 16;
    static constexpr int SJ = TN / 16;
    static constexpr int kABytes = BM * 128;
    static constexpr int kBBytes = BN * 128;
    // per-step scales in LDS: BS fp32 per row of A and <= 64 weight-block scales; MX one packed
    // dword per row of each operand; PT none (its scales are applied once, in the epilogue)
    static constexpr int kSABytes = ROUTE == kRoutePT ? 0 : BM * 4;
    static constexpr int kSBBytes = ROUTE == kRoutePT ? 0 : ROUTE == kRouteBS ? 256 : BN * 4;
    static constexpr int kStageBytes = kABytes + kBBytes + kSABytes + kSBBytes;
    static constexpr int kLoadsA = BM / 8 / kLoaders;  // 1 KB (8-row) loads per loading wave per step
    static constexpr int kLoadsB = BN / 8 / kLoaders;
    static constexpr int kScaleLoadsA = ROUTE == kRoutePT ? 0 : BM / 64;  // 256-byte loads
    static constexpr int kScaleLoadsB = ROUTE == kRoutePT ? 0 : ROUTE == kRouteBS ? 1 : BN / 64;
    static constexpr int kScaleLoads = kScaleLoadsA + kScaleLoadsB;
    static constexpr int kLoadsS = (kScaleLoads + kLoaders - 1) / kLoaders;
    static constexpr int kLoadsPerStep = kLoadsA + kLoadsB + kLoadsS;
    static_assert(BM % (8 * kLoaders) == 0 && BN % (8 * kLoaders) == 0, "whole 8-row groups per wave");
    static_assert(BM % 64 == 0 && TM % 16 == 0 && TN % 64 == 0, "16x16 sub-tiles, 64-row scale loads, "
                  "whole 64-column windows of the prepared weight order per wave");
    static_assert(ROUTE == kRouteMX   ? (TM % 64 == 0 && TN % 64 == 0)
                  : ROUTE == kRouteBS ? (TN <= 128 && 128 % TN == 0)
                                      : true,
                  "MX: whole 64-row packed scale groups; BS: a wave's columns in one weight-scale block");
    static_assert(STAGES >= 2 && STAGES <= 4, "2 to 4 LDS stages");
    static_assert(STAGES * kStageBytes <= kLdsCapacity, "LDS capacity");
    static_assert(kLoadsPerStep * (STAGES - 1) <= 63, "vmcnt range");
    static_assert(PP != 1 || (STAGES == 2 && kWaves == 8), "ping-pong: two stages, two groups of four waves");
    static_assert(PP < 2 || kMathWaves == 4 || kMathWaves == 8, "warp-specialised: 4 or 8 math waves");
    static_assert(PP <= 2, "schedules 0 to 2");
};

// s_waitcnt for vmcnt <= N and lgkmcnt == 0 (expcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// s_waitcnt for lgkmcnt == 0 only.
__device__ __forceinline__ void wait_lgkm0()
{
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));
}

// Cache-policy bits of a vector memory store: sc1 alone is device scope (written through the
// XCD's L2, which other XCDs do not see), nt marks the line non-temporal (streamed, not kept).
constexpr int kCpolThrough = 16;             // sc1
constexpr int kCpolStreamThrough = 16 | 2;   // sc1 nt

// Buffer resource for a byte buffer starting at `base` (range check at 2^31 - 1 bytes).
__device__ __forceinline__ v4i buffer_desc(const void* base)
{
    const uint64_t a = (uint64_t)base;
    return v4i{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), 0x7FFFFFFF, 0x00020000};
}

// Global -> LDS copy of BYTES (16 or 4) per lane: lane l reads rs[voff + soff] and writes LDS
// byte address dst + BYTES * l. Issued through inline assembly, so the compiler tracks neither
// the LDS write nor the vmcnt it adds: every read of the stage it fills waits for it with an
// explicit vmcnt wait and barrier (the compiler's own tracking loses the stage at loop
// back-edges and would wait for loads that were just issued). dst and soff are uniform.
template <int BYTES>
__device__ __forceinline__ void lds_dma(const v4i& rs, uint32_t dst, int voff, int soff)
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

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1, unrolled at compile time.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Tile u of the persistent order -> output tile (tm, tn). Workgroup ids are dispatched
// round-robin over the 8 XCDs, so with a grid that is a multiple of 8, tile u runs on XCD u % 8,
// and tiles [r*grid, (r+1)*grid) run at the same time (round r). The base order t visits
// group_m tile rows at a time, row index fastest, so a window of consecutive t is a compact
// block of the output. The mapping u -> t is a permutation of [0, T):
//  * xcd_remap 0: t = u (the XCDs interleave tile by tile);
//  * xcd_remap 1: XCD x owns the contiguous range [x*T/8, (x+1)*T/8) of t (needs T % 8 == 0);
//  * xcd_remap 2: within each full round, XCD x owns the contiguous eighth
//    [r*grid + x*grid/8, r*grid + (x+1)*grid/8): every XCD works on its own compact block of
//    the same window of the output at the same time (a partial last round keeps t = u).
__device__ __forceinline__ void tile_of(int u, int grid, int tiles_m, int tiles_n, int group_m, int xcd_remap,
                                        int& tm, int& tn)
{
    const int T = tiles_m * tiles_n;
    int t = u;
    if (xcd_remap == 1 && (T & 7) == 0) {
        t = (u & 7) * (T >> 3) + (u >> 3);
    } else if (xcd_remap == 2 && (grid & 7) == 0) {
        const int r0 = u - u % grid;
        if (r0 + grid <= T) {
            const int l = u - r0;
            t = r0 + (l & 7) * (grid >> 3) + (l >> 3);
        }
    }
    const int per_group = group_m * tiles_n;
    const int g = t / per_group;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int r = t - g * per_group;
    tm = first_m + r % gm;
    tn = r / gm;
}

// SPLIT: split K. Each output tile's K blocks are cut into ksplit equal ranges, each computed by
// its own work unit (unit = split * tiles + tile), which writes its fp32 sums (route PT: before
// the row and column scales) to partial[split][M][N] instead of C; splitk_reduce_kernel adds the
// ranges in order and rounds to bf16.
template <int ROUTE, int BM, int BN, int WM, int WN, int STAGES, int PP, bool SPLIT = false>
__global__ void __launch_bounds__((WM * WN + (PP >= 2 ? 4 : 0)) * 64)
gemm_kernel(const uint8_t* __restrict__ A, const void* __restrict__ a_scale,
            const uint8_t* __restrict__ B, const void* __restrict__ b_scale,
            uint16_t* __restrict__ C, int M, int N, int K, int tiles_m, int tiles_n,
            int group_m, int xcd_remap, int ksplit, float* __restrict__ partial, int c_store)
{
    using T = Tile<ROUTE, BM, BN, WM, WN, STAGES, PP>;
    // One LDS array per stage: the stage of every read is known at compile time, so the
    // compiler can tell LDS-DMA writes to one stage from reads of another and adds no waits.
    __shared__ __attribute__((aligned(1024))) uint8_t st0[T::kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[T::kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t st2[STAGES > 2 ? T::kStageBytes : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t st3[STAGES > 3 ? T::kStageBytes : 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM;
    const int wn = wave / WM;
    const int lw = PP >= 2 ? wave - T::kMathWaves : wave;  // index among the loading waves
    const int T_total = tiles_m * tiles_n;
    const int n_split = SPLIT ? ksplit : 1;
    const int KB = (K >> 7) / n_split;  // K blocks per work unit
    const int U_total = T_total * n_split;
    const int grid = gridDim.x;
    // number of work units (tiles, or tile K ranges) this workgroup owns, and the length of its
    // step stream
    const int my_tiles = (int)blockIdx.x < U_total ? (U_total - 1 - (int)blockIdx.x) / grid + 1 : 0;
    const int total = my_tiles * KB;
    // unit i of this workgroup's list -> output tile (tm, tn) and its K range
    auto unit_of = [&](int i, int& tm, int& tn, int& split) FP8BS_INLINE {
        const int u = (int)blockIdx.x + i * grid;
        split = SPLIT ? u / T_total : 0;
        tile_of(SPLIT ? u - split * T_total : u, grid, tiles_m, tiles_n, group_m, xcd_remap, tm, tn);
    };

    const v4i rsA = buffer_desc(A);
    const v4i rsB = buffer_desc(B);
    const v4i rsSA = buffer_desc(a_scale);
    const v4i rsSB = buffer_desc(b_scale);

    // ---- per-tile load descriptors (recomputed when the stream enters a new tile) ---------
    // A wave's load g covers 8 rows (1 KB): lane l writes physical chunk l&7 of row l>>3, which
    // holds logical K chunk (l&7) ^ swz(row); rows past M re-read row M-1 (never stored).
    uint32_t voffA[T::kLoadsA];
    uint32_t voffB[T::kLoadsB];
    uint32_t voffS[T::kLoadsS > 0 ? T::kLoadsS : 1];  // scale loads: byte offset without the K-block term
    uint32_t kstrS[T::kLoadsS > 0 ? T::kLoadsS : 1];  // bytes per K block of that scale array
    int load_tile = -1;          // tile index (in this workgroup's list) the descriptors describe
    int load_kb0 = 0;            // its first K block
    auto setup_loads = [&](int i) FP8BS_INLINE {
        int tm, tn, split;
        unit_of(i, tm, tn, split);
        load_kb0 = split * KB;
        const int m0 = tm * BM, n0 = tn * BN;
#pragma unroll
        for (int g = 0; g < T::kLoadsA; ++g) {
            const int row = (lw * T::kLoadsA + g) * 8 + (lane >> 3);
            const int m = min(m0 + row, M - 1);
            voffA[g] = (uint32_t)m * (uint32_t)K + ((((uint32_t)lane & 7u) ^ swz(row)) << 4);
        }
#pragma unroll
        for (int g = 0; g < T::kLoadsB; ++g) {
            const int row = (lw * T::kLoadsB + g) * 8 + (lane >> 3);
            voffB[g] = (uint32_t)(n0 + row) * (uint32_t)K + ((((uint32_t)lane & 7u) ^ swz(row)) << 4);
        }
#pragma unroll
        for (int g = 0; g < T::kLoadsS; ++g) {
            const int u = min(lw * T::kLoadsS + g, T::kScaleLoads - 1);
            if (u < T::kScaleLoadsA) {
                if constexpr (ROUTE == kRouteBS) {  // a_scale[kb*M + m], fp32
                    voffS[g] = (uint32_t)min(m0 + 64 * u + lane, M - 1) * 4u;
                } else {  // packed dword ((kb*M/64 + group)*64 + lane)
                    voffS[g] = ((uint32_t)min((m0 >> 6) + u, (M >> 6) - 1) * 64u + (uint32_t)lane) * 4u;
                }
                kstrS[g] = (uint32_t)M * 4u;
            } else {
                if constexpr (ROUTE == kRouteBS) {  // b_scale[nb*(K/128) + kb], fp32
                    voffS[g] = (uint32_t)((n0 >> 7) + min(lane, (BN + 127) / 128 - 1)) * (uint32_t)(K >> 7) * 4u;
                    kstrS[g] = 4u;
                } else {
                    voffS[g] = ((uint32_t)((n0 >> 6) + (u - T::kScaleLoadsA)) * 64u + (uint32_t)lane) * 4u;
                    kstrS[g] = (uint32_t)N * 4u;
                }
            }
        }
        load_tile = i;
    };
    // Loads are issued in stream order, one group (kLoadsPerStep loads per wave) per step;
    // (ld_tile, ld_kb) is the next step to load. Past the end of the stream a group is still
    // issued, as an in-bounds re-read of the last loaded tile's first K block into a stage that
    // no later step reads, so that every step issues exactly one group and every vmcnt wait is
    // a compile-time constant.
    int ld_tile = 0, ld_kb = 0;
    int ld_kbv = 0;  // K block of the planned group
    auto plan_loads = [&](bool real) FP8BS_INLINE {
        int kb = 0;
        if (real) {
            if (ld_tile != load_tile)
                setup_loads(ld_tile);
            kb = ld_kb;
            if (++ld_kb == KB) {
                ld_kb = 0;
                ++ld_tile;
            }
        }
        ld_kbv = load_kb0 + kb;
    };
    // Load g of the planned group into stage st: A rows, then B rows, then block scales.
    auto lds_addr = [&](lds_u8* p) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)p); };
    auto issue_load = [&](auto G, lds_u8* st) FP8BS_INLINE {
        constexpr int g = decltype(G)::value;
        const int koff = __builtin_amdgcn_readfirstlane(ld_kbv * 128);
        if constexpr (g < T::kLoadsA) {
            lds_dma<16>(rsA, lds_addr(st + (lw * T::kLoadsA + g) * 1024), (int)voffA[g], koff);
        } else if constexpr (g < T::kLoadsA + T::kLoadsB) {
            constexpr int gb = g - T::kLoadsA;
            lds_dma<16>(rsB, lds_addr(st + T::kABytes + (lw * T::kLoadsB + gb) * 1024), (int)voffB[gb], koff);
        } else {
            constexpr int gs = g - T::kLoadsA - T::kLoadsB;
            lds_u8* sS = st + T::kABytes + T::kBBytes;
            const int u = min(lw * T::kLoadsS + gs, T::kScaleLoads - 1);  // uniform
            const int soff = __builtin_amdgcn_readfirstlane(ld_kbv * (int)kstrS[gs]);
            const bool is_a = u < T::kScaleLoadsA;
            const v4i rs = is_a ? rsSA : rsSB;
            lds_u8* dst = is_a ? sS + u * 256 : sS + T::kSABytes + (u - T::kScaleLoadsA) * 256;
            lds_dma<4>(rs, lds_addr(dst), (int)voffS[gs], soff);
        }
    };
    auto issue_group = [&](lds_u8* st) FP8BS_INLINE {
        static_for<T::kLoadsPerStep>([&](auto G) { issue_load(G, st); });
    };

    v4f acc[T::SI][T::SJ];
#pragma unroll
    for (int i = 0; i < T::SI; ++i)
#pragma unroll
        for (int j = 0; j < T::SJ; ++j)
            acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int frow = lane & 15;
    const uint32_t q = (uint32_t)lane >> 4;
    // this lane's LDS byte offsets of chunk q and chunk q+4 for a row with (row & 15) == frow
    const uint32_t c_lo = ((q ^ swz(frow)) << 4) + frow * 128u;
    const uint32_t c_hi = (((q + 4u) ^ swz(frow)) << 4) + frow * 128u;
    auto frag = [&](const uint8_t* base) -> v8i {
        const v4i lo = *(const v4i*)(base + c_lo);
        const v4i hi = *(const v4i*)(base + c_hi);
        return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    };

    // ---- epilogue: fp32 -> bf16 (nearest even) -------------------------------------------
    // The prepared weight rows are ordered so that sub-tiles j and j+1 (j even) hand lane
    // group q output columns 32*(j/2) + 8q .. +7 of the wave's 64-column window: one 16-byte
    // store per lane and pair, sixteen rows x 64 contiguous bytes per store instruction.
    auto store_tile = [&](int i) FP8BS_INLINE {
        int tm, tn, split;
        unit_of(i, tm, tn, split);
        const int mbase = tm * BM + wm * T::TM + frow;
        const int nbase = tn * BN + wn * T::TN + 8 * (int)q;
        if constexpr (SPLIT) {
            // this K range's fp32 sums, unscaled for route PT: lane group q holds columns
            // 32*(sj/2) + 8q .. +7 of the wave's window, registers of sub-tile sj then sj + 1
            float* P = partial + (size_t)split * M * N;
#pragma unroll
            for (int si = 0; si < T::SI; ++si) {
                const int m = mbase + 16 * si;
                if (m < M) {
                    float* prow = P + (size_t)m * N + nbase;
#pragma unroll
                    for (int sj = 0; sj < T::SJ; sj += 2) {
                        *(v4f*)(prow + 32 * (sj >> 1)) = acc[si][sj];
                        *(v4f*)(prow + 32 * (sj >> 1) + 4) = acc[si][sj + 1];
                    }
                }
#pragma unroll
                for (int sj = 0; sj < T::SJ; ++sj)
                    acc[si][sj] = v4f{0.f, 0.f, 0.f, 0.f};
            }
            return;
        }
        // Route PT: C = acc * (a_s[m] * b_s[n]), with the row and column scales read here, once
        // per tile, before any store of the tile, and waited for at once (the empty asm uses):
        // no store then sits between a scale load and its use.
        float rs[ROUTE == kRoutePT ? T::SI : 1];
        v4f cs[ROUTE == kRoutePT ? T::SJ : 1];
        if constexpr (ROUTE == kRoutePT) {
            const float* as = (const float*)a_scale;
            const float* bs = (const float*)b_scale;
#pragma unroll
            for (int si = 0; si < T::SI; ++si)
                rs[si] = as[min(mbase + 16 * si, M - 1)];
#pragma unroll
            for (int sj = 0; sj < T::SJ; ++sj)
                cs[sj] = *(const v4f*)(bs + nbase + 32 * (sj >> 1) + 4 * (sj & 1));
#pragma unroll
            for (int si = 0; si < T::SI; ++si)
                asm volatile("" : "+v"(rs[si]));
#pragma unroll
            for (int sj = 0; sj < T::SJ; ++sj)
                asm volatile("" : "+v"(cs[sj]));
        }
#pragma unroll
        for (int si = 0; si < T::SI; ++si) {
            const int m = mbase + 16 * si;
            // the 16 rows of this sub-tile row through one buffer resource based at its first
            // row: byte offsets stay below 16 rows * 2N bytes <= 2^29 (N * K < 2^31, K >= 128)
            const int mblk = tm * BM + wm * T::TM + 16 * si;
            const __amdgpu_buffer_rsrc_t crs =
                __builtin_amdgcn_make_buffer_rsrc(C + (size_t)mblk * N, 0, 0x7fffffff, 0x00020000);
            const int cbyte = (frow * N + nbase) * 2;
            if (m < M) {
#pragma unroll
                for (int sj = 0; sj < T::SJ; sj += 2) {
                    v4f lo = acc[si][sj];
                    v4f hi = acc[si][sj + 1];
                    if constexpr (ROUTE == kRoutePT) {
                        lo = lo * (cs[sj] * rs[si]);
                        hi = hi * (cs[sj + 1] * rs[si]);
                    }
                    v4i packed;
                    packed.x = (int)pack_bf16x2(lo.x, lo.y);
                    packed.y = (int)pack_bf16x2(lo.z, lo.w);
                    packed.z = (int)pack_bf16x2(hi.x, hi.y);
                    packed.w = (int)pack_bf16x2(hi.z, hi.w);
                    // the policy is an immediate of the instruction; c_store is uniform
                    const int off = cbyte + 64 * (sj >> 1);
                    if (c_store == 2)
                        __builtin_amdgcn_raw_buffer_store_b128(packed, crs, off, 0, kCpolStreamThrough);
                    else if (c_store == 1)
                        __builtin_amdgcn_raw_buffer_store_b128(packed, crs, off, 0, kCpolThrough);
                    else
                        __builtin_amdgcn_raw_buffer_store_b128(packed, crs, off, 0, 0);
                }
            }
#pragma unroll
            for (int sj = 0; sj < T::SJ; ++sj)
                acc[si][sj] = v4f{0.f, 0.f, 0.f, 0.f};
        }
    };

    if constexpr (PP == 1) {
    // ---- ping-pong schedule ------------------------------------------------------------------
    // Waves w and w+4 share a SIMD, so the two groups (waves 0-3 and 4-7) each hold one wave of
    // every SIMD. Each group alternates a memory phase (read all of the step's fragments and
    // scales from LDS into registers) with a matrix phase (the step's matrix instructions on
    // those registers), with a barrier after each phase; group 1 starts one barrier late, so on
    // every SIMD one wave runs matrix instructions while the other reads its next operands.
    // With phase 2t = group 0 reading step t and phase 2t+1 = group 0 computing step t while
    // group 1 reads it, stage t % 2 is read in phases 2t and 2t+1 and is free from phase 2t+2.
    // The loads of step t+1 go out from phase 2t: group 0's share at the start of its memory
    // phase for step t, group 1's share during its matrix phase for step t-1 (one load per
    // matrix instruction). Each wave waits for its own share before the barrier that opens
    // phase 2t+2, so every load of step t+1 has landed when group 0 starts reading it.
    constexpr int GA = (T::SI + 3) / 4;  // MX: packed scale dwords per wave (one per 64 rows)
    constexpr int GB = (T::SJ + 3) / 4;
    struct Frags {
        v8i a[T::SI];
        v8i b[T::SJ];
        float sa[ROUTE == kRouteBS ? T::SI : 1];  // BS: a_s of this lane's row in sub-tile row i
        float sb;                                  // BS: b_s of the wave's weight block
        int ia[GA];                                // MX: packed activation scale dwords
        int ib[GB];                                // MX: packed weight scale dwords
    };
    auto read_all = [&](const uint8_t* st, Frags& F) FP8BS_INLINE {
        const uint8_t* sA = st + (wm * T::TM) * 128;
        const uint8_t* sB = st + T::kABytes + (wn * T::TN) * 128;
        const uint8_t* sS = st + T::kABytes + T::kBBytes;
#pragma unroll
        for (int i = 0; i < T::SI; ++i)
            F.a[i] = frag(sA + i * 16 * 128);
#pragma unroll
        for (int j = 0; j < T::SJ; ++j)
            F.b[j] = frag(sB + j * 16 * 128);
        if constexpr (ROUTE == kRouteBS) {
            const float* sa = (const float*)sS + wm * T::TM + frow;
#pragma unroll
            for (int i = 0; i < T::SI; ++i)
                F.sa[i] = sa[16 * i];
            F.sb = ((const float*)(sS + T::kSABytes))[(wn * T::TN) >> 7];
        } else if constexpr (ROUTE == kRouteMX) {
#pragma unroll
            for (int g = 0; g < GA; ++g)
                F.ia[g] = ((const int*)sS)[(wm * T::TM / 64 + g) * 64 + lane];
#pragma unroll
            for (int g = 0; g < GB; ++g)
                F.ib[g] = ((const int*)(sS + T::kSABytes))[(wn * T::TN / 64 + g) * 64 + lane];
        }
    };
    // The step's matrix instructions, sub-tile row by row (route BS: each promote two
    // instructions behind its instruction); hook(t) runs after instruction t.
    v4f p[3];
    auto mma = [&](const Frags& F, auto&& hook) FP8BS_INLINE {
        float srow[T::SI];
        if constexpr (ROUTE == kRouteBS) {
#pragma unroll
            for (int i = 0; i < T::SI; ++i)
                srow[i] = F.sa[i] * F.sb;
        }
        auto promote = [&](auto Tc) {
            constexpr int t = decltype(Tc)::value;
            promote_fma(acc[t / T::SJ][t % T::SJ], p[t % 3], srow[t / T::SJ]);
        };
        static_for<T::SI>([&](auto I) {
            constexpr int i = decltype(I)::value;
            static_for<T::SJ>([&](auto J) {
                constexpr int j = decltype(J)::value;
                constexpr int t = i * T::SJ + j;
                if constexpr (ROUTE == kRouteBS) {
                    p[t % 3] = mfma_f8(F.b[j], F.a[i], v4f{0.f, 0.f, 0.f, 0.f});
                    if constexpr (t >= 2)
                        promote(std::integral_constant<int, t - 2>{});
                } else if constexpr (ROUTE == kRoutePT) {
                    acc[i][j] = mfma_f8(F.b[j], F.a[i], acc[i][j]);
                } else {
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        F.b[j], F.a[i], acc[i][j], kFmtE4M3, kFmtE4M3, j & 3, F.ib[j / 4], i & 3, F.ia[i / 4]);
                }
                hook(std::integral_constant<int, t>{});
                __builtin_amdgcn_sched_barrier(0);
            });
        });
        if constexpr (ROUTE == kRouteBS) {
            constexpr int n = T::SI * T::SJ;
            promote(std::integral_constant<int, n - 2>{});
            promote(std::integral_constant<int, n - 1>{});
        }
        // keep every instruction of the phase inside the phase (the optimiser would otherwise
        // sink them below the following branches)
#pragma unroll
        for (int i = 0; i < T::SI; ++i)
#pragma unroll
            for (int j = 0; j < T::SJ; ++j)
                asm volatile("" : "+v"(acc[i][j]));
    };
    int cp_tile = 0, cp_kb = 0;  // the step being computed
    auto finish_step = [&]() FP8BS_INLINE {
        if (++cp_kb == KB) {
            store_tile(cp_tile);
            cp_kb = 0;
            ++cp_tile;
        }
    };
    const int grp = wave >> 2;
    if (total > 0) {
        plan_loads(true);
        issue_group((lds_u8*)st0);  // step 0, every wave
        if (grp == 1) {
            plan_loads(1 < total);
            issue_group((lds_u8*)st1);  // group 1's share of step 1
        }
        // (group 1 waits for its share of step 1 too: with nothing in flight at the top of the
        // step loop, the compiler's own LDS waits there stay exact)
        wait_vmcnt_lgkm<0>();
        __builtin_amdgcn_s_barrier();
        Frags F;
        if (grp == 0) {
            auto step0 = [&](auto S, int t) {
                constexpr int k = decltype(S)::value;
                uint8_t* cur = k == 0 ? st0 : st1;
                uint8_t* oth = k == 0 ? st1 : st0;
                // memory phase: this group's share of step t+1's loads, then step t's operands
                plan_loads(t + 1 < total);
                issue_group((lds_u8*)oth);
                read_all(cur, F);
                wait_lgkm0();
                __builtin_amdgcn_s_barrier();
                // matrix phase
                mma(F, [&](auto) {});
                finish_step();
                wait_vmcnt_lgkm<0>();  // own loads of step t+1
                __builtin_amdgcn_s_barrier();
            };
            for (int t = 0; t < total; t += 2) {
                step0(std::integral_constant<int, 0>{}, t);
                if (t + 1 < total)
                    step0(std::integral_constant<int, 1>{}, t + 1);
            }
            __builtin_amdgcn_s_barrier();  // matches group 1's extra first barrier
        } else {
            __builtin_amdgcn_s_barrier();  // one phase behind group 0
            auto step1 = [&](auto S, int t) {
                constexpr int k = decltype(S)::value;
                uint8_t* cur = k == 0 ? st0 : st1;
                // memory phase: step t's operands; own loads of step t+1 must have landed
                read_all(cur, F);
                wait_vmcnt_lgkm<0>();
                __builtin_amdgcn_s_barrier();
                // matrix phase, issuing this group's share of step t+2 into the stage just read
                plan_loads(t + 2 < total);
                mma(F, [&](auto Tc) {
                    constexpr int tt = decltype(Tc)::value;
                    if constexpr (tt < T::kLoadsPerStep)
                        issue_load(std::integral_constant<int, tt>{}, (lds_u8*)cur);
                });
                if constexpr (T::kLoadsPerStep > T::SI * T::SJ) {
                    static_for<T::kLoadsPerStep - T::SI * T::SJ>([&](auto G) {
                        issue_load(std::integral_constant<int, T::SI * T::SJ + decltype(G)::value>{}, (lds_u8*)cur);
                    });
                }
                finish_step();
                __builtin_amdgcn_s_barrier();
            };
            for (int t = 0; t < total; t += 2) {
                step1(std::integral_constant<int, 0>{}, t);
                if (t + 1 < total)
                    step1(std::integral_constant<int, 1>{}, t + 1);
            }
        }
    }
    // the trailing load groups write LDS: let them land before the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(0);
    } else {
    // ---- registers of the step being computed ----------------------------------------------
    // The operand with fewer fragments per wave is held whole; the other is streamed through a
    // two-deep ring (fragment o+1 is read while the instructions of fragment o run).
    constexpr bool kStreamA = T::SI >= T::SJ;
    constexpr int NO = kStreamA ? T::SI : T::SJ;  // streamed fragments (outer loop)
    constexpr int NH = kStreamA ? T::SJ : T::SI;  // held fragments (inner loop)
    constexpr int GA = (T::SI + 3) / 4;           // MX: packed scale dwords per wave (one per 64 rows)
    constexpr int GB = (T::SJ + 3) / 4;
    v8i held[NH];
    v8i ring[2];
    float sa_r[ROUTE == kRouteBS ? T::SI : 1];  // BS: a_s of this lane's row in sub-tile row i
    float sb_r = 0.f;                            // BS: b_s of the wave's weight block
    int ia[GA];                                  // MX: packed activation scale dwords
    int ib[GB];                                  // MX: packed weight scale dwords
    // Schedule 2 holds every fragment of a step in registers where they fit beside the
    // accumulators (64 x 64 per wave: 8 fragments, 64 registers; the 168 registers of a SIMD
    // running three waves hold them), reading the next step's into each as it falls free.
    constexpr bool kFullHold = PP == 2 && (T::SI + T::SJ) * 8 + T::SI * T::SJ * 4 <= 128;
    v8i outer[kFullHold ? NO : 1];  // every fragment of the outer operand (the ring is unused)
    int ia_n[kFullHold ? GA : 1];   // MX: the next step's scales while the current ones are in use
    int ib_n[kFullHold ? GB : 1];

    auto a_base = [&](const uint8_t* st) { return st + (wm * T::TM) * 128; };
    auto b_base = [&](const uint8_t* st) { return st + T::kABytes + (wn * T::TN) * 128; };
    auto streamed = [&](const uint8_t* st) { return kStreamA ? a_base(st) : b_base(st); };
    auto held_base = [&](const uint8_t* st) { return kStreamA ? b_base(st) : a_base(st); };

    // The head of a step: what its first matrix instruction needs (held fragment 0 and streamed
    // fragment 0), the scales, then the rest of the held fragments.
    // The block scales of the step in stage st (route BS: into sa_r / sb_r; MX: into ia / ib, or
    // into ia_n / ib_n when `next`, while the current ones are still in use).
    auto read_scales = [&](const uint8_t* st, bool next) FP8BS_INLINE {
        const uint8_t* sS = st + T::kABytes + T::kBBytes;
        if constexpr (ROUTE == kRouteBS) {
            const float* sa = (const float*)sS + wm * T::TM + frow;
#pragma unroll
            for (int i = 0; i < T::SI; ++i)
                sa_r[i] = sa[16 * i];
            sb_r = ((const float*)(sS + T::kSABytes))[(wn * T::TN) >> 7];
        } else if constexpr (ROUTE == kRouteMX) {
            int* da = next ? ia_n : ia;
            int* db = next ? ib_n : ib;
#pragma unroll
            for (int g = 0; g < GA; ++g)
                da[g] = ((const int*)sS)[(wm * T::TM / 64 + g) * 64 + lane];
#pragma unroll
            for (int g = 0; g < GB; ++g)
                db[g] = ((const int*)(sS + T::kSABytes))[(wn * T::TN / 64 + g) * 64 + lane];
        }
    };
    auto read_head = [&](const uint8_t* st) FP8BS_INLINE {
        held[0] = frag(held_base(st));
        ring[0] = frag(streamed(st));
        read_scales(st, false);
#pragma unroll
        for (int h = 1; h < NH; ++h)
            held[h] = frag(held_base(st) + h * 16 * 128);
    };

    // ---- one step's matrix work ---------------------------------------------------------------
    // Route BS: matrix instruction t (in issue order) writes a fresh partial, and its promote
    // (acc += partial * a_s*b_s) is issued two instructions later, once the result is ready, so
    // the matrix core never waits on the vector ALU. Scheduling barriers keep that order.
    // `transition` runs after the last instruction is issued and before the last two promotes.
    // With three or more stages the loads of a step have a whole extra step to land, so they
    // are spread evenly over the step; with two they must land by the end of the step that
    // issues them, so they go out from its first instruction on.
    constexpr int kLoadSpacing =
        STAGES >= 3 && NO * NH >= 2 * T::kLoadsPerStep ? (NO * NH) / T::kLoadsPerStep : 1;
    v4f p[3];
    auto rows = [&](const uint8_t* st, lds_u8* load_st, auto&& transition) FP8BS_INLINE {
        const uint8_t* sO = streamed(st);
        float srow[T::SI];
        if constexpr (ROUTE == kRouteBS) {
#pragma unroll
            for (int i = 0; i < T::SI; ++i)
                srow[i] = sa_r[i] * sb_r;
        }
        auto promote = [&](auto Tc) {
            constexpr int t = decltype(Tc)::value;
            constexpr int o = t / NH, h = t % NH;
            constexpr int i = kStreamA ? o : h;
            constexpr int j = kStreamA ? h : o;
            promote_fma(acc[i][j], p[t % 3], srow[i]);
        };
        static_for<NO>([&](auto O) {
            constexpr int o = decltype(O)::value;
            if constexpr (o + 1 < NO)
                ring[(o + 1) & 1] = frag(sO + (o + 1) * 16 * 128);
            static_for<NH>([&](auto H) {
                constexpr int h = decltype(H)::value;
                constexpr int t = o * NH + h;
                constexpr int i = kStreamA ? o : h;
                constexpr int j = kStreamA ? h : o;
                const v8i& a = kStreamA ? ring[o & 1] : held[h];
                const v8i& b = kStreamA ? held[h] : ring[o & 1];
                if constexpr (ROUTE == kRouteBS) {
                    p[t % 3] = mfma_f8(b, a, v4f{0.f, 0.f, 0.f, 0.f});
                    if constexpr (t >= 2)
                        promote(std::integral_constant<int, t - 2>{});
                } else if constexpr (ROUTE == kRoutePT) {
                    // one unscaled accumulation over all of K; the scales come in the epilogue
                    acc[i][j] = mfma_f8(b, a, acc[i][j]);
                } else {
                    // weights first: the weight scale byte of sub-tile j, the activation byte of row i
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        b, a, acc[i][j], kFmtE4M3, kFmtE4M3, j & 3, ib[j / 4], i & 3, ia[i / 4]);
                }
                // the next load group goes out spread over the step (kLoadSpacing instructions
                // apart): a burst of loads fills the memory path's in-flight capacity and
                // stalls the issuing wave, matrix instructions and all
                if constexpr (PP == 0 && t % kLoadSpacing == 0 && t / kLoadSpacing < T::kLoadsPerStep)
                    issue_load(std::integral_constant<int, t / kLoadSpacing>{}, load_st);
                __builtin_amdgcn_sched_barrier(0);
            });
        });
        if constexpr (PP == 0 && T::kLoadsPerStep > NO * NH) {
            static_for<T::kLoadsPerStep - NO * NH>(
                [&](auto G) { issue_load(std::integral_constant<int, NO * NH + decltype(G)::value>{}, load_st); });
        }
        // Every matrix instruction of the step is issued before the transition: without these
        // (empty) uses the optimiser sinks them below its branches, into the next step.
#pragma unroll
        for (int i = 0; i < T::SI; ++i)
#pragma unroll
            for (int j = 0; j < T::SJ; ++j)
                asm volatile("" : "+v"(acc[i][j]));
        if constexpr (ROUTE == kRouteBS) {
            asm volatile("" : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]));
        }
        transition();
        if constexpr (ROUTE == kRouteBS) {
            constexpr int n = T::SI * T::SJ;
            if constexpr (n >= 2)
                promote(std::integral_constant<int, n - 2>{});
            promote(std::integral_constant<int, n - 1>{});
        }
    };

    // ---- schedule 2 with kFullHold: one step with all of its fragments in registers ----------
    // Every fragment of step s is in registers before its first instruction (read during step
    // s-1). After the first row of instructions the wave waits for its outstanding reads (the
    // last ones of step s) and meets the others at the barrier; after it, stage nxt (step s+1)
    // is complete for everyone and stage st is free for the loaders. The next step's fragments
    // are then read into the registers as they fall free: outer fragment o after row o, held
    // fragment h after the last row's instruction h, the last outer fragment after the row.
    auto read_full = [&](const uint8_t* st) FP8BS_INLINE {
        read_scales(st, false);
#pragma unroll
        for (int o = 0; o < (kFullHold ? NO : 0); ++o)
            outer[o] = frag(streamed(st) + o * 16 * 128);
#pragma unroll
        for (int h = 0; h < NH; ++h)
            held[h] = frag(held_base(st) + h * 16 * 128);
    };
    auto rows_full = [&](const uint8_t* nxt, auto&& transition) FP8BS_INLINE {
        float srow[T::SI];
        if constexpr (ROUTE == kRouteBS) {
#pragma unroll
            for (int i = 0; i < T::SI; ++i)
                srow[i] = sa_r[i] * sb_r;
        }
        auto promote = [&](auto Tc) {
            constexpr int t = decltype(Tc)::value;
            constexpr int o = t / NH, h = t % NH;
            constexpr int i = kStreamA ? o : h;
            constexpr int j = kStreamA ? h : o;
            promote_fma(acc[i][j], p[t % 3], srow[i]);
        };
        static_for<NO>([&](auto O) {
            constexpr int o = decltype(O)::value;
            static_for<NH>([&](auto H) {
                constexpr int h = decltype(H)::value;
                constexpr int t = o * NH + h;
                constexpr int i = kStreamA ? o : h;
                constexpr int j = kStreamA ? h : o;
                const v8i& a = kStreamA ? outer[o] : held[h];
                const v8i& b = kStreamA ? held[h] : outer[o];
                if constexpr (ROUTE == kRouteBS) {
                    p[t % 3] = mfma_f8(b, a, v4f{0.f, 0.f, 0.f, 0.f});
                    if constexpr (t >= 2)
                        promote(std::integral_constant<int, t - 2>{});
                } else if constexpr (ROUTE == kRoutePT) {
                    acc[i][j] = mfma_f8(b, a, acc[i][j]);
                } else {
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        b, a, acc[i][j], kFmtE4M3, kFmtE4M3, j & 3, ib[j / 4], i & 3, ia[i / 4]);
                }
                if constexpr (o == NO - 1)
                    held[h] = frag(held_base(nxt) + h * 16 * 128);
                __builtin_amdgcn_sched_barrier(0);
            });
            if constexpr (o == 0) {
                transition();
                __builtin_amdgcn_sched_barrier(0);
                read_scales(nxt, true);
            }
            if constexpr (o < NO - 1)
                outer[o] = frag(streamed(nxt) + o * 16 * 128);
            __builtin_amdgcn_sched_barrier(0);
        });
        outer[NO - 1] = frag(streamed(nxt) + (NO - 1) * 16 * 128);
#pragma unroll
        for (int i = 0; i < T::SI; ++i)
#pragma unroll
            for (int j = 0; j < T::SJ; ++j)
                asm volatile("" : "+v"(acc[i][j]));
        if constexpr (ROUTE == kRouteBS) {
            asm volatile("" : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]));
            constexpr int n = T::SI * T::SJ;
            promote(std::integral_constant<int, n - 2>{});
            promote(std::integral_constant<int, n - 1>{});
        } else if constexpr (ROUTE == kRouteMX) {
#pragma unroll
            for (int g = 0; g < GA; ++g)
                ia[g] = ia_n[g];
#pragma unroll
            for (int g = 0; g < GB; ++g)
                ib[g] = ib_n[g];
        }
    };

    // ---- the step stream ---------------------------------------------------------------------
    // Step s reads stage s % STAGES, and while its matrix instructions run it issues the loads
    // of step s + STAGES - 1 into stage (s - 1) % STAGES. Between the last matrix row of step s
    // and the first of step s+1 every wave (1) has finished its reads of stage s, (2) waits for
    // its own loads of step s+1 (vmcnt), then (3) meets the others at the barrier: after it,
    // step s+1's operands are in LDS for everyone and stage s is free for the loads that step
    // s+1 issues. Loads complete in order among themselves but not in order with the C stores
    // of an epilogue, so the first wait after an epilogue is for everything.
    int cp_tile = 0, cp_kb = 0;  // the step being computed
    int stores_pending = 0;
    auto wait_groups = [&]() {  // all but the STAGES-2 most recent load groups have landed
        if (stores_pending)
            wait_vmcnt_lgkm<0>();
        else
            wait_vmcnt_lgkm<(STAGES - 2) * T::kLoadsPerStep>();
        stores_pending = 0;
    };
    auto stage_ptr = [&](auto S) -> uint8_t* {
        constexpr int k = decltype(S)::value;
        return k == 0 ? st0 : k == 1 ? st1 : k == 2 ? st2 : st3;
    };
    auto step = [&](auto S, int s) FP8BS_INLINE {
        constexpr int kS = decltype(S)::value;
        uint8_t* cur = stage_ptr(S);
        uint8_t* nxt = stage_ptr(std::integral_constant<int, (kS + 1) % STAGES>{});
        uint8_t* ld = stage_ptr(std::integral_constant<int, (kS + STAGES - 1) % STAGES>{});
        plan_loads(s + STAGES - 1 < total);
        // (unconditional: after the last step it waits for the trailing loads and reads a
        // stage nobody uses, which keeps the control flow, and the compiler's own LDS waits,
        // simple)
        rows(cur, (lds_u8*)ld, [&]() {
            wait_groups();
            __builtin_amdgcn_s_barrier();
            read_head(nxt);
        });
        if (++cp_kb == KB) {
            store_tile(cp_tile);
            stores_pending = 1;
            cp_kb = 0;
            ++cp_tile;
        }
    };
    if constexpr (PP >= 2) {
        // Warp-specialised: waves kMathWaves.. only move data, the others only compute. Every
        // wave passes one barrier before the first step and one per step. The math waves issue
        // no loads, so their C stores are never waited for inside the loop.
        if (wave >= T::kMathWaves) {
            // With a few K blocks per tile the computing waves' C stores come every few steps and
            // compete with these waves' loads for issue; a higher issue priority puts the loads
            // first (16384 x 7168 x 768: 100.0-100.2 against 102.7-103.0 us; 4096 x 8192 x 1536:
            // 49.7-50.0 against 50.3-50.7; at K = 7168 it changed nothing or cost up to 0.8%).
            if (KB <= 12)
                __builtin_amdgcn_s_setprio(1);
            if (total > 0) {
                static_for<STAGES - 1>([&](auto S) {
                    plan_loads(decltype(S)::value < total);
                    issue_group((lds_u8*)stage_ptr(S));
                });
                wait_vmcnt_lgkm<(STAGES - 2) * T::kLoadsPerStep>();
                __builtin_amdgcn_s_barrier();
            }
            // in step s: the loads of step s + STAGES - 1 into the stage step s - 1 used, then
            // wait until those of step s + 1 have landed
            auto lstep = [&](auto S, int s) FP8BS_INLINE {
                constexpr int kS = decltype(S)::value;
                plan_loads(s + STAGES - 1 < total);
                issue_group((lds_u8*)stage_ptr(std::integral_constant<int, (kS + STAGES - 1) % STAGES>{}));
                wait_vmcnt_lgkm<(STAGES - 2) * T::kLoadsPerStep>();
                __builtin_amdgcn_s_barrier();
            };
            for (int s = 0; s < total; s += STAGES) {
                lstep(std::integral_constant<int, 0>{}, s);
                if (s + 1 < total)
                    lstep(std::integral_constant<int, 1>{}, s + 1);
                if constexpr (STAGES > 2) {
                    if (s + 2 < total)
                        lstep(std::integral_constant<int, 2>{}, s + 2);
                }
                if constexpr (STAGES > 3) {
                    if (s + 3 < total)
                        lstep(std::integral_constant<int, 3>{}, s + 3);
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
            return;
        }
        auto mstep = [&](auto S, int s) FP8BS_INLINE {
            constexpr int kS = decltype(S)::value;
            uint8_t* cur = stage_ptr(S);
            uint8_t* nxt = stage_ptr(std::integral_constant<int, (kS + 1) % STAGES>{});
            if constexpr (kFullHold) {
                rows_full(nxt, [&]() {
                    wait_lgkm0();  // the last reads of this step's stage are done
                    __builtin_amdgcn_s_barrier();
                });
            } else {
                rows(cur, (lds_u8*)nullptr, [&]() {
                    wait_lgkm0();  // this wave's reads of the stage are done
                    __builtin_amdgcn_s_barrier();
                    read_head(nxt);
                });
            }
            if (++cp_kb == KB) {
                store_tile(cp_tile);
                cp_kb = 0;
                ++cp_tile;
            }
        };
        if (total > 0) {
            __builtin_amdgcn_s_barrier();
            if constexpr (kFullHold)
                read_full(st0);
            else
                read_head(st0);
        }
        for (int s = 0; s < total; s += STAGES) {
            mstep(std::integral_constant<int, 0>{}, s);
            if (s + 1 < total)
                mstep(std::integral_constant<int, 1>{}, s + 1);
            if constexpr (STAGES > 2) {
                if (s + 2 < total)
                    mstep(std::integral_constant<int, 2>{}, s + 2);
            }
            if constexpr (STAGES > 3) {
                if (s + 3 < total)
                    mstep(std::integral_constant<int, 3>{}, s + 3);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }
    if (total > 0) {
        static_for<STAGES - 1>([&](auto S) {
            plan_loads(decltype(S)::value < total);
            issue_group((lds_u8*)stage_ptr(S));
        });
        wait_groups();
        __builtin_amdgcn_s_barrier();
        read_head(st0);
    }
    for (int s = 0; s < total; s += STAGES) {
        step(std::integral_constant<int, 0>{}, s);
        if (s + 1 < total)
            step(std::integral_constant<int, 1>{}, s + 1);
        if constexpr (STAGES > 2) {
            if (s + 2 < total)
                step(std::integral_constant<int, 2>{}, s + 2);
        }
        if constexpr (STAGES > 3) {
            if (s + 3 < total)
                step(std::integral_constant<int, 3>{}, s + 3);
        }
    }
    // the trailing load groups write LDS: let them land before the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(0);
    }
}

// ---- host side ---------------------------------------------------------------------------

// Compute units of each device, read once per device (std::call_once: the first calls may come
// from several host threads at once).

int device_cus()
{
    static std::once_flag once[kMaxDevices];
    static int cus[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return 256;
    std::call_once(once[dev], [dev] {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cus[dev] = n;
    });
    return cus[dev];
}

template <int ROUTE, int BM, int BN, int WM, int WN, int STAGES, int PP, bool SPLIT = false>
static hipError_t launch_tile(const GemmArgs& a, const GemmConfig& c, int splits = 1, float* partial = nullptr)
{
    using T = Tile<ROUTE, BM, BN, WM, WN, STAGES, PP>;
    auto kernel = gemm_kernel<ROUTE, BM, BN, WM, WN, STAGES, PP, SPLIT>;
    // workgroups of this kernel that fit on one CU at once (LDS and registers), once per device
    static std::once_flag once[kMaxDevices];
    static int per_cu[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::call_once(once[dev], [&] {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, T::kThreads, 0) != hipSuccess || n < 1)
            n = 1;
        per_cu[dev] = n;
    });
    const int tiles_m = (a.M + BM - 1) / BM;
    const int tiles_n = a.N / BN;
    const int units = tiles_m * tiles_n * (SPLIT ? splits : 1);
    int grid = device_cus() * per_cu[dev];
    if (c.persistent == 0 || grid > units)
        grid = units;
    return launch_kernel(kernel, dim3(grid), dim3(T::kThreads), a.stream, (const uint8_t*)a.A, a.a_scale,
                         (const uint8_t*)a.B, a.b_scale, (uint16_t*)a.C, a.M, a.N, a.K, tiles_m, tiles_n,
                         c.group_m > 0 ? c.group_m : 1, c.xcd_remap, SPLIT ? splits : 1, partial, c.c_store);
}

// Instantiated shapes: {BM, BN, WM, WN, STAGES, ping-pong}. Index = GemmConfig::variant.
#define FP8BS_VARIANTS(X)        \
    X(0, 128, 128, 2, 2, 3, 0)   \
    X(1, 256, 256, 4, 2, 2, 0)   \
    X(2, 256, 256, 2, 4, 2, 0)   \
    X(3, 128, 256, 2, 2, 3, 0)   \
    X(4, 256, 128, 2, 2, 3, 0)   \
    X(5, 128, 256, 2, 4, 3, 0)   \
    X(6, 256, 128, 4, 2, 3, 0)   \
    X(7, 128, 64, 2, 1, 3, 0)    \
    X(8, 256, 128, 4, 2, 2, 0)   \
    X(9, 128, 128, 2, 2, 4, 0)   \
    X(10, 128, 128, 2, 2, 2, 0)  \
    X(11, 256, 128, 4, 2, 2, 1)  \
    X(12, 128, 256, 2, 4, 2, 1)  \
    X(13, 256, 128, 4, 2, 3, 2)  \
    X(14, 128, 256, 2, 4, 3, 2)  \
    X(15, 256, 128, 2, 2, 3, 2)  \
    X(16, 128, 128, 2, 2, 3, 2)

const VariantInfo* variant_info(int v)
{
    static const VariantInfo table[] = {
#define X(id, bm, bn, wm, wn, st, pp) {bm, bn, wm, wn, st, pp},
        FP8BS_VARIANTS(X)
#undef X
    };
    if (v < 0 || v >= (int)(sizeof(table) / sizeof(table[0])))
        return nullptr;
    return &table[v];
}

template <int BM, int BN, int WM, int WN, int ST>
static constexpr bool mx_fits()
{
    return (BM / WM) % 64 == 0 && (BN / WN) % 64 == 0 && ST * (BM * 132 + BN * 132) <= kLdsCapacity;
}

template <int BM, int BN, int WM, int WN, int ST, int PP>
static hipError_t launch_variant(int route, const GemmArgs& a, const GemmConfig& c)
{
    constexpr int TN = BN / WN;
    if (route == kRouteBS) {
        if constexpr (TN <= 128 && 128 % TN == 0)
            return launch_tile<kRouteBS, BM, BN, WM, WN, ST, PP>(a, c);
        else
            return hipErrorInvalidValue;
    }
    if (route == kRoutePT)
        return launch_tile<kRoutePT, BM, BN, WM, WN, ST, PP>(a, c);
    if constexpr (mx_fits<BM, BN, WM, WN, ST>())
        return launch_tile<kRouteMX, BM, BN, WM, WN, ST, PP>(a, c);
    else
        return hipErrorInvalidValue;
}

bool variant_supports(int route, int v)
{
    const VariantInfo* vi = variant_info(v);
    if (!vi)
        return false;
    const int TM = vi->block_m / vi->waves_m, TN = vi->block_n / vi->waves_n;
    if (route == kRouteBS)
        return TN <= 128 && 128 % TN == 0;
    if (route == kRoutePT)
        return true;
    return TM % 64 == 0 && TN % 64 == 0 && vi->stages * (vi->block_m * 132 + vi->block_n * 132) <= kLdsCapacity;
}

// Route BS with K split `splits` ways, fp32 sums into partial[splits][M][N]: the
// warp-specialised tiles only (the selector's choice wherever a shape's tiles leave CUs idle).
bool split_supported(int v)
{
    return v == 13 || v == 14 || v == 16;
}

hipError_t launch_gemm_split(const GemmArgs& a, const GemmConfig& c, int splits, float* partial)
{
    if (splits < 1 || (a.K >> 7) % splits != 0 || !partial)
        return hipErrorInvalidValue;
    switch (c.variant) {
    case 13:
        return launch_tile<kRouteBS, 256, 128, 4, 2, 3, 2, true>(a, c, splits, partial);
    case 14:
        return launch_tile<kRouteBS, 128, 256, 2, 4, 3, 2, true>(a, c, splits, partial);
    case 16:
        return launch_tile<kRouteBS, 128, 128, 2, 2, 3, 2, true>(a, c, splits, partial);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm(int route, const GemmArgs& a, const GemmConfig& c)
{
    switch (c.variant) {
#define X(id, bm, bn, wm, wn, st, pp) \
    case id:                          \
        return launch_variant<bm, bn, wm, wn, st, pp>(route, a, c);
        FP8BS_VARIANTS(X)
#undef X
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace fp8bs
