// api.hip -- the C ABI of libfp8bs (declared in include/fp8bs.h): argument validation on the
// host, then an asynchronous launch on the caller's stream. Nothing here allocates memory or
// synchronises the host.
#include "fp8bs.h"
#include "launch.hpp"

#include <cstring>

#include <stdint.h>

namespace {

constexpr int kVersion = 10200;  // 1.2.0: fp8bs_config.c_store

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? FP8BS_OK : FP8BS_E_HIP; }

// The kernels address operands with 32-bit byte offsets.
bool fits_offsets(int M, int N, int K)
{
    return (int64_t)M * K < (int64_t)1 << 31 && (int64_t)N * K < (int64_t)1 << 31;
}

// Shape rules of route BS: K in whole 128-wide blocks, N in whole 128-row weight blocks.
int check_bs_shape(int M, int N, int K)
{
    if (M < 0 || N < 128 || K < 128 || N % 128 != 0 || K % 128 != 0 || !fits_offsets(M, N, K))
        return FP8BS_E_SHAPE;
    return FP8BS_OK;
}

// Shape rules of route MX (page "aiter PR #6370", Constraints): M and N in whole 64-row packed
// scale groups, K in whole 128-wide steps and at least two of them.
int check_mx_shape(int M, int N, int K)
{
    if (M < 0 || M % 64 != 0 || N < 64 || N % 64 != 0 || K < 256 || K % 128 != 0 || !fits_offsets(M, N, K))
        return FP8BS_E_SHAPE;
    return FP8BS_OK;
}

// Shape rules of route PT: weight rows in whole 64-row windows of the prepared order, K in
// whole 128-wide steps; any M (the last row tile masks its stores).
int check_pt_shape(int M, int N, int K)
{
    if (M < 0 || N < 64 || N % 64 != 0 || K < 128 || K % 128 != 0 || !fits_offsets(M, N, K))
        return FP8BS_E_SHAPE;
    return FP8BS_OK;
}

int find_variant(const fp8bs_config& c)
{
    for (int v = 0;; ++v) {
        const fp8bs::VariantInfo* vi = fp8bs::variant_info(v);
        if (!vi)
            return -1;
        if (vi->block_m == c.block_m && vi->block_n == c.block_n && vi->waves_m == c.waves_m &&
            vi->waves_n == c.waves_n && vi->stages == c.stages && vi->pingpong == c.pingpong)
            return v;
    }
}

fp8bs_config make_config(int variant, int group_m, int xcd_remap, int persistent, int c_store)
{
    const fp8bs::VariantInfo* vi = fp8bs::variant_info(variant);
    fp8bs_config c;
    c.block_m = vi->block_m;
    c.block_n = vi->block_n;
    c.waves_m = vi->waves_m;
    c.waves_n = vi->waves_n;
    c.stages = vi->stages;
    c.pingpong = vi->pingpong;
    c.group_m = group_m;
    c.xcd_remap = xcd_remap;
    c.persistent = persistent;
    c.small_m = 0;
    c.c_store = c_store;
    return c;
}

// Rows the small-M kernel takes: chunks of kDecodeMaxRows rows, at most kDecodeMaxChunks of them.
bool small_m_rows_ok(int M)
{
    return M >= 1 && (M + fp8bs::kDecodeMaxRows - 1) / fp8bs::kDecodeMaxRows <= fp8bs::kDecodeMaxChunks;
}

// The small-M kernel: the tile fields do not apply to it and are zeroed.
fp8bs_config small_m_config()
{
    fp8bs_config c;
    memset(&c, 0, sizeof(c));
    c.small_m = fp8bs::kDecodeAuto;
    return c;
}

// Shape-driven choice of the workgroup tile (page "Flydsl Fp8 Blockscale Gemm", Per-shape
// recipes: selection by (M, N, K) alone, never by layer). Prefer the 256x256 tile when it
// still gives at least two workgroups per CU, else the 256x128 / 128x256 tiles (warp-
// specialised schedule) when they fill the 256 CUs, else 128x128 (or 128x64 for MX with N not
// a multiple of 128).
fp8bs_config select(int route, int M, int N, int K)
{
    const int kCUs = 256;
    const int group_m = 4;
    auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * (N / bn); };
    // XCD mapping 1 (each XCD walks its own contiguous eighth of the tile order) keeps the
    // tiles one XCD runs at the same time next to each other, which pays while a band of
    // group_m tile rows holds at most about two waves of resident workgroups. On wider outputs
    // mapping 2 puts every XCD on its own block of the same window of the output at once, so a
    // weight panel is reused by the tile rows that need it while it is still cached (measured
    // on the 4096 x 65536 x 1536 shape: about 12% faster than mapping 1, 5% faster than
    // round-robin; on the 16384 x 8192 x 1280 shape mapping 1 is 6% faster than mapping 2).
    // C store policy by the size of C (all three give the same bits; each policy forced through
    // the *_with_config entry, alternating, on several boxes):
    //  * larger than the 256 MiB memory-side cache: written through as non-temporal lines (2),
    //    which keeps C from pushing the operands out of that cache (4096 x 65536 x 1536:
    //    392.8 against 403.3 us; written through without the hint, 423 against 413; 16384 x
    //    16384 x 1536 on 128 x 256 tiles: 399 against 514);
    //  * at most 64 MiB: written through the L2 (1). Such a C is written in few rounds of tiles,
    //    close to the kernel's end, and what is still dirty in the L2s then is written back
    //    after the last tile (4096 x 2048 x 7168: 51.0 against 52.5 us, the route-PT twin 43.8
    //    against 45.5; 4096 x 8192 x 1536: 50.2 against 51.9, on 128 x 256 tiles 51.2 against
    //    53.5; 16384 x 1536 x 7168: 148.5 against 149.4);
    //  * in between, the ordinary write-back stores, which the L2 absorbs round by round
    //    (16384 x 5120 x 2048: 137.6 against 138.5 written through, 140.5 non-temporal;
    //    16384 x 7168 x 768: from 3% faster to 5% slower written through depending on the box,
    //    on 128 x 256 tiles 109.4 against 103.1; 8192 x 8192 x 2048 and 4096 x 16384 x 7168 on
    //    128 x 256 tiles: 127.7 against 127.6, 416.9 against 406.2).
    const int64_t c_bytes = (int64_t)M * N * 2;
    const int c_store = c_bytes > ((int64_t)256 << 20) ? 2 : c_bytes <= ((int64_t)64 << 20) ? 1 : 0;
    auto cfg = [&](int variant, int block_n, int gm = group_m) {
        const int xcd = gm * (N / block_n) <= 2 * kCUs ? 1 : 2;
        return make_config(variant, gm, xcd, 1, c_store);
    };
    // The small-M kernel against the main kernel. With few rows the main kernel runs one round
    // of 128-row tiles whose time is set by the K loop (warp-specialised 128 x 128 tiles, route
    // BS: about 3.7 us + 0.47 us per K block, whatever N), while the small-M kernel splits K over its waves
    // and spreads the work over chunks x N/16 workgroups: its time grows with W = chunks x N/16 x
    // ceil(min(M, 64)/16), the 16 x 16 x 128 products per K block. It always wins for M <= 4
    // (the weights streamed once: 1 x 65536 x 1536 15.8 against 19.2 us); up to 16 rows, where
    // its cost is streaming the weights, unless one row of 128 x 256 main-kernel tiles already
    // fills the CUs (M = 8 and 16 with 65536 x 1536 weights: 17.5 against 18.5 us); from 17 rows
    // while W stays within a limit: 3072 for route BS from K = 2048, else 2048 (routes MX and PT,
    // whose main kernel has no promote, and route BS below K = 2048). Examples, main kernel
    // against small-M kernel: BS M = 128, 2048 x 2048 weights: 11.2 against 4.2 us (W = 1024);
    // BS M = 384, 2048 x 2048: 11.2 against 9.9 (W = 3072), M = 512: 11.3 against 12.8 (W =
    // 4096); BS M = 48, 16384 x 1024: 7.2 against 8.4 (W = 3072, K = 1024); BS M = 128, 7168 x
    // 7168: 29.9 against 31.5 (W = 3584); MX M = 128, 2048 x 2048: 9.2 against 4.4 (W = 1024),
    // M = 192, 4096 x 4096: 14.8 against 17.2 (W = 3072); PT M = 192, 4096 x 4096: 14.2 against
    // 16.6; BS M = 64, 28672 x 8192: 43.3 against 59.5 (W = 7168).
    if (small_m_rows_ok(M)) {
        if (M <= 4)
            return small_m_config();
        if (M <= 16) {
            if (!(N % 256 == 0 && N / 256 >= kCUs))
                return small_m_config();
        } else {
            const int64_t W = (int64_t)((M + fp8bs::kDecodeMaxRows - 1) / fp8bs::kDecodeMaxRows) * (N / 16) *
                              ((std::min(M, fp8bs::kDecodeMaxRows) + 15) / 16);
            const bool lean = route == fp8bs::kRouteMX || route == fp8bs::kRoutePT;
            const int64_t limit = !lean && K >= 2048 ? 3072 : 2048;
            if (W <= limit)
                return small_m_config();
        }
    }
    if ((route == fp8bs::kRouteMX || route == fp8bs::kRoutePT) && N % 128 != 0)
        return cfg(7, 64);
    auto rounds = [&](int bm, int bn) { return (tiles(bm, bn) + kCUs - 1) / kCUs; };
    // 128 x 128 tiles run warp-specialised (four math waves, one per SIMD, beside four loader
    // waves). Grids of one round are bound by each tile's K loop, which the loader waves shorten:
    // BS 512 x 7168 x 7168 31.8 us against 39.4 with every wave loading (and 39.6 with 128 x 64
    // tiles), 1024 x 3072 x 7168 31.4 against 39.3, 128 x 16384 x 1536 9.8 against 11.5; MX
    // 512 x 7168 x 7168 26.5 against 32.1, 1024 x 2048 x 7168 24.3 against 31.1; with more
    // rounds too (BS 1024 x 16384 x 1536: 32.0 against 38.9).
    auto square = [&]() { return cfg(16, 128); };
    // when one row of 128-row tiles covers M, 256-row tiles would only add padding: 128 x 256
    // (warp-specialised) where those fill the CUs or need fewer rounds of them, else 128 x 128
    // (M = 64: 65536 x 1536 weights 18.9 us against 27 us with 256 x 128 tiles; 32768 x 1536
    // 11.5 against 15.3 us; 32768 x 7168 39.7 against 55.3 us; 36864 x 7168, 144 tiles of
    // 128 x 256 in one round against 288 of 128 x 128 in two: 49.1 against 74.7 us)
    if (M <= 128)
        return N % 256 == 0 && (tiles(128, 256) >= kCUs || rounds(128, 256) < rounds(128, 128)) ? cfg(14, 256)
                                                                                                : square();
    // 256 x 256 tiles when they fill at least one round of the CUs and their rounds, each as
    // long as two of 256 x 128 tiles, are no more than those tiles would need (65536 x 1536
    // weights, M = 256: one round, MX 28.3 against 32.0 us with 256 x 128 tiles; route BS,
    // 24576 x 1536, M = 1024: 384 tiles in two rounds, 51.4 against 42.5 for 768 of 256 x 128
    // in three; 36864 x 7168, M = 1024: 576 tiles in three rounds, 286.7 against 258.6 for 1152
    // in five)
    // Route BS at K <= 1536 takes the warp-specialised 128 x 256 tile there instead where those
    // make at least four rounds of the CUs, walked in bands of 8 tile rows (1024 rows, as 4 rows
    // of 256-row tiles): with few K blocks per tile and several tiles per workgroup, its loader
    // waves keep the next tile's operands coming while the computing waves store C
    // (16384 x 7168 x 768: 103.1 against 105.7 us; 4096 x 65536 x 1536: 408.4 against 421.1;
    // 4096 x 8192 x 1536: 51.2 against 51.4; 16384 x 16384 x 1536: 399.2 against 393.4, whose
    // runs spread over 393-406). Deeper K keeps the 256 x 256
    // tile (8192 x 8192 x 2048: 127.6 against 126.4; 4096 x 16384 x 7168: 406.2 against 386.1),
    // and so do routes MX and PT, which have no promote (route PT, 4096 x 65536 x 1536: 418.1
    // against 396.0).
    if (N % 256 == 0 && tiles(256, 256) >= kCUs && 2 * rounds(256, 256) <= rounds(256, 128))
        return route == fp8bs::kRouteBS && K <= 1536 && tiles(128, 256) >= 4 * kCUs ? cfg(14, 256, 8)
                                                                                    : cfg(2, 256);
    // the 256x128 / 128x256 tiles run warp-specialised (four loader waves beside the eight
    // math waves): measured 5-7% faster than the same tiles with every wave loading on the
    // 4096 x 2048 x 7168 and 16384 x 1536 x 7168 shapes
    // 256 x 128 tiles just past one round (257 to 384: two rounds, the second mostly idle):
    // three rounds of the warp-specialised 128 x 128 tiles finish sooner, a round of those
    // costing about 1.25x half a round of 256 x 128 tiles (BS 1280 x 7168 x 2048: 30.1 against
    // 32.5 us, 2304 x 3840 x 4096: 54.0 against 56.9; MX 4352 x 2048 x 7168: 72.9 against 80.3)
    if (tiles(256, 128) > kCUs && 2 * tiles(256, 128) <= 3 * kCUs)
        return square();
    // of the two, 128 x 256 where it fills the CUs as well: 1-2.5% faster with the same waves
    // (4096 x 2048 x 7168 52.8 against 53.6 us, 16384 x 1536 x 7168 151.7 against 153.7,
    // 8192 x 1024 x 4096 32.6 against 33.5, 2048 x 4096 x 7168 52.9 against 53.4)
    if (tiles(256, 128) >= kCUs)
        return N % 256 == 0 && tiles(128, 256) >= kCUs ? cfg(14, 256) : cfg(13, 128);
    if (N % 256 == 0 && tiles(128, 256) >= kCUs)
        return cfg(14, 256);
    // 128x128 tiles, unless they would need more rounds of the CUs than the larger ones (7168 x
    // 7168 weights, M = 640: 280 tiles in two rounds, 74.6 us, against 168 tiles of 256 x 128 in
    // one, 46.1 us)
    if (rounds(256, 128) < rounds(128, 128))
        return cfg(13, 128);
    if (N % 256 == 0 && rounds(128, 256) < rounds(128, 128))
        return cfg(14, 256);
    return square();
}

// Split K for route BS: the number of equal K ranges per output tile. With the tiles the
// selector picks (cfg), a shape whose tiles number fewer than the CUs, at K > 4096, takes the
// most ranges that keep every work unit within one round of the CUs and at least 8 K blocks deep
// (K/128 must divide evenly); 1 (no split) otherwise. The second pass and its launch cost about
// 4 us, which shallower K does not repay (measured, 128 x 128 tiles, plain against split:
// 256 x 7168 x 7168 25.8 us against 23.2 with 2 ranges; 128 x 7168 x 7168 25.8 against 19.0
// with 4; 1000 x 1536 x 7168 25.7 against 21.4 with 2; 1024 x 2048 x 7168 25.7 against 25.6
// with 2; 512 x 2048 x 4096 16.2 against 17.5 with 2 and 17.8 with 4; 256 x 4096 x 2048 10.0
// against 14.4 with 2).
int choose_splits(int M, int N, int K, const fp8bs_config& cfg)
{
    const int kCUs = 256;
    if (cfg.small_m != 0 || K <= 4096)
        return 1;
    const int v = find_variant(cfg);
    if (v < 0 || !fp8bs::split_supported(v))
        return 1;
    const int tiles = ((M + cfg.block_m - 1) / cfg.block_m) * (N / cfg.block_n);
    const int KB = K >> 7;
    int best = 1;
    for (int s = 2; s <= 8; ++s)
        if (KB % s == 0 && KB / s >= 8 && (int64_t)tiles * s <= kCUs)
            best = s;
    return best;
}

size_t splitk_bytes(int M, int N, int splits)
{
    return splits > 1 ? (size_t)splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

int check_config(int route, const fp8bs_config* c, int N, fp8bs::GemmConfig* out)
{
    if (!c)
        return FP8BS_E_NULL;
    if (c->small_m != 0)
        return FP8BS_E_CONFIG;  // handled by run()
    const int v = find_variant(*c);
    if (v < 0 || !fp8bs::variant_supports(route, v) || c->group_m < 1 || N % c->block_n != 0 ||
        (c->xcd_remap < 0 || c->xcd_remap > 2) || (c->persistent != 0 && c->persistent != 1) ||
        (c->c_store < 0 || c->c_store > 2))
        return FP8BS_E_CONFIG;
    out->variant = v;
    out->group_m = c->group_m;
    out->xcd_remap = c->xcd_remap;
    out->persistent = c->persistent;
    out->c_store = c->c_store;
    return FP8BS_OK;
}

int run(int route, const void* A, const void* a_scale, const void* B_prep, const void* b_scale, void* C,
        int M, int N, int K, const fp8bs_config* cfg, hipStream_t stream)
{
    fp8bs::GemmArgs args{A, a_scale, B_prep, b_scale, C, M, N, K, stream};
    if (cfg && cfg->small_m >= fp8bs::kDecodeAuto && cfg->small_m <= fp8bs::kDecodeLdsPair) {
        // the route-MX entry points that come here carry the packed activation scales
        if (!small_m_rows_ok(M) ||
            (cfg->small_m == fp8bs::kDecodeLdsPair && (std::min(M, fp8bs::kDecodeMaxRows) > 32 || N % 32 != 0)))
            return FP8BS_E_CONFIG;
        const int r = route == fp8bs::kRouteMX ? fp8bs::kRouteMXPacked : route;
        return hip_status(fp8bs::launch_decode(r, args, cfg->small_m));
    }
    fp8bs::GemmConfig gc;
    int st = check_config(route, cfg, N, &gc);
    if (st != FP8BS_OK)
        return st;
    return hip_status(fp8bs::launch_gemm(route, args, gc));
}

int check_bs_args(const void* A, const float* a_scale, const void* B_prep, const float* b_scale, void* C,
                  int M, int N, int K)
{
    int st = check_bs_shape(M, N, K);
    if (st != FP8BS_OK)
        return st;
    if (M == 0)
        return -1;  // nothing to do
    if (!A || !a_scale || !B_prep || !b_scale || !C)
        return FP8BS_E_NULL;
    if (!aligned(A, 16) || !aligned(B_prep, 16) || !aligned(C, 16) || !aligned(a_scale, 4) ||
        !aligned(b_scale, 4))
        return FP8BS_E_ALIGN;
    return FP8BS_OK;
}

int check_mx_args(const void* A, const void* a_scale_packed, const void* B_prep, const void* b_scale_packed,
                  void* C, int M, int N, int K)
{
    int st = check_mx_shape(M, N, K);
    if (st != FP8BS_OK)
        return st;
    if (M == 0)
        return -1;
    if (!A || !a_scale_packed || !B_prep || !b_scale_packed || !C)
        return FP8BS_E_NULL;
    if (!aligned(A, 16) || !aligned(B_prep, 16) || !aligned(C, 16) || !aligned(a_scale_packed, 16) ||
        !aligned(b_scale_packed, 16))
        return FP8BS_E_ALIGN;
    return FP8BS_OK;
}

int check_pt_args(const void* A, const float* a_scale, const void* B_prep, const float* b_scale, void* C,
                  int M, int N, int K)
{
    int st = check_pt_shape(M, N, K);
    if (st != FP8BS_OK)
        return st;
    if (M == 0)
        return -1;
    if (!A || !a_scale || !B_prep || !b_scale || !C)
        return FP8BS_E_NULL;
    if (!aligned(A, 16) || !aligned(B_prep, 16) || !aligned(C, 16) || !aligned(a_scale, 4) ||
        !aligned(b_scale, 16))
        return FP8BS_E_ALIGN;
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
    case FP8BS_E_CONFIG: return "invalid kernel configuration for this shape or route";
    case FP8BS_E_HIP: return "the HIP runtime reported an error while enqueueing work";
    case FP8BS_E_WORKSPACE: return "the workspace is missing, misaligned or smaller than the call needs";
    default: return "unknown status";
    }
}

size_t fp8bs_prep_weight_bytes(int N, int K)
{
    if (N <= 0 || K <= 0)
        return 0;
    return (size_t)N * (size_t)K;
}

size_t fp8bs_prep_bytes(int N, int K) { return fp8bs_prep_weight_bytes(N, K); }

int fp8bs_prep_weights(const void* B, void* B_prep, int N, int K, hipStream_t stream)
{
    if (N < 64 || N % 64 != 0 || K < 128 || K % 128 != 0)
        return FP8BS_E_SHAPE;
    if (!B || !B_prep)
        return FP8BS_E_NULL;
    if (!aligned(B, 16) || !aligned(B_prep, 16))
        return FP8BS_E_ALIGN;
    return hip_status(fp8bs::launch_prep_weights(B, B_prep, N, K, stream));
}

int fp8bs_select_config(int route, int M, int N, int K, fp8bs_config* out)
{
    if (!out)
        return FP8BS_E_NULL;
    if (route != FP8BS_ROUTE_BS && route != FP8BS_ROUTE_MX && route != FP8BS_ROUTE_PT)
        return FP8BS_E_CONFIG;
    int st = route == FP8BS_ROUTE_BS   ? check_bs_shape(M, N, K)
             : route == FP8BS_ROUTE_MX ? check_mx_shape(M, N, K)
                                       : check_pt_shape(M, N, K);
    if (st != FP8BS_OK)
        return st;
    *out = select(route, M, N, K);
    return FP8BS_OK;
}

int fp8bs_gemm(const void* A, const float* a_scale, const void* B_prep, const float* b_scale, void* C,
               int M, int N, int K, hipStream_t stream)
{
    int st = check_bs_args(A, a_scale, B_prep, b_scale, C, M, N, K);
    if (st != FP8BS_OK)
        return st < 0 ? FP8BS_OK : st;
    const fp8bs_config cfg = select(fp8bs::kRouteBS, M, N, K);
    return run(fp8bs::kRouteBS, A, a_scale, B_prep, b_scale, C, M, N, K, &cfg, stream);
}

int fp8bs_gemm_with_config(const void* A, const float* a_scale, const void* B_prep, const float* b_scale,
                           void* C, int M, int N, int K, const fp8bs_config* config, hipStream_t stream)
{
    int st = check_bs_args(A, a_scale, B_prep, b_scale, C, M, N, K);
    if (st != FP8BS_OK)
        return st < 0 ? FP8BS_OK : st;
    return run(fp8bs::kRouteBS, A, a_scale, B_prep, b_scale, C, M, N, K, config, stream);
}

size_t fp8bs_splitk_workspace_bytes(int M, int N, int K, int splits)
{
    if (check_bs_shape(M, N, K) != FP8BS_OK || M == 0)
        return 0;
    const fp8bs_config cfg = select(fp8bs::kRouteBS, M, N, K);
    if (splits <= 0)
        splits = choose_splits(M, N, K, cfg);
    return splitk_bytes(M, N, splits);
}

}  // extern "C"

namespace {

// fp8bs_gemm_splitk's work with workspace ws of ws_bytes (ws may be null when nothing splits);
// `noalloc`: ws is the library's scratch, and a call that needs more returns FP8BS_E_WORKSPACE
int splitk_run(const void* A, const float* a_scale, const void* B_prep, const float* b_scale, void* C, int M,
               int N, int K, int splits, void* ws, size_t ws_bytes, bool noalloc, hipStream_t stream)
{
    int st = check_bs_args(A, a_scale, B_prep, b_scale, C, M, N, K);
    if (st != FP8BS_OK)
        return st < 0 ? FP8BS_OK : st;
    const fp8bs_config cfg = select(fp8bs::kRouteBS, M, N, K);
    if (splits <= 0)
        splits = choose_splits(M, N, K, cfg);
    if (splits > 1 && (cfg.small_m != 0 || !fp8bs::split_supported(find_variant(cfg)) || (K >> 7) % splits != 0 ||
                       splits > 64))
        return FP8BS_E_CONFIG;
    if (splits == 1)
        return run(fp8bs::kRouteBS, A, a_scale, B_prep, b_scale, C, M, N, K, &cfg, stream);
    const size_t need = splitk_bytes(M, N, splits);
    if (noalloc) {
        if (need > ws_bytes)
            return FP8BS_E_WORKSPACE;
        ws = fp8bs::splitk_scratch();
        if (!ws)
            return FP8BS_E_HIP;
    }
    if (!ws || !aligned(ws, 256) || ws_bytes < need)
        return FP8BS_E_WORKSPACE;
    fp8bs::GemmConfig gc;
    st = check_config(fp8bs::kRouteBS, &cfg, N, &gc);
    if (st != FP8BS_OK)
        return st;
    fp8bs::GemmArgs args{A, a_scale, B_prep, b_scale, C, M, N, K, stream};
    hipError_t e = fp8bs::launch_gemm_split(args, gc, splits, (float*)ws);
    if (e != hipSuccess)
        return FP8BS_E_HIP;
    return hip_status(fp8bs::launch_splitk_reduce((const float*)ws, splits, C, M, N, stream));
}

}  // namespace

extern "C" {

int fp8bs_gemm_splitk(const void* A, const float* a_scale, const void* B_prep, const float* b_scale, void* C,
                      int M, int N, int K, int splits, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    return splitk_run(A, a_scale, B_prep, b_scale, C, M, N, K, splits, workspace, workspace_bytes, false, stream);
}

int fp8bs_gemm_splitk_noalloc(const void* A, const float* a_scale, const void* B_prep, const float* b_scale,
                              void* C, int M, int N, int K, int splits, hipStream_t stream)
{
    return splitk_run(A, a_scale, B_prep, b_scale, C, M, N, K, splits, nullptr, fp8bs::kSplitkScratchBytes, true,
                      stream);
}

size_t fp8mx_packed_scale_bytes(int rows, int K)
{
    if (rows <= 0 || K <= 0)
        return 0;
    return (size_t)rows * (size_t)(K / 32);
}

size_t fp8mx_scale_bytes(int rows, int K) { return fp8mx_packed_scale_bytes(rows, K); }

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
    return hip_status(fp8bs::launch_pack_scales(a_e8m0, a_scale_packed, M, K, 0, stream));
}

int fp8mx_prep_weights(const void* B, const void* b_e8m0, void* B_prep, void* b_scale_packed, int N, int K,
                       hipStream_t stream)
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
    return hip_status(fp8bs::launch_pack_scales(b_e8m0, b_scale_packed, N, K, 1, stream));
}

int fp8mx_gemm(const void* A, const void* a_scale_packed, const void* B_prep, const void* b_scale_packed,
               void* C, int M, int N, int K, hipStream_t stream)
{
    int st = check_mx_args(A, a_scale_packed, B_prep, b_scale_packed, C, M, N, K);
    if (st != FP8BS_OK)
        return st < 0 ? FP8BS_OK : st;
    const fp8bs_config cfg = select(fp8bs::kRouteMX, M, N, K);
    return run(fp8bs::kRouteMX, A, a_scale_packed, B_prep, b_scale_packed, C, M, N, K, &cfg, stream);
}

int fp8mx_gemm_with_config(const void* A, const void* a_scale_packed, const void* B_prep,
                           const void* b_scale_packed, void* C, int M, int N, int K, const fp8bs_config* config,
                           hipStream_t stream)
{
    int st = check_mx_args(A, a_scale_packed, B_prep, b_scale_packed, C, M, N, K);
    if (st != FP8BS_OK)
        return st < 0 ? FP8BS_OK : st;
    return run(fp8bs::kRouteMX, A, a_scale_packed, B_prep, b_scale_packed, C, M, N, K, config, stream);
}

int fp8pt_gemm(const void* A, const float* a_scale, const void* B_prep, const float* b_scale, void* C,
               int M, int N, int K, hipStream_t stream)
{
    int st = check_pt_args(A, a_scale, B_prep, b_scale, C, M, N, K);
    if (st != FP8BS_OK)
        return st < 0 ? FP8BS_OK : st;
    const fp8bs_config cfg = select(fp8bs::kRoutePT, M, N, K);
    return run(fp8bs::kRoutePT, A, a_scale, B_prep, b_scale, C, M, N, K, &cfg, stream);
}

int fp8pt_gemm_with_config(const void* A, const float* a_scale, const void* B_prep, const float* b_scale,
                           void* C, int M, int N, int K, const fp8bs_config* config, hipStream_t stream)
{
    int st = check_pt_args(A, a_scale, B_prep, b_scale, C, M, N, K);
    if (st != FP8BS_OK)
        return st < 0 ? FP8BS_OK : st;
    return run(fp8bs::kRoutePT, A, a_scale, B_prep, b_scale, C, M, N, K, config, stream);
}

static int quantize(int route, const void* x, int x_dtype, void* codes, void* scales, int M, int K, int group,
                    size_t scale_align, hipStream_t stream)
{
    if (M < 0 || K < group || K % group != 0)
        return FP8BS_E_SHAPE;
    if (x_dtype != FP8BS_IN_F32 && x_dtype != FP8BS_IN_BF16)
        return FP8BS_E_CONFIG;
    if (M == 0)
        return FP8BS_OK;
    if (!x || !codes || !scales)
        return FP8BS_E_NULL;
    if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, scale_align))
        return FP8BS_E_ALIGN;
    return hip_status(fp8bs::launch_quantize(route, x, x_dtype == FP8BS_IN_BF16, codes, scales, M, K, stream));
}

int fp8bs_quantize_act(const void* x, int x_dtype, void* A_codes, float* a_scale, int M, int K, hipStream_t stream)
{
    return quantize(fp8bs::kRouteBS, x, x_dtype, A_codes, a_scale, M, K, 128, 4, stream);
}

int fp8mx_quantize_act(const void* x, int x_dtype, void* A_codes, void* a_e8m0, int M, int K, hipStream_t stream)
{
    return quantize(fp8bs::kRouteMX, x, x_dtype, A_codes, a_e8m0, M, K, 32, 1, stream);
}

int fp8mx_gemm_small_m(const void* A, const void* a_e8m0, const void* B_prep, const void* b_scale_packed, void* C,
                       int M, int N, int K, hipStream_t stream)
{
    if (M < 0 || (M > 0 && !small_m_rows_ok(M)) || N < 64 || N % 64 != 0 || K < 256 || K % 128 != 0 ||
        !fits_offsets(M, N, K))
        return FP8BS_E_SHAPE;
    if (M == 0)
        return FP8BS_OK;
    if (!A || !a_e8m0 || !B_prep || !b_scale_packed || !C)
        return FP8BS_E_NULL;
    if (!aligned(A, 16) || !aligned(B_prep, 16) || !aligned(C, 16) || !aligned(b_scale_packed, 16))
        return FP8BS_E_ALIGN;
    fp8bs::GemmArgs args{A, a_e8m0, B_prep, b_scale_packed, C, M, N, K, stream};
    return hip_status(fp8bs::launch_decode(fp8bs::kRouteMX, args, fp8bs::kDecodeAuto));
}

int fp8bs_mfma_ceiling(const void* A, const void* B_prep, int M, int N, int K, int iters, float* sink, int sink_len,
                       long long* flops, hipStream_t stream)
{
    if (M < 64 || N < 64 || K < 128 || K % 128 != 0 || iters < 1 || sink_len < 8 || !fits_offsets(M, N, K))
        return FP8BS_E_SHAPE;
    if (!A || !B_prep || !sink)
        return FP8BS_E_NULL;
    if (!aligned(A, 16) || !aligned(B_prep, 16) || !aligned(sink, 4))
        return FP8BS_E_ALIGN;
    return hip_status(fp8bs::launch_mfma_ceiling(A, B_prep, M, N, K, iters, sink, sink_len, flops, stream));
}

size_t fp8bs_loop_probe_out_bytes(int parts)
{
    return fp8bs::loop_probe_parts_ok(parts) ? fp8bs::loop_probe_out_bytes(parts) : 0;
}

int fp8bs_loop_probe(int parts, const void* A, const void* B_prep, int M, int N, int K, int steps, void* out,
                     size_t out_bytes, float* sink, int sink_len, long long* flops, hipStream_t stream)
{
    if (!fp8bs::loop_probe_parts_ok(parts))
        return FP8BS_E_CONFIG;
    const size_t step_bytes = (parts & 16) ? 64 * 1024 : 48 * 1024;
    if (M < 1 || N < 1 || K < 128 || K % 128 != 0 || steps < 1 || !fits_offsets(M, N, K) ||
        (size_t)M * K < std::max<size_t>(step_bytes, 32 * 1024) || (size_t)N * K < 32 * 1024)
        return FP8BS_E_SHAPE;
    const size_t need = fp8bs::loop_probe_out_bytes(parts);
    if (!A || !B_prep || !sink || (need && !out))
        return FP8BS_E_NULL;
    if (!aligned(A, 16) || !aligned(B_prep, 16) || !aligned(sink, 4) || (need && !aligned(out, 16)))
        return FP8BS_E_ALIGN;
    if (need > out_bytes || sink_len < 8 * 256)
        return FP8BS_E_WORKSPACE;
    return hip_status(fp8bs::launch_loop_probe(parts, A, B_prep, (size_t)M * K, steps, out, out_bytes, sink, sink_len,
                                               flops, stream));
}

}  // extern "C"
