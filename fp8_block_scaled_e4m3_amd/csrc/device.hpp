// device.hpp -- gfx950 device helpers shared by the GEMM kernels of libfp8bs.
//
// Matrix-core facts used throughout (checked on the device by the parity tests):
//  * v_mfma_f32_16x16x128_f8f6f4 with e4m3 operands multiplies a 16x128 tile by a 128x16 tile.
//    Each lane supplies 32 fp8 bytes (8 VGPRs) of one row of each operand: operand row =
//    lane % 16; with q = lane / 16, bytes 0..15 are K [16q, 16q+16) and bytes 16..31 are
//    K [64+16q, 64+16q+16). So one lane's 32 bytes are two 16-byte chunks, q and q+4, of the
//    row's 128-byte K block.
//  * The scaled form takes one ue8m0 byte per lane and operand (op_sel picks the byte of the
//    32-bit register): lane i + 16g scales row i over the 32-wide K group [32g, 32g+32).
//  * The matrix core's internal sum of the 128 fp8 products is not exact fp32: on operands
//    spanning the whole e4m3 range it deviates by up to ~1.4e-4 of the sum of |products|.
//  * The 16x16 fp32 result lands as lane l, register r = D[4*(l/16) + r][l % 16].
//  * Swapping the operands (weights first) therefore hands each lane four consecutive
//    output COLUMNS of one output row, so a lane owns 8 contiguous bytes of a bf16 C row
//    (page "aiter PR #6370", "Why it is faster", first bullet).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

// e4m3 operand format code of the f8f6f4 instructions (0 = fp8 e4m3, 1 = bf8 e5m2).
constexpr int kFmtE4M3 = 0;
// ue8m0 exponent byte meaning x1.
constexpr int kScaleOne = 127;

// Unscaled fp8 MFMA: 16x16 += 16x128 * 128x16. The scaled builtin with unit scales folds to
// the plain v_mfma_f32_16x16x128_f8f6f4 opcode.
__device__ __forceinline__ v4f mfma_f8(const v8i& a, const v8i& b, const v4f& c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, kFmtE4M3, kFmtE4M3, 0, 0, 0, 0);
}

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair, round to nearest even: one v_cvt_pk_bf16_f32 (converted as a
// pair; two separate conversions cost a shift and an or besides).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{lo, hi}, v2bf));
}

// Row order of the prepared weight buffer inside each 64-row window: prepared row
// rho = 16j + 4a + r (sub-tile j, output lane group a, register r of the swap-AB result) holds
// weight row 32*(j/2) + 8a + 4*(j%2) + r. With this order the result registers of sub-tiles
// j and j+1 (j even) in lane group a are output columns 32*(j/2) + 8a .. +7 of the window.
__host__ __device__ __forceinline__ int weight_row_perm(int rho)
{
    const int j = rho >> 4, a = (rho >> 2) & 3, r = rho & 3;
    return 32 * (j >> 1) + 8 * a + 4 * (j & 1) + r;
}

}  // namespace fp8bs
