/*
 * fp8bs.h -- C ABI of the MI355X (gfx950) fp8 block-scaled GEMM library (libfp8bs.so).
 *
 * Two routes compute C[M,N] (bf16, row-major) from fp8 OCP e4m3 operands A[M,K] (activations)
 * and B[N,K] (weights), both row-major with K contiguous:
 *
 *   route BS  fp8bs_gemm: fp32 block scales, one per 1x128 group of A (a_s[m,kb]) and one
 *             per 128x128 block of B (b_s[nb,kb]):
 *               C[m,n] = bf16( sum_kb a_s[m,kb] * b_s[n/128,kb] * sum_{k in kb} A[m,k]*B[n,k] )
 *             The fp8 products run unscaled on the matrix cores and the fp32 scales are applied
 *             in software to each 128-wide K block's partial sum, never folded into the
 *             hardware's power-of-two scale operands (page "Flydsl Fp8 Blockscale Gemm",
 *             Mechanism A; Procedure step 3).
 *
 *   route MX  fp8mx_gemm: ue8m0 (power-of-two) scales, one per 1x32 group along K for each
 *             row of A and of B, applied by the scaled matrix-core instruction:
 *               C[m,n] = bf16( sum_g 2^(ea[m,g]-127) * 2^(eb[n,g]-127) * sum_{k in g} A[m,k]*B[n,k] )
 *             (page "aiter PR #6370", "Why it is faster").
 *
 *   route PT  fp8pt_gemm: the promote-free twin of route BS, one fp32 scale per row of A and per
 *             row of B (per token / per output channel):
 *               C[m,n] = bf16( a_s[m] * b_s[n] * sum_k A[m,k]*B[n,k] )
 *             The same matrix-core work as route BS with the scales applied once, in the
 *             epilogue: the instrument that separates the cost of the per-block promote from
 *             the rest of the kernel (page "Flydsl Fp8 Blockscale Gemm", Bottleneck diagnosis,
 *             item 2; page "aiter PR #6370" calls such a kernel "ptpc").
 *
 * Conventions shared by every entry point:
 *   - Pointers are device pointers unless stated otherwise; the caller owns every buffer.
 *     No call allocates, frees or keeps per-call state (fp8bs_gemm_splitk_noalloc uses a fixed
 *     static device array instead of a workspace).
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream). No call synchronises
 *     the host, so calls may be captured into a HIP graph.
 *   - Every call returns an fp8bs_status. Pointer, shape and alignment checks run on the host
 *     before anything is launched; on failure nothing is enqueued and outputs are untouched.
 *     A failure of the call's own kernel launch is reported as FP8BS_E_HIP (an error that
 *     earlier work left pending in the HIP runtime is neither reported nor cleared). No call
 *     aborts or throws.
 *   - Shapes that break a constraint are rejected, never padded (page "aiter PR #6370",
 *     Constraints).
 */
#ifndef FP8BS_H
#define FP8BS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FP8BS_OK = 0,
    FP8BS_E_NULL = 1,    /* a required pointer is NULL                                  */
    FP8BS_E_SHAPE = 2,   /* M, N or K violates the route's constraints                   */
    FP8BS_E_ALIGN = 3,   /* a pointer is not 16-byte aligned                             */
    FP8BS_E_CONFIG = 4,  /* an explicit kernel configuration is invalid for the shape    */
    FP8BS_E_HIP = 5,     /* the HIP runtime reported an error when enqueueing the work   */
    FP8BS_E_WORKSPACE = 6 /* a workspace is missing, misaligned or too small             */
} fp8bs_status;

/* Version of this ABI (major * 10000 + minor * 100 + patch). 1.2.0 added the c_store field
 * at the end of fp8bs_config (the struct grew by 4 bytes). */
int fp8bs_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char *fp8bs_strerror(int status);

/* ------------------------------------------------------------------------------------------
 * Weight preparation (one-time, untimed; page "Flydsl Fp8 Blockscale Gemm", Procedure steps
 * 2 and 6: weights are laid out once at set-up and the buffers reused every call).
 * ------------------------------------------------------------------------------------------ */

/* Bytes of the prepared weight buffer for an N x K e4m3 weight (same for both routes); 0 when
 * N or K is not positive. fp8bs_prep_bytes is the same function under a shorter name. */
size_t fp8bs_prep_weight_bytes(int N, int K);
size_t fp8bs_prep_bytes(int N, int K);

/* Lay out B [N,K] (e4m3, row-major) into B_prep, the opaque layout that fp8bs_gemm and
 * fp8mx_gemm consume. B_prep must hold fp8bs_prep_weight_bytes(N, K) bytes and must not
 * overlap B. Constraints: N % 64 == 0, K % 128 == 0, K >= 128; B and B_prep 16-byte aligned. */
int fp8bs_prep_weights(const void *B, void *B_prep, int N, int K, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Activation quantisers (the step before the GEMM: page "Flydsl Fp8 Blockscale Gemm",
 * Procedure step 6; page "aiter PR #6370", Integration). x is [M, K] row-major, bf16 or fp32.
 * e4m3 codes are the nearest value, ties to the even mantissa, saturating at +-448; a NaN
 * element encodes as NaN and is left out of its group's amax. Memory-bound, one pass.
 * ------------------------------------------------------------------------------------------ */

enum { FP8BS_IN_F32 = 0, FP8BS_IN_BF16 = 1 };

/* Route BS activations: per 1x128 group of a row, scale = amax / 448 (fp32; 1 for an all-zero
 * group), codes = e4m3(x / scale) with the division correctly rounded in fp32.
 *   A_codes [M, K] e4m3 (the A operand of fp8bs_gemm); a_scale [K/128, M] fp32, K-block-major
 *   (the a_scale operand of fp8bs_gemm).
 * Constraints: M >= 0, K % 128 == 0, K >= 128; x and A_codes 16-byte aligned, a_scale 4-byte
 * aligned; x_dtype is FP8BS_IN_F32 or FP8BS_IN_BF16 (else FP8BS_E_CONFIG). */
int fp8bs_quantize_act(const void *x, int x_dtype, void *A_codes, float *a_scale, int M, int K,
                       hipStream_t stream);

/* Route MX activations: per 1x32 group, the smallest integer e with amax <= 448 * 2^e
 * (clamped to [-127, 127]; 0 for an all-zero group), stored as the ue8m0 byte e + 127;
 * codes = e4m3(x * 2^-e).
 *   A_codes [M, K] e4m3; a_e8m0 [M, K/32] bytes, row-major (pack it with fp8mx_pack_a_scale).
 * Constraints: M >= 0, K % 32 == 0, K >= 32; x and A_codes 16-byte aligned. */
int fp8mx_quantize_act(const void *x, int x_dtype, void *A_codes, void *a_e8m0, int M, int K,
                       hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Route BS.
 * ------------------------------------------------------------------------------------------ */

/* C[M,N] = blockscaled(A, B).
 *   A        [M, K] e4m3, row-major (lda = K).
 *   a_scale  [K/128, M] fp32, K-block-major: a_scale[kb*M + m] scales A[m, 128kb : 128kb+128]
 *            (page "Flydsl Fp8 Blockscale Gemm", Procedure step 6: the activation scale is fed
 *            transposed, K block outermost).
 *   B_prep   the output of fp8bs_prep_weights for B [N, K].
 *   b_scale  [N/128, K/128] fp32, row-major: b_scale[nb*(K/128) + kb] scales B[128nb : 128nb+128,
 *            128kb : 128kb+128].
 *   C        [M, N] bf16, row-major (ldc = N); every element is written.
 * Constraints: M >= 0 (M == 0 is a no-op), N % 128 == 0, K % 128 == 0, K >= 128, N >= 128;
 * A, B_prep and C 16-byte aligned; a_scale and b_scale 4-byte aligned. Any M is accepted: the
 * last row tile masks its stores. Results are bitwise deterministic run to run. */
int fp8bs_gemm(const void *A, const float *a_scale, const void *B_prep, const float *b_scale,
               void *C, int M, int N, int K, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Route BS with split K: for shapes whose output tiles are too few to occupy the CUs while K
 * is deep (a grid of few workgroups is bound by each tile's K loop: page "Flydsl Fp8 Blockscale
 * Gemm", Bottleneck diagnosis), each tile's 128-wide K blocks are cut into `splits` equal ranges
 * computed by separate workgroups; their fp32 sums go to a caller-provided workspace and a
 * second kernel adds them in range order and rounds once to bf16. The result is deterministic
 * and meets the same bar as fp8bs_gemm; its last bits can differ from fp8bs_gemm's (the fp32
 * sums are grouped by range), and are those of fp8bs_gemm with splits == 1.
 * ------------------------------------------------------------------------------------------ */

/* Workspace bytes fp8bs_gemm_splitk needs: splits x M x N x 4 (0 when it does not split).
 * splits <= 0 asks for the library's choice for the shape (the same choice fp8bs_gemm_splitk
 * makes with splits <= 0). 0 as well for shapes route BS rejects. */
size_t fp8bs_splitk_workspace_bytes(int M, int N, int K, int splits);

/* fp8bs_gemm with K split `splits` ways (splits <= 0: the library's choice; 1: exactly
 * fp8bs_gemm, no workspace used). Operands, layouts and constraints as fp8bs_gemm; in addition
 * (K/128) % splits == 0, splits <= 64, and the shape's tiles must be ones the split kernels
 * have (the warp-specialised tiles the selector takes for grids smaller than the CUs), else
 * FP8BS_E_CONFIG. workspace: device memory of at least fp8bs_splitk_workspace_bytes(M, N, K,
 * splits) bytes, 256-byte aligned, owned by the caller and overwritten; FP8BS_E_WORKSPACE if
 * it is NULL, misaligned or too small (only checked when the call splits). Two kernels are
 * enqueued on `stream`; the workspace must not be used by other work until they finish. */
int fp8bs_gemm_splitk(const void *A, const float *a_scale, const void *B_prep, const float *b_scale,
                      void *C, int M, int N, int K, int splits, void *workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* fp8bs_gemm_splitk without a workspace argument, for callers that cannot allocate (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation). The partial tiles
 * go to the library's own scratch: a static device array of FP8BS_SPLITK_SCRATCH_BYTES on each
 * GPU it runs on, held until the process ends. The call allocates and frees nothing. A call
 * whose partial tiles need more (fp8bs_splitk_workspace_bytes(M, N, K, splits) above the
 * limit) returns FP8BS_E_WORKSPACE and launches nothing. Every call on one GPU shares that
 * array and leaves the last call's partial tiles in it: calls that overlap on one GPU (from
 * different streams or host threads) race, and the caller must order them. Other arguments,
 * constraints and results as fp8bs_gemm_splitk, whose kernels this call runs. */
#define FP8BS_SPLITK_SCRATCH_BYTES ((size_t)32 << 20)
int fp8bs_gemm_splitk_noalloc(const void *A, const float *a_scale, const void *B_prep, const float *b_scale,
                              void *C, int M, int N, int K, int splits, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Route MX.
 * ------------------------------------------------------------------------------------------ */

/* Bytes of a packed ue8m0 scale buffer for `rows` rows and K columns (K/32 scales per row); 0
 * when rows or K is not positive. fp8mx_scale_bytes is the same function under a shorter name. */
size_t fp8mx_packed_scale_bytes(int rows, int K);
size_t fp8mx_scale_bytes(int rows, int K);

/* Pack B's ue8m0 scales b_e8m0 [N, K/32] (uint8, biased by 127, row-major) into the
 * K-block-major, four-to-a-dword layout the scaled instruction consumes (page "aiter PR
 * #6370", "Why it is faster", second bullet), and lay out B as fp8bs_prep_weights does.
 * Constraints: N % 64 == 0, K % 128 == 0, K >= 256. */
int fp8mx_prep_weights(const void *B, const void *b_e8m0, void *B_prep, void *b_scale_packed,
                       int N, int K, hipStream_t stream);

/* Pack A's ue8m0 scales a_e8m0 [M, K/32] into a_scale_packed (fp8mx_packed_scale_bytes(M, K)
 * bytes). Constraints: M % 64 == 0 (the packed group is 64 rows), K % 128 == 0, K >= 256. */
int fp8mx_pack_a_scale(const void *a_e8m0, void *a_scale_packed, int M, int K, hipStream_t stream);

/* C[M,N] = mx(A, B). A [M, K] e4m3 row-major; a_scale_packed from fp8mx_pack_a_scale;
 * B_prep and b_scale_packed from fp8mx_prep_weights; C [M, N] bf16 row-major.
 * Constraints: M % 64 == 0, N % 64 == 0, K % 128 == 0, K >= 256; A, B_prep, C and the packed
 * scales 16-byte aligned. Crossing the two packed scale buffers is not detectable (they have
 * the same size and type) and computes a wrong result rather than failing. */
int fp8mx_gemm(const void *A, const void *a_scale_packed, const void *B_prep,
               const void *b_scale_packed, void *C, int M, int N, int K, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Route PT.
 * ------------------------------------------------------------------------------------------ */

/* C[M,N] = bf16(a_s[m] * b_s[n] * (A B^T)[m,n]).
 *   A        [M, K] e4m3, row-major.
 *   a_scale  [M] fp32: a_scale[m] scales row m of A.
 *   B_prep   the output of fp8bs_prep_weights for B [N, K] (the same buffer route BS uses).
 *   b_scale  [N] fp32: b_scale[n] scales row n of B (output column n).
 *   C        [M, N] bf16, row-major; every element is written.
 * Constraints: M >= 0 (M == 0 is a no-op), N % 64 == 0, N >= 64, K % 128 == 0, K >= 128;
 * A, B_prep, C and b_scale 16-byte aligned, a_scale 4-byte aligned. */
int fp8pt_gemm(const void *A, const float *a_scale, const void *B_prep, const float *b_scale,
               void *C, int M, int N, int K, hipStream_t stream);

/* Route MX through the small-M kernel (meant for few rows, the decode regime; it streams the
 * weights once per 64-row chunk of A, so it also serves M that is not a multiple of 64). The
 * activation exponents are taken row-major, a_e8m0 [M, K/32] bytes (biased by 127; the packed
 * layout of fp8mx_pack_a_scale needs whole 64-row groups); B_prep and b_scale_packed come from
 * fp8mx_prep_weights. Constraints: 0 <= M <= 64 * 65535, N % 64 == 0, K % 128 == 0, K >= 256;
 * A, B_prep, C and b_scale_packed 16-byte aligned. */
int fp8mx_gemm_small_m(const void *A, const void *a_e8m0, const void *B_prep, const void *b_scale_packed,
                       void *C, int M, int N, int K, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Kernel configuration (introspection and ablation). The plain entry points pick a
 * configuration from (M, N, K) alone (page "Flydsl Fp8 Blockscale Gemm", Per-shape recipes:
 * selection by shape, never by layer name); the *_with_config entry points run an explicit one
 * so that tile shapes and the XCD mapping can be measured one against another (same page,
 * Bottleneck diagnosis: ablation is the ground truth).
 * ------------------------------------------------------------------------------------------ */

enum { FP8BS_ROUTE_BS = 0, FP8BS_ROUTE_MX = 1, FP8BS_ROUTE_PT = 2 };

typedef struct {
    int block_m;     /* rows of C per workgroup tile                                           */
    int block_n;     /* columns of C per workgroup tile (N must be a multiple)                 */
    int waves_m;     /* wave grid inside the workgroup: waves_m x waves_n waves of 64 lanes    *
                      * that compute (plus 4 loading waves with schedule 2)                    */
    int waves_n;
    int stages;      /* LDS buffers in the load ring (prefetch depth stages-1 K blocks)        */
    int group_m;     /* tile rows walked together by consecutive tiles (>= 1)                  */
    int xcd_remap;   /* tile order over the 8 XCDs (each has its own L2): 0 round-robin,       *
                      * 1 each XCD a contiguous eighth of all tiles, 2 each XCD a contiguous   *
                      * eighth of every set of tiles resident at the same time                 */
    int persistent;  /* 1: one workgroup per CU slot walks several tiles; 0: one per tile      */
    int pingpong;    /* schedule. 0: every wave loads and computes; 1: the two halves of an    *
                      * 8-wave workgroup alternate, one running its matrix instructions while  *
                      * the other reads its next operands (2 stages); 2: warp-specialised,     *
                      * four extra waves issue every global -> LDS load, the others compute    *
                      * (with 64 x 64 per computing wave, all of a step's operand fragments    *
                      * held in registers and the next step's read as registers free up)      */
    int small_m;     /* non-zero: the small-M kernel (every other field is ignored): one        *
                      * workgroup per 16 output columns and 64-row chunk of A streams the      *
                      * weights, its waves split K (M <= 64 * 65535; route MX with the packed  *
                      * activation scales of its main entry, or fp8mx_gemm_small_m for         *
                      * row-major ones).                                                       *
                      * 1: variant chosen by shape; 2: fragments loaded straight into          *
                      * registers; 3: operands staged through LDS; 4: as 3 with two 16-row     *
                      * weight sub-tiles per workgroup (at most 32 rows per launch chunk, N %  *
                      * 32 == 0). Same results for all up to 48 rows; other values, or 4 where *
                      * it does not apply, are rejected with FP8BS_E_CONFIG                    */
    int c_store;     /* cache policy of the main kernel's C stores (the small-M kernel and the  *
                      * split-K partial sums ignore it). 0: ordinary stores, kept in the       *
                      * XCD's write-back L2 until evicted; 1: written through the L2 at device *
                      * scope; 2: written through and marked non-temporal, so C streams past  *
                      * the caches instead of displacing the operands held there. Same bits   *
                      * for all three; any other value is rejected with FP8BS_E_CONFIG        */
} fp8bs_config;

/* The configuration fp8bs_gemm (route FP8BS_ROUTE_BS), fp8mx_gemm (FP8BS_ROUTE_MX) or
 * fp8pt_gemm (FP8BS_ROUTE_PT) uses for this shape. Host-only and pure; returns FP8BS_E_SHAPE for shapes the route rejects. */
int fp8bs_select_config(int route, int M, int N, int K, fp8bs_config *out);

/* fp8bs_gemm / fp8mx_gemm with an explicit configuration. The (block_m, block_n, waves_m,
 * waves_n, stages, pingpong) tuple must be one the library instantiates and valid for the route, and N
 * must be a multiple of block_n; otherwise FP8BS_E_CONFIG and nothing is launched. Every
 * configuration performs the same per-element arithmetic in the same order, so results are
 * bitwise identical to the plain entry point's. */
int fp8bs_gemm_with_config(const void *A, const float *a_scale, const void *B_prep, const float *b_scale,
                           void *C, int M, int N, int K, const fp8bs_config *config, hipStream_t stream);
int fp8mx_gemm_with_config(const void *A, const void *a_scale_packed, const void *B_prep,
                           const void *b_scale_packed, void *C, int M, int N, int K,
                           const fp8bs_config *config, hipStream_t stream);
int fp8pt_gemm_with_config(const void *A, const float *a_scale, const void *B_prep, const float *b_scale,
                           void *C, int M, int N, int K, const fp8bs_config *config, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Diagnostic (not part of the GEMM): the matrix core's sustained fp8 rate on the caller's own
 * operand bytes, with no memory traffic in the timed loop. On gfx950 the matrix-core rate
 * depends on how much the operand bits change between instructions, so this is the ceiling
 * the GEMM can reach on this data (page "Flydsl Fp8 Blockscale Gemm", Bottleneck diagnosis:
 * an identical-MFMA-work instrument). One workgroup of 8 waves per CU; each wave runs
 * iters x 16 instructions on fragments read from A [M,K] and B_prep (fp8bs_prep_weights).
 * sink: device buffer of sink_len floats (>= 8 per workgroup launched; at most one
 * workgroup per CU is launched and fewer if sink_len is short); flops (host, may be NULL)
 * receives the FLOP count of the launch. Time it with events on `stream`. */
int fp8bs_mfma_ceiling(const void *A, const void *B_prep, int M, int N, int K, int iters, float *sink,
                       int sink_len, long long *flops, hipStream_t stream);

/* Diagnostic (not part of the GEMM): a skeleton of the GEMM mainloop with its parts switched on
 * one at a time, to measure what each costs the matrix core (page "Flydsl Fp8 Blockscale Gemm",
 * Bottleneck diagnosis: identical matrix work, phases added one by one). One workgroup per CU,
 * eight computing waves, `steps` steps of (TM/16) x 4 instructions of 16x16x128 per wave on
 * operand bytes taken from A [M,K] and B_prep. parts, a mask:
 *   1 (FP8BS_LP_READS)   every step reads the wave's operand fragments from LDS (the GEMM's
 *                        swizzled 16-byte reads), else the operands stay in registers;
 *   2 (FP8BS_LP_LOADS)   48 KB per step (64 KB with FP8BS_LP_BIG) of A's bytes go global -> LDS
 *                        (buffer_load ... lds) by four extra loader waves (by the computing waves
 *                        with FP8BS_LP_BIG), with one workgroup barrier per step;
 *   4 (FP8BS_LP_PROMOTE) route BS's promote after each instruction;
 *   8 (FP8BS_LP_STORES)  every 6 steps each computing wave stores its TM x 64 block (2 bytes an
 *                        element) to `out`;
 *  16 (FP8BS_LP_BIG)     TM = 128 instead of 64.
 * Instantiated masks: 0, 1, 3, 5, 7, 15, 17, 19, 23, 31; others return FP8BS_E_CONFIG. The
 * results are meaningless; only the launch time is (time it with events on `stream`).
 * Needs M*K >= 64 KB and N*K >= 32 KB; out: fp8bs_loop_probe_out_bytes(parts) bytes or more
 * (rotated over whole slots of that size), 16-byte aligned, NULL allowed when that is 0;
 * sink: >= 8 floats per CU; flops (may be NULL) receives the launch's matrix FLOP count.
 * FP8BS_E_WORKSPACE if out or sink is short. */
#define FP8BS_LP_READS 1
#define FP8BS_LP_LOADS 2
#define FP8BS_LP_PROMOTE 4
#define FP8BS_LP_STORES 8
#define FP8BS_LP_BIG 16
size_t fp8bs_loop_probe_out_bytes(int parts);
int fp8bs_loop_probe(int parts, const void *A, const void *B_prep, int M, int N, int K, int steps, void *out,
                     size_t out_bytes, float *sink, int sink_len, long long *flops, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8BS_H */
