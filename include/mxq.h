/*
 * mxq.h -- C ABI of libmxq.so: single-pass block-scaled (MX) quantization
 * on AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages):
 *   [MXFP8] pytorch/ao PR #4995, "[moe_training] Fused dual-axis MXFP8
 *           quantization with correct metadata".
 *   [MX9]   AMD-AGI/ALTO PR #33, "feat: mx9: add fused MX9 quantization
 *           kernel with pack/unpack".
 *   [GG]    AMD-AGI/ALTO PR #31, "Add MXFP8 grouped GEMM (E4M3) for
 *           routed-expert MoE training".
 *
 * Conventions shared by every entry point
 *   - Pointers named x, q*, s*, offs, err, y, max_exp and prime are DEVICE
 *     pointers.  The caller allocates and owns every buffer; the library
 *     allocates nothing, keeps no state between calls and never waits on the
 *     device.
 *   - stream is a hipStream_t passed as void*; NULL means the default stream.
 *     All work is enqueued on that stream only, so a call may be captured in a
 *     HIP graph.
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     nonzero return (an mx_status) therefore means nothing was launched and
 *     no output byte was written; MX_E_LAUNCH reports a failed launch.
 *   - Buffers of an empty call (a zero dimension) may be NULL.
 *   - Byte intervals of all buffers passed to one call must be pairwise
 *     disjoint (MX_E_OVERLAP).  Sizes are in elements unless stated.
 *   - Calls on different streams that share an output buffer race.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mx_status {
    MX_OK = 0,
    MX_E_NULL = 1,      /* a required pointer is NULL                        */
    MX_E_DTYPE = 2,     /* unsupported element type (fp16 and others)        */
    MX_E_BLOCK = 3,     /* block_size is not the format's (32 MXFP8, 16 MX9)  */
    MX_E_MODE = 4,      /* scaling_mode other than RCEIL                     */
    MX_E_SHAPE = 5,     /* dimensions negative, too large, or not multiples   */
    MX_E_STRIDE = 6,    /* row pitch smaller than the row or misaligned       */
    MX_E_ALIGN = 7,     /* pointer alignment                                  */
    MX_E_OVERLAP = 8,   /* two buffers of one call overlap                    */
    MX_E_LAUNCH = 9     /* the HIP launch failed                              */
} mx_status;

enum { MX_DTYPE_F32 = 0, MX_DTYPE_BF16 = 1 };
enum { MX_SCALE_RCEIL = 0 };

/* Codes the grouped cast writes to *err (device side). */
enum { MX_OFFS_OK = 0, MX_OFFS_ORDER = 1, MX_OFFS_ALIGN = 2, MX_OFFS_BOUNDS = 3 };

/*
 * mx_quantize_2d_dual -- fused dual-axis MXFP8 cast ([MXFP8], PR
 * description: one read of the bf16 input, four outputs; the
 * "Bug-compatible" list and the NaN paragraph fix the special values).
 *
 *   x      bf16 bit patterns, [M, N] row-major with row pitch ld_x elements.
 *   q_row  uint8 E4M3FN codes [M, N] (pitch N): rowwise 1x32 blocks.
 *   s_row  uint8 E8M0 scales  [M, N/32] (pitch N/32).
 *   q_col  uint8 E4M3FN codes [N, M] (pitch M): colwise 32x1 blocks, stored
 *          transposed, so q_col[n][m] encodes x[m][n].
 *   s_col  uint8 E8M0 scales  [M/32, N] (pitch N).
 *   block_size must be 32, scaling_mode MX_SCALE_RCEIL.
 *
 * Per block: RCEIL scale byte b (smallest power of two that brings the block
 * maximum to <= 448, byte 0 for an all-zero block); element = E4M3FN of
 * x * 2^(127-b), nearest-even.  NaN in a block: scale 255, every code 0x7F,
 * on both axes.  Inf (no NaN): rowwise scale 255 with 0x7F codes; colwise
 * scale 254 with +-Inf -> +-448 and the other elements scaled by 2^-127.
 *
 * Errors: MX_E_NULL (a pointer NULL while M, N > 0), MX_E_BLOCK, MX_E_MODE,
 * MX_E_SHAPE (M or N negative, not a multiple of 128, or above 2^24, or
 * more than 2^23 128x128 tiles: each tile is one workgroup of 512 threads),
 * MX_E_STRIDE (ld_x < N, not a multiple of 8, or above 2^24), MX_E_ALIGN
 * (any pointer not 16-byte aligned), MX_E_OVERLAP.  M == 0 or N == 0 is a
 * no-op.  The call enqueues one kernel on the stream.
 */
int mx_quantize_2d_dual(const uint16_t *x, int64_t M, int64_t N, int64_t ld_x,
                        int32_t block_size, int32_t scaling_mode,
                        uint8_t *q_row, uint8_t *s_row,
                        uint8_t *q_col, uint8_t *s_col, void *stream);

/*
 * mx_quantize_grouped -- the dual-axis cast of a MoE activation buffer
 * whose rows are split into G groups by cumulative ends offs[0..G-1]
 * ([MXFP8], PR description, "Uncovered tail" paragraph; review reply on
 * offset validation).
 *
 * Outputs are exactly those of mx_quantize_2d_dual on the whole buffer,
 * except that s_col rows i >= offs[G-1]/32 (the uncovered tail) are zero.
 * Tail rows are still quantized on both axes; empty groups change nothing.
 * G == 0 is the dense cast (offs may then be NULL).
 *
 *   offs  int32 device array [G]; valid when 0 <= offs[0] <= ... <=
 *         offs[G-1] <= M and every entry is a multiple of 128.
 *   err   int32 device word or NULL.  When non-NULL the call writes
 *         MX_OFFS_OK, or the code of the first invalid entry (bounds are
 *         checked before alignment, alignment before order).  With invalid
 *         offsets the outputs are unspecified, but nothing outside the four
 *         output buffers and *err is written.
 *
 * Host-side errors as for mx_quantize_2d_dual, plus MX_E_SHAPE for G < 0
 * and MX_E_NULL for G > 0 with offs == NULL; offs and err take part in the
 * overlap check.
 */
int mx_quantize_grouped(const uint16_t *x, int64_t M, int64_t N, int64_t ld_x,
                        int32_t block_size, int32_t scaling_mode,
                        const int32_t *offs, int32_t G,
                        uint8_t *q_row, uint8_t *s_row,
                        uint8_t *q_col, uint8_t *s_col,
                        int32_t *err, void *stream);

/*
 * Matrix-core scale layout.  The _mfma variants below write (casts) or read
 * (contractions) E8M0 scales in the order in which the gfx950 scaled matrix
 * instruction (16x16x128, E4M3 operands) takes them, so that a consumer
 * loads one dword per lane per 128-wide step and no rearrangement runs
 * between the cast and the contraction ([MXFP8], PR description: the kernel
 * emits the consumer's swizzled scale layout directly).  For an operand of R
 * rows (R a multiple of 64) and K/32 blocks per row (K a multiple of 128),
 * scale (r, b) is the byte
 *
 *     ((r/64 * K/128 + b/4) * 64 + 16 * (b%4) + r%16) * 4 + (r%64)/16
 *
 * of an R * K/32 byte buffer: each 64-row group and 4-block step owns 256
 * contiguous bytes, dword L of which holds, in byte q, the scale of row
 * 64 (r/64) + 16 q + L%16 for block 4 (b/4) + L/16.
 */

/*
 * mx_quantize_2d_dual_mfma -- mx_quantize_2d_dual with both scale tensors in
 * the matrix-core layout: s_row as the operand [M rows, N/32 blocks] (the
 * scales of q_row), s_col as the operand [N rows, M/32 blocks] (the scales
 * of q_col, whose rows are the input's columns).  Byte for byte the same
 * scale values as mx_quantize_2d_dual, permuted; q_row and q_col identical.
 * Arguments and errors as for mx_quantize_2d_dual.  One kernel.
 */
int mx_quantize_2d_dual_mfma(const uint16_t *x, int64_t M, int64_t N, int64_t ld_x,
                             int32_t block_size, int32_t scaling_mode,
                             uint8_t *q_row, uint8_t *s_row,
                             uint8_t *q_col, uint8_t *s_col, void *stream);

/*
 * mx_quantize_grouped_mfma -- mx_quantize_grouped with the scales of
 * mx_quantize_2d_dual_mfma; the zeroed tail is the same set of s_col bytes
 * (blocks b >= offs[G-1]/32 of every row of the [N, M/32] operand).
 * Arguments and errors as for mx_quantize_grouped.
 */
int mx_quantize_grouped_mfma(const uint16_t *x, int64_t M, int64_t N, int64_t ld_x,
                             int32_t block_size, int32_t scaling_mode,
                             const int32_t *offs, int32_t G,
                             uint8_t *q_row, uint8_t *s_row,
                             uint8_t *q_col, uint8_t *s_col,
                             int32_t *err, void *stream);

/*
 * mx9_pack -- MX9 pack along the last axis, block 16 ([MX9], Summary and
 * Key design choices).
 *
 *   x        fp32 (dtype MX_DTYPE_F32) or bf16 (MX_DTYPE_BF16) bit patterns,
 *            [rows, cols] row-major, row pitch ld_x elements.
 *   q        int8 [nb, 16], nb = rows * ceil(cols/16), blocks numbered
 *            row-major over (row, block within the row).
 *   max_exp  uint8 [nb]: shared exponent as E8M0 (true exponent + 127), the
 *            true exponent taken from the input's own exponent field and
 *            raised to at least -126, so the byte is in [1, 254] for
 *            finite input.
 *   prime    uint8 [nb]: bit j (LSB first) set when pair j (elements 2j,
 *            2j+1) lies wholly below 2^E and is quantized on the finer grid.
 *   q = round-half-even(x / 2^(E - 6 - p)) clamped to [-127, 127].  A block
 *   holding Inf or NaN gets max_exp 255, q 0 and prime 0.  A trailing
 *   partial block is padded with +0.
 *
 * Errors: MX_E_NULL, MX_E_DTYPE (dtype not F32/BF16), MX_E_BLOCK
 * (block_size != 16), MX_E_SHAPE (negative or too large), MX_E_STRIDE
 * (ld_x < cols, or x spanning more than 2^48 bytes), MX_E_ALIGN (x not
 * aligned to its element size, q not
 * 16-byte aligned), MX_E_OVERLAP.  rows == 0 or cols == 0 is a no-op.
 */
int mx9_pack(const void *x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld_x,
             int32_t block_size, int8_t *q, uint8_t *max_exp, uint8_t *prime,
             void *stream);

/*
 * mx9_unpack -- inverse of mx9_pack ([MX9], convert_from_mx9; the caller
 * passes the shape back because it is not stored).
 *
 *   y = q * 2^(max_exp - 127 - 6 - p) for max_exp != 255, written as fp32
 *   (out_dtype MX_DTYPE_F32; exact, IEEE overflow to Inf for the one
 *   combination q = -128, max_exp = 254, p = 0 that pack never emits) or
 *   bf16 (MX_DTYPE_BF16; nearest-even, exact for everything pack emits).
 *   max_exp == 255 gives the quiet NaN 0x7FC00000 / 0x7FC0.
 *   y is [rows, cols] with row pitch ld_y elements; only the first cols
 *   columns of each row are written.
 *
 * Errors: MX_E_NULL, MX_E_DTYPE, MX_E_BLOCK, MX_E_SHAPE, MX_E_STRIDE
 * (ld_y < cols, or y spanning more than 2^48 bytes), MX_E_ALIGN (q not
 * 16-byte aligned, y not aligned to its
 * element size), MX_E_OVERLAP.  rows == 0 or cols == 0 is a no-op.
 */
int mx9_unpack(const int8_t *q, const uint8_t *max_exp, const uint8_t *prime,
               int64_t rows, int64_t cols, int32_t block_size, int32_t out_dtype,
               void *y, int64_t ld_y, void *stream);

/*
 * mx9_pack_strided -- mx9_pack writing each of its three outputs at a row
 * pitch of the caller's choice ([MX9], review comments on the output offsets,
 * which ask why the output tensors take no strides).  Same blocks, same
 * bytes as mx9_pack; only where row r's bytes go changes:
 *
 *   q        block j of row r at q + r * ld_q + 16 j   (ld_q in bytes, a
 *            multiple of 16 and >= 16 * ceil(cols/16)),
 *   max_exp  at max_exp + r * ld_e + j                 (ld_e >= ceil(cols/16)),
 *   prime    at prime + r * ld_pr + j                  (ld_pr >= ceil(cols/16)).
 *
 * Bytes between the rows' used ranges are not written.  mx9_pack is this call
 * with ld_q = 16 * ceil(cols/16) and ld_e = ld_pr = ceil(cols/16).
 * Errors as for mx9_pack, plus MX_E_STRIDE for a pitch below its row or an ld_q
 * that is not a multiple of 16; the byte ranges spanned by the three pitched
 * outputs take part in the overlap check.
 */
int mx9_pack_strided(const void *x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld_x,
                     int32_t block_size, int8_t *q, int64_t ld_q, uint8_t *max_exp, int64_t ld_e,
                     uint8_t *prime, int64_t ld_pr, void *stream);

/*
 * mx9_unpack_strided -- mx9_unpack reading q, max_exp and prime at the row
 * pitches of mx9_pack_strided.  Errors as for mx9_unpack, plus the pitch
 * checks of mx9_pack_strided.
 */
int mx9_unpack_strided(const int8_t *q, int64_t ld_q, const uint8_t *max_exp, int64_t ld_e,
                       const uint8_t *prime, int64_t ld_pr, int64_t rows, int64_t cols,
                       int32_t block_size, int32_t out_dtype, void *y, int64_t ld_y, void *stream);

/*
 * mx9_pack_axis -- MX9 pack in blocks of 16 along any axis ([MX9], the
 * calls' axis argument; the shape and the axis are not stored, so the caller
 * passes them back to the unpack).
 *
 *   x        contiguous fp32 or bf16 array viewed as [outer, len, inner]: the
 *            blocked axis has len elements, outer is the product of the
 *            dimensions before it and inner of those after it (inner == 1 is
 *            the last axis, identical to mx9_pack with rows = outer).
 *   Reading (the page does not print the block order): the axis is moved
 *   last before blocking, so block (o, i, j) holds x[o][16j .. 16j+15][i],
 *   padded with +0 past len, and is numbered (o * inner + i) * nbl + j,
 *   nbl = ceil(len / 16).
 *   q, max_exp, prime  as for mx9_pack, nb = outer * inner * nbl blocks.
 *
 * Errors: MX_E_NULL, MX_E_DTYPE, MX_E_BLOCK (block_size != 16), MX_E_SHAPE
 * (a negative or too large dimension, more than 2^32 blocks, or, for
 * inner > 1, a view whose tiles -- one workgroup of up to 512 threads per
 * tile of 64 or 128 inner positions -- need a grid beyond 2^32 threads),
 * MX_E_ALIGN (x not aligned to its element size, q not 16-byte aligned),
 * MX_E_OVERLAP.  A zero dimension is a no-op.
 */
int mx9_pack_axis(const void *x, int32_t dtype, int64_t outer, int64_t len, int64_t inner,
                  int32_t block_size, int8_t *q, uint8_t *max_exp, uint8_t *prime, void *stream);

/*
 * mx9_unpack_axis -- inverse of mx9_pack_axis: y (contiguous [outer, len,
 * inner], fp32 or bf16 by out_dtype) gets every element, computed as in
 * mx9_unpack.  Errors as for mx9_unpack, with the shape checks of
 * mx9_pack_axis.
 */
int mx9_unpack_axis(const int8_t *q, const uint8_t *max_exp, const uint8_t *prime, int64_t outer,
                    int64_t len, int64_t inner, int32_t block_size, int32_t out_dtype, void *y,
                    void *stream);

/*
 * mx9_pack_records -- MX9 in one byte tensor ([MX9], commit "refactor: mx:
 * pack mx9 into a single uint8 tensor", which stores the exponent byte at
 * the start of each block's record).
 *
 *   x       as for mx9_pack_axis (blocks along the middle axis of [outer,
 *           len, inner]; inner == 1 is the last axis).
 *   packed  uint8, outer * inner rows of nbl records at a pitch of ld_p
 *           bytes (ld_p >= 18 * nbl); row o * inner + i holds the blocks
 *           (o, i, 0 .. nbl-1).  A record is 18 bytes: the exponent byte,
 *           q[0..15], the prime byte (reading: the page fixes only the
 *           exponent byte's place).  Bytes past 18 * nbl in a row are not
 *           written.  9 bits per element.
 *
 * Errors: MX_E_NULL, MX_E_DTYPE, MX_E_BLOCK, MX_E_SHAPE, MX_E_STRIDE
 * (ld_p < 18 * nbl or above 2^40, or the records spanning more than 2^48
 * bytes), MX_E_ALIGN (x not aligned to its element
 * size), MX_E_OVERLAP.  A zero dimension is a no-op.  Contiguous records of
 * a last-axis pack whose len is a multiple of 16, with x and packed 16-byte
 * aligned, take the fastest path.
 */
int mx9_pack_records(const void *x, int32_t dtype, int64_t outer, int64_t len, int64_t inner,
                     int32_t block_size, uint8_t *packed, int64_t ld_p, void *stream);

/*
 * mx9_unpack_records -- inverse of mx9_pack_records into a contiguous
 * [outer, len, inner] y of out_dtype (fp32 or bf16), computed as in
 * mx9_unpack.  Errors: MX_E_NULL, MX_E_DTYPE, MX_E_BLOCK, MX_E_SHAPE,
 * MX_E_STRIDE (as for mx9_pack_records), MX_E_ALIGN (y not aligned to its
 * element size), MX_E_OVERLAP.
 */
int mx9_unpack_records(const uint8_t *packed, int64_t ld_p, int64_t outer, int64_t len, int64_t inner,
                       int32_t block_size, int32_t out_dtype, void *y, void *stream);

/*
 * mx_gemm_nt -- MXFP8 block-scaled contraction, the consumer of the
 * dual-axis cast's outputs ([GG], description: E4M3 operands with E8M0
 * scales per 32 elements of the contraction).
 *
 *   C[m][n] = sum_k e4m3(A[m][k]) 2^(sA(m, k/32) - 127) e4m3(B[n][k]) 2^(sB(n, k/32) - 127)
 *
 *   A      E4M3 codes [M, K], contraction contiguous, row pitch lda bytes
 *          (q_row of the cast, or q_col for a contraction over tokens).
 *   sA     E8M0 bytes, sA(m, b) = sA[m * sa_rs + b * sa_bs]: (K/32, 1) for the
 *          cast's s_row, (1, M) for its s_col read as the scales of q_col.
 *   B, sB  the same for the second operand, [N, K] with pitch ldb.
 *   C      [M, N], fp32 (out_dtype MX_DTYPE_F32) or bf16 (MX_DTYPE_BF16,
 *          nearest-even), row pitch ldc elements; computed on the matrix
 *          cores with fp32 accumulation (summation order unspecified).
 *   M, N, K multiples of 128 (at most 2^24); lda, ldb multiples of 16.
 *
 * Any scale strides are accepted.  The fast (pipelined) kernel runs when
 * both operands' scales have block stride 1 and a row stride that is a
 * multiple of 4, or both have row stride 1 and a block stride that is a
 * multiple of 4 (the cast's s_row and s_col as above), the scale pointers
 * are 4-byte aligned and C rows are whole 16-byte pieces; other views take
 * a slower general kernel with the same results.  Block-stride-1 scales
 * whose pointers and row strides are multiples of 16 bytes, with K a
 * multiple of 512, load faster (four contraction steps per request) in
 * this call and the row-grouped forward.
 *
 * Errors: MX_E_NULL, MX_E_DTYPE (out_dtype), MX_E_SHAPE (also when a kernel's
 * grid would exceed 2^32 threads), MX_E_STRIDE (a pitch
 * below its row or misaligned, a negative scale stride), MX_E_ALIGN (A or B
 * not 16-byte aligned, C not aligned to its element), MX_E_OVERLAP (C
 * overlaps an input).  M == 0 or N == 0 is a no-op.
 */
int mx_gemm_nt(const uint8_t *A, int64_t lda, const uint8_t *sA, int64_t sa_rs, int64_t sa_bs,
               const uint8_t *B, int64_t ldb, const uint8_t *sB, int64_t sb_rs, int64_t sb_bs,
               int64_t M, int64_t N, int64_t K, void *C, int64_t ldc, int32_t out_dtype, void *stream);

/*
 * mx_grouped_gemm_rows -- the routed-expert forward ([GG]: 1-D cumulative
 * offsets over a padded activation buffer, one weight operand per expert).
 * Rows offs[g-1] <= m < offs[g] of A (offs[-1] = 0) are contracted with
 * expert g's operand B + g * b_gs (codes [N, K], pitch ldb) and its scales
 * sB + g * sb_gs; rows m >= offs[G-1] (the uncovered tail) give 0 (reading:
 * the padding belongs to no expert).  offs (device int32 [G], G >= 1) must
 * satisfy the grouped cast's rule (ascending multiples of 128 within
 * [0, M]); otherwise the rows' expert is unspecified but every access stays
 * inside the operands.  Other arguments and errors as for mx_gemm_nt, plus
 * MX_E_SHAPE for G < 1, MX_E_NULL for offs NULL, MX_E_STRIDE for a negative
 * group stride.  The pipelined kernel also needs sb_gs to be a multiple of 4.
 */
int mx_grouped_gemm_rows(const uint8_t *A, int64_t lda, const uint8_t *sA, int64_t sa_rs, int64_t sa_bs,
                         const uint8_t *B, int64_t ldb, int64_t b_gs, const uint8_t *sB, int64_t sb_rs,
                         int64_t sb_bs, int64_t sb_gs, const int32_t *offs, int32_t G, int64_t M, int64_t N,
                         int64_t K, void *C, int64_t ldc, int32_t out_dtype, void *stream);

/*
 * mx_grouped_gemm_k -- the routed-expert weight gradient: the contraction
 * runs over the token axis, grouped by the same offsets.  Group g writes
 * C + g * c_gs ([M, N], pitch ldc, elements) with the sum over
 * offs[g-1] <= k < offs[g]; an empty group writes 0; k >= offs[G-1] is not
 * read.  A [M, K] and B [N, K] hold the contraction contiguous (the cast's
 * q_col of the two token-major operands), sA and sB their scales (the
 * cast's s_col, as (1, M) and (1, N) strided views).  Invalid offsets are
 * clamped to multiples of 128 inside [0, K]: the results are then
 * unspecified, the accesses stay inside the operands.  Errors as for
 * mx_gemm_nt, plus MX_E_SHAPE (G < 1, or a grid of more than 2^32 threads),
 * MX_E_STRIDE (c_gs smaller than one group's C).
 */
int mx_grouped_gemm_k(const uint8_t *A, int64_t lda, const uint8_t *sA, int64_t sa_rs, int64_t sa_bs,
                      const uint8_t *B, int64_t ldb, const uint8_t *sB, int64_t sb_rs, int64_t sb_bs,
                      const int32_t *offs, int32_t G, int64_t M, int64_t N, int64_t K, void *C, int64_t ldc,
                      int64_t c_gs, int32_t out_dtype, void *stream);

/*
 * mx_gemm_nt_mfma, mx_grouped_gemm_rows_mfma, mx_grouped_gemm_k_mfma -- the
 * three contractions above with sA, sB in the matrix-core scale layout (sA
 * for the operand [M rows, K/32 blocks], sB for [N rows, K/32 blocks]; for
 * the row-grouped form expert g's scales start at sB + g * sb_gs), which the
 * _mfma casts emit: s_row for q_row, s_col for q_col.  The scale pointers
 * must be 16-byte aligned (MX_E_ALIGN).  Results, other arguments and
 * errors as for the strided-view forms.
 */
int mx_gemm_nt_mfma(const uint8_t *A, int64_t lda, const uint8_t *sA, const uint8_t *B, int64_t ldb,
                    const uint8_t *sB, int64_t M, int64_t N, int64_t K, void *C, int64_t ldc,
                    int32_t out_dtype, void *stream);
int mx_grouped_gemm_rows_mfma(const uint8_t *A, int64_t lda, const uint8_t *sA, const uint8_t *B, int64_t ldb,
                              int64_t b_gs, const uint8_t *sB, int64_t sb_gs, const int32_t *offs, int32_t G,
                              int64_t M, int64_t N, int64_t K, void *C, int64_t ldc, int32_t out_dtype,
                              void *stream);
int mx_grouped_gemm_k_mfma(const uint8_t *A, int64_t lda, const uint8_t *sA, const uint8_t *B, int64_t ldb,
                           const uint8_t *sB, const int32_t *offs, int32_t G, int64_t M, int64_t N, int64_t K,
                           void *C, int64_t ldc, int64_t c_gs, int32_t out_dtype, void *stream);

/*
 * mx_scales_to_mfma -- rewrite rows x blocks E8M0 scales given as a strided
 * view (byte (r, b) at s[r * rs + b * bs], rs, bs >= 0) into the matrix-core
 * scale layout described above (out: rows * blocks bytes, 4-byte aligned),
 * so that scales held in a plain layout can feed the _mfma contractions.
 * rows must be a multiple of 64 and blocks of 4.
 * mx_scales_from_mfma -- the inverse: the flat matrix-core buffer `in` is
 * written to the strided view s, whose positions must be distinct (rs, bs
 * >= 1 and rs >= blocks * bs or bs >= rows * rs).
 *
 * Errors: MX_E_NULL, MX_E_SHAPE (negative, not multiples of 64 / 4, or above
 * 2^30), MX_E_STRIDE (a negative or too large stride, or a written view that
 * aliases itself), MX_E_ALIGN (flat buffer not 4-byte aligned),
 * MX_E_OVERLAP.  rows == 0 or blocks == 0 is a no-op.
 */
int mx_scales_to_mfma(const uint8_t *s, int64_t rs, int64_t bs, int64_t rows, int64_t blocks, uint8_t *out,
                      void *stream);
int mx_scales_from_mfma(const uint8_t *in, int64_t rows, int64_t blocks, uint8_t *s, int64_t rs, int64_t bs,
                        void *stream);

/* Host function: a static, human-readable name for an mx_status value. */
const char *mx_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */
