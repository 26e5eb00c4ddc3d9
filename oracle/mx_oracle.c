/*
 * mx_oracle.c -- plain, slow CPU oracle for single-pass MX quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU product path
 * never calls it, links it or shares code with it.
 *
 * Every value is handled as an exact real number in IEEE binary64:
 * bf16 / fp32 / E4M3 values decode exactly into a double, and scaling by a
 * power of two with ldexp() is exact in the ranges used here.  Rounding to
 * E4M3 is a nearest-value search over the format's finite values; the RCEIL
 * exponent is found by comparison against exact powers of two.  There is no
 * bit trick for any step of the method.
 *
 * Sources (web pages):
 *   [MXFP8] pytorch/ao PR #4995, "[moe_training] Fused dual-axis MXFP8
 *           quantization with correct metadata".
 *   [MX9]   AMD-AGI/ALTO PR #33, "feat: mx9: add fused MX9 quantization kernel
 *           with pack/unpack".
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - E4M3 is the OCP E4M3FN variant (max 448, no Inf, NaN = S.1111.111).
 *   - A poisoned MXFP8 block (scale byte 255) holds 0x7F in every byte.
 *   - Colwise Inf block: scale byte 254 and the exact multiplier 2^-127, so
 *     the data stays finite (+-Inf -> +-448).
 *   - A zero block gets scale byte 0.
 *   - Scale layouts are plain row-major: s_row [M][N/32], s_col [M/32][N];
 *     colwise data is transposed: q_col [N][M].
 *   - MX9 pair bit: 1 ("demoted") when the pair's largest magnitude is below
 *     2^E, the block's shared power of two; bit j belongs to pair j, LSB first.
 *   - MX9 non-finite block: max_exp 255, q all 0, prime 0, unpacks to NaN.
 *   - MX9 trailing partial block is padded with +0.
 *   - MX9 along another axis: the axis is moved last (movedim) before
 *     blocking, which fixes the block order.
 *   - MX9 in one byte tensor: 18-byte records, exponent byte, q[16], prime.
 *
 * Parity unpinned (oracle-defined; no passage and no independent source fixes
 * them): the 0x7F byte of poisoned MXFP8 blocks, the row-major s_col layout,
 * the MX9 pair-bit polarity and bit order, the MX9 poison values, the block
 * order for a non-last axis and the place of q and prime inside an MX9
 * record.  Every
 * other result is pinned by the test suite against the pages' constants,
 * hand-derived blocks, torch's float8 codec, closed forms or exact rationals.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number formats, decoded from their field definitions.                     */
/* ------------------------------------------------------------------------ */

/* bfloat16: sign bit 15, 8-bit exponent (bias 127) in bits 14..7, 7-bit
 * fraction in bits 6..0.  Returns the exact value; sets *kind to 0 finite,
 * 1 infinite, 2 NaN. */
static double bf16_decode(uint16_t bits, int *kind)
{
    int sign = (bits >> 15) & 1;
    int e = (bits >> 7) & 0xFF;
    int f = bits & 0x7F;
    double mag;
    if (e == 0xFF) {
        *kind = f ? 2 : 1;
        return f ? NAN : (sign ? -INFINITY : INFINITY);
    }
    *kind = 0;
    if (e == 0)
        mag = ldexp((double)f, -126 - 7);              /* subnormal: 0.f * 2^-126 */
    else
        mag = ldexp((double)(128 + f), e - 127 - 7);    /* normal: 1.f * 2^(e-127) */
    return sign ? -mag : mag;
}

/* IEEE binary32: sign bit 31, 8-bit exponent in bits 30..23, 23-bit fraction. */
static double fp32_decode(uint32_t bits, int *kind)
{
    int sign = (bits >> 31) & 1;
    int e = (bits >> 23) & 0xFF;
    uint32_t f = bits & 0x7FFFFF;
    double mag;
    if (e == 0xFF) {
        *kind = f ? 2 : 1;
        return f ? NAN : (sign ? -INFINITY : INFINITY);
    }
    *kind = 0;
    if (e == 0)
        mag = ldexp((double)f, -126 - 23);
    else
        mag = ldexp((double)((1u << 23) + f), e - 127 - 23);
    return sign ? -mag : mag;
}

/* OCP E4M3FN: sign bit 7, 4-bit exponent (bias 7) in bits 6..3, 3-bit
 * fraction.  Exponent 15 with fraction 7 is NaN; there is no infinity. */
double oref_e4m3_value(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int f = code & 7;
    double mag;
    if (e == 15 && f == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)f, -6 - 3);
    else
        mag = ldexp((double)(8 + f), e - 7 - 3);
    return sign ? -mag : mag;
}

/* Round v to E4M3FN: nearest finite value, ties to the even code; magnitudes
 * beyond the largest finite value (448), infinities included, saturate to it.
 * The sign is copied from v, so -0 and tiny negatives give 0x80.  v must not
 * be NaN. */
uint8_t oref_e4m3_encode(double v)
{
    int sign = signbit(v) ? 1 : 0;
    double a = fabs(v);
    int best = 0;
    double best_err = INFINITY;
    int c;
    if (a > 448.0)
        a = 448.0;
    for (c = 0; c <= 0x7E; c++) {           /* every positive finite code */
        double err = fabs(oref_e4m3_value((uint8_t)c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best_err = err;
            best = c;
        }
    }
    return (uint8_t)((sign << 7) | best);
}

/* ------------------------------------------------------------------------ */
/* MXFP8 (block 32, E4M3 data, E8M0 scale, RCEIL)   [MXFP8]                   */
/* ------------------------------------------------------------------------ */

/* RCEIL scale byte for a finite block maximum A >= 0: the smallest power of
 * two 2^k with A / 2^k <= 448, i.e. k = ceil(log2(A / 448)), clamped to the
 * E8M0 exponent range [-127, 127] and biased by 127.  A zero block gets 0.
 * The comparison A <= 448 * 2^k is exact in binary64.  ([MXFP8], the scale
 * 0/1 cutoff at 448 * 2^-127 given in the review reply.) */
int oref_rceil_byte(double amax)
{
    int k;
    if (amax == 0.0)
        return 0;
    for (k = -300; k <= 300; k++)
        if (amax <= ldexp(448.0, k))
            break;
    if (k < -127) k = -127;
    if (k > 127) k = 127;
    return 127 + k;
}

/* One 32-element block, gathered with a stride (1 for a rowwise block, the
 * row pitch for a colwise block).  colwise selects the colwise rules:
 *   - NaN anywhere: scale 255, every data byte 0x7F, on both axes (the fused
 *     kernel poisons the colwise block; the rowwise cast converts NOSAT).
 *   - Inf, no NaN: rowwise scale 255 and all-NaN data (NOSAT); colwise scale
 *     254 with finite data (SATFINITE).
 *   - otherwise: RCEIL scale byte b; element = E4M3(x * 2^(127 - b)), which
 *     for b = 0 is the 2^127 multiplier of the pages' byte-0 rule.
 * ([MXFP8] PR description: the "Bug-compatible" list and the NaN paragraph.) */
static void mxfp8_block(const uint16_t *x, int64_t stride, int colwise,
                        uint8_t *q, int64_t q_stride, uint8_t *s)
{
    int has_nan = 0, has_inf = 0, i, kind, b;
    double amax = 0.0;
    for (i = 0; i < 32; i++) {
        double v = bf16_decode(x[i * stride], &kind);
        if (kind == 2) has_nan = 1;
        else if (kind == 1) has_inf = 1;
        else if (fabs(v) > amax) amax = fabs(v);
    }
    if (has_nan)
        b = 255;
    else if (has_inf)
        b = colwise ? 254 : 255;
    else
        b = oref_rceil_byte(amax);
    *s = (uint8_t)b;
    for (i = 0; i < 32; i++) {
        if (b == 255) {
            q[i * q_stride] = 0x7F;
        } else {
            double v = bf16_decode(x[i * stride], &kind);
            q[i * q_stride] = oref_e4m3_encode(ldexp(v, 127 - b));
        }
    }
}

/* Rowwise 1x32 cast of bf16 x[M][N] (row pitch ld_x elements):
 * q_row[m][n] (pitch N) and s_row[m][j] (pitch N/32).  N % 32 == 0. */
void oref_mxfp8_rowwise(const uint16_t *x, int64_t M, int64_t N, int64_t ld_x,
                        uint8_t *q_row, uint8_t *s_row)
{
    int64_t m, j;
    for (m = 0; m < M; m++)
        for (j = 0; j < N / 32; j++)
            mxfp8_block(x + m * ld_x + 32 * j, 1, 0,
                        q_row + m * N + 32 * j, 1, s_row + m * (N / 32) + j);
}

/* Colwise 32x1 cast: block (i, n) holds x[32i .. 32i+31][n].  Data is stored
 * transposed, q_col[n][m] (pitch M); scales s_col[i][n] (pitch N).
 * M % 32 == 0. */
void oref_mxfp8_colwise(const uint16_t *x, int64_t M, int64_t N, int64_t ld_x,
                        uint8_t *q_col, uint8_t *s_col)
{
    int64_t i, n;
    for (i = 0; i < M / 32; i++)
        for (n = 0; n < N; n++)
            mxfp8_block(x + 32 * i * ld_x + n, ld_x, 1,
                        q_col + n * M + 32 * i, 1, s_col + i * N + n);
}

/* The fused dual-axis cast: all four outputs of one bf16 matrix. */
void oref_mxfp8_dual(const uint16_t *x, int64_t M, int64_t N, int64_t ld_x,
                     uint8_t *q_row, uint8_t *s_row, uint8_t *q_col, uint8_t *s_col)
{
    oref_mxfp8_rowwise(x, M, N, ld_x, q_row, s_row);
    oref_mxfp8_colwise(x, M, N, ld_x, q_col, s_col);
}

/* Validity of cumulative group ends offs[0..G-1] for an M-row buffer:
 * 0 valid; 1 not ascending; 2 not a multiple of 128; 3 outside [0, M].
 * The first failing group decides; within a group, bounds are checked
 * first, then alignment, then order.  ([MXFP8] review reply: validation of
 * ascending, in-bounds offsets; PR description: every group size a multiple
 * of 128.) */
int oref_offs_check(const int32_t *offs, int32_t G, int64_t M)
{
    int32_t g;
    for (g = 0; g < G; g++) {
        if (offs[g] < 0 || offs[g] > M) return 3;
        if (offs[g] % 128 != 0) return 2;
        if (g > 0 && offs[g] < offs[g - 1]) return 1;
    }
    return 0;
}

/* Grouped cast: identical to the dense cast except that the colwise scale
 * bytes of the uncovered tail, rows at or past offs[G-1], are zero.  Tail
 * rows are still quantized on both axes.  Empty groups change nothing.
 * Returns the oref_offs_check code; outputs are only written when it is 0.
 * ([MXFP8] PR description, "Uncovered tail" paragraph.) */
int oref_mxfp8_grouped(const uint16_t *x, int64_t M, int64_t N, int64_t ld_x,
                       const int32_t *offs, int32_t G,
                       uint8_t *q_row, uint8_t *s_row, uint8_t *q_col, uint8_t *s_col)
{
    int rc = oref_offs_check(offs, G, M);
    int64_t covered, i, n;
    if (rc != 0)
        return rc;
    oref_mxfp8_dual(x, M, N, ld_x, q_row, s_row, q_col, s_col);
    covered = G > 0 ? offs[G - 1] : M;
    for (i = covered / 32; i < M / 32; i++)
        for (n = 0; n < N; n++)
            s_col[i * N + n] = 0;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* MX9 pack / unpack (block 16)   [MX9]                                       */
/* ------------------------------------------------------------------------ */

/* Pack one block of 16 elements.  val[i] are exact values, ef[i] the biased
 * exponent fields read from the input's own dtype bits, kind[i] as above.
 * Steps, in the order the MX9 page gives them:
 *   1. the shared exponent is the largest exponent field, raised to at least
 *      1 (true exponent clamped at -126, the fp32-normal minimum), stored
 *      as an E8M0 byte (true exponent + 127);
 *   2. a pair whose larger magnitude is below 2^E is demoted one step onto
 *      the finer grid 2^(E-7) and its prime bit set;
 *   3. q = round-half-even(x / 2^(E - 6 - p)), clamped symmetrically to
 *      [-127, 127].
 * A non-finite element poisons the block: max_exp 255, q all 0, prime 0. */
static void mx9_block(const double *val, const int *ef, const int *kind,
                      int8_t *q, uint8_t *max_exp, uint8_t *prime)
{
    int i, j, S = 0, E, poison = 0;
    unsigned bits = 0;
    for (i = 0; i < 16; i++) {
        if (kind[i] != 0) poison = 1;
        if (ef[i] > S) S = ef[i];
    }
    if (poison) {
        for (i = 0; i < 16; i++) q[i] = 0;
        *max_exp = 255;
        *prime = 0;
        return;
    }
    if (S < 1) S = 1;
    E = S - 127;
    for (j = 0; j < 8; j++) {
        double pm = fmax(fabs(val[2 * j]), fabs(val[2 * j + 1]));
        int p = pm < ldexp(1.0, E);
        if (p) bits |= 1u << j;
        for (i = 2 * j; i < 2 * j + 2; i++) {
            double r = rint(ldexp(val[i], 6 + p - E));   /* half to even */
            if (r > 127.0) r = 127.0;
            if (r < -127.0) r = -127.0;
            q[i] = (int8_t)r;
        }
    }
    *max_exp = (uint8_t)S;
    *prime = (uint8_t)bits;
}

/* Pack x[rows][cols] (row pitch ld_x elements; dtype 0 = fp32 bits, 1 = bf16
 * bits) along the last axis.  Blocks are numbered row-major over (row, block
 * within row), ceil(cols/16) per row; a trailing partial block is padded with
 * +0.  q is [nb][16], max_exp [nb], prime [nb]. */
void oref_mx9_pack(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                   int8_t *q, uint8_t *max_exp, uint8_t *prime)
{
    int64_t nbr = (cols + 15) / 16, r, b;
    for (r = 0; r < rows; r++) {
        for (b = 0; b < nbr; b++) {
            double val[16];
            int ef[16], kind[16], i;
            int64_t blk = r * nbr + b;
            for (i = 0; i < 16; i++) {
                int64_t c = 16 * b + i;
                if (c >= cols) {                       /* padding: +0 */
                    val[i] = 0.0; ef[i] = 0; kind[i] = 0;
                } else if (dtype == 0) {
                    uint32_t w = ((const uint32_t *)x)[r * ld_x + c];
                    val[i] = fp32_decode(w, &kind[i]);
                    ef[i] = (w >> 23) & 0xFF;
                } else {
                    uint16_t h = ((const uint16_t *)x)[r * ld_x + c];
                    val[i] = bf16_decode(h, &kind[i]);
                    ef[i] = (h >> 7) & 0xFF;
                }
            }
            mx9_block(val, ef, kind, q + 16 * blk, max_exp + blk, prime + blk);
        }
    }
}

/* Round an exact value to bfloat16, nearest with ties to even, and return its
 * bits.  The value's quantum is 2^(floor(log2|y|) - 7) in the normal range and
 * 2^-133 below 2^-126; rint() rounds half to even. */
static uint16_t bf16_round(double y)
{
    double a = fabs(y), quantum, r;
    int ex;
    float f;
    uint32_t w;
    if (a == 0.0) {
        r = 0.0;
    } else {
        if (a < ldexp(1.0, -126)) {
            quantum = ldexp(1.0, -133);
        } else {
            frexp(a, &ex);                 /* a = m * 2^ex, m in [0.5, 1) */
            quantum = ldexp(1.0, ex - 1 - 7);
        }
        r = rint(a / quantum) * quantum;
    }
    f = (float)(signbit(y) ? -r : r);      /* exact: r is a bf16 value */
    memcpy(&w, &f, 4);
    return (uint16_t)(w >> 16);
}

/* Unpack: y = q * 2^(max_exp - 127 - 6 - p) for max_exp != 255, NaN for 255.
 * out_dtype 0 = fp32 (exact), 1 = bf16 (round to nearest even).  Writes the
 * first cols columns of each row of y (row pitch ld_y elements).  NaN is the
 * quiet NaN 0x7FC00000 (fp32) / 0x7FC0 (bf16). */
void oref_mx9_unpack(const int8_t *q, const uint8_t *max_exp, const uint8_t *prime,
                     int64_t rows, int64_t cols, int out_dtype, void *y, int64_t ld_y)
{
    int64_t nbr = (cols + 15) / 16, r, c;
    for (r = 0; r < rows; r++) {
        for (c = 0; c < cols; c++) {
            int64_t blk = r * nbr + c / 16;
            int i = (int)(c % 16);
            int S = max_exp[blk];
            int p = (prime[blk] >> (i / 2)) & 1;
            if (out_dtype == 0) {
                uint32_t w;
                if (S == 255) {
                    w = 0x7FC00000u;
                } else {
                    float f = (float)ldexp((double)q[16 * blk + i], S - 127 - 6 - p);
                    memcpy(&w, &f, 4);
                }
                ((uint32_t *)y)[r * ld_y + c] = w;
            } else {
                uint16_t h = S == 255 ? 0x7FC0
                           : bf16_round(ldexp((double)q[16 * blk + i], S - 127 - 6 - p));
                ((uint16_t *)y)[r * ld_y + c] = h;
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* MX9 along any axis   [MX9] (the axis argument of the MX9 calls)          */
/* ------------------------------------------------------------------------ */

/* The array is contiguous and viewed as x[outer][len][inner]; blocks of 16
 * run along len.  Reading: the axis is first moved to the last position
 * (movedim(axis, -1)), so row (o, i) of the moved array is x[o][0..len-1][i]
 * and the block order is (o, i, j), j = block within the row,
 * ceil(len/16) blocks per row.  Each row is packed exactly as
 * oref_mx9_pack packs one row.  This call handles the rows with
 * i0 <= i < i1, for every o. */
void oref_mx9_pack_axis(const void *x, int dtype, int64_t outer, int64_t len, int64_t inner,
                        int64_t i0, int64_t i1, int8_t *q, uint8_t *max_exp, uint8_t *prime)
{
    int64_t nbl = (len + 15) / 16, o, i, l;
    size_t es = dtype == 0 ? 4 : 2;
    unsigned char row[4 * 16 * 1024];      /* one moved row, in chunks of 16 Ki elements */
    for (o = 0; o < outer; o++) {
        for (i = i0; i < i1; i++) {
            int64_t blk0 = (o * inner + i) * nbl, done;
            for (done = 0; done < len; done += 16 * 1024) {
                int64_t n = len - done < 16 * 1024 ? len - done : 16 * 1024;
                for (l = 0; l < n; l++)
                    memcpy(row + l * es, (const unsigned char *)x + (size_t)((o * len + done + l) * inner + i) * es, es);
                oref_mx9_pack(row, dtype, 1, n, n, q + 16 * (blk0 + done / 16),
                              max_exp + blk0 + done / 16, prime + blk0 + done / 16);
            }
        }
    }
}

/* Inverse of oref_mx9_pack_axis: unpack row (o, i) as oref_mx9_unpack unpacks
 * one row and place element l at y[o][l][i]. */
void oref_mx9_unpack_axis(const int8_t *q, const uint8_t *max_exp, const uint8_t *prime,
                          int64_t outer, int64_t len, int64_t inner, int64_t i0, int64_t i1,
                          int out_dtype, void *y)
{
    int64_t nbl = (len + 15) / 16, o, i, l;
    size_t es = out_dtype == 0 ? 4 : 2;
    unsigned char row[4 * 16 * 1024];
    for (o = 0; o < outer; o++) {
        for (i = i0; i < i1; i++) {
            int64_t blk0 = (o * inner + i) * nbl, done;
            for (done = 0; done < len; done += 16 * 1024) {
                int64_t n = len - done < 16 * 1024 ? len - done : 16 * 1024;
                oref_mx9_unpack(q + 16 * (blk0 + done / 16), max_exp + blk0 + done / 16,
                                prime + blk0 + done / 16, 1, n, out_dtype, row, n);
                for (l = 0; l < n; l++)
                    memcpy((unsigned char *)y + (size_t)((o * len + done + l) * inner + i) * es, row + l * es, es);
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* MX9 in one byte tensor   [MX9] (commit "pack mx9 into a single uint8     */
/* tensor"; the exponent byte is stored at blk * N_PACKED_BYTES)            */
/* ------------------------------------------------------------------------ */

/* One 18-byte record per block: the E8M0 exponent byte first (the pages
 * place it at the record's start), then q[0..15], then the prime byte
 * (reading: the order of q and prime inside the record is not printed).
 * Rows of bpr records sit at a pitch of ld_p bytes; bytes past 18 * bpr in a
 * row are not touched. */
void oref_mx9_to_records(const int8_t *q, const uint8_t *max_exp, const uint8_t *prime,
                         int64_t rows, int64_t bpr, uint8_t *packed, int64_t ld_p)
{
    int64_t r, b;
    for (r = 0; r < rows; r++) {
        for (b = 0; b < bpr; b++) {
            int64_t blk = r * bpr + b;
            uint8_t *rec = packed + r * ld_p + 18 * b;
            rec[0] = max_exp[blk];
            memcpy(rec + 1, q + 16 * blk, 16);
            rec[17] = prime[blk];
        }
    }
}

/* Inverse of oref_mx9_to_records. */
void oref_mx9_from_records(const uint8_t *packed, int64_t ld_p, int64_t rows, int64_t bpr,
                           int8_t *q, uint8_t *max_exp, uint8_t *prime)
{
    int64_t r, b;
    for (r = 0; r < rows; r++) {
        for (b = 0; b < bpr; b++) {
            int64_t blk = r * bpr + b;
            const uint8_t *rec = packed + r * ld_p + 18 * b;
            max_exp[blk] = rec[0];
            memcpy(q + 16 * blk, rec + 1, 16);
            prime[blk] = rec[17];
        }
    }
}

/* ------------------------------------------------------------------------ */
/* MXFP8 block-scaled contraction   [MXFP8 GG] (AMD-AGI/ALTO PR #31: the     */
/* E4M3 grouped GEMM whose operands are MXFP8 data with E8M0 block-32       */
/* scales along the contraction)                                             */
/* ------------------------------------------------------------------------ */

/* E8M0 scale byte b: 2^(b - 127); 255 is NaN. */
static double e8m0_value(uint8_t b)
{
    return b == 255 ? NAN : ldexp(1.0, (int)b - 127);
}

/* "NT" form: both operands are stored with the contraction index contiguous.
 *   C[m][n] = sum over k in [k0, k1) of
 *             e4m3(A[m][k]) * 2^(sA(m, k/32) - 127) * e4m3(B[n][k]) * 2^(sB(n, k/32) - 127)
 * with sA(m, b) = sA[m * sa_rs + b * sa_bs] and sB(n, b) = sB[n * sb_rs + b * sb_bs],
 * for rows m0 <= m < m1 and all n < N; k0 and k1 are multiples of 32.
 * Each product is exact in binary64 and the sum is accumulated in binary64
 * in k order.  absC, when non-NULL, receives the sum of |product|: the
 * quantity any other summation order's rounding error is proportional to.
 * NaN codes and scale byte 255 propagate as NaN. */
void oref_mx_gemm_nt(const uint8_t *A, int64_t lda, const uint8_t *sA, int64_t sa_rs, int64_t sa_bs,
                     const uint8_t *B, int64_t ldb, const uint8_t *sB, int64_t sb_rs, int64_t sb_bs,
                     int64_t m0, int64_t m1, int64_t N, int64_t k0, int64_t k1,
                     double *C, double *absC, int64_t ldc)
{
    double dec[256], sc[256];
    int64_t m, n, k;
    int i;
    for (i = 0; i < 256; i++) {
        dec[i] = oref_e4m3_value((uint8_t)i);
        sc[i] = e8m0_value((uint8_t)i);
    }
    for (m = m0; m < m1; m++) {
        for (n = 0; n < N; n++) {
            double acc = 0.0, mag = 0.0;
            for (k = k0; k < k1; k++) {
                double a = dec[A[m * lda + k]] * sc[sA[m * sa_rs + (k / 32) * sa_bs]];
                double b = dec[B[n * ldb + k]] * sc[sB[n * sb_rs + (k / 32) * sb_bs]];
                acc += a * b;
                mag += fabs(a * b);
            }
            C[m * ldc + n] = acc;
            if (absC)
                absC[m * ldc + n] = mag;
        }
    }
}
