// mxq_abi.cpp -- the C ABI declared in include/mxq.h.
//
// Every entry point validates its arguments on the host, in the order the
// header documents, before enqueuing anything; a nonzero status therefore
// means no output byte was written.  Nothing here allocates, synchronizes or
// keeps state.
#include "../../include/mxq.h"

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mxq_kernels.h"

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 30;
constexpr int64_t kMaxDual = int64_t(1) << 24;   // dual-axis: 32-bit per-lane offsets within a tile
constexpr uint64_t kMaxThreads = 0xFFFFFFFFull - 256;   // grid.x * block.x must fit 32 bits

struct Span {
    uintptr_t p;
    uint64_t n;   // bytes
};

bool overlap(const Span& a, const Span& b) {
    return a.n != 0 && b.n != 0 && a.p < b.p + b.n && b.p < a.p + a.n;
}

bool any_overlap(const Span* s, int k) {
    for (int i = 0; i < k; ++i)
        for (int j = i + 1; j < k; ++j)
            if (overlap(s[i], s[j])) return true;
    return false;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

uintptr_t addr(const void* p) { return reinterpret_cast<uintptr_t>(p); }

// No device buffer spans more bytes than a 48-bit virtual address space.
constexpr uint64_t kMaxSpan = uint64_t(1) << 48;
constexpr uint64_t kTooLarge = ~uint64_t(0);

// Bytes spanned by a [rows, cols] matrix with row pitch ld (elements), or
// kTooLarge when that exceeds kMaxSpan (computed without overflow).
uint64_t matrix_bytes(int64_t rows, int64_t cols, int64_t ld, int64_t esz) {
    if (rows <= 0 || cols <= 0) return 0;
    const unsigned __int128 b =
        (static_cast<unsigned __int128>(rows - 1) * uint64_t(ld) + uint64_t(cols)) * uint64_t(esz);
    return b > kMaxSpan ? kTooLarge : uint64_t(b);
}

int check_dual(const uint16_t* x, int64_t M, int64_t N, int64_t ld_x, int32_t block_size,
               int32_t scaling_mode, const uint8_t* q_row, const uint8_t* s_row,
               const uint8_t* q_col, const uint8_t* s_col) {
    const bool empty = M == 0 || N == 0;   // empty buffers may be NULL
    if (!empty && (!x || !q_row || !s_row || !q_col || !s_col)) return MX_E_NULL;
    if (block_size != 32) return MX_E_BLOCK;
    if (scaling_mode != MX_SCALE_RCEIL) return MX_E_MODE;
    if (M < 0 || N < 0 || M > kMaxDual || N > kMaxDual || M % 128 != 0 || N % 128 != 0)
        return MX_E_SHAPE;
    if (uint64_t(M / 128) * uint64_t(N / 128) * 512 > kMaxThreads) return MX_E_SHAPE;   // one 512-thread workgroup per tile
    if (ld_x < N || ld_x % 8 != 0 || ld_x > kMaxDual) return MX_E_STRIDE;
    if (!empty && (!aligned(x, 16) || !aligned(q_row, 16) || !aligned(s_row, 16) ||
                   !aligned(q_col, 16) || !aligned(s_col, 16)))
        return MX_E_ALIGN;
    return MX_OK;
}

int dual_call(const uint16_t* x, int64_t M, int64_t N, int64_t ld_x, int32_t block_size,
              int32_t scaling_mode, uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
              bool mfma_scales, void* stream) {
    int rc = check_dual(x, M, N, ld_x, block_size, scaling_mode, q_row, s_row, q_col, s_col);
    if (rc != MX_OK) return rc;
    const uint64_t mn = uint64_t(M) * uint64_t(N);
    const Span s[5] = {{addr(x), matrix_bytes(M, N, ld_x, 2)}, {addr(q_row), mn}, {addr(s_row), mn / 32},
                       {addr(q_col), mn}, {addr(s_col), mn / 32}};
    if (any_overlap(s, 5)) return MX_E_OVERLAP;
    if (M == 0 || N == 0) return MX_OK;
    hipError_t e = mxq::launch_dual_axis(x, M, N, ld_x, q_row, s_row, q_col, s_col, nullptr, 0, nullptr, false,
                                         mfma_scales, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MX_OK : MX_E_LAUNCH;
}

int grouped_call(const uint16_t* x, int64_t M, int64_t N, int64_t ld_x, int32_t block_size,
                 int32_t scaling_mode, const int32_t* offs, int32_t G, uint8_t* q_row, uint8_t* s_row,
                 uint8_t* q_col, uint8_t* s_col, int32_t* err, bool mfma_scales, void* stream) {
    int rc = check_dual(x, M, N, ld_x, block_size, scaling_mode, q_row, s_row, q_col, s_col);
    if (rc != MX_OK) return rc;
    if (G < 0) return MX_E_SHAPE;
    if (G > 0 && !offs) return MX_E_NULL;
    if (G > 0 && !aligned(offs, 4)) return MX_E_ALIGN;
    if (err && !aligned(err, 4)) return MX_E_ALIGN;
    const uint64_t mn = uint64_t(M) * uint64_t(N);
    const Span s[7] = {{addr(x), matrix_bytes(M, N, ld_x, 2)}, {addr(q_row), mn}, {addr(s_row), mn / 32},
                       {addr(q_col), mn}, {addr(s_col), mn / 32},
                       {addr(offs), G > 0 ? uint64_t(G) * 4 : 0}, {addr(err), err ? 4u : 0u}};
    if (any_overlap(s, 7)) return MX_E_OVERLAP;
    hipError_t e = hipSuccess;
    if (M == 0 || N == 0) {
        if (err) e = mxq::launch_offs_validate(offs, G, M, err, static_cast<hipStream_t>(stream));
    } else {
        e = mxq::launch_dual_axis(x, M, N, ld_x, q_row, s_row, q_col, s_col, offs, G, err, true, mfma_scales,
                                  static_cast<hipStream_t>(stream));
    }
    return e == hipSuccess ? MX_OK : MX_E_LAUNCH;
}

// Shared checks of the axis and record calls; nb receives the block count.
int check_mx9_view(int32_t dtype, int64_t outer, int64_t len, int64_t inner, int32_t block_size,
                   uint64_t* nb) {
    if (dtype != MX_DTYPE_F32 && dtype != MX_DTYPE_BF16) return MX_E_DTYPE;
    if (block_size != 16) return MX_E_BLOCK;
    if (outer < 0 || len < 0 || inner < 0 || len > kMaxDim || outer > kMaxDim || inner > kMaxDim)
        return MX_E_SHAPE;
    const uint64_t elems = uint64_t(outer) * uint64_t(len) * uint64_t(inner);
    if (elems > (uint64_t(1) << 40)) return MX_E_SHAPE;
    *nb = uint64_t(outer) * uint64_t(inner) * uint64_t((len + 15) / 16);
    if (*nb > kMaxThreads) return MX_E_SHAPE;
    // the tile kernels of a non-last axis: one workgroup per tile
    if (*nb > 0 && inner > 1 && mxq::mx9_axis_grid_threads(outer, len, inner) > kMaxThreads) return MX_E_SHAPE;
    return MX_OK;
}

// Bytes spanned by a strided scale view of rows x blocks (non-negative strides).
uint64_t scale_span(int64_t rows, int64_t blocks, int64_t rs, int64_t bs) {
    if (rows <= 0 || blocks <= 0) return 0;
    return uint64_t((rows - 1) * rs + (blocks - 1) * bs + 1);
}

constexpr int64_t kMaxGemm = int64_t(1) << 24;

// Checks shared by the contraction calls: operand pitches and alignment,
// scale strides, the output type and pitch.  K is the contraction extent.
int check_gemm(const uint8_t* A, int64_t lda, const uint8_t* sA, int64_t sa_rs, int64_t sa_bs,
               const uint8_t* B, int64_t ldb, const uint8_t* sB, int64_t sb_rs, int64_t sb_bs,
               int64_t M, int64_t N, int64_t K, const void* C, int64_t ldc, int32_t out_dtype, bool mfma) {
    const bool empty = M == 0 || N == 0;
    if (!empty && (!A || !sA || !B || !sB || !C)) return MX_E_NULL;
    if (out_dtype != MX_DTYPE_F32 && out_dtype != MX_DTYPE_BF16) return MX_E_DTYPE;
    if (M < 0 || N < 0 || K < 0 || M > kMaxGemm || N > kMaxGemm || K > kMaxGemm ||
        M % 128 != 0 || N % 128 != 0 || K % 128 != 0)
        return MX_E_SHAPE;
    if (lda < K || ldb < K || lda % 16 != 0 || ldb % 16 != 0 || lda > kMaxGemm || ldb > kMaxGemm || ldc < N ||
        ldc > kMaxGemm || sa_rs < 0 || sa_bs < 0 || sb_rs < 0 || sb_bs < 0)
        return MX_E_STRIDE;
    const uintptr_t esz = out_dtype == MX_DTYPE_F32 ? 4 : 2;
    if (!empty && (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, esz))) return MX_E_ALIGN;
    if (!empty && mfma && (!aligned(sA, 16) || !aligned(sB, 16))) return MX_E_ALIGN;
    return MX_OK;
}

// Whether every contraction kernel the call may launch has a grid whose
// thread count fits 32 bits: the general kernel (128 x 128 tiles of 256
// threads), the pipelined kernel (256 x 256 tiles of 512 threads, or for row
// groups 8 XCD shares of at most ceil(M/128/8) + 1 row tiles of 128 x 256),
// times the group count for contraction groups.
bool gemm_grid_fits(int64_t M, int64_t N, int32_t G, bool row_groups, bool k_groups) {
    const uint64_t g = k_groups ? uint64_t(G) : 1u;
    const uint64_t general = uint64_t(M / 128) * uint64_t(N / 128) * g * 256u;
    const uint64_t pipe = row_groups ? 8u * (uint64_t(M / 128 + 7) / 8u + 1u) * uint64_t((N + 255) / 256) * 512u
                                     : uint64_t((M + 255) / 256) * uint64_t((N + 255) / 256) * g * 512u;
    return general <= kMaxThreads && pipe <= kMaxThreads;
}

// Bytes of one operand's scales: a strided view, or rows * K/32 in the matrix-core layout.
uint64_t scale_bytes(bool mfma, int64_t rows, int64_t K, int64_t rs, int64_t bs) {
    return mfma ? uint64_t(rows) * uint64_t(K / 32) : scale_span(rows, K / 32, rs, bs);
}

int gemm_call(const uint8_t* A, int64_t lda, const uint8_t* sA, int64_t sa_rs, int64_t sa_bs,
              const uint8_t* B, int64_t ldb, const uint8_t* sB, int64_t sb_rs, int64_t sb_bs,
              int64_t M, int64_t N, int64_t K, void* C, int64_t ldc, int32_t out_dtype, bool mfma, void* stream) {
    int rc = check_gemm(A, lda, sA, sa_rs, sa_bs, B, ldb, sB, sb_rs, sb_bs, M, N, K, C, ldc, out_dtype, mfma);
    if (rc != MX_OK) return rc;
    if (!gemm_grid_fits(M, N, 1, false, false)) return MX_E_SHAPE;
    const uint64_t esz = out_dtype == MX_DTYPE_F32 ? 4 : 2;
    const uint64_t cb = matrix_bytes(M, N, ldc, int64_t(esz));
    const Span s[5] = {{addr(C), cb}, {addr(A), matrix_bytes(M, K, lda, 1)}, {addr(B), matrix_bytes(N, K, ldb, 1)},
                       {addr(sA), scale_bytes(mfma, M, K, sa_rs, sa_bs)}, {addr(sB), scale_bytes(mfma, N, K, sb_rs, sb_bs)}};
    for (int i = 1; i < 5; ++i)
        if (overlap(s[0], s[i])) return MX_E_OVERLAP;
    if (M == 0 || N == 0) return MX_OK;
    hipError_t e = mxq::launch_mx_gemm(A, lda, sA, sa_rs, sa_bs, B, ldb, 0, sB, sb_rs, sb_bs, 0, C, ldc, 0, M, N, K,
                                       nullptr, 1, 0, out_dtype, mfma, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MX_OK : MX_E_LAUNCH;
}

int gemm_rows_call(const uint8_t* A, int64_t lda, const uint8_t* sA, int64_t sa_rs, int64_t sa_bs,
                   const uint8_t* B, int64_t ldb, int64_t b_gs, const uint8_t* sB, int64_t sb_rs,
                   int64_t sb_bs, int64_t sb_gs, const int32_t* offs, int32_t G, int64_t M, int64_t N,
                   int64_t K, void* C, int64_t ldc, int32_t out_dtype, bool mfma, void* stream) {
    int rc = check_gemm(A, lda, sA, sa_rs, sa_bs, B, ldb, sB, sb_rs, sb_bs, M, N, K, C, ldc, out_dtype, mfma);
    if (rc != MX_OK) return rc;
    if (G < 1 || G > (1 << 20)) return MX_E_SHAPE;
    if (!gemm_grid_fits(M, N, G, true, false)) return MX_E_SHAPE;
    if (!offs) return MX_E_NULL;
    if (!aligned(offs, 4)) return MX_E_ALIGN;
    if (b_gs < 0 || sb_gs < 0) return MX_E_STRIDE;
    const uint64_t esz = out_dtype == MX_DTYPE_F32 ? 4 : 2;
    const Span s[6] = {{addr(C), matrix_bytes(M, N, ldc, int64_t(esz))}, {addr(A), matrix_bytes(M, K, lda, 1)},
                       {addr(B), uint64_t(G - 1) * uint64_t(b_gs) + matrix_bytes(N, K, ldb, 1)},
                       {addr(sA), scale_bytes(mfma, M, K, sa_rs, sa_bs)},
                       {addr(sB), uint64_t(G - 1) * uint64_t(sb_gs) + scale_bytes(mfma, N, K, sb_rs, sb_bs)},
                       {addr(offs), uint64_t(G) * 4}};
    for (int i = 1; i < 6; ++i)
        if (overlap(s[0], s[i])) return MX_E_OVERLAP;
    if (M == 0 || N == 0) return MX_OK;
    hipError_t e = mxq::launch_mx_gemm(A, lda, sA, sa_rs, sa_bs, B, ldb, b_gs, sB, sb_rs, sb_bs, sb_gs, C, ldc, 0,
                                       M, N, K, offs, G, 0, out_dtype, mfma, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MX_OK : MX_E_LAUNCH;
}

int gemm_k_call(const uint8_t* A, int64_t lda, const uint8_t* sA, int64_t sa_rs, int64_t sa_bs,
                const uint8_t* B, int64_t ldb, const uint8_t* sB, int64_t sb_rs, int64_t sb_bs,
                const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K, void* C, int64_t ldc,
                int64_t c_gs, int32_t out_dtype, bool mfma, void* stream) {
    int rc = check_gemm(A, lda, sA, sa_rs, sa_bs, B, ldb, sB, sb_rs, sb_bs, M, N, K, C, ldc, out_dtype, mfma);
    if (rc != MX_OK) return rc;
    if (G < 1 || G > (1 << 20)) return MX_E_SHAPE;
    if (!offs) return MX_E_NULL;
    if (!aligned(offs, 4)) return MX_E_ALIGN;
    const uint64_t esz = out_dtype == MX_DTYPE_F32 ? 4 : 2;
    const uint64_t slab = matrix_bytes(M, N, ldc, 1);                  // elements of one group's C
    if (c_gs < int64_t(slab)) return MX_E_STRIDE;
    if (!gemm_grid_fits(M, N, G, false, true)) return MX_E_SHAPE;
    const Span s[6] = {{addr(C), (uint64_t(G - 1) * uint64_t(c_gs) + slab) * esz},
                       {addr(A), matrix_bytes(M, K, lda, 1)}, {addr(B), matrix_bytes(N, K, ldb, 1)},
                       {addr(sA), scale_bytes(mfma, M, K, sa_rs, sa_bs)}, {addr(sB), scale_bytes(mfma, N, K, sb_rs, sb_bs)},
                       {addr(offs), uint64_t(G) * 4}};
    for (int i = 1; i < 6; ++i)
        if (overlap(s[0], s[i])) return MX_E_OVERLAP;
    if (M == 0 || N == 0) return MX_OK;
    hipError_t e = mxq::launch_mx_gemm(A, lda, sA, sa_rs, sa_bs, B, ldb, 0, sB, sb_rs, sb_bs, 0, C, ldc, c_gs, M, N,
                                       K, offs, G, 1, out_dtype, mfma, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MX_OK : MX_E_LAUNCH;
}

// Checks of the scale-layout conversions: view (rs, bs) of rows x blocks
// plain scales, flat buffer of rows * blocks bytes in the matrix-core layout.
// A view that is written (the inverse conversion) must not alias itself.
int check_scale_conversion(const uint8_t* view, int64_t rs, int64_t bs, int64_t rows, int64_t blocks,
                           const uint8_t* flat, bool view_written) {
    const bool empty = rows == 0 || blocks == 0;
    if (!empty && (!view || !flat)) return MX_E_NULL;
    if (rows < 0 || blocks < 0 || rows % 64 != 0 || blocks % 4 != 0 || rows > kMaxDim || blocks > kMaxDim)
        return MX_E_SHAPE;
    if (uint64_t(rows) * uint64_t(blocks) / 4 > kMaxThreads) return MX_E_SHAPE;
    if (rs < 0 || bs < 0 || rs > kMaxDim || bs > kMaxDim) return MX_E_STRIDE;
    if (view_written && !empty &&
        !(rs >= 1 && bs >= 1 && (rs >= blocks * bs || bs >= rows * rs)))
        return MX_E_STRIDE;
    if (!empty && !aligned(flat, 4)) return MX_E_ALIGN;
    const Span a{addr(view), scale_span(rows, blocks, rs, bs)}, b{addr(flat), empty ? 0u : uint64_t(rows * blocks)};
    if (overlap(a, b)) return MX_E_OVERLAP;
    return MX_OK;
}

}  // namespace

extern "C" {

const char* mx_status_string(int status) {
    switch (status) {
        case MX_OK: return "MX_OK: success";
        case MX_E_NULL: return "MX_E_NULL: a required pointer is NULL";
        case MX_E_DTYPE: return "MX_E_DTYPE: unsupported element type (fp32 or bf16 only)";
        case MX_E_BLOCK: return "MX_E_BLOCK: unsupported block size (32 for MXFP8, 16 for MX9)";
        case MX_E_MODE: return "MX_E_MODE: unsupported scaling mode (RCEIL only)";
        case MX_E_SHAPE: return "MX_E_SHAPE: unsupported shape (MXFP8 needs M, N multiples of 128)";
        case MX_E_STRIDE: return "MX_E_STRIDE: row pitch smaller than the row or misaligned";
        case MX_E_ALIGN: return "MX_E_ALIGN: pointer misaligned";
        case MX_E_OVERLAP: return "MX_E_OVERLAP: buffers of one call overlap";
        case MX_E_LAUNCH: return "MX_E_LAUNCH: kernel launch failed";
        default: return "unknown mx_status";
    }
}

int mx_quantize_2d_dual(const uint16_t* x, int64_t M, int64_t N, int64_t ld_x,
                        int32_t block_size, int32_t scaling_mode,
                        uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                        void* stream) {
    return dual_call(x, M, N, ld_x, block_size, scaling_mode, q_row, s_row, q_col, s_col, false, stream);
}

int mx_quantize_2d_dual_mfma(const uint16_t* x, int64_t M, int64_t N, int64_t ld_x,
                             int32_t block_size, int32_t scaling_mode,
                             uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                             void* stream) {
    return dual_call(x, M, N, ld_x, block_size, scaling_mode, q_row, s_row, q_col, s_col, true, stream);
}

int mx_quantize_grouped(const uint16_t* x, int64_t M, int64_t N, int64_t ld_x,
                        int32_t block_size, int32_t scaling_mode,
                        const int32_t* offs, int32_t G,
                        uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                        int32_t* err, void* stream) {
    return grouped_call(x, M, N, ld_x, block_size, scaling_mode, offs, G, q_row, s_row, q_col, s_col, err,
                        false, stream);
}

int mx_quantize_grouped_mfma(const uint16_t* x, int64_t M, int64_t N, int64_t ld_x,
                             int32_t block_size, int32_t scaling_mode,
                             const int32_t* offs, int32_t G,
                             uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                             int32_t* err, void* stream) {
    return grouped_call(x, M, N, ld_x, block_size, scaling_mode, offs, G, q_row, s_row, q_col, s_col, err,
                        true, stream);
}

int mx9_pack_strided(const void* x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld_x,
                     int32_t block_size, int8_t* q, int64_t ld_q, uint8_t* max_exp, int64_t ld_e,
                     uint8_t* prime, int64_t ld_pr, void* stream) {
    const bool empty = rows == 0 || cols == 0;   // empty buffers may be NULL
    if (!empty && (!x || !q || !max_exp || !prime)) return MX_E_NULL;
    if (dtype != MX_DTYPE_F32 && dtype != MX_DTYPE_BF16) return MX_E_DTYPE;
    if (block_size != 16) return MX_E_BLOCK;
    if (rows < 0 || cols < 0 || rows > (int64_t(1) << 40) || cols > kMaxDim) return MX_E_SHAPE;
    const int64_t bpr = (cols + 15) / 16;
    const uint64_t nb = uint64_t(rows) * uint64_t(bpr);
    if (nb > kMaxThreads) return MX_E_SHAPE;
    if (ld_x < cols || ld_x > (int64_t(1) << 40)) return MX_E_STRIDE;
    if (ld_q < 16 * bpr || ld_q % 16 != 0 || ld_e < bpr || ld_pr < bpr || ld_q > (int64_t(1) << 40) ||
        ld_e > (int64_t(1) << 40) || ld_pr > (int64_t(1) << 40))
        return MX_E_STRIDE;
    const int64_t esz = dtype == MX_DTYPE_F32 ? 4 : 2;
    const uint64_t xb = matrix_bytes(rows, cols, ld_x, esz);
    const uint64_t qb = matrix_bytes(rows, 16 * bpr, ld_q, 1);
    const uint64_t eb = matrix_bytes(rows, bpr, ld_e, 1);
    const uint64_t pb = matrix_bytes(rows, bpr, ld_pr, 1);
    if (xb == kTooLarge || qb == kTooLarge || eb == kTooLarge || pb == kTooLarge) return MX_E_STRIDE;
    if (!empty && (!aligned(x, uintptr_t(esz)) || !aligned(q, 16))) return MX_E_ALIGN;
    const Span s[4] = {{addr(x), xb}, {addr(q), qb}, {addr(max_exp), eb}, {addr(prime), pb}};
    if (any_overlap(s, 4)) return MX_E_OVERLAP;
    if (nb == 0) return MX_OK;
    hipError_t e = mxq::launch_mx9_pack(x, dtype, rows, cols, ld_x, q, ld_q, max_exp, ld_e, prime, ld_pr,
                                        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MX_OK : MX_E_LAUNCH;
}

int mx9_unpack_strided(const int8_t* q, int64_t ld_q, const uint8_t* max_exp, int64_t ld_e,
                       const uint8_t* prime, int64_t ld_pr, int64_t rows, int64_t cols, int32_t block_size,
                       int32_t out_dtype, void* y, int64_t ld_y, void* stream) {
    const bool empty = rows == 0 || cols == 0;   // empty buffers may be NULL
    if (!empty && (!q || !max_exp || !prime || !y)) return MX_E_NULL;
    if (out_dtype != MX_DTYPE_F32 && out_dtype != MX_DTYPE_BF16) return MX_E_DTYPE;
    if (block_size != 16) return MX_E_BLOCK;
    if (rows < 0 || cols < 0 || rows > (int64_t(1) << 40) || cols > kMaxDim) return MX_E_SHAPE;
    const int64_t bpr = (cols + 15) / 16;
    const uint64_t nb = uint64_t(rows) * uint64_t(bpr);
    if (nb > kMaxThreads) return MX_E_SHAPE;
    if (ld_y < cols || ld_y > (int64_t(1) << 40)) return MX_E_STRIDE;
    if (ld_q < 16 * bpr || ld_q % 16 != 0 || ld_e < bpr || ld_pr < bpr || ld_q > (int64_t(1) << 40) ||
        ld_e > (int64_t(1) << 40) || ld_pr > (int64_t(1) << 40))
        return MX_E_STRIDE;
    const int64_t esz = out_dtype == MX_DTYPE_F32 ? 4 : 2;
    const uint64_t yb = matrix_bytes(rows, cols, ld_y, esz);
    const uint64_t qb = matrix_bytes(rows, 16 * bpr, ld_q, 1);
    const uint64_t eb = matrix_bytes(rows, bpr, ld_e, 1);
    const uint64_t pb = matrix_bytes(rows, bpr, ld_pr, 1);
    if (yb == kTooLarge || qb == kTooLarge || eb == kTooLarge || pb == kTooLarge) return MX_E_STRIDE;
    if (!empty && (!aligned(q, 16) || !aligned(y, uintptr_t(esz)))) return MX_E_ALIGN;
    const Span s[4] = {{addr(q), qb}, {addr(max_exp), eb}, {addr(prime), pb}, {addr(y), yb}};
    if (any_overlap(s, 4)) return MX_E_OVERLAP;
    if (nb == 0) return MX_OK;
    hipError_t e = mxq::launch_mx9_unpack(q, ld_q, max_exp, ld_e, prime, ld_pr, rows, cols, out_dtype, y, ld_y,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MX_OK : MX_E_LAUNCH;
}

int mx9_pack(const void* x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld_x,
             int32_t block_size, int8_t* q, uint8_t* max_exp, uint8_t* prime, void* stream) {
    const int64_t bpr = cols > 0 && cols <= kMaxDim ? (cols + 15) / 16 : 0;   // others: MX_E_SHAPE
    return mx9_pack_strided(x, dtype, rows, cols, ld_x, block_size, q, 16 * bpr, max_exp, bpr, prime, bpr, stream);
}

int mx9_unpack(const int8_t* q, const uint8_t* max_exp, const uint8_t* prime,
               int64_t rows, int64_t cols, int32_t block_size, int32_t out_dtype,
               void* y, int64_t ld_y, void* stream) {
    const int64_t bpr = cols > 0 && cols <= kMaxDim ? (cols + 15) / 16 : 0;   // others: MX_E_SHAPE
    return mx9_unpack_strided(q, 16 * bpr, max_exp, bpr, prime, bpr, rows, cols, block_size, out_dtype, y, ld_y,
                              stream);
}

int mx9_pack_axis(const void* x, int32_t dtype, int64_t outer, int64_t len, int64_t inner,
                  int32_t block_size, int8_t* q, uint8_t* max_exp, uint8_t* prime, void* stream) {
    const bool empty = outer == 0 || len == 0 || inner == 0;
    if (!empty && (!x || !q || !max_exp || !prime)) return MX_E_NULL;
    uint64_t nb = 0;
    int rc = check_mx9_view(dtype, outer, len, inner, block_size, &nb);
    if (rc != MX_OK) return rc;
    const uint64_t esz = dtype == MX_DTYPE_F32 ? 4 : 2;
    if (!empty && (!aligned(x, uintptr_t(esz)) || !aligned(q, 16))) return MX_E_ALIGN;
    const Span s[4] = {{addr(x), uint64_t(outer) * uint64_t(len) * uint64_t(inner) * esz}, {addr(q), nb * 16},
                       {addr(max_exp), nb}, {addr(prime), nb}};
    if (any_overlap(s, 4)) return MX_E_OVERLAP;
    if (nb == 0) return MX_OK;
    hipError_t e = mxq::launch_mx9_pack_axis(x, dtype, outer, len, inner, q, max_exp, prime,
                                             static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MX_OK : MX_E_LAUNCH;
}

int mx9_unpack_axis(const int8_t* q, const uint8_t* max_exp, const uint8_t* prime, int64_t outer,
                    int64_t len, int64_t inner, int32_t block_size, int32_t out_dtype, void* y,
                    void* stream) {
    const bool empty = outer == 0 || len == 0 || inner == 0;
    if (!empty && (!q || !max_exp || !prime || !y)) return MX_E_NULL;
    uint64_t nb = 0;
    int rc = check_mx9_view(out_dtype, outer, len, inner, block_size, &nb);
    if (rc != MX_OK) return rc;
    const uint64_t esz = out_dtype == MX_DTYPE_F32 ? 4 : 2;
    if (!empty && (!aligned(q, 16) || !aligned(y, uintptr_t(esz)))) return MX_E_ALIGN;
    const Span s[4] = {{addr(q), nb * 16}, {addr(max_exp), nb}, {addr(prime), nb},
                       {addr(y), uint64_t(outer) * uint64_t(len) * uint64_t(inner) * esz}};
    if (any_overlap(s, 4)) return MX_E_OVERLAP;
    if (nb == 0) return MX_OK;
    hipError_t e = mxq::launch_mx9_unpack_axis(q, max_exp, prime, outer, len, inner, out_dtype, y,
                                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MX_OK : MX_E_LAUNCH;
}

int mx9_pack_records(const void* x, int32_t dtype, int64_t outer, int64_t len, int64_t inner,
                     int32_t block_size, uint8_t* packed, int64_t ld_p, void* stream) {
    const bool empty = outer == 0 || len == 0 || inner == 0;
    if (!empty && (!x || !packed)) return MX_E_NULL;
    uint64_t nb = 0;
    int rc = check_mx9_view(dtype, outer, len, inner, block_size, &nb);
    if (rc != MX_OK) return rc;
    const int64_t row_bytes = 18 * ((len + 15) / 16);
    if (ld_p < row_bytes || ld_p > (int64_t(1) << 40)) return MX_E_STRIDE;
    const uint64_t pb = matrix_bytes(outer * inner, row_bytes, ld_p, 1);
    if (pb == kTooLarge) return MX_E_STRIDE;
    const uint64_t esz = dtype == MX_DTYPE_F32 ? 4 : 2;
    if (!empty && !aligned(x, uintptr_t(esz))) return MX_E_ALIGN;
    const Span s[2] = {{addr(x), uint64_t(outer) * uint64_t(len) * uint64_t(inner) * esz}, {addr(packed), pb}};
    if (any_overlap(s, 2)) return MX_E_OVERLAP;
    if (nb == 0) return MX_OK;
    hipError_t e = mxq::launch_mx9_pack_records(x, dtype, outer, len, inner, packed, ld_p,
                                                static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MX_OK : MX_E_LAUNCH;
}

int mx9_unpack_records(const uint8_t* packed, int64_t ld_p, int64_t outer, int64_t len, int64_t inner,
                       int32_t block_size, int32_t out_dtype, void* y, void* stream) {
    const bool empty = outer == 0 || len == 0 || inner == 0;
    if (!empty && (!packed || !y)) return MX_E_NULL;
    uint64_t nb = 0;
    int rc = check_mx9_view(out_dtype, outer, len, inner, block_size, &nb);
    if (rc != MX_OK) return rc;
    const int64_t row_bytes = 18 * ((len + 15) / 16);
    if (ld_p < row_bytes || ld_p > (int64_t(1) << 40)) return MX_E_STRIDE;
    const uint64_t pb = matrix_bytes(outer * inner, row_bytes, ld_p, 1);
    if (pb == kTooLarge) return MX_E_STRIDE;
    const uint64_t esz = out_dtype == MX_DTYPE_F32 ? 4 : 2;
    if (!empty && !aligned(y, uintptr_t(esz))) return MX_E_ALIGN;
    const Span s[2] = {{addr(packed), pb}, {addr(y), uint64_t(outer) * uint64_t(len) * uint64_t(inner) * esz}};
    if (any_overlap(s, 2)) return MX_E_OVERLAP;
    if (nb == 0) return MX_OK;
    hipError_t e = mxq::launch_mx9_unpack_records(packed, ld_p, outer, len, inner, out_dtype, y,
                                                  static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MX_OK : MX_E_LAUNCH;
}

int mx_gemm_nt(const uint8_t* A, int64_t lda, const uint8_t* sA, int64_t sa_rs, int64_t sa_bs,
               const uint8_t* B, int64_t ldb, const uint8_t* sB, int64_t sb_rs, int64_t sb_bs,
               int64_t M, int64_t N, int64_t K, void* C, int64_t ldc, int32_t out_dtype, void* stream) {
    return gemm_call(A, lda, sA, sa_rs, sa_bs, B, ldb, sB, sb_rs, sb_bs, M, N, K, C, ldc, out_dtype, false, stream);
}

int mx_gemm_nt_mfma(const uint8_t* A, int64_t lda, const uint8_t* sA, const uint8_t* B, int64_t ldb,
                    const uint8_t* sB, int64_t M, int64_t N, int64_t K, void* C, int64_t ldc, int32_t out_dtype,
                    void* stream) {
    return gemm_call(A, lda, sA, 0, 0, B, ldb, sB, 0, 0, M, N, K, C, ldc, out_dtype, true, stream);
}

int mx_grouped_gemm_rows(const uint8_t* A, int64_t lda, const uint8_t* sA, int64_t sa_rs, int64_t sa_bs,
                         const uint8_t* B, int64_t ldb, int64_t b_gs, const uint8_t* sB, int64_t sb_rs,
                         int64_t sb_bs, int64_t sb_gs, const int32_t* offs, int32_t G, int64_t M, int64_t N,
                         int64_t K, void* C, int64_t ldc, int32_t out_dtype, void* stream) {
    return gemm_rows_call(A, lda, sA, sa_rs, sa_bs, B, ldb, b_gs, sB, sb_rs, sb_bs, sb_gs, offs, G, M, N, K, C,
                          ldc, out_dtype, false, stream);
}

int mx_grouped_gemm_rows_mfma(const uint8_t* A, int64_t lda, const uint8_t* sA, const uint8_t* B, int64_t ldb,
                              int64_t b_gs, const uint8_t* sB, int64_t sb_gs, const int32_t* offs, int32_t G,
                              int64_t M, int64_t N, int64_t K, void* C, int64_t ldc, int32_t out_dtype,
                              void* stream) {
    return gemm_rows_call(A, lda, sA, 0, 0, B, ldb, b_gs, sB, 0, 0, sb_gs, offs, G, M, N, K, C, ldc, out_dtype,
                          true, stream);
}

int mx_grouped_gemm_k(const uint8_t* A, int64_t lda, const uint8_t* sA, int64_t sa_rs, int64_t sa_bs,
                      const uint8_t* B, int64_t ldb, const uint8_t* sB, int64_t sb_rs, int64_t sb_bs,
                      const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K, void* C, int64_t ldc,
                      int64_t c_gs, int32_t out_dtype, void* stream) {
    return gemm_k_call(A, lda, sA, sa_rs, sa_bs, B, ldb, sB, sb_rs, sb_bs, offs, G, M, N, K, C, ldc, c_gs,
                       out_dtype, false, stream);
}

int mx_grouped_gemm_k_mfma(const uint8_t* A, int64_t lda, const uint8_t* sA, const uint8_t* B, int64_t ldb,
                           const uint8_t* sB, const int32_t* offs, int32_t G, int64_t M, int64_t N, int64_t K,
                           void* C, int64_t ldc, int64_t c_gs, int32_t out_dtype, void* stream) {
    return gemm_k_call(A, lda, sA, 0, 0, B, ldb, sB, 0, 0, offs, G, M, N, K, C, ldc, c_gs, out_dtype, true, stream);
}

int mx_scales_to_mfma(const uint8_t* s, int64_t rs, int64_t bs, int64_t rows, int64_t blocks, uint8_t* out,
                      void* stream) {
    int rc = check_scale_conversion(s, rs, bs, rows, blocks, out, false);
    if (rc != MX_OK) return rc;
    if (rows == 0 || blocks == 0) return MX_OK;
    hipError_t e = mxq::launch_scales_to_mfma(s, rs, bs, rows, blocks, out, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MX_OK : MX_E_LAUNCH;
}

int mx_scales_from_mfma(const uint8_t* in, int64_t rows, int64_t blocks, uint8_t* s, int64_t rs, int64_t bs,
                        void* stream) {
    int rc = check_scale_conversion(s, rs, bs, rows, blocks, in, true);
    if (rc != MX_OK) return rc;
    if (rows == 0 || blocks == 0) return MX_OK;
    hipError_t e = mxq::launch_scales_from_mfma(in, rows, blocks, s, rs, bs, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MX_OK : MX_E_LAUNCH;
}

}  // extern "C"
