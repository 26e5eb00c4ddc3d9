// Internal launch interface between the C-ABI layer (mxq_abi.cpp) and the
// HIP kernels.  Arguments arrive already validated; each launcher enqueues
// on the given stream and returns the launch's hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

// Fused dual-axis MXFP8 cast of a bf16 [M, N] matrix (M, N > 0, multiples
// of 128).  offs == nullptr selects the dense cast; otherwise G >= 0 group
// ends drive the uncovered-tail rule and *err (when non-null) receives the
// offset validation code.
hipError_t launch_dual_axis(const uint16_t* x, int64_t M, int64_t N, int64_t ld_x,
                            uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                            const int32_t* offs, int32_t G, int32_t* err, bool grouped,
                            bool mfma_scales, hipStream_t stream);

// Offset validation alone, for a grouped call on an empty matrix.
hipError_t launch_offs_validate(const int32_t* offs, int32_t G, int64_t M, int32_t* err,
                                hipStream_t stream);

// MX9 pack of [rows, cols] (rows, cols > 0); dtype 0 = fp32, 1 = bf16.
// Row r's blocks go to q + r * ld_q (bytes, a multiple of 16), max_exp +
// r * ld_e and prime + r * ld_pr; the three-part form passes ld_q = 16 *
// ceil(cols/16) and ld_e = ld_pr = ceil(cols/16).
hipError_t launch_mx9_pack(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                           int8_t* q, int64_t ld_q, uint8_t* max_exp, int64_t ld_e, uint8_t* prime,
                           int64_t ld_pr, hipStream_t stream);

// MX9 unpack to [rows, cols] (rows, cols > 0); out_dtype 0 = fp32, 1 = bf16;
// the parts are read with the pitches of launch_mx9_pack.
hipError_t launch_mx9_unpack(const int8_t* q, int64_t ld_q, const uint8_t* max_exp, int64_t ld_e,
                             const uint8_t* prime, int64_t ld_pr, int64_t rows, int64_t cols, int out_dtype,
                             void* y, int64_t ld_y, hipStream_t stream);

// MX9 in blocks of 16 along the middle axis of a contiguous [outer, len,
// inner] array (all > 0), blocks numbered (o * inner + i) * ceil(len/16) + j.
hipError_t launch_mx9_pack_axis(const void* x, int dtype, int64_t outer, int64_t len, int64_t inner,
                                int8_t* q, uint8_t* max_exp, uint8_t* prime, hipStream_t stream);
hipError_t launch_mx9_unpack_axis(const int8_t* q, const uint8_t* max_exp, const uint8_t* prime,
                                  int64_t outer, int64_t len, int64_t inner, int out_dtype, void* y,
                                  hipStream_t stream);

// The largest grid, in threads, that the axis and record calls may launch
// for an [outer, len, inner] view with inner > 1 (tile kernels), over both
// lane layouts; the caller rejects views whose grid would not fit 32 bits.
uint64_t mx9_axis_grid_threads(int64_t outer, int64_t len, int64_t inner);

// The same blocks as 18-byte records (exponent byte, q[16], prime byte); the
// records of one (o, i) form a row, rows at a pitch of ld_p bytes.
hipError_t launch_mx9_pack_records(const void* x, int dtype, int64_t outer, int64_t len, int64_t inner,
                                   uint8_t* packed, int64_t ld_p, hipStream_t stream);
hipError_t launch_mx9_unpack_records(const uint8_t* packed, int64_t ld_p, int64_t outer, int64_t len,
                                     int64_t inner, int out_dtype, void* y, hipStream_t stream);

// MXFP8 block-scaled contraction C = A B^T (codes with the contraction
// contiguous, E8M0 scales per 32 through strided views).  mode 0: dense
// (offs == nullptr) or row groups (group g's rows use B + g * b_gs, rows past
// offs[G-1] give 0); mode 1: contraction groups (group g writes C + g * c_gs
// from its contraction range).  M, N, K are multiples of 128.
hipError_t launch_mx_gemm(const uint8_t* A, int64_t lda, const uint8_t* sA, int64_t sa_rs, int64_t sa_bs,
                          const uint8_t* B, int64_t ldb, int64_t b_gs, const uint8_t* sB, int64_t sb_rs,
                          int64_t sb_bs, int64_t sb_gs, void* C, int64_t ldc, int64_t c_gs, int64_t M, int64_t N,
                          int64_t K, const int32_t* offs, int32_t G, int mode, int out_dtype, bool mfma_scales,
                          hipStream_t stream);

hipError_t launch_scales_to_mfma(const uint8_t* s, int64_t rs, int64_t bs, int64_t rows, int64_t blocks, uint8_t* out,
                                 hipStream_t stream);
hipError_t launch_scales_from_mfma(const uint8_t* in, int64_t rows, int64_t blocks, uint8_t* s, int64_t rs, int64_t bs,
                                   hipStream_t stream);

}  // namespace mxq
