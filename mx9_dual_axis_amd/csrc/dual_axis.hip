// dual_axis.hip -- fused dual-axis MXFP8 cast for gfx950 (CDNA4).
//
// Operation: pytorch/ao PR #4995, "[moe_training] Fused dual-axis MXFP8
// quantization with correct metadata" (PR description).  One read of a bf16
// matrix produces rowwise 1x32 and colwise 32x1 E4M3 data with E8M0 RCEIL
// scales; colwise data is stored transposed.
//
// Work decomposition: one workgroup (8 wave64s) per 128x128 tile.
//   * load   : each thread holds four 16-byte row segments (8 bf16 each); a
//              wave's load instruction covers four full 256-byte tile rows.
//              (8 waves of 4 loads measured 1% faster than 4 waves of 8 on
//              the stress shape, with the same LDS footprint per tile.)
//   * rowwise: a 1x32 block is four adjacent lanes; the block maximum is a
//              packed u16 max of the sign-masked bf16 patterns followed by a
//              two-step DPP quad reduction.  Masking the sign makes the
//              integer order NaN > Inf > finite, so the special cases need no
//              per-element test.  The cast runs from registers.
//   * LDS    : the tile is written once (32 KiB).  The 16-byte chunk index of
//              each row is XORed with a function of the row's 16-row chunk c
//              (2c + c/4, lds_chunk_xor), so that the lanes of a colwise
//              dword read (8 chunks x 8 column pairs per wave) hit distinct
//              banks (with 2c alone, a two-way conflict took 31% of the
//              LDS-active cycles).  What conflicts remain (7% of the
//              LDS-active cycles of a stress call) come from the small scale
//              stagings; the kernel is bound by memory, not by LDS.
//   * colwise: a unit is (column pair, 16-row chunk); each thread takes one.
//              A packed u16 max over 16 LDS dwords plus one DPP step between
//              the two chunks of a 32-row block gives both column maxima;
//              v_perm regroups (row m, row m+1) pairs of one column so the
//              packed scaled cast yields m-contiguous bytes.  The eight lanes
//              that share a column pair hold its eight chunks, so every
//              16-byte store of a wave lands in full 128-byte lines of the
//              transposed output.
//   * cast   : v_cvt_scalef32_pk_fp8_bf16 divides by the E8M0 scale 2^(b-127)
//              given as fp32 bits b<<23 (byte 0 acts as 2^-127, i.e. the 2^127
//              multiplier) and rounds to nearest even; it does not saturate,
//              so the colwise Inf block (scale 254) maps its NaN bytes to
//              +-448 afterwards, and poisoned blocks are overwritten with 0x7F.
//   * order  : consecutive workgroups take consecutive tile rows.  A call
//              that moves more than twice the memory-side cache visits the
//              tiles in a diagonal order (each tile row shifted one tile
//              column), which spreads the concurrently active row segments of
//              the input and of both outputs over the HBM channels; a smaller
//              call goes down whole tile columns (column-major), which the
//              cache serves better (measured on the workloads' shapes).
//   * s_col  : a tile owns 128 contiguous scale bytes in each of 4 block
//              rows; they are staged in LDS and leave as whole 128-byte lines
//              (one 16-byte store per lane), instead of 128 two-byte stores.
//   * s_row  : a tile owns 4 scale bytes of each of its 128 rows, written as
//              one 4-byte store per row.  Consecutive workgroups go to
//              consecutive XCDs, so with a tile-row count that is a multiple
//              of 8 (every workload here) the order below keeps all tiles of
//              a tile row on one XCD and close in time, and that L2 merges
//              the stores into whole sectors: WRITE_SIZE of a stress call is
//              within 1.4% of the algorithmic bytes (an earlier order showed
//              each store as a 32-byte write, and a staged layout with a
//              second, transposing kernel was slower than this).
//   * caching: the input and the outputs are touched once, and how their
//              lines travel through the L2 and the 256 MB memory-side cache
//              decides the speed far more than the arithmetic does.  The tile
//              loads and every q_col store carry the non-temporal (streaming)
//              hint.  q_row stores carry it in the tile rows whose index mod 8
//              is set in row_stream_mask, the others are ordinary write-back
//              stores.  The host streams q_row in 6 of 8 tile rows when a call
//              moves more than twice the memory-side cache (the write-back
//              share is then too large for the cache to absorb) and in none
//              otherwise (the cache absorbs q_row and drains it while the
//              call still runs).  Measured on MI355X with rotating buffers:
//              the bf16 [32768, 8192] call runs in 193 us instead of 213 us
//              with ordinary accesses, [8192, 7168] in 43.5 us instead of 53.6.
//   * matrix-core scale layout (optional): both scale tensors written in
//              the order in which the scaled 16x16x128 matrix instruction
//              takes them, so a contraction reads one dword per lane and
//              128-wide step.  For an operand with R rows and kb = K/32 blocks
//              per row, scale (r, b) sits at byte
//                ((r/64 * kb/4 + b/4) * 64 + 16 (b%4) + r%16) * 4 + (r%64)/16,
//              i.e. a 64-row group and a 4-block step own 256 contiguous
//              bytes, one dword per lane.  s_row is the operand [M rows, N/32
//              blocks]; s_col belongs to q_col, the operand [N rows, M/32
//              blocks].  A tile owns exactly two such runs of each tensor, so
//              it stages its scale bytes in LDS and writes four 256-byte runs;
//              no second pass is needed.
//   * offsets: per-tile bases are uniform buffer resources and per-lane
//              offsets are 32-bit, which the host guarantees by limiting M, N
//              and the row pitch to 2^24.
#include "mxq_kernels.h"

#include <limits.h>

namespace mxq {
namespace {

constexpr int kTile = 128;
constexpr int kThreads = 512;
constexpr int kLoads = kTile * 16 / kThreads;   // 16-byte loads per thread (a tile is 2048 of them)
constexpr int kRowsPerLoad = kThreads / 16;     // tile rows one load round covers
constexpr double kMemorySideCacheBytes = 256.0 * 1024 * 1024;   // MI355X last-level (MALL) capacity

// How a call writes its scales.
constexpr int kScalesPlain = 0;    // s_row [M][N/32], s_col [M/32][N]
constexpr int kScalesMfma = 1;     // both tensors in the matrix-core layout

typedef short v2i16 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Cache-policy operand of the buffer instructions on gfx950: bit 0 sc0,
// bit 1 nt (non-temporal / streaming), bit 4 sc1.
constexpr int kPolicyDefault = 0;
constexpr int kPolicyStream = 2;

// Raw (untyped, stride 0) buffer resource over [base, base + 2^32 - 1).
// Word 3 selects the 32-bit data format, which CDNA needs for untyped
// accesses to be performed.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(0xFFFFFFFFu), 0x00020000);
}

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

// RCEIL scale byte from the largest sign-masked finite bf16 pattern a of a
// block.  448 = 1.75 * 2^8, so ceil(log2(A / 448)) = (e - 135) + [1.m > 1.75]
// for a normal A with exponent field e and fraction m; biased by 127 and
// clamped below at 0 (zero and tiny blocks).  Largest finite result: 247.
__device__ __forceinline__ uint32_t rceil_byte(uint32_t a) {
    const int b = int(a >> 7) - 8 + ((a & 0x7Fu) > 0x60u ? 1 : 0);
    return b > 0 ? uint32_t(b) : 0u;
}

// Rowwise scale: the 1x32 cast converts without saturation, so Inf as well
// as NaN makes the whole block NaN with scale 255.
__device__ __forceinline__ uint32_t row_scale(uint32_t a) {
    return a >= 0x7F80u ? 255u : rceil_byte(a);
}

// Colwise scale: NaN poisons (255); Inf without NaN saturates (254).
__device__ __forceinline__ uint32_t col_scale(uint32_t a) {
    return a > 0x7F80u ? 255u : (a == 0x7F80u ? 254u : rceil_byte(a));
}

// E8M0 byte as the fp32 scale operand of the scaled conversion.
__device__ __forceinline__ float e8m0_operand(uint32_t b) {
    return __uint_as_float((b < 254u ? b : 254u) << 23);
}

// Four bf16 (two packed pairs, in order) -> four E4M3 bytes, x / 2^(b-127).
__device__ __forceinline__ uint32_t cvt4(uint32_t pair01, uint32_t pair23, float scale) {
    v2i16 r = {0, 0};
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(v2bf16, pair01), scale, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(v2bf16, pair23), scale, true);
    return __builtin_bit_cast(uint32_t, r);
}

// In a colwise Inf block the only NaN bytes (0x7F / 0xFF) come from +-Inf;
// satfinite turns them into +-448 (0x7E / 0xFE).  Adding 1 to the low seven
// bits carries into bit 7 exactly for those bytes.
__device__ __forceinline__ uint32_t nan_bytes_to_max(uint32_t w) {
    const uint32_t t = (w & 0x7F7F7F7Fu) + 0x01010101u;
    return w - ((t & 0x80808080u) >> 7);
}

// Offset validation code of group g: bounds, then alignment, then order.
__device__ __forceinline__ int32_t offs_code(const int32_t* offs, int32_t g, int64_t M) {
    const int32_t o = offs[g];
    if (o < 0 || int64_t(o) > M) return 3;
    if (o % 128 != 0) return 2;
    if (g > 0 && o < offs[g - 1]) return 1;
    return 0;
}

// Whole workgroup: first invalid group's code (0 if none) into *err.
__device__ void validate_offsets(const int32_t* offs, int32_t G, int64_t M, int32_t* err) {
    __shared__ int32_t first_bad;
    if (threadIdx.x == 0) first_bad = INT_MAX;
    __syncthreads();
    for (int32_t g = threadIdx.x; g < G; g += kThreads)
        if (offs_code(offs, g, M) != 0) atomicMin(&first_bad, g);
    __syncthreads();
    if (threadIdx.x == 0) *err = first_bad == INT_MAX ? 0 : offs_code(offs, first_bad, M);
}

// XOR applied to the 16-byte chunk index of the tile rows of 16-row chunk c
// (0..7) in LDS: 2c | c/4.  A colwise dword read covers 4 column pairs of 8
// chunks per half wave; 2c spreads the chunks over bits 3..5 of the dword
// column and c/4 over bit 2, so the half wave's 32 dwords fall in 32 banks.
__device__ __forceinline__ uint32_t lds_chunk_xor(uint32_t c) {
    c &= 7u;
    return (c << 1) | (c >> 2);
}

// Byte of the tile's 512-byte staging run for local row r (0..127) and local
// block j (0..3) in the matrix-core scale layout: run r/64, then lane
// 16 j + r%16, byte (r%64)/16 of its dword.
__device__ __forceinline__ uint32_t mfma_scale_slot(uint32_t r, uint32_t j) {
    return (r >> 6) * 256u + (16u * j + (r & 15u)) * 4u + ((r >> 4) & 3u);
}

template <bool kGrouped, int kScales>
__global__ __launch_bounds__(kThreads)
void dual_axis_kernel(const uint16_t* __restrict__ x, int64_t ld_x, int64_t M, int64_t N,
                      uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
                      uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col,
                      uint32_t tiles_n, uint32_t tiles, uint32_t row_stream_mask, bool diagonal,
                      const int32_t* __restrict__ offs, int32_t G, int32_t* __restrict__ err) {
    __shared__ uint4 lds_tile[kTile * 16];     // [128 rows][16 x 16 bytes]
    __shared__ uint32_t lds_srow[kTile];       // the tile's 512 rowwise scale bytes
    __shared__ uint32_t lds_scol[kTile];       // the tile's 512 colwise scale bytes (either layout)

    const uint32_t t = threadIdx.x;
    const uint32_t bid = blockIdx.x;
    const uint32_t tiles_m = tiles / tiles_n;
    const uint32_t tm = bid % tiles_m;
    const uint32_t tn = diagonal ? (bid / tiles_m + tm) % tiles_n : bid / tiles_m;
    const int64_t m0 = int64_t(tm) * kTile;
    const int64_t n0 = int64_t(tn) * kTile;

    // first block row of the uncovered tail (grouped only)
    int64_t tail_br = M / 32;
    if (kGrouped) {
        if (G > 0) {
            int64_t last = offs[G - 1];
            last = last < 0 ? 0 : (last > M ? M : last);
            tail_br = last / 32;
        }
        if (err != nullptr && bid == 0) validate_offsets(offs, G, M, err);
    }

    // ---- load the tile: rows kRowsPerLoad * k + rsub, columns c8 .. c8+7 ----
    const uint32_t rsub = t >> 4;
    const uint32_t c8 = (t & 15u) * 8u;
    const __amdgpu_buffer_rsrc_t rx = raw_rsrc(x + m0 * ld_x + n0);
    const __amdgpu_buffer_rsrc_t rq_row = raw_rsrc(q_row + m0 * N + n0);
    const __amdgpu_buffer_rsrc_t rq_col = raw_rsrc(q_col + n0 * M + m0);
    const bool stream_row = ((row_stream_mask >> (tm & 7u)) & 1u) != 0u;
    const uint32_t ldb = uint32_t(ld_x) * 2u;          // row pitch in bytes (<= 2^25)
    uint4 d[kLoads];
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t(kRowsPerLoad) * k + rsub) * ldb + 2u * c8, 0,
                                                              kPolicyStream);
        d[k] = make_uint4(v.x, v.y, v.z, v.w);
    }

    // ---- rowwise 1x32 pass ----
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
        const uint32_t r = uint32_t(kRowsPerLoad) * k + rsub;
        lds_tile[r * 16u + ((t & 15u) ^ lds_chunk_xor(r >> 4))] = d[k];
        const uint32_t mx = pk_max_u16(pk_max_u16(d[k].x & 0x7FFF7FFFu, d[k].y & 0x7FFF7FFFu),
                                       pk_max_u16(d[k].z & 0x7FFF7FFFu, d[k].w & 0x7FFF7FFFu));
        uint32_t a = max(mx & 0xFFFFu, mx >> 16);
        a = max(a, uint32_t(__builtin_amdgcn_mov_dpp(int(a), 0xB1, 0xF, 0xF, true)));  // lane ^ 1
        a = max(a, uint32_t(__builtin_amdgcn_mov_dpp(int(a), 0x4E, 0xF, 0xF, true)));  // lane ^ 2
        const uint32_t b = row_scale(a);
        const float sc = e8m0_operand(b);
        u32x2 o;
        o.x = cvt4(d[k].x, d[k].y, sc);
        o.y = cvt4(d[k].z, d[k].w, sc);
        if (b == 255u) o.x = o.y = 0x7F7F7F7Fu;
        const uint32_t off = r * uint32_t(N) + c8;
        if (stream_row) __builtin_amdgcn_raw_buffer_store_b64(o, rq_row, off, 0, kPolicyStream);
        else __builtin_amdgcn_raw_buffer_store_b64(o, rq_row, off, 0, kPolicyDefault);
        if ((t & 3u) == 0u) {
            const uint32_t j = (t & 15u) >> 2;
            reinterpret_cast<uint8_t*>(lds_srow)[kScales == kScalesMfma ? mfma_scale_slot(r, j) : r * 4u + j] = uint8_t(b);
        }
    }
    __syncthreads();

    if (kScales == kScalesMfma) {
        // runs (2 tm + h) * tiles_n + tn of the [M rows, N/32 blocks] operand, h = 0, 1
        if (t < 32) {
            const int64_t run = (2 * int64_t(tm) + (t >> 4)) * tiles_n + tn;
            *reinterpret_cast<uint4*>(s_row + run * 256 + 16 * (t & 15u)) = reinterpret_cast<const uint4*>(lds_srow)[t];
        }
    } else if (t < kTile) {
        *reinterpret_cast<uint32_t*>(s_row + (m0 + t) * (N / 32) + n0 / 32) = lds_srow[t];
    }

    // ---- colwise 32x1 pass ----
    // Unit = (column pair cp, 16-row chunk c); each thread takes one unit.
    // Eight lanes share a column pair and hold its eight chunks, so each
    // 16-byte store of a column lands in one full 128-byte line per 8 lanes.
    // The two chunks of a 32-row block sit in lanes l, l^1 (one DPP step).
    const uint32_t lane = t & 63u, wave = t >> 6;
    const uint32_t c = lane & 7u;
    const uint32_t* lt = reinterpret_cast<const uint32_t*>(lds_tile);
    {
        const uint32_t cp = ((lane >> 3) & 7u) + 8u * wave;
        const uint32_t* src = lt + (16u * c) * 64u + (cp ^ (4u * lds_chunk_xor(c)));
        uint32_t v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = src[i * 64];
        uint32_t cm = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) cm = pk_max_u16(cm, v[i] & 0x7FFF7FFFu);
        cm = pk_max_u16(cm, uint32_t(__builtin_amdgcn_mov_dpp(int(cm), 0xB1, 0xF, 0xF, true)));  // lane ^ 1
        const uint32_t b_lo = col_scale(cm & 0xFFFFu);
        const uint32_t b_hi = col_scale(cm >> 16);
        const float s_lo = e8m0_operand(b_lo), s_hi = e8m0_operand(b_hi);
        uint32_t w_lo[4], w_hi[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t lo01 = __builtin_amdgcn_perm(v[4 * q + 1], v[4 * q], 0x05040100u);
            const uint32_t hi01 = __builtin_amdgcn_perm(v[4 * q + 1], v[4 * q], 0x07060302u);
            const uint32_t lo23 = __builtin_amdgcn_perm(v[4 * q + 3], v[4 * q + 2], 0x05040100u);
            const uint32_t hi23 = __builtin_amdgcn_perm(v[4 * q + 3], v[4 * q + 2], 0x07060302u);
            w_lo[q] = cvt4(lo01, lo23, s_lo);
            w_hi[q] = cvt4(hi01, hi23, s_hi);
        }
        if (__any(b_lo >= 254u || b_hi >= 254u)) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                w_lo[q] = b_lo == 255u ? 0x7F7F7F7Fu : nan_bytes_to_max(w_lo[q]);
                w_hi[q] = b_hi == 255u ? 0x7F7F7F7Fu : nan_bytes_to_max(w_hi[q]);
            }
        }
        const uint32_t off = 2u * cp * uint32_t(M) + 16u * c;   // q_col row n0 + 2cp, column m0 + 16c
        const u32x4 lo = {w_lo[0], w_lo[1], w_lo[2], w_lo[3]};
        const u32x4 hi = {w_hi[0], w_hi[1], w_hi[2], w_hi[3]};
        __builtin_amdgcn_raw_buffer_store_b128(lo, rq_col, off, 0, kPolicyStream);
        __builtin_amdgcn_raw_buffer_store_b128(hi, rq_col, off + uint32_t(M), 0, kPolicyStream);
        if ((c & 1u) == 0u) {
            const int64_t sbr = m0 / 32 + (c >> 1);
            const bool tail = kGrouped && sbr >= tail_br;
            if (kScales == kScalesMfma) {
                uint8_t* ls = reinterpret_cast<uint8_t*>(lds_scol);
                ls[mfma_scale_slot(2u * cp, c >> 1)] = tail ? uint8_t(0) : uint8_t(b_lo);
                ls[mfma_scale_slot(2u * cp + 1u, c >> 1)] = tail ? uint8_t(0) : uint8_t(b_hi);
            } else {
                // block row c/2 of the tile, columns 2 cp and 2 cp + 1
                reinterpret_cast<uint16_t*>(lds_scol)[(c >> 1) * 64u + cp] =
                    tail ? uint16_t(0) : uint16_t(b_lo | (b_hi << 8));
            }
        }
    }
    __syncthreads();
    if (t < 32) {
        const uint4 piece = reinterpret_cast<const uint4*>(lds_scol)[t];
        if (kScales == kScalesMfma) {
            // runs (2 tn + h) * tiles_m + tm of the [N rows, M/32 blocks] operand
            const int64_t run = (2 * int64_t(tn) + (t >> 4)) * tiles_m + tm;
            *reinterpret_cast<uint4*>(s_col + run * 256 + 16 * (t & 15u)) = piece;
        } else {
            // block row m0/32 + t/8, bytes n0 + 16 (t%8) .. + 15
            *reinterpret_cast<uint4*>(s_col + (m0 / 32 + (t >> 3)) * N + n0 + 16 * (t & 7u)) = piece;
        }
    }
}

__global__ __launch_bounds__(kThreads)
void offs_validate_kernel(const int32_t* __restrict__ offs, int32_t G, int64_t M, int32_t* __restrict__ err) {
    validate_offsets(offs, G, M, err);
}

}  // namespace

hipError_t launch_dual_axis(const uint16_t* x, int64_t M, int64_t N, int64_t ld_x,
                            uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                            const int32_t* offs, int32_t G, int32_t* err, bool grouped,
                            bool mfma_scales, hipStream_t stream) {
    const uint32_t tiles_n = uint32_t(N / kTile);
    const uint32_t tiles = uint32_t((M / kTile) * (N / kTile));
    const int scales = mfma_scales ? kScalesMfma : kScalesPlain;
    // q_row streaming share by the call's size against the memory-side cache
    const double call_bytes = 4.0625 * double(M) * double(N);
    const bool large = call_bytes > 2.0 * kMemorySideCacheBytes;
    const uint32_t row_stream = large ? 0x3Fu : 0x00u;
    if (!grouped) {
        offs = nullptr;
        G = 0;
        err = nullptr;
    }
    const dim3 grid(tiles), block(kThreads);
#define MXQ_LAUNCH(GR, SC)                                                                                   \
    hipLaunchKernelGGL((dual_axis_kernel<GR, SC>), grid, block, 0, stream, x, ld_x, M, N, q_row, s_row, q_col, \
                       s_col, tiles_n, tiles, row_stream, large, offs, G, err)
    if (grouped) {
        if (scales == kScalesMfma) MXQ_LAUNCH(true, kScalesMfma);
        else MXQ_LAUNCH(true, kScalesPlain);
    } else {
        if (scales == kScalesMfma) MXQ_LAUNCH(false, kScalesMfma);
        else MXQ_LAUNCH(false, kScalesPlain);
    }
#undef MXQ_LAUNCH
    return hipGetLastError();
}

hipError_t launch_offs_validate(const int32_t* offs, int32_t G, int64_t M, int32_t* err,
                                hipStream_t stream) {
    hipLaunchKernelGGL(offs_validate_kernel, dim3(1), dim3(kThreads), 0, stream, offs, G, M, err);
    return hipGetLastError();
}

}  // namespace mxq
