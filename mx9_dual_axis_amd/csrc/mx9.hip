// mx9.hip -- MX9 pack / unpack for gfx950 (CDNA4).
//
// Format: AMD-AGI/ALTO PR #33, "feat: mx9: add fused MX9 quantization kernel
// with pack/unpack" (Summary, Key design choices).  Blocks of 16 along the
// last axis; q int8 in [-127, 127]; max_exp an E8M0 byte (true exponent +
// 127, true exponent read from the input's own exponent field and clamped at
// -126); prime one bit per pair of elements, set when the pair lies wholly
// below 2^E and uses the finer grid 2^(E-7).
//
// Contiguous inputs (row pitch == cols, cols % 16 == 0) take the flat
// kernels: a block is split over 2 lanes (bf16) or 4 lanes (fp32) so that
// every wave-wide load and store is one contiguous range, and the block's
// exponent maximum and prime bits are combined with DPP.  Strided or ragged
// inputs take one thread per block.  bf16 inputs are widened exactly to fp32
// bit patterns (bf16 is the upper half of binary32), so one code path serves
// both input types.  The quotient x / 2^(E-6-p) is rounded half-to-even
// in one fused multiply-add with 1.5 * 2^23 (its reciprocal is a normal
// float for every block whose exponent byte is at least 9; smaller blocks
// form it exactly with v_ldexp_f32), and clamped with one median.  A lane of
// the flat pack issues eight (large calls) or four 16-byte loads before it
// quantizes any of them.
//
// Cache policy of the flat kernels (each byte is touched once): the pack
// reads its input and writes q with the non-temporal hint, the unpack writes
// its output with it.  Measured on MI355X, ordinary write-back stores of the
// bulk streams leave the memory-side cache full of dirty lines that the next
// kernel pays for: in the sequence cast -> pack -> unpack the streaming
// policy brings the step from 5.59 to 5.85 TB/s and the cast after it from
// 206 to 196 us, and the unpack alone from 0.65-0.68 to 0.84 of peak.  The
// pack's max_exp and prime bytes (1/16 of its output each) are the
// exception: ordinary stores, which the cache merges into whole lines, are
// faster in that sequence than streaming single bytes.
#include "mxq_kernels.h"
#include "mx9_codec.h"

namespace mxq {
namespace {

using namespace mx9;

constexpr int kThreads = 256;



// Where the per-block kernels put block j of row r: q bytes at
// q + r * ld_q + 16 j (ld_q a multiple of 16), the exponent byte at
// max_exp + r * ld_e + j, the prime byte at prime + r * ld_pr + j.  The
// contiguous three-part form is ld_q = 16 * blocks_per_row, ld_e = ld_pr =
// blocks_per_row.
struct Mx9Pitch {
    int64_t q, e, pr;
};

// Vector path: cols % 16 == 0 and 16-byte aligned block starts.
template <int kDtype>
__global__ __launch_bounds__(kThreads)
void mx9_pack_vec(const void* __restrict__ xv, int64_t ld_x, uint32_t blocks_per_row, uint64_t nb,
                  int8_t* __restrict__ q, uint8_t* __restrict__ max_exp, uint8_t* __restrict__ prime,
                  Mx9Pitch ld) {
    const uint64_t blk = uint64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (blk >= nb) return;
    const uint64_t row = blk / blocks_per_row;
    const uint64_t jb = blk - row * blocks_per_row;
    const uint64_t col = jb * 16;
    uint32_t w[16];
    if (kDtype == 0) {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint32_t*>(xv) + row * ld_x + col);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint4 d = src[k];
            w[4 * k] = d.x; w[4 * k + 1] = d.y; w[4 * k + 2] = d.z; w[4 * k + 3] = d.w;
        }
    } else {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xv) + row * ld_x + col);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const uint4 d = src[k];
            const uint32_t dd[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w[8 * k + 2 * i] = dd[i] << 16;
                w[8 * k + 2 * i + 1] = dd[i] & 0xFFFF0000u;
            }
        }
    }
    uint32_t qd[4], me, pr;
    pack16(w, qd, me, pr);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(q) + row * ld.q + col) = make_uint4(qd[0], qd[1], qd[2], qd[3]);
    max_exp[row * ld.e + jb] = uint8_t(me);
    prime[row * ld.pr + jb] = uint8_t(pr);
}

// General path: any cols (trailing partial block padded with +0), any ld_x.
template <int kDtype>
__global__ __launch_bounds__(kThreads)
void mx9_pack_any(const void* __restrict__ xv, int64_t ld_x, int64_t cols, uint32_t blocks_per_row,
                  uint64_t nb, int8_t* __restrict__ q, uint8_t* __restrict__ max_exp,
                  uint8_t* __restrict__ prime, Mx9Pitch ld) {
    const uint64_t blk = uint64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (blk >= nb) return;
    const uint64_t row = blk / blocks_per_row;
    const uint64_t jb = blk - row * blocks_per_row;
    const int64_t col = int64_t(jb) * 16;
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t c = col + i;
        if (c < cols) {
            if (kDtype == 0) w[i] = static_cast<const uint32_t*>(xv)[row * ld_x + c];
            else w[i] = uint32_t(static_cast<const uint16_t*>(xv)[row * ld_x + c]) << 16;
        } else {
            w[i] = 0u;
        }
    }
    uint32_t qd[4], me, pr;
    pack16(w, qd, me, pr);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(q) + row * ld.q + jb * 16) = make_uint4(qd[0], qd[1], qd[2], qd[3]);
    max_exp[row * ld.e + jb] = uint8_t(me);
    prime[row * ld.pr + jb] = uint8_t(pr);
}

// ---------------------------------------------------------------------------
// Flat paths: the input is one contiguous run of nb blocks (ld == cols and
// cols % 16 == 0).  A block is shared by L = 16 * esz / 16 lanes (2 for bf16,
// 4 for fp32) that each hold one 16-byte piece, so every wave-wide load and
// store covers a contiguous range.  The block's exponent maximum and its
// prime bits are combined across the L lanes with DPP quad permutes.
// ---------------------------------------------------------------------------

// Groups of 64 / kLanes blocks (one wave-wide 1 KiB load) that one wave of
// the flat pack takes; their loads are all issued before the first group is
// quantized.  Eight groups when that still leaves kPackWideMinWgs workgroups,
// four otherwise (fewer, longer workgroups leave a larger share of the last
// round idle).  Measured on MI355X: bf16 [32768, 8192] 127 us with eight, 129
// us with four; the [4096, 14336] weights 47.5 us (fp32) and 29.9 us (bf16)
// with four, 49.5 us and 31.0 us with eight.
constexpr uint64_t kPackWideMinWgs = 8192;

// Quantize one loaded 16-byte piece (this lane's share of block blk) and store
// its outputs: q with the non-temporal hint, the max_exp and prime bytes with
// ordinary write-back stores (the cache merges the wave's 1-byte stores).
template <int kDtype>
__device__ __forceinline__ void pack_piece_store(uint4 d, uint64_t blk, uint32_t part, int8_t* __restrict__ q,
                                                 uint8_t* __restrict__ max_exp, uint8_t* __restrict__ prime) {
    using P = FlatPiece<kDtype>;
    const P r = pack_flat_piece<kDtype>(d, part);
    uint8_t* qb = reinterpret_cast<uint8_t*>(q) + blk * 16 + part * P::kElems;
    typedef unsigned int u2 __attribute__((ext_vector_type(2)));
    if (P::kElems == 8) __builtin_nontemporal_store(u2{r.qd[0], r.qd[1]}, reinterpret_cast<u2*>(qb));
    else __builtin_nontemporal_store(r.qd[0], reinterpret_cast<uint32_t*>(qb));
    if (part == 0) max_exp[blk] = uint8_t(r.S);
    if (part == 1) prime[blk] = uint8_t(r.prime);
}

// kDtype 0: fp32, 4 lanes x 4 elements per block.  1: bf16, 2 lanes x 8.
// Each wave owns kPackGroups groups of 64 / kLanes consecutive blocks; group k
// is one contiguous 1 KiB load.  A lane issues its kPackGroups streaming loads
// before it quantizes anything, so a wave keeps up to 8 KiB of reads in flight.
// Measured on MI355X (bf16 [32768, 8192], rotating buffers): one group per
// wave 157 us, two 133 us, eight 127 us; in the cast -> pack -> unpack
// sequence the step went from 471 us to 452 us.  Streaming the max_exp and
// prime bytes as well costs 4% (one group) to 7% (two groups) in the step.
template <int kDtype, int kPackGroups>
__global__ __launch_bounds__(kThreads)
void mx9_pack_flat(const void* __restrict__ xv, uint64_t nb, int8_t* __restrict__ q,
                   uint8_t* __restrict__ max_exp, uint8_t* __restrict__ prime) {
    constexpr int kLanes = kDtype == 0 ? 4 : 2;
    constexpr uint32_t kGroup = 64 / kLanes;
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t part = lane % kLanes;
    const uint64_t blk0 = (uint64_t(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6)) * (kPackGroups * kGroup);
    const u4* src = reinterpret_cast<const u4*>(xv) + blk0 * kLanes + lane;
    if (blk0 + kPackGroups * kGroup <= nb) {
        u4 v[kPackGroups];
#pragma unroll
        for (int k = 0; k < kPackGroups; ++k) v[k] = __builtin_nontemporal_load(src + k * 64);
#pragma unroll
        for (int k = 0; k < kPackGroups; ++k)
            pack_piece_store<kDtype>(make_uint4(v[k].x, v[k].y, v[k].z, v[k].w), blk0 + k * kGroup + lane / kLanes,
                                     part, q, max_exp, prime);
    } else {
        // the last wave: groups past nb are skipped, a partial group is guarded per block
        for (int k = 0; k < kPackGroups; ++k) {
            const uint64_t blk = blk0 + k * kGroup + lane / kLanes;
            if (blk0 + k * kGroup >= nb) break;
            uint4 d = make_uint4(0u, 0u, 0u, 0u);
            if (blk < nb) {
                const u4 v = __builtin_nontemporal_load(src + k * 64);
                d = make_uint4(v.x, v.y, v.z, v.w);
            }
            // every lane of the wave takes part in the DPP combines; only live blocks store
            using P = FlatPiece<kDtype>;
            const P r = pack_flat_piece<kDtype>(d, part);
            if (blk < nb) {
                uint8_t* qb = reinterpret_cast<uint8_t*>(q) + blk * 16 + part * P::kElems;
                typedef unsigned int u2 __attribute__((ext_vector_type(2)));
                if (P::kElems == 8) __builtin_nontemporal_store(u2{r.qd[0], r.qd[1]}, reinterpret_cast<u2*>(qb));
                else __builtin_nontemporal_store(r.qd[0], reinterpret_cast<uint32_t*>(qb));
                if (part == 0) max_exp[blk] = uint8_t(r.S);
                if (part == 1) prime[blk] = uint8_t(r.prime);
            }
        }
    }
}

// kOut 0: fp32 output, 4 lanes x 4 elements per block.  1: bf16, 2 lanes x 8.
template <int kOut>
__global__ __launch_bounds__(kThreads)
void mx9_unpack_flat(const int8_t* __restrict__ q, const uint8_t* __restrict__ max_exp,
                     const uint8_t* __restrict__ prime, uint64_t nb, void* __restrict__ yv) {
    constexpr int kLanes = kOut == 0 ? 4 : 2;
    constexpr int kElems = 16 / kLanes;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t part = lane % kLanes;
    const uint64_t wave_blk0 = (uint64_t(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6)) * 64;
#pragma unroll
    for (int k = 0; k < kLanes; ++k) {
        const uint64_t blk = wave_blk0 + uint64_t(k) * (64 / kLanes) + lane / kLanes;
        if (blk >= nb) continue;
        const uint8_t* qb = reinterpret_cast<const uint8_t*>(q) + blk * 16 + part * kElems;
        uint32_t qd[2];
        if (kElems == 8) { const uint2 t2 = *reinterpret_cast<const uint2*>(qb); qd[0] = t2.x; qd[1] = t2.y; }
        else { qd[0] = *reinterpret_cast<const uint32_t*>(qb); qd[1] = 0u; }
        const uint32_t S = max_exp[blk];
        const uint32_t pr = uint32_t(prime[blk]) >> ((kElems / 2) * part);
        float y[kElems];
#pragma unroll
        for (int i = 0; i < kElems; ++i) {
            const int qi = int(int8_t(uint8_t(qd[i >> 2] >> (8 * (i & 3)))));
            const int p = int((pr >> (i >> 1)) & 1u);
            y[i] = __builtin_ldexpf(float(qi), int(S) - 133 - p);
        }
        if (kOut == 0) {
            float4 o = make_float4(y[0], y[1], y[2], y[3]);
            if (S == 255u) o = make_float4(__uint_as_float(0x7FC00000u), __uint_as_float(0x7FC00000u),
                                           __uint_as_float(0x7FC00000u), __uint_as_float(0x7FC00000u));
            store_out16(reinterpret_cast<float4*>(yv) + blk * 4 + part, make_uint4(__float_as_uint(o.x), __float_as_uint(o.y), __float_as_uint(o.z), __float_as_uint(o.w)));
        } else {
            uint4 o = make_uint4(bf16_pair(y[0], y[1]), bf16_pair(y[2], y[3]), bf16_pair(y[4], y[5]), bf16_pair(y[6], y[7]));
            if (S == 255u) o = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
            store_out16(reinterpret_cast<uint4*>(yv) + blk * 2 + part, o);
        }
    }
}

template <int kOut, bool kVec>
__global__ __launch_bounds__(kThreads)
void mx9_unpack_kernel(const int8_t* __restrict__ q, const uint8_t* __restrict__ max_exp,
                       const uint8_t* __restrict__ prime, int64_t cols, uint32_t blocks_per_row,
                       uint64_t nb, void* __restrict__ yv, int64_t ld_y, Mx9Pitch ld) {
    const uint64_t blk = uint64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (blk >= nb) return;
    const uint64_t row = blk / blocks_per_row;
    const uint64_t jb = blk - row * blocks_per_row;
    const int64_t col = int64_t(jb) * 16;
    const uint4 qv = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(q) + row * ld.q + jb * 16);
    const uint32_t S = max_exp[row * ld.e + jb];
    const uint32_t pr = prime[row * ld.pr + jb];
    float y[16];
    unpack16(qv, S, pr, y);
    if (kOut == 0) {
        float* dst = static_cast<float*>(yv) + row * ld_y + col;
        if (kVec) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                reinterpret_cast<float4*>(dst)[k] = make_float4(y[4 * k], y[4 * k + 1], y[4 * k + 2], y[4 * k + 3]);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (col + i < cols) dst[i] = y[i];
        }
    } else {
        uint32_t h[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) h[k] = bf16_pair(y[2 * k], y[2 * k + 1]);
        if (S == 255u) {
#pragma unroll
            for (int k = 0; k < 8; ++k) h[k] = 0x7FC07FC0u;
        }
        uint16_t* dst = static_cast<uint16_t*>(yv) + row * ld_y + col;
        if (kVec) {
            reinterpret_cast<uint4*>(dst)[0] = make_uint4(h[0], h[1], h[2], h[3]);
            reinterpret_cast<uint4*>(dst)[1] = make_uint4(h[4], h[5], h[6], h[7]);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (col + i < cols) dst[i] = uint16_t(h[i >> 1] >> (16 * (i & 1)));
        }
    }
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

hipError_t launch_mx9_pack(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                           int8_t* q, int64_t ld_q, uint8_t* max_exp, int64_t ld_e, uint8_t* prime,
                           int64_t ld_pr, hipStream_t stream) {
    const int64_t esz = dtype == 0 ? 4 : 2;
    const uint32_t bpr = uint32_t((cols + 15) / 16);
    const uint64_t nb = uint64_t(rows) * bpr;
    const dim3 grid(uint32_t((nb + kThreads - 1) / kThreads));
    const bool vec = cols % 16 == 0 && aligned16(x) && (ld_x * esz) % 16 == 0;
    const bool packed_out = (ld_q == 16 * int64_t(bpr) && ld_e == int64_t(bpr) && ld_pr == int64_t(bpr)) || rows == 1;
    const Mx9Pitch ld{ld_q, ld_e, ld_pr};
    if (vec && ld_x == cols && aligned16(q) && packed_out) {
        // groups * 64 / kLanes blocks per wave, 4 waves per workgroup
        const uint64_t per_group_wg = uint64_t(kThreads / 64) * (dtype == 0 ? 16 : 32);
        const bool wide = (nb + 8 * per_group_wg - 1) / (8 * per_group_wg) >= kPackWideMinWgs;
        const uint64_t per_wg = per_group_wg * (wide ? 8 : 4);
        const dim3 fgrid(uint32_t((nb + per_wg - 1) / per_wg));
        if (dtype == 0) {
            if (wide) hipLaunchKernelGGL((mx9_pack_flat<0, 8>), fgrid, dim3(kThreads), 0, stream, x, nb, q, max_exp, prime);
            else hipLaunchKernelGGL((mx9_pack_flat<0, 4>), fgrid, dim3(kThreads), 0, stream, x, nb, q, max_exp, prime);
        } else {
            if (wide) hipLaunchKernelGGL((mx9_pack_flat<1, 8>), fgrid, dim3(kThreads), 0, stream, x, nb, q, max_exp, prime);
            else hipLaunchKernelGGL((mx9_pack_flat<1, 4>), fgrid, dim3(kThreads), 0, stream, x, nb, q, max_exp, prime);
        }
        return hipGetLastError();
    }
    if (dtype == 0) {
        if (vec) hipLaunchKernelGGL(mx9_pack_vec<0>, grid, dim3(kThreads), 0, stream, x, ld_x, bpr, nb, q, max_exp, prime, ld);
        else hipLaunchKernelGGL(mx9_pack_any<0>, grid, dim3(kThreads), 0, stream, x, ld_x, cols, bpr, nb, q, max_exp, prime, ld);
    } else {
        if (vec) hipLaunchKernelGGL(mx9_pack_vec<1>, grid, dim3(kThreads), 0, stream, x, ld_x, bpr, nb, q, max_exp, prime, ld);
        else hipLaunchKernelGGL(mx9_pack_any<1>, grid, dim3(kThreads), 0, stream, x, ld_x, cols, bpr, nb, q, max_exp, prime, ld);
    }
    return hipGetLastError();
}

hipError_t launch_mx9_unpack(const int8_t* q, int64_t ld_q, const uint8_t* max_exp, int64_t ld_e,
                             const uint8_t* prime, int64_t ld_pr, int64_t rows, int64_t cols, int out_dtype,
                             void* y, int64_t ld_y, hipStream_t stream) {
    const int64_t esz = out_dtype == 0 ? 4 : 2;
    const uint32_t bpr = uint32_t((cols + 15) / 16);
    const uint64_t nb = uint64_t(rows) * bpr;
    const dim3 grid(uint32_t((nb + kThreads - 1) / kThreads));
    const bool vec = cols % 16 == 0 && aligned16(y) && (ld_y * esz) % 16 == 0;
    const bool packed_in = (ld_q == 16 * int64_t(bpr) && ld_e == int64_t(bpr) && ld_pr == int64_t(bpr)) || rows == 1;
    const Mx9Pitch ld{ld_q, ld_e, ld_pr};
    if (vec && ld_y == cols && aligned16(q) && packed_in) {
        const dim3 fgrid(uint32_t((nb + 255) / 256));
        if (out_dtype == 0) hipLaunchKernelGGL(mx9_unpack_flat<0>, fgrid, dim3(kThreads), 0, stream, q, max_exp, prime, nb, y);
        else hipLaunchKernelGGL(mx9_unpack_flat<1>, fgrid, dim3(kThreads), 0, stream, q, max_exp, prime, nb, y);
        return hipGetLastError();
    }
    if (out_dtype == 0) {
        if (vec) hipLaunchKernelGGL((mx9_unpack_kernel<0, true>), grid, dim3(kThreads), 0, stream, q, max_exp, prime, cols, bpr, nb, y, ld_y, ld);
        else hipLaunchKernelGGL((mx9_unpack_kernel<0, false>), grid, dim3(kThreads), 0, stream, q, max_exp, prime, cols, bpr, nb, y, ld_y, ld);
    } else {
        if (vec) hipLaunchKernelGGL((mx9_unpack_kernel<1, true>), grid, dim3(kThreads), 0, stream, q, max_exp, prime, cols, bpr, nb, y, ld_y, ld);
        else hipLaunchKernelGGL((mx9_unpack_kernel<1, false>), grid, dim3(kThreads), 0, stream, q, max_exp, prime, cols, bpr, nb, y, ld_y, ld);
    }
    return hipGetLastError();
}

}  // namespace mxq
