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
// both input types.  The quotient x / 2^(E-6-p) is formed with v_ldexp_f32,
// exact because the divisor is a power of two and |quotient| < 2^8, then
// rounded half-to-even by v_rndne_f32; fp32 denormals are kept (no flush),
// so subnormal inputs quantize exactly.
#include "mxq_kernels.h"

namespace mxq {
namespace {

constexpr int kThreads = 256;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));


// round-half-even(x * 2^shift) clamped to [-127, 127], returned in the low
// byte of the result (two's complement).  |x * 2^shift| < 2^8 for every
// element of a block, and ldexp is exact there.  Clamping to +-127 before
// rounding equals clamping after (the bounds are integers).  Adding 1.5*2^23
// rounds half-to-even to an integer held in the low mantissa bits, whose low
// byte is the two's-complement int8 of the rounded value.
__device__ __forceinline__ uint32_t qbits(uint32_t w, int shift) {
    float t = __builtin_ldexpf(__uint_as_float(w), shift);
    t = __builtin_fminf(__builtin_fmaxf(t, -127.0f), 127.0f);
    return __float_as_uint(t + 12582912.0f);
}

// Low bytes of four qbits results -> one dword, element a in byte 0.
__device__ __forceinline__ uint32_t pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0C0C0400u);
    const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0C0C0400u);
    return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// Quantize pairs of fp32 patterns against the block's shared exponent byte S.
// A pair is demoted (p = 1) when its larger magnitude is below 2^(S-127),
// i.e. when its larger magnitude pattern is below S << 23 (magnitudes and
// their bit patterns order alike).  Returns the q bytes of kPairs pairs in
// kPairs / 2 dwords and the pair bits in *bits (LSB = first pair).
template <int kPairs>
__device__ __forceinline__ void quantize_pairs(const uint32_t (&w)[2 * kPairs], uint32_t S,
                                               uint32_t (&qd)[kPairs / 2], uint32_t& bits) {
    uint32_t qb[2 * kPairs];
    bits = 0;
#pragma unroll
    for (int j = 0; j < kPairs; ++j) {
        const uint32_t pm = max(w[2 * j] & 0x7FFFFFFFu, w[2 * j + 1] & 0x7FFFFFFFu);
        const uint32_t p = pm < (S << 23) ? 1u : 0u;
        bits |= p << j;
        const int shift = 133 + int(p) - int(S);          // 6 + p - E, E = S - 127
        qb[2 * j] = qbits(w[2 * j], shift);
        qb[2 * j + 1] = qbits(w[2 * j + 1], shift);
    }
#pragma unroll
    for (int k = 0; k < kPairs / 2; ++k) qd[k] = pack4(qb[4 * k], qb[4 * k + 1], qb[4 * k + 2], qb[4 * k + 3]);
}

// Largest magnitude pattern of n fp32 patterns (NaN > Inf > finite).
template <int kN>
__device__ __forceinline__ uint32_t max_magnitude(const uint32_t (&w)[kN]) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < kN; ++i) m = max(m, w[i] & 0x7FFFFFFFu);
    return m;
}

// Pack 16 fp32 patterns: q bytes (4 dwords), max_exp byte, prime byte.
// The shared exponent byte is the largest exponent field raised to >= 1;
// an Inf or NaN (exponent field 255) poisons the block.
__device__ __forceinline__ void pack16(const uint32_t (&w)[16], uint32_t (&qd)[4], uint32_t& me,
                                       uint32_t& pr) {
    const uint32_t mmax = max_magnitude(w);
    const uint32_t S = max(mmax >> 23, 1u);
    quantize_pairs<8>(w, S, qd, pr);
    me = S;
    if (mmax >= 0x7F800000u) {          // Inf or NaN: poisoned block
        qd[0] = qd[1] = qd[2] = qd[3] = 0u;
        me = 255u;
        pr = 0u;
    }
}

// Vector path: cols % 16 == 0 and 16-byte aligned block starts.
template <int kDtype>
__global__ __launch_bounds__(kThreads)
void mx9_pack_vec(const void* __restrict__ xv, int64_t ld_x, uint32_t blocks_per_row, uint64_t nb,
                  int8_t* __restrict__ q, uint8_t* __restrict__ max_exp, uint8_t* __restrict__ prime) {
    const uint64_t blk = uint64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (blk >= nb) return;
    const uint64_t row = blk / blocks_per_row;
    const uint64_t col = (blk - row * blocks_per_row) * 16;
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
    reinterpret_cast<uint4*>(q)[blk] = make_uint4(qd[0], qd[1], qd[2], qd[3]);
    max_exp[blk] = uint8_t(me);
    prime[blk] = uint8_t(pr);
}

// General path: any cols (trailing partial block padded with +0), any ld_x.
template <int kDtype>
__global__ __launch_bounds__(kThreads)
void mx9_pack_any(const void* __restrict__ xv, int64_t ld_x, int64_t cols, uint32_t blocks_per_row,
                  uint64_t nb, int8_t* __restrict__ q, uint8_t* __restrict__ max_exp,
                  uint8_t* __restrict__ prime) {
    const uint64_t blk = uint64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (blk >= nb) return;
    const uint64_t row = blk / blocks_per_row;
    const int64_t col = int64_t(blk - row * blocks_per_row) * 16;
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
    reinterpret_cast<uint4*>(q)[blk] = make_uint4(qd[0], qd[1], qd[2], qd[3]);
    max_exp[blk] = uint8_t(me);
    prime[blk] = uint8_t(pr);
}

// Unpack one block to 16 fp32 values: q * 2^(S - 133 - p); S == 255 -> NaN.
__device__ __forceinline__ void unpack16(uint4 qv, uint32_t S, uint32_t pr, float (&y)[16]) {
    const uint32_t qd[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int qi = int(int8_t(uint8_t(qd[i >> 2] >> (8 * (i & 3)))));
        const int p = int((pr >> (i >> 1)) & 1u);
        y[i] = __builtin_ldexpf(float(qi), int(S) - 133 - p);
    }
    if (S == 255u) {
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] = __uint_as_float(0x7FC00000u);
    }
}

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
    const bf16x2 r = {__bf16(lo), __bf16(hi)};
    return __builtin_bit_cast(uint32_t, r);
}

// ---------------------------------------------------------------------------
// Flat paths: the input is one contiguous run of nb blocks (ld == cols and
// cols % 16 == 0).  A block is shared by L = 16 * esz / 16 lanes (2 for bf16,
// 4 for fp32) that each hold one 16-byte piece, so every wave-wide load and
// store covers a contiguous range.  The block's exponent maximum and its
// prime bits are combined across the L lanes with DPP quad permutes.
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) {
    return uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) {
    return uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x4E, 0xF, 0xF, true));
}

// One pass of the flat pack: this lane's 16-byte piece of block blk.
template <int kDtype, bool kGuard>
__device__ __forceinline__ void pack_piece(const void* __restrict__ xv, uint64_t nb, uint64_t blk,
                                           uint32_t part, int8_t* __restrict__ q,
                                           uint8_t* __restrict__ max_exp, uint8_t* __restrict__ prime) {
    constexpr int kLanes = kDtype == 0 ? 4 : 2;          // lanes per block
    constexpr int kElems = 16 / kLanes;                   // elements per lane
    const bool live = !kGuard || blk < nb;
    uint32_t w[kElems];
    uint4 d = make_uint4(0u, 0u, 0u, 0u);
    if (live) d = reinterpret_cast<const uint4*>(xv)[blk * kLanes + part];
    if (kDtype == 0) {
        w[0] = d.x; w[1] = d.y; w[2] = d.z; w[3] = d.w;
    } else {
        const uint32_t dd[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) { w[2 * i] = dd[i] << 16; w[2 * i + 1] = dd[i] & 0xFFFF0000u; }
    }
    uint32_t mmax = max_magnitude(w);
    mmax = max(mmax, dpp_xor1(mmax));
    if (kLanes == 4) mmax = max(mmax, dpp_xor2(mmax));
    const uint32_t S = max(mmax >> 23, 1u);
    uint32_t qd[kElems / 4], bits;
    quantize_pairs<kElems / 2>(w, S, qd, bits);
    // the block's prime byte: this lane's pairs start at bit (kElems / 2) * part
    uint32_t pr = bits << ((kElems / 2) * part);
    pr |= dpp_xor1(pr);
    if (kLanes == 4) pr |= dpp_xor2(pr);
    const bool poison = mmax >= 0x7F800000u;
    if (live) {
        uint8_t* qb = reinterpret_cast<uint8_t*>(q) + blk * 16 + part * kElems;
        if (kElems == 8) *reinterpret_cast<uint2*>(qb) = poison ? make_uint2(0u, 0u) : make_uint2(qd[0], qd[1]);
        else *reinterpret_cast<uint32_t*>(qb) = poison ? 0u : qd[0];
        if (part == 0) max_exp[blk] = uint8_t(poison ? 255u : S);
        if (part == 1) prime[blk] = uint8_t(poison ? 0u : pr);
    }
}

// kDtype 0: fp32, 4 lanes x 4 elements per block.  1: bf16, 2 lanes x 8.
// Each wave owns 64 / kLanes consecutive blocks: one contiguous 1 KiB load.
template <int kDtype>
__global__ __launch_bounds__(kThreads)
void mx9_pack_flat(const void* __restrict__ xv, uint64_t nb, int8_t* __restrict__ q,
                   uint8_t* __restrict__ max_exp, uint8_t* __restrict__ prime) {
    constexpr int kLanes = kDtype == 0 ? 4 : 2;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t part = lane % kLanes;
    const uint64_t wave_blk0 = (uint64_t(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6)) * (64 / kLanes);
    if (wave_blk0 + 64 / kLanes <= nb)
        pack_piece<kDtype, false>(xv, nb, wave_blk0 + lane / kLanes, part, q, max_exp, prime);
    else
        pack_piece<kDtype, true>(xv, nb, wave_blk0 + lane / kLanes, part, q, max_exp, prime);
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
            reinterpret_cast<float4*>(yv)[blk * 4 + part] = o;
        } else {
            uint4 o = make_uint4(bf16_pair(y[0], y[1]), bf16_pair(y[2], y[3]), bf16_pair(y[4], y[5]), bf16_pair(y[6], y[7]));
            if (S == 255u) o = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
            reinterpret_cast<uint4*>(yv)[blk * 2 + part] = o;
        }
    }
}

template <int kOut, bool kVec>
__global__ __launch_bounds__(kThreads)
void mx9_unpack_kernel(const int8_t* __restrict__ q, const uint8_t* __restrict__ max_exp,
                       const uint8_t* __restrict__ prime, int64_t cols, uint32_t blocks_per_row,
                       uint64_t nb, void* __restrict__ yv, int64_t ld_y) {
    const uint64_t blk = uint64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (blk >= nb) return;
    const uint64_t row = blk / blocks_per_row;
    const int64_t col = int64_t(blk - row * blocks_per_row) * 16;
    const uint4 qv = reinterpret_cast<const uint4*>(q)[blk];
    const uint32_t S = max_exp[blk];
    const uint32_t pr = prime[blk];
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
                           int8_t* q, uint8_t* max_exp, uint8_t* prime, hipStream_t stream) {
    const int64_t esz = dtype == 0 ? 4 : 2;
    const uint32_t bpr = uint32_t((cols + 15) / 16);
    const uint64_t nb = uint64_t(rows) * bpr;
    const dim3 grid(uint32_t((nb + kThreads - 1) / kThreads));
    const bool vec = cols % 16 == 0 && aligned16(x) && (ld_x * esz) % 16 == 0;
    if (vec && ld_x == cols && aligned16(q)) {
        // 64 / kLanes blocks per wave, 4 waves per workgroup
        const dim3 fgrid(uint32_t((nb + (dtype == 0 ? 63 : 127)) / (dtype == 0 ? 64 : 128)));
        if (dtype == 0) hipLaunchKernelGGL(mx9_pack_flat<0>, fgrid, dim3(kThreads), 0, stream, x, nb, q, max_exp, prime);
        else hipLaunchKernelGGL(mx9_pack_flat<1>, fgrid, dim3(kThreads), 0, stream, x, nb, q, max_exp, prime);
        return hipGetLastError();
    }
    if (dtype == 0) {
        if (vec) hipLaunchKernelGGL(mx9_pack_vec<0>, grid, dim3(kThreads), 0, stream, x, ld_x, bpr, nb, q, max_exp, prime);
        else hipLaunchKernelGGL(mx9_pack_any<0>, grid, dim3(kThreads), 0, stream, x, ld_x, cols, bpr, nb, q, max_exp, prime);
    } else {
        if (vec) hipLaunchKernelGGL(mx9_pack_vec<1>, grid, dim3(kThreads), 0, stream, x, ld_x, bpr, nb, q, max_exp, prime);
        else hipLaunchKernelGGL(mx9_pack_any<1>, grid, dim3(kThreads), 0, stream, x, ld_x, cols, bpr, nb, q, max_exp, prime);
    }
    return hipGetLastError();
}

hipError_t launch_mx9_unpack(const int8_t* q, const uint8_t* max_exp, const uint8_t* prime,
                             int64_t rows, int64_t cols, int out_dtype, void* y, int64_t ld_y,
                             hipStream_t stream) {
    const int64_t esz = out_dtype == 0 ? 4 : 2;
    const uint32_t bpr = uint32_t((cols + 15) / 16);
    const uint64_t nb = uint64_t(rows) * bpr;
    const dim3 grid(uint32_t((nb + kThreads - 1) / kThreads));
    const bool vec = cols % 16 == 0 && aligned16(y) && (ld_y * esz) % 16 == 0;
    if (vec && ld_y == cols && aligned16(q)) {
        const dim3 fgrid(uint32_t((nb + 255) / 256));
        if (out_dtype == 0) hipLaunchKernelGGL(mx9_unpack_flat<0>, fgrid, dim3(kThreads), 0, stream, q, max_exp, prime, nb, y);
        else hipLaunchKernelGGL(mx9_unpack_flat<1>, fgrid, dim3(kThreads), 0, stream, q, max_exp, prime, nb, y);
        return hipGetLastError();
    }
    if (out_dtype == 0) {
        if (vec) hipLaunchKernelGGL((mx9_unpack_kernel<0, true>), grid, dim3(kThreads), 0, stream, q, max_exp, prime, cols, bpr, nb, y, ld_y);
        else hipLaunchKernelGGL((mx9_unpack_kernel<0, false>), grid, dim3(kThreads), 0, stream, q, max_exp, prime, cols, bpr, nb, y, ld_y);
    } else {
        if (vec) hipLaunchKernelGGL((mx9_unpack_kernel<1, true>), grid, dim3(kThreads), 0, stream, q, max_exp, prime, cols, bpr, nb, y, ld_y);
        else hipLaunchKernelGGL((mx9_unpack_kernel<1, false>), grid, dim3(kThreads), 0, stream, q, max_exp, prime, cols, bpr, nb, y, ld_y);
    }
    return hipGetLastError();
}

}  // namespace mxq
