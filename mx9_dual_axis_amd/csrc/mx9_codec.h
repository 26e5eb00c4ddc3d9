// mx9_codec.h -- the MX9 block codec shared by the MX9 kernels (device code).
//
// Format: AMD-AGI/ALTO PR #33, "feat: mx9: add fused MX9 quantization kernel
// with pack/unpack" (Summary, Key design choices).  A block is 16 values; its
// shared exponent byte S is the largest exponent field of the block raised to
// at least 1 (true exponent E = S - 127 >= -126); the pair bit of elements
// (2j, 2j+1) is set when both lie below 2^E, and the pair is then quantized
// on the grid 2^(E-7) instead of 2^(E-6); q = round-half-even(x / grid)
// clamped to [-127, 127].  A block with Inf or NaN is poisoned: S = 255,
// q = 0, prime = 0, and it unpacks to NaN.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {
namespace mx9 {

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

// round-half-even(x * scale) clamped to [-127, 127] in the low byte, for a
// power-of-two scale.  The fused multiply-add forms x * scale + 1.5 * 2^23
// exactly and rounds it once; |x * scale| < 2^8, so the sum lies in
// [2^23, 2^24), where floats are the integers, and the rounding is the
// half-even rounding of x * scale (1.5 * 2^23 is even).  The median then
// clamps the integer to 1.5 * 2^23 +- 127.
__device__ __forceinline__ uint32_t qbits_scaled(uint32_t w, float scale) {
    const float t = __builtin_fmaf(__uint_as_float(w), scale, 12582912.0f);
    return __float_as_uint(__builtin_amdgcn_fmed3f(t, 12582785.0f, 12583039.0f));
}

// Quantize pairs of fp32 patterns against the block's shared exponent byte S.
// A pair is demoted (p = 1) when its larger magnitude is below 2^(S-127),
// i.e. when its larger magnitude pattern is below S << 23 (magnitudes and
// their bit patterns order alike).  Returns the q bytes of kPairs pairs in
// kPairs / 2 dwords and the pair bits in *bits (LSB = first pair).
//
// The grid's reciprocal is 2^(133 + p - S).  For S >= 9 it is a normal float
// (at most 2^125) and the quantization is one fused multiply-add and one
// median per element; an element below the smallest normal then has
// |x * scale| < 1/2 and rounds to 0 whether or not the hardware keeps it
// subnormal.  Blocks with S < 9 (largest magnitude below 2^-118) take the
// exact ldexp route.
template <int kPairs>
__device__ __forceinline__ void quantize_pairs(const uint32_t (&w)[2 * kPairs], uint32_t S,
                                               uint32_t (&qd)[kPairs / 2], uint32_t& bits) {
    uint32_t qb[2 * kPairs];
    bits = 0;
    const uint32_t thr = S << 23;
    if (S >= 9u) {
        const uint32_t base = (260u - S) << 23;        // 2^(133 - S) as a float pattern
#pragma unroll
        for (int j = 0; j < kPairs; ++j) {
            const uint32_t pm = max(w[2 * j] & 0x7FFFFFFFu, w[2 * j + 1] & 0x7FFFFFFFu);
            const uint32_t p = (pm - thr) >> 31;        // pm < thr; both are below 2^31
            bits |= p << j;
            const float scale = __uint_as_float(base + (p << 23));
            qb[2 * j] = qbits_scaled(w[2 * j], scale);
            qb[2 * j + 1] = qbits_scaled(w[2 * j + 1], scale);
        }
    } else {
#pragma unroll
        for (int j = 0; j < kPairs; ++j) {
            const uint32_t pm = max(w[2 * j] & 0x7FFFFFFFu, w[2 * j + 1] & 0x7FFFFFFFu);
            const uint32_t p = pm < thr ? 1u : 0u;
            bits |= p << j;
            const int shift = 133 + int(p) - int(S);      // 6 + p - E, E = S - 127
            qb[2 * j] = qbits(w[2 * j], shift);
            qb[2 * j + 1] = qbits(w[2 * j + 1], shift);
        }
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

// A 16-byte piece of unpacked output, written with the non-temporal hint:
// the output is touched once, and ordinary write-back lines left in the
// memory-side cache slow the kernel that runs next (measured on MI355X).
__device__ __forceinline__ void store_out16(void* p, uint4 v) {
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(u4{v.x, v.y, v.z, v.w}, reinterpret_cast<u4*>(p));
}

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
    const bf16x2 r = {__bf16(lo), __bf16(hi)};
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) {
    return uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) {
    return uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x4E, 0xF, 0xF, true));
}

// One lane's share of a block in the flat layout: kLanes adjacent lanes of
// a wave (4 for fp32, 2 for bf16) hold one block, each a 16-byte piece of 16 /
// kLanes elements.  Returns the lane's q bytes, and the block's exponent byte
// S and prime byte (identical in all kLanes lanes); a block holding Inf or
// NaN comes back poisoned (S = 255, q = 0, prime = 0).
template <int kDtype>
struct FlatPiece {
    static constexpr int kLanes = kDtype == 0 ? 4 : 2;
    static constexpr int kElems = 16 / kLanes;
    uint32_t qd[kElems / 4];
    uint32_t S;
    uint32_t prime;
};

template <int kDtype>
__device__ __forceinline__ FlatPiece<kDtype> pack_flat_piece(uint4 d, uint32_t part) {
    using P = FlatPiece<kDtype>;
    constexpr int kLanes = P::kLanes, kElems = P::kElems;
    uint32_t w[kElems];
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
    P r;
    r.S = max(mmax >> 23, 1u);
    uint32_t bits;
    quantize_pairs<kElems / 2>(w, r.S, r.qd, bits);
    // the block's prime byte: this lane's pairs start at bit (kElems / 2) * part
    uint32_t pr = bits << ((kElems / 2) * part);
    pr |= dpp_xor1(pr);
    if (kLanes == 4) pr |= dpp_xor2(pr);
    r.prime = pr;
    if (mmax >= 0x7F800000u) {          // Inf or NaN: poisoned block
#pragma unroll
        for (int k = 0; k < kElems / 4; ++k) r.qd[k] = 0u;
        r.S = 255u;
        r.prime = 0u;
    }
    return r;
}

// Unpack kElems consecutive q bytes (qd[0] holds the first four) whose pair
// bits start at bit 0 of pr: q * 2^(S - 133 - p).  S == 255 is handled by the
// caller (the block unpacks to NaN).
template <int kElems>
__device__ __forceinline__ void unpack_piece(const uint32_t (&qd)[2], uint32_t S, uint32_t pr, float (&y)[kElems]) {
#pragma unroll
    for (int i = 0; i < kElems; ++i) {
        const int qi = int(int8_t(uint8_t(qd[i >> 2] >> (8 * (i & 3)))));
        const int p = int((pr >> (i >> 1)) & 1u);
        y[i] = __builtin_ldexpf(float(qi), int(S) - 133 - p);
    }
}

}  // namespace mx9
}  // namespace mxq
