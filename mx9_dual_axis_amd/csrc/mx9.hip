// mx9.hip -- MX9 pack / unpack for gfx950 (CDNA4).
//
// Format: AMD-AGI/ALTO PR #33, "feat: mx9: add fused MX9 quantization kernel
// with pack/unpack" (Summary, Key design choices).  Blocks of 16 along the
// last axis; q int8 in [-127, 127]; max_exp an E8M0 byte (true exponent +
// 127, true exponent read from the input's own exponent field and clamped at
// -126); prime one bit per pair of elements, set when the pair lies wholly
// below 2^E and uses the finer grid 2^(E-7).
//
// One thread per block of 16.  bf16 inputs are widened exactly to fp32 bit
// patterns (bf16 is the upper half of binary32), so one code path serves
// both input types.  The quotient x / 2^(E-6-p) is formed with v_ldexp_f32,
// exact because the divisor is a power of two and |quotient| < 2^8, then
// rounded half-to-even by v_rndne_f32; fp32 denormals are kept (no flush),
// so subnormal inputs quantize exactly.
#include "mxq_kernels.h"

namespace mxq {
namespace {

constexpr int kThreads = 256;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t efield(uint32_t w) { return (w >> 23) & 0xFFu; }

__device__ __forceinline__ uint32_t qbyte(uint32_t w, int shift) {
    int q = int(__builtin_rintf(__builtin_ldexpf(__uint_as_float(w), shift)));
    q = q < -127 ? -127 : (q > 127 ? 127 : q);
    return uint32_t(q) & 0xFFu;
}

// Pack 16 fp32 patterns: q bytes (4 dwords), max_exp byte, prime byte.
__device__ __forceinline__ void pack16(const uint32_t (&w)[16], uint32_t (&qd)[4], uint32_t& me,
                                       uint32_t& pr) {
    uint32_t ef[16];
    uint32_t emax = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        ef[i] = efield(w[i]);
        emax = max(emax, ef[i]);
    }
    if (emax == 255u) {                 // Inf or NaN: poisoned block
        qd[0] = qd[1] = qd[2] = qd[3] = 0u;
        me = 255u;
        pr = 0u;
        return;
    }
    const uint32_t S = max(emax, 1u);
    uint32_t bits = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t p = max(ef[2 * j], ef[2 * j + 1]) < S ? 1u : 0u;
        bits |= p << j;
        const int shift = 133 + int(p) - int(S);          // 6 + p - E, E = S - 127
        const uint32_t pair = qbyte(w[2 * j], shift) | (qbyte(w[2 * j + 1], shift) << 8);
        if (j & 1) qd[j >> 1] |= pair << 16;
        else qd[j >> 1] = pair;
    }
    me = S;
    pr = bits;
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
