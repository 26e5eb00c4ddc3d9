// scale_layout.hip -- conversion between plain E8M0 scale views and the
// matrix-core scale layout.
//
// The matrix-core layout is the order in which v_mfma_scale_f32_16x16x128
// takes its scale operand (the layout the _mfma casts emit and the _mfma
// contractions read; the pages' cast likewise emits its consumer's swizzled
// layout directly, pytorch/ao PR #4995, description).  For an operand of R
// rows and kb blocks per row, scale (r, b) is the byte
//     ((r/64 * kb/4 + b/4) * 64 + 16 (b%4) + r%16) * 4 + (r%64)/16,
// i.e. dword i (run i / 64, lane L = i % 64) holds in byte q the scale of row
// 64 g + 16 q + L % 16 and block 4 t + L / 16, where run = g * kb/4 + t.
//
// One thread per dword: the forward conversion gathers four bytes from the
// strided view and writes the dword (a wave writes 256 contiguous bytes);
// the inverse reads the dword and scatters its bytes.
#include "mxq_kernels.h"

namespace mxq {
namespace {

constexpr int kThreads = 256;

struct ScaleView {
    int64_t rs, bs;        // strides of the plain view, in bytes
    uint64_t runs_per_group;   // kb / 4
    uint64_t dwords;       // rows * kb / 4
};

__device__ __forceinline__ void dword_coords(const ScaleView& v, uint64_t i, int64_t& r0, int64_t& b) {
    const uint64_t run = i >> 6, lane = i & 63u;
    const uint64_t grp = run / v.runs_per_group, step = run - grp * v.runs_per_group;
    r0 = int64_t(64 * grp + (lane & 15u));          // row of byte 0; byte q adds 16 q
    b = int64_t(4 * step + (lane >> 4));
}

__global__ __launch_bounds__(kThreads)
void scales_to_mfma_kernel(const uint8_t* __restrict__ s, ScaleView v, uint32_t* __restrict__ out) {
    const uint64_t i = uint64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (i >= v.dwords) return;
    int64_t r0, b;
    dword_coords(v, i, r0, b);
    const uint8_t* p = s + r0 * v.rs + b * v.bs;
    const int64_t step16 = 16 * v.rs;
    out[i] = uint32_t(p[0]) | (uint32_t(p[step16]) << 8) | (uint32_t(p[2 * step16]) << 16) |
             (uint32_t(p[3 * step16]) << 24);
}

__global__ __launch_bounds__(kThreads)
void scales_from_mfma_kernel(const uint32_t* __restrict__ in, ScaleView v, uint8_t* __restrict__ s) {
    const uint64_t i = uint64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (i >= v.dwords) return;
    int64_t r0, b;
    dword_coords(v, i, r0, b);
    const uint32_t d = in[i];
    uint8_t* p = s + r0 * v.rs + b * v.bs;
    const int64_t step16 = 16 * v.rs;
    p[0] = uint8_t(d);
    p[step16] = uint8_t(d >> 8);
    p[2 * step16] = uint8_t(d >> 16);
    p[3 * step16] = uint8_t(d >> 24);
}

ScaleView make_scale_view(int64_t rows, int64_t blocks, int64_t rs, int64_t bs) {
    ScaleView v;
    v.rs = rs;
    v.bs = bs;
    v.runs_per_group = uint64_t(blocks / 4);
    v.dwords = uint64_t(rows) * uint64_t(blocks) / 4;
    return v;
}

}  // namespace

hipError_t launch_scales_to_mfma(const uint8_t* s, int64_t rs, int64_t bs, int64_t rows, int64_t blocks, uint8_t* out,
                                 hipStream_t stream) {
    const ScaleView v = make_scale_view(rows, blocks, rs, bs);
    const dim3 grid(uint32_t((v.dwords + kThreads - 1) / kThreads));
    hipLaunchKernelGGL(scales_to_mfma_kernel, grid, dim3(kThreads), 0, stream, s, v, reinterpret_cast<uint32_t*>(out));
    return hipGetLastError();
}

hipError_t launch_scales_from_mfma(const uint8_t* in, int64_t rows, int64_t blocks, uint8_t* s, int64_t rs, int64_t bs,
                                   hipStream_t stream) {
    const ScaleView v = make_scale_view(rows, blocks, rs, bs);
    const dim3 grid(uint32_t((v.dwords + kThreads - 1) / kThreads));
    hipLaunchKernelGGL(scales_from_mfma_kernel, grid, dim3(kThreads), 0, stream, reinterpret_cast<const uint32_t*>(in),
                       v, s);
    return hipGetLastError();
}

}  // namespace mxq
