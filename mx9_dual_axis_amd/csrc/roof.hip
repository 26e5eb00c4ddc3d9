// roof.hip -- measurement helpers for the benchmark (not part of the
// quantization path and not part of libmxq.so's C ABI).
//
// The benchmark reports the dual-axis cast against MI355X's published HBM
// peak and, for context, against what the same box achieves for a plain
// stream of the same byte volume.  These kernels are those streams, written
// for the access pattern that measured fastest on MI355X: each workgroup
// (4 waves) moves one 4 KiB chunk with one 16-byte non-temporal load and/or
// store per lane, and consecutive workgroups take consecutive chunks.  Since
// workgroups are dealt to the 8 XCDs in turn, XCD k then handles the chunks
// whose index is k mod 8; a copy with eight 16-byte loads per lane over
// contiguous 32 KiB per workgroup measured 4-14% slower (write streams most).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void roof_copy(const u4* __restrict__ src, u4* __restrict__ dst) {
    const uint64_t i = uint64_t(blockIdx.x) * 256 + threadIdx.x;
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(256) void roof_read(const u4* __restrict__ src, u4* __restrict__ sink) {
    const uint64_t i = uint64_t(blockIdx.x) * 256 + threadIdx.x;
    const u4 v = __builtin_nontemporal_load(src + i);
    // never true for the benchmark's zero-filled buffers, but keeps the load
    if ((v.x & v.y & v.z & v.w) == 0xFFFFFFFFu && threadIdx.x == 0) sink[blockIdx.x & 255u] = v;
}

__global__ __launch_bounds__(256) void roof_write(u4* __restrict__ dst) {
    const uint64_t i = uint64_t(blockIdx.x) * 256 + threadIdx.x;
    __builtin_nontemporal_store(u4{uint32_t(i), blockIdx.x, threadIdx.x, 0u}, dst + i);
}

}  // namespace

extern "C" {

// kind 0: copy `bytes` from src to dst; 1: read `bytes` of src (dst receives
// at most 4 KiB, and only for all-ones data); 2: write `bytes` to dst.
// bytes must be a positive multiple of 4096 below 2^43 and the pointers
// 16-byte aligned.  Returns 0, -1 for invalid arguments, or the HIP error of
// the launch.  Enqueued on `stream`.
int mxq_roof(int kind, const void* src, void* dst, int64_t bytes, void* stream) {
    if (bytes <= 0 || bytes % 4096 != 0 || bytes >= (int64_t(1) << 43)) return -1;
    if ((kind != 2 && (!src || reinterpret_cast<uintptr_t>(src) % 16 != 0)) || !dst ||
        reinterpret_cast<uintptr_t>(dst) % 16 != 0)
        return -1;
    const dim3 grid(uint32_t(bytes / 4096)), block(256);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (kind == 0) hipLaunchKernelGGL(roof_copy, grid, block, 0, st, static_cast<const u4*>(src), static_cast<u4*>(dst));
    else if (kind == 1) hipLaunchKernelGGL(roof_read, grid, block, 0, st, static_cast<const u4*>(src), static_cast<u4*>(dst));
    else if (kind == 2) hipLaunchKernelGGL(roof_write, grid, block, 0, st, static_cast<u4*>(dst));
    else return -1;
    return int(hipGetLastError());
}

}  // extern "C"
