// roof.hip -- measurement helpers for the benchmark (not part of the
// quantization path and not part of libmxq.so's C ABI).
//
// The benchmark reports the dual-axis cast against MI355X's published HBM
// peak and, for context, against what the same GPU achieves for a plain
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

// The three streams of the dual-axis cast, each alone, with the cast's tile
// order and per-lane accesses (one 512-thread workgroup per 128 x 128 tile;
// a call that moves more than twice the memory-side cache visits the tiles
// diagonally, each tile row shifted one tile column):
//   stream 0: the tiled read of the bf16 input, rows of 256 bytes at pitch 2N;
//   stream 1: the q_row write, rows of 128 bytes at pitch N, 8 bytes per lane;
//   stream 2: the q_col write, rows of 128 bytes at pitch M, 16 bytes per lane.
// The cast's time against the sum of these three separates the cost of its
// access pattern from the cost of combining the streams in one kernel.
__device__ __forceinline__ void tile_of(uint32_t bid, uint32_t tiles_m, uint32_t tiles_n, bool diagonal, uint32_t& tm,
                                        uint32_t& tn) {
    tm = bid % tiles_m;
    tn = diagonal ? (bid / tiles_m + tm) % tiles_n : bid / tiles_m;
}

__global__ __launch_bounds__(512) void stream_x_read(const uint8_t* __restrict__ x, int64_t N, uint32_t tiles_m,
                                                     uint32_t tiles_n, bool diagonal, u4* __restrict__ sink) {
    uint32_t tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, diagonal, tm, tn);
    const uint32_t t = threadIdx.x;
    const uint8_t* base = x + (uint64_t(tm) * 128 * uint64_t(N) + uint64_t(tn) * 128) * 2;
    u4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 4; ++k)
        acc ^= __builtin_nontemporal_load(reinterpret_cast<const u4*>(base + uint64_t(32 * k + (t >> 4)) * 2 * N) + (t & 15u));
    if ((acc.x & acc.y & acc.z & acc.w) == 0xFFFFFFFFu && t == 0) sink[blockIdx.x & 255u] = acc;
}

__global__ __launch_bounds__(512) void stream_q_row(uint8_t* __restrict__ q, int64_t N, uint32_t tiles_m,
                                                    uint32_t tiles_n, bool diagonal) {
    typedef unsigned int u2 __attribute__((ext_vector_type(2)));
    uint32_t tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, diagonal, tm, tn);
    const uint32_t t = threadIdx.x;
    uint8_t* base = q + uint64_t(tm) * 128 * uint64_t(N) + uint64_t(tn) * 128;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        __builtin_nontemporal_store(u2{t, uint32_t(k)}, reinterpret_cast<u2*>(base + uint64_t(32 * k + (t >> 4)) * N) + (t & 15u));
}

__global__ __launch_bounds__(512) void stream_q_col(uint8_t* __restrict__ q, int64_t M, uint32_t tiles_m,
                                                    uint32_t tiles_n, bool diagonal) {
    uint32_t tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, diagonal, tm, tn);
    const uint32_t t = threadIdx.x, lane = t & 63u, c = lane & 7u;
    const uint32_t cp = ((lane >> 3) & 7u) + 8u * (t >> 6);
    uint8_t* base = q + uint64_t(tn) * 128 * uint64_t(M) + uint64_t(tm) * 128;
    u4* lo = reinterpret_cast<u4*>(base + uint64_t(2 * cp) * M + 16 * c);
    u4* hi = reinterpret_cast<u4*>(base + uint64_t(2 * cp + 1) * M + 16 * c);
    __builtin_nontemporal_store(u4{t, 1u, 2u, 3u}, lo);
    __builtin_nontemporal_store(u4{t, 4u, 5u, 6u}, hi);
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

// One stream of the dual-axis cast on an [M, N] problem (M, N positive
// multiples of 128 below 2^24): stream 0 reads buf as the bf16 input [M, N]
// (sink receives at most 4 KiB, only for all-ones data), 1 writes buf as
// q_row [M, N], 2 writes buf as q_col [N, M].  The tile order is the cast's
// for this size.  Returns 0, -1 for invalid arguments, or the launch's HIP error.
int mxq_roof_cast_stream(int stream_id, void* buf, void* sink, int64_t M, int64_t N, void* stream) {
    if (M <= 0 || N <= 0 || M % 128 != 0 || N % 128 != 0 || M >= (int64_t(1) << 24) || N >= (int64_t(1) << 24)) return -1;
    if (!buf || reinterpret_cast<uintptr_t>(buf) % 16 != 0 || (stream_id == 0 && !sink)) return -1;
    const uint64_t tiles = uint64_t(M / 128) * uint64_t(N / 128);
    if (tiles * 512 > 0xFFFFFFFFull) return -1;
    const uint32_t tm = uint32_t(M / 128), tn = uint32_t(N / 128);
    const bool diagonal = 4.0625 * double(M) * double(N) > 2.0 * 256.0 * 1024 * 1024;
    const dim3 grid(static_cast<uint32_t>(tiles)), block(512);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (stream_id == 0)
        hipLaunchKernelGGL(stream_x_read, grid, block, 0, st, static_cast<const uint8_t*>(buf), N, tm, tn, diagonal,
                           static_cast<u4*>(sink));
    else if (stream_id == 1) hipLaunchKernelGGL(stream_q_row, grid, block, 0, st, static_cast<uint8_t*>(buf), N, tm, tn, diagonal);
    else if (stream_id == 2) hipLaunchKernelGGL(stream_q_col, grid, block, 0, st, static_cast<uint8_t*>(buf), M, tm, tn, diagonal);
    else return -1;
    return int(hipGetLastError());
}

}  // extern "C"
