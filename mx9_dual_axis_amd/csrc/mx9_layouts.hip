// mx9_layouts.hip -- MX9 along any axis and in the single-byte-tensor form,
// for gfx950 (CDNA4).
//
// Format and calls: AMD-AGI/ALTO PR #33, "feat: mx9: add fused MX9
// quantization kernel with pack/unpack": the calls take an axis argument and
// do not store the shape or the axis (the caller passes them back), and the
// commit "refactor: mx: pack mx9 into a single uint8 tensor" stores each
// block as one record that starts with its exponent byte (the kernel writes
// it at blk * N_PACKED_BYTES).  Readings taken here: the axis is moved last
// before blocking, so block (o, i, j) of a contiguous [outer, len, inner]
// array covers x[o][16j .. 16j+15][i] and is numbered (o * inner + i) * nbl
// + j with nbl = ceil(len / 16); a record is 18 bytes: the exponent byte,
// q[0..15], then the prime byte; records of one (o, i) form a row, and rows
// sit at a caller-given pitch.
//
// Kernels:
//   * flat records: contiguous input blocks and contiguous records.  The
//     lanes hold blocks exactly as the flat three-part pack does (a block
//     over 2 lanes for bf16, 4 for fp32; every wave-wide load is one
//     contiguous range).  A wave of the pack takes 64 contiguous blocks (two
//     groups of 32 for bf16, four of 16 for fp32) and issues all their loads
//     first; its records are assembled in the wave's own slice of LDS with
//     16-bit writes and written as 16-byte chunks, so the 18-byte records
//     cost no unaligned global stores.  The unpack stages a workgroup's records the same way.
//   * axis tiles (inner > 1): a workgroup takes 64 consecutive inner
//     positions i of one o and 32 consecutive blocks j (128 and 16 when the
//     inner extent is even: a lane then takes two adjacent i, so one 32-bit
//     load carries two bf16 elements and one 64-bit load two fp32).  The 64
//     lanes of a wave take consecutive i, so every load instruction reads a
//     contiguous run of the inner axis.  The tile's outputs are staged in
//     LDS (rows padded so the column-wise writes do not collide in the banks)
//     and written row by row: each (o, i) receives 512 contiguous q bytes
//     (576 record bytes) and 32 max_exp and prime bytes (256, 288 and 16 with
//     two positions per lane), so q lines are never assembled from pieces of
//     different workgroups.  The unpack reads a tile's rows the same way and
//     writes each element row of the tile as one contiguous run of the inner
//     axis.
//   * strided (inner == 1): records with a pitch or a ragged row, one thread
//     per block.
#include <algorithm>

#include "mxq_kernels.h"
#include "mx9_codec.h"

namespace mxq {
namespace {

using namespace mx9;

constexpr int kThreads = 256;
constexpr int kRec = 18;          // bytes per block record: exponent, q[16], prime

__device__ __forceinline__ uint32_t load_bits(const void* xv, uint64_t idx, int dtype) {
    return dtype == 0 ? static_cast<const uint32_t*>(xv)[idx]
                      : uint32_t(static_cast<const uint16_t*>(xv)[idx]) << 16;
}

// ---------------------------------------------------------------------------
// Flat records
// ---------------------------------------------------------------------------

// Groups of 64 / kLanes blocks (one wave-wide 1 KiB load) that one wave of
// the flat record pack takes: four for fp32, two for bf16, so that a wave's
// records are 64 blocks, 1,152 bytes, either way.  A wave's blocks are
// contiguous, so are its records, and it stages them in its own slice of
// LDS: no workgroup barrier.  Measured on MI355X for the [4096, 14336]
// weights (byte-identical output): one workgroup-wide stage of 8 x 256
// lanes' blocks 58-60 us (fp32) and 32.5-32.8 us (bf16); per-wave stages of
// 4 groups 54.4 us and 30.1 us; with the 16-bit staging below, 2, 4 and 8
// groups took 50.2, 49.8 and 50.3-50.9 us (fp32) and 30.5, 31.0-31.1 and
// 32.0-32.2 us (bf16).
template <int kDtype>
constexpr int kRecGroups = kDtype == 0 ? 4 : 2;

// Stage one lane's share of a record as 16-bit LDS writes.  A record starts
// at an even LDS offset, so its bytes pair up as (exponent, q0), (q1, q2),
// ..., (q15, prime): pair m holds q[2m - 1] and q[2m].  The lane holding
// q[e0 .. e0 + kE - 1] (e0 = kE * part) writes pairs kE/2 * part ..
// kE/2 * (part + 1) - 1, whose first byte is the last q byte of the lane
// below (the exponent for part 0), and the last lane adds (q15, prime).
// Measured on MI355X for the [4096, 14336] weights, byte-identical output:
// 57.3 -> 49.3 us (fp32) and 31.8 -> 31.3 us (bf16) against byte writes.
template <int kDtype>
__device__ __forceinline__ void stage_record_piece(uint8_t* rec, const FlatPiece<kDtype>& r, uint32_t part,
                                                   uint32_t below) {
    using P = FlatPiece<kDtype>;
    constexpr int kE = P::kElems;
    uint16_t* rec16 = reinterpret_cast<uint16_t*>(rec);
    const uint32_t first = part == 0 ? r.S : below;
#pragma unroll
    for (int h = 0; h < kE / 2; ++h) {
        const uint32_t lo = h == 0 ? first : (r.qd[(2 * h - 1) >> 2] >> (8 * ((2 * h - 1) & 3))) & 0xFFu;
        const uint32_t hi = (r.qd[(2 * h) >> 2] >> (8 * ((2 * h) & 3))) & 0xFFu;
        rec16[(kE / 2) * part + h] = uint16_t(lo | (hi << 8));
    }
    if (part == P::kLanes - 1) {
        const uint32_t last = (r.qd[(kE - 1) >> 2] >> (8 * ((kE - 1) & 3))) & 0xFFu;
        rec16[8] = uint16_t(last | (r.prime << 8));
    }
}

template <int kDtype>
__global__ __launch_bounds__(kThreads)
void mx9_pack_records_flat(const void* __restrict__ xv, uint64_t nb, uint8_t* __restrict__ packed) {
    using P = FlatPiece<kDtype>;
    constexpr int kGB = 64 / P::kLanes;                          // blocks per group (16 or 32)
    constexpr int kG = kRecGroups<kDtype>;
    constexpr int kWB = kG * kGB;                                // blocks per wave (64)
    constexpr int kBytes = kWB * kRec;                           // record bytes per wave (1152)
    static_assert(kBytes % 16 == 0, "a wave's records are whole 16-byte chunks");
    __shared__ uint4 stage[kThreads / 64][kBytes / 16];
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    uint8_t* st = reinterpret_cast<uint8_t*>(stage[wave]);
    const uint64_t blk0 = (uint64_t(blockIdx.x) * (kThreads / 64) + wave) * kWB;
    if (blk0 >= nb) return;                                      // uniform across the wave
    const uint32_t part = lane % P::kLanes, lb = lane / P::kLanes;
    const u4* src = reinterpret_cast<const u4*>(xv) + blk0 * P::kLanes + lane;
    u4 v[kG];
#pragma unroll
    for (int k = 0; k < kG; ++k) {
        v[k] = u4{0u, 0u, 0u, 0u};
        if (blk0 + k * kGB + lb < nb) v[k] = __builtin_nontemporal_load(src + k * 64);
    }
#pragma unroll
    for (int k = 0; k < kG; ++k) {
        const P r = pack_flat_piece<kDtype>(make_uint4(v[k].x, v[k].y, v[k].z, v[k].w), part);
        // the last q byte of the lane below (row_shr:1; lanes of a block are
        // adjacent and a block never spans two rows of 16 lanes)
        const uint32_t last = (r.qd[(P::kElems - 1) >> 2] >> (8 * ((P::kElems - 1) & 3))) & 0xFFu;
        const uint32_t below = uint32_t(__builtin_amdgcn_mov_dpp(int(last), 0x111, 0xF, 0xF, false));
        stage_record_piece<kDtype>(st + kRec * (k * kGB + lb), r, part, below);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);                         // lgkmcnt(0): the wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
    // the wave's records are one contiguous, 16-byte aligned range
    const uint32_t nbytes = uint32_t(nb - blk0 < uint64_t(kWB) ? nb - blk0 : uint64_t(kWB)) * kRec;
    uint8_t* out = packed + blk0 * kRec;
    for (uint32_t c = lane; c * 16u < nbytes; c += 64u) {
        if (c * 16u + 16u <= nbytes) {
            const uint4 w = stage[wave][c];
            __builtin_nontemporal_store(u4{w.x, w.y, w.z, w.w}, reinterpret_cast<u4*>(out) + c);
        } else {
            for (uint32_t b = c * 16u; b < nbytes; ++b) out[b] = st[b];
        }
    }
}

template <int kOut>
__global__ __launch_bounds__(kThreads)
void mx9_unpack_records_flat(const uint8_t* __restrict__ packed, uint64_t nb, void* __restrict__ yv) {
    constexpr int kLanes = kOut == 0 ? 4 : 2;
    constexpr int kElems = 16 / kLanes;
    constexpr int kBlocks = kThreads / kLanes;
    __shared__ uint4 stage[kBlocks * kRec / 16];
    uint8_t* st = reinterpret_cast<uint8_t*>(stage);
    const uint64_t blk0 = uint64_t(blockIdx.x) * kBlocks;
    const uint32_t nbytes = uint32_t(nb - blk0 < uint64_t(kBlocks) ? nb - blk0 : uint64_t(kBlocks)) * kRec;
    const uint8_t* in = packed + blk0 * kRec;
    for (uint32_t c = threadIdx.x; c * 16u < nbytes; c += kThreads) {
        if (c * 16u + 16u <= nbytes) {
            stage[c] = reinterpret_cast<const uint4*>(in)[c];
        } else {
            for (uint32_t b = c * 16u; b < nbytes; ++b) st[b] = in[b];
        }
    }
    __syncthreads();
    const uint32_t lb = threadIdx.x / kLanes, part = threadIdx.x % kLanes;
    const uint64_t blk = blk0 + lb;
    if (blk >= nb) return;
    const uint8_t* rec = st + kRec * lb;
    const uint32_t S = rec[0];
    const uint32_t pr = uint32_t(rec[kRec - 1]) >> ((kElems / 2) * part);
    uint32_t qd[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < kElems; ++k) qd[k >> 2] |= uint32_t(rec[1 + part * kElems + k]) << (8 * (k & 3));
    float y[kElems];
    unpack_piece<kElems>(qd, S, pr, y);
    if (kOut == 0) {
        float4 o = make_float4(y[0], y[1], y[2], y[3]);
        if (S == 255u) o = make_float4(__uint_as_float(0x7FC00000u), __uint_as_float(0x7FC00000u),
                                       __uint_as_float(0x7FC00000u), __uint_as_float(0x7FC00000u));
        store_out16(reinterpret_cast<float4*>(yv) + blk * kLanes + part, make_uint4(__float_as_uint(o.x), __float_as_uint(o.y), __float_as_uint(o.z), __float_as_uint(o.w)));
    } else {
        uint4 o = make_uint4(bf16_pair(y[0], y[1]), bf16_pair(y[2], y[3]), bf16_pair(y[4], y[5]), bf16_pair(y[6], y[7]));
        if (S == 255u) o = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
        store_out16(reinterpret_cast<uint4*>(yv) + blk * kLanes + part, o);
    }
}

// ---------------------------------------------------------------------------
// Strided: any [outer, len, inner] view, three-part or record output
// ---------------------------------------------------------------------------

struct StridedView {
    uint64_t outer, inner;
    int64_t len;
    uint32_t nbl;         // blocks per row, ceil(len / 16)
    uint32_t groups;      // ceil(nbl / kJ)
    uint64_t nthreads;    // outer * inner * groups
};

template <int kDtype, bool kRecords, int kJ>
__global__ __launch_bounds__(kThreads)
void mx9_pack_strided(const void* __restrict__ xv, StridedView v, int8_t* __restrict__ q,
                      uint8_t* __restrict__ max_exp, uint8_t* __restrict__ prime,
                      uint8_t* __restrict__ packed, int64_t ld_p) {
    const uint64_t t = uint64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (t >= v.nthreads) return;
    const uint64_t i = t % v.inner;
    const uint64_t rest = t / v.inner;
    const uint32_t g = uint32_t(rest % v.groups);
    const uint64_t o = rest / v.groups;
    const uint64_t row = o * v.inner + i;
    for (int jj = 0; jj < kJ; ++jj) {
        const uint32_t j = g * kJ + uint32_t(jj);
        if (j >= v.nbl) break;
        uint32_t w[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int64_t l = int64_t(16) * j + k;
            w[k] = l < v.len ? load_bits(xv, (o * uint64_t(v.len) + uint64_t(l)) * v.inner + i, kDtype) : 0u;
        }
        uint32_t qd[4], me, pr;
        pack16(w, qd, me, pr);
        if (kRecords) {
            uint8_t* rec = packed + row * uint64_t(ld_p) + uint64_t(kRec) * j;
            rec[0] = uint8_t(me);
#pragma unroll
            for (int k = 0; k < 16; ++k) rec[1 + k] = uint8_t(qd[k >> 2] >> (8 * (k & 3)));
            rec[kRec - 1] = uint8_t(pr);
        } else {
            const uint64_t blk = row * v.nbl + j;
            reinterpret_cast<uint4*>(q)[blk] = make_uint4(qd[0], qd[1], qd[2], qd[3]);
            max_exp[blk] = uint8_t(me);
            prime[blk] = uint8_t(pr);
        }
    }
}

template <int kOut, bool kRecords, int kJ>
__global__ __launch_bounds__(kThreads)
void mx9_unpack_strided(const int8_t* __restrict__ q, const uint8_t* __restrict__ max_exp,
                        const uint8_t* __restrict__ prime, const uint8_t* __restrict__ packed, int64_t ld_p,
                        StridedView v, void* __restrict__ yv) {
    const uint64_t t = uint64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (t >= v.nthreads) return;
    const uint64_t i = t % v.inner;
    const uint64_t rest = t / v.inner;
    const uint32_t g = uint32_t(rest % v.groups);
    const uint64_t o = rest / v.groups;
    const uint64_t row = o * v.inner + i;
    for (int jj = 0; jj < kJ; ++jj) {
        const uint32_t j = g * kJ + uint32_t(jj);
        if (j >= v.nbl) break;
        uint4 qv;
        uint32_t S, pr;
        if (kRecords) {
            const uint8_t* rec = packed + row * uint64_t(ld_p) + uint64_t(kRec) * j;
            uint32_t qd[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int k = 0; k < 16; ++k) qd[k >> 2] |= uint32_t(rec[1 + k]) << (8 * (k & 3));
            qv = make_uint4(qd[0], qd[1], qd[2], qd[3]);
            S = rec[0];
            pr = rec[kRec - 1];
        } else {
            const uint64_t blk = row * v.nbl + j;
            qv = reinterpret_cast<const uint4*>(q)[blk];
            S = max_exp[blk];
            pr = prime[blk];
        }
        float y[16];
        unpack16(qv, S, pr, y);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int64_t l = int64_t(16) * j + k;
            if (l >= v.len) break;
            const uint64_t idx = (o * uint64_t(v.len) + uint64_t(l)) * v.inner + i;
            if (kOut == 0) {
                static_cast<float*>(yv)[idx] = y[k];
            } else {
                const uint16_t h = S == 255u ? uint16_t(0x7FC0u) : __builtin_bit_cast(uint16_t, __bf16(y[k]));
                static_cast<uint16_t*>(yv)[idx] = h;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Axis tiles: 64 * kPer inner positions x 32 / kPer blocks of one o per
// workgroup (8 / kPer blocks for the three-part unpack).  A lane takes kPer
// adjacent inner positions (kPer = 2 when the inner extent is even: one
// 32-bit load carries two bf16 elements, one 64-bit load two fp32 elements).  The element reads of the pack and the element
// writes of the unpack (each touched once, in segments scattered over many
// rows) carry the non-temporal hint; measured on MI355X for [4096, 14336]
// along axis 0, pack goes from 0.49 to 0.59 of peak (fp32) and unpack from
// 0.47 to 0.71.  Streaming the other side as well is slower.
// ---------------------------------------------------------------------------

template <int kPer, int kTJ = 32, int kWaves = 4>
struct Tile {
    static constexpr int kI = 64 * kPer;                 // inner positions per tile
    static constexpr int kJ = kTJ / kPer;                // blocks per tile row
    static constexpr int kJW = kJ / kWaves;              // blocks per wave
    static constexpr int kQPitch = kJ * 16 + 16;         // q row in LDS (bytes)
    static constexpr int kEPitch = kJ + 4;               // max_exp / prime row in LDS
    static constexpr int kRPitch = kJ * kRec + 16;       // record row in LDS
    static constexpr int kQBytes = kI * kQPitch;
    static constexpr int kLds = kI * kRPitch > kI * (kQPitch + 2 * kEPitch) ? kI * kRPitch : kI * (kQPitch + 2 * kEPitch);
};

// The axis pack runs 8 waves per tile (kJ / 8 blocks each): measured on
// MI355X this is 1-5% faster than 4 waves of kJ / 4 blocks, with fewer
// registers per wave and the same LDS stage.
constexpr int kPackThreads = 512;

// The unpack of the three-part form takes tiles of 8 / kPer blocks per row:
// their LDS stage is a quarter of the pack's, so four times as many
// workgroups fit a CU, and measured on MI355X for [4096, 14336] along axis 0
// the unpack goes from 0.70-0.73 to 0.76-0.85 of peak (the pack is slower
// with small tiles and keeps 32 / kPer).  Records keep 32 / kPer blocks, so
// that every row's run of records starts 16-byte aligned.
template <bool kRecords>
constexpr int kUnpackTJ = kRecords ? 32 : 8;

struct AxisTiles {
    uint64_t outer, inner;
    int64_t len;
    uint32_t nbl;         // blocks per row, ceil(len / 16)
    uint32_t tiles_i;     // ceil(inner / kI)
    uint32_t tiles_j;     // ceil(nbl / kJ)
};

struct TileCoord {
    uint64_t o, i0;
    uint32_t j0, rows, nj;    // rows: live inner positions, nj: live blocks per row
};

// The pack's order: tile row (o, ti) -- the tiles of one inner range --
// runs on one XCD, which walks its blocks' tiles tj in turn.  Workgroups are
// dealt to the 8 XCDs round-robin, so workgroup wg runs on XCD x = wg % 8 and
// is that XCD's k-th (k = wg / 8); XCD x takes tile rows x, x + 8, x + 16,
// ...  The max_exp and prime lines of a row (8 tiles' 16-byte pieces) are
// then completed in one L2 by consecutive tiles, and the 8 XCDs read
// adjacent column ranges of the same element rows.  Workgroups past the last
// tile row (when the row count is not a multiple of 8) return at once.
// Measured on MI355X for [4096, 14336] along axis 0 (byte-identical output):
// 57.3 -> 51.7 us (fp32) and 37.3 -> 33.8 us (bf16) against the order below.
template <int kPer, int kTJ = 32>
__device__ __forceinline__ bool tile_coord_walk(const AxisTiles& v, TileCoord& c) {
    using T = Tile<kPer, kTJ>;
    const uint64_t x = blockIdx.x & 7u, k = blockIdx.x >> 3;
    const uint64_t row = 8 * (k / v.tiles_j) + x;          // tile row: o * tiles_i + ti
    if (row >= v.outer * v.tiles_i) return false;
    const uint32_t tj = uint32_t(k % v.tiles_j);
    const uint32_t ti = uint32_t(row % v.tiles_i);
    c.o = row / v.tiles_i;
    c.i0 = uint64_t(ti) * T::kI;
    c.j0 = tj * T::kJ;
    c.rows = uint32_t(v.inner - c.i0 < uint64_t(T::kI) ? v.inner - c.i0 : uint64_t(T::kI));
    c.nj = v.nbl - c.j0 < uint32_t(T::kJ) ? v.nbl - c.j0 : uint32_t(T::kJ);
    return true;
}

// Grid of the pack's order: 8 XCDs x ceil(tile rows / 8) x tiles_j.
inline uint64_t walk_grid(const AxisTiles& v) {
    return 8 * ((v.outer * v.tiles_i + 7) / 8) * v.tiles_j;
}

template <int kPer, int kTJ = 32>
__device__ __forceinline__ TileCoord tile_coord(const AxisTiles& v) {
    using T = Tile<kPer, kTJ>;
    TileCoord c;
    // the unpack's order: consecutive workgroups take consecutive inner
    // ranges of the same element rows, so the rows' segments are read (and
    // written) together
    const uint64_t wg = blockIdx.x;
    const uint32_t ti = uint32_t(wg % v.tiles_i);
    const uint64_t rest = wg / v.tiles_i;
    const uint32_t tj = uint32_t(rest % v.tiles_j);
    c.o = rest / v.tiles_j;
    c.i0 = uint64_t(ti) * T::kI;
    c.j0 = tj * T::kJ;
    c.rows = uint32_t(v.inner - c.i0 < uint64_t(T::kI) ? v.inner - c.i0 : uint64_t(T::kI));
    c.nj = v.nbl - c.j0 < uint32_t(T::kJ) ? v.nbl - c.j0 : uint32_t(T::kJ);
    return c;
}

// One load of kPer adjacent elements x[idx], x[idx + 1] (idx is even when
// kPer == 2): a raw word, widened to fp32 bit patterns by raw_elem.
template <int kDtype, int kPer>
struct Raw {
    using type = uint32_t;
};
template <>
struct Raw<0, 2> {
    using type = uint2;
};

template <int kDtype, int kPer>
__device__ __forceinline__ typename Raw<kDtype, kPer>::type load_raw(const void* xv, uint64_t idx) {
    if constexpr (kDtype == 0 && kPer == 2) {
        typedef unsigned int u2 __attribute__((ext_vector_type(2)));
        const u2 v = __builtin_nontemporal_load(reinterpret_cast<const u2*>(static_cast<const uint32_t*>(xv) + idx));
        return make_uint2(v.x, v.y);
    } else if constexpr (kDtype == 1 && kPer == 2) {
        return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(xv) + idx));
    } else if constexpr (kDtype == 0) {
        return __builtin_nontemporal_load(static_cast<const uint32_t*>(xv) + idx);
    } else {
        return uint32_t(__builtin_nontemporal_load(static_cast<const uint16_t*>(xv) + idx)) << 16;
    }
}

#if defined(__HIP_DEVICE_COMPILE__)
// The same load through a buffer resource: byte offset voff (per lane) plus
// soff (wave-uniform, a scalar register), so a batch of rows costs no vector
// address arithmetic.  The resource never clips (num_records is 2^32 - 1);
// callers keep every offset inside the tensor.
template <int kDtype, int kPer>
__device__ __forceinline__ typename Raw<kDtype, kPer>::type load_raw_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                                         uint32_t soff) {
    constexpr int kNt = 2;   // the non-temporal hint
    if constexpr (kDtype == 0 && kPer == 2) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, int(voff), int(soff), kNt);
        return make_uint2(v[0], v[1]);
    } else if constexpr (kDtype == 1 && kPer == 1) {
        return uint32_t(__builtin_amdgcn_raw_buffer_load_b16(r, int(voff), int(soff), kNt)) << 16;
    } else {
        return __builtin_amdgcn_raw_buffer_load_b32(r, int(voff), int(soff), kNt);
    }
}
#endif

template <int kDtype, int kPer>
__device__ __forceinline__ uint32_t raw_elem(typename Raw<kDtype, kPer>::type r, int e) {
    if constexpr (kDtype == 0 && kPer == 2) {
        return e == 0 ? r.x : r.y;
    } else if constexpr (kDtype == 1 && kPer == 2) {
        return e == 0 ? r << 16 : r & 0xFFFF0000u;
    } else {
        return r;
    }
}

// Stage one packed block in the tile's LDS row r, block slot jl.
template <int kPer, bool kRecords>
__device__ __forceinline__ void stage_block(uint8_t* ls, uint32_t r, uint32_t jl, const uint32_t (&qd)[4],
                                            uint32_t me, uint32_t pr) {
    using T = Tile<kPer>;
    if (kRecords) {
        uint8_t* rec = ls + r * T::kRPitch + kRec * jl;
        rec[0] = uint8_t(me);
#pragma unroll
        for (int k = 0; k < 16; ++k) rec[1 + k] = uint8_t(qd[k >> 2] >> (8 * (k & 3)));
        rec[kRec - 1] = uint8_t(pr);
    } else {
        *reinterpret_cast<uint4*>(ls + r * T::kQPitch + 16 * jl) = make_uint4(qd[0], qd[1], qd[2], qd[3]);
        ls[T::kQBytes + r * T::kEPitch + jl] = uint8_t(me);
        ls[T::kQBytes + T::kI * T::kEPitch + r * T::kEPitch + jl] = uint8_t(pr);
    }
}

template <int kDtype, bool kRecords, int kPer>
__global__ __launch_bounds__(kPackThreads)
void mx9_pack_axis_tile(const void* __restrict__ xv, AxisTiles v, int8_t* __restrict__ q,
                        uint8_t* __restrict__ max_exp, uint8_t* __restrict__ prime,
                        uint8_t* __restrict__ packed, int64_t ld_p, bool vec_out) {
    using T = Tile<kPer, 32, kPackThreads / 64>;
    __shared__ uint4 lds[T::kLds / 16];
    uint8_t* ls = reinterpret_cast<uint8_t*>(lds);
    TileCoord c;
    if (!tile_coord_walk<kPer>(v, c)) return;       // uniform across the workgroup, before any barrier
    const uint32_t il = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t r0 = il * kPer;                  // the lane's first row in the tile
    const bool live_i = r0 < c.rows;                // kPer == 2: rows come in pairs (inner is even)
    const uint64_t i = c.i0 + r0;
    constexpr uint32_t kEsz = kDtype == 0 ? 4u : 2u;
    // The offsets of a batch (64 element rows) fit 32 bits when an element
    // row is below 2^26 bytes; longer rows take the general route below.
    const bool small_row = v.inner * kEsz < (uint64_t(1) << 26);
    // Batches of kU blocks: every load of a batch is issued before any of its
    // blocks is computed, so 16 * kU loads per lane are in flight.
    using RawT = typename Raw<kDtype, kPer>::type;
    constexpr int kU = T::kJW < 4 ? T::kJW : 4;
    static_assert(T::kJW % kU == 0, "batches divide the wave's blocks");
#pragma unroll 1
    for (int b0 = 0; b0 < T::kJW; b0 += kU) {
        const uint32_t jl0 = wave * T::kJW + uint32_t(b0);
        if (jl0 >= c.nj) break;                     // uniform across the wave
        RawT raw[kU][16];
        const int64_t l_first = int64_t(16) * (c.j0 + jl0);
        if (small_row && jl0 + kU <= c.nj && l_first + 16 * kU <= v.len) {
            // Every row of the batch exists: a load's address is the batch's
            // first row (wave-uniform) plus the row's offset (wave-uniform)
            // plus the lane's position, and no load is predicated.  Lanes past
            // the tile's live rows read position i0 (which exists); their
            // results are never written out.
#if defined(__HIP_DEVICE_COMPILE__)
            const uint32_t voff = uint32_t(live_i ? i : c.i0) * kEsz;
            const char* rows = static_cast<const char*>(xv) +
                               (c.o * uint64_t(v.len) + uint64_t(l_first)) * v.inner * kEsz;
            const __amdgpu_buffer_rsrc_t rs =
                __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(rows), 0, int(0xFFFFFFFFu), 0x00020000);
            const uint32_t pitch = uint32_t(v.inner) * kEsz;
#pragma unroll
            for (int u = 0; u < kU; ++u) {
#pragma unroll
                for (int k = 0; k < 16; ++k)
                    raw[u][k] = load_raw_buf<kDtype, kPer>(rs, voff, uint32_t(16 * u + k) * pitch);
            }
#endif
        } else {
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int64_t l0 = l_first + 16 * u;
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const int64_t l = l0 + k;
                    raw[u][k] = RawT{};
                    if (live_i && jl0 + u < c.nj && l < v.len)
                        raw[u][k] = load_raw<kDtype, kPer>(xv, (c.o * uint64_t(v.len) + uint64_t(l)) * v.inner + i);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if (jl0 + u >= c.nj) break;
#pragma unroll
            for (int e = 0; e < kPer; ++e) {
                uint32_t w[16];
#pragma unroll
                for (int k = 0; k < 16; ++k) w[k] = raw_elem<kDtype, kPer>(raw[u][k], e);
                uint32_t qd[4], me, pr;
                pack16(w, qd, me, pr);
                stage_block<kPer, kRecords>(ls, r0 + e, jl0 + u, qd, me, pr);
            }
        }
    }
    __syncthreads();
    const uint64_t row0 = c.o * v.inner + c.i0;      // output row of the tile's first inner position
    if (kRecords) {
        const uint32_t rb = kRec * c.nj;            // record bytes per row
        const uint32_t chunks = (rb + 15) / 16;
        for (uint32_t t = threadIdx.x; t < c.rows * chunks; t += kPackThreads) {
            const uint32_t r = t / chunks, k = t - r * chunks;
            uint8_t* dst = packed + (row0 + r) * uint64_t(ld_p) + uint64_t(kRec) * c.j0 + 16u * k;
            const uint8_t* src = ls + r * T::kRPitch + 16u * k;
            const uint32_t n = rb - 16u * k < 16u ? rb - 16u * k : 16u;
            if (vec_out && n == 16u) {
                *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
            } else {
                for (uint32_t b = 0; b < n; ++b) dst[b] = src[b];
            }
        }
    } else {
        const uint8_t* ls_e = ls + T::kQBytes;
        const uint8_t* ls_p = ls_e + T::kI * T::kEPitch;
        for (uint32_t t = threadIdx.x; t < c.rows * c.nj; t += kPackThreads) {
            const uint32_t r = t / c.nj, k = t - r * c.nj;
            const uint64_t blk = (row0 + r) * v.nbl + c.j0 + k;
            reinterpret_cast<uint4*>(q)[blk] = *reinterpret_cast<const uint4*>(ls + r * T::kQPitch + 16u * k);
            max_exp[blk] = ls_e[r * T::kEPitch + k];
            prime[blk] = ls_p[r * T::kEPitch + k];
        }
    }
}

// Store kPer consecutive outputs y[idx], y[idx + 1] (idx is even when kPer == 2);
// an element of a poisoned block (nan[e]) is the quiet NaN.
template <int kOut, int kPer>
__device__ __forceinline__ void store_run(void* yv, uint64_t idx, const float (&y)[kPer], const bool (&nan)[kPer]) {
    if (kOut == 0) {
        uint32_t b[kPer];
#pragma unroll
        for (int e = 0; e < kPer; ++e) b[e] = nan[e] ? 0x7FC00000u : __float_as_uint(y[e]);
        typedef unsigned int u2 __attribute__((ext_vector_type(2)));
        if (kPer == 1) __builtin_nontemporal_store(b[0], static_cast<uint32_t*>(yv) + idx);
        else __builtin_nontemporal_store(u2{b[0], b[kPer - 1]}, reinterpret_cast<u2*>(static_cast<uint32_t*>(yv) + idx));
    } else {
        uint16_t h[kPer];
#pragma unroll
        for (int e = 0; e < kPer; ++e) h[e] = nan[e] ? uint16_t(0x7FC0u) : __builtin_bit_cast(uint16_t, __bf16(y[e]));
        if (kPer == 1) __builtin_nontemporal_store(h[0], static_cast<uint16_t*>(yv) + idx);
        else __builtin_nontemporal_store(uint32_t(h[0]) | (uint32_t(h[kPer - 1]) << 16),
                                         reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(yv) + idx));
    }
}

template <int kOut, bool kRecords, int kPer>
__global__ __launch_bounds__(kThreads)
void mx9_unpack_axis_tile(const int8_t* __restrict__ q, const uint8_t* __restrict__ max_exp,
                          const uint8_t* __restrict__ prime, const uint8_t* __restrict__ packed, int64_t ld_p,
                          AxisTiles v, void* __restrict__ yv, bool vec_in) {
    using T = Tile<kPer, kUnpackTJ<kRecords>>;
    __shared__ uint4 lds[T::kLds / 16];
    uint8_t* ls = reinterpret_cast<uint8_t*>(lds);
    uint8_t* ls_e = ls + T::kQBytes;
    uint8_t* ls_p = ls_e + T::kI * T::kEPitch;
    const TileCoord c = tile_coord<kPer, kUnpackTJ<kRecords>>(v);
    const uint64_t row0 = c.o * v.inner + c.i0;
    if (kRecords) {
        const uint32_t rb = kRec * c.nj;
        const uint32_t chunks = (rb + 15) / 16;
        for (uint32_t t = threadIdx.x; t < c.rows * chunks; t += kThreads) {
            const uint32_t r = t / chunks, k = t - r * chunks;
            const uint8_t* src = packed + (row0 + r) * uint64_t(ld_p) + uint64_t(kRec) * c.j0 + 16u * k;
            uint8_t* dst = ls + r * T::kRPitch + 16u * k;
            const uint32_t n = rb - 16u * k < 16u ? rb - 16u * k : 16u;
            if (vec_in && n == 16u) {
                *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
            } else {
                for (uint32_t b = 0; b < n; ++b) dst[b] = src[b];
            }
        }
    } else {
        for (uint32_t t = threadIdx.x; t < c.rows * c.nj; t += kThreads) {
            const uint32_t r = t / c.nj, k = t - r * c.nj;
            const uint64_t blk = (row0 + r) * v.nbl + c.j0 + k;
            *reinterpret_cast<uint4*>(ls + r * T::kQPitch + 16u * k) = reinterpret_cast<const uint4*>(q)[blk];
            ls_e[r * T::kEPitch + k] = max_exp[blk];
            ls_p[r * T::kEPitch + k] = prime[blk];
        }
    }
    __syncthreads();
    const uint32_t il = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t r0 = il * kPer;
    if (r0 >= c.rows) return;                       // no barrier follows
    const uint64_t i = c.i0 + r0;
#pragma unroll 2
    for (int b = 0; b < T::kJW; ++b) {
        const uint32_t jl = wave * T::kJW + uint32_t(b);
        if (jl >= c.nj) break;
        float y[kPer][16];
        bool nan[kPer];
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const uint32_t r = r0 + e;
            uint4 qv;
            uint32_t S, pr;
            if (kRecords) {
                const uint8_t* rec = ls + r * T::kRPitch + kRec * jl;
                uint32_t qd[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int k = 0; k < 16; ++k) qd[k >> 2] |= uint32_t(rec[1 + k]) << (8 * (k & 3));
                qv = make_uint4(qd[0], qd[1], qd[2], qd[3]);
                S = rec[0];
                pr = rec[kRec - 1];
            } else {
                qv = *reinterpret_cast<const uint4*>(ls + r * T::kQPitch + 16 * jl);
                S = ls_e[r * T::kEPitch + jl];
                pr = ls_p[r * T::kEPitch + jl];
            }
            unpack16(qv, S, pr, y[e]);
            nan[e] = S == 255u;
        }
        const int64_t l0 = int64_t(16) * (c.j0 + jl);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int64_t l = l0 + k;
            if (l >= v.len) break;
            const uint64_t idx = (c.o * uint64_t(v.len) + uint64_t(l)) * v.inner + i;
            float run[kPer];
#pragma unroll
            for (int e = 0; e < kPer; ++e) run[e] = y[e][k];
            store_run<kOut, kPer>(yv, idx, run, nan);
        }
    }
}

AxisTiles make_tiles(int64_t outer, int64_t len, int64_t inner, int per, int tile_tj) {
    AxisTiles v;
    v.outer = uint64_t(outer);
    v.inner = uint64_t(inner);
    v.len = len;
    v.nbl = uint32_t((len + 15) / 16);
    const int ti = 64 * per, tj = tile_tj / per;
    v.tiles_i = uint32_t((inner + ti - 1) / ti);
    v.tiles_j = (v.nbl + uint32_t(tj) - 1) / uint32_t(tj);
    return v;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

StridedView make_view(int64_t outer, int64_t len, int64_t inner, int kJ) {
    StridedView v;
    v.outer = uint64_t(outer);
    v.inner = uint64_t(inner);
    v.len = len;
    v.nbl = uint32_t((len + 15) / 16);
    v.groups = (v.nbl + uint32_t(kJ) - 1) / uint32_t(kJ);
    v.nthreads = v.outer * v.inner * v.groups;
    return v;
}

dim3 grid_for(uint64_t nthreads) { return dim3(uint32_t((nthreads + kThreads - 1) / kThreads)); }

// kPer = 2 needs an even inner extent (then a lane's two inner positions are
// one aligned 32- or 64-bit word of every element row).
inline int per_lane(int64_t inner, const void* buf, int esz) {
    return inner % 2 == 0 && (reinterpret_cast<uintptr_t>(buf) & uintptr_t(2 * esz - 1)) == 0 ? 2 : 1;
}

template <bool kRecords>
void launch_pack_tiles(const void* x, int dtype, int64_t outer, int64_t len, int64_t inner, int8_t* q,
                       uint8_t* max_exp, uint8_t* prime, uint8_t* packed, int64_t ld_p, hipStream_t stream) {
    const int per = per_lane(inner, x, dtype == 0 ? 4 : 2);
    const AxisTiles v = make_tiles(outer, len, inner, per, 32);
    const dim3 grid(uint32_t(walk_grid(v)));
    const bool vec = aligned16(packed) && ld_p % 16 == 0;
    if (dtype == 0 && per == 2) hipLaunchKernelGGL((mx9_pack_axis_tile<0, kRecords, 2>), grid, dim3(kPackThreads), 0, stream, x, v, q, max_exp, prime, packed, ld_p, vec);
    else if (dtype == 0) hipLaunchKernelGGL((mx9_pack_axis_tile<0, kRecords, 1>), grid, dim3(kPackThreads), 0, stream, x, v, q, max_exp, prime, packed, ld_p, vec);
    else if (per == 2) hipLaunchKernelGGL((mx9_pack_axis_tile<1, kRecords, 2>), grid, dim3(kPackThreads), 0, stream, x, v, q, max_exp, prime, packed, ld_p, vec);
    else hipLaunchKernelGGL((mx9_pack_axis_tile<1, kRecords, 1>), grid, dim3(kPackThreads), 0, stream, x, v, q, max_exp, prime, packed, ld_p, vec);
}

template <bool kRecords>
void launch_unpack_tiles(const int8_t* q, const uint8_t* max_exp, const uint8_t* prime, const uint8_t* packed,
                         int64_t ld_p, int64_t outer, int64_t len, int64_t inner, int out_dtype, void* y,
                         hipStream_t stream) {
    const int per = per_lane(inner, y, out_dtype == 0 ? 4 : 2);
    const AxisTiles v = make_tiles(outer, len, inner, per, kUnpackTJ<kRecords>);
    const dim3 grid(uint32_t(v.outer * v.tiles_i * v.tiles_j));
    const bool vec = aligned16(packed) && ld_p % 16 == 0;
    if (out_dtype == 0 && per == 2) hipLaunchKernelGGL((mx9_unpack_axis_tile<0, kRecords, 2>), grid, dim3(kThreads), 0, stream, q, max_exp, prime, packed, ld_p, v, y, vec);
    else if (out_dtype == 0) hipLaunchKernelGGL((mx9_unpack_axis_tile<0, kRecords, 1>), grid, dim3(kThreads), 0, stream, q, max_exp, prime, packed, ld_p, v, y, vec);
    else if (per == 2) hipLaunchKernelGGL((mx9_unpack_axis_tile<1, kRecords, 2>), grid, dim3(kThreads), 0, stream, q, max_exp, prime, packed, ld_p, v, y, vec);
    else hipLaunchKernelGGL((mx9_unpack_axis_tile<1, kRecords, 1>), grid, dim3(kThreads), 0, stream, q, max_exp, prime, packed, ld_p, v, y, vec);
}

// Records of a last-axis pack with a pitch or a ragged row: one thread per block.
void launch_pack_records_rows(const void* x, int dtype, int64_t rows, int64_t len, uint8_t* packed, int64_t ld_p,
                              hipStream_t stream) {
    const StridedView v = make_view(rows, len, 1, 1);
    if (dtype == 0) hipLaunchKernelGGL((mx9_pack_strided<0, true, 1>), grid_for(v.nthreads), dim3(kThreads), 0, stream, x, v, nullptr, nullptr, nullptr, packed, ld_p);
    else hipLaunchKernelGGL((mx9_pack_strided<1, true, 1>), grid_for(v.nthreads), dim3(kThreads), 0, stream, x, v, nullptr, nullptr, nullptr, packed, ld_p);
}

void launch_unpack_records_rows(const uint8_t* packed, int64_t ld_p, int64_t rows, int64_t len, int out_dtype,
                                void* y, hipStream_t stream) {
    const StridedView v = make_view(rows, len, 1, 1);
    if (out_dtype == 0) hipLaunchKernelGGL((mx9_unpack_strided<0, true, 1>), grid_for(v.nthreads), dim3(kThreads), 0, stream, nullptr, nullptr, nullptr, packed, ld_p, v, y);
    else hipLaunchKernelGGL((mx9_unpack_strided<1, true, 1>), grid_for(v.nthreads), dim3(kThreads), 0, stream, nullptr, nullptr, nullptr, packed, ld_p, v, y);
}

}  // namespace

uint64_t mx9_axis_grid_threads(int64_t outer, int64_t len, int64_t inner) {
    uint64_t most = 0;
    for (int per = 1; per <= 2; ++per) {
        const uint64_t pack = walk_grid(make_tiles(outer, len, inner, per, 32)) * kPackThreads;
        const AxisTiles u3 = make_tiles(outer, len, inner, per, kUnpackTJ<false>);
        const AxisTiles ur = make_tiles(outer, len, inner, per, kUnpackTJ<true>);
        const uint64_t unpack = std::max(u3.outer * u3.tiles_i * u3.tiles_j, ur.outer * ur.tiles_i * ur.tiles_j) * kThreads;
        most = std::max(most, std::max(pack, unpack));
    }
    return most;
}

hipError_t launch_mx9_pack_axis(const void* x, int dtype, int64_t outer, int64_t len, int64_t inner,
                                int8_t* q, uint8_t* max_exp, uint8_t* prime, hipStream_t stream) {
    if (inner == 1)   // the last axis: rows of len elements
        return launch_mx9_pack(x, dtype, outer, len, len, q, 16 * ((len + 15) / 16), max_exp, (len + 15) / 16, prime,
                               (len + 15) / 16, stream);
    launch_pack_tiles<false>(x, dtype, outer, len, inner, q, max_exp, prime, nullptr, 0, stream);
    return hipGetLastError();
}

hipError_t launch_mx9_unpack_axis(const int8_t* q, const uint8_t* max_exp, const uint8_t* prime,
                                  int64_t outer, int64_t len, int64_t inner, int out_dtype, void* y,
                                  hipStream_t stream) {
    if (inner == 1)
        return launch_mx9_unpack(q, 16 * ((len + 15) / 16), max_exp, (len + 15) / 16, prime, (len + 15) / 16, outer, len,
                                 out_dtype, y, len, stream);
    launch_unpack_tiles<false>(q, max_exp, prime, nullptr, 0, outer, len, inner, out_dtype, y, stream);
    return hipGetLastError();
}

hipError_t launch_mx9_pack_records(const void* x, int dtype, int64_t outer, int64_t len, int64_t inner,
                                   uint8_t* packed, int64_t ld_p, hipStream_t stream) {
    const int64_t nbl = (len + 15) / 16;
    if (inner == 1 && len % 16 == 0 && ld_p == kRec * nbl && aligned16(x) && aligned16(packed)) {
        const uint64_t nb = uint64_t(outer) * uint64_t(nbl);
        const uint64_t per_wg = uint64_t(kThreads / 64) * 64u;   // 64 blocks per wave, either dtype
        const dim3 grid(uint32_t((nb + per_wg - 1) / per_wg));
        if (dtype == 0) hipLaunchKernelGGL(mx9_pack_records_flat<0>, grid, dim3(kThreads), 0, stream, x, nb, packed);
        else hipLaunchKernelGGL(mx9_pack_records_flat<1>, grid, dim3(kThreads), 0, stream, x, nb, packed);
        return hipGetLastError();
    }
    if (inner == 1) launch_pack_records_rows(x, dtype, outer, len, packed, ld_p, stream);
    else launch_pack_tiles<true>(x, dtype, outer, len, inner, nullptr, nullptr, nullptr, packed, ld_p, stream);
    return hipGetLastError();
}

hipError_t launch_mx9_unpack_records(const uint8_t* packed, int64_t ld_p, int64_t outer, int64_t len,
                                     int64_t inner, int out_dtype, void* y, hipStream_t stream) {
    const int64_t nbl = (len + 15) / 16;
    if (inner == 1 && len % 16 == 0 && ld_p == kRec * nbl && aligned16(packed) && aligned16(y)) {
        const uint64_t nb = uint64_t(outer) * uint64_t(nbl);
        const uint32_t per_wg = out_dtype == 0 ? 64u : 128u;
        const dim3 grid(uint32_t((nb + per_wg - 1) / per_wg));
        if (out_dtype == 0) hipLaunchKernelGGL(mx9_unpack_records_flat<0>, grid, dim3(kThreads), 0, stream, packed, nb, y);
        else hipLaunchKernelGGL(mx9_unpack_records_flat<1>, grid, dim3(kThreads), 0, stream, packed, nb, y);
        return hipGetLastError();
    }
    if (inner == 1) launch_unpack_records_rows(packed, ld_p, outer, len, out_dtype, y, stream);
    else launch_unpack_tiles<true>(nullptr, nullptr, nullptr, packed, ld_p, outer, len, inner, out_dtype, y, stream);
    return hipGetLastError();
}

}  // namespace mxq
