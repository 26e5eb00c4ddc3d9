// mx_gemm.hip -- MXFP8 block-scaled contraction on gfx950 matrix cores.
//
// Operation: AMD-AGI/ALTO PR #31, "Add MXFP8 grouped GEMM (E4M3) for
// routed-expert MoE training" (description): E4M3 operands with E8M0 scales
// per 32 elements of the contraction, groups given by 1-D cumulative
// offsets.  Both operands are stored with the contraction index contiguous
// ("NT"), which is what the dual-axis cast emits: q_row [M, K] for the
// forward and q_col [K, M] (tokens contiguous) for the weight gradient.
//
//   C[m][n] = sum_k e4m3(A[m][k]) 2^(sA(m, k/32) - 127) e4m3(B[n][k]) 2^(sB(n, k/32) - 127)
//
// Matrix-core layout of v_mfma_scale_f32_16x16x128_f8f6f4 (identified on
// MI355X with one-hot probes): lane L of a wave holds row L % 16 of the
// 16 x 128 operand; with g = L / 16 its bytes 0..15 are k = 16g .. 16g+15
// and bytes 16..31 are k = 64 + 16g .. 64 + 16g + 15, and its scale operand
// is the E8M0 byte of k-block [32g, 32g + 32).  The result C[4 (L/16) + v]
// [L % 16] is element v of lane L's four accumulators.  The same layout for
// A and B means each lane reads two 16-byte pieces of one stored row.
//
// Two kernels.  mx_gemm_pipe_kernel (further below) is the fast path: it
// takes the matrix-core scale layout, or plain scales whose blocks of a row
// are adjacent (the rowwise cast's s_row) or whose rows of a block are
// adjacent (the colwise cast's s_col read through its transpose), with both
// operands in one form and C rows in 16-byte pieces (rows-form scales with
// 16-byte aligned rows are loaded four steps at a time).  mx_gemm_kernel
// (below) takes any strided scale views and any C pitch.
//
// mx_gemm_kernel: one workgroup (4 wave64s) per 128 x 128 tile of C; wave w
// computes the 64 x 64 quarter (w / 2, w % 2) as 4 x 4 instructions per
// 128-wide step of the contraction.
//   * staging: the A and B tiles of a step (128 rows x 128 bytes each) are
//     loaded with 16-byte global loads (a wave covers eight whole 128-byte
//     rows) into double-buffered LDS; the 16-byte chunk index of a row is
//     XORed with row % 8 so that the 16 rows a fragment read touches at one
//     chunk offset fall in different banks.  The next step's loads are in
//     flight while the current step computes.
//   * scales: a lane needs one A byte per 16-row sub-tile and one B byte per
//     16-column sub-tile per step; the four A bytes (and the four B bytes)
//     are packed into one register and the instruction's op_sel picks the
//     byte.  They are fetched one step ahead, like the data.  From strided
//     scale views (the cast's plain layouts) that takes four byte loads per
//     operand; from the matrix-core scale layout (scale (r, b) at byte
//     ((r/64 * K/128 + b/4) * 64 + 16 (b%4) + r%16) * 4 + (r%64)/16) the
//     register is one dword, and a wave's 64 dwords are one 256-byte run.
//   * groups: row groups (the forward: rows of group g use expert g's
//     operand, rows past the last offset give 0) find their group from the
//     tile's first row, since groups are multiples of 128 rows; contraction
//     groups (the weight gradient) give each group its own C and run the
//     group's range of the contraction.
#include "mxq_kernels.h"

#include <utility>

namespace mxq {
namespace {

constexpr int kTile = 128;
constexpr int kThreads = 256;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
    const uint8_t* A;
    int64_t lda;
    const uint8_t* sA;
    int64_t sa_rs, sa_bs;     // strided view; in the matrix-core layout sa_rs is the bytes per 64 rows
    const uint8_t* B;
    int64_t ldb, b_gs;
    const uint8_t* sB;
    int64_t sb_rs, sb_bs, sb_gs;
    void* C;
    int64_t ldc, c_gs;
    int64_t M, N, K;          // rows of A and C, rows of B, contraction extent
    const int32_t* offs;
    int32_t G;
    int32_t mode;             // 0: dense or row groups, 1: contraction groups
    uint32_t tiles_m, tiles_n;
};

template <int MS, int NS>
__device__ __forceinline__ void mma(v4f (&acc)[4][4], const v8i (&a)[4], const v8i (&b)[4], int sa, int sb) {
    acc[MS][NS] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[MS], b[NS], acc[MS][NS], 0, 0, MS, sa, NS, sb);
}

template <int MS>
__device__ __forceinline__ void mma_row(v4f (&acc)[4][4], const v8i (&a)[4], const v8i (&b)[4], int sa, int sb) {
    mma<MS, 0>(acc, a, b, sa, sb);
    mma<MS, 1>(acc, a, b, sa, sb);
    mma<MS, 2>(acc, a, b, sa, sb);
    mma<MS, 3>(acc, a, b, sa, sb);
}

// Clamp a group end to [lo, hi] and down to a multiple of the tile, so that
// invalid offsets can never move an access outside the operands.
__device__ __forceinline__ int64_t clamp_end(int64_t v, int64_t lo, int64_t hi) {
    v = v < lo ? lo : (v > hi ? hi : v);
    return v - (v - lo) % kTile;
}

template <int kOut, bool kMfmaScales>
__global__ __launch_bounds__(kThreads, 2)
void mx_gemm_kernel(GemmArgs p) {
    __shared__ uint4 lds[2][2][kTile * 8];      // [buffer][A, B][row * 8 + chunk]

    const uint32_t t = threadIdx.x;
    const uint32_t lane = t & 63u, wave = t >> 6;
    const uint32_t wm = wave >> 1, wn = wave & 1u;

    // ---- which tile, which group, which range of the contraction ----
    uint32_t tm, tn;
    int64_t k_lo = 0, k_hi = p.K;
    const uint8_t* B = p.B;
    const uint8_t* sB = p.sB;
    char* C = static_cast<char*>(p.C);
    bool zero = false;
    if (p.mode == 0) {
        tm = blockIdx.x % p.tiles_m;
        tn = blockIdx.x / p.tiles_m;
        if (p.offs != nullptr) {
            const int64_t row = int64_t(tm) * kTile;
            int32_t g = 0;
            while (g < p.G && int64_t(p.offs[g]) <= row) ++g;      // first group ending after the row
            if (g == p.G) {
                zero = true;                                        // the uncovered tail
            } else {
                B += int64_t(g) * p.b_gs;
                sB += int64_t(g) * p.sb_gs;
            }
        }
    } else {
        const uint32_t per = p.tiles_m * p.tiles_n;
        const uint32_t g = blockIdx.x / per, r = blockIdx.x - g * per;
        tm = r % p.tiles_m;
        tn = r / p.tiles_m;
        k_lo = g == 0 ? 0 : clamp_end(p.offs[g - 1], 0, p.K);
        k_hi = clamp_end(p.offs[g], k_lo, p.K);
        C += int64_t(g) * p.c_gs * (kOut == 0 ? 4 : 2);
    }
    const int64_t m0 = int64_t(tm) * kTile, n0 = int64_t(tn) * kTile;

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    if (!zero && k_lo < k_hi) {
        uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
        // scale rows of this lane's four A sub-tiles and four B sub-tiles
        const uint8_t* sa_row = p.sA + (m0 + wm * 64 + (lane & 15u)) * p.sa_rs;
        const uint8_t* sb_row = sB + (n0 + wn * 64 + (lane & 15u)) * p.sb_rs;
        const int64_t kgrp = int64_t(lane >> 4);                   // the lane's 32-wide k-block of a step
        // matrix-core layout: this lane's dword of its 64-row group, one 256-byte run per step
        const uint32_t* sa_run = reinterpret_cast<const uint32_t*>(p.sA + int64_t(2 * tm + wm) * p.sa_rs) + lane;
        const uint32_t* sb_run = reinterpret_cast<const uint32_t*>(sB + int64_t(2 * tn + wn) * p.sb_rs) + lane;
        // this thread's four staging chunks: c = t + 256 i, row c / 8, 16-byte piece c % 8
        const uint32_t r0 = t >> 3, ch = t & 7u;                    // rows r0, r0 + 32, r0 + 64, r0 + 96
        const uint8_t* ga = p.A + (m0 + r0) * p.lda + 16 * ch;
        const uint8_t* gb = B + (n0 + r0) * p.ldb + 16 * ch;
        const int64_t lda32 = 32 * p.lda, ldb32 = 32 * p.ldb;
        const uint32_t slot0 = r0 * 8u + (ch ^ (r0 & 7u));         // (r0 + 32 i) % 8 == r0 % 8
#define MXQ_LOAD_STEP(k, SA, SB)                                                              \
        do {                                                                                  \
            ra0 = *reinterpret_cast<const uint4*>(ga + (k));                                  \
            ra1 = *reinterpret_cast<const uint4*>(ga + lda32 + (k));                          \
            ra2 = *reinterpret_cast<const uint4*>(ga + 2 * lda32 + (k));                      \
            ra3 = *reinterpret_cast<const uint4*>(ga + 3 * lda32 + (k));                      \
            rb0 = *reinterpret_cast<const uint4*>(gb + (k));                                  \
            rb1 = *reinterpret_cast<const uint4*>(gb + ldb32 + (k));                          \
            rb2 = *reinterpret_cast<const uint4*>(gb + 2 * ldb32 + (k));                      \
            rb3 = *reinterpret_cast<const uint4*>(gb + 3 * ldb32 + (k));                      \
            if (kMfmaScales) {                                                                \
                SA = int(sa_run[((k) / kTile) * 64]);                                         \
                SB = int(sb_run[((k) / kTile) * 64]);                                         \
            } else {                                                                          \
                const int64_t blk_ = (k) / 32 + kgrp;                                         \
                uint32_t a4_ = 0, b4_ = 0;                                                    \
                for (int s_ = 0; s_ < 4; ++s_) {                                              \
                    a4_ |= uint32_t(sa_row[16 * s_ * p.sa_rs + blk_ * p.sa_bs]) << (8 * s_);  \
                    b4_ |= uint32_t(sb_row[16 * s_ * p.sb_rs + blk_ * p.sb_bs]) << (8 * s_);  \
                }                                                                             \
                SA = int(a4_);                                                                \
                SB = int(b4_);                                                                \
            }                                                                                 \
        } while (0)
#define MXQ_STORE_STEP(buf)                                                                   \
        do {                                                                                  \
            lds[buf][0][slot0] = ra0;                                                         \
            lds[buf][0][slot0 + 256] = ra1;                                                   \
            lds[buf][0][slot0 + 512] = ra2;                                                   \
            lds[buf][0][slot0 + 768] = ra3;                                                   \
            lds[buf][1][slot0] = rb0;                                                         \
            lds[buf][1][slot0 + 256] = rb1;                                                   \
            lds[buf][1][slot0 + 512] = rb2;                                                   \
            lds[buf][1][slot0 + 768] = rb3;                                                   \
        } while (0)

        int sa_cur, sb_cur, sa_nxt = 0, sb_nxt = 0;
        MXQ_LOAD_STEP(k_lo, sa_cur, sb_cur);
        MXQ_STORE_STEP(0);
        __syncthreads();
        int buf = 0;
        for (int64_t k = k_lo; k < k_hi; k += kTile) {
            const bool more = k + kTile < k_hi;
            if (more) MXQ_LOAD_STEP(k + kTile, sa_nxt, sb_nxt);
            v8i af[4], bf[4];
            const uint32_t g = lane >> 4;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint32_t ar = wm * 64 + 16 * s + (lane & 15u);
                const uint4 alo = lds[buf][0][ar * 8u + (g ^ (ar & 7u))];
                const uint4 ahi = lds[buf][0][ar * 8u + ((4u + g) ^ (ar & 7u))];
                af[s] = v8i{int(alo.x), int(alo.y), int(alo.z), int(alo.w), int(ahi.x), int(ahi.y), int(ahi.z), int(ahi.w)};
                const uint32_t br = wn * 64 + 16 * s + (lane & 15u);
                const uint4 blo = lds[buf][1][br * 8u + (g ^ (br & 7u))];
                const uint4 bhi = lds[buf][1][br * 8u + ((4u + g) ^ (br & 7u))];
                bf[s] = v8i{int(blo.x), int(blo.y), int(blo.z), int(blo.w), int(bhi.x), int(bhi.y), int(bhi.z), int(bhi.w)};
            }
            mma_row<0>(acc, af, bf, sa_cur, sb_cur);
            mma_row<1>(acc, af, bf, sa_cur, sb_cur);
            mma_row<2>(acc, af, bf, sa_cur, sb_cur);
            mma_row<3>(acc, af, bf, sa_cur, sb_cur);
            if (more) {
                MXQ_STORE_STEP(buf ^ 1);
                sa_cur = sa_nxt;
                sb_cur = sb_nxt;
            }
            __syncthreads();
            buf ^= 1;
        }
#undef MXQ_LOAD_STEP
#undef MXQ_STORE_STEP
    }

    // ---- epilogue: C[m0 + 64 wm + 16 ms + 4 (lane / 16) + v][n0 + 64 wn + 16 ns + lane % 16] ----
    const int64_t col0 = n0 + wn * 64 + (lane & 15u);
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t row = m0 + wm * 64 + 16 * ms + 4 * (lane >> 4) + v;
#pragma unroll
            for (int ns = 0; ns < 4; ++ns) {
                const float x = acc[ms][ns][v];
                const int64_t idx = row * p.ldc + col0 + 16 * ns;
                if (kOut == 0) reinterpret_cast<float*>(C)[idx] = x;
                else reinterpret_cast<__bf16*>(C)[idx] = __bf16(x);
            }
        }
    }
}


// Scale forms of the pipelined kernel.  kScalesMfma: 64-row groups of
// 256-byte runs in the matrix-core layout.  kScalesRows: plain scales with
// the blocks of a row adjacent (block stride 1, row stride a multiple of 4),
// as the rowwise cast writes them.  kScalesBlocks: plain scales with the rows
// of a block adjacent (row stride 1, block stride a multiple of 4), as the
// colwise cast's s_col read through its transpose.  A plain run is the 64
// rows x 4 blocks of one contraction step, loaded as 64 dwords (one row's 4
// blocks, or 4 rows of one block) and gathered into the matrix-core dword at
// read time (four byte reads).
//
// kScalesRows4 is the rows form loaded four steps at a time: when every
// row's scales are 16-byte aligned and the contraction is whole periods of
// four steps (K a multiple of 512, contraction starting at 0), a run's load
// is one 16-byte piece per row covering four steps, into a period buffer
// of its own (two buffers, one period ahead).  A per-step dword per row
// touches one cache line per row and step; measured on MI355X, the
// row-grouped forward spends a quarter of its time on those requests
// (234 us against 174-180 us with the same number of contiguous loads);
// in four-step periods it takes 184-189 us, with byte-identical results.
constexpr int kScalesMfma = 0, kScalesRows = 1, kScalesBlocks = 2, kScalesRows4 = 3;

// A plain run's contribution to a lane's scale dword: byte q of the dword is
// the scale of run row 16 q + lane % 16, block lane / 16.  The four bytes lie
// in four dwords at a fixed stride (64 bytes in the rows form, 16 in the
// blocks form), read as two pairs; plain_scale_pick then takes the lane's
// byte of each with byte permutes.
template <int kSF>
__device__ __forceinline__ void plain_scale_read(const uint8_t* run, uint32_t lane, uint32_t (&raw)[4]) {
    constexpr uint32_t kStride = kSF == kScalesRows ? 16u : 4u;   // dwords
    const uint32_t* d = reinterpret_cast<const uint32_t*>(run) +
                        (kSF == kScalesRows ? (lane & 15u) : 16u * (lane >> 4) + ((lane & 15u) >> 2));
#pragma unroll
    for (int q = 0; q < 4; ++q) raw[q] = d[q * kStride];
}

// The same four dwords from a period buffer of the rows form: row r's
// 16 bytes at 16 r, the step's dword `sub` (0..3) of them.
__device__ __forceinline__ void period_scale_read(const uint8_t* run, uint32_t lane, uint32_t sub, uint32_t (&raw)[4]) {
    const uint32_t* d = reinterpret_cast<const uint32_t*>(run) + 4u * (lane & 15u) + sub;
#pragma unroll
    for (int q = 0; q < 4; ++q) raw[q] = d[64 * q];
}

template <int kSF>
__device__ __forceinline__ uint32_t plain_scale_sel(uint32_t lane) {
    const uint32_t b = kSF == kScalesRows ? (lane >> 4) : (lane & 3u);    // byte within each dword
    return b | ((4u + b) << 8) | 0x0C0C0000u;
}

__device__ __forceinline__ int plain_scale_pick(const uint32_t (&raw)[4], uint32_t sel) {
    const uint32_t lo = __builtin_amdgcn_perm(raw[1], raw[0], sel);
    const uint32_t hi = __builtin_amdgcn_perm(raw[3], raw[2], sel);
    return int(__builtin_amdgcn_perm(hi, lo, 0x05040100u));
}

// acc[i][J] += a[i] x b for every i (J, the column sub-tile, is fixed).
template <int J, int MS, int NS, int... I>
__device__ __forceinline__ void mma_col(v4f (&acc)[MS][NS], const v8i (&a)[MS], const v8i& b, const int (&sa)[MS / 4],
                                        int sb, std::integer_sequence<int, I...>) {
    ((acc[I][J] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[I], b, acc[I][J], 0, 0, I & 3, sa[I >> 2], J & 3,
                                                                   sb)),
     ...);
}

// B fragment of column sub-tile J (rows b_row0 + 16 J .. + 15) from LDS.
template <int J>
__device__ __forceinline__ v8i b_frag(const uint4* sb_lds, uint32_t b_row0, uint32_t lane) {
    const uint32_t g = lane >> 4, sw = lane & 7u;
    const uint32_t r = b_row0 + 16u * J + (lane & 15u);
    const uint4 lo = sb_lds[r * 8u + (g ^ sw)];
    const uint4 hi = sb_lds[r * 8u + ((4u + g) ^ sw)];
    return v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
}

// Column sub-tile J: the next column's B fragment is read from LDS while
// this column's instructions run (only two B fragments are ever live; the
// scheduling barriers keep the compiler from hoisting every read of the
// step, which would not fit the registers).
template <int J, int MS, int NS>
__device__ __forceinline__ void mma_b(v4f (&acc)[MS][NS], const v8i (&a)[MS], v8i& b, const uint4* sb_lds,
                                      uint32_t b_row0, uint32_t lane, const int (&sa)[MS / 4],
                                      const int (&sb)[NS / 4]) {
    v8i nb;
    if constexpr (J + 1 < NS) nb = b_frag<J + 1>(sb_lds, b_row0, lane);
    __builtin_amdgcn_sched_barrier(0);
    mma_col<J>(acc, a, b, sa, sb[J >> 2], std::make_integer_sequence<int, MS>{});
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (J + 1 < NS) b = nb;
}

// One 128-wide step from one LDS stage: all A fragments of the wave, then
// the B fragments one column sub-tile at a time.
template <int MS, int NS, int... J>
__device__ __forceinline__ void mma_step(v4f (&acc)[MS][NS], const uint4* sa_lds, const uint4* sb_lds, uint32_t a_row0,
                                         uint32_t b_row0, uint32_t lane, const int (&sa)[MS / 4],
                                         const int (&sb)[NS / 4], std::integer_sequence<int, J...>) {
    const uint32_t g = lane >> 4, sw = lane & 7u;           // a fragment row's index mod 8 is lane % 8
    v8i a[MS];
#pragma unroll
    for (int i = 0; i < MS; ++i) {
        const uint32_t r = a_row0 + 16u * i + (lane & 15u);
        const uint4 lo = sa_lds[r * 8u + (g ^ sw)];
        const uint4 hi = sa_lds[r * 8u + ((4u + g) ^ sw)];
        a[i] = v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
    }
    v8i b = b_frag<0>(sb_lds, b_row0, lane);
    (mma_b<J>(acc, a, b, sb_lds, b_row0, lane, sa, sb), ...);
}

// The same step with plain-form scales: their raw dwords were read before
// this step's fragments, and are combined only after every fragment read of
// the step's first column is issued, so that the combining waits for the
// scale reads alone.
template <int MS, int NS, int... J>
__device__ __forceinline__ void mma_step_plain(v4f (&acc)[MS][NS], const uint4* sa_lds, const uint4* sb_lds,
                                               uint32_t a_row0, uint32_t b_row0, uint32_t lane,
                                               const uint32_t (&ra)[MS / 4][4], const uint32_t (&rb)[NS / 4][4],
                                               uint32_t sel, std::integer_sequence<int, J...>) {
    const uint32_t g = lane >> 4, sw = lane & 7u;
    v8i a[MS];
#pragma unroll
    for (int i = 0; i < MS; ++i) {
        const uint32_t r = a_row0 + 16u * i + (lane & 15u);
        const uint4 lo = sa_lds[r * 8u + (g ^ sw)];
        const uint4 hi = sa_lds[r * 8u + ((4u + g) ^ sw)];
        a[i] = v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
    }
    v8i b = b_frag<0>(sb_lds, b_row0, lane);
    __builtin_amdgcn_sched_barrier(0);
    int sa[MS / 4], sb[NS / 4];
#pragma unroll
    for (int j = 0; j < MS / 4; ++j) sa[j] = plain_scale_pick(ra[j], sel);
#pragma unroll
    for (int j = 0; j < NS / 4; ++j) sb[j] = plain_scale_pick(rb[j], sel);
    (mma_b<J>(acc, a, b, sb_lds, b_row0, lane, sa, sb), ...);
}

// ---------------------------------------------------------------------------
// Form for scales in the matrix-core layout (the default consumer path).
//
// Measured on MI355X, mx_gemm_kernel is bound by LDS throughput: a 64 x 64
// wave tile reads 16 KB of fragments per 16 instructions.  Counters showed
// the LDS data FIFO full 58% of cycles, no bank conflicts and the matrix
// cores busy 30%.  This form changes four things:
//   * wave tiles of 64 x (16 NS): NS = 8 (64 x 128, a 256 x 256 tile of 8
//     waves, 2 per SIMD) reads a quarter fewer LDS bytes per instruction;
//     row groups use NS = 4 (128 x 256 tiles, since a group unit is 128 rows).
//     128 x 128 wave tiles (4 waves, accumulators in the AGPRs) were slower:
//     one wave per SIMD does not hide the LDS and barrier latency;
//   * operands and the step's scale dwords go straight from global memory
//     into LDS (buffer loads with the LDS destination); no registers stage
//     them and no LDS writes are issued;
//   * those loads and the workgroup barrier are written as instructions with
//     explicit waits.  The compiler's barrier waits for every outstanding
//     load, which would limit the pipeline to one step ahead; loads complete
//     in issue order, so at step s a wave waits until only the later steps'
//     loads are outstanding.  With three stages (NS = 4) loads run two steps
//     ahead; the 256 x 256 tile fits two stages;
//   * the result goes through LDS and leaves as full 16-byte pieces of C
//     rows with non-temporal stores (the weight gradient, whose groups are
//     short, is bound by writing C).
// Each wave issues the same number of loads per step (its A and B pieces
// and its scale runs; runs past the last repeat it into a spare slot), which
// is what the waits count.
// ---------------------------------------------------------------------------

typedef int v4i __attribute__((ext_vector_type(4)));

// Buffer resource for base (uniform): raw, 4 GiB range.
__device__ __forceinline__ v4i pipe_rsrc(const uint8_t* base) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    v4i r;
    r.x = __builtin_amdgcn_readfirstlane(int(uint32_t(b)));
    r.y = __builtin_amdgcn_readfirstlane(int(uint32_t(b >> 32)));
    r.z = -1;
    r.w = 0x00020000;
    return r;
}

// 16 (or 4) bytes per lane from the buffer at voff + soff into LDS at
// lds + 16 (or 4) * lane; lds and soff are uniform.
__device__ __forceinline__ void pipe_load16(v4i r, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(lds)
                 : "memory");
}
// The same with the non-temporal hint, for operands each CU reads once
// (the experts' weights of a row-grouped contraction).
__device__ __forceinline__ void pipe_load16_nt(v4i r, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen nt lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(lds)
                 : "memory");
}
__device__ __forceinline__ void pipe_load4(v4i r, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(lds)
                 : "memory");
}

// Wait until at most kLeft of this wave's loads are outstanding and its LDS
// reads are done, then synchronize the workgroup.
template <int kLeft>
__device__ __forceinline__ void pipe_sync() {
    static_assert(kLeft >= 0 && kLeft < 16, "vmcnt immediate");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kLeft) : "memory");
}

// Configuration: WM x WN waves of (16 MS) x (16 NS) each; the tile is
// (16 MS WM) x (16 NS WN).  Every wave issues kLoads loads per step: its
// share of the A and B pieces and kRpw scale runs (runs past the last repeat
// it into spare slots).
template <int MS, int NS, int WM, int WN>
struct Pipe {
    static constexpr int kWaves = WM * WN, kThreads = 64 * kWaves;
    static constexpr int kTM = 16 * MS * WM, kTN = 16 * NS * WN;
    static constexpr int kLA = 2 * MS / WN, kLB = 2 * NS / WM;   // 16-byte loads per wave and step
    static constexpr int kRunsA = kTM / 64, kRuns = kTM / 64 + kTN / 64;
    static constexpr int kRpw = (kRuns + kWaves - 1) / kWaves;    // scale runs per wave
    static constexpr uint32_t kA = 0, kB = uint32_t(kTM) * 128, kS = kB + uint32_t(kTN) * 128;
    static constexpr uint32_t kStage = kS + uint32_t(kWaves * kRpw) * 256;
    static constexpr int kStages = (160 * 1024) / kStage >= 3 ? 3 : 2;
    static constexpr int kLoads = kLA + kLB + kRpw;
    static_assert(kLA * WN == 2 * MS && kLB * WM == 2 * NS, "pieces divide evenly over the waves");
    static_assert(kStages == 2 || kLoads < 16, "vmcnt immediate");
};

// Group ends of a row-grouped contraction, read 64 at a time (one load per
// lane, then a prefix maximum across the wave).  The ends are rounded down
// to multiples of 128 and clamped to an ascending sequence inside [0, M]
// (valid offsets already are), so the row tiles they delimit partition the
// rows whatever offs holds.  Returns the last clamped end (the first row of
// the uncovered tail); with row >= 0, *group receives the number of ends at
// or below `row`, i.e. the group whose rows contain it (G for the tail).
// Every wave of a workgroup computes the same values, held wave-uniform, so
// no barrier is needed.
__device__ __forceinline__ int32_t uniform(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ int32_t group_ends(const GemmArgs& p, int64_t row, int32_t* group) {
    const uint32_t lane = threadIdx.x & 63u;
    int32_t c_carry = 0;
    int32_t below = 0;
    for (int32_t base = 0; base < p.G; base += 64) {
        const int32_t g = base + int32_t(lane);
        int32_t c = 0;
        if (g < p.G) {
            const int64_t o = (int64_t(p.offs[g]) / 128) * 128;
            c = int32_t(o < 0 ? 0 : (o > p.M ? p.M : o));
        }
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int32_t o = __shfl_up(c, d, 64);
            if (lane >= uint32_t(d)) c = max(c, o);
        }
        c = max(c, c_carry);
        if (row >= 0) below += uniform(__builtin_popcountll(__ballot(g < p.G && int64_t(c) <= row)));
        c_carry = uniform(__shfl(c, 63, 64));
    }
    if (row >= 0) *group = below;
    return c_carry;
}

// kStreamB: B's loads carry the non-temporal hint.  The row-grouped forward
// streams each expert's weights through the CUs of one or two row tiles;
// measured on MI355X (byte-identical output) the hint takes it from
// 182-184 us to 172-177 us, while it slows the dense product (455 -> 492 us)
// and the contraction-grouped weight gradient (331 -> 411 us), whose B tiles
// are re-read from the caches.
template <int kOut, int MS, int NS, int WM, int WN, int kSF, bool kStreamB>
__global__ __launch_bounds__(64 * WM * WN, WM * WN >= 8 ? 2 : 1)
void mx_gemm_pipe_kernel(GemmArgs p) {
    using P = Pipe<MS, NS, WM, WN>;
    constexpr int kEsz = kOut == 0 ? 4 : 2;
    constexpr int kPitch = 16 * NS * kEsz + 16;                 // staged result row, bytes
    // kScalesRows4: stages hold operands only; two period buffers of the
    // scale runs (1 KiB each: 64 rows x 16 bytes) follow them
    constexpr bool kPer = kSF == kScalesRows4;
    constexpr uint32_t kStageB = kPer ? P::kS : P::kStage;
    constexpr uint32_t kPA = P::kStages * kStageB;
    constexpr uint32_t kRunB = 1024u;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kPA + (kPer ? 2u * P::kRuns * kRunB : 0u)];
    static_assert(kPA + (kPer ? 2u * P::kRuns * kRunB : 0u) <= 160u * 1024u, "LDS");

    const uint32_t t = threadIdx.x, lane = t & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const uint32_t wm = wave / WN, wn = wave % WN;

    // ---- which tile, which group, which range of the contraction ----
    int64_t m0;
    uint32_t tn;
    int64_t k_lo = 0, k_hi = p.K;
    const uint8_t* B = p.B;
    const uint8_t* sB = p.sB;
    char* C = static_cast<char*>(p.C);
    bool zero = false;
    if (p.mode == 0) {
        if (p.offs != nullptr) {
            // Row groups (launched with 128-row tiles only: one group unit).
            // Workgroups are dealt to the 8 XCDs in turn, each with its own
            // L2.  XCD x (workgroups x, x + 8, ...) takes a contiguous range of the
            // covered row tiles, every column tile of one row tile in a row,
            // then its share of the uncovered tail (written as 0).  A row
            // tile's activations are then fetched into one L2 only, and
            // neighbouring row tiles, which mostly belong to one group, share
            // their expert's weights there.  The ranges partition the row
            // tiles; workgroups past their XCD's share exit.
            const uint32_t xcd = blockIdx.x & 7u, j = blockIdx.x >> 3;
            const uint32_t lr = j / p.tiles_n;
            tn = j - lr * p.tiles_n;
            const uint32_t cov = uint32_t(group_ends(p, -1, nullptr)) / 128u;
            const uint32_t tail = p.tiles_m - cov;
            const uint32_t c0 = cov * xcd / 8u, c1 = cov * (xcd + 1u) / 8u;
            const uint32_t t0 = cov + tail * xcd / 8u, t1 = cov + tail * (xcd + 1u) / 8u;
            uint32_t tm;
            if (lr < c1 - c0) tm = c0 + lr;
            else if (lr < (c1 - c0) + (t1 - t0)) tm = t0 + (lr - (c1 - c0));
            else return;                                         // uniform: the whole workgroup
            m0 = int64_t(tm) * P::kTM;
            int32_t g = p.G;
            group_ends(p, m0, &g);
            if (g >= p.G) {
                zero = true;
            } else {
                B += int64_t(g) * p.b_gs;
                sB += int64_t(g) * p.sb_gs;
            }
        } else {
            m0 = int64_t(blockIdx.x % p.tiles_m) * P::kTM;
            tn = blockIdx.x / p.tiles_m;
        }
    } else {
        const uint32_t per = p.tiles_m * p.tiles_n;
        const uint32_t g = blockIdx.x / per, r = blockIdx.x - g * per;
        m0 = int64_t(r % p.tiles_m) * P::kTM;
        tn = r / p.tiles_m;
        k_lo = g == 0 ? 0 : clamp_end(p.offs[g - 1], 0, p.K);
        k_hi = clamp_end(p.offs[g], k_lo, p.K);
        C += int64_t(g) * p.c_gs * kEsz;
    }
    const int64_t n0 = int64_t(tn) * P::kTN;
    const int64_t n = zero ? 0 : (k_hi - k_lo) / kTile;

    // ---- load plan (all offsets fit 32 bits: a tile spans <= 256 rows of <= 2^24 bytes) ----
    const uint32_t lda = uint32_t(p.lda), ldb = uint32_t(p.ldb);
    const uint32_t lr = lane >> 3, lc = (lane & 7u) ^ (lane >> 3);
    const uint32_t voa = lr * lda + 16u * lc, vob = lr * ldb + 16u * lc;
    // M and N are multiples of 128: rows past a ragged last tile wrap onto valid rows
    const uint32_t a_mask = uint32_t(min(int64_t(P::kTM), p.M - m0)) - 1u;
    const uint32_t b_mask = uint32_t(min(int64_t(P::kTN), p.N - n0)) - 1u;
    const v4i ra = pipe_rsrc(p.A + m0 * p.lda);
    const v4i rb = pipe_rsrc(B + n0 * p.ldb);
    // scale runs of this wave (A groups first, then B groups; groups past a
    // ragged last tile clamp to the last one; runs past the last repeat it)
    const int64_t ga_max = p.M / 64 - 1 - m0 / 64, gb_max = p.N / 64 - 1 - n0 / 64;
    // the scales of the tile's first row, and per run: the run's offset from
    // there, the offset added per contraction step and the lane's offset
    constexpr bool kRowsForm = kSF == kScalesRows || kSF == kScalesRows4;
    const int64_t a_org = kSF == kScalesMfma ? (m0 / 64) * p.sa_rs : kRowsForm ? m0 * p.sa_rs : m0;
    const int64_t b_org = kSF == kScalesMfma ? (n0 / 64) * p.sb_rs : kRowsForm ? n0 * p.sb_rs : n0;
    const v4i rs_a = pipe_rsrc(p.sA + a_org);
    const v4i rs_b = pipe_rsrc(sB + b_org);
    bool run_a[P::kRpw];
    uint32_t s_run_off[P::kRpw], s_step[P::kRpw], v_run[P::kRpw], slot[P::kRpw];
#pragma unroll
    for (int r = 0; r < P::kRpw; ++r) {
        const uint32_t run = min(wave * uint32_t(P::kRpw) + uint32_t(r), uint32_t(P::kRuns - 1));
        slot[r] = run;
        run_a[r] = run < uint32_t(P::kRunsA);
        const uint32_t g = run_a[r] ? uint32_t(min(int64_t(run), ga_max)) : uint32_t(min(int64_t(run - P::kRunsA), gb_max));
        const uint32_t rs = uint32_t(run_a[r] ? p.sa_rs : p.sb_rs), bs = uint32_t(run_a[r] ? p.sa_bs : p.sb_bs);
        if constexpr (kSF == kScalesMfma) {
            s_run_off[r] = g * rs; s_step[r] = 256u; v_run[r] = 4u * lane;
        } else if constexpr (kRowsForm) {
            s_run_off[r] = 64u * g * rs; s_step[r] = 4u; v_run[r] = lane * rs;
        } else {
            s_run_off[r] = 64u * g; s_step[r] = 4u * bs; v_run[r] = (lane >> 4) * bs + 4u * (lane & 15u);
        }
    }
    const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(lds));
    const uint32_t plain_sel = plain_scale_sel<kSF == kScalesMfma || kPer ? kScalesRows : kSF>(lane);
#define MXQ_PIPE_ISSUE(step)                                                                     \
    do {                                                                                         \
        const uint32_t k_ = uint32_t(k_lo + int64_t(step) * kTile);                              \
        const uint32_t st_ = lds0 + uint32_t((step) % P::kStages) * kStageB;                     \
        _Pragma("unroll") for (int q_ = 0; q_ < P::kLA; ++q_) {                                  \
            const uint32_t j_ = uint32_t(P::kLA) * wave + q_;                                    \
            pipe_load16(ra, st_ + P::kA + 1024u * j_, voa, ((8u * j_) & a_mask) * lda + k_);     \
        }                                                                                        \
        _Pragma("unroll") for (int q_ = 0; q_ < P::kLB; ++q_) {                                  \
            const uint32_t j_ = uint32_t(P::kLB) * wave + q_;                                    \
            if constexpr (kStreamB) pipe_load16_nt(rb, st_ + P::kB + 1024u * j_, vob, ((8u * j_) & b_mask) * ldb + k_); \
            else pipe_load16(rb, st_ + P::kB + 1024u * j_, vob, ((8u * j_) & b_mask) * ldb + k_); \
        }                                                                                        \
        if constexpr (!kPer)                                                                     \
            _Pragma("unroll") for (int r_ = 0; r_ < P::kRpw; ++r_)                               \
                pipe_load4(run_a[r_] ? rs_a : rs_b, st_ + P::kS + 256u * (wave * P::kRpw + r_), v_run[r_], \
                           s_run_off[r_] + (k_ / uint32_t(kTile)) * s_step[r_]);                  \
    } while (0)
    // kScalesRows4: the scale runs of steps 4 q .. 4 q + 3, 16 bytes per row,
    // into period buffer q % 2 (the contraction starts at 0)
#define MXQ_PERIOD_ISSUE(q)                                                                      \
    do {                                                                                         \
        _Pragma("unroll") for (int r_ = 0; r_ < P::kRpw; ++r_)                                   \
            pipe_load16(run_a[r_] ? rs_a : rs_b,                                                 \
                        lds0 + kPA + uint32_t((q) & 1) * (P::kRuns * kRunB) + kRunB * slot[r_], v_run[r_], \
                        s_run_off[r_] + 16u * uint32_t(q));                                      \
    } while (0)

    v4f acc[MS][NS];
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // Every step's issue group is its operand loads (and, without kPer, its
    // scale runs).  With kPer, period 0 goes out with step 0 and period
    // q + 1 with the group issued at step 4 q, ahead of its operand loads.
    constexpr int kOps = P::kLA + P::kLB;
#pragma unroll
    for (int s0 = 0; s0 < P::kStages - 1; ++s0) {
        if (s0 < n) {
            if constexpr (kPer)
                if (s0 == 0) MXQ_PERIOD_ISSUE(0);
            MXQ_PIPE_ISSUE(s0);
        }
    }
    for (int64_t s = 0; s < n; ++s) {
        // step s's loads are in LDS (the later issued steps may still be in
        // flight) and the stage step s - 1 used is free
        if constexpr (P::kStages == 3) {
            if constexpr (kPer) {
                // what may stay in flight: the group issued at step s - 1
                const bool ops = s + 1 < n;
                const bool per = s >= 1 && (s - 1) % 4 == 0 && 4 * ((s - 1) / 4 + 1) < n;
                if (ops && per) pipe_sync<kOps + P::kRpw>();
                else if (ops) pipe_sync<kOps>();
                else if (per) pipe_sync<P::kRpw>();
                else pipe_sync<0>();
            } else {
                if (s + 1 < n) pipe_sync<P::kLoads>();
                else pipe_sync<0>();
            }
        } else {
            pipe_sync<0>();
        }
        if constexpr (kPer)
            if (s % 4 == 0 && 4 * (s / 4 + 1) < n) MXQ_PERIOD_ISSUE(s / 4 + 1);
        if (s + P::kStages - 1 < n) MXQ_PIPE_ISSUE(s + P::kStages - 1);
        const uint8_t* st = lds + uint32_t(s % P::kStages) * kStageB;
        const uint8_t* sc = kPer ? lds + kPA + uint32_t((s / 4) & 1) * (P::kRuns * kRunB) : st + P::kS;
        constexpr uint32_t kRunStride = kPer ? kRunB : 256u;
        const uint8_t* runs_a = sc + kRunStride * ((MS / 4) * wm);
        const uint8_t* runs_b = sc + kRunStride * (P::kRunsA + (NS / 4) * wn);
        if constexpr (kSF == kScalesMfma) {
            int sa[MS / 4], sb[NS / 4];
#pragma unroll
            for (int j = 0; j < MS / 4; ++j) sa[j] = *reinterpret_cast<const int*>(runs_a + 256u * j + 4u * lane);
#pragma unroll
            for (int j = 0; j < NS / 4; ++j) sb[j] = *reinterpret_cast<const int*>(runs_b + 256u * j + 4u * lane);
            mma_step<MS, NS>(acc, reinterpret_cast<const uint4*>(st + P::kA),
                             reinterpret_cast<const uint4*>(st + P::kB), wm * 16u * MS, wn * 16u * NS, lane, sa, sb,
                             std::make_integer_sequence<int, NS>{});
        } else {
            uint32_t ra[MS / 4][4], rb[NS / 4][4];
            if constexpr (kPer) {
                const uint32_t sub = uint32_t(s) & 3u;
#pragma unroll
                for (int j = 0; j < MS / 4; ++j) period_scale_read(runs_a + kRunB * j, lane, sub, ra[j]);
#pragma unroll
                for (int j = 0; j < NS / 4; ++j) period_scale_read(runs_b + kRunB * j, lane, sub, rb[j]);
            } else {
#pragma unroll
                for (int j = 0; j < MS / 4; ++j) plain_scale_read<kSF>(runs_a + 256u * j, lane, ra[j]);
#pragma unroll
                for (int j = 0; j < NS / 4; ++j) plain_scale_read<kSF>(runs_b + 256u * j, lane, rb[j]);
            }
            __builtin_amdgcn_sched_barrier(0);
            mma_step_plain<MS, NS>(acc, reinterpret_cast<const uint4*>(st + P::kA),
                                   reinterpret_cast<const uint4*>(st + P::kB), wm * 16u * MS, wn * 16u * NS, lane,
                                   ra, rb, plain_sel, std::make_integer_sequence<int, NS>{});
        }
    }
#undef MXQ_PIPE_ISSUE
#undef MXQ_PERIOD_ISSUE
    __syncthreads();

    // ---- epilogue through LDS: 16 rows of the wave tile at a time, 16-byte non-temporal stores ----
    // acc[i][j][v] is C[m0 + 16 MS wm + 16 i + 4 (lane / 16) + v][n0 + 16 NS wn + 16 j + lane % 16]
    uint8_t* ep = lds + wave * (16 * kPitch);
    constexpr int kPieces = 16 * NS * kEsz / 16;               // 16-byte pieces per staged row
#pragma unroll
    for (int i = 0; i < MS; ++i) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const uint32_t row = 4u * (lane >> 4) + v, col = 16u * j + (lane & 15u);
                const float x = acc[i][j][v];
                if (kOut == 0) *reinterpret_cast<float*>(ep + row * kPitch + col * 4u) = x;
                else *reinterpret_cast<__bf16*>(ep + row * kPitch + col * 2u) = __bf16(x);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);                     // lgkmcnt(0): this wave's staging writes done
        __builtin_amdgcn_wave_barrier();
        const int64_t row0 = m0 + 16 * MS * wm + 16 * i;
        const int64_t col0 = n0 + 16 * NS * wn;
#pragma unroll
        for (int q = 0; q < 16 * kPieces / 64; ++q) {
            const uint32_t piece = 64u * q + lane;
            const uint32_t row = piece / kPieces, pc = piece % kPieces;
            const int64_t grow = row0 + row, gcol = col0 + pc * (16 / kEsz);
            const uint4 val = *reinterpret_cast<const uint4*>(ep + row * kPitch + 16u * pc);
            if (grow < p.M && gcol < p.N) {
                const u32x4 vv = {val.x, val.y, val.z, val.w};
                __builtin_nontemporal_store(vv, reinterpret_cast<u32x4*>(C + (grow * p.ldc + gcol) * kEsz));
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);                     // reads done before the next chunk's writes
        __builtin_amdgcn_wave_barrier();
    }
}

// The plain scale form a view allows the pipelined kernel to load, or -1:
// rows form (block stride 1, row stride a multiple of 4), blocks form (row
// stride 1, block stride a multiple of 4); the base and the per-group stride
// keep every dword 4-byte aligned, and every offset fits 31 bits.
int plain_scale_form(const uint8_t* s, int64_t rs, int64_t bs, int64_t K, int64_t gs) {
    if (reinterpret_cast<uintptr_t>(s) % 4 != 0 || gs % 4 != 0) return -1;
    if (bs == 1 && rs > 0 && rs % 4 == 0 && rs < (int64_t(1) << 24)) return kScalesRows;
    if (rs == 1 && bs > 0 && bs % 4 == 0 && (K / 32 + 4) * bs < (int64_t(1) << 31)) return kScalesBlocks;
    return -1;
}

// Row groups: 128-row tiles (one group unit) of 8 waves; otherwise 256 x 256.
template <int kSF>
hipError_t launch_pipe(GemmArgs& p, int out_dtype, hipStream_t stream) {
    if (p.mode == 0 && p.offs != nullptr) {
        // 128 x 256 tiles (a group unit is 128 rows).  Each XCD's share is at
        // most ceil(tiles_m / 8) + 1 row tiles (its covered range and its
        // tail range are each at most a ceiling).  (Measured on MI355X for the
        // workload's 64 groups: covering the pairs of units inside a group with
        // 256 x 256 tiles in a second launch, whose 64 x 128 wave tiles run the
        // matrix cores faster, took 259 us instead of 187 us: 280 such tiles
        // need two rounds of the 256 CUs, and the odd units a third.)
        using P = Pipe<4, 4, 2, 4>;
        p.tiles_m = uint32_t(p.M / P::kTM);
        p.tiles_n = uint32_t((p.N + P::kTN - 1) / P::kTN);
        const dim3 grid(8u * ((p.tiles_m + 7u) / 8u + 1u) * p.tiles_n), block(P::kThreads);
        if (out_dtype == 0) hipLaunchKernelGGL((mx_gemm_pipe_kernel<0, 4, 4, 2, 4, kSF, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((mx_gemm_pipe_kernel<1, 4, 4, 2, 4, kSF, true>), grid, block, 0, stream, p);
    } else {
        using P = Pipe<4, 8, 4, 2>;
        p.tiles_m = uint32_t((p.M + P::kTM - 1) / P::kTM);
        p.tiles_n = uint32_t((p.N + P::kTN - 1) / P::kTN);
        const dim3 grid(p.tiles_m * p.tiles_n * uint32_t(p.mode == 1 ? p.G : 1)), block(P::kThreads);
        if (out_dtype == 0) hipLaunchKernelGGL((mx_gemm_pipe_kernel<0, 4, 8, 4, 2, kSF, false>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((mx_gemm_pipe_kernel<1, 4, 8, 4, 2, kSF, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_gemm(const uint8_t* A, int64_t lda, const uint8_t* sA, int64_t sa_rs, int64_t sa_bs,
                          const uint8_t* B, int64_t ldb, int64_t b_gs, const uint8_t* sB, int64_t sb_rs,
                          int64_t sb_bs, int64_t sb_gs, void* C, int64_t ldc, int64_t c_gs, int64_t M, int64_t N,
                          int64_t K, const int32_t* offs, int32_t G, int mode, int out_dtype, bool mfma_scales,
                          hipStream_t stream) {
    GemmArgs p;
    p.A = A; p.lda = lda; p.sA = sA; p.sa_rs = sa_rs; p.sa_bs = sa_bs;
    p.B = B; p.ldb = ldb; p.b_gs = b_gs; p.sB = sB; p.sb_rs = sb_rs; p.sb_bs = sb_bs; p.sb_gs = sb_gs;
    p.C = C; p.ldc = ldc; p.c_gs = c_gs;
    p.M = M; p.N = N; p.K = K; p.offs = offs; p.G = G; p.mode = mode;
    if (mfma_scales) {
        // the K/32 scale bytes of each of 64 rows
        p.sa_rs = p.sb_rs = 2 * K;
        p.sa_bs = p.sb_bs = 0;
    }
    // the pipelined kernel stores 16-byte pieces of C rows, and loads plain
    // scales as dwords of one row's 4 blocks or of one block's 4 rows
    const int64_t esz = out_dtype == 0 ? 4 : 2;
    const bool rows16 = (reinterpret_cast<uintptr_t>(C) % 16 == 0) && (ldc * esz) % 16 == 0 &&
                        (mode != 1 || (c_gs * esz) % 16 == 0);
    int sf = kScalesMfma;
    if (!mfma_scales) {
        const bool row_groups = mode == 0 && offs != nullptr;
        const int fa = plain_scale_form(sA, sa_rs, sa_bs, K, 0);
        const int fb = plain_scale_form(sB, sb_rs, sb_bs, K, row_groups ? sb_gs : 0);
        sf = fa == fb ? fa : -1;
    }
    if (sf >= 0 && rows16) {
        if (sf == kScalesMfma) return launch_pipe<kScalesMfma>(p, out_dtype, stream);
        if (sf == kScalesRows) {
            // four steps of scales per load: 16-byte aligned rows, whole periods
            // from the contraction's start (row groups: each expert's scales too)
            const bool per = mode == 0 && K % 512 == 0 && reinterpret_cast<uintptr_t>(sA) % 16 == 0 &&
                             reinterpret_cast<uintptr_t>(sB) % 16 == 0 && sa_rs % 16 == 0 && sb_rs % 16 == 0 &&
                             (offs == nullptr || sb_gs % 16 == 0);
            if (per) return launch_pipe<kScalesRows4>(p, out_dtype, stream);
            return launch_pipe<kScalesRows>(p, out_dtype, stream);
        }
        return launch_pipe<kScalesBlocks>(p, out_dtype, stream);
    }
    p.tiles_m = uint32_t(M / kTile);
    p.tiles_n = uint32_t(N / kTile);
    const uint32_t tiles = p.tiles_m * p.tiles_n * uint32_t(mode == 1 ? G : 1);
    const dim3 grid(tiles), block(kThreads);
    if (out_dtype == 0) {
        if (mfma_scales) hipLaunchKernelGGL((mx_gemm_kernel<0, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((mx_gemm_kernel<0, false>), grid, block, 0, stream, p);
    } else {
        if (mfma_scales) hipLaunchKernelGGL((mx_gemm_kernel<1, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((mx_gemm_kernel<1, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace mxq
