// Dense FP32 GEMM for AMD MI355X (gfx950 / CDNA4): kernels and the C ABI.
//
// C[M x N] = A[M x K] . B[K x N], row-major binary32 (the product of the
// UIUC ECE408 Lecture 12 final-project page, project_template.cu section 2).
//
// Kernels:
//
//  * gemm_f32_mfma_dma<Tile, SK, SPLIT, STRIP, WB>: the main kernel.  One workgroup per
//    BM x BN tile of C; K is walked in BK-deep panels that buffer loads write
//    straight into a ring of LDS buffers, so later panels are fetched while
//    the matrix cores work on the current one (one barrier per panel).  Each
//    wave owns a (BM/WAVES_M) x (BN/WAVES_N) block of C held in 32 x 32
//    accumulators of v_mfma_f32_32x32x2_f32; optional K-split wave groups
//    inside the workgroup, stream-K across workgroups (SK) and split-K
//    through a caller's workspace (SPLIT).  The largest tiles (4 waves of
//    128 x 128 or 64 x 64) and the K-split tile of one-wave groups run a
//    software-pipelined round loop (PIPE) that interleaves fragment reads
//    and panel loads with the MFMAs.  Ragged edges are zero-filled on load
//    and masked on store, so every shape runs on this path.  C is written
//    with streaming stores, or (WB twins, for a large C whose rows are not
//    16-byte aligned) with ordinary write-back stores.
//  * gemm_f32_mfma<Tile, VEC_A, VEC_B>: the same tiling with panels staged
//    global -> VGPR -> LDS, for rows too long for 32-bit buffer offsets.
//  * gemm_f32_valu: a 64 x 64 LDS-tiled vector-FMA kernel (4 x 4 outputs per
//    thread) for problems too small to fill a matrix-core tile.
//  * fill_zero (K = 0), zero_shared_tiles (stream-K) and splitk_reduce
//    (split-K) as helpers.
//
// The pages' kernels (Lecture 5 and 12 notes, the cuda-gemm README) were
// written for NVIDIA parts; what carries over is the structure -- output
// tiling, K-panels in on-chip memory, register blocking, vector loads, double
// buffering -- while the inner product runs on CDNA4 FP32 matrix cores with
// 64-wide waves.

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <atomic>
#include <type_traits>
#include <stdio.h>
#include <string.h>

#include "gemm_f32.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaveSize = 64;
constexpr int64_t kMaxGrid = 1 << 20;  // workgroups per launch; larger jobs loop

struct GemmArgs {
    const float *A;
    const float *B;
    float *C;
    int64_t lda, ldb, ldc;
    int M, N, K;
    int tiles_m, tiles_n;
    int slices;          // K slices of a split-K launch (1 otherwise)
    int64_t slab;        // floats between two slices' partial products in C
    int strip_rows;      // rows M - strip_rows .. M-1 lie below the tile grid
                         // (tiles_m * BM = M - strip_rows): every workgroup
                         // computes a share of their columns with FMAs
    int strip_cols;      // likewise columns N - strip_cols .. N-1, right of
                         // the grid, every workgroup a share of their rows
                         // above the row strip (which holds the corner)
    int xcds;            // dies the device hands workgroups to round-robin
};

// Most rows (columns) a remainder strip may hold, and the most columns
// (rows) of it one workgroup sums.
constexpr int kMaxStripRows = 4;
constexpr int kMaxBothStripsK = 3072;   // largest K planned with a row and a column strip
constexpr int kMaxStripSpread = 8;
constexpr int kMaxThreads = 1024;      // threads of the largest workgroup
// LDS floats a strip block's partial sums take (strip_block), at most.
constexpr int kStripRed = kMaxStripSpread * kMaxStripSpread * (kMaxThreads / 4 + 1);

// ---------------------------------------------------------------------------
// Tile scheduling
// ---------------------------------------------------------------------------

// Workgroups are handed to the XCDs round-robin (on a whole MI355X, workgroup
// w runs on XCD w mod 8), and each XCD has its own L2.  Renumber so that each
// XCD receives a contiguous range of logical tiles; neighbouring tiles share
// A rows and B columns, so their panels are fetched once per L2.
__device__ inline int xcd_contiguous(int w, int total, int xcds)
{
    const int per = total / xcds;
    const int rem = total % xcds;
    const int xcd = w % xcds;
    return xcd * per + (xcd < rem ? xcd : rem) + w / xcds;
}

// Logical tile id -> (tile row, tile column), walking groups of `group` tile
// rows column by column so that concurrently running tiles form a compact
// block of C.
__device__ inline void tile_coords(int t, int tiles_m, int tiles_n, int group,
                                   int &tm, int &tn)
{
    const int per_group = group * tiles_n;
    const int first_m = (t / per_group) * group;
    const int rows = min(tiles_m - first_m, group);
    const int r = t % per_group;
    tm = first_m + r % rows;
    tn = r / rows;
}

// Stream-K work split: the iters = tiles x K-panels units of work, taken in
// tile order, are cut into `workers` contiguous ranges of nearly equal length;
// range b is [floor(b*iters/workers), floor((b+1)*iters/workers)), computed
// without forming the 128-bit product.  When there are at least as many tiles
// as workers every range is at least one tile's panels long, so a tile meets
// at most two ranges.
__device__ inline void streamk_range(int b, int workers, int64_t iters, int64_t &lo, int64_t &hi)
{
    const int64_t q = iters / workers, r = iters % workers;
    lo = q * b + r * b / workers;
    hi = q * (b + 1) + r * (b + 1) / workers;
}

// Epilogue store of one C element.  C is written once and not read again by
// the kernel, so the store is normally marked non-temporal: it streams to
// memory instead of displacing the A and B panels other workgroups still read
// from L2 (measured +1 % on the store-heavy 8192 x 8192 x 128 and on 2048^3).
// With WB (write-back) it is an ordinary store instead: when C's rows are
// not 16-byte aligned, the 128-byte row pieces a store instruction writes
// straddle cache lines, and for a large C streamed partial lines cost far
// more than lines completed in L2 before they are written back
// (4119 x 4789 x 77: 40.6 us against 70.8; 8191 x 8191 x 128: 162 against
// 212).
template <bool WB = false>
__device__ inline void store_c(float *p, float v)
{
    if constexpr (WB)
        *p = v;
    else
        __builtin_nontemporal_store(v, p);
}

// Elements of C from which rows that are not 16-byte aligned are written
// with ordinary stores (the WB kernel instances); below it the partial lines
// still stream (1023 x 1025 x 1000: 28.9 us against 30.7 with ordinary
// stores).  2^23 floats are 32 MiB, the eight L2 caches together.
constexpr int64_t kWriteBackFromElems = int64_t(1) << 23;

// ---------------------------------------------------------------------------
// Guarded loads: 4 consecutive elements of one row, +0.0 outside the matrix.
// VEC = true needs a 16-byte aligned address and a row length that is a
// multiple of 4, so a 4-element chunk is entirely inside or outside.
// ---------------------------------------------------------------------------
template <bool VEC>
__device__ inline f32x4 load_row4(const float *p, bool row_ok, int col, int ncols)
{
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (VEC) {
        if (row_ok && col < ncols)
            v = *reinterpret_cast<const f32x4 *>(p);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (row_ok && col + e < ncols)
                v[e] = p[e];
    }
    return v;
}

// ---------------------------------------------------------------------------
// Tile parameters, and the register-staged matrix-core kernel
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int KSPLIT_ = 1, int STAGES_ = 2,
          int GROUP_ = 8, int LOADERS_ = 0, int PIPE_ = 0, int LOADER_WAVE_ = 0>
struct MfmaTile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    // K-split inside the workgroup: KSPLIT groups of WAVES_M x WAVES_N waves
    // each accumulate every KSPLIT-th K-panel of the same output tile.
    static constexpr int kSplit = KSPLIT_;
    static constexpr int kGroupWaves = WAVES_M * WAVES_N;
    // Software-pipelined tiles may add LOADER_WAVES waves that issue all
    // panel loads while the others only read LDS and run MFMAs.
    static constexpr int kLoaderWaves = LOADER_WAVE_;
    static constexpr bool kLoaderWave = kLoaderWaves != 0;
    static constexpr int kThreads = (kGroupWaves * kSplit + kLoaderWaves) * kWaveSize;
    static constexpr int kWaveM = BM / WAVES_M;      // C rows per wave
    static constexpr int kWaveN = BN / WAVES_N;      // C columns per wave
    static constexpr int kFragM = kWaveM / 32;       // 32x32 accumulators down
    static constexpr int kFragN = kWaveN / 32;       // 32x32 accumulators across
    // Register-staged kernel's LDS panels.  A is kept row-major ([m][k], k
    // contiguous) so one 128-bit read gives a lane 4 consecutive k of its row;
    // the +4 pad makes the 32 rows read by a half-wave fall on distinct banks.
    // B is kept row-major ([k][n]); lanes read consecutive n, and the +8 pad
    // puts the two half-waves (k and k+4) on different banks.
    static constexpr int kStrideA = BK + 4;
    static constexpr int kStrideB = BN + 8;
    static constexpr int kLdsA = BM * kStrideA;
    static constexpr int kLdsB = BK * kStrideB;
    // 4-element chunks each thread moves per panel (register-staged kernel).
    static constexpr int kChunksA = BM * BK / 4 / kThreads;
    static constexpr int kChunksB = BK * BN / 4 / kThreads;
    static constexpr int kGroup = GROUP_;            // tile rows per raster group
    static constexpr int kStages = STAGES_;          // LDS panel buffers per K-split group
    // Waves of each group that issue the direct-to-LDS panel loads (the
    // lowest-numbered ones; 0: all of them).
    static constexpr int kLoaders = LOADERS_ ? LOADERS_ : WAVES_M * WAVES_N;
    // Software-pipelined rounds (direct-to-LDS kernel, 4-wave tiles): see
    // the pipelined branch of gemm_f32_mfma_dma.
    static constexpr bool kPipe = PIPE_ != 0;

    static_assert(BM % (32 * WAVES_M) == 0 && BN % (32 * WAVES_N) == 0, "wave tile");
    static_assert(BK % 8 == 0, "BK feeds k in groups of 8");
    static_assert(kLoaders >= 1 && kLoaders <= WAVES_M * WAVES_N, "loader waves");
    static_assert(!kLoaderWave || (PIPE_ != 0 && KSPLIT_ == 1), "loader waves serve one pipelined group");
};

// The tile that also computes remainder strips (64 x 64, 8 software-
// pipelined one-wave K-split groups on 16-deep panels): the only one the
// shape rule pairs with a strip.  The strip code lives in a separate
// instantiation of its kernel (STRIP), so the plain one keeps its registers.
using StripTile = MfmaTile<64, 64, 16, 1, 1, 8, 2, 8, 0, 1>;

// Whether a tile's panel buffers hold a strip block's partial sums.
template <class T>
constexpr bool strip_fits()
{
    constexpr int stage = T::BM * T::BK + T::BK * T::BN;
    return T::kThreads <= kMaxThreads && kStripRed <= T::kSplit * T::kStages * stage;
}
static_assert(strip_fits<StripTile>(), "strip space in the strip tile's panel buffers");

// One v_mfma_f32_32x32x2_f32 adds, for the 32 x 32 block it accumulates,
// sum over t in {0,1} of a(i,t) * b(t,j), where lane l supplies a(l%32, l/32)
// and b(l/32, l%32).  Lane half h = l/32 therefore plays the role of k.  The
// kernel pairs k = 8g + 4h + s (s = 0..3) in the s-th instruction of k-group
// g: each lane reads its 4 A values with one 128-bit LDS read, every k of the
// panel is used exactly once, and only the order of the sum changes.
//
// Accumulator layout (16 floats per lane): register r of lane l holds
// C(8*(r/4) + 4*(l/32) + r%4, l%32) of the block.
template <class T, bool VEC_A, bool VEC_B>
__global__ __launch_bounds__(T::kThreads) void gemm_f32_mfma(GemmArgs g)
{
    constexpr int BM = T::BM, BN = T::BN, BK = T::BK;
    constexpr int NT = T::kThreads;
    static_assert(T::kSplit == 1 && T::kStages == 2, "the register-staged kernel is double-buffered, unsplit");
    static_assert(BM * BK % (4 * NT) == 0 && T::kChunksA >= 1, "A panel split");
    static_assert(BK * BN % (4 * NT) == 0 && T::kChunksB >= 1, "B panel split");
    static_assert(2 * (T::kLdsA + T::kLdsB) * 4 <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) float lds_a[2][T::kLdsA];
    __shared__ __attribute__((aligned(16))) float lds_b[2][T::kLdsB];

    const int tid = threadIdx.x;
    const int lane = tid % kWaveSize;
    const int wave = tid / kWaveSize;
    const int wave_m = wave / T::WAVES_N;
    const int wave_n = wave % T::WAVES_N;
    const int li = lane % 32;        // row (A) / column (B) within a 32-block
    const int lh = lane / 32;        // lane half: selects k = 8g + 4*lh + s

    const int total = g.tiles_m * g.tiles_n;
    for (int w = blockIdx.x; w < total; w += gridDim.x) {
        const int t = (int)gridDim.x == total ? xcd_contiguous(w, total, g.xcds) : w;
        int tm, tn;
        tile_coords(t, g.tiles_m, g.tiles_n, T::kGroup, tm, tn);
        const int m0 = tm * BM;
        const int n0 = tn * BN;

        // Per-thread panel coordinates (fixed over the K loop).
        int a_row[T::kChunksA], a_col[T::kChunksA];
        int b_row[T::kChunksB], b_col[T::kChunksB];
#pragma unroll
        for (int r = 0; r < T::kChunksA; ++r) {
            const int f = tid + r * NT;
            a_row[r] = f / (BK / 4);
            a_col[r] = (f % (BK / 4)) * 4;
        }
#pragma unroll
        for (int r = 0; r < T::kChunksB; ++r) {
            const int f = tid + r * NT;
            b_row[r] = f / (BN / 4);
            b_col[r] = (f % (BN / 4)) * 4;
        }

        f32x4 stage_a[T::kChunksA];
        f32x4 stage_b[T::kChunksB];
        auto fetch = [&](int k0) {
#pragma unroll
            for (int r = 0; r < T::kChunksA; ++r) {
                const int m = m0 + a_row[r];
                const float *p = g.A + (int64_t)m * g.lda + (k0 + a_col[r]);
                stage_a[r] = load_row4<VEC_A>(p, m < g.M, k0 + a_col[r], g.K);
            }
#pragma unroll
            for (int r = 0; r < T::kChunksB; ++r) {
                const int k = k0 + b_row[r];
                const float *p = g.B + (int64_t)k * g.ldb + (n0 + b_col[r]);
                stage_b[r] = load_row4<VEC_B>(p, k < g.K, n0 + b_col[r], g.N);
            }
        };
        auto stash = [&](int buf) {
#pragma unroll
            for (int r = 0; r < T::kChunksA; ++r)
                *reinterpret_cast<f32x4 *>(&lds_a[buf][a_row[r] * T::kStrideA + a_col[r]]) = stage_a[r];
#pragma unroll
            for (int r = 0; r < T::kChunksB; ++r)
                *reinterpret_cast<f32x4 *>(&lds_b[buf][b_row[r] * T::kStrideB + b_col[r]]) = stage_b[r];
        };

        f32x16 acc[T::kFragM][T::kFragN];
#pragma unroll
        for (int i = 0; i < T::kFragM; ++i)
#pragma unroll
            for (int j = 0; j < T::kFragN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[i][j][r] = 0.f;

        const int ktiles = (g.K + BK - 1) / BK;
        fetch(0);
        stash(0);
        if (ktiles > 1)
            fetch(BK);
        __syncthreads();

        for (int kt = 0; kt < ktiles; ++kt) {
            const int cur = kt & 1;
            // Buffer cur^1 was last read before the previous barrier.
            if (kt + 1 < ktiles) {
                stash(cur ^ 1);
                if (kt + 2 < ktiles)
                    fetch((kt + 2) * BK);
            }
            const float *la = lds_a[cur] + (wave_m * T::kWaveM + li) * T::kStrideA + 4 * lh;
            const float *lb = lds_b[cur] + (4 * lh) * T::kStrideB + wave_n * T::kWaveN + li;
#pragma unroll
            for (int kg = 0; kg < BK / 8; ++kg) {
                f32x4 a[T::kFragM];
                float b[4][T::kFragN];
#pragma unroll
                for (int i = 0; i < T::kFragM; ++i)
                    a[i] = *reinterpret_cast<const f32x4 *>(la + i * 32 * T::kStrideA + 8 * kg);
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int j = 0; j < T::kFragN; ++j)
                        b[s][j] = lb[(8 * kg + s) * T::kStrideB + j * 32];
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int i = 0; i < T::kFragM; ++i)
#pragma unroll
                        for (int j = 0; j < T::kFragN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][s], b[s][j], acc[i][j], 0, 0, 0);
            }
            __syncthreads();
        }

        // Epilogue: each store instruction writes two 128-byte row segments.
#pragma unroll
        for (int i = 0; i < T::kFragM; ++i) {
#pragma unroll
            for (int j = 0; j < T::kFragN; ++j) {
                const int col = n0 + wave_n * T::kWaveN + j * 32 + li;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + wave_m * T::kWaveM + i * 32 + 8 * (r / 4) + 4 * lh + (r % 4);
                    if (row < g.M && col < g.N)
                        store_c(&g.C[(int64_t)row * g.ldc + col], acc[i][j][r]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Matrix-core kernel with direct-to-LDS operand loads.
//
// gfx950 buffer loads can write their result straight into LDS
// (buffer_load_dwordx4 ... lds): lane l of a wave deposits its 16 bytes at
// LDS base + 16*l, so one wave instruction fills 1 KB of LDS with no VGPR
// staging and no ds_write.  The global side only needs 4-byte alignment, so
// every operand takes this path.  Which global element lands in which LDS
// slot is chosen through the per-lane global offset, which is how the
// bank-conflict-avoiding layouts below are produced.  A buffer offset
// outside the resource's range reads as zero (dword by dword), so ragged
// rows, columns and K-tails are zero-filled by pointing their lanes at an
// out-of-range offset.
//
// LDS layouts (per panel, BK = 16, 32 or 64):
//  * A: [BM][BK] floats, the BK/4 16-byte chunks of row r permuted by
//    chunk ^ swz_a<BK>(r), so that the 128-bit fragment reads (32 rows, one
//    chunk per lane half) run without bank conflicts.
//  * B: [BK][BN] floats; in rows with bit 2 of k set, columns are stored at
//    col ^ 32.  The two lane halves read rows k and k+4 (same columns), which
//    the swap moves onto different banks.
// Buffer resources are rebased on every panel (A at row m0 / column k0, B at
// row k0 / column n0), so every in-range offset stays below 2^31.
// ---------------------------------------------------------------------------
constexpr uint32_t kOutOfRange = 0x80000000u;   // buffer offset that reads as 0
constexpr int kRawBufferFlags = 0x00020000;      // dword 3 of a raw buffer resource

// Debug build (-DGEMM_F32_POISON_LDS): every LDS slot a panel load is about
// to fill is first set to NaN by the wave that issues the load, and every
// fold, band and strip region is set to NaN before it is written.  A read of
// a slot before its data has landed, or of a region slot nobody wrote, then
// carries NaN into C, which every parity check catches; with the normal
// build such a read would pick up stale but finite values.
#ifdef GEMM_F32_POISON_LDS
constexpr bool kPoisonLds = true;
#else
constexpr bool kPoisonLds = false;
#endif

__device__ inline void poison16(float *p)
{
    const float nan = __builtin_nanf("");
    *reinterpret_cast<f32x4 *>(p) = f32x4{nan, nan, nan, nan};
}

// NaN over `floats` floats of LDS from `base` (16-byte aligned, a multiple
// of 4 floats), by `threads` threads of which this is thread `t`.
__device__ inline void poison_region(float *base, int floats, int t, int threads)
{
    for (int e = 4 * t; e < floats; e += 4 * threads)
        poison16(base + e);
}

// One workgroup's block of a remainder strip: C[ar0 + r][bc0 + c] =
// sum over k of A[ar0 + r][k] * B[k][bc0 + c] for r < nr <= R, c < nc <= CW,
// with vector FMAs.  Lane groups of CW threads share a k and take one column
// each (c = tid % CW), so a wave's B loads cover 64 / CW rows of CW
// consecutive columns and its A loads 64 / CW consecutive k of a row.
// Thread tid takes k = tid / CW, + NT / CW, ..., loads kBatch = 64 / R of
// them at a time (one memory latency per batch; R x kBatch A values in
// registers) and sums them in k order; the NT / CW sums of each output are then added through
// LDS (`red`, kStripRed floats) in thread order, 16 runs of consecutive
// threads' sums and then the runs, so the result does not depend on
// scheduling.  All NT threads call it (it has barriers).  Kept
// out of line so that the tile kernel around it keeps its registers.
template <int NT, int CW, int R>
__device__ __noinline__ void strip_block(const float *A, int64_t lda, const float *B, int64_t ldb, float *C,
                                         int64_t ldc, int K, int ar0, int nr, int bc0, int nc, float *red, int tid)
{
    static_assert(R <= kMaxStripSpread, "rows of a block");
    constexpr int KS = NT / CW;                // k's one pass covers
    constexpr int PAD = KS + 1;                // sums per output, padded against bank conflicts
    constexpr int kBatch = 64 / R;             // k's per thread loaded at once (R x kBatch A values)
    static_assert(NT % CW == 0 && (R * CW * PAD + 3) / 4 * 4 <= kStripRed, "strip sums fit");
    // A and B are global memory: address them as such (global instead of
    // flat loads).
    using gfloat = const __attribute__((address_space(1))) float;
    gfloat *ga = (gfloat *)A, *gb = (gfloat *)B;
    const int c = tid % CW, kk = tid / CW;
    const bool on = c < nc && nr > 0;
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        acc[r] = 0.f;
    if (on) {
        for (int k0 = kk; k0 < K; k0 += kBatch * KS) {
            float a[kBatch][R], b[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int k = k0 + u * KS;
                b[u] = k < K ? gb[(int64_t)k * ldb + bc0 + c] : 0.f;
#pragma unroll
                for (int r = 0; r < R; ++r)
                    a[u][r] = k < K && r < nr ? ga[(int64_t)(ar0 + r) * lda + k] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                if (k0 + u * KS < K) {
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        acc[r] = fmaf(a[u][r], b[u], acc[r]);
                }
        }
    }
    __syncthreads();
    if constexpr (kPoisonLds) {
        poison_region(red, (R * CW * PAD + 3) / 4 * 4, tid, NT);
        __syncthreads();
    }
    // `red` is LDS: address it as such (ds_* instead of flat accesses).
    using lds_float = __attribute__((address_space(3))) float;
    lds_float *sums = (lds_float *)red;
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (on && r < nr)
            sums[(r * CW + c) * PAD + kk] = acc[r];
    __syncthreads();
    // Each output's KS sums in kChunks runs of consecutive threads' sums,
    // then the runs' totals, both in thread order.
    // (A block has at most kMaxStripRows x kMaxStripSpread outputs.)
    constexpr int kChunks = 16, kRun = KS / kChunks;
    static_assert(KS % kChunks == 0 && NT >= kMaxStripRows * kMaxStripSpread * kChunks, "chunked sums");
    float part = 0.f;
    const int o = tid / kChunks, j = tid % kChunks;               // output o = r * nc + cc
    if (o < nr * nc) {
        const lds_float *v = sums + ((o / nc) * CW + o % nc) * PAD + j * kRun;
        part = v[0];
#pragma unroll
        for (int i = 1; i < kRun; ++i)
            part += v[i];
    }
    __syncthreads();
    if (o < nr * nc)
        sums[o * kChunks + j] = part;
    __syncthreads();
    if (tid < nr * nc) {
        const lds_float *v = sums + tid * kChunks;
        float sum = v[0];
#pragma unroll
        for (int i = 1; i < kChunks; ++i)
            sum += v[i];
        store_c(&C[(int64_t)(ar0 + tid / nc) * ldc + bc0 + tid % nc], sum);
    }
    __syncthreads();
}

// Chunk permutation of A-panel row r (BK/4 chunks of 16 bytes per row).
// Chosen by measurement (SQ_LDS_BANK_CONFLICT on 128-bit fragment reads of
// 32 consecutive rows): for 64-byte rows, rows four apart share banks and
// (r >> 2) & 3 rotates them onto different chunks, which reads with no
// conflict cycles; for 128-byte rows (r ^ (r >> 3)) & 7 does, and for
// 256-byte rows r & 15.
template <int BK>
__device__ inline int swz_a(int r)
{
    static_assert(BK == 16 || BK == 32 || BK == 64, "A-panel swizzles exist for 16-, 32- and 64-deep panels");
    return BK == 16 ? (r >> 2) & 3 : BK == 32 ? (r ^ (r >> 3)) & 7 : r & 15;
}

// One wave instruction: lane l's 16 bytes at buffer offset `offset` land at
// lds_base + 16*l.
__device__ inline void buffer_to_lds(__amdgpu_buffer_rsrc_t rsrc, float *lds_base, uint32_t offset)
{
    auto *dst = (__attribute__((address_space(3))) void *)lds_base;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, offset, 0, 0, 0);
}

template <class T, bool SK = false, bool SPLIT = false, bool STRIP = false, bool WB = false>
__global__ __launch_bounds__(T::kThreads) void gemm_f32_mfma_dma(GemmArgs g)
{
    constexpr int BM = T::BM, BN = T::BN, BK = T::BK;
    constexpr int NW = T::kGroupWaves;                // waves per K-split group
    constexpr int KS = T::kSplit;
    constexpr int FM = T::kFragM, FN = T::kFragN;
    static_assert(!(SK && SPLIT), "one way of splitting K across workgroups at a time");
    static_assert(!STRIP || (std::is_same<T, StripTile>::value && !SK && !SPLIT),
                  "remainder strips: data-parallel launches of the strip tile");
    static_assert(BK == 16 || BK == 32 || BK == 64, "the A layout permutes the 16-byte chunks of 16-, 32- or 64-deep rows");
    // B panels 64 or more columns wide swap 32-column halves between rows
    // with bit 2 of k set and clear; 32-wide ones swap neighbouring rows.
    static_assert(BN % 64 == 0 || BN == 32, "B-panel layouts exist for 32 and multiples of 64 columns");
    constexpr bool kNarrowB = BN == 32;
    constexpr int kA = BM * BK;                       // floats per A panel
    constexpr int kB = BK * BN;                       // floats per B panel
    constexpr int kStage = kA + kB;
    constexpr int kVecA = 4, kVecB = 4;               // floats per lane per load (16 bytes)
    constexpr int kSpanA = kWaveSize * kVecA;         // floats one instruction moves
    constexpr int kSpanB = kWaveSize * kVecB;
    // Load instructions per panel, dealt in order to the group's first NL
    // waves; when a panel has fewer instructions than NL times the per-wave
    // count, the last of them skip the missing ones.  With 16 waves, letting
    // only the first 8 load measured fastest: those waves issue first after
    // each barrier, so the loads start at once, while the other 8 go straight
    // to their fragment reads and MFMAs instead of queueing behind the loads
    // (+3.6 % at 2048^3, +1.4 % at 8192^3; 4 or 12 loaders, or the last 8 or
    // every other wave as loaders, were slower).
    // With a loader wave (LW) that wave issues every load instruction of a
    // panel and the group's waves issue none.
    constexpr bool LW = T::kLoaderWave;
    constexpr int NL = LW ? 1 : T::kLoaders;
    constexpr int kInstA = kA / kSpanA, kInstB = kB / kSpanB;
    constexpr int kLoadsA = (kInstA + NL - 1) / NL;   // instructions per loader wave per panel
    constexpr int kLoadsB = (kInstB + NL - 1) / NL;
    constexpr bool kEvenA = kInstA % NL == 0, kEvenB = kInstB % NL == 0;
    static_assert(kA % kSpanA == 0 && kB % kSpanB == 0, "panel split");
    constexpr int S = T::kStages;
    constexpr int kLoads = kLoadsA + kLoadsB;         // per wave per round
    // The 128-bit C epilogue stages kWaveM x BN floats in the panel buffers.
    // It pays where writing C weighs most, the 4-wave tiles chosen for short
    // K; on the 16-wave tiles of long-K problems it measured 0.4-0.8 % slower.
    constexpr bool kBandEpilogue = KS == 1 && NW == 4 && BN >= 64 && T::kWaveM * BN <= S * kStage;
    static_assert(S >= 2 && (LW || (S - 2) * kLoads <= 63), "vmcnt range");
    static_assert(S == 2 || (kEvenA && kEvenB), "partial vmcnt waits need equal per-wave load counts");
    static_assert(KS * S * kStage * 4 <= 160 * 1024, "LDS budget");
    static_assert(KS == 1 || KS * S * kStage >= BM * BN, "the K-split reduction reuses the panel buffers");
    // Each K-split group owns S panel buffers, used as a ring.
    __shared__ __attribute__((aligned(1024))) float lds[KS][S][kStage];

    const int tid = threadIdx.x;
    const int lane = tid % kWaveSize;
    // The wave index is the same in every lane; saying so keeps everything
    // derived from it (LDS destinations of the panel loads, K-split group,
    // loader role) in scalar registers instead of per-lane loops.
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWaveSize);
    const int group = KS == 1 ? 0 : wave / NW;        // K-split group
    const int gw = KS == 1 ? wave : wave % NW;        // wave within its group
    const int wave_m = gw / T::WAVES_N;
    const int wave_n = gw % T::WAVES_N;
    const int li = lane % 32;
    const int lh = lane / 32;

    // Slot -> source element maps, fixed for the whole kernel (loader waves).
    const bool loader = !LW && gw < NL;
    const int lw = loader ? gw : 0;
    uint32_t a_off[kLoadsA];     // byte offset from the panel's (m0, k0) corner
    int a_r[kLoadsA], a_k[kLoadsA];
#pragma unroll
    for (int j = 0; j < kLoadsA; ++j) {
        const int f = (lw * kLoadsA + j) * kSpanA + lane * kVecA;   // LDS slot (float index)
        const int r = f / BK, e = f % BK;
        const int k = 4 * ((e / 4) ^ swz_a<BK>(r)) + e % 4;
        a_r[j] = r;
        a_k[j] = k;
        a_off[j] = (uint32_t)(r * g.lda + k) * 4u;
    }
    uint32_t b_off[kLoadsB];
    int b_k[kLoadsB], b_c[kLoadsB];
#pragma unroll
    for (int j = 0; j < kLoadsB; ++j) {
        const int f = (lw * kLoadsB + j) * kSpanB + lane * kVecB;
        // Wide panels: slot (k, col) holds B(k, col ^ 32) in rows with bit 2
        // of k set.  32-wide panels: slot row p holds B row p ^ bit 2 of p
        // (rows 4..7 of every 8 swapped in pairs), so the two lane halves of
        // a fragment read (rows k and k + 4) fall on different banks.
        const int k = kNarrowB ? (f / BN) ^ ((f / BN >> 2) & 1) : f / BN;
        const int c = kNarrowB ? f % BN : (f % BN) ^ (((k >> 2) & 1) * 32);
        b_k[j] = k;
        b_c[j] = c;
        b_off[j] = (uint32_t)(k * g.ldb + c) * 4u;
    }
    // Fragment read addresses (floats within a panel buffer).
    const int a_frag = (wave_m * T::kWaveM + li) * BK;
    int a_swz[FM];             // chunk permutation of each fragment's row
#pragma unroll
    for (int i = 0; i < FM; ++i)
        a_swz[i] = swz_a<BK>(wave_m * T::kWaveM + i * 32 + li);
    // Column of fragment j after the half swap of rows with bit 2 of k set
    // (k = 8q + 4*lh + s, so that bit is lh); the fragment base is a multiple
    // of 32, so the swap only flips its bit 5.
    // For 32-wide panels, row 8q + 4*lh + s sits in slot row 8q + 4*lh +
    // (s ^ lh): b_frag then holds the lane's slot in row 8q + 4*lh and
    // b_s[s] the offset of its s-th row.
    int b_frag[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j)
        b_frag[j] = kNarrowB ? kA + (4 * lh) * BN + li
                             : kA + (4 * lh) * BN + (((wave_n * T::kWaveN + 32 * j) ^ (32 * lh)) + li);
    int b_s[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
        b_s[s] = (kNarrowB ? (s ^ lh) : s) * BN;

    float (*stage)[kStage] = lds[group];   // this group's ring of S buffers

    const int total = g.tiles_m * g.tiles_n;
    const int ktiles = (g.K + BK - 1) / BK;

    // Output tile t over K-panels [p_begin, p_end), written to cbase (C, or
    // a K slice's partial product in the workspace).  A tile whose panels are
    // split between two workgroups (stream-K) adds its partial sum to C,
    // which holds +0.0 there beforehand; every other tile stores.
    float *cbase = g.C;
    auto work = [&](int t, int p_begin, int p_end) {
        const bool c_vec = ((uintptr_t)cbase & 15u) == 0 && (g.ldc & 3) == 0;
        int tm, tn;
        tile_coords(t, g.tiles_m, g.tiles_n, T::kGroup, tm, tn);
        const int m0 = tm * BM;
        const int n0 = tn * BN;

        // The loads of one panel: prepare() works out the panel corners and
        // per-lane offsets, fire() builds the buffer resources and issues the
        // loads (loader waves only).
        struct Panel {
            const float *a, *b;          // panel corners
            int a_range, b_range;        // bytes of A from a on, of B from b on
            uint32_t oa[kLoadsA], ob[kLoadsB];
        };
        auto prepare = [&](int k0) {
            Panel p;
            p.a = g.A + ((int64_t)m0 * g.lda + k0);
            // Likewise for A when K % 4 != 0: in the panel holding column
            // K-1 a chunk can run past it (the elements it picks up there are
            // cleared in LDS before use, see clear_a_tail); for the tile
            // holding row M-1 that panel's A range ends after A's last
            // element.
            p.a_range = (g.K & 3) && k0 + BK >= g.K && m0 + BM >= g.M
                            ? 4 * ((g.M - 1 - m0) * (int)g.lda + (g.K - k0))
                            : (int)kOutOfRange;
#pragma unroll
            for (int j = 0; j < kLoadsA; ++j)
                p.oa[j] = m0 + a_r[j] < g.M && k0 + a_k[j] < g.K ? a_off[j] : kOutOfRange;
            // When N % 4 != 0 a 4-float chunk can start before column N and
            // run past it.  Past column N of rows before K-1 it still reads
            // inside B; for the panel that holds row K-1 the B range ends
            // after B's last element (K-1, N-1), so there such a chunk reads
            // zeros instead of memory beyond B.  That panel's range is under
            // (BK-1)*ldb + BN floats, which the 32-bit offsets already need.
            p.b = g.B + ((int64_t)k0 * g.ldb + n0);
            p.b_range = (g.N & 3) && k0 + BK >= g.K ? 4 * ((g.K - 1 - k0) * (int)g.ldb + (g.N - n0))
                                                     : (int)kOutOfRange;
#pragma unroll
            for (int j = 0; j < kLoadsB; ++j)
                p.ob[j] = k0 + b_k[j] < g.K && n0 + b_c[j] < g.N ? b_off[j] : kOutOfRange;
            return p;
        };
        auto fire = [&](int buf, const Panel &p) {
            if (NL < NW && !loader)
                return;
            if constexpr (kPoisonLds) {
#pragma unroll
                for (int j = 0; j < kLoadsA; ++j)
                    if (kEvenA || lw * kLoadsA + j < kInstA)
                        poison16(&stage[buf][(lw * kLoadsA + j) * kSpanA + lane * kVecA]);
#pragma unroll
                for (int j = 0; j < kLoadsB; ++j)
                    if (kEvenB || lw * kLoadsB + j < kInstB)
                        poison16(&stage[buf][kA + (lw * kLoadsB + j) * kSpanB + lane * kVecB]);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
            const __amdgpu_buffer_rsrc_t ra =
                __builtin_amdgcn_make_buffer_rsrc((void *)p.a, 0, p.a_range, kRawBufferFlags);
            const __amdgpu_buffer_rsrc_t rb =
                __builtin_amdgcn_make_buffer_rsrc((void *)p.b, 0, p.b_range, kRawBufferFlags);
#pragma unroll
            for (int j = 0; j < kLoadsA; ++j) {
                if (!kEvenA && lw * kLoadsA + j >= kInstA)
                    break;
                buffer_to_lds(ra, &stage[buf][(lw * kLoadsA + j) * kSpanA], p.oa[j]);
            }
#pragma unroll
            for (int j = 0; j < kLoadsB; ++j) {
                if (!kEvenB && lw * kLoadsB + j >= kInstB)
                    break;
                buffer_to_lds(rb, &stage[buf][kA + (lw * kLoadsB + j) * kSpanB], p.ob[j]);
            }
        };

        f32x16 acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[i][j][r] = 0.f;

        // One k-group (8 k) of MFMA operands: A rows and B columns of this
        // wave's 32 x 32 blocks.
        struct Frag {
            f32x4 a[FM];
            float b[4][FN];
        };
        auto read_frag = [&](Frag &f, int buf, int q) {
            const float *pa = stage[buf] + a_frag;
            const float *pb = stage[buf];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                f.a[i] = *reinterpret_cast<const f32x4 *>(pa + i * 32 * BK + 4 * ((2 * q + lh) ^ a_swz[i]));
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    f.b[s][j] = pb[b_frag[j] + 8 * q * BN + b_s[s]];
        };
        // The instructions s0 .. s1-1 of a k-group (all 32 x 32 blocks).
        auto mma_part = [&](const Frag &f, int s0, int s1) {
#pragma unroll
            for (int s = s0; s < s1; ++s)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[i][s], f.b[s][j], acc[i][j], 0, 0, 0);
        };
        auto mma = [&](const Frag &f) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[i][s], f.b[s][j], acc[i][j], 0, 0, 0);
        };

        // Group `group` takes panels p_begin + group, + KS, + 2*KS, ...;
        // round `it` is its panel p_begin + it*KS + group, held in buffer
        // it % S.
        const int npanels = p_end - p_begin;
        const int rounds = (npanels + KS - 1) / KS;
        auto exists = [&](int it) { return it < rounds && (KS == 1 || it * KS + group < npanels); };
        auto panel_k = [&](int it) { return (p_begin + it * KS + group) * BK; };
        // With 128-bit A loads and K % 4 != 0, the chunk of each A row that
        // holds column K-1 also brings 1 to 3 elements past it (the row's
        // padding or the next row's first elements), which would meet B's
        // zero-filled rows >= K: harmless if finite, NaN if not.  Once the
        // panel holding column K-1 (round tail_round of group tail_group) is
        // in LDS, those elements are set to +0.0, followed by one barrier.
        const bool a_tail = (g.K & 3) && p_end == ktiles;
        const int tail_round = (ktiles - 1 - p_begin) / KS;
        const int tail_group = (ktiles - 1 - p_begin) % KS;
        auto clear_a_tail = [&](int buf) {
            const int valid = g.K - (ktiles - 1) * BK;       // columns of the panel below K
            const int chunk = valid / 4, first = valid % 4;
            constexpr int NT = NW * kWaveSize;                // threads of the group
            const int gt = tid - group * NT;
            for (int e = gt; e < BM * 4; e += NT) {
                const int r = e / 4, x = e % 4;
                if (x >= first)
                    stage[buf][r * BK + 4 * (chunk ^ swz_a<BK>(r)) + x] = 0.f;
            }
        };
        if constexpr (T::kPipe) {
            // Software-pipelined rounds, for 4-wave tiles and for K-split
            // tiles of one-wave groups.  With one or two waves per SIMD,
            // little else fills the matrix core while a wave waits: the
            // wave's own instruction stream must keep it busy.
            //  - Fragments are read one k-group ahead (two Frag sets), and
            //    each read is issued between two MFMAs of the k-group before.
            //  - The panel loads of round it+1 are spread through the MFMAs
            //    of round it, one load every kGap MFMAs from the first
            //    k-groups on, into the buffer round it-1 used (with loader
            //    waves, those waves issue them and the MFMA waves none).
            //  - One barrier per round, halfway through the last k-group: the
            //    wave's own loads have landed (vmcnt), all waves are done
            //    with the buffer of round it (their last reads fed the MFMAs
            //    before it), and the first fragments of round it+1 are read
            //    while the second half of those MFMAs runs.  A one-wave
            //    group owns its buffers and only waits for its own loads.
            //    (8 such groups on a 64 x 64 tile: 16384 x 64 x 4096 in 72 us
            //    against 79 for 4 groups of 4 waves.)
            //  - Per round only scalars change.  The per-lane offsets are the
            //    tile's (rows past M-1 and columns past N-1 read as zero);
            //    in the last panel (k0 + BK > K) B's range ends after B's
            //    last element, so its rows past K-1 read as zero, and A's
            //    columns past K-1 are set to +0.0 in LDS once the panel has
            //    landed (A's range also ends after A's last element when that
            //    is within the panel's reach).  Past the last round the
            //    ranges are empty and the loads only write zeros into the
            //    idle buffer.
            // The sched_group_barrier masks: 0x008 MFMA, 0x100 LDS read,
            // 0x060 buffer load (a direct-to-LDS load counts as a load and
            // a store).  Measured at 8192^3: 7.30 ms against 7.45 for the
            // 16-wave 256 x 256 tile; 2048^3 with 128 x 128 x 64 tiles:
            // 125 us against 132.6 for the 16-wave K-split tile.
            constexpr int Q = BK / 8;                            // k-groups per panel
            constexpr int kMfma = 4 * FM * FN;                   // MFMAs per k-group
            constexpr int kReads = FM + 2 * FN;                  // LDS reads per k-group (B in pairs)
            // MFMAs before each panel load: 3 where the loads fit, fewer for
            // small wave tiles, which have few MFMAs per load.
            constexpr int kGapFit = (kMfma - kReads) * (Q - 1) / kLoads;
            constexpr int kGap = kGapFit < 3 ? (kGapFit < 1 ? 1 : kGapFit) : 3;
            constexpr int kPerBlock = (kMfma - kReads) / kGap;   // panel loads per k-group
            // The per-round barrier is a workgroup barrier, so only a tile
            // with a single group (KS == 1) may use it: K-split groups can
            // have different round counts, and one-wave groups (NW == 1)
            // therefore run their rounds without any barrier.
            static_assert((KS == 1 || NW == 1) && (S == 2 || LW) && Q % 2 == 0 &&
                              (LW || (NL == NW && kEvenA && kEvenB)),
                          "pipelined rounds: one group of all-loading waves (or loader waves), or one-wave "
                          "groups; two buffers (a deeper ring with loader waves); even k-group count");
            static_assert(LW || (kPerBlock >= 1 && (kLoads + kPerBlock - 1) / kPerBlock <= Q - 1),
                          "the panel loads fit in the k-groups before the barrier");
            uint32_t oa_t[kLoadsA], ob_t[kLoadsB];
#pragma unroll
            for (int j = 0; j < kLoadsA; ++j)
                oa_t[j] = m0 + a_r[j] < g.M ? a_off[j] : kOutOfRange;
#pragma unroll
            for (int j = 0; j < kLoadsB; ++j)
                ob_t[j] = n0 + b_c[j] < g.N ? b_off[j] : kOutOfRange;
            struct Rsrc {
                __amdgpu_buffer_rsrc_t a, b;
            };
            // This group's rounds: panels p_begin + group, + KS, ... below
            // p_end; the panel holding column K-1 is its round tail_round if
            // the group is tail_group.
            const int my_rounds = npanels > group ? (npanels - group + KS - 1) / KS : 0;
            const bool cols_tail = g.K % BK != 0 && p_end == ktiles && group == tail_group;
            // The ranges of the panel holding column K-1, worked out once:
            // per round only selects and the panel's base addresses remain,
            // with no branch (so that they can sit between MFMAs).
            const int k_last = (ktiles - 1) * BK;
            const int64_t a_end = 4 * ((int64_t)(g.M - 1 - m0) * g.lda + (g.K - k_last));
            const int ar_last = a_end < (int64_t)kOutOfRange ? (int)a_end : (int)kOutOfRange;
            const int br_last = 4 * ((g.K - 1 - k_last) * (int)g.ldb + (g.N - n0));
            // Round it's panels start at a_at(it) and b_at(it).
            auto a_at = [&](int it) { return g.A + ((int64_t)m0 * g.lda + panel_k(it)); };
            auto b_at = [&](int it) { return g.B + ((int64_t)panel_k(it) * g.ldb + n0); };
            auto rsrc_from = [&](const float *pa, const float *pb, int it) {
                const bool on = it < my_rounds, last = cols_tail && it == tail_round;
                const int ar = on ? (last ? ar_last : (int)kOutOfRange) : 0;
                const int br = on ? (last ? br_last : (int)kOutOfRange) : 0;
                return Rsrc{__builtin_amdgcn_make_buffer_rsrc((void *)pa, 0, ar, kRawBufferFlags),
                            __builtin_amdgcn_make_buffer_rsrc((void *)pb, 0, br, kRawBufferFlags)};
            };
            auto rsrc = [&](int it) { return rsrc_from(a_at(it), b_at(it), it); };
            // Load x of a wave's panel share (A's loads first, then B's).
            // Debug build: NaN into every slot this wave's loads of one
            // round fill, before they are issued.
            auto poison_loads = [&](int buf) {
                if constexpr (kPoisonLds) {
#pragma unroll
                    for (int x = 0; x < kLoadsA; ++x)
                        poison16(&stage[buf][(lw * kLoadsA + x) * kSpanA + lane * kVecA]);
#pragma unroll
                    for (int x = 0; x < kLoadsB; ++x)
                        poison16(&stage[buf][kA + (lw * kLoadsB + x) * kSpanB + lane * kVecB]);
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                }
            };
            auto load_one = [&](int buf, const Rsrc &r, int x) {
                if (x < kLoadsA)
                    buffer_to_lds(r.a, &stage[buf][(lw * kLoadsA + x) * kSpanA], oa_t[x]);
                else
                    buffer_to_lds(r.b, &stage[buf][kA + (lw * kLoadsB + x - kLoadsA) * kSpanB], ob_t[x - kLoadsA]);
            };
            constexpr int NT = NW * kWaveSize;                   // threads of the group
            auto clear_cols = [&](int buf) {
                const int valid = g.K - (ktiles - 1) * BK;
                for (int e = tid - group * NT; e < BM * BK; e += NT) {
                    const int r = e / BK, c = e % BK;
                    if (c >= valid)
                        stage[buf][r * BK + 4 * ((c / 4) ^ swz_a<BK>(r)) + c % 4] = 0.f;
                }
            };
            // A one-wave group needs no barrier: its LDS reads and writes are
            // in program order, and vmcnt covers its own loads.
            auto group_sync = [&]() {
                if constexpr (NW > 1)
                    __syncthreads();
            };
            // Loader waves (LW): they issue every load of a panel, in the
            // group's round structure -- with a ring of S buffers, round
            // it+S-1 goes into the buffer round it-1 used right after round
            // it-1's barrier; each loader waits until its loads of round
            // it+1 have landed and meets the MFMA waves at round it's barrier
            // (and at the tail clearing's).  The MFMA waves' side of the
            // loop is the same as without loader waves, minus the loads.
            // The panel's load instructions (A's, then B's) are dealt to the
            // loader waves in equal runs.
            if (LW && gw >= NW) {
                constexpr int NLW = LW ? T::kLoaderWaves : 1;
                constexpr int kPer = (kInstA + kInstB) / NLW;
                static_assert((kInstA + kInstB) % NLW == 0, "equal loader shares");
                static_assert(S == 2 || (S - 1) * kPer <= 63, "a deeper ring keeps its rounds' loads within vmcnt");
                auto loader_rounds = [&](auto lv_c) {
                    constexpr int lv = decltype(lv_c)::value;
                    uint32_t off[kPer];
#pragma unroll
                    for (int j = 0; j < kPer; ++j) {
                        const int x = lv * kPer + j;
                        if (x < kInstA) {
                            const int f = x * kSpanA + lane * kVecA;
                            const int r = f / BK, e = f % BK;
                            const int k = 4 * ((e / 4) ^ swz_a<BK>(r)) + e % 4;
                            off[j] = m0 + r < g.M ? (uint32_t)(r * g.lda + k) * 4u : kOutOfRange;
                        } else {
                            const int f = (x - kInstA) * kSpanB + lane * kVecB;
                            const int k = kNarrowB ? (f / BN) ^ ((f / BN >> 2) & 1) : f / BN;
                            const int c = kNarrowB ? f % BN : (f % BN) ^ (((k >> 2) & 1) * 32);
                            off[j] = n0 + c < g.N ? (uint32_t)(k * g.ldb + c) * 4u : kOutOfRange;
                        }
                    }
                    auto slot = [](int x) { return x < kInstA ? x * kSpanA : kA + (x - kInstA) * kSpanB; };
                    auto issue = [&](int buf, const Rsrc &r) {
                        if constexpr (kPoisonLds) {
#pragma unroll
                            for (int j = 0; j < kPer; ++j)
                                poison16(&stage[buf][slot(lv * kPer + j) + lane * 4]);
                            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                        }
                        // vmcnt counts at most 63 loads in flight: past
                        // that, each load waits for the oldest to land.
#pragma unroll
                        for (int j = 0; j < kPer; ++j) {
                            const int x = lv * kPer + j;
                            if (j >= 63)
                                asm volatile("s_waitcnt vmcnt(62)" ::: "memory");
                            buffer_to_lds(x < kInstA ? r.a : r.b, &stage[buf][slot(x)], off[j]);
                        }
                    };
                    // Rounds 0 .. S-2 first; then, after round it-1's
                    // barrier, round it+S-1 into the buffer round it-1
                    // used.  Before round it's barrier round it+1 must have
                    // landed: the S-2 rounds after it may still be in flight.
#pragma unroll
                    for (int r = 0; r + 1 < S; ++r)
                        issue(r, rsrc(r));
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((S - 2) * kPer) : "memory");
                    __builtin_amdgcn_s_barrier();
                    if (cols_tail && tail_round == 0)
                        group_sync();
                    for (int it = 0; it < my_rounds; ++it) {
                        issue((it + S - 1) % S, rsrc(it + S - 1));
                        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((S - 2) * kPer) : "memory");
                        __builtin_amdgcn_s_barrier();
                        if (cols_tail && it + 1 == tail_round)
                            group_sync();
                    }
                };
                if (my_rounds > 0) {
                    if (gw == NW)
                        loader_rounds(std::integral_constant<int, 0>{});
                    else if constexpr (NLW > 1)
                        loader_rounds(std::integral_constant<int, 1>{});
                    static_assert(NLW <= 2, "one or two loader waves");
                }
            } else if (my_rounds > 0) {
            if constexpr (!LW) {
                const Rsrc r0 = rsrc(0);
                poison_loads(0);
#pragma unroll
                for (int x = 0; x < kLoads; ++x)
                    load_one(0, r0, x);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            if constexpr (NW > 1)
                __builtin_amdgcn_s_barrier();
            if (cols_tail && tail_round == 0) {
                clear_cols(0);
                group_sync();
            }
            Frag F[2];
            read_frag(F[0], 0, 0);
            // Round it+1's panels, advanced by one round's step in round it.
            const float *pa = a_at(1), *pb = b_at(1);
            const int64_t step_b = (int64_t)KS * BK * g.ldb;
            Rsrc nx;
            if constexpr (!LW)
                nx = rsrc_from(pa, pb, 1);
            for (int it = 0; it < my_rounds; ++it) {
                const int buf = it % S, nbuf = (it + 1) % S;
                if constexpr (!LW)
                    poison_loads(nbuf);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int q = 0; q + 1 < Q; ++q) {
                    read_frag(F[(q + 1) & 1], buf, q + 1);
                    if constexpr (!LW) {
#pragma unroll
                        for (int x = q * kPerBlock; x < (q + 1) * kPerBlock; ++x)
                            if (x < kLoads)
                                load_one(nbuf, nx, x);
                    }
                    mma(F[q & 1]);
#pragma unroll
                    for (int r = 0; r < kReads; ++r) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                    if constexpr (!LW) {
#pragma unroll
                        for (int x = q * kPerBlock; x < (q + 1) * kPerBlock; ++x)
                            if (x < kLoads) {
                                __builtin_amdgcn_sched_group_barrier(0x008, kGap, 0);
                                __builtin_amdgcn_sched_group_barrier(0x060, 1, 0);
                            }
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, kMfma, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
                mma_part(F[(Q - 1) & 1], 0, 2);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (LW)
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                else
                    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
                if constexpr (NW > 1)
                    __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
                if (cols_tail && it + 1 == tail_round) {
                    clear_cols(nbuf);
                    group_sync();
                }
                read_frag(F[0], nbuf, 0);
                // The next round's buffer descriptors, worked out here
                // between MFMAs rather than ahead of the next round's first.
                Rsrc nn;
                if constexpr (!LW) {
                    pa += KS * BK;
                    pb += step_b;
                    nn = rsrc_from(pa, pb, it + 2);
                }
                mma_part(F[(Q - 1) & 1], 2, 4);
#pragma unroll
                for (int r = 0; r < kReads; ++r) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
#pragma unroll
                for (int r = kReads; r < kMfma / 2; ++r) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x004, 2, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (!LW)
                    nx = nn;
            }
            }
        } else {
        // Rounds it+1 .. it+S-1 are in flight while round it is computed.
#pragma unroll
        for (int it = 0; it < S - 1; ++it)
            if (exists(it))
                fire(it, prepare(panel_k(it)));
        for (int it = 0; it < rounds; ++it) {
            const bool more = exists(it + S - 1);
            const Panel next = prepare(panel_k(it + S - 1));
            // Round it has landed once no more than the loads of the rounds
            // after it (up to S-2 of them, kLoads each) are outstanding; the
            // LDS reads of round it-1 are complete as well.  Then the barrier
            // makes every wave's panel visible and frees buffer (it-1) % S.
            // A one-wave group owns its buffers, loads its own panels and
            // reads and writes LDS in program order: it needs no barrier.
            if (S > 2 && exists(it + S - 2))
                asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((S - 2) * kLoads) : "memory");
            else
                asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
            if constexpr (NW > 1)
                __builtin_amdgcn_s_barrier();
            if (more)
                fire((it + S - 1) % S, next);
            if (a_tail && it == tail_round) {
                if (group == tail_group)
                    clear_a_tail(it % S);
                if constexpr (NW > 1)
                    __syncthreads();
            }
            if (exists(it)) {
#pragma unroll
                for (int q = 0; q < BK / 8; ++q) {
                    Frag f;
                    read_frag(f, it % S, q);
                    mma(f);
                }
            }
        }
        }
        // Every wave is done with the panel buffers before they are reused
        // (by the K-split reduction, or by the next tile's first loads).
        __syncthreads();

        const bool shared = SK && (p_begin != 0 || p_end != ktiles);
        if constexpr (KS > 1) {
            // Fold the groups' partial sums and write C: every group stores
            // its partial tile into a region of its own (the panel buffers
            // are free: the loop ended with a barrier), then, after one
            // barrier, each thread adds a 4-column chunk of the groups'
            // partials in group order 0, 1, ..., KS-1 -- a fixed order, so
            // the result does not depend on scheduling -- and writes it to
            // C as one 128-bit store (element by element in edge tiles, for
            // unaligned rows, and as atomic adds in stream-K's shared
            // tiles).  In a region, rows with bit 2 set have their columns
            // swapped in 32-float halves (32-wide tiles: their rows swapped
            // in pairs), so the two lane halves of an accumulator write
            // (rows 4 apart) fall on different banks.
            static_assert(KS * BM * BN <= KS * S * kStage, "every group's partial tile fits in the panel buffers");
            float *part = &lds[0][0][0];
            auto slot = [](int row, int col) {
                return kNarrowB ? (row ^ ((row >> 2) & 1)) * BN + col : row * BN + (col ^ ((row & 4) ? 32 : 0));
            };
            float *mine = part + group * (BM * BN);
            if constexpr (kPoisonLds) {
                poison_region(part, KS * BM * BN, tid, T::kThreads);
                __syncthreads();
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = wave_m * T::kWaveM + i * 32 + 8 * (r / 4) + 4 * lh + (r % 4);
                        mine[slot(row, wave_n * T::kWaveN + j * 32 + li)] = acc[i][j][r];
                    }
            __syncthreads();
            auto sum = [&](int at) {
                float v = part[at];
#pragma unroll
                for (int q = 1; q < KS; ++q)
                    v += part[q * (BM * BN) + at];
                return v;
            };
            if (!shared && c_vec && m0 + BM <= g.M && n0 + BN <= g.N) {
                constexpr int kRowChunks = BN / 4;
                for (int e = tid; e < BM * kRowChunks; e += T::kThreads) {
                    const int lr = e / kRowChunks, lc = 4 * (e % kRowChunks);
                    const int at = slot(lr, lc);
                    f32x4 v = *reinterpret_cast<const f32x4 *>(&part[at]);
#pragma unroll
                    for (int q = 1; q < KS; ++q)
                        v += *reinterpret_cast<const f32x4 *>(&part[q * (BM * BN) + at]);
                    float *c = &cbase[(int64_t)(m0 + lr) * g.ldc + n0 + lc];
                    if constexpr (WB)
                        *reinterpret_cast<f32x4 *>(c) = v;
                    else
                        __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(c));
                }
            } else {
                // Edge tiles, unaligned rows and shared tiles: one element
                // per thread, consecutive threads on consecutive columns, so
                // each store (or atomic add) instruction covers whole runs
                // of a row.
                for (int e = tid; e < BM * BN; e += T::kThreads) {
                    const int lr = e / BN, lc = e % BN;
                    const int row = m0 + lr, col = n0 + lc;
                    if (row < g.M && col < g.N) {
                        const float v = sum(slot(lr, lc));
                        float *c = &cbase[(int64_t)row * g.ldc + col];
                        if (shared)
                            unsafeAtomicAdd(c, v);
                        else
                            store_c<WB>(c, v);
                    }
                }
            }
            // Every thread is done with the regions before the panel buffers
            // are reused (a strip's sums, or the next tile's loads).
            __syncthreads();
        } else {
            if (kBandEpilogue && !shared && c_vec && m0 + BM <= g.M && n0 + BN <= g.N) {
                // Whole tile, 16-byte aligned rows of C: stage one band of
                // kWaveM rows at a time through the (now idle) panel buffers and
                // write C with 128-bit stores of whole rows instead of one
                // 32-bit store per accumulator element (+3.5 to +7 % on
                // 8192 x 8192 x 128, whose time is dominated by writing C).  The
                // band is [kWaveM][BN]; rows with bit 2 set have their columns
                // swapped in 32-float halves, so the two lane halves of an
                // accumulator write (rows 4 apart) fall on different banks.
                float *band = &lds[0][0][0];
                for (int p = 0; p < T::WAVES_M; ++p) {
                    if constexpr (kPoisonLds) {
                        poison_region(band, T::kWaveM * BN, tid, T::kThreads);
                        __syncthreads();
                    }
                    if (wave_m == p) {
#pragma unroll
                        for (int i = 0; i < FM; ++i)
#pragma unroll
                            for (int j = 0; j < FN; ++j)
#pragma unroll
                                for (int r = 0; r < 16; ++r) {
                                    const int lr = i * 32 + 8 * (r / 4) + 4 * lh + (r % 4);
                                    const int lc = (wave_n * T::kWaveN + j * 32 + li) ^ ((lr & 4) ? 32 : 0);
                                    band[lr * BN + lc] = acc[i][j][r];
                                }
                    }
                    __syncthreads();
                    constexpr int kRowChunks = BN / 4;
                    for (int e = tid; e < T::kWaveM * kRowChunks; e += T::kThreads) {
                        const int lr = e / kRowChunks, c4 = e % kRowChunks;
                        const f32x4 v = *reinterpret_cast<const f32x4 *>(&band[lr * BN + ((4 * c4) ^ ((lr & 4) ? 32 : 0))]);
                        float *dst = &cbase[(int64_t)(m0 + p * T::kWaveM + lr) * g.ldc + n0 + 4 * c4];
                        __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(dst));
                    }
                    __syncthreads();
                }
                return;
            }
            if (group == 0 && gw < NW) {    // not the loader wave
#pragma unroll
                for (int i = 0; i < FM; ++i) {
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const int col = n0 + wave_n * T::kWaveN + j * 32 + li;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int row = m0 + wave_m * T::kWaveM + i * 32 + 8 * (r / 4) + 4 * lh + (r % 4);
                            if (row < g.M && col < g.N) {
                                float *c = &cbase[(int64_t)row * g.ldc + col];
                                if (shared)
                                    unsafeAtomicAdd(c, acc[i][j][r]);
                                else
                                    store_c<WB>(c, acc[i][j][r]);
                            }
                        }
                    }
                }
            }
        }

        // Remainder strips (data-parallel launches only): rows M-R .. M-1
        // below the tile grid and columns N-S .. N-1 right of it (either or
        // both) are summed with vector FMAs by every workgroup: the one
        // running tile t takes w = ceil(N / tiles) of the row strip's columns
        // from t * w, and h = ceil((M - R) / tiles) of the column strip's rows
        // from t * h, each at most kMaxStripSpread, so that no workgroup
        // streams much of B (A); the row strip spans all N columns, so the
        // corner is its.  strip_block sums one block.
        if constexpr (STRIP)
        if (g.strip_rows > 0 || g.strip_cols > 0) {
            const int total = g.tiles_m * g.tiles_n;
            float *red = &lds[0][0][0];
            // rows ar0 .. of A and C, columns bc0 .. of B and C
            if (g.strip_rows > 0) {
                const int w = (g.N + total - 1) / total;
                const int bc0 = t * w, nc = max(0, min(w, g.N - bc0));
                __syncthreads();
                if (nc <= 4)
                    strip_block<T::kThreads, 4, kMaxStripRows>(g.A, g.lda, g.B, g.ldb, cbase, g.ldc, g.K,
                                                               g.M - g.strip_rows, g.strip_rows, bc0, nc, red, tid);
                else
                    strip_block<T::kThreads, 8, kMaxStripRows>(g.A, g.lda, g.B, g.ldb, cbase, g.ldc, g.K,
                                                               g.M - g.strip_rows, g.strip_rows, bc0, nc, red, tid);
            }
            if (g.strip_cols > 0) {
                const int rows = g.M - g.strip_rows;
                const int h = (rows + total - 1) / total;
                const int ar0 = t * h;
                __syncthreads();
                strip_block<T::kThreads, 4, kMaxStripSpread>(g.A, g.lda, g.B, g.ldb, cbase, g.ldc, g.K, ar0,
                                                             max(0, min(h, rows - ar0)), g.N - g.strip_cols,
                                                             g.strip_cols, red, tid);
            }
        }
    };

    if (SPLIT) {
        // Split-K: workgroup w computes tile w % tiles over K slice
        // w / tiles and stores it into that slice's slab of the workspace.
        const int slice = blockIdx.x / total;
        cbase = g.C + (int64_t)slice * g.slab;
        work(blockIdx.x % total, (int)((int64_t)slice * ktiles / g.slices),
             (int)((int64_t)(slice + 1) * ktiles / g.slices));
    } else if (SK) {
        int64_t lo, hi;
        streamk_range(xcd_contiguous(blockIdx.x, gridDim.x, g.xcds), gridDim.x, (int64_t)total * ktiles, lo, hi);
        // The range is the end of one tile (from panel lo % ktiles), whole
        // tiles, and the start of another (panels 0 .. hi % ktiles).  Whole
        // tiles go first and the start piece next, so that most workgroups
        // are at the same K-panel at the same time and share the panels'
        // rows of A and columns of B in L2; the end piece goes last.
        const int first = (int)((lo + ktiles - 1) / ktiles);   // first tile starting at or after lo
        const int last = (int)(hi / ktiles);                    // tile holding panel hi (or one past)
        const int p_lo = (int)(lo % ktiles), p_hi = (int)(hi % ktiles);
        if (lo < hi && first > last) {
            work(last, p_lo, p_hi);                             // inside one tile
        } else if (lo < hi) {
            for (int t = first; t < last; ++t)
                work(t, 0, ktiles);
            if (p_hi > 0)
                work(last, 0, p_hi);
            if (p_lo > 0)
                work(first - 1, p_lo, ktiles);
        }
    } else {
        for (int w = blockIdx.x; w < total; w += gridDim.x)
            work((int)gridDim.x == total ? xcd_contiguous(w, total, g.xcds) : w, 0, ktiles);
    }
}

// Stream-K leaves each tile shared by two workgroups to be summed in C: both
// add their partial sums atomically, so C must hold +0.0 there first.  Block
// b looks at the start of workgroup range b + 1; if it falls strictly inside
// a tile, that tile is shared and this block clears it (clipped to M x N).
// As no two range starts fall inside one tile, each tile is cleared once.
// Split-K: C = sum of the slices' partial products, added in slice order
// (slice 0, then 1, ...), so the result does not depend on scheduling.  The
// workspace holds slice s's M x N product at ws + s*slab, rows N apart.
__global__ __launch_bounds__(256) void splitk_reduce(const float *ws, int64_t slab, int slices,
                                                     float *C, int64_t ldc, int M, int N)
{
    const int64_t total = (int64_t)M * N;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        float sum = ws[e];
        for (int s = 1; s < slices; ++s)
            sum += ws[s * slab + e];
        store_c(&C[(e / N) * ldc + e % N], sum);
    }
}

template <class T>
__global__ __launch_bounds__(256) void zero_shared_tiles(GemmArgs g, int workers)
{
    const int ktiles = (g.K + T::BK - 1) / T::BK;
    int64_t start, end;
    streamk_range(blockIdx.x + 1, workers, (int64_t)g.tiles_m * g.tiles_n * ktiles, start, end);
    if (start % ktiles == 0)
        return;
    int tm, tn;
    tile_coords((int)(start / ktiles), g.tiles_m, g.tiles_n, T::kGroup, tm, tn);
    const int rows = min(T::BM, g.M - tm * T::BM), cols = min(T::BN, g.N - tn * T::BN);
    float *c = g.C + (int64_t)tm * T::BM * g.ldc + (int64_t)tn * T::BN;
    for (int e = threadIdx.x; e < rows * T::BN; e += blockDim.x)
        if (e % T::BN < cols)
            c[(int64_t)(e / T::BN) * g.ldc + e % T::BN] = 0.f;
}


// ---------------------------------------------------------------------------
// Vector-FMA kernel: 64 x 64 tile, 256 threads, 4 x 4 outputs per thread.
// ---------------------------------------------------------------------------
constexpr int kValuTile = 64;
constexpr int kValuBK = 16;
constexpr int kValuThreads = 256;

__global__ __launch_bounds__(kValuThreads) void gemm_f32_valu(GemmArgs g)
{
    // Both panels k-major ([k][m], [k][n]) so each thread reads its 4 rows and
    // its 4 columns with one 128-bit LDS read each.
    __shared__ __attribute__((aligned(16))) float sa[kValuBK][kValuTile + 4];
    __shared__ __attribute__((aligned(16))) float sb[kValuBK][kValuTile + 4];

    const int tid = threadIdx.x;
    const int tx = tid % 16;          // output columns 4*tx .. 4*tx+3
    const int ty = tid / 16;          // output rows    4*ty .. 4*ty+3
    const int total = g.tiles_m * g.tiles_n;

    for (int t = blockIdx.x; t < total; t += gridDim.x) {
        const int m0 = (t / g.tiles_n) * kValuTile;
        const int n0 = (t % g.tiles_n) * kValuTile;
        float acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = 0.f;

        for (int k0 = 0; k0 < g.K; k0 += kValuBK) {
#pragma unroll
            for (int q = 0; q < kValuTile * kValuBK / kValuThreads; ++q) {
                const int e = tid + q * kValuThreads;
                const int am = e / kValuBK, ak = e % kValuBK;      // A: along k
                const int m = m0 + am, ka = k0 + ak;
                sa[ak][am] = (m < g.M && ka < g.K) ? g.A[(int64_t)m * g.lda + ka] : 0.f;
                const int bk = e / kValuTile, bn = e % kValuTile;  // B: along n
                const int kb = k0 + bk, n = n0 + bn;
                sb[bk][bn] = (kb < g.K && n < g.N) ? g.B[(int64_t)kb * g.ldb + n] : 0.f;
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < kValuBK; ++k) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(&sa[k][4 * ty]);
                const f32x4 b = *reinterpret_cast<const f32x4 *>(&sb[k][4 * tx]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
            }
            __syncthreads();
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + 4 * ty + i;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = n0 + 4 * tx + j;
                if (row < g.M && col < g.N)
                    g.C[(int64_t)row * g.ldc + col] = acc[i][j];
            }
        }
    }
}

// K == 0: the sum is empty, C's window becomes +0.0.  A kernel rather than a
// memset so the call stays a plain kernel launch (also under graph capture).
__global__ __launch_bounds__(256) void fill_zero(float *C, int64_t ldc, int M, int N)
{
    const int64_t total = (int64_t)M * N;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x)
        C[(e / N) * ldc + (e % N)] = 0.f;
}

// ---------------------------------------------------------------------------
// Configurations
// ---------------------------------------------------------------------------
// Tile shapes (MfmaTile<BM, BN, BK, WAVES_M, WAVES_N, KSPLIT, STAGES, GROUP,
// LOADERS, PIPE>): BM x BN output tile, BK-deep K-panels, WAVES_M x WAVES_N
// waves each owning a (BM/WAVES_M) x (BN/WAVES_N) block; optional K-split
// groups, panel-ring depth, loader-wave count and the software-pipelined
// round loop.
using Tile128x128 = MfmaTile<128, 128, 16, 2, 2>;       // 4 waves of 64 x 64 (staged fallback)
using Tile64x64 = MfmaTile<64, 64, 16, 2, 2>;           // 4 waves of 32 x 32 (staged fallback)
using Tile128x128K32W16 = MfmaTile<128, 128, 32, 4, 4, 1, 2, 8, 8>;  // 16 waves of 32 x 32, 8 load
using Tile64x64K32 = MfmaTile<64, 64, 32, 2, 2>;
using Tile64x64K32S4 = MfmaTile<64, 64, 32, 2, 2, 4>;   // 4 K-split groups of 4 waves
using Tile64x128K32 = MfmaTile<64, 128, 32, 2, 2>;
using Tile128x64K32 = MfmaTile<128, 64, 32, 2, 2>;
using Tile64x64K64 = MfmaTile<64, 64, 64, 2, 2>;         // 64-deep panels
// 2 K-split groups of 8 waves of 32 x 64, 4 of them loading
using Tile128x128K32S2 = MfmaTile<128, 128, 32, 4, 2, 2, 2, 8, 4>;
// Software-pipelined 4-wave tiles: 4 waves of 128 x 128, and 4 waves of
// 64 x 64 on 64-deep panels (128 KiB of LDS) with two more waves that issue
// every panel load (the MFMA waves only read LDS: 2048^3 in 123.0 us against
// 125.6 when the four MFMA waves also load; 2372 x 1619 x 7588: 437 against
// 449; stream-K over 5000 x 2600 x 4096: 792 against 811).  One loader wave
// needs 64 loads per panel, past the 63 vmcnt can count (124.1 us).
using Tile256x256K32P = MfmaTile<256, 256, 32, 2, 2, 1, 2, 8, 0, 1>;
using Tile128x128K64PL2 = MfmaTile<128, 128, 64, 2, 2, 1, 2, 8, 0, 1, 2>;
// 4 waves of 32 x 32 fed by two loader waves through a ring of four 32-deep
// panels (64 KiB of LDS): three rounds of loads in flight.
using Tile64x64K32PL2S4 = MfmaTile<64, 64, 32, 2, 2, 1, 4, 8, 0, 1, 2>;
// Software-pipelined K-split: 8 one-wave groups, each with the whole 64 x 64
// tile for every 8th 16-deep panel
using Tile64x64K16S8P = MfmaTile<64, 64, 16, 1, 1, 8, 2, 8, 0, 1>;
// Software-pipelined 4 waves of 64 x 64 on 16-deep panels (32 KiB of LDS,
// three workgroups per CU)
using Tile128x128K16P = MfmaTile<128, 128, 16, 2, 2, 1, 2, 8, 0, 1>;
// Software-pipelined 4 waves of 64 x 64 on 32-deep panels (64 KiB of LDS,
// two workgroups per CU)
using Tile128x128K32P = MfmaTile<128, 128, 32, 2, 2, 1, 2, 8, 0, 1>;

// 32-row or 32-column tiles of K-split one-wave groups, for problems with
// few output tiles: each wave owns the whole tile for every KS-th K-panel
// and streams those panels through its own ring of LDS buffers, with no
// barrier until the groups' partial sums are folded.
using Tile32x32K32S8 = MfmaTile<32, 32, 32, 1, 1, 8, 2>;   // 8 groups, 128 KiB of LDS
using Tile32x32K32S4 = MfmaTile<32, 32, 32, 1, 1, 4, 2>;   // 4 groups, 64 KiB
using Tile32x64K16S8 = MfmaTile<32, 64, 16, 1, 1, 8, 2>;   // 8 groups of 32 x 64, 96 KiB
using Tile64x32K16S8 = MfmaTile<64, 32, 16, 1, 1, 8, 2>;

// Every configuration is one the shape rule (select_config) picks for some
// shapes, the register-staged fallback for rows too long for 32-bit panel
// offsets, or one of the two plain 64 x 64 stream-K twins, which the rule no
// longer picks (over K <= 512 a second round of tiles beats stream-K) but
// which remain the simplest stream-K kernels (no K-split fold); each also
// runs under gemm_f32_with_config for tests and sweeps.
enum ConfigId {
    kCfgValu64 = 0,
    kCfgStaged128x128,
    kCfgStaged64x64,
    kCfgDma64x64K32,
    kCfgDma64x64K32S4,
    kCfgDma64x128K32,
    kCfgDma128x64K32,
    kCfgDma64x64K32SK,
    kCfgDma128x128K32W16SK,
    kCfgDma64x64K64,
    kCfgDma64x64K64SK,
    kCfgDma128x128K32S2,
    kCfgDma256x256K32P,
    kCfgDma256x256K32PSK,
    kCfgDma128x128K64P,
    kCfgDma128x128K64PSK,
    kCfgDma64x64K16S8P,
    kCfgDma64x64K32S4SK,
    kCfgDma128x128K16P,
    kCfgDma32x32K32S8,
    kCfgDma32x32K32S4,
    kCfgDma32x64K16S8,
    kCfgDma64x32K16S8,
    kCfgDma128x128K32P,
    kCfgDma64x64K32PL2S4,
    kCfgDma64x64K16S8PSK,
    kNumConfigs
};

template <class T, template <class, bool, bool> class Kernel>
struct Launch {
    static hipError_t run(const GemmArgs &g, bool va, bool vb, int grid, hipStream_t s)
    {
        if (va && vb)
            hipLaunchKernelGGL((Kernel<T, true, true>::fn), dim3(grid), dim3(T::kThreads), 0, s, g);
        else if (va)
            hipLaunchKernelGGL((Kernel<T, true, false>::fn), dim3(grid), dim3(T::kThreads), 0, s, g);
        else if (vb)
            hipLaunchKernelGGL((Kernel<T, false, true>::fn), dim3(grid), dim3(T::kThreads), 0, s, g);
        else
            hipLaunchKernelGGL((Kernel<T, false, false>::fn), dim3(grid), dim3(T::kThreads), 0, s, g);
        return hipGetLastError();
    }
    // Resident workgroups per compute unit (the 128-bit-load instance).
    static int occupancy()
    {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, Kernel<T, true, true>::fn, T::kThreads, 0) != hipSuccess)
            return -1;
        return n;
    }
};

// Adapter giving the register-staged kernel the launcher's interface.
template <class T, bool VA, bool VB>
struct PlainKernel {
    static constexpr auto fn = gemm_f32_mfma<T, VA, VB>;
};

// The direct-to-LDS kernel has one instance per tile and mode: it loads 16
// bytes per lane from any 4-byte aligned operand, so the load-width flags
// of the plan do not apply to it.
template <class T, bool SK = false, bool SPLIT = false, bool STRIP = false, bool WB = false>
struct LaunchDma {
    static hipError_t run(const GemmArgs &g, bool, bool, int grid, hipStream_t s)
    {
        hipLaunchKernelGGL((gemm_f32_mfma_dma<T, SK, SPLIT, STRIP, WB>), dim3(grid), dim3(T::kThreads), 0, s, g);
        return hipGetLastError();
    }
    static int occupancy()
    {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_f32_mfma_dma<T, SK, SPLIT, STRIP>, T::kThreads, 0) !=
            hipSuccess)
            return -1;
        return n;
    }
};

// Stream-K: clear the tiles two workgroups will share, then run the
// workers (one per compute unit) on the same stream.
template <class T, bool WB = false>
hipError_t launch_streamk(const GemmArgs &g, bool va, bool vb, int grid, hipStream_t s)
{
    if (grid > 1) {
        zero_shared_tiles<T><<<grid - 1, 256, 0, s>>>(g, grid);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return LaunchDma<T, true, false, false, WB>::run(g, va, vb, grid, s);
}

hipError_t launch_valu(const GemmArgs &g, bool, bool, int grid, hipStream_t s)
{
    gemm_f32_valu<<<grid, kValuThreads, 0, s>>>(g);
    return hipGetLastError();
}

int occupancy_valu()
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_f32_valu, kValuThreads, 0) != hipSuccess)
        return -1;
    return n;
}

struct ConfigInfo {
    const char *name;
    int bm, bn, bk, threads;
    bool dma;                    // direct-to-LDS (32-bit panel offsets)
    hipError_t (*launch)(const GemmArgs &, bool, bool, int, hipStream_t);
    int (*occupancy)();
    bool streamk;                // one worker per CU over all tiles' K-panels
    // The instance with write-back C stores, for a large C whose rows are
    // not 16-byte aligned (nullptr: none, the streaming one runs).
    hipError_t (*launch_wb)(const GemmArgs &, bool, bool, int, hipStream_t);
};

template <class T>
constexpr ConfigInfo config_staged(const char *name)
{
    return {name, T::BM, T::BN, T::BK, T::kThreads, false, &Launch<T, PlainKernel>::run,
            &Launch<T, PlainKernel>::occupancy, false, nullptr};
}

// WB: also build the write-back twin (only for the tiles the shape rule
// picks for problems with a large C).
template <class T, bool WB = false>
constexpr ConfigInfo config_dma(const char *name)
{
    hipError_t (*wb)(const GemmArgs &, bool, bool, int, hipStream_t) = nullptr;
    if constexpr (WB)
        wb = &LaunchDma<T, false, false, false, true>::run;
    return {name, T::BM, T::BN, T::BK, T::kThreads, true, &LaunchDma<T>::run, &LaunchDma<T>::occupancy,
            false, wb};
}

template <class T, bool WB = false>
constexpr ConfigInfo config_streamk(const char *name)
{
    hipError_t (*wb)(const GemmArgs &, bool, bool, int, hipStream_t) = nullptr;
    if constexpr (WB)
        wb = &launch_streamk<T, true>;
    return {name, T::BM, T::BN, T::BK, T::kThreads, true, &launch_streamk<T>,
            &LaunchDma<T, true>::occupancy, true, wb};
}

// Indexed by ConfigId.
const ConfigInfo kConfigs[kNumConfigs] = {
    {"valu_64x64", kValuTile, kValuTile, kValuBK, kValuThreads, false, &launch_valu, &occupancy_valu, false, nullptr},
    config_staged<Tile128x128>("staged_128x128x16"),
    config_staged<Tile64x64>("staged_64x64x16"),
    config_dma<Tile64x64K32, true>("dma_64x64x32"),
    config_dma<Tile64x64K32S4>("dma_64x64x32_ksplit4"),
    config_dma<Tile64x128K32, true>("dma_64x128x32"),
    config_dma<Tile128x64K32, true>("dma_128x64x32"),
    config_streamk<Tile64x64K32, true>("dma_64x64x32_sk"),
    config_streamk<Tile128x128K32W16>("dma_128x128x32_w16_sk"),
    config_dma<Tile64x64K64>("dma_64x64x64"),
    config_streamk<Tile64x64K64>("dma_64x64x64_sk"),
    config_dma<Tile128x128K32S2>("dma_128x128x32_ksplit2"),
    config_dma<Tile256x256K32P, true>("dma_256x256x32_pipe"),
    config_streamk<Tile256x256K32P, true>("dma_256x256x32_pipe_sk"),
    config_dma<Tile128x128K64PL2, true>("dma_128x128x64_pipe_lw2"),
    config_streamk<Tile128x128K64PL2, true>("dma_128x128x64_pipe_lw2_sk"),
    config_dma<Tile64x64K16S8P, true>("dma_64x64x16_ksplit8_pipe"),
    config_streamk<Tile64x64K32S4>("dma_64x64x32_ksplit4_sk"),
    config_dma<Tile128x128K16P, true>("dma_128x128x16_pipe"),
    config_dma<Tile32x32K32S8>("dma_32x32x32_ksplit8"),
    config_dma<Tile32x32K32S4>("dma_32x32x32_ksplit4"),
    config_dma<Tile32x64K16S8>("dma_32x64x16_ksplit8"),
    config_dma<Tile64x32K16S8>("dma_64x32x16_ksplit8"),
    config_dma<Tile128x128K32P, true>("dma_128x128x32_pipe"),
    config_dma<Tile64x64K32PL2S4>("dma_64x64x32_pipe_lw2_s4"),
    config_streamk<Tile64x64K16S8P>("dma_64x64x16_ksplit8_pipe_sk"),
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The device the work runs on, read once per device: its compute units
// (the unit the shape rule balances tiles over, and stream-K's worker count)
// and the dies (XCDs, 32 compute units each on MI355X) workgroups are dealt
// to round-robin.  A whole MI355X has 256 and 8; a partitioned one fewer.
// Without a usable device (plans described on a host without a GPU) the
// whole MI355X is assumed.
struct Machine {
    int64_t cus;
    int xcds;
};
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_cus[kMaxDevices];   // 0: not read yet

Machine machine()
{
    constexpr int kDefaultCus = 256, kCusPerXcd = 32;
    int dev = -1, cu = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        cu = kDefaultCus;
    } else {
        cu = g_device_cus[dev].load(std::memory_order_relaxed);
        if (cu == 0) {
            if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) {
                (void)hipGetLastError();
                cu = kDefaultCus;
            }
            g_device_cus[dev].store(cu, std::memory_order_relaxed);
        }
    }
    return {cu, cu % kCusPerXcd == 0 ? cu / kCusPerXcd : 1};
}

// The direct-to-LDS kernels address each panel with 32-bit buffer offsets
// from its corner: the farthest in-range element of an A panel is
// (BM-1)*lda + BK-1 floats away, of a B panel (BK-1)*ldb + BN-1.
bool dma_offsets_fit(const ConfigInfo &c, int64_t lda, int64_t ldb)
{
    const int64_t limit = (int64_t)kOutOfRange / 4;
    return (c.bm - 1) * lda + c.bk < limit && (c.bk - 1) * ldb + c.bn < limit;
}

// Tile choice by shape, from configuration sweeps (sweep.py) on MI355X: the
// workload shapes, square and mid-size shapes, and three sets of 40-44
// random shapes (M, N log-uniform in 100..8192, K in 64..16384).  Output
// tiles are the unit of parallelism; the rule prefers the biggest tiles of
// which there are enough for the 256 compute units, and a stream-K twin
// (all tiles' K-panels split evenly over one workgroup per CU) where the
// last round of whole tiles would leave too many CUs idle:
//  * K <= 1024 with at least four 128 x 128 tiles per CU: 128 x 128, 4
//    pipelined waves on 16-deep panels, three workgroups per CU (short K:
//    per-tile start-up and the C store weigh more than reuse; 8192 x 8192 x
//    128: 143 us against 146.5 for the same tile unpipelined, 8192 x 8192 x
//    512: 490 against 506);
//  * at least one 256 x 256 tile per CU: 256 x 256 with 4 software-pipelined
//    waves of 128 x 128, 32-deep panels, if they fill their rounds (8192^3:
//    7.31 ms against 7.45 for 16 waves of 64 x 64; 4096 x 4096 x 16384: 3.66
//    against 3.72); their stream-K twin for K >= 3072 with two or more
//    rounds of them if 128 x 128 tiles would not fill their rounds either
//    (7168 x 6656 x 4096: 2649 us against 2676 for the 128 x 128 twin);
//  * at least one 128 x 128 tile per CU, rounds filled: 128 x 128 with 4
//    pipelined waves of 64 x 64 -- one round: 64-deep panels fed by two
//    loader waves (2048^3: 123 us against 125.6 when the MFMA waves load,
//    133 for 16 waves in two K-split groups); two rounds: 32-deep panels,
//    two workgroups per CU (4096 x 2048 x 2048: 243 us against 248); more:
//    16-deep panels, three workgroups per CU (6144 x 2048 x 4096: 717
//    against 727); rounds not filled: the loader-wave tile's stream-K twin
//    for K >= 2048, or K >= 1024 with two or more tiles per CU (3072^3: 428
//    us against 455 for 64 x 64), two rounds of the 32-deep tile for K >=
//    1024 with a second round over four fifths full; otherwise, and for one
//    or two rounds with K < 512, 64 x 64 tiles;
//  * at least three quarters of the CUs busy with 128 x 128 tiles where
//    64 x 64 tiles would take four rounds: one round of the loader-wave
//    128 x 128 tile (1792^3: 109 us against 121 for 64 x 64), of the
//    32-deep one if a 64-deep last panel would be at most half used;
//  * at most one 64 x 64 tile per CU with K > 512 (mid-size squares, skinny
//    shapes): from K = 640 on, K split over 8 software-pipelined one-wave
//    groups (16384 x 64 x 4096: 72 us against 79 for 4 groups of 4 waves;
//    1024 x 1024 x 1280: 25.1 against 27.1 for the loader-wave tile), unless
//    K < 1536 and its 16-deep panels split unevenly over the 8 groups; else
//    4 pipelined waves of 32 x 32 fed by two loader waves through four
//    32-deep panels (1000 x 1000 x 600: 17.6 us against 18.1); a last tile row
//    (column, or both) of 1-4 rows (columns) past one round: one round of
//    the 8 pipelined groups, the remainder computed as strips spread over
//    all workgroups; past one round, 32 x 64 (64 x 32) tiles of 8 one-wave
//    K-split groups where they fill at most two rounds (K < 2560) or where
//    64-wide tiles would pad a side under 192 by a third more;
//  * up to six rounds of 64 x 64 tiles, K >= 950 and idle CU-rounds x K
//    large enough: stream-K over the 8 pipelined groups (1536^3: 70 us
//    against 82 for stream-K over 4 groups; 1025 x 1025 x 4096: 87 against
//    104), over the 4-group K split instead just past one round with K <
//    1536 (32 x 32 tiles of 4 K-split groups below K = 1150); otherwise two
//    rounds with K >= 1024, or three with K >= 2048:
//    whole tiles of the 8 pipelined groups (1300 x 1300 x 4096: 136 us
//    against 149; 2048 x 1536 x 2048: 101 against 110);
//  * otherwise 64-row or 64-column tiles if there are at least two per CU,
//    else 64 x 64.
// Below the largest tile the choices use 32- or 64-deep K-panels: those
// tiles give each wave few MFMAs per panel, so fewer, deeper panels cut the
// per-panel barrier, wait and LDS-latency cost (64-deep: +3 to +5 % at 1280^3
// and 2048 x 1024 x 1024, one or two 64 x 64 tiles per CU).  With deep_ok
// false (64-deep panels too tall for 32-bit offsets at the caller's leading
// dimensions) the 32-deep alternatives are chosen instead.  Where 128-wide
// tiles would cover over a quarter more padded area than 64 x 64 tiles (a
// side of at most 64, or of 129 to 192), only the 64 x 64 choices are
// considered (64 x 32768 x 4096: 154 us against 244).  Problems with
// fewer than 16 rows or columns use the vector-FMA kernel, where a 32-wide
// matrix-core block would be mostly padding.
int select_config(int M, int N, int K, bool dma_ok, bool deep_ok, int64_t CU, int &strip_rows, int &strip_cols)
{
    strip_rows = strip_cols = 0;
    if (M < 16 || N < 16)
        return kCfgValu64;
    auto tiles = [&](int c) { return ceil_div(M, kConfigs[c].bm) * ceil_div(N, kConfigs[c].bn); };
    if (!dma_ok) {
        if (tiles(kCfgStaged128x128) >= 4 * CU)
            return kCfgStaged128x128;
        return kCfgStaged64x64;
    }
    // Few output tiles: while 32 x 32 tiles fit in one round, one workgroup
    // per 32 x 32 tile of 8 K-split one-wave groups keeps every CU busy
    // (512^3: 9.4 us against 15.9 for 64 one-round 64 x 64 tiles; 256 x 256
    // x 8192: 45 against 126; 500^3: 9.8 against 16.3); with K <= 256, 4
    // groups (300 x 400 x 100: 6.7 against 7.2 for 8).  While 32 x 64 (64 x
    // 32) tiles fit in one round, 8 groups of those (640 x 640 x 2048: 25.9
    // us against 39.3; 1024 x 512 x 1024: 17.2 against 24.7), 32 x 64 ones
    // first (their panels' wider B rows: 848 x 383 x 723 13.6 us against 14.2
    // for 64 x 32; 700 x 600 x 1000: 15.8 against 16.2).
    const int64_t t32x32 = ceil_div(M, 32) * ceil_div(N, 32);
    if (t32x32 <= CU)
        return K > 256 ? kCfgDma32x32K32S8 : kCfgDma32x32K32S4;
    if (tiles(kCfgDma32x64K16S8) <= CU)
        return kCfgDma32x64K16S8;
    if (tiles(kCfgDma64x32K16S8) <= CU)
        return kCfgDma64x32K16S8;
    // The busiest CU has ceil(tiles / CUs) tiles.  The last round of tiles
    // leaves more than a fifth of the CU-rounds idle when this is true:
    auto unbalanced = [&](int c) {
        const int64_t t = tiles(c);
        return 5 * t < 4 * ceil_div(t, CU) * CU;
    };
    // Whether stream-K's even split beats whole tiles: over a long K its
    // extra launch and split tiles cost about 3 %, so it pays once the last
    // round leaves more than 4 % of the CU-rounds idle (7168 x 6656 x 4096,
    // 95 % filled: 2688 us against 2785 for 256 x 256 tiles; 5000 x 2600 x
    // 4096, 82 %: 813 against 954 for 128 x 128; 5120 x 5120 x 1536, 89 %:
    // 598 against 627 for the 16-deep 128 x 128 tile; but 3584 x 3456 x
    // 4096, 98 %: 730 against 719); below K = 1024 only past a fifth.
    auto streamk_pays = [&](int c) {
        const int64_t t = tiles(c);
        return K >= 1024 ? 25 * t < 24 * ceil_div(t, CU) * CU : unbalanced(c);
    };
    // Stream-K over the 8 pipelined groups of 64 x 64 tiles (below) pays
    // where, with up to max_rounds rounds of those tiles, the idle share of
    // their CU-rounds times K reaches min_idle_k (320 against the whole-tile
    // choices of the 64 x 64 region), from K = 950 on.
    auto idle_k = [&]() {   // idle share of the CU-rounds of 64 x 64 tiles, times K
        const int64_t t = tiles(kCfgDma64x64K32), r = ceil_div(t, CU);
        return (r * CU - t) * K / (r * CU);
    };
    auto psk_pays = [&](int64_t max_rounds, int64_t min_idle_k) {
        return K >= 950 && tiles(kCfgDma64x64K32) <= max_rounds * CU && idle_k() >= min_idle_k;
    };
    // A side of at most 64 (or 129 to 192) leaves 128-wide tiles a half (a
    // third) padding; once their padded area is over a quarter larger than
    // that of 64 x 64 tiles, only the 64 x 64 choices below are taken
    // (64 x 32768 x 4096: 154 us against 244 for 128 x 128 tiles; 192 x
    // 16384 x 4096: 202 against 243; 64 x 65536 x 1024: 75 against 240 for
    // 256 x 256).
    auto padded = [&](int edge) { return int64_t(ceil_div(M, edge)) * ceil_div(N, edge) * edge * edge; };
    const bool thin = 4 * padded(128) > 5 * padded(64);
    if (!thin && K <= 1024 && tiles(kCfgDma128x128K16P) >= 4 * CU)
        return kCfgDma128x128K16P;
    // 256 x 256 tiles: whole ones when they fill the rounds; stream-K over
    // them only for K >= 3072, at least two rounds of them, and when 128 x
    // 128 tiles would not fill their rounds either (7168 x 6656 x 4096: 2649
    // us against 2676 for stream-K over 128 x 128 tiles; but 5500 x 5500 x
    // 3500, 1.9 rounds: 1561 against 1487; 4451 x 4749 x 4858, 1.3 rounds:
    // 1521 against 1457; and 6478 x 5640 x 3472, 2295 of 2304 128 x 128
    // slots used: 1796 against 1909 for 256 x 256 stream-K); otherwise the
    // 128 x 128 choices (7369 x 2892 x 2379: 794 against 829; 3813 x 6105 x
    // 766: 281 against 354).
    if (!thin && tiles(kCfgDma256x256K32P) >= CU) {
        if (!streamk_pays(kCfgDma256x256K32P))
            return kCfgDma256x256K32P;
        if (K >= 3072 && tiles(kCfgDma256x256K32P) >= 2 * CU && streamk_pays(kCfgDma128x128K64P))
            return kCfgDma256x256K32PSK;
    }
    const int64_t t128 = tiles(kCfgDma128x128K64P);
    if (!thin && t128 >= CU) {
        if (!streamk_pays(kCfgDma128x128K64P)) {
            // Three or more rounds: three resident workgroups of the 16-deep
            // pipelined tile overlap each other's start-up and stores
            // (6000 x 2000 x 1000: 185 us against 198; 6144 x 2048 x 4096: 717
            // against 727 for 64-deep panels; 6478 x 5640 x 3472: 1796 against
            // 1856).  Two rounds: two resident workgroups of the 32-deep one
            // (4096 x 2048 x 2048: 243 against 248 for 64-deep panels and 250
            // for 16-deep ones; 4096 x 2048 x 1024: 125.5 against 128.5).
            if (t128 > 2 * CU || (t128 == 2 * CU && K < 512))
                return kCfgDma128x128K16P;
            // One or two rounds with a short K: a 64-deep panel ring has
            // too few rounds to fill; 64 x 64 tiles balance better
            // (5221 x 1201 x 233: 37.9 us against 50.5).
            if (K < 512)
                return kCfgDma64x64K32;
            if (t128 > CU)
                return kCfgDma128x128K32P;
            return deep_ok ? kCfgDma128x128K64P : kCfgDma128x128K32S2;
        }
        // Stream-K's extra launch and split-tile passes pay off over a long
        // K, from K = 1024 on with two or more tiles per CU; otherwise four
        // or more 64 x 64 tiles per CU balance well enough (2200 x 2200 x
        // 1500, 324 tiles: 135 us against 148 for stream-K; 941 x 4305 x
        // 1100, 272: 81 against 107), unless with K >= 1024 the last round
        // of 128 x 128 tiles is over four fifths full: two rounds of the
        // 32-deep pipelined tile (3428 x 2297 x 1956, 486 tiles: 235 us
        // against 267 for 64 x 64 tiles).
        if (K >= 2048 || (K >= 1024 && t128 >= 2 * CU))
            return deep_ok ? kCfgDma128x128K64PSK : kCfgDma128x128K32W16SK;
        if (K >= 1024 && t128 <= 2 * CU && !unbalanced(kCfgDma128x128K64P))
            return kCfgDma128x128K32P;
        // (Up to six rounds of 64 x 64 tiles, stream-K over the 8 pipelined
        // groups where it pays, here from an idle share x K of 160 on, the
        // 64 x 64 tiles of 4 waves being the alternative: 198 x 16642 x
        // 1898: 149.5 us against 166.7; 2600 x 2000 x 1800: 169.5 against
        // 184.3; 3317 x 1235 x 1323: 111.1 against 118.7; but 1500 x 3500 x
        // 1050, 148: 119.2 against 110.3.)
        return psk_pays(6, 160) ? kCfgDma64x64K16S8PSK : kCfgDma64x64K32;
    }
    // At least three quarters of the CUs busy with 128 x 128 tiles: one
    // round of them where 64 x 64 tiles would take four rounds, as much
    // work per CU, the bigger tiles doing it faster (2372 x 1619 x 7588, 247
    // tiles: 443 us against 504 for 64 x 64 tiles; 1746 x 1863 x 3494, 210:
    // 211 against 235; 3394 x 1064 x 960, 918 64 x 64 tiles: 62.9 against
    // 69.5; but 3072 x 1024 x 2048, 192 (768): 126 against 109; 1551 x 1838
    // x 1619, 195 (725): 104.6 against 88.3); the loader-wave tile's 64-deep
    // panels unless the last one would be at most half used and its padding
    // over 1/32 of K, then 32-deep ones (2286 x 1396 x 758: 53.6 us against
    // 54.0; 2282 x 1391 x 771: 57.6 against 60.1; but 1800 x 1800 x 2500:
    // 152.9 against 155.2 for 32-deep panels).  Not where the fourth round of 64 x 64 tiles is nearly
    // empty and K long, idle share x K >= 1000: stream-K over the 8
    // pipelined groups then does less (1664 x 1950 x 11185: 603 us against
    // 636; 1700 x 1900 x 5000: 276 against 292; but 2000 x 1700 x 4000,
    // 625: 237.6 against 234.6).
    if (!thin && K > 512 && 4 * t128 >= 3 * CU && ceil_div(tiles(kCfgDma64x64K32), CU) >= 4 &&
        !psk_pays(6, 1000))
        return deep_ok && (64 * ceil_div(K, 64) == 32 * ceil_div(K, 32) || 32 * (64 * ceil_div(K, 64) - K) <= K)
                   ? kCfgDma128x128K64P
                   : kCfgDma128x128K32P;
    // 64 x 64 tiles with K > 512 (one round: K >= 400), up to three rounds
    // of them.  One tile per CU: 8 pipelined one-wave K-split groups from K
    // = 640 on (and from 400 to 512), unless the
    // 16-deep panels split unevenly over the groups (the busiest group's
    // rounds span over 9/8 of K rounded up to 32-deep panels) while K < 1536;
    // otherwise 4 pipelined waves of 32 x 32 fed by two loader waves through
    // a ring of four 32-deep panels (1024 x 1024 x 1280: 25.1 us for the 8
    // groups against 27.1; 1000^3: 23.7 against 24.0, 25.1 for 4 K-split
    // groups of 4 waves; 1024 x 1024 x 640: 16.0 against 17.2; but 800 x
    // 1200 x 650, 41 panels over 8 groups: 18.8 against 18.3, and 1000 x
    // 1000 x 600: 18.1 against 17.6).  Past one round: stream-K over the 8
    // pipelined groups where enough of the rounds would idle, over the
    // 4-group K split just past one round; else whole tiles of the 8 groups
    // for two rounds with K >= 1024 or three with K >= 2048.
    const int64_t t32 = tiles(kCfgDma64x64K32);
    // A last tile row of at most kMaxStripRows rows that alone takes the
    // tiles past one round: those rows become a strip computed with FMAs,
    // spread over all workgroups, and the rest runs as one round of the 8
    // pipelined K-split groups.  Strips stay from K = 257 up to rows x K =
    // 4096, and each workgroup's share of the strip's columns up to
    // kMaxStripSpread (1025 x 1023 x 1000: 26.8 us against 29.7 for the
    // strip summed by the last tile row of 4-group K-split tiles, 37.3 for
    // stream-K; 1000 x 1028 x 1000: 26.7 against 35.0; 1025 x 1023 x 3000:
    // 58.2 against 65.2 for stream-K over the 8 pipelined groups; 1028 x 1000
    // x 400: 17.3 against 20.7 for two rounds of 64 x 64 tiles; but 1023 x
    // 1025 x 256: 15.3 against 15.3).
    const int64_t t_full = (M / 64) * ceil_div(N, 64);
    static_assert(std::is_same<Tile64x64K16S8P, StripTile>::value, "the strip tile is the 8-group pipelined K split");
    if (K > 256 && M % 64 != 0 && M % 64 <= kMaxStripRows && (M % 64) * K <= 4096 &&
        t_full <= CU && t32 > CU && ceil_div(N, t_full) <= kMaxStripSpread) {
        strip_rows = M % 64;
        return kCfgDma64x64K16S8P;
    }
    // Both a last tile row and a last tile column of 1-4 rows (columns):
    // both as strips, the row strip spanning all N columns, up to K =
    // kMaxBothStripsK (1025 x 1025 x 1000: 30.7 us against 39.8 for stream-K
    // over the 4-group K split; 1025 x 1025 x 2000: 47.6 against 54.5 and
    // 1025 x 1025 x 3000: 66.0 against 71.7 for stream-K over the 8
    // pipelined groups; but 1025 x 1025 x 4096: 91.4 against 86.9).
    const int64_t t_inner = (M / 64) * (N / 64);
    if (K > 256 && K <= kMaxBothStripsK && M % 64 != 0 && M % 64 <= kMaxStripRows && N % 64 != 0 &&
        N % 64 <= kMaxStripRows && (M % 64) * K <= 4096 && (N % 64) * K <= 4096 && t_inner <= CU && t32 > CU &&
        ceil_div(N, t_inner) <= kMaxStripSpread && ceil_div(M, t_inner) <= kMaxStripSpread) {
        strip_rows = M % 64;
        strip_cols = N % 64;
        return kCfgDma64x64K16S8P;
    }
    // The same for a last tile column of at most kMaxStripRows columns.
    const int64_t t_full_n = ceil_div(M, 64) * (N / 64);
    if (K > 256 && N % 64 != 0 && N % 64 <= kMaxStripRows && (N % 64) * K <= 4096 &&
        t_full_n <= CU && t32 > CU && ceil_div(M, t_full_n) <= kMaxStripSpread) {
        strip_cols = N % 64;
        return kCfgDma64x64K16S8P;
    }
    // (From K = 400 to 512 the 8 groups win whatever the split: 1024 x 1024
    // x 512: 14.1 us against 16.2 for dma_64x64x64; 1024 x 1024 x 448: 13.3
    // against 14.3 for the loader-wave tile; 1000 x 1000 x 400: 13.9 against
    // 14.9;
    // below, 64 x 64 tiles of 4 waves: 1024 x 1024 x 300: 12.2 against 12.5.)
    if (K >= 400 && t32 <= CU) {
        const int64_t k8 = 128 * ceil_div(ceil_div(K, 16), 8);   // K the busiest of the 8 groups covers
        const int64_t k4 = 32 * ceil_div(K, 32);                  // K the loader-wave tile covers
        return K <= 512 || K >= 1536 || (K >= 640 && 8 * k8 <= 9 * k4) ? kCfgDma64x64K16S8P : kCfgDma64x64K32PL2S4;
    }
    // Past one round, 32 x 64 (64 x 32) tiles of the 8 one-wave K-split
    // groups that fill at most two rounds (a last tile row of at most 32
    // rows) give no CU more work than one round of 64 x 64 tiles would; for
    // 256 < K < 2560 that beats stream-K and a second round of 64 x 64 tiles
    // (535 x 1913 x 2314: 53.0 us against 60.0 for stream-K over the 8
    // pipelined groups; 1620 x 634 x 695: 22.1 against 30.4 for stream-K
    // over the 4-group K split; 4157 x 207 x 1519: 38.4 against 44.1; 535 x
    // 1913 x 450: 18.7 against 22.6 for dma_64x64x32; but 1247 x 792 x 4980:
    // 99.2 against 91.1).
    if (K > 256 && K < 2560 && t32 > CU && tiles(kCfgDma32x64K16S8) <= 2 * CU)
        return kCfgDma32x64K16S8;
    if (K > 256 && K < 2560 && t32 > CU && tiles(kCfgDma64x32K16S8) <= 2 * CU)
        return kCfgDma64x32K16S8;
    // Past one round, a side under 192 that 64-wide tiles pad a third more
    // than 32-wide ones: 32 x 64 (64 x 32) tiles of the 8 one-wave K-split
    // groups, in up to three rounds, do less work (95 x 8926 x 1248: 32.5 us
    // against 41.4 for stream-K; 8926 x 95 x 1248: 33.3 against 42.0; 80 x
    // 12000 x 2000: 65.9 against 69.6; 15133 x 90 x 3196: 101.4 against 106.8
    // for 64 x 64 tiles of the 8 pipelined groups).
    auto pads_third_more = [](int side) { return side < 192 && 3 * ceil_div(side, 64) * 64 >= 4 * ceil_div(side, 32) * 32; };
    if (K > 512 && t32 <= 3 * CU) {
        if (pads_third_more(M) && tiles(kCfgDma32x64K16S8) <= 3 * CU)
            return kCfgDma32x64K16S8;
        if (pads_third_more(N) && tiles(kCfgDma64x32K16S8) <= 3 * CU)
            return kCfgDma64x32K16S8;
    }
    // Stream-K over the 8 pipelined groups where the idle share of the
    // CU-rounds times K reaches 320 (from K = 950 on; 1025 x 1025 x 4096: 87
    // us against 104 for the 4-group K split; 808 x 1496 x 6456: 135 against
    // 166; 868 x 1930 x 5448, last round 70 % full: 157 against 170 for whole
    // tiles of the 8 groups; 1249 x 1618 x 999: 55.0 against 57.7; but 1197 x
    // 2414 x 2779, 94 % full: 142 against 141, and 3280 x 682 x 1149, 75 %:
    // 66.6 against 64.4 for 64 x 64 tiles), except just past one round with
    // K < 1536, where the 4-group K split's lighter pieces win (574 x 1850 x
    // 1256: 40.6 us against 43.0), and below K = 1150 32 x 32 tiles of 4
    // one-wave K-split groups, two workgroups per CU, without stream-K's
    // extra launch (660 x 1684 x 979: 35.6 us against 38.3; 789 x 1518 x
    // 1137: 40.6 against 43.7; on 10 random shapes of 257-320 64 x 64 tiles
    // with K in 513-950: 0.1 % above the per-shape best, against 10 % for
    // stream-K; but 1993 x 539 x 1078: 39.8 against 39.4).
    if (psk_pays(6, 320) && (t32 > 5 * CU / 4 || K >= 1536))
        return kCfgDma64x64K16S8PSK;
    if (K > 512 && t32 <= 5 * CU / 4)
        return K < 1150 ? kCfgDma32x32K32S4 : kCfgDma64x64K32S4SK;
    // Two rounds favour the 8 pipelined groups from K = 1024 on (2048 x
    // 1024 x 1024: 39.3 us against 42.1 for 64 x 64 tiles of 4 waves; 1600
    // x 1200 x 1200: 45.2 against 48.5; 2048 x 1024 x 1100: 45.5 against
    // 45.3; but 1400 x 1400 x 1000: 43.6 against 42.3), three rounds with a
    // fuller last one from K = 2048 on (2048 x 1536 x 2048: 101.2 against
    // 109.5; 5932 x 460 x 2048: 101.7 against 109.4; but 1900 x 1600 x 1500:
    // 83.2 against 81.7).
    if (K >= 1024 && t32 <= 2 * CU)
        return kCfgDma64x64K16S8P;
    if (K >= 2048 && t32 <= 3 * CU)
        return kCfgDma64x64K16S8P;
    // 64 x 128 (128 x 64) tiles with at least two per CU, unless a side
    // pads 128-wide tiles a quarter more (48857 x 138 x 860: 146.6 us
    // against 137.0 for 64 x 64 tiles; 33933 x 157 x 708: 104.3 against
    // 92.0; but 64 x 65536 x 1024, exactly two rounds of 64 x 128 tiles:
    // 74.8 against 74.3).
    const int wide = N >= M ? kCfgDma64x128K32 : kCfgDma128x64K32;
    if (!thin && tiles(wide) >= 2 * CU)
        return wide;
    // 64 x 64 tiles.  Up to two per CU, the one or two 4-wave workgroups
    // leave each SIMD one or two waves, and 64-deep panels halve the
    // per-panel barrier stalls that then show, unless their last panel is
    // at most half used (K % 64 in 1..32), which 32-deep panels avoid, or K
    // is under 256 (600 x 3000 x 200: 14.2 us against 15.6; 956 x 1597 x
    // 331: 18.9 against 20.1; 1590 x 744 x 100: 11.0 against 11.4; but 1280
    // x 1280 x 512: 23.7 against 24.1 for 32-deep panels, 1000 x 1000 x 300:
    // 12.6 against 12.8); with more, several
    // workgroups share a CU and the smaller 32-deep panels (more resident
    // workgroups) win.  Stream-K does not pay here, even barely past one
    // round: with K <= 512 its clearing launch and split tiles cost more
    // than the second round (1025 x 1023 x 300: 22.1 us against 17.6;
    // 1590 x 744 x 100: 17.1 against 11.0).
    const int64_t t64 = tiles(kCfgDma64x64K64);
    if (t64 <= 2 * CU)
        return deep_ok && K >= 256 && 64 * ceil_div(K, 64) == 32 * ceil_div(K, 32) ? kCfgDma64x64K64 : kCfgDma64x64K32;
    return kCfgDma64x64K32;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

struct Plan {
    int config;
    bool vec_a, vec_b;
    bool wb_c;           // run the configuration's write-back C-store twin
    int tiles_m, tiles_n;
    int grid;
    int strip_rows;      // rows below the tile grid, computed as a strip
    int strip_cols;      // columns right of it, computed as a strip
    int xcds;            // the device's dies (tile order)
    bool shares_tiles;   // stream-K: some tiles are summed in C by two
                         // workgroups with atomic adds
};

// Validates the arguments (sizes, leading dimensions, configuration index,
// NULL pointers, alignment, in that order) and fills `plan`; returns a
// GEMM_F32_* code.
int make_plan(int config, int M, int N, int K, const float *A, int lda,
              const float *B, int ldb, const float *C, int ldc, Plan *plan)
{
    if (M < 0 || N < 0 || K < 0)
        return GEMM_F32_ERR_DIM;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1))
        return GEMM_F32_ERR_LD;
    if (config < -1 || config >= kNumConfigs)
        return GEMM_F32_ERR_CONFIG;
    plan->config = -1;
    plan->vec_a = plan->vec_b = false;
    plan->wb_c = false;
    plan->tiles_m = plan->tiles_n = plan->grid = 0;
    plan->strip_rows = plan->strip_cols = 0;
    plan->xcds = 1;
    plan->shares_tiles = false;
    if (M == 0 || N == 0)
        return GEMM_F32_OK;
    if (C == nullptr || (K > 0 && (A == nullptr || B == nullptr)))
        return GEMM_F32_ERR_NULL;
    if (((uintptr_t)C & 3u) || (K > 0 && (((uintptr_t)A & 3u) || ((uintptr_t)B & 3u))))
        return GEMM_F32_ERR_ALIGN;
    if (K == 0) {
        plan->grid = (int)(ceil_div((int64_t)M * N, 256) < 4096 ? ceil_div((int64_t)M * N, 256) : 4096);
        return GEMM_F32_OK;
    }
    int c = config;
    int strip = 0, strip_c = 0;
    const Machine mach = machine();
    plan->xcds = mach.xcds;
    if (c < 0) {
        // The rule's direct-to-LDS choice; if its panels are too tall or deep
        // for 32-bit offsets at these leading dimensions, its choice among
        // 32-deep panels, and failing that the register-staged kernel.
        c = select_config(M, N, K, true, true, mach.cus, strip, strip_c);
        if (kConfigs[c].dma && !dma_offsets_fit(kConfigs[c], lda, ldb))
            c = select_config(M, N, K, true, false, mach.cus, strip, strip_c);
        if (kConfigs[c].dma && !dma_offsets_fit(kConfigs[c], lda, ldb))
            c = select_config(M, N, K, false, false, mach.cus, strip, strip_c);
    } else if (kConfigs[c].dma && !dma_offsets_fit(kConfigs[c], lda, ldb)) {
        return GEMM_F32_ERR_CONFIG;   // this kernel cannot address such wide rows
    }
    // The strip kernel sums at most kMaxStripRows rows (columns), and each
    // workgroup at most kMaxStripSpread columns (rows) of them; the rule
    // never plans more.
    if (strip > kMaxStripRows || strip_c > kMaxStripRows)
        return GEMM_F32_ERR_CONFIG;
    const int64_t tm = strip ? (M - strip) / kConfigs[c].bm : ceil_div(M, kConfigs[c].bm);
    const int64_t tn = strip_c ? (N - strip_c) / kConfigs[c].bn : ceil_div(N, kConfigs[c].bn);
    if (tm * tn > INT32_MAX)
        return GEMM_F32_ERR_DIM;
    if ((strip && ceil_div(N, tm * tn) > kMaxStripSpread) || (strip_c && ceil_div(M, tm * tn) > kMaxStripSpread))
        return GEMM_F32_ERR_CONFIG;
    plan->config = c;
    plan->strip_rows = strip;
    plan->strip_cols = strip_c;
    plan->tiles_m = (int)tm;
    plan->tiles_n = (int)tn;
    if (kConfigs[c].streamk) {
        plan->grid = (int)(tm * tn < mach.cus ? tm * tn : mach.cus);
        // A tile is shared when a worker's range starts inside it (the
        // workers' ranges as streamk_range cuts them).
        const int64_t ktiles = ceil_div(K, kConfigs[c].bk), iters = tm * tn * ktiles;
        for (int b = 1; b < plan->grid && !plan->shares_tiles; ++b) {
            const int64_t lo = iters / plan->grid * b + iters % plan->grid * b / plan->grid;
            plan->shares_tiles = lo % ktiles != 0;
        }
    } else
        plan->grid = (int)(tm * tn < kMaxGrid ? tm * tn : kMaxGrid);
    plan->wb_c = kConfigs[c].launch_wb != nullptr && !strip && !strip_c &&
                 !(aligned16(C) && ldc % 4 == 0) && (int64_t)M * N >= kWriteBackFromElems;
    if (kConfigs[c].dma) {
        // Direct-to-LDS loads move 16 bytes from any 4-byte aligned address
        // (checked on gfx950 together with the per-dword range check).  A
        // chunk of B that crosses column N only feeds C columns >= N, which
        // are never stored; a chunk of A that crosses column K has the
        // elements past it cleared in LDS before use.  The panels' buffer
        // ranges end at A's and B's last elements, so nothing beyond them is
        // read.
        plan->vec_a = true;
        plan->vec_b = true;
    } else {
        plan->vec_a = aligned16(A) && lda % 4 == 0 && K % 4 == 0;
        plan->vec_b = aligned16(B) && ldb % 4 == 0 && N % 4 == 0;
    }
    return GEMM_F32_OK;
}

int run(int config, int M, int N, int K, const float *A, int lda, const float *B,
        int ldb, float *C, int ldc, hipStream_t stream)
{
    Plan p;
    const int rc = make_plan(config, M, N, K, A, lda, B, ldb, C, ldc, &p);
    if (rc != GEMM_F32_OK || p.grid == 0)
        return rc;
    if (K == 0) {
        fill_zero<<<p.grid, 256, 0, stream>>>(C, ldc, M, N);
        return hipGetLastError() == hipSuccess ? GEMM_F32_OK : GEMM_F32_ERR_LAUNCH;
    }
    GemmArgs g;
    g.A = A;
    g.B = B;
    g.C = C;
    g.lda = lda;
    g.ldb = ldb;
    g.ldc = ldc;
    g.M = M;
    g.N = N;
    g.K = K;
    g.tiles_m = p.tiles_m;
    g.tiles_n = p.tiles_n;
    g.slices = 1;
    g.slab = 0;
    g.strip_rows = p.strip_rows;
    g.strip_cols = p.strip_cols;
    g.xcds = p.xcds;
    // A plan with a remainder strip runs the strip tile's strip kernel (the
    // rule pairs strips with that tile only).
    const hipError_t err = p.strip_rows > 0 || p.strip_cols > 0
                               ? LaunchDma<StripTile, false, false, true>::run(g, true, true, p.grid, stream)
                           : p.wb_c ? kConfigs[p.config].launch_wb(g, p.vec_a, p.vec_b, p.grid, stream)
                                    : kConfigs[p.config].launch(g, p.vec_a, p.vec_b, p.grid, stream);
    return err == hipSuccess ? GEMM_F32_OK : GEMM_F32_ERR_LAUNCH;
}

// Split-K with a caller's workspace, for problems with few output tiles and
// a long K: the 64 x 64 K-split tiles run as `slices` independent
// workgroups per tile, each over a contiguous K slice, writing partial
// products to the workspace; a second kernel adds them in slice order.
using TileSplitK = Tile64x64K32S4;
constexpr int kSplitKMinPanels = 8;     // 32-deep panels per slice, at least

// Slices for this shape, or 1 when split-K does not apply: only while the
// 64 x 64 tiles fill at most half of the CUs, as many slices as fill them,
// each at least kSplitKMinPanels panels deep (640 x 640 x 8192, 100 tiles:
// 147 us without, 82 us with two slices).
int splitk_slices(int M, int N, int K)
{
    if (M < 16 || N < 16 || K <= 0)
        return 1;
    const int64_t cus = machine().cus;
    const int64_t t = ceil_div(M, TileSplitK::BM) * ceil_div(N, TileSplitK::BN);
    if (2 * t > cus)
        return 1;
    int64_t slices = cus / t;
    const int64_t by_depth = ceil_div(K, TileSplitK::BK) / kSplitKMinPanels;
    if (by_depth < slices)
        slices = by_depth;
    return slices >= 2 ? (int)slices : 1;
}

size_t splitk_bytes(int M, int N, int K)
{
    const int slices = splitk_slices(M, N, K);
    return slices < 2 ? 0 : (size_t)slices * (size_t)M * (size_t)N * sizeof(float);
}

int run_workspace(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                  float *C, int ldc, void *ws, size_t ws_bytes, hipStream_t stream)
{
    Plan p;
    int rc = make_plan(-1, M, N, K, A, lda, B, ldb, C, ldc, &p);
    if (rc != GEMM_F32_OK || p.grid == 0 || K == 0)
        return run(-1, M, N, K, A, lda, B, ldb, C, ldc, stream);
    const int slices = splitk_slices(M, N, K);
    const size_t need = splitk_bytes(M, N, K);
    // Slices of at least 2048 of K run the pipelined 8-group K-split tile
    // (640 x 640 x 8192, two slices: 74 us against 83; 512 x 512 x 8192:
    // 45 against 47), shorter ones the 4-group tile (130 x 70 x 5000, 19
    // slices: 21.6 us against 25).  Both cover the same 64 x 64 tiles.
    static_assert(Tile64x64K16S8P::BM == TileSplitK::BM && Tile64x64K16S8P::BN == TileSplitK::BN, "same tiles");
    const bool pipe = K / slices >= 2048;
    const ConfigInfo &cfg = kConfigs[pipe ? kCfgDma64x64K16S8P : kCfgDma64x64K32S4];
    if (slices < 2 || ws == nullptr || ws_bytes < need || ((uintptr_t)ws & 15u) ||
        !dma_offsets_fit(cfg, lda, ldb))
        return run(-1, M, N, K, A, lda, B, ldb, C, ldc, stream);
    GemmArgs g;
    g.A = A;
    g.B = B;
    g.C = (float *)ws;
    g.lda = lda;
    g.ldb = ldb;
    g.ldc = N;
    g.M = M;
    g.N = N;
    g.K = K;
    g.tiles_m = (int)ceil_div(M, TileSplitK::BM);
    g.tiles_n = (int)ceil_div(N, TileSplitK::BN);
    g.slices = slices;
    g.slab = (int64_t)M * N;
    g.strip_rows = g.strip_cols = 0;
    g.xcds = p.xcds;
    const int grid = g.tiles_m * g.tiles_n * slices;
    hipError_t err = pipe ? LaunchDma<Tile64x64K16S8P, false, true>::run(g, true, true, grid, stream)
                          : LaunchDma<TileSplitK, false, true>::run(g, true, true, grid, stream);
    if (err != hipSuccess)
        return GEMM_F32_ERR_LAUNCH;
    const int64_t elems = (int64_t)M * N;
    const int rgrid = (int)(ceil_div(elems, 256) < 4096 ? ceil_div(elems, 256) : 4096);
    splitk_reduce<<<rgrid, 256, 0, stream>>>((const float *)ws, g.slab, slices, C, ldc, M, N);
    return hipGetLastError() == hipSuccess ? GEMM_F32_OK : GEMM_F32_ERR_LAUNCH;
}

// Split-K scratch that the library owns, for callers that cannot allocate
// (gemm_f32_ws_noalloc): one array per device, held until the process ends.
// A split plan runs at most one 64 x 64 tile slice per compute unit, so its
// slabs hold at most 256 x 64 x 64 floats on a whole MI355X: 4 MiB covers
// every split plan there (a device with more compute units can need more,
// and such plans are refused).  In host code `scratch` names a host-side
// stand-in, never the device array: kernels and copies get the per-device
// address hipGetSymbolAddress returns.
constexpr size_t kScratchBytes = GEMM_F32_SCRATCH_BYTES;
static_assert(kScratchBytes == size_t(256) * 64 * 64 * sizeof(float), "one 64 x 64 slab per compute unit");
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

std::atomic<void *> g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (resolved on the first call on that
// device, with it current), or nullptr if it cannot be resolved.
void *scratch_on_current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    void *ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
    return ptr;
}

int run_noalloc(int M, int N, int K, const float *A, int lda, const float *B, int ldb, float *C, int ldc,
                hipStream_t stream)
{
    Plan p;
    const int rc = make_plan(-1, M, N, K, A, lda, B, ldb, C, ldc, &p);
    if (rc != GEMM_F32_OK || p.grid == 0 || K == 0)
        return run(-1, M, N, K, A, lda, B, ldb, C, ldc, stream);   // nothing split, nothing allocated
    if (splitk_bytes(M, N, K) > kScratchBytes)
        return GEMM_F32_ERR_SCRATCH;
    void *ws = scratch_on_current_device();
    if (ws == nullptr)
        return GEMM_F32_ERR_LAUNCH;
    return run_workspace(M, N, K, A, lda, B, ldb, C, ldc, ws, kScratchBytes, stream);
}

}  // namespace

extern "C" {

int gemm_f32_ws_noalloc(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                        float *C, int ldc, hipStream_t stream)
{
    return run_noalloc(M, N, K, A, lda, B, ldb, C, ldc, stream);
}

size_t gemm_f32_ws_size(int M, int N, int K)
{
    return M < 0 || N < 0 || K < 0 ? 0 : splitk_bytes(M, N, K);
}

int gemm_f32_ws(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                float *C, int ldc, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return run_workspace(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes, stream);
}

int gemm_f32(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
             float *C, int ldc, hipStream_t stream)
{
    return run(-1, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int gemm_f32_with_config(int config, int M, int N, int K, const float *A, int lda,
                         const float *B, int ldb, float *C, int ldc, hipStream_t stream)
{
    return run(config, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int gemm_f32_num_configs(void) { return kNumConfigs; }

int gemm_f32_config_info(int config, int *bm, int *bn, int *bk, int *threads, int *blocks_per_cu)
{
    if (config < 0 || config >= kNumConfigs)
        return GEMM_F32_ERR_CONFIG;
    const ConfigInfo &c = kConfigs[config];
    if (bm) *bm = c.bm;
    if (bn) *bn = c.bn;
    if (bk) *bk = c.bk;
    if (threads) *threads = c.threads;
    if (blocks_per_cu) {
        const int n = kConfigs[config].occupancy();
        if (n < 0)
            return GEMM_F32_ERR_LAUNCH;
        *blocks_per_cu = n;
    }
    return GEMM_F32_OK;
}

int gemm_f32_device_peak(int device, int *compute_units, int *clock_khz, double *tflops)
{
    // One v_mfma_f32_32x32x2_f32 is 32 * 32 * 2 multiply-adds (4096 FLOP)
    // and occupies a SIMD's matrix core for 64 cycles; a compute unit has 4
    // SIMDs, so 256 FLOP per clock.
    constexpr double kFlopPerClockPerCU = 4 * 4096.0 / 64;
    int cu = 0, khz = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeClockRate, device) != hipSuccess) {
        (void)hipGetLastError();
        return GEMM_F32_ERR_LAUNCH;
    }
    if (compute_units) *compute_units = cu;
    if (clock_khz) *clock_khz = khz;
    if (tflops) *tflops = cu * kFlopPerClockPerCU * (khz * 1e3) / 1e12;
    return GEMM_F32_OK;
}

const char *gemm_f32_config_name(int config)
{
    return (config >= 0 && config < kNumConfigs) ? kConfigs[config].name : "";
}

int gemm_f32_describe(int config, int M, int N, int K, const float *A, int lda,
                      const float *B, int ldb, const float *C, int ldc, char *buf, int buflen)
{
    Plan p;
    const int rc = make_plan(config, M, N, K, A, lda, B, ldb, C, ldc, &p);
    if (buf == nullptr || buflen <= 0)
        return rc;
    if (rc != GEMM_F32_OK)
        snprintf(buf, (size_t)buflen, "invalid: %s", gemm_f32_status_string(rc));
    else if (p.config < 0)
        snprintf(buf, (size_t)buflen, "%s", p.grid ? "fill_zero" : "none");
    else {
        const int n = snprintf(buf, (size_t)buflen, "%s tiles=%dx%d grid=%d threads=%d load_a=%s load_b=%s",
                               kConfigs[p.config].name, p.tiles_m, p.tiles_n, p.grid,
                               kConfigs[p.config].threads, p.vec_a ? "x4" : "x1", p.vec_b ? "x4" : "x1");
        if (p.strip_rows > 0 && n >= 0 && n < buflen)
            snprintf(buf + n, (size_t)(buflen - n), " strip_rows=%d", p.strip_rows);
        int used = (int)strlen(buf);
        if (p.strip_cols > 0 && used + 1 < buflen)
            snprintf(buf + used, (size_t)(buflen - used), " strip_cols=%d", p.strip_cols);
        used = (int)strlen(buf);
        if (p.wb_c && used + 1 < buflen)
            snprintf(buf + used, (size_t)(buflen - used), " c_store=write_back");
        used = (int)strlen(buf);
        if (p.shares_tiles && used + 1 < buflen)
            snprintf(buf + used, (size_t)(buflen - used), " c_accumulate=atomic_add");
        used = (int)strlen(buf);
        if (kPoisonLds && used + 1 < buflen)
            snprintf(buf + used, (size_t)(buflen - used), " lds=poisoned");
    }
    return rc;
}

const char *gemm_f32_status_string(int status)
{
    switch (status) {
    case GEMM_F32_OK: return "ok";
    case GEMM_F32_ERR_DIM: return "M, N or K is negative or the problem is too large to tile";
    case GEMM_F32_ERR_LD: return "a leading dimension is smaller than its row length";
    case GEMM_F32_ERR_NULL: return "a required pointer is NULL";
    case GEMM_F32_ERR_LAUNCH: return "kernel launch failed";
    case GEMM_F32_ERR_CONFIG: return "unknown kernel configuration";
    case GEMM_F32_ERR_ALIGN: return "a pointer is not 4-byte aligned";
    case GEMM_F32_ERR_SCRATCH: return "the split plan needs more than the library's static scratch holds";
    default: return "unknown status";
    }
}

}  // extern "C"
