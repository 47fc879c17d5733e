// Device code of the dense GEMM: C = A . B on gfx950 matrix cores.
//
// One kernel template serves both input types:
//   fp32 inputs  -> v_mfma_f32_32x32x2_f32    (fp32 products, fp32 accumulate)
//   bf16 inputs  -> v_mfma_f32_32x32x16_bf16  (exact products, fp32 accumulate)
//
// Structure (the tiling of "Learning to develop for GPUs through the GEMM
// operation", sections "Making the GPU implementation better" through "How to
// do even better", rebuilt for CDNA4 wave64 matrix cores):
//   * each workgroup owns a BM x BN block of C and walks K in tiles of BK;
//   * each tile of A (BM x BK) and B (BK x BN) is copied from HBM with 16-byte
//     loads into LDS, double buffered, so the copy of tile t+1 overlaps the
//     products of tile t and one barrier per tile suffices;
//   * LDS rows are padded (or XOR-swizzled) so the 16-byte fragment reads of a
//     wave spread over all banks ("How to do even better": padding moves rows
//     onto different banks);
//   * each wave owns a (BM/WM) x (BN/WN) sub-block held as 32x32 accumulator
//     fragments in registers and reuses every A and B fragment it reads across
//     that sub-block (the register blocking of "Improving the solution and
//     balancing memory work");
//   * blocks that cross the M, N or K edge take a masked path that loads zeros
//     outside the matrix and stores only inside it; the branch is uniform over
//     the workgroup.
//
// k-slot assignment.  A 32x32 MFMA pairs, in each of its k slots, the A value a
// lane supplies with the B value the same-numbered lane half supplies.  Lanes
// 0-31 feed one slot group and lanes 32-63 the other.  Within one tile, lane
// half h takes the contiguous k range [h*BK/2, (h+1)*BK/2), so a lane's A
// values for a whole tile are contiguous in an LDS row and come in 16-byte
// reads.  B is laid out so that the same k reaches the same slot, so every
// product A[i][k]*B[k][j] of the definition is formed exactly once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Arguments of one launch.  The grid is 1-D: splits * tiles_m * tiles_n blocks.
struct KernelArgs {
    const void *A;
    const void *B;
    float *C;       // final output (splits == 1)
    float *ws;      // split-K partial sums, slice-major, ld = N (splits > 1)
    int64_t lda, ldb, ldc;
    int M, N, K;
    int tiles_m, tiles_n;
    int splits;       // number of K slices
    int k_per_split;  // K extent of a slice, a multiple of the k-tile
    int group_m;      // tile rows per raster group (L2 reuse of B columns)
};

// Element-type policy.
template <bool BF16>
struct Op;

template <>
struct Op<false> {               // fp32 inputs
    using In = float;
    static constexpr int BK = 32;   // k extent of one tile
    static constexpr int VEC = 4;   // elements per 16-byte chunk
};

template <>
struct Op<true> {                // bf16 inputs (raw 16-bit patterns)
    using In = uint16_t;
    static constexpr int BK = 64;
    static constexpr int VEC = 8;
};

// Tile geometry and LDS layout for one configuration.
template <bool BF16, int BM_, int BN_, int WM_, int WN_>
struct Geo {
    using O = Op<BF16>;
    using In = typename O::In;
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int BK = O::BK, VEC = O::VEC;
    static constexpr int NT = 64 * WM * WN;          // threads per workgroup
    static constexpr int WTM = BM / WM, WTN = BN / WN; // wave sub-block
    static constexpr int FM = WTM / 32, FN = WTN / 32; // 32x32 fragments per wave
    static constexpr int KH = BK / 2;                 // k values per lane half and tile
    static constexpr int STEPS = 4;                   // fragment steps per tile
    static constexpr int KS = KH / STEPS;             // k values per lane and step (4 or 8)
    static_assert(KS * (int)sizeof(In) == 16, "one step is one 16-byte read per lane");

    // A tile: BM rows of BK elements = 8 chunks of 16 bytes, padded to 144 bytes
    // so that 16 consecutive rows read at the same column land on distinct banks.
    static constexpr int A_ROW_BYTES = BK * (int)sizeof(In) + 16;
    static constexpr int A_BYTES = BM * A_ROW_BYTES;
    static constexpr int A_CHUNKS = BM * 8;
    static_assert(A_CHUNKS % NT == 0, "A chunks must divide evenly over the threads");
    static constexpr int A_PER_THREAD = A_CHUNKS / NT;

    // B tile, fp32: BK rows of BN floats, row-major; the 32-float halves of a
    // row swap places in rows 16..31 so the two lane halves of a fragment read
    // (rows k and k+16, same columns) hit different banks.
    // B tile, bf16: stored transposed, BN rows of BK k-values (same padded
    // layout as A), filled from 8x8 blocks transposed in registers.
    static constexpr int B_ROW_BYTES = BF16 ? A_ROW_BYTES : BN * 4;
    static constexpr int B_BYTES = BF16 ? BN * A_ROW_BYTES : BK * BN * 4;
    static constexpr int B_UNITS = BF16 ? (BK / 8) * (BN / 8) : BK * BN / 4;  // 8x8 blocks or chunks
    static constexpr int B_PER_THREAD = (B_UNITS + NT - 1) / NT;
    static_assert(B_UNITS % 64 == 0, "B units must fill whole waves");
    static_assert(BF16 || BN % 64 == 0, "fp32 B swizzle needs BN a multiple of 64");
    static_assert(BF16 || B_UNITS % NT == 0, "fp32 B chunks must divide evenly over the threads");

    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int SMEM_BYTES = 2 * STAGE_BYTES;
    static_assert(SMEM_BYTES <= 160 * 1024, "LDS budget of one workgroup exceeded");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave sub-block must be whole fragments");
};

// ------------------------------------------------------------ small helpers --

__device__ __forceinline__ u32x4 load16(const void *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ void lds_store16(unsigned char *smem, int off, u32x4 v)
{
    *reinterpret_cast<u32x4 *>(smem + off) = v;
}

__device__ __forceinline__ u32x4 lds_load16(const unsigned char *smem, int off)
{
    return *reinterpret_cast<const u32x4 *>(smem + off);
}

__device__ __forceinline__ float lds_loadf(const unsigned char *smem, int off)
{
    return *reinterpret_cast<const float *>(smem + off);
}

// Masked 16-byte chunk: elements [k, k+VEC) of one row, zero where the row is
// outside the matrix (row_ok false) or k+e >= kend.  Never dereferences an
// address outside the matrix.
template <typename In, int VEC, bool ALIGNED>
__device__ __forceinline__ u32x4 load_chunk_masked(const In *row, bool row_ok, int k, int kend)
{
    if (ALIGNED && row_ok && k + VEC <= kend) return load16(row + k);
    union {
        u32x4 v;
        In e[VEC];
    } u;
#pragma unroll
    for (int e = 0; e < VEC; ++e) u.e[e] = (row_ok && k + e < kend) ? row[k + e] : In(0);
    return u.v;
}

// Transpose an 8x8 block of 16-bit values held as 8 rows of 16 bytes:
// out[c] holds column c, i.e. (in[0][c], in[1][c], ..., in[7][c]).
__device__ __forceinline__ void transpose8x8_b16(const u32x4 in[8], u32x4 out[8])
{
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int d = c >> 1;         // dword holding column c in each row
        const int hi = (c & 1) * 16;  // which half of that dword
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const unsigned lo_row = (in[2 * q][d] >> hi) & 0xFFFFu;
            const unsigned hi_row = (in[2 * q + 1][d] >> hi) & 0xFFFFu;
            out[c][q] = lo_row | (hi_row << 16);
        }
    }
}

// Map a linear block id to (slice, tile row, tile column).
//
// The hardware hands consecutive workgroups to the 8 XCDs in turn, and each
// XCD has its own L2.  Renumbering so that consecutive logical ids run on one
// XCD, then rastering tiles in groups of group_m tile rows, makes the blocks
// resident on an XCD at one time share rows of A and columns of B in its L2.
__device__ __forceinline__ void block_coords(const KernelArgs &p, int &slice, int &tm, int &tn)
{
    const int nblk = (int)gridDim.x;
    int bid = (int)blockIdx.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
    const int tiles = p.tiles_m * p.tiles_n;
    slice = bid / tiles;
    const int t = bid - slice * tiles;
    const int per_group = p.group_m * p.tiles_n;
    const int group = t / per_group;
    const int first_m = group * p.group_m;
    const int gsize = min(p.tiles_m - first_m, p.group_m);
    const int in_group = t - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

// ------------------------------------------------------------------ kernel --

template <bool BF16, int BM, int BN, int WM, int WN, bool ALIGNED>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_kernel(KernelArgs p)
{
    using G = Geo<BF16, BM, BN, WM, WN>;
    using In = typename G::In;
    constexpr int BK = G::BK, VEC = G::VEC, NT = G::NT;
    constexpr int FM = G::FM, FN = G::FN, KS = G::KS;

    __shared__ __attribute__((aligned(16))) unsigned char smem[G::SMEM_BYTES];

    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wrow = wave / WN, wcol = wave % WN;
    const int half = lane >> 5;   // which k half this lane feeds
    const int l32 = lane & 31;    // row (A) or column (B) within a fragment

    int slice, tm, tn;
    block_coords(p, slice, tm, tn);
    const int bm = tm * BM, bn = tn * BN;
    const int kbeg = slice * p.k_per_split;
    const int kend = min(p.K, kbeg + p.k_per_split);
    const int ntiles = (kend - kbeg + BK - 1) / BK;

    const In *__restrict__ A = static_cast<const In *>(p.A);
    const In *__restrict__ B = static_cast<const In *>(p.B);
    const bool edge = !ALIGNED || bm + BM > p.M || bn + BN > p.N;

    // ---- per-thread global offsets (fixed across tiles; k0 is added per tile)
    // A: chunk u covers row (tid/8 + u*NT/8), columns (tid%8)*VEC .. +VEC
    int a_row[G::A_PER_THREAD];
    const int a_col = (tid & 7) * VEC;
#pragma unroll
    for (int u = 0; u < G::A_PER_THREAD; ++u) a_row[u] = (tid >> 3) + u * (NT / 8);

    // ---- registers holding the next tile between its global load and LDS store
    u32x4 ga[G::A_PER_THREAD];
    u32x4 gb[BF16 ? 8 * G::B_PER_THREAD : G::B_PER_THREAD];

    auto global_load = [&](int k0) {
        const bool full = !edge && k0 + BK <= kend;
#pragma unroll
        for (int u = 0; u < G::A_PER_THREAD; ++u) {
            const int gi = bm + a_row[u];
            const In *row = A + (int64_t)gi * p.lda;
            if (full)
                ga[u] = load16(row + k0 + a_col);
            else
                ga[u] = load_chunk_masked<In, VEC, ALIGNED>(row, gi < p.M, k0 + a_col, kend);
        }
        if constexpr (BF16) {
            // 8x8 blocks: block b covers k rows (b%8)*8..+8, n columns (b/8)*8..+8
#pragma unroll
            for (int u = 0; u < G::B_PER_THREAD; ++u) {
                const int b = tid + u * NT;
                if (G::B_UNITS % NT == 0 || b < G::B_UNITS) {
                    const int kr = (b & 7) * 8;
                    const int gn = bn + (b >> 3) * 8;
#pragma unroll
                    for (int rr = 0; rr < 8; ++rr) {
                        const int gk = k0 + kr + rr;
                        const In *row = B + (int64_t)gk * p.ldb;
                        if (full)
                            gb[u * 8 + rr] = load16(row + gn);
                        else
                            gb[u * 8 + rr] = load_chunk_masked<In, VEC, ALIGNED>(
                                row, gk < kend, gn, p.N);
                    }
                }
            }
        } else {
            // chunks: chunk c covers k row c/(BN/4), columns (c%(BN/4))*4 .. +4
#pragma unroll
            for (int u = 0; u < G::B_PER_THREAD; ++u) {
                const int c = tid + u * NT;
                const int kr = c / (BN / 4);
                const int gn = bn + (c % (BN / 4)) * 4;
                const int gk = k0 + kr;
                const In *row = B + (int64_t)gk * p.ldb;
                if (full)
                    gb[u] = load16(row + gn);
                else
                    gb[u] = load_chunk_masked<In, VEC, ALIGNED>(row, gk < kend, gn, p.N);
            }
        }
    };

    auto lds_store = [&](int stage) {
        unsigned char *sa = smem + stage * G::STAGE_BYTES;
        unsigned char *sb = sa + G::A_BYTES;
#pragma unroll
        for (int u = 0; u < G::A_PER_THREAD; ++u)
            lds_store16(sa, a_row[u] * G::A_ROW_BYTES + a_col * (int)sizeof(In), ga[u]);
        if constexpr (BF16) {
#pragma unroll
            for (int u = 0; u < G::B_PER_THREAD; ++u) {
                const int b = tid + u * NT;
                if (G::B_UNITS % NT == 0 || b < G::B_UNITS) {
                    u32x4 t[8];
                    transpose8x8_b16(&gb[u * 8], t);
                    const int kr = (b & 7) * 8;
                    const int n0 = (b >> 3) * 8;
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        lds_store16(sb, (n0 + c) * G::B_ROW_BYTES + kr * 2, t[c]);
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < G::B_PER_THREAD; ++u) {
                const int c = tid + u * NT;
                const int kr = c / (BN / 4);
                const int n = ((c % (BN / 4)) * 4) ^ (((kr >> 4) & 1) * 32);
                lds_store16(sb, kr * G::B_ROW_BYTES + n * 4, gb[u]);
            }
        }
    };

    // ---- fragments of one step: A as 16 bytes per fragment row, B likewise
    // (bf16) or as KS single floats (fp32).
    struct Frags {
        u32x4 a[FM];
        u32x4 b[FN];   // fp32: the KS floats of one column; bf16: 8 k values
    };

    auto load_frags = [&](int stage, int step, Frags &f) {
        const unsigned char *sa = smem + stage * G::STAGE_BYTES;
        const unsigned char *sb = sa + G::A_BYTES;
        const int kk = half * G::KH + step * KS;  // first k of this lane's slot range
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int row = wrow * G::WTM + fm * 32 + l32;
            f.a[fm] = lds_load16(sa, row * G::A_ROW_BYTES + kk * (int)sizeof(In));
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int col = wcol * G::WTN + fn * 32 + l32;
            if constexpr (BF16) {
                f.b[fn] = lds_load16(sb, col * G::B_ROW_BYTES + kk * 2);
            } else {
                const int n = col ^ (half * 32);  // rows kk.. have bit 4 == half
#pragma unroll
                for (int e = 0; e < KS; ++e)
                    f.b[fn][e] = __float_as_uint(lds_loadf(sb, (kk + e) * G::B_ROW_BYTES + n * 4));
            }
        }
    };

    floatx16 acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[fm][fn][r] = 0.0f;

    auto mma = [&](const Frags &f) {
        if constexpr (BF16) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, f.a[fm]), __builtin_bit_cast(bf16x8, f.b[fn]),
                        acc[fm][fn], 0, 0, 0);
        } else {
#pragma unroll
            for (int e = 0; e < KS; ++e)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
                        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            __uint_as_float(f.a[fm][e]), __uint_as_float(f.b[fn][e]),
                            acc[fm][fn], 0, 0, 0);
        }
    };

    // ---- prologue: tile 0 into stage 0
    global_load(kbeg);
    lds_store(0);
    __syncthreads();
    Frags cur, nxt;
    load_frags(0, 0, cur);

    // ---- main loop: one barrier per tile.  Stage s = t&1 is read while the
    // other stage receives tile t+1; fragments of step j+1 are read before the
    // products of step j are issued, and the first fragments of tile t+1 are
    // read right after the barrier, under the last products of tile t.
    for (int t = 0; t < ntiles; ++t) {
        const int stage = t & 1;
        const bool more = t + 1 < ntiles;
        if (more) global_load(kbeg + (t + 1) * BK);
#pragma unroll
        for (int step = 0; step < G::STEPS - 1; ++step) {
            load_frags(stage, step + 1, nxt);
            mma(cur);
            cur = nxt;
        }
        if (more) lds_store(stage ^ 1);
        __syncthreads();
        if (more) load_frags(stage ^ 1, 0, nxt);
        mma(cur);
        cur = nxt;
    }

    // ---- epilogue: accumulator element r of a 32x32 fragment sits at row
    // 8*(r/4) + 4*half + r%4 and column l32 of that fragment.
    float *out;
    int64_t ldo;
    if (p.splits > 1) {
        out = p.ws + (int64_t)slice * p.M * p.N;
        ldo = p.N;
    } else {
        out = p.C;
        ldo = p.ldc;
    }
    const bool store_edge = bm + BM > p.M || bn + BN > p.N;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int gj = bn + wcol * G::WTN + fn * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gi = bm + wrow * G::WTM + fm * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (!store_edge || (gi < p.M && gj < p.N)) out[(int64_t)gi * ldo + gj] = acc[fm][fn][r];
            }
        }
    }
}

}  // namespace dg
