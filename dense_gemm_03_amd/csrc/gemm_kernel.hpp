// Device code of the dense GEMM on gfx950 matrix cores:
//
//     C := alpha * op(A) * op(B) + beta * C,   op(X) = X or X^T
//
// the generalised product of "Learning to develop for GPUs through the GEMM
// operation", section "Generalized matrix multiplication GEMM"; the plain
// product C = A.B of its section "Matrix product" is alpha = 1, beta = 0 and
// no transposes.  One kernel template serves both input types:
//   fp32 inputs  -> v_mfma_f32_32x32x2_f32    (fp32 products, fp32 accumulate)
//   bf16 inputs  -> v_mfma_f32_32x32x16_bf16  (exact products, fp32 accumulate)
// and writes C as fp32 or as bf16 (rounded to nearest, ties to even).
//
// Structure (the tiling of the GEMM page, sections "Making the GPU
// implementation better" through "How to do even better", rebuilt for CDNA4
// wave64 matrix cores):
//   * each workgroup owns a BM x BN block of C and walks K in tiles of BK;
//   * tiles of op(A) (BM x BK) and op(B) (BK x BN) stream from HBM into a ring
//     of LDS stages with direct global->LDS 16-byte loads, several tiles ahead
//     of the products, one barrier per tile;
//   * LDS rows are XOR-swizzled so the fragment reads of a wave spread over
//     all 64 banks ("How to do even better": shifting rows across banks
//     removes the conflicts);
//   * each wave owns a (BM/WM) x (BN/WN) sub-block held as 32x32 accumulator
//     fragments in registers and reuses every A and B fragment it reads across
//     that sub-block (the register blocking of "Improving the solution and
//     balancing memory work");
//   * blocks that cross the M or N edge, the partial last k-tile and
//     unaligned operands take a masked path that loads zeros outside the
//     matrix (through registers) and stores only inside it; the choice is
//     uniform over the workgroup.
//
// Operand tiles.  Both operands are described by one template (OpTile): a
// tile of OUTER (m for A, n for B) by BK elements, stored in memory either
// k-contiguous (KMAJOR: A as given, or B given transposed as N x K) or
// outer-contiguous (MNMAJOR: B as given, or A given transposed as K x M).
// LDS keeps the memory orientation, so the global->LDS copy is a plain
// 16-byte copy either way; the fragment read adapts: a KMAJOR fragment is one
// 16-byte LDS read per lane, an MNMAJOR one is 4 single-float reads (fp32) or
// two LDS transpose reads (bf16).
//
// k-slot assignment.  A 32x32 MFMA pairs, in each of its k slots, the A value a
// lane supplies with the B value the same-numbered lane half supplies.  Lanes
// 0-31 feed one slot group and lanes 32-63 the other.  Within one tile, lane
// half h takes the contiguous k range [h*BK/2, (h+1)*BK/2) of both operands,
// so every product op(A)[i][k]*op(B)[k][j] of the definition is formed
// exactly once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace dg {

// f(std::integral_constant<int, I>) for I = B .. E-1, expanded at compile
// time: loops over accumulator fragments whose bodies are too large for the
// unroller would otherwise index the accumulators dynamically (and move them
// to scratch memory).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>());
        static_for<B + 1, E>(f);
    }
}

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Memory orientation of an operand tile.
enum Layout { KMAJOR = 0, MNMAJOR = 1 };

// Where op(B) comes from: a matrix in memory, or tiles of a convolution
// matrix formed from an image inside the loader (implicit GEMM).
enum BSource {
    B_MATRIX = 0,
    B_CONV_FWD = 1,    // op(B) = cols (C_in R S x P Q): B points at the image
    B_CONV_WGRAD = 2,  // op(B) = cols^T (P Q x C_in R S), read as the k-contiguous
                       // B^T tile (rows C_in R S, columns P Q)
    // The same two sources with the per-k terms looked up in a table made
    // before the launch (ConvGeom::tab) instead of computed in the loader.
    B_CONV_FWD_TAB = 3,
    B_CONV_WGRAD_TAB = 4,
    // Volume (3-D) forms of the first two, analytic terms: image [C_in][D][H][W],
    // taps (ci, t, r, s), output positions (o, p, q).
    B_CONV3_FWD = 5,
    B_CONV3_WGRAD = 6,
    // The analytic 2-D and volume forms reading a zero-padded copy of the
    // image: every position a tile touches lies inside it, so the loader
    // makes no range checks (the geometry describes the padded image, with
    // no padding).
    B_CONV_FWD_PAD = 7,
    B_CONV_WGRAD_PAD = 8,
    B_CONV3_FWD_PAD = 9,
    B_CONV3_WGRAD_PAD = 10,
    // forward product, 2-D, unit horizontal stride and dilation: B fragments
    // read from a window of the zero-bordered image held in LDS (see
    // ConvWindow); A is the filters with each filter row padded to S' taps
    B_CONV_FWD_WIN = 11,
    // filter gradient, 2-D, unit horizontal stride and dilation: the same
    // windows, with A the output gradient with rows padded to Q' positions
    // and C the gradient of the filters with rows padded to S' taps
    B_CONV_WGRAD_WIN = 12,
    // Four spatial dimensions: the volume sources with one more, outermost
    // dimension u -- image [C_in][U][D][H][W], taps (ci, ku, t, r, s), output
    // positions (ou, o, p, q) -- analytic terms, on the image or on its
    // zero-padded copy.
    B_CONV4_FWD = 13,
    B_CONV4_WGRAD = 14,
    B_CONV4_FWD_PAD = 15,
    B_CONV4_WGRAD_PAD = 16,
};

__host__ __device__ constexpr bool conv_fwd_source(int b)
{
    return b == B_CONV_FWD || b == B_CONV_FWD_TAB || b == B_CONV3_FWD || b == B_CONV_FWD_PAD ||
           b == B_CONV3_FWD_PAD || b == B_CONV_FWD_WIN || b == B_CONV4_FWD || b == B_CONV4_FWD_PAD;
}
__host__ __device__ constexpr bool conv_table_source(int b) { return b == B_CONV_FWD_TAB || b == B_CONV_WGRAD_TAB; }
__host__ __device__ constexpr bool conv_4d_source(int b) { return b >= B_CONV4_FWD && b <= B_CONV4_WGRAD_PAD; }
__host__ __device__ constexpr bool conv_volume_source(int b)
{
    return b == B_CONV3_FWD || b == B_CONV3_WGRAD || b == B_CONV3_FWD_PAD || b == B_CONV3_WGRAD_PAD ||
           conv_4d_source(b);
}
__host__ __device__ constexpr bool conv_padded_source(int b)
{
    return (b >= B_CONV_FWD_PAD && b <= B_CONV3_WGRAD_PAD) || b == B_CONV4_FWD_PAD ||
           b == B_CONV4_WGRAD_PAD;
}

// Geometry of the convolution behind an implicit op(B), for one image
// [C_in][H][W]: matrix row (ci R + r) S + s, column p Q + q holds
// image[ci][p sh - ph + r dh][q sw - pw + s dw], zero outside the image.
// Volume sources add a leading dimension: image [C_in][D][H][W], row
// ((ci T + t) R + r) S + s, column (o P + p) Q + q, depth o sz - pz + t lz.
struct ConvGeom {
    int h, w, r, s, ph, pw, sh, sw, dh, dw, q, pq, crs;
    uint64_t q_magic, rs_magic, s_magic;  // j / Q, k / (R S), k / S (exact below 2^31)
    int q_shift, rs_shift, s_shift;
    int img_bytes;                        // C_in (D) H W element bytes (< 2^31)
    // volume sources only
    int d, t, pz, sz, lz, p;              // depth, filter depth, its padding, stride, dilation; P
    uint64_t trs_magic, pq_magic;         // k / (T R S), j / (P Q)
    int trs_shift, pq_shift;
    // four-dimensional sources only: the outermost dimension's size, filter
    // size, padding, stride and dilation, O P Q (positions per outermost
    // output index), and k / (KU T R S), j / (O P Q)
    int du, ku, pu, su, lu, opq;
    uint64_t ktrs_magic, opq_magic;
    int ktrs_shift, opq_shift;
    // Window source only (all on the zero-bordered image: h, w are its padded
    // sizes): sp = S' taps per filter row (S rounded up to a 16-byte slot and
    // dividing BK; s >= S are zero filter taps), cr = C_in R filter rows, nr
    // output rows per window, and the divisions they need.
    int sp, cr, nr;
    uint64_t sp_magic, r_magic, w_magic;  // k / S', filter row / R, slot / W'
    int sp_shift, r_shift, w_shift;
    // filter-gradient window: output rows padded to qp = Q' positions (a
    // multiple of BK), k / Q'
    int qp;
    uint64_t qp_magic;
    int qp_shift;
    // Table sources only: the terms that change along K, one entry per k --
    // per tap (ci, r, s) for the forward product, per output position (p, q)
    // for the filter gradient: {y | x << 16 (signed 16-bit each), byte offset}.
    const int2 *tab;
};

// Arguments of one launch.  The grid is 1-D: splits * tiles_m * tiles_n blocks.
struct KernelArgs {
    const void *A;    // op(A) = A (M x K, k-contiguous) or A^T (A stored K x M)
    const void *B;    // op(B) = B (K x N, n-contiguous) or B^T (B stored N x K)
    void *C;          // final output (splits == 1): fp32, or bf16 when out_bf16
    float *ws;        // split-K partial sums, slice-major, ld = N (splits > 1)
    int64_t lda, ldb, ldc;
    int M, N, K;
    // outer extents the loads may read (>= M, N): for an operand stored with
    // M or N along its rows, up to its row width when its rows are padded
    // (the values there feed only outputs that are not stored); M and N for
    // the others
    int m_load, n_load;
    int tiles_m, tiles_n;
    int splits;       // number of K slices
    int k_per_split;  // K extent of a slice, a multiple of the k-tile
    int group_m;      // tile rows per raster group (L2 reuse of B columns)
    int direct_ok;    // per-thread byte offsets of a tile fit in 32 bits
    float alpha, beta;
    int out_bf16;     // C holds bf16 bit patterns (1) or fp32 (0)
    ConvGeom conv;    // used by the implicit (convolution) B sources only
};

// ----------------------------------------------------------- operand tile --

// One operand tile in LDS: OUTER x BK elements of op(A) (OUTER = BM) or of
// op(B) (OUTER = BN).
//
// LDS banks (measured on gfx950 with the bank-conflict counter): 64 banks of
// 4 bytes, and a 16-byte read serves 16 lanes per pass, so the 16 addresses of
// a pass must cover 256 bytes that fall on distinct banks.
//
//   KMAJOR:  OUTER rows of BK elements (64 to 1024 bytes).  Chunk c of row r
//            sits in slot c ^ ((r / RPL) % CPR), RPL rows sharing a 256-byte
//            bank line (RPL = 1 for longer rows): the 16 rows a 16-lane pass
//            reads at one chunk cover all 64 banks once, and so do the writes.
//   MNMAJOR: BK rows of OUTER elements, row-major as in memory.
//     fp32:  the two 32-float halves of each 64-float group swap places in
//            rows with bit 4 set, so the two lane halves of a fragment read
//            (rows k and k+16, same columns) use different banks.
//     bf16:  read with the LDS transpose load, 4 rows x 16 columns per 16
//            lanes; the 64-byte segments of row k are XOR-permuted by (k & 3)
//            so those 4 rows land on 4 different bank quarters.
template <bool BF16_, int OUTER_, int BK_, int LAYOUT_, int NT_, int NW_>
struct OpTile {
    static constexpr bool BF16 = BF16_;
    using In = typename std::conditional<BF16, uint16_t, float>::type;
    static constexpr int OUTER = OUTER_, BK = BK_, LAYOUT = LAYOUT_, NT = NT_, NW = NW_;
    static constexpr int ES = (int)sizeof(In);
    static constexpr int VEC = 16 / ES;                   // elements per 16-byte chunk
    static constexpr int ROWS = LAYOUT == KMAJOR ? OUTER : BK;
    static constexpr int ROW_BYTES = (LAYOUT == KMAJOR ? BK : OUTER) * ES;
    static constexpr int BYTES = ROWS * ROW_BYTES;
    static constexpr int CPR = ROW_BYTES / 16;            // 16-byte chunks per row
    static constexpr int CHUNKS = ROWS * CPR;
    static_assert(CHUNKS % NT == 0, "tile chunks must divide evenly over the threads");
    static constexpr int PER_THREAD = CHUNKS / NT;
    // Direct global->LDS loads write 64 lanes x 16 bytes = 1 KiB contiguous
    // LDS bytes per instruction; the tile is cut into such pieces.
    static constexpr int PIECES = BYTES / 1024;
    static_assert(PIECES % NW == 0, "direct loads must divide over the waves");
    static_assert(ROW_BYTES <= 1024 && 1024 % ROW_BYTES == 0, "rows must tile a 1 KiB piece");
    static constexpr int ROWS_PER_PIECE = 1024 / ROW_BYTES;
    // KMAJOR rows per 256-byte bank line (1 for rows of 256 bytes or more)
    static constexpr int RPL = ROW_BYTES >= 256 ? 1 : 256 / ROW_BYTES;
    static_assert(LAYOUT != KMAJOR || ROW_BYTES >= 256 || CPR * RPL == 16,
                  "k-contiguous rows of 64 bytes or more");
    static constexpr int SEGMASK = (OUTER / 32 >= 4) ? 3 : (OUTER / 32 - 1);
    static_assert(LAYOUT != MNMAJOR || BF16 || (OUTER % 64 == 0 && BK == 32),
                  "fp32 outer-contiguous tiles: OUTER % 64 == 0, BK == 32");
    static_assert(LAYOUT != MNMAJOR || !BF16 || (OUTER % 32 == 0 && (OUTER & (OUTER - 1)) == 0),
                  "bf16 outer-contiguous tiles: a power-of-two count of 32-column segments");

    // Byte offset of element `e` of LDS row `row` (e a multiple of 4 for the
    // bf16 MNMAJOR transpose reads, of VEC for KMAJOR).
    static __device__ __forceinline__ int off(int row, int e)
    {
        if constexpr (LAYOUT == KMAJOR)
            return row * ROW_BYTES + (((e / VEC) ^ ((row / RPL) % CPR)) << 4);
        else if constexpr (BF16)
            return row * ROW_BYTES + (((e >> 5) ^ (row & SEGMASK)) << 6) + ((e & 31) << 1);
        else
            return row * ROW_BYTES + ((e ^ (((row >> 4) & 1) << 5)) << 2);
    }

    // Logical element held at the 16-byte-aligned physical element position
    // `phys` of LDS row `row`: the inverse of off(), which is the same XOR.
    static __device__ __forceinline__ int logical(int row, int phys)
    {
        if constexpr (LAYOUT == KMAJOR)
            return ((phys / VEC) ^ ((row / RPL) % CPR)) * VEC;
        else if constexpr (BF16)
            return (((phys >> 5) ^ (row & SEGMASK)) << 5) | (phys & 31);
        else
            return phys ^ (((row >> 4) & 1) << 5);
    }

    // The same for any physical element position (the swizzles move whole
    // 16-byte chunks, or for fp32 outer-contiguous tiles flip bit 5 of the
    // element, so an element keeps its place inside its chunk).
    static __device__ __forceinline__ int logical_elem(int row, int phys)
    {
        if constexpr (LAYOUT == KMAJOR)
            return logical(row, phys - phys % VEC) + phys % VEC;
        else
            return logical(row, phys);
    }

    // LDS reads per fragment and step.
    static constexpr int READS = LAYOUT == KMAJOR ? 1 : (BF16 ? 2 : VEC);
};

// Tile geometry of one configuration.
template <bool BF16_, int BM_, int BN_, int BK_, int WM_, int WN_, int STAGES_, int LA_, int LB_>
struct Geo {
    static constexpr bool BF16 = BF16_;
    using In = typename std::conditional<BF16, uint16_t, float>::type;
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int STAGES = STAGES_, LA = LA_, LB = LB_;
    static constexpr int ES = (int)sizeof(In);         // element bytes
    static constexpr int VEC = 16 / ES;                // elements per 16-byte chunk
    static constexpr int NW = WM * WN;                 // waves
    static constexpr int NT = 64 * NW;                 // threads per workgroup
    static constexpr int WTM = BM / WM, WTN = BN / WN; // wave sub-block
    static constexpr int FM = WTM / 32, FN = WTN / 32; // 32x32 fragments per wave
    static constexpr int KH = BK / 2;                  // k values per lane half and tile
    static constexpr int KS = VEC;                     // k values per lane and step
    static constexpr int STEPS = KH / KS;              // fragment steps per tile
    static_assert(KH % KS == 0 && STEPS >= 2, "a tile needs at least two fragment steps");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave sub-block must be whole fragments");

    using TA = OpTile<BF16, BM, BK, LA, NT, NW>;
    using TB = OpTile<BF16, BN, BK, LB, NT, NW>;
    static constexpr int A_BYTES = TA::BYTES;
    static constexpr int STAGE_BYTES = TA::BYTES + TB::BYTES;

    // MFMAs and LDS fragment reads per step and wave; direct loads per tile
    // and wave.
    static constexpr int N_MMA = BF16 ? FM * FN : KS * FM * FN;
    static constexpr int N_DS = FM * TA::READS + FN * TB::READS;
    // Interleave hints for the main loop (interleave_step), bf16 only: with
    // the compiler's own order bf16 8192^3 ran 1.5-2% slower, while the fp32
    // blocks ran as fast or faster (alternating runs: 4096^3 -0.9%,
    // 4097 x 4095 x 4099 -1.7%, 2048^3 -1.7%, 1000^3 -3%, the tall and
    // im2col shapes within noise).
    static constexpr bool HINTS = BF16;
    static constexpr int LOADS_PER_TILE = (TA::PIECES + TB::PIECES) / NW;

    // Direct loads of 4 bytes per lane (256 B per instruction), range-checked
    // buffer loads, for rows at any 4-byte alignment and for blocks crossing
    // the M or N edge: a lane's dword is one fp32 element or two consecutive
    // bf16 elements (the kernel takes this form for bf16 only when every row
    // starts 4-byte aligned and no pair straddles an edge).  The entry must
    // split its tiles into whole 256-byte pieces per wave, keep k-contiguous
    // rows within one 256-byte bank line (so a piece's rows share one swizzle
    // key), and count its loads in flight within vmcnt's range.
    static constexpr int LOADS4_PER_TILE = (TA::BYTES / 256 + TB::BYTES / 256) / NW;
    static constexpr bool DMA4 =
        (TA::BYTES / 256) % NW == 0 && (TB::BYTES / 256) % NW == 0 &&
        (LA == MNMAJOR || TA::ROW_BYTES <= 256) && (LB == MNMAJOR || TB::ROW_BYTES <= 256) &&
        LOADS4_PER_TILE * (STAGES - 2) <= 63;

    static_assert(STAGES >= 2 && STAGES <= 4, "2 to 4 LDS stages");
    static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "LDS budget of one workgroup exceeded");
    static_assert(LOADS_PER_TILE * (STAGES - 2) <= 63, "vmcnt counts at most 63 loads");
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

// LDS transpose load (gfx950): within each group of 16 lanes, lane s names
// row s/4, columns 4*(s%4)..+3 of a 4 x 16 block of 16-bit values, and lane i
// receives column i of that block (its 4 rows).
__device__ __forceinline__ v4i16 lds_read_tr16(const unsigned char *smem, int off)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)((__attribute__((address_space(3))) unsigned char *)smem + off));
}

// One direct global->LDS load: each lane copies 16 bytes from base + voff
// (base uniform, voff a per-lane 32-bit byte offset), and the 64 lanes' bytes
// land contiguously at LDS byte address lds_addr + 16 * lane (measured on
// gfx950).  It is written as an instruction rather than the compiler builtin:
// the builtin makes every later LDS transpose read wait for all such loads
// in flight, which would undo the multi-stage pipeline.  The code that uses
// it waits for the loads itself (s_waitcnt vmcnt before each barrier).  M0
// carries the LDS address; nothing else in these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void direct_load16(const void *base, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(base)
                 : "m0");
}

// One range-checked direct load of 4 bytes per lane: lane l's dword at
// rsrc.base + voff lands at LDS byte address lds_addr + 4 * l; a lane whose
// offset is at or past the resource's size reads zero and touches no memory.
__device__ __forceinline__ void direct_load4(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                             uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rsrc)
                 : "m0");
}
#pragma clang diagnostic pop

// LDS byte address of a __shared__ location (the offset inside the
// workgroup's LDS allocation).
__device__ __forceinline__ uint32_t lds_addr(const unsigned char *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char *)p;
}

// s_waitcnt immediate that waits until at most `vm` vector-memory loads are
// outstanding and every LDS access has completed (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 left at its maximum, lgkmcnt 11:8 = 0).
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4); }

// Masked 16-byte chunk: elements [e0, e0+VEC) of one row, zero where the row
// is outside the matrix (row_ok false) or e0+e >= eend.  Element loads never
// touch an address outside the matrix.  A whole bf16 chunk of an unaligned
// row (2-byte aligned, as rows at an odd leading dimension are every other
// row) comes from the five 4-byte-aligned dwords that cover it, shifted
// into place: each of them holds at least one element of the chunk, so it
// lies on a page the matrix occupies, and its bytes outside the chunk are
// discarded.
template <typename In, int VEC, bool ALIGNED>
__device__ __forceinline__ u32x4 load_chunk_masked(const In *row, bool row_ok, int e0, int eend)
{
    if (ALIGNED && row_ok && e0 + VEC <= eend) return load16(row + e0);
    if constexpr (!ALIGNED && sizeof(In) == 2) {
        if (row_ok && e0 + VEC <= eend) {
            const unsigned char *s = reinterpret_cast<const unsigned char *>(row + e0);
            const uint32_t mis = (uint32_t)reinterpret_cast<uintptr_t>(s) & 2;
            const uint32_t *q = reinterpret_cast<const uint32_t *>(s - mis);
            const uint32_t sh = mis * 8;                 // 0 or 16 bits
            const uint32_t w0 = q[0], w1 = q[1], w2 = q[2], w3 = q[3];
            const uint32_t w4 = q[sh ? 4 : 3];           // past the chunk only when shifted
            u32x4 v;
            v[0] = __builtin_amdgcn_alignbit(w1, w0, sh);
            v[1] = __builtin_amdgcn_alignbit(w2, w1, sh);
            v[2] = __builtin_amdgcn_alignbit(w3, w2, sh);
            v[3] = __builtin_amdgcn_alignbit(w4, w3, sh);
            return v;
        }
    }
    union {
        u32x4 v;
        In e[VEC];
    } u;
#pragma unroll
    for (int e = 0; e < VEC; ++e) u.e[e] = (row_ok && e0 + e < eend) ? row[e0 + e] : In(0);
    return u.v;
}

// Two fp32 values -> bf16 bit patterns (lo in the low half), rounded to
// nearest with ties to even; a NaN stays a NaN with its sign and leading
// payload bits and the quiet bit set.  In integer terms: u -> (u + 0x7FFF +
// ((u >> 16) & 1)) >> 16 for numbers, u -> (u >> 16) | 0x40 for NaNs.  gfx950
// converts a pair in one instruction (v_cvt_pk_bf16_f32); on the GPU it gave
// exactly those integer results for 2^20 bit patterns (every upper half with
// 16 lower halves: ties, half-ulp neighbours, NaN payloads, denormals), and
// costs a sixth of the VALU work of the integer form.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{lo, hi}, bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    return (uint16_t)f32x2_to_bf16x2_rne(f, 0.0f);
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

// ---------------------------------------------------------- block context --

// Per-block state shared by the main-loop helpers.
template <class G>
struct BlockCtx {
    using In = typename G::In;
    const In *A;
    const In *B;
    int64_t lda, ldb;
    int M, N;     // outer extents the loads may read (KernelArgs::m_load, n_load)
    int bm, bn;   // block origin in C
    int kend;     // end of this block's K range
    int tid, lane, wrow, wcol;
    int rot;      // interior k-tile the block may start at (see main_loop_direct)
    int64_t a_end, b_end;  // bytes from A / B to just past their last element
};

// Fragments of one step: per 32-row A fragment 16 bytes (4 fp32 or 8 bf16 k
// values of the lane's row); per 32-column B fragment the same k values of
// the lane's column.
template <class G>
struct Frags {
    u32x4 a[G::FM];
    u32x4 b[G::FN];
};

// One operand fragment: the KS k values from kk of outer index ob + lane%32.
template <class T>
__device__ __forceinline__ u32x4 read_frag(const unsigned char *tile, int lane, int ob, int kk)
{
    if constexpr (T::LAYOUT == KMAJOR) {
        return lds_load16(tile, T::off(ob + (lane & 31), kk));
    } else if constexpr (T::BF16) {
        // two transpose loads: k = kk..kk+3 and kk+4..kk+7 of outer index
        // ob + lane%32
        const int s = lane & 15, g = (lane >> 4) & 1;
        const int col = ob + 16 * g + 4 * (s & 3);
        const int k = kk + (s >> 2);
        const v4i16 lo = lds_read_tr16(tile, T::off(k, col));
        const v4i16 hi = lds_read_tr16(tile, T::off(k + 4, col));
        return u32x4{(unsigned)(unsigned short)lo[0] | ((unsigned)(unsigned short)lo[1] << 16),
                     (unsigned)(unsigned short)lo[2] | ((unsigned)(unsigned short)lo[3] << 16),
                     (unsigned)(unsigned short)hi[0] | ((unsigned)(unsigned short)hi[1] << 16),
                     (unsigned)(unsigned short)hi[2] | ((unsigned)(unsigned short)hi[3] << 16)};
    } else {
        u32x4 v;
        const int col = ob + (lane & 31);
#pragma unroll
        for (int e = 0; e < T::VEC; ++e) v[e] = __float_as_uint(lds_loadf(tile, T::off(kk + e, col)));
        return v;
    }
}

// Fragments of step `step` of the tile in `stage`.  Lane half h (lanes
// 32h..32h+31) supplies k = h*BK/2 + step*KS .. +KS of the tile.
template <class G>
__device__ __forceinline__ void load_frags(const unsigned char *stage, const BlockCtx<G> &c,
                                           int step, Frags<G> &f)
{
    const unsigned char *sb = stage + G::A_BYTES;
    const int kk = (c.lane >> 5) * G::KH + step * G::KS;
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm)
        f.a[fm] = read_frag<typename G::TA>(stage, c.lane, c.wrow * G::WTM + fm * 32, kk);
#pragma unroll
    for (int fn = 0; fn < G::FN; ++fn)
        f.b[fn] = read_frag<typename G::TB>(sb, c.lane, c.wcol * G::WTN + fn * 32, kk);
}

template <class G>
__device__ __forceinline__ void mma(const Frags<G> &f, floatx16 (&acc)[G::FM][G::FN])
{
    if constexpr (G::BF16) {
#pragma unroll
        for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < G::FN; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, f.a[fm]), __builtin_bit_cast(bf16x8, f.b[fn]),
                    acc[fm][fn], 0, 0, 0);
    } else {
#pragma unroll
        for (int e = 0; e < G::KS; ++e)
#pragma unroll
            for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < G::FN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                        __uint_as_float(f.a[fm][e]), __uint_as_float(f.b[fn][e]), acc[fm][fn], 0,
                        0, 0);
    }
}

// Instruction interleave for one step: each MFMA is followed by up to one
// direct global->LDS load and one LDS fragment read, so the loads and reads
// issue while the matrix core is busy instead of in a burst after it.
template <int N_MMA, int N_DS, int N_VMEM>
__device__ __forceinline__ void interleave_step()
{
#pragma unroll
    for (int i = 0; i < N_MMA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA
        if (i < N_VMEM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
        if (i < N_DS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // DS read
    }
    if (N_DS > N_MMA) __builtin_amdgcn_sched_group_barrier(0x100, N_DS - N_MMA, 0);
    if (N_VMEM > N_MMA) __builtin_amdgcn_sched_group_barrier(0x020, N_VMEM - N_MMA, 0);
}

// -------------------------------------------------- interior (direct) path --

// Per-thread byte offsets of one operand's direct loads, relative to the tile
// origin, for loads of DW bytes per lane (16: one 1 KiB piece of the tile
// per instruction; 4: one 256-byte piece).  They do not change from one
// k-tile to the next, so they are computed once per block and the per-tile
// address is a uniform base plus a 32-bit offset.
template <class T, int DW>
struct TileOffsets {
    static constexpr int PIECE = 64 * DW;
    static constexpr int PER_WAVE = T::BYTES / PIECE / T::NW;
    uint32_t v[PER_WAVE];
};

// The LDS side of a direct load is fixed -- lane l at byte DW*l of the piece
// -- so each lane fetches the global element(s) that the tile's swizzle places
// at its LDS position.  LDS row r is memory row r of the tile (an outer index
// for KMAJOR, a k for MNMAJOR).
//
// 16-byte loads of a block at the M or N edge fetch in-bounds data for the
// positions past the edge: a KMAJOR row past the last outer index reads the
// last row, and an MNMAJOR chunk past the edge reads the last chunk (the
// caller takes this form only when that outer extent is a whole number of
// chunks, so no chunk straddles the edge).  Those LDS positions only feed
// outputs past the edge, which are never stored.  outer0 is the block's
// first outer index, n_outer the matrix's outer extent; for interior blocks
// the clamps change nothing.
template <class T, int DW>
__device__ __forceinline__ void tile_offsets(int wave, int lane, int64_t ld, int outer0,
                                             int n_outer, TileOffsets<T, DW> &o)
{
    using O = TileOffsets<T, DW>;
#pragma unroll
    for (int i = 0; i < O::PER_WAVE; ++i) {
        const int piece = wave + T::NW * i;
        const int byte = piece * O::PIECE + DW * lane;
        int row = byte / T::ROW_BYTES;
        int e = T::logical_elem(row, (byte % T::ROW_BYTES) / T::ES);
        if constexpr (DW == 16) {
            if constexpr (T::LAYOUT == KMAJOR)
                row = min(outer0 + row, n_outer - 1) - outer0;
            else
                e = min(outer0 + e, n_outer - T::VEC) - outer0;
        }
        o.v[i] = (uint32_t)(((int64_t)row * ld + e) * T::ES);
    }
}

template <class G, int DW>
struct DirectOffsets {
    TileOffsets<typename G::TA, DW> a;
    TileOffsets<typename G::TB, DW> b;
    static constexpr int LOADS_PER_TILE =
        TileOffsets<typename G::TA, DW>::PER_WAVE + TileOffsets<typename G::TB, DW>::PER_WAVE;
};

// Byte offset of the origin of one operand's k-tile from the matrix start:
// KMAJOR rows are outer indices (origin row outer0, column k0), MNMAJOR rows
// are k (origin row k0, column outer0).
template <class T>
__device__ __forceinline__ int64_t tile_origin_bytes(int64_t ld, int outer0, int k0)
{
    if constexpr (T::LAYOUT == KMAJOR)
        return ((int64_t)outer0 * ld + k0) * T::ES;
    else
        return ((int64_t)k0 * ld + outer0) * T::ES;
}

// Bytes from the start of a stored operand to just past its last element:
// the range a buffer load may touch.
template <class T>
__device__ __forceinline__ int64_t operand_end_bytes(int64_t ld, int n_outer, int K)
{
    if constexpr (T::LAYOUT == KMAJOR)
        return ((int64_t)(n_outer - 1) * ld + K) * T::ES;
    else
        return ((int64_t)(K - 1) * ld + n_outer) * T::ES;
}

// Range-checked buffer resource over one operand's k-tile: from the tile
// origin to the end of the matrix, capped at 4 GiB - 1 bytes (the tile's own
// offsets are below 2^32, so a cap never cuts into the tile).
template <class T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const typename T::In *X, int64_t ld,
                                                            int64_t end, int outer0, int k0)
{
    const int64_t org = tile_origin_bytes<T>(ld, outer0, k0);
    const int64_t left = end - org;
    const uint32_t size = (uint32_t)(left < 0xFFFFFFFFll ? left : 0xFFFFFFFFll);
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char *>(reinterpret_cast<const unsigned char *>(X) + org), 0, (int)size,
        0x00020000);  // gfx9 raw-buffer format word
}

// Direct copy of the k-tile at k0 into `stage`.  DW = 16: every address is
// inside the matrix and 16-byte aligned (interior blocks of aligned
// operands).  DW = 4: range-checked loads (one fp32 element or two bf16
// elements per lane); elements of rows or columns
// past the M or N edge read other in-bounds elements or zero, and only feed
// outputs that are never stored.
template <class G, int DW>
__device__ __forceinline__ void direct_tile_load(unsigned char *stage, const BlockCtx<G> &c,
                                                 const DirectOffsets<G, DW> &o, int k0)
{
    using TA = typename G::TA;
    using TB = typename G::TB;
    constexpr int NW = G::NW;
    constexpr int PIECE = 64 * DW;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(c.tid >> 6);
    const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_addr(stage)) + PIECE * wave;
    if constexpr (DW == 16) {
        const unsigned char *a_base =
            reinterpret_cast<const unsigned char *>(c.A) + tile_origin_bytes<TA>(c.lda, c.bm, k0);
        const unsigned char *b_base =
            reinterpret_cast<const unsigned char *>(c.B) + tile_origin_bytes<TB>(c.ldb, c.bn, k0);
#pragma unroll
        for (int i = 0; i < decltype(o.a)::PER_WAVE; ++i)
            direct_load16(a_base, o.a.v[i], lds + PIECE * NW * i);
#pragma unroll
        for (int i = 0; i < decltype(o.b)::PER_WAVE; ++i)
            direct_load16(b_base, o.b.v[i], lds + G::A_BYTES + PIECE * NW * i);
    } else {
        static_assert(DW == 4 && G::DMA4, "4-byte direct loads: entries with whole 256-byte pieces");
        const auto ra = tile_rsrc<TA>(c.A, c.lda, c.a_end, c.bm, k0);
        const auto rb = tile_rsrc<TB>(c.B, c.ldb, c.b_end, c.bn, k0);
#pragma unroll
        for (int i = 0; i < decltype(o.a)::PER_WAVE; ++i)
            direct_load4(ra, o.a.v[i], lds + PIECE * NW * i);
#pragma unroll
        for (int i = 0; i < decltype(o.b)::PER_WAVE; ++i)
            direct_load4(rb, o.b.v[i], lds + G::A_BYTES + PIECE * NW * i);
    }
}

// One interior k-tile: multiply the tile in `stage` while the tile at k_load
// streams into `load` (STAGES-1 tiles ahead).  The tile ends with a wait for
// the next tile's loads -- only those: the later tiles stay in flight -- and
// a barrier, after which the next tile's first fragments are read under the
// last products of this one.  (Past the last tile the caller passes an
// in-bounds k_load again, so the code has no branch.)
template <class G, int DW>
__device__ __forceinline__ void direct_tile(const unsigned char *stage, const unsigned char *next,
                                            unsigned char *load,
                                            const BlockCtx<G> &c, const DirectOffsets<G, DW> &o,
                                            int k_load, Frags<G> &cur,
                                            floatx16 (&acc)[G::FM][G::FN])
{
    constexpr int LOADS = DirectOffsets<G, DW>::LOADS_PER_TILE;
    Frags<G> nxt;
    direct_tile_load(load, c, o, k_load);
    load_frags(stage, c, 1, nxt);
    // The two waves of a SIMD keep the default priority: raising it around
    // the MFMA bursts measured 0.7-0.9% slower on the large products (fp32
    // 4096^3, bf16 8192^3, alternating runs).
    mma(cur, acc);
    if constexpr (G::HINTS) interleave_step<G::N_MMA, G::N_DS, LOADS>();
    cur = nxt;
#pragma unroll
    for (int step = 1; step < G::STEPS - 1; ++step) {
        load_frags(stage, c, step + 1, nxt);
        mma(cur, acc);
        if constexpr (G::HINTS) interleave_step<G::N_MMA, G::N_DS, 0>();
        cur = nxt;
    }
    // The next tile's loads were issued STAGES-2 tiles before the ones just
    // issued; every wave waits for its own share before the barrier, so after
    // it the whole tile is in LDS.  lgkmcnt(0): this tile's reads are done
    // before anyone may overwrite the stage.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(LOADS * (G::STAGES - 2)));
    __builtin_amdgcn_s_barrier();
    load_frags(next, c, 0, nxt);
    mma(cur, acc);
    if constexpr (G::HINTS) interleave_step<G::N_MMA, G::N_DS, 0>();
    cur = nxt;
}

// Interior k-tiles [0, ntiles) from k_first, STAGES tiles per loop iteration
// so that each stage is always the same array.  The block visits the tiles
// in rotated order, rot, rot+1, .., ntiles-1, 0, .., rot-1 (rot < ntiles):
// blocks that share a row of A or a column of B on one XCD start at
// different tiles, so one of them takes the L2 miss on each shared tile and
// the others, a tile later, hit, instead of all waiting on the same miss.  The stages are distinct
// __shared__ arrays passed as restrict pointers of this one function: the
// alias scopes this gives every LDS read and direct load let the compiler see
// that reading one stage need not wait for loads into the others.  On entry
// no wave may read or load any stage; on exit no load is in flight.
template <class G, int DW>
__device__ __forceinline__ void main_loop_direct(unsigned char *__restrict__ s0,
                                                 unsigned char *__restrict__ s1,
                                                 unsigned char *__restrict__ s2,
                                                 unsigned char *__restrict__ s3,
                                                 const BlockCtx<G> &c, int k_first, int ntiles,
                                                 floatx16 (&acc)[G::FM][G::FN])
{
    constexpr int S = G::STAGES, BK = G::BK;
    constexpr int LOADS = DirectOffsets<G, DW>::LOADS_PER_TILE;
    static_assert(LOADS * (S - 2) <= 63, "vmcnt counts at most 63 loads");
    unsigned char *const st[4] = {s0, s1, s2, s3};
    Frags<G> cur;
    DirectOffsets<G, DW> o;
    tile_offsets(c.tid >> 6, c.lane, c.lda, c.bm, c.M, o.a);
    tile_offsets(c.tid >> 6, c.lane, c.ldb, c.bn, c.N, o.b);
    // k of the next tile to load; past the last tile the loads wrap round to
    // tiles already done (never read, and in bounds), so the code has no branch
    // rotated start for bf16 blocks with 64-byte tile rows (measured: +3-6% on
    // large square products; fp32, which needs an eighth of the bytes per flop,
    // gains nothing, and the 64-deep bf16 blocks, which request whole 128-byte
    // lines, ran 0.8% faster without it at 8192^3), only on long K loops,
    // where the wrapped tiles are few
    int kt = G::BF16 && BK == 32 && ntiles >= 32 ? c.rot : 0;
    auto next_k = [&]() {
        const int k = k_first + kt * BK;
        kt = kt + 1 == ntiles ? 0 : kt + 1;
        return k;
    };
    // prologue: tiles 0 .. S-2 in flight, tile 0 complete
#pragma unroll
    for (int s = 0; s < S - 1; ++s) direct_tile_load(st[s], c, o, next_k());
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(LOADS * (S - 2)));
    __builtin_amdgcn_s_barrier();
    load_frags(st[0], c, 0, cur);

    for (int t = 0; t < ntiles; t += S) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            if (s == 0 || t + s < ntiles)
                direct_tile(st[s], st[(s + 1) % S], st[(s + S - 1) % S], c, o, next_k(), cur, acc);
        }
    }
    // drain the loads issued past the last tile before the stages are reused
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    __builtin_amdgcn_s_barrier();
}

// ------------------------------------------------------------ masked path --

// The operand tiles of one k-tile, between their global load and LDS store.
template <class G>
struct StageRegs {
    u32x4 a[G::TA::PER_THREAD];
    u32x4 b[G::TB::PER_THREAD];
};

// Global -> registers for one operand's k-tile at k0, zero outside the
// matrix.  Chunk u of a thread is ch = tid + u*NT: memory row ch/CPR of the
// tile, elements (ch%CPR)*VEC .. +VEC, so consecutive lanes read consecutive
// 16-byte chunks of a row (coalesced).  KMAJOR rows are outer indices (valid
// below n_outer) and k runs along the row (valid below kend); MNMAJOR rows
// are k and the outer index runs along the row.
template <bool ALIGNED, class T>
__device__ __forceinline__ void load_tile_masked(const typename T::In *X, int64_t ld, int outer0,
                                                 int n_outer, int k0, int kend, int tid,
                                                 u32x4 (&r)[T::PER_THREAD])
{
    using In = typename T::In;
#pragma unroll
    for (int u = 0; u < T::PER_THREAD; ++u) {
        const int ch = tid + u * T::NT;
        const int row = ch / T::CPR, e = (ch % T::CPR) * T::VEC;
        if constexpr (T::LAYOUT == KMAJOR) {
            const int go = outer0 + row;
            r[u] = load_chunk_masked<In, T::VEC, ALIGNED>(X + (int64_t)go * ld, go < n_outer,
                                                          k0 + e, kend);
        } else {
            const int gk = k0 + row;
            r[u] = load_chunk_masked<In, T::VEC, ALIGNED>(X + (int64_t)gk * ld, gk < kend,
                                                          outer0 + e, n_outer);
        }
    }
}

template <class T>
__device__ __forceinline__ void store_tile(unsigned char *tile, int tid,
                                           const u32x4 (&r)[T::PER_THREAD])
{
#pragma unroll
    for (int u = 0; u < T::PER_THREAD; ++u) {
        const int ch = tid + u * T::NT;
        lds_store16(tile, T::off(ch / T::CPR, (ch % T::CPR) * T::VEC), r[u]);
    }
}

template <bool ALIGNED, class G>
__device__ __forceinline__ void global_load_masked(const BlockCtx<G> &c, int k0, StageRegs<G> &r)
{
    load_tile_masked<ALIGNED, typename G::TA>(c.A, c.lda, c.bm, c.M, k0, c.kend, c.tid, r.a);
    load_tile_masked<ALIGNED, typename G::TB>(c.B, c.ldb, c.bn, c.N, k0, c.kend, c.tid, r.b);
}

template <class G>
__device__ __forceinline__ void lds_store(unsigned char *stage, int tid, const StageRegs<G> &r)
{
    store_tile<typename G::TA>(stage, tid, r.a);
    store_tile<typename G::TB>(stage + G::A_BYTES, tid, r.b);
}

// `ntiles` masked k-tiles from k_first, double buffered through registers
// (stage t&1 is read while stage (t+1)&1 receives tile t+1); `load(k0, regs)`
// fetches the tiles of the k-tile at k0.  On entry no wave may still use
// stages 0 and 1.
template <class G, class Loader>
__device__ __forceinline__ void main_loop_masked(unsigned char *smem0, unsigned char *smem1,
                                                 const BlockCtx<G> &c, int k_first, int ntiles,
                                                 floatx16 (&acc)[G::FM][G::FN], Loader &&load)
{
    StageRegs<G> regs;
    Frags<G> cur, nxt;
    load(k_first, regs);
    lds_store(smem0, c.tid, regs);
    __syncthreads();
    load_frags(smem0, c, 0, cur);
    for (int t = 0; t < ntiles; ++t) {
        unsigned char *stage = (t & 1) ? smem1 : smem0;
        unsigned char *other = (t & 1) ? smem0 : smem1;
        const bool more = t + 1 < ntiles;
        if (more) load(k_first + (t + 1) * G::BK, regs);
#pragma unroll
        for (int step = 0; step < G::STEPS - 1; ++step) {
            load_frags(stage, c, step + 1, nxt);
            mma(cur, acc);
            cur = nxt;
        }
        if (more) lds_store(other, c.tid, regs);
        __syncthreads();
        if (more) load_frags(other, c, 0, nxt);
        mma(cur, acc);
        cur = nxt;
    }
}

// ------------------------------------------------- implicit (convolution) B --

// Exact floor(j / d) for 0 <= j < 2^31 from host-made constants.
__device__ __forceinline__ int div_magic(int j, uint64_t m, int shift)
{
    return (int)(((uint64_t)(uint32_t)j * m) >> shift);
}

// Loader of B tiles of the convolution matrix, formed from the image ("Three
// X's: large convolutions in PyTorch for model training", section "CUTLASS":
// the implicit GEMM builds the matrix tiles inside the blocks, from output
// coordinates (p, q) and filter taps (ci, r, s), instead of materialising the
// matrix).  The terms that change along K are computed on the fly (the page's
// analytic iterator) or, for the table sources, looked up in a table made once
// per call (its optimized iterator, which precomputes offsets into lookup
// tables).
//
// Every matrix element is image[ci][y][x] with y = (p sh - ph) + r dh and
// x = (q sw - pw) + s dw (volume sources: image[ci][z][y][x], z likewise): a
// column term (from the output position) plus a row term (from the tap).  A thread's chunks share their column positions across its chunk
// rows (NT is a multiple of the chunks per tile row), so in the forward tile
// (rows k = taps, columns n = outputs) the column terms are fixed for the
// whole K loop and the row terms change per k-tile; in the filter-gradient
// tile (rows n = taps, columns k = outputs) it is the other way round.
// Elements in the padding, or past K or N, read at an offset beyond the
// image's buffer resource, which the hardware answers with zero.
template <class G, int MODE>
struct ConvGather {
    using T = typename G::TB;
    using In = typename G::In;
    static constexpr int U = T::PER_THREAD, V = T::VEC, RSTEP = T::NT / T::CPR;
    static constexpr bool FWD = conv_fwd_source(MODE);
    static constexpr bool TAB = conv_table_source(MODE);
    static constexpr bool VOL = conv_volume_source(MODE);
    static constexpr bool V4 = conv_4d_source(MODE);
    static constexpr bool PAD = conv_padded_source(MODE);
    static constexpr int ES = (int)sizeof(In);
    static_assert(T::NT % T::CPR == 0, "a thread's chunks must share their columns");
    static_assert((FWD && T::LAYOUT == MNMAJOR) || (!FWD && T::LAYOUT == KMAJOR),
                  "tile orientation of the convolution source");

    // Image coordinates (depth z for volume sources only, the outermost u for
    // four-dimensional ones) and byte offset of a term; an element's
    // coordinates and offset are the sums of its column term and its row term.
    struct Term {
        int u, z, y, x, o;
    };

    __amdgpu_buffer_rsrc_t rsrc;
    const ConvGeom *g;
    int row0, e0;      // first chunk row of this thread, first element in the row
    // Fixed terms -- column terms (forward) or row terms (filter gradient) --
    // plus whether that column / row lies inside the matrix.
    static constexpr int NF = FWD ? V : U;
    Term f[NF];
    bool fok[NF];
    // Table sources: the per-k entries of the next k-tile, loaded one tile
    // ahead so that their latency hides behind the current tile's gathers.
    static constexpr int NK = FWD ? U : V;   // k values per thread and tile
    int2 nxt[TAB ? NK : 1];
    // Forward: whether this thread's V columns are V consecutive output
    // positions of one output row with unit horizontal stride, so that for
    // every tap they read V consecutive image elements.
    bool run = false;

    // Terms of tap k = (ci R + r) S + s (volume: ((ci T + t) R + r) S + s;
    // four dimensions: (((ci KU + ku) T + t) R + r) S + s): u = ku lu,
    // z = t lz, y = r dh, x = s dw and the offset of (ci, u, z, y, x).
    __device__ __forceinline__ Term tap_terms(int k) const
    {
        Term e;
        int ci, rem;
        e.u = 0;
        if constexpr (V4) {
            ci = div_magic(k, g->ktrs_magic, g->ktrs_shift);
            rem = k - ci * g->ku * g->t * g->r * g->s;
            const int uu = div_magic(rem, g->trs_magic, g->trs_shift);
            rem -= uu * g->t * g->r * g->s;
            e.u = uu * g->lu;
            const int tt = div_magic(rem, g->rs_magic, g->rs_shift);
            rem -= tt * g->r * g->s;
            e.z = tt * g->lz;
        } else if constexpr (VOL) {
            ci = div_magic(k, g->trs_magic, g->trs_shift);
            rem = k - ci * g->t * g->r * g->s;
            const int tt = div_magic(rem, g->rs_magic, g->rs_shift);
            rem -= tt * g->r * g->s;
            e.z = tt * g->lz;
        } else {
            ci = div_magic(k, g->rs_magic, g->rs_shift);
            rem = k - ci * g->r * g->s;
            e.z = 0;
        }
        const int r = div_magic(rem, g->s_magic, g->s_shift);
        const int s = rem - r * g->s;
        e.y = r * g->dh;
        e.x = s * g->dw;
        const int plane = V4 ? (ci * g->du + e.u) * g->d + e.z : VOL ? ci * g->d + e.z : ci;
        e.o = ((plane * g->h + e.y) * g->w + e.x) * ES;
        return e;
    }
    // Terms of output position j = p Q + q (volume: (o P + p) Q + q; four
    // dimensions: ((ou O + o) P + p) Q + q): u = ou su - pu, z = o sz - pz,
    // y = p sh - ph, x = q sw - pw and the (possibly negative) offset of
    // (u, z, y, x).
    __device__ __forceinline__ Term out_terms(int j) const
    {
        Term e;
        int rem = j;
        e.u = 0;
        if constexpr (V4) {
            const int ou = div_magic(j, g->opq_magic, g->opq_shift);
            rem = j - ou * g->opq;
            e.u = ou * g->su - g->pu;
        }
        if constexpr (VOL) {
            const int o = div_magic(rem, g->pq_magic, g->pq_shift);
            rem -= o * g->pq;
            e.z = o * g->sz - g->pz;
        } else {
            e.z = 0;
        }
        const int p = div_magic(rem, g->q_magic, g->q_shift);
        const int q = rem - p * g->q;
        e.y = p * g->sh - g->ph;
        e.x = q * g->sw - g->pw;
        e.o = (((VOL ? ((V4 ? e.u * g->d : 0) + e.z) * g->h : 0) + e.y) * g->w + e.x) * ES;
        return e;
    }
    // Per-k terms of k (clamped into the matrix by the caller).
    __device__ __forceinline__ Term k_terms(int k) const
    {
        if constexpr (FWD)
            return tap_terms(k);
        else
            return out_terms(k);
    }
    static __device__ __forceinline__ Term unpack(int2 e)
    {
        return Term{0, 0, (e.x << 16) >> 16, e.x >> 16, e.y};
    }
    // k of this thread's i-th per-k slot in the k-tile at k0.
    __device__ __forceinline__ int k_of(int k0, int i) const
    {
        return FWD ? k0 + row0 + i * RSTEP : k0 + e0 + i;
    }
    __device__ __forceinline__ void prefetch(int k0, int kend)
    {
        if constexpr (TAB) {
#pragma unroll
            for (int i = 0; i < NK; ++i) nxt[i] = g->tab[min(k_of(k0, i), kend - 1)];
        }
    }
    // V consecutive terms that read V consecutive image elements of one row.
    static __device__ __forceinline__ bool is_run(const Term &a, const Term &b)
    {
        return (!V4 || a.u == b.u) & (!VOL || a.z == b.z) & (a.y == b.y) & (b.x == a.x + (V - 1));
    }

    __device__ __forceinline__ ConvGather(const KernelArgs &a, int bn, int tid, int kbeg, int kend)
        : g(&a.conv)
    {
        rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.B), 0, a.conv.img_bytes,
                                                 0x00020000);  // gfx9 raw-buffer format word
        row0 = tid / T::CPR;
        e0 = (tid % T::CPR) * V;
        if constexpr (FWD) {
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const int n = bn + e0 + e;
                fok[e] = n < a.N;
                f[e] = out_terms(min(n, a.N - 1));
            }
            run = fok[V - 1] & is_run(f[0], f[V - 1]);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int n = bn + row0 + u * RSTEP;
                fok[u] = n < a.N;
                f[u] = tap_terms(min(n, a.N - 1));
            }
        }
        prefetch(kbeg, kend);
    }

    // Whether image position (u, z, y, x) lies inside the image: unsigned
    // compares joined without short-circuits.
    __device__ __forceinline__ bool inside(int u, int z, int y, int x) const
    {
        if constexpr (PAD) return true;  // the padded image holds every position
        bool in = ((unsigned)y < (unsigned)g->h) & ((unsigned)x < (unsigned)g->w);
        if constexpr (VOL) in = in & ((unsigned)z < (unsigned)g->d);
        if constexpr (V4) in = in & ((unsigned)u < (unsigned)g->du);
        return in;
    }

    // The element of column term c and row term k, or zero when ok is false
    // or it lies in the padding.
    __device__ __forceinline__ In fetch(bool ok, const Term &c, const Term &k) const
    {
        const bool in = ok & inside(c.u + k.u, c.z + k.z, c.y + k.y, c.x + k.x);
        const int vo = in ? c.o + k.o : (int)0x80000000u;
        if constexpr (ES == 4)
            return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc, vo, 0, 0));
        else
            return (In)__builtin_amdgcn_raw_buffer_load_b16(rsrc, vo, 0, 0);
    }

    // 16 bytes of the image at byte offset off (inside the image; element
    // aligned, not necessarily 16-byte aligned).
    __device__ __forceinline__ u32x4 load_run(int off) const
    {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
        return u32x4{v[0], v[1], v[2], v[3]};
    }

    // The B tile of the k-tile at k0 (k below kend), chunk u of this thread in
    // r[u].  Called for consecutive k-tiles, starting at the constructor's kbeg.
    __device__ __forceinline__ void load(int k0, int kend, u32x4 (&r)[U])
    {
        union Chunk {
            u32x4 v;
            In e[V];
        };
        Term kt[NK];
        bool kok[NK];
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int k = k_of(k0, i);
            kok[i] = k < kend;
            if constexpr (TAB)
                kt[i] = unpack(nxt[i]);
            else
                kt[i] = k_terms(min(k, kend - 1));
        }
        prefetch(k0 + G::BK, kend);
        // A chunk whose V elements are V consecutive image elements of one
        // image row, all inside the image, is one 16-byte load; any other
        // chunk (crossing the padding, an output-row end, or with a stride)
        // is gathered element by element.
        if constexpr (FWD) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const Term &t = kt[u];
                const bool whole = run & kok[u] &
                                   inside(f[0].u + t.u, f[0].z + t.z, f[0].y + t.y,
                                          f[0].x + t.x) &
                                   (PAD || f[V - 1].x + t.x < g->w);
                if (whole) {
                    r[u] = load_run(f[0].o + t.o);
                } else {
                    Chunk c;
#pragma unroll
                    for (int e = 0; e < V; ++e) c.e[e] = fetch(kok[u] & fok[e], f[e], t);
                    r[u] = c.v;
                }
            }
        } else {
            const bool krun = kok[V - 1] & is_run(kt[0], kt[V - 1]);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const Term &t = f[u];
                const bool whole = krun & fok[u] &
                                   inside(t.u + kt[0].u, t.z + kt[0].z, t.y + kt[0].y,
                                          t.x + kt[0].x) &
                                   (PAD || t.x + kt[V - 1].x < g->w);
                if (whole) {
                    r[u] = load_run(t.o + kt[0].o);
                } else {
                    Chunk c;
#pragma unroll
                    for (int e = 0; e < V; ++e) c.e[e] = fetch(fok[u] & kok[e], kt[e], t);
                    r[u] = c.v;
                }
            }
        }
    }
};

// B fragments of the forward convolution product from a window of the image
// in LDS ("Three X's: large convolutions in PyTorch for model training",
// section "CUTLASS": the implicit GEMM forms the matrix tiles in the block;
// here for unit horizontal stride and dilation, where the matrix element of
// tap (ci, r, s) and output (p, q) is image[ci][p sh + r dh][q + s] of the
// zero-bordered image).  A lane's fragment holds KS consecutive taps
// s0 .. s0 + KS - 1 of one filter row for one output position, which are KS
// consecutive image elements from x = q + s0.  Filter rows are padded to S'
// taps (a multiple of KS dividing BK), so every k-tile covers NP = BK / S'
// whole filter rows, and its B values all come from NP x NR image rows (filter
// row kp, output row p): one window per k-tile instead of BK x BN gathered
// elements.  Window slot (j, i, x), at j NRWP + i W' + x (NRWP = NR W'
// rounded up to the thread count), holds the KS elements from x of the row of
// filter row kp0 + j and output row p_first + i; every fragment is one
// aligned 16-byte LDS read and consecutive lanes (consecutive q) read
// consecutive slots.  Because S' divides BK, a fragment step's filter row j
// and first tap s0 are the same in every k-tile, and so is the slot of a
// thread's u-th staged load within its filter row: all of it is computed once
// per block.  Taps s >= S (zero filter taps, only in a row's last slot) are
// zeroed in the fragment, so a non-finite pixel is never multiplied by them;
// filter rows past C_in R load zeros.
template <class G>
struct ConvWindow {
    using In = typename G::In;
    static constexpr int KS = G::KS;             // taps per slot and fragment
    static constexpr int U = G::TB::PER_THREAD;  // staged slots per thread
    static_assert(G::TB::CHUNKS == U * G::NT, "window slots fill the B stage");

    __amdgpu_buffer_rsrc_t rsrc;
    const ConvGeom *g;
    int nrwp, vrows;  // slots per filter row of the window (a multiple of NT), NT-rows of them
    int jrow[U];      // per staged load u: its filter row in the window, u / vrows (uniform)
    int pos[G::FN];   // per B fragment: i W' + q of this lane's output position
    int col[U];       // per staged load u: element offset of its slot within a filter
                      // row's image rows, (p_first + i) sh W' + x, or -1 past them
    int base[G::STEPS];      // per fragment step: j NRWP + s0 of this lane's half
    bool last[G::STEPS];     // per fragment step: the slot holds zero taps
    uint32_t keep[4];        // the real taps of such a slot, as a mask of its dwords

    __device__ __forceinline__ ConvWindow(const KernelArgs &a, int bn, int tid, int wcol, int lane)
        : g(&a.conv)
    {
        rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.B), 0, a.conv.img_bytes,
                                                 0x00020000);  // gfx9 raw-buffer format word
        const int p_first = div_magic(bn, g->q_magic, g->q_shift);
        const int nrw = g->nr * g->w;
        vrows = (nrw + G::NT - 1) / G::NT;
        nrwp = vrows * G::NT;
#pragma unroll
        for (int fn = 0; fn < G::FN; ++fn) {
            // columns past N repeat the last position (their outputs are not stored)
            const int n = min(bn + wcol * G::WTN + fn * 32 + (lane & 31), a.N - 1);
            const int p = div_magic(n, g->q_magic, g->q_shift);
            pos[fn] = (p - p_first) * g->w + (n - p * g->q);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            jrow[u] = u / vrows;
            const int in = tid + (u - jrow[u] * vrows) * G::NT;  // slot within its filter row
            const int i = div_magic(in, g->w_magic, g->w_shift);
            col[u] = in < nrw ? (p_first + i) * g->sh * g->w + (in - i * g->w) : -1;
        }
        const int h = lane >> 5;
#pragma unroll
        for (int st = 0; st < G::STEPS; ++st) {
            const int kk = h * G::KH + st * KS;  // k within the k-tile
            const int j = div_magic(kk, g->sp_magic, g->sp_shift);
            const int s0 = kk - j * g->sp;
            base[st] = j * nrwp + s0;
            last[st] = s0 + KS > g->s;
        }
        const int real = g->s - (g->sp - KS);  // real taps of a row's last slot
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            if constexpr (KS == 8)  // bf16: two taps per dword
                keep[d] = (2 * d < real ? 0x0000FFFFu : 0u) | (2 * d + 1 < real ? 0xFFFF0000u : 0u);
            else
                keep[d] = d < real ? 0xFFFFFFFFu : 0u;
        }
    }

    // The window of the k-tile at k0 (a multiple of BK), slot tid + u NT in
    // r[u]: staged load u serves filter row j = u / vrows (uniform), whose
    // image-row offset is computed once per filter row on the scalar unit.
    __device__ __forceinline__ void load(int k0, u32x4 (&r)[U]) const
    {
        const int kp0 = div_magic(k0, g->sp_magic, g->sp_shift);
        const int np = G::BK / g->sp;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = jrow[u];
            if (j >= np) break;  // past the window: no load (block-uniform)
            const int kp = kp0 + j;
            const int ci = div_magic(kp, g->r_magic, g->r_shift);
            const int rr = kp - ci * g->r;
            const int row = (ci * g->h + rr * g->dh) * g->w;  // element offset of the filter row
            const bool ok = (kp < g->cr) & (col[u] >= 0);
            const int off = ok ? (row + col[u]) * (int)sizeof(In) : (int)0x80000000u;
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
            r[u] = u32x4{v[0], v[1], v[2], v[3]};
        }
    }

    __device__ __forceinline__ void store(unsigned char *win, int tid, const u32x4 (&r)[U]) const
    {
        const int np = G::BK / g->sp;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (jrow[u] >= np) break;
            lds_store16(win, (tid + u * G::NT) * 16, r[u]);
        }
    }

    __device__ __forceinline__ u32x4 frag(const unsigned char *win, int st, int fn) const
    {
        const u32x4 v = lds_load16(win, (base[st] + pos[fn]) * 16);
        if (!last[st]) return v;
        return u32x4{v[0] & keep[0], v[1] & keep[1], v[2] & keep[2], v[3] & keep[3]};
    }
};

// The filter-gradient product from the same windows ("Three X's", section
// "CUTLASS", the implicit GEMM of the weight gradient): dW'[co][kp S' + s] =
// sum over positions k of dY'[co][k] X[k][kp S' + s], k = p Q' + q with every
// output row padded to Q' positions (a multiple of BK; dY' is zero at q >= Q)
// and the taps of every filter row padded to S' (their columns are dropped by
// the caller).  A lane's B fragment holds KS consecutive positions
// q .. q + KS - 1 of one output row for one tap (kp, s): KS consecutive
// image elements from x = q + s of image row (ci, p sh + r dh).  A block's
// BN columns are BN / S' whole filter rows, fixed for the block; a k-tile's
// BK positions lie in one output row p, from qa = k0 - p Q'.  So the window
// of a k-tile is, per filter row j of the block, the BK + S' - 1 elements of
// its image row from qa: slot (j, x') holds the KS elements from qa + x', at
// j LP + x' (LP = BK + S' - 1 rounded up to the thread count).  A fragment is
// slot (j, q_local + s): its offset is fixed per lane and step; per k-tile
// only the uniform term (p sh W' + qa) changes.  Positions q >= Q are zeroed
// in the fragment (dY' is zero there and a non-finite pixel must not meet
// it).
template <class G>
struct ConvWindowW {
    using In = typename G::In;
    static constexpr int KS = G::KS;
    static constexpr int U = G::TB::PER_THREAD;
    static_assert(G::TB::CHUNKS == U * G::NT, "window slots fill the B stage");

    __amdgpu_buffer_rsrc_t rsrc;
    const ConvGeom *g;
    int vrows, lp;       // NT-rows of slots per filter row, LP slots per filter row
    int jrow[U];         // per staged load u: its filter row (uniform)
    int col[U];          // element offset of its slot within the image for qa = 0,
                         // p = 0: (ci Hp + r dh) W' + x', or -1 (no load)
    int pos[G::FN];      // per B fragment: j LP + s of this lane's tap column

    __device__ __forceinline__ ConvWindowW(const KernelArgs &a, int bn, int tid, int wcol, int lane)
        : g(&a.conv)
    {
        rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.B), 0, a.conv.img_bytes,
                                                 0x00020000);  // gfx9 raw-buffer format word
        const int len = G::BK + g->sp - 1;  // window slots per filter row
        vrows = (len + G::NT - 1) / G::NT;
        lp = vrows * G::NT;
        const int kp_first = div_magic(bn, g->sp_magic, g->sp_shift);
#pragma unroll
        for (int fn = 0; fn < G::FN; ++fn) {
            // columns past N repeat the last tap (their sums are not stored)
            const int t = min(bn + wcol * G::WTN + fn * 32 + (lane & 31), a.N - 1) - bn;
            const int j = div_magic(t, g->sp_magic, g->sp_shift);
            pos[fn] = j * lp + (t - j * g->sp);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            jrow[u] = u / vrows;
            const int xo = tid + (u - jrow[u] * vrows) * G::NT;  // slot within its filter row
            const int kp = kp_first + jrow[u];
            const int ci = div_magic(min(kp, g->cr - 1), g->r_magic, g->r_shift);
            const int rr = min(kp, g->cr - 1) - ci * g->r;
            col[u] = ((xo < len) & (kp < g->cr)) ? (ci * g->h + rr * g->dh) * g->w + xo : -1;
        }
    }

    // The window of the k-tile at k0 (a multiple of BK, inside one output row).
    __device__ __forceinline__ void load(int k0, u32x4 (&r)[U]) const
    {
        const int p = div_magic(k0, g->qp_magic, g->qp_shift);
        const int shift = p * g->sh * g->w + (k0 - p * g->qp);  // uniform
        const int npb = G::BN / g->sp;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (jrow[u] >= npb) break;  // past the window: no load (block-uniform)
            const int off = col[u] >= 0 ? (col[u] + shift) * (int)sizeof(In) : (int)0x80000000u;
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
            r[u] = u32x4{v[0], v[1], v[2], v[3]};
        }
    }

    __device__ __forceinline__ void store(unsigned char *win, int tid, const u32x4 (&r)[U]) const
    {
        const int npb = G::BN / g->sp;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (jrow[u] >= npb) break;
            lds_store16(win, (tid + u * G::NT) * 16, r[u]);
        }
    }

    // Fragment step st of the k-tile at k0: positions q = qa + kk .. + KS - 1.
    __device__ __forceinline__ u32x4 frag(const unsigned char *win, int k0, int st, int fn,
                                          int lane) const
    {
        const int kk = (lane >> 5) * G::KH + st * KS;
        const u32x4 v = lds_load16(win, (pos[fn] + kk) * 16);
        const int p = div_magic(k0, g->qp_magic, g->qp_shift);
        const int real = g->q - (k0 - p * g->qp) - kk;  // positions of the fragment below Q
        if (real >= KS) return v;
        uint32_t keep[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            if constexpr (KS == 8)
                keep[d] = (2 * d < real ? 0x0000FFFFu : 0u) | (2 * d + 1 < real ? 0xFFFF0000u : 0u);
            else
                keep[d] = d < real ? 0xFFFFFFFFu : 0u;
        }
        return u32x4{v[0] & keep[0], v[1] & keep[1], v[2] & keep[2], v[3] & keep[3]};
    }
};

template <class G>
__device__ __forceinline__ u32x4 window_frag(const ConvWindow<G> &win, const unsigned char *w,
                                             int, int st, int fn, int)
{
    return win.frag(w, st, fn);
}
template <class G>
__device__ __forceinline__ u32x4 window_frag(const ConvWindowW<G> &win, const unsigned char *w,
                                             int k0, int st, int fn, int lane)
{
    return win.frag(w, k0, st, fn, lane);
}

template <class G, class W>
__device__ __forceinline__ void load_frags_window(const unsigned char *stage, const BlockCtx<G> &c,
                                                  const W &win, int k0, int step, Frags<G> &f)
{
    const int kk = (c.lane >> 5) * G::KH + step * G::KS;
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm)
        f.a[fm] = read_frag<typename G::TA>(stage, c.lane, c.wrow * G::WTM + fm * 32, kk);
#pragma unroll
    for (int fn = 0; fn < G::FN; ++fn)
        f.b[fn] = window_frag<G>(win, stage + G::A_BYTES, k0, step, fn, c.lane);
}

// main_loop_masked with a window source: A tiles as there, B from windows.
template <bool ALIGNED, class G, class W>
__device__ __forceinline__ void main_loop_window(unsigned char *smem0, unsigned char *smem1,
                                                 const BlockCtx<G> &c, const W &win,
                                                 int k_first, int ntiles,
                                                 floatx16 (&acc)[G::FM][G::FN])
{
    StageRegs<G> regs;
    Frags<G> cur, nxt;
    auto load = [&](int k0) {
        load_tile_masked<ALIGNED, typename G::TA>(c.A, c.lda, c.bm, c.M, k0, c.kend, c.tid, regs.a);
        win.load(k0, regs.b);
    };
    auto store = [&](unsigned char *stage) {
        store_tile<typename G::TA>(stage, c.tid, regs.a);
        win.store(stage + G::A_BYTES, c.tid, regs.b);
    };
    load(k_first);
    store(smem0);
    __syncthreads();
    load_frags_window(smem0, c, win, k_first, 0, cur);
    for (int t = 0; t < ntiles; ++t) {
        unsigned char *stage = (t & 1) ? smem1 : smem0;
        unsigned char *other = (t & 1) ? smem0 : smem1;
        const int k0 = k_first + t * G::BK;
        const bool more = t + 1 < ntiles;
        if (more) load(k0 + G::BK);
#pragma unroll
        for (int step = 0; step < G::STEPS - 1; ++step) {
            load_frags_window(stage, c, win, k0, step + 1, nxt);
            mma(cur, acc);
            cur = nxt;
        }
        if (more) store(other);
        __syncthreads();
        if (more) load_frags_window(other, c, win, k0 + G::BK, 0, nxt);
        mma(cur, acc);
        cur = nxt;
    }
}

// --------------------------------------------------------------- epilogue --

// Final value of one element of C: alpha * sum, plus beta * (old C) when
// beta != 0 (C is not read when beta == 0, so it may hold anything then),
// stored as fp32 or as bf16.
__device__ __forceinline__ void store_out(void *C, int64_t idx, float sum, float alpha, float beta,
                                          bool out_bf16)
{
    float v = alpha * sum;
    if (out_bf16) {
        uint16_t *c = static_cast<uint16_t *>(C);
        if (beta != 0.0f) v += beta * __uint_as_float((uint32_t)c[idx] << 16);
        c[idx] = f32_to_bf16_rne(v);
    } else {
        float *c = static_cast<float *>(C);
        if (beta != 0.0f) v += beta * c[idx];
        c[idx] = v;
    }
}

// Finished C through LDS, for interior blocks (the cases are listed where
// the epilogue picks it): the fragment layout gives each lane single elements
// of 32 columns, so element-wise stores (and, with beta != 0, loads of the
// old C) would move 4 or 2 bytes per lane.  After the main loop the stages
// are free: each wave writes one 32-row fragment row of its sub-block
// (32 x WTN fp32) to its own LDS scratch, reads it back as 16-byte row pieces
// (4 consecutive columns), and loads, scales and stores C in those pieces of
// 4 elements -- a wave's row run of WTN elements in one piece per lane, or,
// with `halves`, each piece as two stores of 2 elements (C rows 8-byte
// aligned for fp32, 4-byte for bf16).  The scratch is row-major with the 32-column halves of
// each 64-column group swapped in rows with bit 2 set, so the two lane halves
// of a fragment write (rows i and i+4) fall on different banks and the
// 16-byte reads of 16 lanes cover 256 contiguous bytes.
template <class G>
struct StagedOut {
    static constexpr int BYTES = 32 * G::WTN * 4;                // one wave's scratch
    static constexpr int PER_STAGE = G::STAGE_BYTES / BYTES;     // scratches per stage array
    static constexpr int CPR = G::WTN / 4;                       // 16-byte pieces per row
    static constexpr int PER_LANE = 32 * CPR / 64;               // pieces per lane and row block
    // Blocks of at most 64 rows (the skinny, wide and small classes, and most
    // convolution products) keep the element-wise epilogue: their outputs are
    // split-K partials or plain products almost always, and the staged code
    // alone, never executed, measured 3% slower on the 64 x 256 entry's
    // streaming product (64 x 16384 x 61504 in 8 K slices).
    static constexpr bool OK =
        G::BM > 64 && G::WTN % 64 == 0 && PER_STAGE * G::STAGES >= G::NW;
};

template <class G>
__device__ __forceinline__ int staged_col(int row, int col)
{
    return col ^ (((row >> 2) & 1) << 5);
}

template <class G>
__device__ __forceinline__ void staged_epilogue(unsigned char *l0, unsigned char *l1,
                                                unsigned char *l2, unsigned char *l3,
                                                const BlockCtx<G> &c, const KernelArgs &p,
                                                const floatx16 (&acc)[G::FM][G::FN], bool halves)
{
    using S = StagedOut<G>;
    const int wave = __builtin_amdgcn_readfirstlane(c.tid >> 6);
    const int arr = wave / S::PER_STAGE;
    unsigned char *scr = (arr == 0 ? l0 : arr == 1 ? l1 : arr == 2 ? l2 : l3) +
                         (wave % S::PER_STAGE) * S::BYTES;
    const int half = c.lane >> 5, l32 = c.lane & 31;
    const bool out_bf16 = p.out_bf16 != 0, read_c = p.beta != 0.0f;
    const float alpha = p.alpha, beta = p.beta;
    // the stages' last readers are done before any wave writes its scratch
    __syncthreads();
    static_for<0, G::FM>([&](auto fm) {
#pragma unroll
        for (int fn = 0; fn < G::FN; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 8 * (r >> 2) + 4 * half + (r & 3);
                *reinterpret_cast<float *>(scr + 4 * (row * G::WTN +
                                                      staged_col<G>(row, fn * 32 + l32))) =
                    acc[fm][fn][r];
            }
        // A wave's LDS accesses complete in order: the reads below see the
        // writes above, and the next row block's writes follow these reads.
        // Pieces go in groups of four (16 registers of old C per group), so
        // the epilogue does not raise the kernel's register count past what
        // its main loop needs.
        const int64_t row0 = c.bm + c.wrow * G::WTM + fm * 32;
        const int col0 = c.bn + c.wcol * G::WTN;
        constexpr int GRP = S::PER_LANE < 4 ? S::PER_LANE : 4;
#pragma unroll
        for (int u0 = 0; u0 < S::PER_LANE; u0 += GRP) {
            u32x4 old[GRP];
            if (read_c) {
#pragma unroll
                for (int g = 0; g < GRP; ++g) {
                    const int ch = c.lane + 64 * (u0 + g), rr = ch / S::CPR, cc = ch % S::CPR;
                    const int64_t idx = (row0 + rr) * p.ldc + col0 + 4 * cc;
                    if (out_bf16) {
                        const uint32_t *q = reinterpret_cast<const uint32_t *>(
                            static_cast<const uint16_t *>(p.C) + idx);
                        const uint32_t w0 = q[0], w1 = q[1];
                        old[g] = u32x4{w0 << 16, w0 & 0xFFFF0000u, w1 << 16, w1 & 0xFFFF0000u};
                    } else if (halves) {
                        const u32x2 *q = reinterpret_cast<const u32x2 *>(
                            static_cast<const float *>(p.C) + idx);
                        const u32x2 lo = q[0], hi = q[1];
                        old[g] = u32x4{lo[0], lo[1], hi[0], hi[1]};
                    } else {
                        old[g] = load16(static_cast<const float *>(p.C) + idx);
                    }
                }
            }
#pragma unroll
            for (int g = 0; g < GRP; ++g) {
                const int ch = c.lane + 64 * (u0 + g), rr = ch / S::CPR, cc = ch % S::CPR;
                const u32x4 raw = lds_load16(scr, 4 * (rr * G::WTN + staged_col<G>(rr, 4 * cc)));
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = alpha * __uint_as_float(raw[e]);
                    if (read_c) v[e] += beta * __uint_as_float(old[g][e]);
                }
                const int64_t idx = (row0 + rr) * p.ldc + col0 + 4 * cc;
                // non-temporal, as on the plain path: C is not read again here
                if (out_bf16) {
                    const uint32_t w0 = f32x2_to_bf16x2_rne(v[0], v[1]);
                    const uint32_t w1 = f32x2_to_bf16x2_rne(v[2], v[3]);
                    uint16_t *out = static_cast<uint16_t *>(p.C) + idx;
                    if (halves) {
                        __builtin_nontemporal_store(w0, reinterpret_cast<uint32_t *>(out));
                        __builtin_nontemporal_store(w1, reinterpret_cast<uint32_t *>(out + 2));
                    } else {
                        __builtin_nontemporal_store(u32x2{w0, w1}, reinterpret_cast<u32x2 *>(out));
                    }
                } else {
                    float *out = static_cast<float *>(p.C) + idx;
                    if (halves) {
                        __builtin_nontemporal_store(u32x2{__float_as_uint(v[0]), __float_as_uint(v[1])},
                                                    reinterpret_cast<u32x2 *>(out));
                        __builtin_nontemporal_store(u32x2{__float_as_uint(v[2]), __float_as_uint(v[3])},
                                                    reinterpret_cast<u32x2 *>(out + 2));
                    } else {
                        __builtin_nontemporal_store(
                            u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                  __float_as_uint(v[3])},
                            reinterpret_cast<u32x4 *>(out));
                    }
                }
            }
        }
    });
}

// The staged epilogue for bf16 C with beta == 0 and C rows 16-byte aligned:
// the scaled values are rounded to bf16 before they go through the wave's
// scratch (the same single rounding of alpha * acc as above), so the scratch
// holds half the bytes and each lane stores whole 16-byte pieces of 8
// columns.  Same swizzle as the fp32 scratch: the two lane halves of a write
// (rows 4 apart) fall on different banks, and a 16-lane read covers 256
// contiguous bytes.
template <class G>
__device__ __forceinline__ void staged_epilogue_bf16(unsigned char *l0, unsigned char *l1,
                                                     unsigned char *l2, unsigned char *l3,
                                                     const BlockCtx<G> &c, const KernelArgs &p,
                                                     const floatx16 (&acc)[G::FM][G::FN])
{
    using S = StagedOut<G>;
    constexpr int CPR = G::WTN / 8;               // 16-byte pieces per row
    constexpr int PER_LANE = 32 * CPR / 64;       // pieces per lane and row block
    const int wave = __builtin_amdgcn_readfirstlane(c.tid >> 6);
    const int arr = wave / S::PER_STAGE;
    unsigned char *scr = (arr == 0 ? l0 : arr == 1 ? l1 : arr == 2 ? l2 : l3) +
                         (wave % S::PER_STAGE) * S::BYTES;
    const int half = c.lane >> 5, l32 = c.lane & 31;
    const float alpha = p.alpha;
    // the stages' last readers are done before any wave writes its scratch
    __syncthreads();
    static_for<0, G::FM>([&](auto fm) {
#pragma unroll
        for (int fn = 0; fn < G::FN; ++fn)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                // rows `row` and `row + 1` of one column, rounded as a pair
                const int row = 8 * (r >> 2) + 4 * half + (r & 3);
                const uint32_t w =
                    f32x2_to_bf16x2_rne(alpha * acc[fm][fn][r], alpha * acc[fm][fn][r + 1]);
                *reinterpret_cast<uint16_t *>(scr + 2 * (row * G::WTN +
                                                         staged_col<G>(row, fn * 32 + l32))) =
                    (uint16_t)w;
                *reinterpret_cast<uint16_t *>(
                    scr + 2 * ((row + 1) * G::WTN + staged_col<G>(row + 1, fn * 32 + l32))) =
                    (uint16_t)(w >> 16);
            }
        // in-order LDS accesses of one wave: the reads see the writes above,
        // and the next row block's writes follow these reads
        const int64_t row0 = c.bm + c.wrow * G::WTM + fm * 32;
        const int col0 = c.bn + c.wcol * G::WTN;
#pragma unroll
        for (int u = 0; u < PER_LANE; ++u) {
            const int ch = c.lane + 64 * u, rr = ch / CPR, cc = ch % CPR;
            const u32x4 v = lds_load16(scr, 2 * (rr * G::WTN + staged_col<G>(rr, 8 * cc)));
            uint16_t *out = static_cast<uint16_t *>(p.C) + (row0 + rr) * p.ldc + col0 + 8 * cc;
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(out));
        }
    });
}

// ------------------------------------------------------------------ kernel --

template <bool BF16, int BM, int BN, int BK, int WM, int WN, int STAGES, int LA, int LB,
          bool ALIGNED, int BSRC = B_MATRIX>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_kernel(KernelArgs p)
{
    using G = Geo<BF16, BM, BN, BK, WM, WN, STAGES, LA, LB>;
    using In = typename G::In;

    // One __shared__ array per stage (unused ones are one byte).
    __shared__ __attribute__((aligned(1024))) unsigned char lds0[G::STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) unsigned char lds1[G::STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) unsigned char lds2[STAGES > 2 ? G::STAGE_BYTES : 1];
    __shared__ __attribute__((aligned(1024))) unsigned char lds3[STAGES > 3 ? G::STAGE_BYTES : 1];

    BlockCtx<G> c;
    c.tid = (int)threadIdx.x;
    c.lane = c.tid & 63;
    const int wave = c.tid >> 6;
    c.wrow = wave / WN;
    c.wcol = wave % WN;

    int slice, tm, tn;
    block_coords(p, slice, tm, tn);
    c.bm = tm * BM;
    c.bn = tn * BN;
    c.A = static_cast<const In *>(p.A);
    c.B = static_cast<const In *>(p.B);
    c.lda = p.lda;
    c.ldb = p.ldb;
    c.M = p.m_load;
    c.N = p.n_load;
    const int kbeg = slice * p.k_per_split;
    c.kend = min(p.K, kbeg + p.k_per_split);
    const int ntiles = (c.kend - kbeg + BK - 1) / BK;

    floatx16 acc[G::FM][G::FN];
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < G::FN; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[fm][fn][r] = 0.0f;

    // Interior blocks run their whole k-tiles without bounds checks; the
    // partial last k-tile, blocks crossing the M or N edge, unaligned operands
    // and leading dimensions too large for 32-bit tile offsets take the
    // masked loads.  The choice is uniform per workgroup.
    if constexpr (BSRC == B_MATRIX) {
        // Whole k-tiles go through direct global->LDS loads: 16 bytes per lane
        // for aligned operands, in interior blocks and in blocks crossing the
        // M or N edge when each outer-contiguous operand's outer extent is a
        // whole number of 16-byte chunks (see tile_offsets); 4 range-checked
        // bytes per lane for the other edge blocks and for rows at any 4-byte
        // alignment.  Other cases, and the partial last k-tile, take the
        // masked loads.
        const bool edge_mn = c.bm + BM > c.M || c.bn + BN > c.N;
        const bool edge16 = (G::LA == KMAJOR || c.M % G::VEC == 0) &&
                            (G::LB == KMAJOR || c.N % G::VEC == 0);
        const bool x4 = ALIGNED && p.direct_ok && (!edge_mn || edge16);
        // bf16 dwords are element pairs (k, k+1) of a k-contiguous row or
        // (n, n+1) of an outer-contiguous one: rows must start 4-byte aligned,
        // and an outer-contiguous extent must be even, so that the last pair
        // of the last row does not reach past the operand (a range check
        // that cut it would zero a valid element).  Pairs along k stay inside
        // K: only whole k-tiles, which start at even k, take these loads.
        const bool pairs_ok =
            !G::BF16 || (((p.lda | p.ldb) & 1) == 0 && (((uintptr_t)p.A | (uintptr_t)p.B) & 3) == 0 &&
                         (G::LA == KMAJOR || (c.M & 1) == 0) && (G::LB == KMAJOR || (c.N & 1) == 0));
        const bool dw = G::DMA4 && p.direct_ok && pairs_ok && !x4;
        const int nfast = x4 || dw ? (c.kend - kbeg) / BK : 0;
        c.rot = (tm + tn) % 8;
        if constexpr (G::DMA4) {
            c.a_end = operand_end_bytes<typename G::TA>(p.lda, c.M, p.K);
            c.b_end = operand_end_bytes<typename G::TB>(p.ldb, c.N, p.K);
            if (dw && nfast > 0)
                main_loop_direct<G, 4>(lds0, lds1, lds2, lds3, c, kbeg, nfast, acc);
        }
        if constexpr (ALIGNED) {
            if (x4 && nfast > 0)
                main_loop_direct<G, 16>(lds0, lds1, lds2, lds3, c, kbeg, nfast, acc);
        }
        if (ntiles > nfast)
            main_loop_masked(lds0, lds1, c, kbeg + nfast * BK, ntiles - nfast, acc,
                             [&](int k0, StageRegs<G> &r) { global_load_masked<ALIGNED>(c, k0, r); });
    } else if constexpr (BSRC == B_CONV_FWD_WIN) {
        // implicit GEMM: A from memory, B fragments from image windows in LDS
        ConvWindow<G> win(p, c.bn, c.tid, c.wcol, c.lane);
        main_loop_window<ALIGNED>(lds0, lds1, c, win, kbeg, ntiles, acc);
    } else if constexpr (BSRC == B_CONV_WGRAD_WIN) {
        ConvWindowW<G> win(p, c.bn, c.tid, c.wcol, c.lane);
        main_loop_window<ALIGNED>(lds0, lds1, c, win, kbeg, ntiles, acc);
    } else {
        // implicit GEMM: A from memory, B tiles formed from the image
        ConvGather<G, BSRC> gather(p, c.bn, c.tid, kbeg, c.kend);
        main_loop_masked(lds0, lds1, c, kbeg, ntiles, acc, [&](int k0, StageRegs<G> &r) {
            load_tile_masked<ALIGNED, typename G::TA>(c.A, c.lda, c.bm, c.M, k0, c.kend, c.tid, r.a);
            gather.load(k0, c.kend, r.b);
        });
    }

    // Epilogue: element r of a 32x32 accumulator fragment sits at row
    // 8*(r/4) + 4*(lane/32) + r%4 and column lane%32 of that fragment.  With
    // split-K the raw partial sums go to the workspace (the reduce applies
    // alpha, beta and the output type); otherwise they are finished here.
    const int half = c.lane >> 5, l32 = c.lane & 31;
    const bool store_edge = c.bm + BM > p.M || c.bn + BN > p.N;
    const bool partial = p.splits > 1;
    if (partial) {
        // raw sums of this slice, read back by the reduce kernel
        float *out = p.ws + (int64_t)slice * p.M * p.N;
#pragma unroll
        for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < G::FN; ++fn) {
                const int gj = c.bn + c.wcol * G::WTN + fn * 32 + l32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int gi =
                        c.bm + c.wrow * G::WTM + fm * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                    if (!store_edge || (gi < p.M && gj < p.N))
                        out[(int64_t)gi * p.N + gj] = acc[fm][fn][r];
                }
            }
        return;
    }
    // Interior blocks of entries with a staged epilogue finish C through LDS
    // in 4-element row pieces when the rows hold whole pieces (16 bytes fp32,
    // 8 bytes bf16) or half pieces ("halves": rows 8- or 4-byte aligned,
    // each piece stored in two halves): the outputs other than the plain
    // fp32 product always, and the plain product when C's rows are not whole
    // 128-byte lines.  Then a wave's 32-element row runs straddle two lines
    // each, and the element-wise stores below issue twice as many partial-line
    // writes as the staged pieces (measured: bf16 8192 x 30520 x 768,
    // 587 -> 793 TF/s; 8192 x 8184 x 8192, 1288 -> 1311).
    int staged = 0;   // 0: no, 1: whole pieces, 2: halves, 3: bf16 pieces of 8 (beta == 0)
    if constexpr (StagedOut<G>::OK) {
        const int64_t piece = p.out_bf16 ? 8 : 16;
        const bool plain = p.alpha == 1.0f && p.beta == 0.0f && !p.out_bf16;
        const bool lines = (p.ldc * 4) % 128 == 0 && (uintptr_t)p.C % 128 == 0;
        if (!store_edge && !(plain && lines)) {
            const int64_t esz = p.out_bf16 ? 2 : 4;
            if (p.out_bf16 && p.beta == 0.0f && (p.ldc * 2) % 16 == 0 && (uintptr_t)p.C % 16 == 0)
                staged = 3;
            else if ((p.ldc * esz) % piece == 0 && (uintptr_t)p.C % piece == 0)
                staged = 1;
            else if ((p.ldc * esz) % (piece / 2) == 0 && (uintptr_t)p.C % (piece / 2) == 0)
                staged = 2;
        }
    }
    if (staged == 3) {
        staged_epilogue_bf16<G>(lds0, lds1, lds2, lds3, c, p, acc);
        return;
    }
    if (staged) {
        staged_epilogue<G>(lds0, lds1, lds2, lds3, c, p, acc, staged == 2);
        return;
    }
    if (p.alpha == 1.0f && p.beta == 0.0f && !p.out_bf16) {
        // the plain product into fp32 C.  C is written once and not read
        // again here: non-temporal stores keep it from evicting the operand
        // tiles other blocks still stream through the caches (measured
        // 1-2.5% on bf16 8192^3, 8% in a later build).
        float *out = static_cast<float *>(p.C);
#pragma unroll
        for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < G::FN; ++fn) {
                const int gj = c.bn + c.wcol * G::WTN + fn * 32 + l32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int gi =
                        c.bm + c.wrow * G::WTM + fm * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                    if (!store_edge || (gi < p.M && gj < p.N))
                        __builtin_nontemporal_store(acc[fm][fn][r], &out[(int64_t)gi * p.ldc + gj]);
                }
            }
        return;
    }
    static_for<0, G::FM>([&](auto fm) {
        static_for<0, G::FN>([&](auto fn) {
            const int gj = c.bn + c.wcol * G::WTN + fn * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gi = c.bm + c.wrow * G::WTM + fm * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (!store_edge || (gi < p.M && gj < p.N))
                    store_out(p.C, (int64_t)gi * p.ldc + gj, acc[fm][fn][r], p.alpha, p.beta,
                              p.out_bf16 != 0);
            }
        });
    });
}

}  // namespace dg
