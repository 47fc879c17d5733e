// C ABI of the dense GEMM library: argument checks, shape-class dispatch over
// the tile table, split-K workspace, launches.  Declared in include/gemm.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>
#include <vector>

#include "gemm.h"
#include "gemm_configs.hpp"
#include "gemm_internal.hpp"

namespace dg {
namespace {

constexpr int64_t kMaxDim = int64_t(1) << 30;  // keeps all in-kernel int math exact
// Compute units assumed when no device can be queried (the tile-table hooks on
// a host without a GPU): MI355X, 8 XCDs x 32 CUs.
constexpr int kDefaultComputeUnits = 256;
constexpr int kMaxStreamSplits = 16;
// LDS bytes of one compute unit (gfx950).
constexpr int64_t kLdsBytes = 160 * 1024;
constexpr int kMaxDevices = 64;

// Compute units of the current device (hipDeviceGetAttribute, cached per
// device), or kDefaultComputeUnits when no device is visible.
int compute_units()
{
    static std::atomic<int> cached[kMaxDevices];
    int device = -1;
    if (hipGetDevice(&device) != hipSuccess || device < 0 || device >= kMaxDevices) {
        (void)hipGetLastError();
        return kDefaultComputeUnits;
    }
    int cus = cached[device].load(std::memory_order_relaxed);
    if (cus > 0) return cus;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        cus <= 0) {
        (void)hipGetLastError();
        return kDefaultComputeUnits;
    }
    cached[device].store(cus, std::memory_order_relaxed);
    return cus;
}

const TileConfig *table(int dtype, int *count)
{
    if (dtype == GEMM_DTYPE_F32) return f32_configs(count);
    if (dtype == GEMM_DTYPE_BF16) return bf16_configs(count);
    *count = 0;
    return nullptr;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Index of the table entry called `name`, or -1 when the table has no such
// entry (the dispatcher's names and the tables disagree: an internal error
// that the callers report as GEMM_ERR_INTERNAL).  The tables are fixed, so each
// lookup result is cached by the caller.
int config_index(int dtype, const char *name)
{
    int count = 0;
    const TileConfig *tab = table(dtype, &count);
    for (int i = 0; i < count; ++i)
        if (std::strcmp(tab[i].name, name) == 0) return i;
    std::fprintf(stderr, "dense_gemm: tile table has no entry \"%s\"\n", name);
    return -1;
}

// Fraction of the GPU's block slots a grid of `tiles` blocks keeps busy over
// its rounds: tiles / (rounds * slots), slots = compute units x resident
// blocks per unit.
double fill(int64_t tiles, int64_t slots)
{
    const int64_t rounds = (tiles + slots - 1) / slots;
    return (double)tiles / (double)(rounds * slots);
}

// Rows (or columns) of the product given to full blocks of `b` when the last
// block row (column) would hold only a thin remainder -- at most an eighth of
// a block: those few rows then run as a separate, small product, so that the
// main grid has no block row doing a full K loop for a handful of outputs.
int64_t main_extent(int64_t M, int b)
{
    const int64_t r = M % b;
    return r > 0 && 8 * r <= b && M > r ? M - r : M;
}

struct Candidate {
    const char *name;
    int per_cu;        // resident blocks per compute unit (LDS-limited)
    double measured;   // fraction of the dtype's matrix peak on a full-chip run
};

// Among `cands`, the entry with the best measured efficiency times the fill
// of its grid for this M x N on `cus` compute units (-1 if a name is missing).
int best_of(int dtype, const Candidate *cands, int n, int64_t M, int64_t N, int cus,
            bool whole_grids = false)
{
    int count = 0;
    const TileConfig *tab = table(dtype, &count);
    int best = -1;
    double best_score = -1.0;
    for (int i = 0; i < n; ++i) {
        const int idx = config_index(dtype, cands[i].name);
        if (idx < 0) return -1;
        // the grid of the main part (thin remainders run apart, see run_call)
        const int64_t tiles = ceil_div(main_extent(M, tab[idx].bm), tab[idx].bm) *
                              ceil_div(main_extent(N, tab[idx].bn), tab[idx].bn);
        // whole_grids: entries of one resident block per CU whose grid leaves
        // CUs idle would run K-sliced; left out where that is slow
        if (whole_grids && cands[i].per_cu == 1 && tiles < cus) continue;
        const double score = cands[i].measured * fill(tiles, (int64_t)cus * cands[i].per_cu);
        if (score > best_score) {
            best_score = score;
            best = idx;
        }
    }
    return best;
}

// Shape classes -> table entry (-1 if an entry it names is missing).  The
// "measured" factors are the fractions of peak each tile shape reached on
// 4096^3 fp32 / 8192^3 bf16 (full grids), so the choice trades per-block
// efficiency against quantisation of the grid over the `cus` compute units.
int select_config(int dtype, int layout, int64_t M, int64_t N, int64_t K, int cus)
{
    (void)K;
    // Skinny products (a few dozen rows, wide N, usually long K: the
    // convolution GEMMs with few output channels) stream the large operand
    // once; 32-row blocks waste no matrix-core work at M <= 32, and when that
    // operand is read k-contiguous (B^T) rows of 256 (bf16 64-row blocks: 512)
    // bytes per k-tile keep its reads long.
    const bool skinny = M <= 32 && N >= 1024;
    if (dtype == GEMM_DTYPE_F32) {
        static const int tall = config_index(dtype, "f32_128x64_w2x2_s2");
        // wide: A . B takes two LDS stages (80 KB: two resident blocks per
        // CU, so one block's loads run under the other's products; measured
        // 3-11% faster than three stages at M = 64, N 8192-16384, and equal
        // at N = 2048); the other operand forms have the three-stage entry
        static const int wide_nn = config_index(dtype, "f32_64x256_w1x4_s2");
        static const int wide = config_index(dtype, "f32_64x256_w1x4_s3");
        // wide A . B^T: 64x64 blocks with 256-byte k-contiguous rows (64 KB of
        // LDS: two resident blocks per CU); measured 4-5% faster than 64x128
        // blocks at M = 64, N 8192-61504, K = 16384
        static const int wide_t = config_index(dtype, "f32_64x64x64_w2x2_s2");
        static const int skinny_n = config_index(dtype, "f32_32x128_w1x4_s3");
        static const int skinny_t = config_index(dtype, "f32_32x128x64_w1x4_s2");
        static const int narrow = config_index(dtype, "f32_128x64_w2x1_s2");
        static const int small = config_index(dtype, "f32_64x64_w2x2_s2");
        static const int small3 = config_index(dtype, "f32_64x64_w2x2_s3");
        // The efficiency figures rank the entries under the fill model; they
        // were set against a sweep of A . B at M, N of 2048-4096 (every
        // entry and split): 64x64 blocks in two stages (two resident per CU)
        // where their grid fills whole rounds better than the three-stage
        // ones (2048^3: 127 against 159 us; 2560^3: 274 against 326 for
        // 256x128 blocks in three K slices; 3584^3: 699 against 712), three
        // stages where they fill whole rounds (3072^3: 425 against 460), and
        // the 256-column blocks where their grid covers the chip.  One-block
        // entries whose grid would not cover the chip are left out: K-sliced,
        // they lost (2560^3 above).
        static const Candidate large[] = {
            {"f32_256x256_w4x2_s2", 1, 0.93},
            {"f32_256x128_w4x2_s2", 1, 0.885},
            {"f32_64x64_w2x2_s3", 3, 0.89},
            {"f32_64x64_w2x2_s2", 2, 0.88},
        };
        if (N <= 64 && M >= 4096) return tall;   // tall-skinny: many 64-row blocks
        if (skinny && layout == LAYOUT_NN) return skinny_n;
        if (skinny && layout == LAYOUT_NT) return skinny_t;
        if (M <= 64 && N >= 1024)  // split-K
            return layout == LAYOUT_NT ? wide_t : layout == LAYOUT_NN ? wide_nn : wide;
        if (M >= 2048 && N >= 2048) return best_of(dtype, large, 4, M, N, cus, true);
        if (N <= 64) return narrow;
        // at most one 64x64 block per compute unit and a K loop of 24 or more
        // k-tiles: three stages hide more of the load latency (1000^3: 24.7
        // against 26.2 us); with more blocks per unit the third stage's LDS
        // costs resident blocks (1024 x 4096 x 1024: 82 against 66 us)
        if (ceil_div(M, 64) * ceil_div(N, 64) <= cus && ceil_div(K, 32) >= 24) return small3;
        return small;
    }
    // 128x128 blocks: two stages (64 KB, two resident per CU) where the grid
    // needs more than one block per CU, three (96 KB, one per CU) where it
    // fits in one round, so the third stage costs no residency: 2048^3 A . B
    // 552 -> 740 TF/s, 2048 x 2048 x 4096 642 -> 849; at 2560^3 (400 blocks)
    // three stages lost, 651 against 860 (harness, one box).  The efficiency
    // figures rank the entries by the fill model; three stages rank just
    // below two at equal fill.
    static const Candidate large[] = {
        {"bf16_256x256x32_w4x2_s4", 1, 0.52},
        {"bf16_128x128x64_w2x2_s2", 2, 0.42},
        {"bf16_128x128x64_w2x2_s3", 1, 0.40},
    };
    // A read k-contiguous (A . B, A . B^T): 64-deep k-tiles in two stages
    // read whole 128-byte lines of A (and of B^T, whose 64-byte pieces kept
    // the data-return path 97% busy at 8192^3 A . B^T); measured against the
    // 32-deep four-stage block: A . B^T +5% at 4096^3 and 8192^3, A . B
    // +1.9% at 8192^3 and +1.2% at 4096^3 (alternating, two boxes).  A^T . B
    // lost 2% with it, and A^T . B^T's element-wise variant spilled.
    // 192 x 256 blocks (8 waves of 96 x 64) cover outputs that 256 x 256
    // blocks leave a quarter or more of the chip idle on: 3072^2 is 192 of
    // them against 144, 6144^2 three whole rounds against 2.25.  Measured
    // against the previous choice (median of single calls, one box): A . B
    // 3072^3 70.5 -> 60.2 us, 4608^3 203.6 -> 180.5, 6144^3 426.7 -> 381.4,
    // 3072 x 3072 x 8192 152.6 -> 136.7; A . B^T 8-11% faster at the same
    // shapes.  On a full grid they reach 0.48 of the peak (6144^3), against
    // 0.55 for 256 x 256, which therefore stays at 4096^3 and 8192^3.
    static const Candidate large_ak[] = {
        {"bf16_256x256x64_w4x2_s2", 1, 0.55},
        {"bf16_128x128x64_w2x2_s2", 2, 0.42},
        {"bf16_128x128x64_w2x2_s3", 1, 0.40},
        {"bf16_192x256x64_w2x4_s2", 1, 0.48},
    };
    static const int medium = config_index(dtype, "bf16_128x128x64_w2x2_s2");
    static const int medium3 = config_index(dtype, "bf16_128x128x64_w2x2_s3");
    static const int small = config_index(dtype, "bf16_64x64x64_w2x2_s2");
    static const int small_deep = config_index(dtype, "bf16_64x64x64_w2x2_s4");
    static const int wide = config_index(dtype, "bf16_64x256x64_w1x4_s3");
    // wide A . B^T: 64x64 blocks, four stages of 64 k (64 KB of LDS: two
    // resident blocks per CU); measured 3% faster than 256-deep k-tiles
    // (128 KB, one block per CU) at N = 61504 and 17% at N = 8192, K = 16384
    static const int wide_t = config_index(dtype, "bf16_64x64x64_w2x2_s4");
    static const int skinny_n = config_index(dtype, "bf16_32x256x64_w1x4_s3");
    static const int skinny_t = config_index(dtype, "bf16_32x256x128_w1x4_s2");
    if (skinny && layout == LAYOUT_NN) return skinny_n;
    if (skinny && layout == LAYOUT_NT) return skinny_t;
    if (M <= 64 && N >= 1024) return layout == LAYOUT_NT ? wide_t : wide;  // split-K
    if (M >= 2048 && N >= 2048)
        return layout == LAYOUT_NN || layout == LAYOUT_NT ? best_of(dtype, large_ak, 4, M, N, cus)
                                                          : best_of(dtype, large, 3, M, N, cus);
    // Mid-size and small products, from a sweep of A . B and A . B^T at M, N
    // of 512-2048 and K of 512-8192: 128x128 blocks (K-sliced when they do
    // not fill the chip) where they fill it or K is long; 64x64 blocks where
    // the 128x128 grid would leave compute units idle and K is at most 2048
    // (1536^3: 16.8 us against 24.4 with 128x128 blocks in two slices); four
    // stages when even the 64x64 grid or the 128x128 one is small and K is
    // longer (1024 x 1024 x 4096: 18.0 us against 23.2).
    const int64_t t128 = ceil_div(M, 128) * ceil_div(N, 128), t64 = ceil_div(M, 64) * ceil_div(N, 64);
    const int64_t kt = ceil_div(K, 64);
    // a 128x128 grid of exactly one block per CU: one round, so the third
    // stage costs no residency (as in the large class)
    if (t128 >= cus || kt >= 96) return t128 == cus ? medium3 : medium;
    if (kt <= 32) return t64 >= cus ? small : small_deep;
    return 4 * t128 <= cus ? small_deep : medium;
}

// Entry for an implicit-GEMM convolution product (the entries built with
// implicit kernels), by the number of output channels M.
int select_implicit(int dtype, int64_t M)
{
    if (dtype == GEMM_DTYPE_F32) {
        static const int skinny = config_index(dtype, "f32_32x128_w1x4_s3");
        static const int wide = config_index(dtype, "f32_64x256_w1x4_s3");
        static const int mid = config_index(dtype, "f32_128x128_w2x2_s2");
        static const int large = config_index(dtype, "f32_256x128_w4x2_s2");
        return M <= 32 ? skinny : M <= 64 ? wide : M <= 128 ? mid : large;
    }
    static const int skinny = config_index(dtype, "bf16_32x256x64_w1x4_s3");
    static const int wide = config_index(dtype, "bf16_64x256x64_w1x4_s3");
    static const int mid = config_index(dtype, "bf16_128x128x64_w2x2_s2");
    static const int large = config_index(dtype, "bf16_256x128x64_w2x2_s2");
    return M <= 32 ? skinny : M <= 64 ? wide : M <= 128 ? mid : large;
}

// Number of K slices.  Large blocks: 1 when the output alone yields enough
// blocks to fill the chip; otherwise enough slices for about two blocks per
// compute unit.  Blocks of at most 64 rows (the skinny and wide classes) carry
// little work each and stream their large operand: at most 16 slices, and when
// B is read k-contiguous (B^T, rows of a few hundred bytes per k-tile) they
// aim at six blocks per compute unit even when the output alone fills the
// chip, since each block then sustains less bandwidth.  Every slice keeps at
// least four k-tiles.  bf16 blocks of more than 64 rows whose blocks at the M
// and N edges also take the direct loads (edges_direct: both operands have
// 16-byte-aligned rows, whose loads may run to the next 16 bytes past M or N
// when those lie along the rows) split only as far as
// one round of resident blocks and twelve k-tiles per slice allow: on 128 x
// 128 blocks at M, N of 1024-2048 (K 512-8192) a split that adds a round of
// blocks, or leaves shorter slices, costs more in partial sums and pipeline
// fill than it gains (1536^3: 30.3 us with the four slices of the two-blocks-
// per-CU target, 21.3 us unsplit).  forced > 0 overrides the target.
void plan_split(const TileConfig &c, int layout, int64_t M, int64_t N, int64_t K, int forced,
                int cus, int esize, bool edges_direct, int *splits, int *k_per_split)
{
    const int64_t target_blocks = 2 * (int64_t)cus, stream_blocks = 6 * (int64_t)cus;
    const int64_t tiles = ceil_div(M, c.bm) * ceil_div(N, c.bn);
    const int64_t ktiles = ceil_div(K, c.bk);
    const bool streaming = c.bm <= 64 && M <= 64;   // the skinny and wide classes
    const bool b_kcontig = layout == LAYOUT_NT || layout == LAYOUT_TT;
    int64_t s;
    if (forced > 0) {
        s = forced;
    } else if (tiles >= cus && !(streaming && b_kcontig)) {
        s = 1;
    } else if (esize == 2 && !streaming && edges_direct) {
        const int64_t lds = (int64_t)c.stages * (c.bm + c.bn) * c.bk * esize;
        const int64_t per_cu = std::max<int64_t>(1, kLdsBytes / lds);
        // 64-row blocks serve small outputs with K below 6144: unsplit
        s = c.bm <= 64 && ktiles < 96 ? 1 : std::min((int64_t)cus * per_cu / tiles, ktiles / 12);
    } else {
        s = ceil_div(streaming && b_kcontig ? stream_blocks : target_blocks, tiles);
        int64_t max_s = ktiles / 4;
        if (streaming && max_s > kMaxStreamSplits) max_s = kMaxStreamSplits;
        if (s > max_s) s = max_s;
    }
    if (s < 1) s = 1;
    if (s > ktiles) s = ktiles;
    const int64_t kps = ceil_div(ktiles, s) * c.bk;  // whole k-tiles per slice
    *k_per_split = (int)kps;
    *splits = (int)ceil_div(K, kps);                 // every slice non-empty
}

// Library-owned device buffers, one per (device, stream, slot), so that calls
// on different streams never share one: slot 0 holds split-K partial sums,
// slot 1 the convolution tables of the implicit GEMM, slot 2 its zero-padded
// image, slot 3 its filters with padded rows (or, for the filter gradient,
// the output gradient with padded rows), slot 4 that filter gradient with
// padded rows, slot 5 row-aligned copies of bf16 GEMM operands.  A buffer only grows, by at least half its size each time.
// The buffer it replaces is retired, not freed: a HIP graph captured earlier
// on that stream still holds its address, so it stays valid until the
// stream's buffers are released (gemm_release_buffers) or the library is
// unloaded.  Growth during stream capture would call hipMalloc inside the
// capture, so it is refused (GEMM_ERR_CAPTURING).
struct Workspace {
    void *ptr = nullptr;
    size_t bytes = 0;
    std::vector<void *> retired;
};
std::mutex g_ws_mutex;
std::map<std::tuple<int, hipStream_t, int>, Workspace> g_ws;

struct WorkspaceReleaser {
    ~WorkspaceReleaser()
    {
        // At unload the runtime may already be gone; freeing is best effort.
        for (auto &kv : g_ws) {
            if (kv.second.ptr) (void)hipFree(kv.second.ptr);
            for (void *p : kv.second.retired) (void)hipFree(p);
        }
    }
} g_ws_releaser;

// Whether work enqueued on `stream` is being captured into a graph.
bool capturing(hipStream_t stream)
{
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &st) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return st != hipStreamCaptureStatusNone;
}

int get_buffer(int slot, int device, hipStream_t stream, size_t bytes, void **out)
{
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace &w = g_ws[std::make_tuple(device, stream, slot)];
    if (w.bytes < bytes) {
        if (capturing(stream)) return GEMM_ERR_CAPTURING;
        const size_t want = bytes > w.bytes + w.bytes / 2 ? bytes : w.bytes + w.bytes / 2;
        void *p = nullptr;
        if (hipMalloc(&p, want) != hipSuccess) {
            (void)hipGetLastError();
            return GEMM_ERR_OUT_OF_MEMORY;
        }
        if (w.ptr) w.retired.push_back(w.ptr);
        w.ptr = p;
        w.bytes = want;
    }
    *out = w.ptr;
    return GEMM_OK;
}

// Frees every buffer (current and retired) of `stream` on the current device.
int release_buffers(hipStream_t stream)
{
    int device = -1;
    if (hipGetDevice(&device) != hipSuccess) {
        (void)hipGetLastError();
        return GEMM_ERR_NO_DEVICE;
    }
    if (capturing(stream)) return GEMM_ERR_CAPTURING;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    int rc = GEMM_OK;
    for (auto it = g_ws.begin(); it != g_ws.end();) {
        if (std::get<0>(it->first) == device && std::get<1>(it->first) == stream) {
            // hipFree waits for the device, so work still using a buffer is done
            if (it->second.ptr && hipFree(it->second.ptr) != hipSuccess) rc = GEMM_ERR_HIP;
            for (void *p : it->second.retired)
                if (hipFree(p) != hipSuccess) rc = GEMM_ERR_HIP;
            it = g_ws.erase(it);
        } else {
            ++it;
        }
    }
    if (rc != GEMM_OK) (void)hipGetLastError();
    return rc;
}

int get_workspace(int device, hipStream_t stream, size_t bytes, float **out)
{
    void *p = nullptr;
    const int rc = get_buffer(0, device, stream, bytes, &p);
    *out = static_cast<float *>(p);
    return rc;
}

int elem_size(int dtype) { return dtype == GEMM_DTYPE_F32 ? 4 : 2; }

bool valid_dtype(int dtype) { return dtype == GEMM_DTYPE_F32 || dtype == GEMM_DTYPE_BF16; }

using Call = GemmCall;

int check_args(const Call &c, bool with_c = true)
{
    if (!valid_dtype(c.dtype) || (with_c && !valid_dtype(c.dtype_c))) return GEMM_ERR_INVALID_ARG;
    if ((c.transa != GEMM_OP_N && c.transa != GEMM_OP_T) ||
        (c.transb != GEMM_OP_N && c.transb != GEMM_OP_T))
        return GEMM_ERR_INVALID_ARG;
    if (c.M < 0 || c.N < 0 || c.K < 0) return GEMM_ERR_INVALID_ARG;
    if (c.M > kMaxDim || c.N > kMaxDim || c.K > kMaxDim) return GEMM_ERR_INVALID_ARG;
    // Row lengths of the stored matrices: A is M x K (or K x M when
    // transposed), B is K x N (or N x K), C is M x N.
    const int64_t a_row = c.transa == GEMM_OP_T ? c.M : c.K;
    const int64_t b_row = c.transb == GEMM_OP_T ? c.K : c.N;
    const bool implicit = c.bsrc != B_MATRIX;
    if (implicit && (c.bsrc < B_CONV_FWD || c.bsrc > B_CONV4_WGRAD_PAD || c.conv == nullptr ||
                     c.transa != GEMM_OP_N ||
                     c.transb != (conv_fwd_source(c.bsrc) ? GEMM_OP_N : GEMM_OP_T) ||
                     (conv_table_source(c.bsrc) && c.conv->tab == nullptr)))
        return GEMM_ERR_INVALID_ARG;
    if (c.lda < (a_row > 0 ? a_row : 1) || (!implicit && c.ldb < (b_row > 0 ? b_row : 1)) ||
        (with_c && c.ldc < (c.N > 0 ? c.N : 1)))
        return GEMM_ERR_INVALID_ARG;
    if (with_c && c.M > 0 && c.N > 0 && c.C == nullptr) return GEMM_ERR_INVALID_ARG;
    if (c.M > 0 && c.N > 0 && c.K > 0 && (c.A == nullptr || c.B == nullptr))
        return GEMM_ERR_INVALID_ARG;
    const uintptr_t esz = (uintptr_t)elem_size(c.dtype);
    if ((uintptr_t)c.A % esz || (uintptr_t)c.B % esz ||
        (with_c && (uintptr_t)c.C % (uintptr_t)elem_size(c.dtype_c)))
        return GEMM_ERR_INVALID_ARG;
    return GEMM_OK;
}

// Fixed split-K scratch of gemm_ex_noalloc: one array per GPU (every GPU the
// library runs on holds its own copy until the process ends), for callers
// that cannot allocate.  Host code never passes the array's name to a kernel
// (on the host it is only a stand-in for the symbol): the device address of
// each GPU's copy is looked up once, with that GPU current, and kept.  The
// partial sums need no clearing: every slice writes all of its M x N values
// before the reduce reads them.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

// Device address of `device`'s scratch array (the current device).
int scratch_address(int device, void **out)
{
    if (device < 0 || device >= kMaxDevices) return GEMM_ERR_NO_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[device] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return GEMM_ERR_HIP;
        }
        g_scratch_ptr[device] = p;
    }
    *out = g_scratch_ptr[device];
    return GEMM_OK;
}

// bf16 operands whose rows are not all 4-byte aligned (an odd leading
// dimension, a 2-byte-aligned address, or pairs along an odd outer extent)
// take neither direct load in the kernels: every k-tile goes through
// registers, at a third to a half of the aligned rate.  When the product has
// enough work per byte of the operands whose rows are not 16-byte aligned,
// those are first copied into a library buffer with 16-byte-aligned rows
// (one pass over each at HBM speed) and the product runs on the copies.
// Copying costs an operand's bytes twice in HBM traffic plus a launch, and
// saves time in proportion to the K loop's share of the call; operands read
// outer-contiguous (B, A^T) lose more in place than k-contiguous ones.
// Measured on MI355X against the in-place call: copying a k-contiguous
// operand won from about 190 flops per copied byte (8191 x 192 x 8191, A
// copied: 140 -> 107 us) and lost 9-16% at 128; copying an outer-contiguous
// one won already at 64 (64 x 8191 x 8191, B copied: 115 -> 89 us); with K
// of 255 or less, where writing C dominates, copying lost up to 7%.  So the
// product must do 160 flops per copied byte of a k-contiguous operand plus
// 56 per copied byte of an outer-contiguous one.  Returns whether it
// enqueued copies (then *out is the call on them); a buffer that cannot grow
// (stream capture, out of memory) leaves the call in place.
constexpr double kStageFlopsPerByteK = 160.0;
constexpr double kStageFlopsPerByteOuter = 56.0;
constexpr double kStageMinFlops = double(1 << 26);
constexpr int64_t kStageMinK = 256;
constexpr int64_t kStageAlign = 256;

// Which operands to copy and where: A at the buffer's start, B after it.
struct StagePlan {
    bool a = false, b = false;                 // copy A / B
    bool a_outer = false, b_outer = false;     // stored with M (A^T) / N (B) along rows
    int64_t a_rows = 0, a_cols = 0, a_ld = 0, a_bytes = 0;
    int64_t b_rows = 0, b_cols = 0, b_ld = 0, b_bytes = 0;
};

bool plan_stage(const Call &call, int layout, StagePlan *sp)
{
    if (call.dtype != GEMM_DTYPE_BF16 || call.bsrc != B_MATRIX) return false;
    sp->a_outer = layout == LAYOUT_TN || layout == LAYOUT_TT;
    sp->b_outer = layout == LAYOUT_NN || layout == LAYOUT_TN;
    const bool pairs = ((call.lda | call.ldb) & 1) == 0 &&
                       (((uintptr_t)call.A | (uintptr_t)call.B) & 3) == 0 &&
                       (!sp->a_outer || (call.M & 1) == 0) && (!sp->b_outer || (call.N & 1) == 0);
    const bool a16 = call.lda % 8 == 0 && (uintptr_t)call.A % 16 == 0;
    const bool b16 = call.ldb % 8 == 0 && (uintptr_t)call.B % 16 == 0;
    if (pairs || (a16 && b16)) return false;
    sp->a = !a16;
    sp->b = !b16;
    // stored shapes: A is M x K (K x M transposed), B is K x N (N x K)
    sp->a_rows = call.transa == GEMM_OP_T ? call.K : call.M;
    sp->a_cols = call.transa == GEMM_OP_T ? call.M : call.K;
    sp->b_rows = call.transb == GEMM_OP_T ? call.N : call.K;
    sp->b_cols = call.transb == GEMM_OP_T ? call.K : call.N;
    sp->a_ld = (sp->a_cols + 7) / 8 * 8;
    sp->b_ld = (sp->b_cols + 7) / 8 * 8;
    sp->a_bytes = sp->a ? (sp->a_rows * sp->a_ld * 2 + kStageAlign - 1) / kStageAlign * kStageAlign : 0;
    sp->b_bytes = sp->b ? sp->b_rows * sp->b_ld * 2 : 0;
    const double flops = 2.0 * (double)call.M * (double)call.N * (double)call.K;
    const double need = (sp->a_outer ? kStageFlopsPerByteOuter : kStageFlopsPerByteK) * sp->a_bytes +
                        (sp->b_outer ? kStageFlopsPerByteOuter : kStageFlopsPerByteK) * sp->b_bytes;
    return call.K >= kStageMinK && flops >= kStageMinFlops && flops >= need;
}

bool stage_operands(const Call &call, int layout, int device, hipStream_t stream, Call *out,
                    int *rc)
{
    *rc = GEMM_OK;
    StagePlan sp;
    if (!plan_stage(call, layout, &sp)) return false;
    void *buf = nullptr;
    if (get_buffer(5, device, stream, (size_t)(sp.a_bytes + sp.b_bytes), &buf) != GEMM_OK)
        return false;
    *out = call;
    if (sp.a) {
        if (launch_stage_rows(call.A, call.lda, sp.a_rows, sp.a_cols, 2, buf, sp.a_ld, stream) !=
            hipSuccess) {
            *rc = GEMM_ERR_HIP;
            return true;
        }
        out->A = buf;
        out->lda = sp.a_ld;
    }
    if (sp.b) {
        void *bb = static_cast<char *>(buf) + sp.a_bytes;
        if (launch_stage_rows(call.B, call.ldb, sp.b_rows, sp.b_cols, 2, bb, sp.b_ld, stream) !=
            hipSuccess) {
            *rc = GEMM_ERR_HIP;
            return true;
        }
        out->B = bb;
        out->ldb = sp.b_ld;
    }
    return true;
}

// Where a call's split-K partial sums go: the library's per-(device, stream)
// buffer, grown with hipMalloc on demand, or (no_alloc) the fixed per-device
// scratch array below, never allocating.
int run_call(const Call &call, int forced_cfg, int forced_split, hipStream_t stream,
             bool no_alloc = false)
{
    int rc = check_args(call);
    if (rc != GEMM_OK) return rc;
    int count = 0;
    const TileConfig *tab = table(call.dtype, &count);
    if (tab == nullptr) return GEMM_ERR_INVALID_ARG;
    if (forced_cfg >= count) return GEMM_ERR_INVALID_ARG;
    const int layout = call.transa * 2 + call.transb;
    const int impl = call.bsrc - B_CONV_FWD;  // implicit slot, for bsrc != B_MATRIX
    auto kernel_of = [&](const TileConfig &t, bool aligned) -> launch_fn {
        return call.bsrc == B_MATRIX ? t.fn[layout][aligned ? 0 : 1]
                                     : t.implicit[impl][aligned ? 0 : 1];
    };
    if (forced_cfg >= 0 && kernel_of(tab[forced_cfg], true) == nullptr) return GEMM_ERR_INVALID_ARG;
    const int64_t M = call.M, N = call.N, K = call.K;
    if (M == 0 || N == 0) return GEMM_OK;

    int device = -1;
    if (hipGetDevice(&device) != hipSuccess) {
        (void)hipGetLastError();
        return GEMM_ERR_NO_DEVICE;
    }
    const int out_bf16 = call.dtype_c == GEMM_DTYPE_BF16;
    // The product term vanishes (empty sum, or alpha == 0): A and B are not
    // read and C := beta * C.
    if (K == 0 || call.alpha == 0.0f)
        return launch_scale((int)M, (int)N, call.C, call.ldc, call.beta, out_bf16, stream) ==
                       hipSuccess
                   ? GEMM_OK
                   : GEMM_ERR_HIP;

    const int cus = compute_units();
    const int ci = forced_cfg >= 0             ? forced_cfg
                   : call.bsrc != B_MATRIX ? select_implicit(call.dtype, M)
                                           : select_config(call.dtype, layout, M, N, K, cus);
    if (ci < 0) return GEMM_ERR_INTERNAL;
    const TileConfig &cfg = tab[ci];
    if (kernel_of(cfg, true) == nullptr) return GEMM_ERR_INVALID_ARG;

    // bf16 operands with rows below 4-byte alignment: row-aligned copies
    // (dispatcher's choice only; a forced entry runs on the operands as given)
    if (forced_cfg < 0 && call.bsrc == B_MATRIX && !no_alloc) {
        Call staged;
        if (stage_operands(call, layout, device, stream, &staged, &rc))
            return rc != GEMM_OK ? rc : run_call(staged, -1, 0, stream, false);
    }
    // Outer extents the loads may read.  An operand stored with M (A^T) or N
    // (B) along 16-byte-aligned rows is loaded in whole 16-byte chunks up to
    // the next multiple of 16 bytes: each such chunk holds an element of its
    // row, so it lies within the row's pitch or, in the last row, on the page
    // of that element; the values past M or N feed only outputs that are
    // never stored.  So the blocks at that edge keep the direct loads.
    const int esize = (int)elem_size(call.dtype);
    const int vec = 16 / esize;
    const bool a_rows16 = call.lda % vec == 0 && (uintptr_t)call.A % 16 == 0;
    const bool b_rows16 = call.bsrc == B_MATRIX && call.ldb % vec == 0 && (uintptr_t)call.B % 16 == 0;
    const int64_t m_load = call.transa == GEMM_OP_T && a_rows16 ? ceil_div(M, vec) * vec : M;
    const int64_t n_load = call.transb == GEMM_OP_N && b_rows16 ? ceil_div(N, vec) * vec : N;
    int splits = 1, kps = 0;
    plan_split(cfg, layout, M, N, K, forced_split, cus, esize, a_rows16 && b_rows16, &splits, &kps);

    // Thin remainders (dispatcher's choice only; a forced entry runs as asked):
    // when the last block row or column would hold at most an eighth of a
    // block and leaving it out saves a round of blocks over the chip, the
    // full blocks run as one product and the remainder strips as products of
    // their own (rows M' .. M-1 with all columns, then columns N' .. N-1 of
    // rows 0 .. M'-1), each dispatched for its shape.  The strips write
    // disjoint parts of C, so alpha and beta apply to each as to the whole.
    if (forced_cfg < 0 && call.bsrc == B_MATRIX && splits == 1) {
        const int64_t Mm = main_extent(M, cfg.bm), Nm = main_extent(N, cfg.bn);
        const int64_t slots = (int64_t)cus;  // blocks of the large entries: one per CU
        const int64_t full = ceil_div(M, cfg.bm) * ceil_div(N, cfg.bn);
        const int64_t main = ceil_div(Mm, cfg.bm) * ceil_div(Nm, cfg.bn);
        if ((Mm < M || Nm < N) && ceil_div(main, slots) < ceil_div(full, slots)) {
            const int64_t esz_ab = elem_size(call.dtype), esz_c = elem_size(call.dtype_c);
            auto at = [](const void *p, int64_t elems, int64_t esz) {
                return static_cast<const void *>(static_cast<const char *>(p) + elems * esz);
            };
            Call part = call;
            part.M = Mm;
            part.N = Nm;
            rc = run_call(part, ci, 0, stream, no_alloc);
            if (rc != GEMM_OK) return rc;
            if (Mm < M) {
                Call rows = call;
                rows.M = M - Mm;
                rows.A = at(call.A, call.transa == GEMM_OP_T ? Mm : Mm * call.lda, esz_ab);
                rows.C = const_cast<void *>(at(call.C, Mm * call.ldc, esz_c));
                rc = run_call(rows, -1, 0, stream, no_alloc);
                if (rc != GEMM_OK) return rc;
            }
            if (Nm < N) {
                Call cols = call;
                cols.M = Mm;
                cols.N = N - Nm;
                cols.B = at(call.B, call.transb == GEMM_OP_T ? Nm * call.ldb : Nm, esz_ab);
                cols.C = const_cast<void *>(at(call.C, Nm, esz_c));
                rc = run_call(cols, -1, 0, stream, no_alloc);
            }
            return rc;
        }
    }

    KernelArgs a{};
    a.A = call.A;
    a.B = call.B;
    a.C = call.C;
    a.ws = nullptr;
    a.lda = call.lda;
    a.ldb = call.ldb;
    a.ldc = call.ldc;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.m_load = (int)m_load;
    a.n_load = (int)n_load;
    a.tiles_m = (int)ceil_div(M, cfg.bm);
    a.tiles_n = (int)ceil_div(N, cfg.bn);
    a.splits = splits;
    a.k_per_split = kps;
    a.group_m = cfg.group_m;
    a.alpha = call.alpha;
    a.beta = call.beta;
    a.out_bf16 = out_bf16;
    if (splits > 1) {
        const size_t need = (size_t)splits * (size_t)M * (size_t)N * sizeof(float);
        if (no_alloc) {
            if (need > kScratchBytes) return GEMM_ERR_SCRATCH_LIMIT;
            rc = scratch_address(device, reinterpret_cast<void **>(&a.ws));
        } else {
            rc = get_workspace(device, stream, need, &a.ws);
        }
        if (rc != GEMM_OK) return rc;
    }

    const int64_t esz = esize;
    // (an implicit B is gathered element by element: only A's alignment counts)
    const bool aligned = a_rows16 && (call.bsrc != B_MATRIX || b_rows16);
    // The direct-load path addresses a tile with per-thread 32-bit byte
    // offsets from the tile origin, over the tile's memory rows: BM (A as
    // given) or BK (A transposed) rows of A, BK (B as given) or BN (B
    // transposed) rows of B.
    const int64_t a_rows = call.transa == GEMM_OP_T ? cfg.bk : cfg.bm;
    const int64_t b_rows = call.transb == GEMM_OP_T ? cfg.bn : cfg.bk;
    a.direct_ok = (a_rows * call.lda * esz < (int64_t(1) << 32)) &&
                  (b_rows * call.ldb * esz < (int64_t(1) << 32));
    if (call.bsrc != B_MATRIX) {
        a.conv = *call.conv;
        a.direct_ok = 0;
    }
    const int64_t blocks = (int64_t)splits * a.tiles_m * a.tiles_n;
    if (blocks > INT32_MAX) return GEMM_ERR_INVALID_ARG;
    launch_fn fn = kernel_of(cfg, aligned);
    if (fn(a, (int)blocks, stream) != hipSuccess) return GEMM_ERR_HIP;
    if (splits > 1 && launch_splitk_reduce(a.ws, splits, (int)M, (int)N, call.C, call.ldc,
                                           call.alpha, call.beta, out_bf16, stream) != hipSuccess)
        return GEMM_ERR_HIP;
    return GEMM_OK;
}

// The plain product C := A . B with fp32 C.
Call plain_call(int dtype, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                const void *B, int64_t ldb, float *C, int64_t ldc)
{
    return Call{dtype, GEMM_DTYPE_F32, GEMM_OP_N, GEMM_OP_N, M, N, K, 1.0f, 0.0f,
                A, lda, B, ldb, C, ldc};
}

}  // namespace

int gemm_run(const GemmCall &call, int forced_cfg, int forced_split, hipStream_t stream)
{
    return run_call(call, forced_cfg, forced_split, stream);
}

int conv_table_buffer(hipStream_t stream, size_t bytes, void **out)
{
    int device = -1;
    if (hipGetDevice(&device) != hipSuccess) {
        (void)hipGetLastError();
        return GEMM_ERR_NO_DEVICE;
    }
    return get_buffer(1, device, stream, bytes, out);
}

int conv_padded_buffer(hipStream_t stream, size_t bytes, void **out)
{
    int device = -1;
    if (hipGetDevice(&device) != hipSuccess) {
        (void)hipGetLastError();
        return GEMM_ERR_NO_DEVICE;
    }
    return get_buffer(2, device, stream, bytes, out);
}

int conv_filter_buffer(hipStream_t stream, size_t bytes, void **out)
{
    int device = -1;
    if (hipGetDevice(&device) != hipSuccess) {
        (void)hipGetLastError();
        return GEMM_ERR_NO_DEVICE;
    }
    return get_buffer(3, device, stream, bytes, out);
}

int conv_result_buffer(hipStream_t stream, size_t bytes, void **out)
{
    int device = -1;
    if (hipGetDevice(&device) != hipSuccess) {
        (void)hipGetLastError();
        return GEMM_ERR_NO_DEVICE;
    }
    return get_buffer(4, device, stream, bytes, out);
}

int implicit_tile(int dtype, int64_t M, int *bn, int *bk, int *threads)
{
    int count = 0;
    const TileConfig *tab = table(dtype, &count);
    const int ci = tab ? select_implicit(dtype, M) : -1;
    if (ci < 0) return GEMM_ERR_INTERNAL;
    *bn = tab[ci].bn;
    *bk = tab[ci].bk;
    *threads = tab[ci].threads;
    return GEMM_OK;
}

}  // namespace dg

extern "C" {

int gemm_f32(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
             int64_t ldb, float *C, int64_t ldc, hipStream_t stream)
{
    return dg::gemm_run(dg::plain_call(GEMM_DTYPE_F32, M, N, K, A, lda, B, ldb, C, ldc), -1, 0, stream);
}

int gemm_bf16(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda, const uint16_t *B,
              int64_t ldb, float *C, int64_t ldc, hipStream_t stream)
{
    return dg::gemm_run(dg::plain_call(GEMM_DTYPE_BF16, M, N, K, A, lda, B, ldb, C, ldc), -1, 0, stream);
}

int gemm_f32_with_config(int cfg, int split_k, int64_t M, int64_t N, int64_t K, const float *A,
                         int64_t lda, const float *B, int64_t ldb, float *C, int64_t ldc,
                         hipStream_t stream)
{
    if (cfg < 0) return GEMM_ERR_INVALID_ARG;
    return dg::gemm_run(dg::plain_call(GEMM_DTYPE_F32, M, N, K, A, lda, B, ldb, C, ldc), cfg, split_k,
                   stream);
}

int gemm_bf16_with_config(int cfg, int split_k, int64_t M, int64_t N, int64_t K,
                          const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                          float *C, int64_t ldc, hipStream_t stream)
{
    if (cfg < 0) return GEMM_ERR_INVALID_ARG;
    return dg::gemm_run(dg::plain_call(GEMM_DTYPE_BF16, M, N, K, A, lda, B, ldb, C, ldc), cfg, split_k,
                   stream);
}

int gemm_ex(int dtype_ab, int dtype_c, int transa, int transb, int64_t M, int64_t N, int64_t K,
            float alpha, const void *A, int64_t lda, const void *B, int64_t ldb, float beta,
            void *C, int64_t ldc, hipStream_t stream)
{
    return dg::gemm_run(dg::Call{dtype_ab, dtype_c, transa, transb, M, N, K, alpha, beta, A, lda, B,
                            ldb, C, ldc},
                   -1, 0, stream);
}

int gemm_ex_noalloc(int dtype_ab, int dtype_c, int transa, int transb, int64_t M, int64_t N,
                    int64_t K, float alpha, const void *A, int64_t lda, const void *B,
                    int64_t ldb, float beta, void *C, int64_t ldc, hipStream_t stream)
{
    return dg::run_call(dg::Call{dtype_ab, dtype_c, transa, transb, M, N, K, alpha, beta, A, lda, B,
                                 ldb, C, ldc},
                        -1, 0, stream, true);
}

int gemm_ex_with_config(int cfg, int split_k, int dtype_ab, int dtype_c, int transa, int transb,
                        int64_t M, int64_t N, int64_t K, float alpha, const void *A, int64_t lda,
                        const void *B, int64_t ldb, float beta, void *C, int64_t ldc,
                        hipStream_t stream)
{
    if (cfg < 0) return GEMM_ERR_INVALID_ARG;
    return dg::gemm_run(dg::Call{dtype_ab, dtype_c, transa, transb, M, N, K, alpha, beta, A, lda, B,
                            ldb, C, ldc},
                   cfg, split_k, stream);
}

int gemm_release_buffers(hipStream_t stream) { return dg::release_buffers(stream); }

int gemm_config_layouts(int dtype, int cfg)
{
    int count = 0;
    const dg::TileConfig *tab = dg::table(dtype, &count);
    if (!tab || cfg < 0 || cfg >= count) return GEMM_ERR_INVALID_ARG;
    int mask = 0;
    for (int l = 0; l < 4; ++l)
        if (tab[cfg].fn[l][0] != nullptr) mask |= 1 << l;
    return mask;
}

const char *gemm_status_string(int status)
{
    switch (status) {
    case GEMM_OK: return "success";
    case GEMM_ERR_INVALID_ARG: return "invalid argument";
    case GEMM_ERR_HIP: return "HIP runtime error";
    case GEMM_ERR_NO_DEVICE: return "no HIP device";
    case GEMM_ERR_OUT_OF_MEMORY: return "out of device memory";
    case GEMM_ERR_INTERNAL: return "internal error: a tile-table entry the dispatcher names is missing";
    case GEMM_ERR_SCRATCH_LIMIT:
        return "the call needs more split-K scratch than the fixed array of gemm_ex_noalloc holds";
    case GEMM_ERR_CAPTURING:
        return "a library buffer must grow while the stream is being captured into a graph "
               "(run the call once on this stream before capturing)";
    default: return "unknown status";
    }
}

int gemm_num_configs(int dtype)
{
    int count = 0;
    return dg::table(dtype, &count) ? count : GEMM_ERR_INVALID_ARG;
}

int gemm_select_config(int dtype, int64_t M, int64_t N, int64_t K)
{
    int count = 0;
    if (!dg::table(dtype, &count) || M < 0 || N < 0 || K < 0) return GEMM_ERR_INVALID_ARG;
    const int ci = dg::select_config(dtype, dg::LAYOUT_NN, M, N, K, dg::compute_units());
    return ci < 0 ? GEMM_ERR_INTERNAL : ci;
}

int gemm_select_config_ex(int dtype, int transa, int transb, int64_t M, int64_t N, int64_t K)
{
    int count = 0;
    if (!dg::table(dtype, &count) || M < 0 || N < 0 || K < 0 ||
        (transa != GEMM_OP_N && transa != GEMM_OP_T) || (transb != GEMM_OP_N && transb != GEMM_OP_T))
        return GEMM_ERR_INVALID_ARG;
    const int ci = dg::select_config(dtype, transa * 2 + transb, M, N, K, dg::compute_units());
    return ci < 0 ? GEMM_ERR_INTERNAL : ci;
}

const char *gemm_config_name(int dtype, int cfg)
{
    int count = 0;
    const dg::TileConfig *tab = dg::table(dtype, &count);
    if (!tab || cfg < 0 || cfg >= count) return nullptr;
    return tab[cfg].name;
}

int gemm_split_k(int dtype, int cfg, int64_t M, int64_t N, int64_t K)
{
    int count = 0;
    const dg::TileConfig *tab = dg::table(dtype, &count);
    if (!tab || cfg < 0 || cfg >= count || M < 0 || N < 0 || K < 0) return GEMM_ERR_INVALID_ARG;
    if (M == 0 || N == 0 || K == 0) return 1;
    int splits = 1, kps = 0;
    const int es = dtype == GEMM_DTYPE_BF16 ? 2 : 4;
    dg::plan_split(tab[cfg], dg::LAYOUT_NN, M, N, K, 0, dg::compute_units(), es,
                   true, &splits, &kps);
    return splits;
}

int gemm_split_k_ex(int dtype, int cfg, int transa, int transb, int64_t M, int64_t N, int64_t K)
{
    int count = 0;
    const dg::TileConfig *tab = dg::table(dtype, &count);
    if (!tab || cfg < 0 || cfg >= count || M < 0 || N < 0 || K < 0 ||
        (transa != GEMM_OP_N && transa != GEMM_OP_T) || (transb != GEMM_OP_N && transb != GEMM_OP_T))
        return GEMM_ERR_INVALID_ARG;
    if (M == 0 || N == 0 || K == 0) return 1;
    int splits = 1, kps = 0;
    const int es = dtype == GEMM_DTYPE_BF16 ? 2 : 4;
    dg::plan_split(tab[cfg], transa * 2 + transb, M, N, K, 0, dg::compute_units(), es,
                   true, &splits, &kps);
    return splits;
}

int64_t gemm_operand_copy_bytes(int dtype_ab, int transa, int transb, int64_t M, int64_t N,
                                int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb)
{
    const dg::GemmCall call{dtype_ab, dtype_ab, transa, transb, M, N, K, 1.0f, 0.0f,
                            A, lda, B, ldb, nullptr, 0};
    if (dg::check_args(call, false) != GEMM_OK) return GEMM_ERR_INVALID_ARG;
    if (M == 0 || N == 0 || K == 0) return 0;
    dg::StagePlan sp;
    return dg::plan_stage(call, transa * 2 + transb, &sp) ? sp.a_bytes + sp.b_bytes : 0;
}

}  // extern "C"
