// tc_internal.h -- definitions shared by the host planner (tcgemm.cpp) and
// the gfx950 kernels (gemm_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tcg {

// Element type codes; identical to tc_dtype_t in include/tcgemm.h.
enum Dt : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_I8 = 3, DT_I32 = 4 };

__host__ __device__ constexpr int dt_size(int dt) {
    return dt == DT_F32 ? 4 : dt == DT_I32 ? 4 : dt == DT_I8 ? 1 : 2;
}

// Tile classes.  Every class keeps one LDS row of an operand tile at 128
// bytes of K (64 bf16/f16, 128 int8, 32 f32), so the swizzle and the MFMA
// fragment reads are the same for every element type.  TILE_256_DMA is the
// 256x256 tile of gemm_dma_kernel (direct-to-LDS loads; 16-bit and int8
// inputs with 16-byte aligned rows) with 4 waves of 128x128, TILE_256_DMA8
// the same with 8 waves of 128x64 (two per SIMD), TILE_128_DMA its 128x128
// tile with 4 waves of 64x64 and two workgroups per CU, TILE_128_DMA4 the
// same tile with one workgroup per CU and 4 LDS stages (three K-tiles in
// flight: split-K slices, whose short loops are bound by load latency).
// TILE_256_DMA keeps its operand tiles in a ring of five slots (all 160 KiB
// of LDS; half of each K-tile's loads in each of its two sub-steps).
// TILE_64_KS, TILE_32_KS and TILE_16_KS are 64x64, 32x32 and 16x16 tiles
// whose 4 waves split K among themselves (every wave owns the whole tile and
// takes every 4th K-tile; the four partial tiles are added in LDS): small
// problems with few tiles and a short K.
enum TileClass : int {
    TILE_256 = 0,
    TILE_128 = 1,
    TILE_64 = 2,
    TILE_256_DMA = 3,
    TILE_256_DMA8 = 4,
    TILE_128_DMA = 5,
    TILE_THIN = 6,          // thin_kernel: N <= 16, A K-contiguous; kThinRows rows per workgroup
    TILE_128_DMA4 = 7,
    TILE_64_KS = 8,
    TILE_32_KS = 9,
    TILE_16_KS = 10,
    NUM_TILE_CLASSES = 11
};

__host__ __device__ constexpr bool is_ks_class(int cls) {
    return cls == TILE_64_KS || cls == TILE_32_KS || cls == TILE_16_KS;
}

constexpr int kThinRows = 8;    // output rows per thin_kernel workgroup (2 waves)

__host__ __device__ constexpr bool is_dma_class(int cls) {
    return cls == TILE_256_DMA || cls == TILE_256_DMA8 || cls == TILE_128_DMA ||
           cls == TILE_128_DMA4;
}

__host__ __device__ constexpr int tile_threads(int cls) { return cls == TILE_256_DMA8 ? 512 : 256; }

struct TileShape {
    int bm, bn, wm, wn;   // tile rows/cols, waves along m/n (4 waves = 256 threads)
};

__host__ __device__ constexpr TileShape tile_shape(int cls) {
    return (cls == TILE_256 || cls == TILE_256_DMA || cls == TILE_256_DMA8)
               ? TileShape{256, 256, 2, 2}
         : (cls == TILE_128 || cls == TILE_128_DMA || cls == TILE_128_DMA4) ? TileShape{128, 128, 2, 2}
         : cls == TILE_THIN                         ? TileShape{kThinRows, 16, kThinRows / 4, 1}
         : cls == TILE_64_KS                        ? TileShape{64, 64, 1, 1}
         : cls == TILE_32_KS                        ? TileShape{32, 32, 1, 1}
         : cls == TILE_16_KS                        ? TileShape{16, 16, 1, 1}
                                                    : TileShape{64, 64, 2, 2};
}

constexpr int kLdsRowBytes = 128;      // bytes of K per LDS tile row
constexpr int kXcds = 8;               // MI355X: 8 XCDs x 32 CUs

// Size of the static scratch array of the allocation-free entry point, and
// the devices whose addresses of it are cached.
constexpr int64_t kStaticScratchBytes = 32ll << 20;
constexpr int kMaxDevices = 64;

// Output selector of the GEMM kernel beyond the element types: raw partial
// sums of one split-K slice (fp32, or int32 for int8 inputs).
constexpr int OUT_PARTIAL = 5;

// Fused-epilogue activations (tessl "Architecture", "Fused Epilogue").
constexpr int ACT_NONE = 0, ACT_RELU = 1, ACT_GELU_TANH = 2;

// Everything a GEMM launch needs; passed by value as the kernel argument.
struct GemmArgs {
    const void *A;
    const void *B;
    void *C;
    void *ws;                  // split-K partials [batch][splits][M][N] (4-byte elements)
    int64_t stride_a, stride_b, stride_c;   // elements between batch problems
    int64_t a_extent, b_extent, c_extent;   // bytes spanned by one problem's operand
    int32_t M, N, K;
    int32_t lda, ldb, ldc;     // elements
    int32_t c_dtype;
    float alpha, beta;
    int32_t tiles_m, tiles_n;
    int32_t splits, k_per_split;   // k_per_split is a multiple of the tile K
    int32_t groups;                // batch * splits
    int32_t band;                  // tile-order band height (<= 0: row-major)
    int32_t c_vec_ok;              // 4 complete C values go as one vector access
    int32_t c_dma_ok;              // C rows, batch stride and base are whole 16-byte chunks
    // fused epilogue: out = act(alpha*scale[n]*acc + beta*C_old + bias[n])
    const void *bias;              // N values of c_dtype per problem, or null
    int64_t bias_stride;           // elements between the problems' bias vectors
    const float *scale;            // N per-column fp32 scales per problem, or null
    int64_t scale_stride;          // elements between the problems' scale vectors
    int32_t act;                   // ACT_*
    int32_t epi;                   // bias or scale != null || act != ACT_NONE
    // thin kernel only: output (r, c) of this problem is C[c * ldc + r] (the
    // transposed product of a small-M GEMM); bias and scales then go by r
    int32_t c_trans;
};

// Arguments of the split-K reduction and of the alpha == 0 scaling kernel.
struct EpilogueArgs {
    const void *ws;
    void *C;
    int64_t stride_c;
    int64_t c_extent;
    int32_t M, N, ldc;
    int32_t batch, splits;
    int32_t c_dtype;
    int32_t acc_is_int;
    int32_t c_vec_ok;          // 4 complete C values go as one vector access
    float alpha, beta;
    const void *bias;          // fused epilogue, as in GemmArgs
    int64_t bias_stride;
    const float *scale;
    int64_t scale_stride;
    int32_t act, epi;
};

// Operand repacking: `rows` rows of `row_bytes` bytes, read at pitch
// src_pitch and written at pitch dst_pitch (a multiple of 16, >= row_bytes)
// with the bytes from row_bytes to dst_pitch zeroed, for `batch` problems.
struct PackArgs {
    const void *src;
    void *dst;
    int64_t src_stride, dst_stride;   // bytes between batch problems
    int64_t src_pitch, dst_pitch;     // bytes between rows
    int32_t rows, row_bytes, batch;
    // row packing only, optional (bt == null: none): the bt_cols elements
    // of bt_es bytes that follow each source row's row_bytes, transposed --
    // element n of row r goes to bt[n * bt_pitch + r * bt_es] (the B^T of a
    // thin column strip right after the packed columns)
    void *bt;
    int64_t bt_stride;                // bytes between batch problems
    int32_t bt_pitch, bt_cols, bt_es;
};

// Workgroup -> (tile_m, tile_n, group).
//
// Step 1, XCD regrouping: the hardware hands consecutive workgroup ids to the
// 8 XCDs in turn, so XCD x runs ids x, x+8, x+16, ...  Those are renumbered to
// one contiguous range of logical ids per XCD (a bijection also when n_wg is
// not a multiple of 8), so that the tiles one XCD runs together share operand
// panels in that XCD's L2.
//
// Step 2, group: logical ids are group-major (group = batch element x split
// slice), so one XCD's range stays inside one problem where it can.
//
// Step 3, band order inside a group (tessl "Architecture", "Column-Panel Grid
// Swizzling"): the tile rows are grouped into horizontal bands of `band`
// rows (the last band keeps whatever rows remain), the bands are visited top
// to bottom, and each band is visited in column-major order -- down one tile
// column of the band, then the next column to the right.  A run of
// consecutive ids then touches few B column panels and few A row panels.
// Every band above the one holding id t is full, so t's band is
// t / (band * tiles_n) and t's position inside it the remainder; in a band of
// h rows, position o is tile column o / h and row o % h of the band.
__host__ __device__ inline void tile_of_workgroup(int32_t tiles_m, int32_t tiles_n,
                                                  int32_t band, int64_t wg, int64_t n_wg,
                                                  int32_t *tm, int32_t *tn, int32_t *g) {
    int64_t q = n_wg / kXcds, r = n_wg % kXcds;
    int64_t xcd = wg % kXcds, j = wg / kXcds;
    int64_t logical = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + j;
    int64_t tiles = (int64_t)tiles_m * tiles_n;
    int64_t t = logical % tiles;
    *g = (int32_t)(logical / tiles);
    if (band <= 0) {
        *tm = (int32_t)(t / tiles_n);
        *tn = (int32_t)(t % tiles_n);
        return;
    }
    // (this exact arithmetic keeps the kernels' compile time low: equivalent
    // rewrites of it made each GEMM object compile three times slower)
    int64_t per_band = (int64_t)band * tiles_n;
    int64_t b = t / per_band;
    int64_t rem = t - b * per_band;
    int64_t h = tiles_m - b * band;
    if (h > band) h = band;
    *tm = (int32_t)(b * band + rem % h);
    *tn = (int32_t)(rem / h);
}

}  // namespace tcg

// Launchers (epilogue_kernels.hip and gemm_inst.hip).  They return
// hipSuccess or the launch error; hipErrorInvalidValue for a combination
// that has no instantiation.  `cls` is a TileClass, `dt` the input Dt, `out`
// the output Dt or OUT_PARTIAL.
hipError_t tcg_launch_gemm(int dt, bool ta, bool tb, int cls, int out, const tcg::GemmArgs &args,
                           int64_t grid, hipStream_t stream);
hipError_t tcg_launch_splitk_reduce(const tcg::EpilogueArgs &args, hipStream_t stream);
hipError_t tcg_launch_scale_c(const tcg::EpilogueArgs &args, hipStream_t stream);
hipError_t tcg_launch_pack_rows(const tcg::PackArgs &args, hipStream_t stream);
// B stored [N, K] (K-contiguous rows)
hipError_t tcg_launch_thin(int dt, int out, const tcg::GemmArgs &args, int64_t grid, hipStream_t stream);
// rows = K, row_bytes = N * es of a B stored [K, N]; writes Bt[n][k] rows of
// dst_pitch bytes
hipError_t tcg_launch_thin_pack_bt(const tcg::PackArgs &args, int es, hipStream_t stream);
const char *tcg_kernel_name(int dt, bool ta, bool tb, int cls);
// Device address of the static scratch array (kStaticScratchBytes) on
// `device`, which must be the current device; looked up once per device.
hipError_t tcg_static_scratch(int device, void **ptr);

// One launcher per (input type, layout) object; each dispatches on (cls, out).
#define TCG_DECLARE_LAUNCHER(NAME)                                                       \
    hipError_t NAME(int cls, int out, const tcg::GemmArgs &args, int64_t grid,           \
                    hipStream_t stream);
TCG_DECLARE_LAUNCHER(tcg_launch_f32_nn) TCG_DECLARE_LAUNCHER(tcg_launch_f32_nt)
TCG_DECLARE_LAUNCHER(tcg_launch_f32_tn) TCG_DECLARE_LAUNCHER(tcg_launch_f32_tt)
TCG_DECLARE_LAUNCHER(tcg_launch_f16_nn) TCG_DECLARE_LAUNCHER(tcg_launch_f16_nt)
TCG_DECLARE_LAUNCHER(tcg_launch_f16_tn) TCG_DECLARE_LAUNCHER(tcg_launch_f16_tt)
TCG_DECLARE_LAUNCHER(tcg_launch_bf16_nn) TCG_DECLARE_LAUNCHER(tcg_launch_bf16_nt)
TCG_DECLARE_LAUNCHER(tcg_launch_bf16_tn) TCG_DECLARE_LAUNCHER(tcg_launch_bf16_tt)
TCG_DECLARE_LAUNCHER(tcg_launch_i8_nn) TCG_DECLARE_LAUNCHER(tcg_launch_i8_nt)
TCG_DECLARE_LAUNCHER(tcg_launch_i8_tn) TCG_DECLARE_LAUNCHER(tcg_launch_i8_tt)
#undef TCG_DECLARE_LAUNCHER
