// thin_kernel.hip -- C = alpha * A @ op(B) + beta * C for outputs at most 16
// columns wide, with A stored [M, K] (K-contiguous rows).  A matrix-core tile
// would spend 16 / N of its work on padding here and the problem is bound by
// reading A once, so this is a dot-product kernel on the vector ALUs:
//
//   * a workgroup (2 waves) owns 8 output rows; 16 lanes share one row and
//     walk its K in 16-byte pieces, so a wave reads 4 rows x 256 bytes per
//     load, coalesced; two or more workgroups share a CU, so one computes
//     while another waits for memory;
//   * K runs in chunks: 4, 2 or 1 KiB per row for up to 4, 8 or 16 columns
//     when the grid has few workgroups (each one then needs many loads in
//     flight), 512 bytes for any width when it has many (registers and LDS
//     per workgroup shrink, several workgroups share a CU and hide each
//     other's memory latency).  op(B) is staged in LDS one chunk at a time, transposed to Bt[n][k]
//     (zero past N and past K), in two buffers; a lane's pieces of A for the
//     next chunk are loaded into registers while the current chunk is
//     computed, and one barrier per chunk hands the next B buffer over;
//   * int8 uses v_dot4_i32_i8 (exact int32), fp16 and bf16 the dot2 forms
//     accumulating in fp32, fp32 FMAs; the 16 lanes of a row are then summed
//     with lane shuffles and one lane applies alpha / beta and stores the row.
//
// Same contract as the GEMM kernels (tessl "Architecture", "Cooperative
// Destination Accumulation": C written once; "Edge-Slice Support": k past K
// and rows past M contribute nothing).
#include "gemm_kernel.hpp"

namespace tcg {
namespace {

constexpr int kThinThreads = kThinRows / 4 * 64;   // 4 rows per wave

// Bytes of K per row per chunk for small grids (fewer for more columns, to
// keep the staged B and the two chunks of A in registers).  A lane holds
// CH / 256 pieces of 16 bytes of its row per chunk.
constexpr int thin_chunk_bytes(int ns) { return ns > 8 ? 1024 : ns > 4 ? 2048 : 4096; }
constexpr int kThinNarrowChunk = 512;    // bytes of K per row per chunk, large grids
constexpr int kThinNarrowGrid = 1024;    // workgroups from which the narrow chunk is used

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// The two halves of a 32-bit word.  The word comes in by value: a bit cast
// applied directly to an element of a vector variable would read the
// vector's first element whatever the index.
__device__ inline half2_t as_half2(u32 x) { return __builtin_bit_cast(half2_t, x); }
__device__ inline bf16x2_t as_bf16x2(u32 x) { return __builtin_bit_cast(bf16x2_t, x); }

// acc += dot(16 bytes of A, 16 bytes of B) for one column.
template <int DT>
__device__ inline void thin_dot(u32x4 a, u32x4 b, int &acc) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_sdot4((int)a[j], (int)b[j], acc, false);
}
template <int DT>
__device__ inline void thin_dot(u32x4 a, u32x4 b, float &acc) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (DT == DT_F32) {
            acc = __builtin_fmaf(as_f32(a[j]), as_f32(b[j]), acc);
        } else if constexpr (DT == DT_F16) {
            acc = __builtin_amdgcn_fdot2(as_half2(a[j]), as_half2(b[j]), acc, false);
        } else {
            acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a[j]), as_bf16x2(b[j]), acc, false);
        }
    }
}

// Load this lane's pieces of its A row for the whole chunk starting at kc.
template <int ES, int P>
__device__ inline void thin_load_a(const GemmArgs &args, const char *Ab, int64_t a_org, int rl, int kl,
                                   int kc, u32x4 (&a)[P]) {
    const int64_t a_chunk = a_org + (int64_t)kc * ES;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab + a_chunk, args.a_extent - a_chunk);
    const int row_off = rl * args.lda * ES;
#pragma unroll
    for (int i = 0; i < P; ++i) a[i] = ld128(ra, row_off + (kl + 16 * i) * 16);
}

// B stored [N, K] (K-contiguous), the whole chunk starting at kc: thread t
// holds pieces t, t + threads, ... (16 bytes each) of the chunk's Bt rows.
// Rows n >= N start at or past the end of B (ldb >= K), so the range-checked
// loads return zero there.
template <int ES, int NS, int CH>
__device__ inline void thin_load_bt(const GemmArgs &args, const char *Bb, int kc,
                                    u32x4 (&v)[NS * CH / 16 / kThinThreads]) {
    constexpr int PER_COL = CH / 16;
    constexpr int Q = NS * PER_COL / kThinThreads;
    const int64_t b_org = (int64_t)kc * ES;
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb + b_org, args.b_extent - b_org);
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int piece = threadIdx.x + q * kThinThreads;
        const int n = piece / PER_COL, u = piece % PER_COL;
        v[q] = ld128(rb, n * args.ldb * ES + u * 16);
    }
}

template <int NS, int CH>
__device__ inline void thin_store_bt(char *bt, const u32x4 (&v)[NS * CH / 16 / kThinThreads]) {
    constexpr int Q = NS * CH / 16 / kThinThreads;
#pragma unroll
    for (int q = 0; q < Q; ++q)
        *reinterpret_cast<u32x4 *>(bt + (threadIdx.x + q * kThinThreads) * 16) = v[q];
}

// B stored [N, K], the last chunk (kv < a whole chunk of k valid), one
// piece at a time: Bt[n][k - kc], zero past kv.
template <int ES, int NS, int CH>
__device__ inline void thin_stage_bt_tail(const GemmArgs &args, const char *Bb, int kc, int kv, char *bt) {
    constexpr int PER_COL = CH / 16;
    const int64_t b_org = (int64_t)kc * ES;
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb + b_org, args.b_extent - b_org);
#pragma unroll 1
    for (int piece = threadIdx.x; piece < NS * PER_COL; piece += kThinThreads) {
        const int n = piece / PER_COL, u = piece % PER_COL;
        const int k0 = u * (16 / ES);
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        const int off = n * args.ldb * ES + u * 16;
        if (n < args.N) {
            if (k0 + 16 / ES <= kv) v = ld128(rb, off);
            else if (k0 < kv) v = ld_partial<ES>(rb, off, kv - k0);
        }
        *reinterpret_cast<u32x4 *>(bt + piece * 16) = v;
    }
}

// One 16-byte piece of A (piece u of the chunk) against every staged column.
// The scheduling fence keeps the compiler from hoisting the LDS reads of
// every piece ahead at once (their registers would not fit).
template <int DT, int NS, int CH, typename Acc>
__device__ inline void thin_piece(const char *bt, int u, u32x4 a, Acc (&acc)[NS]) {
    u32x4 b[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) b[n] = *reinterpret_cast<const u32x4 *>(bt + n * CH + u * 16);
#pragma unroll
    for (int n = 0; n < NS; ++n) thin_dot<DT>(a, b[n], acc[n]);
    __builtin_amdgcn_sched_barrier(0);
}

// NS: columns computed (>= N, a multiple of 4); CH: bytes of K per row per
// chunk.  B is stored [N, K] (K-contiguous rows); a B stored [K, N] is
// transposed first (thin_pack_bt_kernel).
template <int DT, int OUT, int NS, int CH>
__global__ __launch_bounds__(kThinThreads) void thin_kernel(const GemmArgs args) {
    constexpr int ES = dt_size(DT);
    constexpr int KCH = CH / ES, P = CH / 256;
    static_assert(NS * CH % (16 * kThinThreads) == 0, "whole pieces of B per thread");
    constexpr int Q = NS * CH / 16 / kThinThreads;
    using Acc = std::conditional_t<DT == DT_I8, int, float>;
    __shared__ __attribute__((aligned(16))) char bt[2][NS * CH];

    const int M = args.M, N = args.N, K = args.K;
    const int mblocks = (M + kThinRows - 1) / kThinRows;
    const int z = blockIdx.x / mblocks;
    const int m0 = (blockIdx.x % mblocks) * kThinRows;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rl = wave * 4 + (lane >> 4);      // row of this lane inside the block
    const int kl = lane & 15;                   // this lane's 16-byte piece of every 256

    // buffer resources are based at the workgroup's rows and the chunk they
    // serve, so every offset stays far below 2^31; rows past M lie past the
    // A extent and read as zero
    const int64_t a_org = (int64_t)m0 * args.lda * ES;
    const char *Ab = static_cast<const char *>(args.A) + z * args.stride_a * ES;
    const char *Bb = static_cast<const char *>(args.B) + z * args.stride_b * ES;

    Acc acc[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) acc[n] = 0;

    // ---- whole chunks: the next chunk's A and B in flight while this one is
    // computed
    const int nfull = K / KCH;
    if (nfull > 0) {
        u32x4 a_cur[P], a_nxt[P];
        thin_load_a<ES, P>(args, Ab, a_org, rl, kl, 0, a_cur);
        {
            u32x4 bv[Q];
            thin_load_bt<ES, NS, CH>(args, Bb, 0, bv);
            thin_store_bt<NS, CH>(bt[0], bv);
        }
        __syncthreads();
#pragma unroll 1
        for (int c = 0; c < nfull; ++c) {
            const bool more = c + 1 < nfull;
            const char *cur = bt[c & 1];
            char *nxt = bt[(c + 1) & 1];
            u32x4 bv[Q];
            if (more) {
                thin_load_a<ES, P>(args, Ab, a_org, rl, kl, (c + 1) * KCH, a_nxt);
                thin_load_bt<ES, NS, CH>(args, Bb, (c + 1) * KCH, bv);
            }
#pragma unroll
            for (int i = 0; i < P; ++i) thin_piece<DT, NS, CH>(cur, kl + 16 * i, a_cur[i], acc);
            if (more) thin_store_bt<NS, CH>(nxt, bv);
            // every wave is done with cur, and nxt is written
            __syncthreads();
#pragma unroll
            for (int i = 0; i < P; ++i) a_cur[i] = a_nxt[i];
        }
    }

    // ---- the last, partial chunk (both buffers are free here)
    const int kc = nfull * KCH, kv = K - kc;
    if (kv > 0) {
        thin_stage_bt_tail<ES, NS, CH>(args, Bb, kc, kv, bt[0]);
        __syncthreads();
        const int64_t a_chunk = a_org + (int64_t)kc * ES;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab + a_chunk, args.a_extent - a_chunk);
        const int row_off = rl * args.lda * ES;
        // four pieces per lane in flight at a time
#pragma unroll 1
        for (int u0 = kl; u0 * (16 / ES) < kv; u0 += 64) {
            u32x4 a[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k0 = (u0 + 16 * q) * (16 / ES);
                const int off = row_off + k0 * ES;
                a[q] = u32x4{0u, 0u, 0u, 0u};
                if (k0 + 16 / ES <= kv) a[q] = ld128(ra, off);
                else if (k0 < kv) a[q] = ld_partial<ES>(ra, off, kv - k0);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (u0 + 16 * q < CH / 16) thin_piece<DT, NS, CH>(bt[0], u0 + 16 * q, a[q], acc);
        }
    }

    // ---- sum the 16 lanes of each row (fixed order: a butterfly)
#pragma unroll
    for (int n = 0; n < NS; ++n)
#pragma unroll
        for (int w = 8; w >= 1; w >>= 1) acc[n] += __shfl_xor(acc[n], w, 16);

    constexpr int CES = dt_size(OUT);
    if (args.c_trans) {
        // the transposed product of a small-M GEMM: row r of this problem is
        // column r of C and its columns n are rows of C (C[n * ldc + r]);
        // the bias and scale of C's column r apply to the whole row
        const int64_t c_org = (int64_t)m0 * CES;
        char *Cb = static_cast<char *>(args.C) + z * args.stride_c * CES + c_org;
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cb, args.c_extent - c_org);
        if (kl != 0 || m0 + rl >= M) return;
        const EpiState ep = make_epi<OUT == DT_I32 ? DT_F32 : OUT>(args, z, M);
        [[maybe_unused]] float b = 0.f, s = 1.f;
        if constexpr (OUT != DT_I32) {
            if (ep.on) load_epi1<OUT>(ep, m0 + rl, M, b, s);
        }
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            if (n >= N) break;
            const int off = n * args.ldc * CES + rl * CES;
            if constexpr (OUT == DT_I32) {
                int v[4] = {acc[n], 0, 0, 0};
                store_i4(rc, off, 1, false, v);
            } else {
                float v[4] = {(float)acc[n], 0.f, 0.f, 0.f};
                if (ep.on) {
                    const float b4[4] = {b, b, b, b}, s4[4] = {s, s, s, s};
                    finish4<OUT>(rc, off, 1, false, args.alpha, args.beta, v, ep, b4, s4);
                } else {
                    finish4<OUT>(rc, off, 1, false, args.alpha, args.beta, v);
                }
            }
        }
        return;
    }
    const int64_t c_org = (int64_t)m0 * args.ldc * CES;
    char *Cb = static_cast<char *>(args.C) + z * args.stride_c * CES + c_org;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cb, args.c_extent - c_org);
    if (kl != 0 || m0 + rl >= M) return;
    const int row_off = rl * args.ldc * CES;
    const EpiState ep = make_epi<OUT == DT_I32 ? DT_F32 : OUT>(args, z, N);
#pragma unroll
    for (int n = 0; n < NS; n += 4) {
        if (n >= N) break;
        const int nvalid = N - n < 4 ? N - n : 4;
        if constexpr (OUT == DT_I32) {
            int v[4] = {acc[n], acc[n + 1], acc[n + 2], acc[n + 3]};
            store_i4(rc, row_off + n * CES, nvalid, args.c_vec_ok != 0, v);
        } else {
            float v[4] = {(float)acc[n], (float)acc[n + 1], (float)acc[n + 2], (float)acc[n + 3]};
            finish4<OUT>(rc, row_off + n * CES, nvalid, args.c_vec_ok != 0, args.alpha, args.beta, v,
                         ep, n);
        }
    }
}

// Transposed copy of a thin B stored [K, N] (N <= NS values per row, rows
// ldb apart): Bt[n][k] with rows dst_pitch bytes apart.  Read straight from
// a wide matrix, each row of B is a cache line of its own; the copy gathers
// them once instead of once per workgroup of the thin kernel.  Thread t of
// workgroup (z, b) takes row k = 256 b + t; the stores of one column are
// coalesced.  Bt[n][k] past K is left unwritten (the thin kernel reads no
// k >= K).
template <int ES, int NS>
__global__ __launch_bounds__(256) void thin_pack_bt_kernel(const PackArgs a) {
    const int kblocks = (a.rows + 255) / 256;
    const int z = blockIdx.x / kblocks;
    const int k0 = (blockIdx.x % kblocks) * 256;
    const int t = threadIdx.x;
    const int nrows = min(256, a.rows - k0);
    // resources based at the workgroup's first row (uniform), offsets < 2^31;
    // the range ends with the last row's N values, past it loads return zero
    const char *src = static_cast<const char *>(a.src) + z * a.src_stride + (int64_t)k0 * a.src_pitch;
    char *dst = static_cast<char *>(a.dst) + z * a.dst_stride + (int64_t)k0 * ES;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, (int64_t)(nrows - 1) * a.src_pitch + a.row_bytes);
    if (t >= nrows) return;
    const int n_cols = a.row_bytes / ES;
    const int off = t * (int)a.src_pitch;
    // NS loads in flight (values past column N are not stored)
    u32 v[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) {
        if constexpr (ES == 4) v[n] = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 4 * n, 0, 0);
        else if constexpr (ES == 2) v[n] = __builtin_amdgcn_raw_buffer_load_b16(rs, off + 2 * n, 0, 0);
        else v[n] = __builtin_amdgcn_raw_buffer_load_b8(rs, off + n, 0, 0);
    }
#pragma unroll
    for (int n = 0; n < NS; ++n) {
        if (n < n_cols) {
            char *d = dst + n * a.dst_pitch + t * ES;
            if constexpr (ES == 4) *reinterpret_cast<u32 *>(d) = v[n];
            else if constexpr (ES == 2) *reinterpret_cast<unsigned short *>(d) = (unsigned short)v[n];
            else *reinterpret_cast<unsigned char *>(d) = (unsigned char)v[n];
        }
    }
}

template <int ES>
hipError_t launch_pack_bt_ns(const PackArgs &args, int64_t blocks, hipStream_t stream) {
    const int n = args.row_bytes / ES;
    if (n <= 4)
        hipLaunchKernelGGL((thin_pack_bt_kernel<ES, 4>), dim3((unsigned)blocks), dim3(256), 0, stream, args);
    else if (n <= 8)
        hipLaunchKernelGGL((thin_pack_bt_kernel<ES, 8>), dim3((unsigned)blocks), dim3(256), 0, stream, args);
    else
        hipLaunchKernelGGL((thin_pack_bt_kernel<ES, 16>), dim3((unsigned)blocks), dim3(256), 0, stream, args);
    return hipGetLastError();
}

template <int DT, int OUT, int NS>
hipError_t launch_thin_ch(const GemmArgs &args, int64_t grid, hipStream_t stream) {
    if (grid >= kThinNarrowGrid)
        hipLaunchKernelGGL((thin_kernel<DT, OUT, NS, kThinNarrowChunk>), dim3((unsigned)grid),
                           dim3(kThinThreads), 0, stream, args);
    else
        hipLaunchKernelGGL((thin_kernel<DT, OUT, NS, thin_chunk_bytes(NS)>), dim3((unsigned)grid),
                           dim3(kThinThreads), 0, stream, args);
    return hipGetLastError();
}

template <int DT, int OUT>
hipError_t launch_thin_ns(const GemmArgs &args, int64_t grid, hipStream_t stream) {
    if (args.N <= 4) return launch_thin_ch<DT, OUT, 4>(args, grid, stream);
    if (args.N <= 8) return launch_thin_ch<DT, OUT, 8>(args, grid, stream);
    return launch_thin_ch<DT, OUT, 16>(args, grid, stream);
}

template <int DT>
hipError_t launch_thin_dt(int out, const GemmArgs &args, int64_t grid, hipStream_t stream) {
    if constexpr (DT == DT_I8) {
        if (out == DT_I32) return launch_thin_ns<DT, DT_I32>(args, grid, stream);
        // float outputs: the dequantizing fused epilogue
        if (!args.epi) return hipErrorInvalidValue;
        if (out == DT_F32) return launch_thin_ns<DT, DT_F32>(args, grid, stream);
        if (out == DT_F16) return launch_thin_ns<DT, DT_F16>(args, grid, stream);
        if (out == DT_BF16) return launch_thin_ns<DT, DT_BF16>(args, grid, stream);
    } else if constexpr (DT == DT_F32) {
        if (out == DT_F32) return launch_thin_ns<DT, DT_F32>(args, grid, stream);
    } else {
        if (out == DT_F32) return launch_thin_ns<DT, DT_F32>(args, grid, stream);
        if (out == DT) return launch_thin_ns<DT, DT>(args, grid, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace
}  // namespace tcg

hipError_t tcg_launch_thin(int dt, int out, const tcg::GemmArgs &args, int64_t grid, hipStream_t stream) {
    using namespace tcg;
    if (args.N < 1 || args.N > 16 || grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    switch (dt) {
    case DT_F32: return launch_thin_dt<DT_F32>(out, args, grid, stream);
    case DT_F16: return launch_thin_dt<DT_F16>(out, args, grid, stream);
    case DT_BF16: return launch_thin_dt<DT_BF16>(out, args, grid, stream);
    case DT_I8: return launch_thin_dt<DT_I8>(out, args, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t tcg_launch_thin_pack_bt(const tcg::PackArgs &args, int es, hipStream_t stream) {
    using namespace tcg;
    const int64_t blocks = (int64_t)args.batch * ((args.rows + 255) / 256);
    if (blocks <= 0 || blocks > 0x7FFFFFFF || args.row_bytes < es || args.row_bytes > 16 * es ||
        args.row_bytes % es != 0 || args.dst_pitch < (int64_t)args.rows * es)
        return hipErrorInvalidValue;
    switch (es) {
    case 4: return launch_pack_bt_ns<4>(args, blocks, stream);
    case 2: return launch_pack_bt_ns<2>(args, blocks, stream);
    case 1: return launch_pack_bt_ns<1>(args, blocks, stream);
    default: return hipErrorInvalidValue;
    }
}
