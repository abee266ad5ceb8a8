// epilogue_kernels.hip -- the split-K reduction, the alpha == 0 kernel, the
// operand packing, the static scratch of the allocation-free entry point, and
// the dispatch from (input type, layout) to the per-object launchers.
#include "gemm_kernel.hpp"

#include <mutex>

// Scratch memory of the allocation-free entry point (split-K partial sums and
// packed operand copies): one array on every GPU the library runs on, there
// from the code object's load until the process ends.  Host code never uses
// the array's name as an address; it asks for the device address once per
// device (tcg_static_scratch) and passes that to kernels.
static __device__ __align__(256) char scratch[tcg::kStaticScratchBytes];

namespace tcg {
namespace {

template <int CDT>
__device__ inline EpiState epi_of(const EpilogueArgs &a, int z) {
    return make_epi<CDT>(a, z, a.N);
}

// Row m of problem z's C as a buffer resource spanning its N values (the
// row's byte address in 64-bit arithmetic).
__device__ inline __amdgpu_buffer_rsrc_t c_row_rsrc(const EpilogueArgs &a, int z, int m) {
    const int64_t ces = dt_size(a.c_dtype);
    char *row = static_cast<char *>(a.C) + ((int64_t)z * a.stride_c + (int64_t)m * a.ldc) * ces;
    return make_rsrc(row, (int64_t)a.N * ces);
}

// ---------------------------------------------------------------------------
// Split-K reduction: C = round(alpha * sum_s partial[s] + beta * C_old), the
// slices summed in ascending s so the result is the same on every run; the
// fused epilogue, when one is on, runs here (the partials have none).
// One thread per 4 consecutive outputs of a row; the workgroups of one
// problem never straddle the next, so the problem's partial sums are one
// workgroup-uniform buffer (no per-lane resource).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const EpilogueArgs a) {
    const int nq = (a.N + 3) / 4;
    const int64_t per = (int64_t)a.M * nq;          // threads of one problem
    const int64_t bpp = (per + 255) / 256;          // workgroups per problem
    const int z = (int)(blockIdx.x / bpp);
    const int64_t rem = (int64_t)(blockIdx.x % bpp) * 256 + threadIdx.x;
    if (z >= a.batch || rem >= per) return;
    const int m = (int)(rem / nq), n = (int)(rem % nq) * 4;
    const int nvalid = a.N - n;
    const int64_t plane = (int64_t)a.M * a.N;
    const char *wsz = static_cast<const char *>(a.ws) + (int64_t)z * a.splits * plane * 4;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(wsz, (int64_t)a.splits * plane * 4);
    const bool wvec = (a.N % 4) == 0;
    const bool cvec = a.c_vec_ok != 0;
    float s4[4] = {0.f, 0.f, 0.f, 0.f};
    int i4[4] = {0, 0, 0, 0};
    if (a.acc_is_int) {
        // exact int32 sums; int32 out as they are, a float out (int8 with a
        // dequantization scale) through the float epilogue below
        for (int s = 0; s < a.splits; ++s) {
            const int off = (int)((s * plane + (int64_t)m * a.N + n) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (e < nvalid) i4[e] += (int)__builtin_amdgcn_raw_buffer_load_b32(rw, off + 4 * e, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) s4[e] = (float)i4[e];
    } else {
        int s = 0;
        if (wvec && nvalid >= 4) {
            // groups of up to 16 slices: a group's loads are in flight
            // together (one memory round trip for up to 16 slices), the adds
            // still run in ascending s
            const int plane_b = (int)(plane * 4);
            const int off0 = (int)(((int64_t)m * a.N + n) * 4);
            for (; s < a.splits; s += 16) {
                u32x4 w[16];
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    if (s + u < a.splits) w[u] = ld128(rw, off0 + (s + u) * plane_b);
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    if (s + u < a.splits)
#pragma unroll
                        for (int e = 0; e < 4; ++e) s4[e] += as_f32(w[u][e]);
            }
        }
        for (; s < a.splits; ++s) {
            const int off = (int)((s * plane + (int64_t)m * a.N + n) * 4);
            if (wvec && nvalid >= 4) {
                u32x4 w = ld128(rw, off);
#pragma unroll
                for (int e = 0; e < 4; ++e) s4[e] += as_f32(w[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (e < nvalid)
                        s4[e] += as_f32(__builtin_amdgcn_raw_buffer_load_b32(rw, off + 4 * e, 0, 0));
            }
        }
    }
    auto finish = [&](const __amdgpu_buffer_rsrc_t &rc, int coff) {
        switch (a.c_dtype) {
        case DT_I32: store_i4(rc, coff, nvalid, cvec, i4); break;
        case DT_F32: finish4<DT_F32>(rc, coff, nvalid, cvec, a.alpha, a.beta, s4, epi_of<DT_F32>(a, z), n); break;
        case DT_BF16: finish4<DT_BF16>(rc, coff, nvalid, cvec, a.alpha, a.beta, s4, epi_of<DT_BF16>(a, z), n); break;
        default: finish4<DT_F16>(rc, coff, nvalid, cvec, a.alpha, a.beta, s4, epi_of<DT_F16>(a, z), n); break;
        }
    };
    // C: the problem's whole C as one workgroup-uniform buffer when every
    // offset in it fits 31 bits, else row m as a buffer of its N values
    // (offsets stay small for a C of any size); nothing past column N is
    // written either way
    const int64_t ces = dt_size(a.c_dtype);
    if (((int64_t)(a.M - 1) * a.ldc + a.N) * ces <= 0x7FFFFFFF)
        finish(make_rsrc(static_cast<char *>(a.C) + (int64_t)z * a.stride_c * ces, a.c_extent),
               (int)(((int64_t)m * a.ldc + n) * ces));
    else
        finish(c_row_rsrc(a, z, m), (int)(n * ces));
}

// alpha == 0: C = beta * C (beta == 0 writes zeros without reading C), then
// the fused epilogue when one is on.
__global__ __launch_bounds__(256) void scale_c_kernel(const EpilogueArgs a) {
    const int nq = (a.N + 3) / 4;
    const int64_t total = (int64_t)a.batch * a.M * nq;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const int z = (int)(idx / ((int64_t)a.M * nq));
    const int64_t rem = idx - (int64_t)z * a.M * nq;
    const int m = (int)(rem / nq), n = (int)(rem % nq) * 4;
    const int nvalid = a.N - n;
    const __amdgpu_buffer_rsrc_t rc = c_row_rsrc(a, z, m);
    const int coff = n * dt_size(a.c_dtype);
    const bool cvec = a.c_vec_ok != 0;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    // alpha = 1 on zeros keeps them zero; finish4 then adds beta * C_old.
    switch (a.c_dtype) {
    case DT_F32: finish4<DT_F32>(rc, coff, nvalid, cvec, 1.f, a.beta, v, epi_of<DT_F32>(a, z), n); break;
    case DT_BF16: finish4<DT_BF16>(rc, coff, nvalid, cvec, 1.f, a.beta, v, epi_of<DT_BF16>(a, z), n); break;
    case DT_F16: finish4<DT_F16>(rc, coff, nvalid, cvec, 1.f, a.beta, v, epi_of<DT_F16>(a, z), n); break;
    default: {
        int iv[4] = {0, 0, 0, 0};
        store_i4(rc, coff, nvalid, cvec, iv);
    }
    }
}

// Operand repacking into 16-byte row pitches, so that an operand whose rows
// do not start on 16-byte boundaries (or whose rows end inside a 16-byte
// chunk) can feed the direct-to-LDS GEMM kernel.  One wave per row (the
// buffer resource of the source row is then wave-uniform), four rows per
// workgroup; each lane moves 16 bytes at a time.  The source may sit at any
// byte address: buffer loads of 16 bytes take unaligned offsets, and the
// last partial chunk of a row is read byte by byte, the rest of it zero.
// With a.bt set, the few elements that follow each row's packed bytes (the
// columns of a thin strip computed by a second GEMM) are written transposed
// to that strip's B^T as well, so the strip needs no gather pass of its own.
__global__ __launch_bounds__(256) void pack_rows_kernel(const PackArgs a) {
    const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= (int64_t)a.batch * a.rows) return;
    const int z = (int)(row / a.rows), r = (int)(row % a.rows);
    const char *src = static_cast<const char *>(a.src) + z * a.src_stride + r * a.src_pitch;
    char *dst = static_cast<char *>(a.dst) + z * a.dst_stride + r * a.dst_pitch;
    const int tail_bytes = a.bt ? a.bt_cols * a.bt_es : 0;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, (int64_t)a.row_bytes + tail_bytes);
    // the transposed tail: lane n loads element n past the packed bytes now,
    // so its latency overlaps the row's
    const int lane = threadIdx.x & 63;
    u32 tail = 0;
    if (lane < (a.bt ? a.bt_cols : 0)) {
        const int off = a.row_bytes + lane * a.bt_es;
        if (a.bt_es == 4) tail = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
        else if (a.bt_es == 2) tail = __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0);
        else tail = __builtin_amdgcn_raw_buffer_load_b8(rs, off, 0, 0);
    }
    const int chunks = (int)(a.dst_pitch / 16), full = a.row_bytes / 16;
    // the whole chunks, eight per lane in flight before their stores (a row
    // of up to 8 KiB costs one memory round trip); no partial chunk among
    // them, so the loads go out with no branch between them
    for (int c0 = lane; c0 < full; c0 += 512) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (c0 + 64 * u < full) v[u] = ld128(rs, 16 * (c0 + 64 * u));
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (c0 + 64 * u < full) *reinterpret_cast<u32x4 *>(dst + 16 * (c0 + 64 * u)) = v[u];
    }
    // the partial chunk at the end of the row (byte by byte) and the zero
    // padding up to the pitch
    for (int c = full + lane; c < chunks; c += 64) {
        const int nb = a.row_bytes - 16 * c;
        const u32x4 v = nb > 0 ? ld_partial<1>(rs, 16 * c, nb) : u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4 *>(dst + 16 * c) = v;
    }
    if (lane < (a.bt ? a.bt_cols : 0)) {
        char *d = static_cast<char *>(a.bt) + z * a.bt_stride + (int64_t)lane * a.bt_pitch +
                  (int64_t)r * a.bt_es;
        if (a.bt_es == 4) *reinterpret_cast<u32 *>(d) = tail;
        else if (a.bt_es == 2) *reinterpret_cast<unsigned short *>(d) = (unsigned short)tail;
        else *reinterpret_cast<unsigned char *>(d) = (unsigned char)tail;
    }
}

using Launcher = hipError_t (*)(int, int, const GemmArgs &, int64_t, hipStream_t);

// [input type][transpose_a * 2 + transpose_b]
const Launcher kLaunchers[4][4] = {
    {tcg_launch_f32_nn, tcg_launch_f32_nt, tcg_launch_f32_tn, tcg_launch_f32_tt},
    {tcg_launch_f16_nn, tcg_launch_f16_nt, tcg_launch_f16_tn, tcg_launch_f16_tt},
    {tcg_launch_bf16_nn, tcg_launch_bf16_nt, tcg_launch_bf16_tn, tcg_launch_bf16_tt},
    {tcg_launch_i8_nn, tcg_launch_i8_nt, tcg_launch_i8_tn, tcg_launch_i8_tt}};

const char *const kDtName[4] = {"f32", "f16", "bf16", "i8"};
const char *const kLayoutName[2][2] = {{"nn", "nt"}, {"tn", "tt"}};
const char *const kTileName[NUM_TILE_CLASSES] = {"256x256", "128x128", "64x64",
                                                   "256x256_dma", "256x256_dma8", "128x128_dma",
                                                   "thin", "128x128_dma4", "64x64_ks", "32x32_ks",
                                                   "16x16_ks"};

char g_names[4][2][2][NUM_TILE_CLASSES][64];
bool g_names_ready = false;

}  // namespace
}  // namespace tcg

using namespace tcg;

hipError_t tcg_launch_gemm(int dt, bool ta, bool tb, int cls, int out, const GemmArgs &args,
                           int64_t grid, hipStream_t stream) {
    if (dt < 0 || dt > 3 || cls < 0 || cls >= NUM_TILE_CLASSES || grid <= 0 || grid > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    return kLaunchers[dt][(ta ? 2 : 0) + (tb ? 1 : 0)](cls, out, args, grid, stream);
}

hipError_t tcg_launch_pack_rows(const PackArgs &args, hipStream_t stream) {
    const int64_t blocks = ((int64_t)args.batch * args.rows + 3) / 4;
    if (blocks <= 0 || blocks > 0x7FFFFFFF || args.dst_pitch % 16 != 0 ||
        args.dst_pitch < args.row_bytes)
        return hipErrorInvalidValue;
    if (args.bt && (args.bt_cols < 1 || args.bt_cols > 16 ||
                    (args.bt_es != 1 && args.bt_es != 2 && args.bt_es != 4) ||
                    args.bt_pitch < (int64_t)args.rows * args.bt_es))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(pack_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, args);
    return hipGetLastError();
}

hipError_t tcg_launch_splitk_reduce(const EpilogueArgs &args, hipStream_t stream) {
    const int64_t per = (int64_t)args.M * ((args.N + 3) / 4);
    const int64_t blocks = (per + 255) / 256 * args.batch;
    if (blocks <= 0 || blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, args);
    return hipGetLastError();
}

hipError_t tcg_static_scratch(int device, void **ptr) {
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    if (device < 0 || device >= kMaxDevices || !ptr) return hipErrorInvalidValue;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[device]) {
        // the caller made `device` current: its own copy of the array
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[device] = p;
    }
    *ptr = addr[device];
    return hipSuccess;
}

hipError_t tcg_launch_scale_c(const EpilogueArgs &args, hipStream_t stream) {
    const int64_t total = (int64_t)args.batch * args.M * ((args.N + 3) / 4);
    const int64_t blocks = (total + 255) / 256;
    if (blocks <= 0 || blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(scale_c_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, args);
    return hipGetLastError();
}

const char *tcg_kernel_name(int dt, bool ta, bool tb, int cls) {
    if (dt < 0 || dt > 3 || cls < 0 || cls >= NUM_TILE_CLASSES) return "";
    if (!g_names_ready) {
        for (int d = 0; d < 4; ++d)
            for (int a = 0; a < 2; ++a)
                for (int b = 0; b < 2; ++b)
                    for (int c = 0; c < NUM_TILE_CLASSES; ++c)
                        snprintf(g_names[d][a][b][c], sizeof g_names[d][a][b][c], "gemm_%s_%s_%s",
                                 kDtName[d], kLayoutName[a][b], kTileName[c]);
        g_names_ready = true;
    }
    return g_names[dt][ta ? 1 : 0][tb ? 1 : 0][cls];
}
