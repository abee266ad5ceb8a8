// gemm_inst.hip -- instantiates the GEMM kernel for one input type and one
// layout and exports that object's launcher.  The build compiles this file
// once per (TCG_DT, TCG_TA, TCG_TB) with TCG_LAUNCHER naming the launcher,
// so the 16 objects compile in parallel.
#include "gemm_dma_kernel.hpp"

#if !defined(TCG_DT) || !defined(TCG_TA) || !defined(TCG_TB) || !defined(TCG_LAUNCHER)
#error "the build defines TCG_DT, TCG_TA, TCG_TB and TCG_LAUNCHER"
#endif

namespace tcg {
namespace {

// Output types that exist for this input type (include/tcgemm.h lists the
// supported tuples); split-K partials only for the classes the planner
// splits (64x64, the 128x128 tiles and the 256x256 ring); the direct-to-LDS
// classes only for 16-bit and int8 inputs.
constexpr bool out_ok(int cls, int out) {
    if (is_dma_class(cls) && TCG_DT == DT_F32) return false;
    if (out == OUT_PARTIAL)
        return cls == TILE_64 || cls == TILE_128 || cls == TILE_128_DMA || cls == TILE_128_DMA4 ||
               cls == TILE_256_DMA;
    if (cls == TILE_THIN) return false;
    // int8 into a float output: the dequantizing fused epilogue only
    if (TCG_DT == DT_I8) return out == DT_I32 || out == DT_F32 || out == DT_F16 || out == DT_BF16;
    if (TCG_DT == DT_F32) return out == DT_F32;
    return out == TCG_DT || out == DT_F32;
}

template <int CLS, int OUT>
hipError_t launch_one(const GemmArgs &args, int64_t grid, hipStream_t stream) {
    if constexpr (is_dma_class(CLS) && out_ok(CLS, OUT)) {
        // the K tail needs per-chunk masks only when K is not a whole number
        // of 128-byte tiles (split-K slices are whole tiles)
        constexpr int T = tile_shape(CLS).bm;
        constexpr int NW = CLS == TILE_256_DMA8 ? 8 : 4;
        constexpr int OCC = CLS == TILE_128_DMA ? 2 : 1;
        // LDS: 4 stages for split-K slices (5, all 160 KiB, measured no
        // faster on the batched 128 x 384 x 16384 split-K shape); the 256 x
        // 256 tile with 4 waves as the ring of 5 slots (measured on the same
        // box, the ring ran 0.5-1.5 % faster than 2 stages on the bf16 NN,
        // fp16 TN and int8 NN 4096^3 shapes, the same on fp16 NT)
        constexpr int NST = CLS == TILE_128_DMA4 ? 4 : CLS == TILE_256_DMA ? 5 : 2;
        // 16 x 16 MFMA blocks: the 32 x 32 form measured 6-8 % slower on the
        // 256 x 256 tile (4096^3 bf16 NN, fp16 TN and NT)
        constexpr int MS = 16;
        // and the epilogue variant: C read only when beta != 0, the fused
        // epilogue only when one is asked for (float outputs)
        constexpr int BK = kLdsRowBytes / dt_size(TCG_DT);
        constexpr bool FLOAT_OUT = OUT == DT_F32 || OUT == DT_F16 || OUT == DT_BF16;
        const bool kmask = args.K % BK != 0;
        const int epi = !FLOAT_OUT ? EPI_PLAIN
                      : args.epi   ? EPI_FUSED
                      : args.beta != 0.f ? EPI_BETA : EPI_PLAIN;
        const dim3 g((unsigned)grid), b(NW * 64);
#define TCG_DMA(KM, EP) \
    hipLaunchKernelGGL((gemm_dma_kernel<TCG_DT, (bool)TCG_TA, (bool)TCG_TB, OUT, T, T, NW, OCC, KM, EP, NST, MS>), \
                       g, b, 0, stream, args)
        if constexpr (FLOAT_OUT && TCG_DT == DT_I8) {
            // int8 sums reach a float output only through the fused epilogue
            if (epi != EPI_FUSED) return hipErrorInvalidValue;
            if (kmask) TCG_DMA(true, EPI_FUSED);
            else TCG_DMA(false, EPI_FUSED);
        } else if constexpr (FLOAT_OUT) {
            if (kmask) {
                if (epi == EPI_FUSED) TCG_DMA(true, EPI_FUSED);
                else if (epi == EPI_BETA) TCG_DMA(true, EPI_BETA);
                else TCG_DMA(true, EPI_PLAIN);
            } else {
                if (epi == EPI_FUSED) TCG_DMA(false, EPI_FUSED);
                else if (epi == EPI_BETA) TCG_DMA(false, EPI_BETA);
                else TCG_DMA(false, EPI_PLAIN);
            }
        } else {
            if (kmask) TCG_DMA(true, EPI_PLAIN);
            else TCG_DMA(false, EPI_PLAIN);
        }
#undef TCG_DMA
        return hipGetLastError();
    } else if constexpr (is_ks_class(CLS) && out_ok(CLS, OUT)) {
        if (TCG_DT == DT_I8 && OUT != DT_I32 && !args.epi) return hipErrorInvalidValue;
        hipLaunchKernelGGL((gemm_ks_kernel<TCG_DT, (bool)TCG_TA, (bool)TCG_TB, OUT, tile_shape(CLS).bm>),
                           dim3((unsigned)grid), dim3(256), 0, stream, args);
        return hipGetLastError();
    } else if constexpr (!is_dma_class(CLS) && !is_ks_class(CLS) && out_ok(CLS, OUT)) {
        if (TCG_DT == DT_I8 && OUT != DT_I32 && OUT != OUT_PARTIAL && !args.epi)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL((gemm_kernel<TCG_DT, (bool)TCG_TA, (bool)TCG_TB, CLS, OUT>),
                           dim3((unsigned)grid), dim3(256), 0, stream, args);
        return hipGetLastError();
    } else {
        return hipErrorInvalidValue;
    }
}

template <int CLS>
hipError_t launch_cls(int out, const GemmArgs &args, int64_t grid, hipStream_t stream) {
    switch (out) {
    case DT_F32: return launch_one<CLS, DT_F32>(args, grid, stream);
    case DT_F16: return launch_one<CLS, DT_F16>(args, grid, stream);
    case DT_BF16: return launch_one<CLS, DT_BF16>(args, grid, stream);
    case DT_I32: return launch_one<CLS, DT_I32>(args, grid, stream);
    case OUT_PARTIAL: return launch_one<CLS, OUT_PARTIAL>(args, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace
}  // namespace tcg

hipError_t TCG_LAUNCHER(int cls, int out, const tcg::GemmArgs &args, int64_t grid,
                        hipStream_t stream) {
    using namespace tcg;
    switch (cls) {
    case TILE_256: return launch_cls<TILE_256>(out, args, grid, stream);
    case TILE_128: return launch_cls<TILE_128>(out, args, grid, stream);
    case TILE_64: return launch_cls<TILE_64>(out, args, grid, stream);
    case TILE_256_DMA: return launch_cls<TILE_256_DMA>(out, args, grid, stream);
    case TILE_256_DMA8: return launch_cls<TILE_256_DMA8>(out, args, grid, stream);
    case TILE_128_DMA: return launch_cls<TILE_128_DMA>(out, args, grid, stream);
    case TILE_128_DMA4: return launch_cls<TILE_128_DMA4>(out, args, grid, stream);
    case TILE_64_KS: return launch_cls<TILE_64_KS>(out, args, grid, stream);
    case TILE_32_KS: return launch_cls<TILE_32_KS>(out, args, grid, stream);
    case TILE_16_KS: return launch_cls<TILE_16_KS>(out, args, grid, stream);
    default: return hipErrorInvalidValue;
    }
}
