// gemm_kernel.hpp -- the dense GEMM kernel template for gfx950 (MI355X, CDNA4).
// Instantiated by gemm_inst.hip (one object per input type and layout).
//
// Computes C = alpha * op(A) @ op(B) + beta * C in BLAS row-major layout
// (tensorcore "GEMM", section "Surface").  The K extent is walked in blocks:
// each block of op(A) rows and op(B) columns is brought on chip, multiplied,
// and added into a running sum (the loop structure of Phobos "Matrix
// products", matmul / matmul_t).  That sum stays in registers from the first
// K block to the last, and C is written once at the end (tessl
// "Architecture", section "Cooperative Destination Accumulation").
//
// Structure of one workgroup (256 threads = 4 wave64s, 2 x 2):
//   * tile (tm, tn, group) from tile_of_workgroup(): XCD-aware regrouping,
//     then the column-panel band order;
//   * per K-tile: every thread loads its share of the A and B tiles from HBM
//     into registers (buffer loads; transposed operands are transposed in
//     registers), writes them to one of two LDS stages, and the waves run MFMA
//     on the other stage -- one barrier per K-tile; the 64x64 class keeps two
//     tiles in flight in two register sets, the larger classes one;
//   * LDS holds both operands K-contiguous: one 128-byte row of K per M (or
//     N) index, its 16-byte chunks XOR-swizzled by the row so that fragment
//     reads and transposed writes do not collide in banks;
//   * each wave owns a (BM/2) x (BN/2) block of C as 16x16 MFMA blocks;
//     operands enter the MFMA swapped (B block as src0, A block as src1) so
//     each lane ends up with 4 consecutive columns of one C row;
//   * epilogue: alpha*acc + beta*C_old (C read only when beta != 0), or the
//     fused form act(alpha*scale[n]*acc + beta*C_old + bias[n]), rounded once
//     to the output type, masked to the M x N extent -- or, for split-K, the
//     raw fp32/int32 partial to the workspace.
//
// Ragged edges (tessl "Architecture", "Edge-Slice Support"): tiles that reach
// past M, N or K take a checked load path that zero-fills everything outside
// the operand, element by element where a 16-byte chunk straddles the end.
// Every global access is a buffer access whose range is the operand's own
// extent, so an access outside it reads 0 or is dropped instead of faulting.

#pragma once

#include <type_traits>

#include "tc_internal.h"

namespace tcg {
namespace {

typedef uint32_t u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Scalar reinterpretation through a by-value parameter.  With this clang,
// __builtin_bit_cast applied directly to an element of an ext_vector_type
// value reads element 0 whatever the index; copying the element into a
// parameter first gives the element that was asked for.
__device__ inline float as_f32(u32 x) { return __builtin_bit_cast(float, x); }
__device__ inline u32 as_u32(float x) { return __builtin_bit_cast(u32, x); }
__device__ inline int as_i32(float x) { return __builtin_bit_cast(int, x); }

// Word 3 of a gfx9-family buffer resource: raw (untyped) 32-bit data.
constexpr int kRsrcWord3 = 0x00020000;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    int32_t n = bytes <= 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, kRsrcWord3);
}

__device__ inline u32x4 ld128(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Load the first `nvalid` elements (of 16 / ES) of a 16-byte chunk one by
// one; the rest of the chunk is zero.  Used where a chunk straddles the end
// of a row or of the operand.
template <int ES>
__device__ inline u32x4 ld_partial(__amdgpu_buffer_rsrc_t r, int off, int nvalid) {
    u32 w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16 / ES; ++e) {
        if (e < nvalid) {
            u32 x;
            if constexpr (ES == 4) {
                x = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * e, 0, 0);
            } else if constexpr (ES == 2) {
                x = __builtin_amdgcn_raw_buffer_load_b16(r, off + 2 * e, 0, 0);
            } else {
                x = __builtin_amdgcn_raw_buffer_load_b8(r, off + e, 0, 0);
            }
            const int bit = e * ES * 8;
            w[bit >> 5] |= x << (bit & 31);
        }
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}

// LDS tile layout: row r (an M or N index) holds 128 bytes of K as 8 chunks
// of 16 bytes; chunk c is stored at position c ^ swz(r).  swz mixes the low
// three bits of the row with the next three, so 8 consecutive rows read at
// one chunk (fragment reads) and rows 8 apart written at one chunk
// (transposed writes) both land on 8 different 16-byte bank groups.
__device__ inline int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ inline int lds_off(int row, int chunk) {
    return row * kLdsRowBytes + ((chunk ^ swz(row)) << 4);
}

// ---------------------------------------------------------------------------
// Operand tile loaders.  A tile is R rows (M or N indices) x 128 bytes of K.
// ---------------------------------------------------------------------------

// K-contiguous operand (A not transposed, B transposed): global row r has the
// tile's K slice at bytes [0, 128) from the tile origin.  8 threads cover one
// 128-byte row, so a wave reads 8 full rows.
template <int ES, int R, int THREADS>
struct RowLoader {
    static constexpr int kChunks = R * 8;
    static constexpr int kPer = (kChunks + THREADS - 1) / THREADS;
    u32x4 v[kPer];

    template <bool CHECK>
    __device__ inline void load(__amdgpu_buffer_rsrc_t r, int tid, int ld_bytes,
                                int rows_valid, int k_valid) {
        constexpr int EPC = 16 / ES;
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int q = tid + u * THREADS;
            if (kChunks % THREADS != 0 && q >= kChunks) break;
            const int row = q >> 3, c = q & 7;
            const int off = row * ld_bytes + c * 16;
            if constexpr (!CHECK) {
                v[u] = ld128(r, off);
            } else {
                const int k0 = c * EPC;
                if (row < rows_valid && k0 + EPC <= k_valid) {
                    v[u] = ld128(r, off);
                } else if (row >= rows_valid || k0 >= k_valid) {
                    v[u] = u32x4{0u, 0u, 0u, 0u};
                } else {
                    v[u] = ld_partial<ES>(r, off, k_valid - k0);
                }
            }
        }
    }

    __device__ inline void store(char *s, int tid) const {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int q = tid + u * THREADS;
            if (kChunks % THREADS != 0 && q >= kChunks) break;
            *reinterpret_cast<u32x4 *>(s + lds_off(q >> 3, q & 7)) = v[u];
        }
    }
};

// M/N-contiguous operand (A transposed, B not transposed): global row k holds
// the tile's R M/N values.  Each thread loads a block of KB rows x 16 bytes
// and transposes it in registers so that LDS again holds K-contiguous rows.
// Threads with consecutive ids take consecutive 16-byte chunks of one k row.
template <int ES, int R, int THREADS>
struct ColLoader {
    static constexpr int EPC = 16 / ES;             // M/N values per chunk
    static constexpr int KB = (ES == 4) ? 4 : 8;    // k rows per block
    static constexpr int BKE = kLdsRowBytes / ES;   // k values per tile
    static constexpr int NMB = R / EPC;
    static constexpr int NKB = BKE / KB;
    static constexpr int kBlocks = NMB * NKB;
    static constexpr int kPer = (kBlocks + THREADS - 1) / THREADS;
    static_assert(R % EPC == 0, "tile rows must hold whole chunks");
    u32x4 in[kPer][KB];

    template <bool CHECK>
    __device__ inline void load(__amdgpu_buffer_rsrc_t r, int tid, int ld_bytes,
                                int mn_valid, int k_valid) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int q = tid + u * THREADS;
            if (kBlocks % THREADS != 0 && q >= kBlocks) break;
            const int mb = q % NMB, kb = q / NMB;
#pragma unroll
            for (int j = 0; j < KB; ++j) {
                const int krow = kb * KB + j;
                const int off = krow * ld_bytes + mb * 16;
                if constexpr (!CHECK) {
                    in[u][j] = ld128(r, off);
                } else {
                    const int mn0 = mb * EPC;
                    if (krow < k_valid && mn0 + EPC <= mn_valid) {
                        in[u][j] = ld128(r, off);
                    } else if (krow >= k_valid || mn0 >= mn_valid) {
                        in[u][j] = u32x4{0u, 0u, 0u, 0u};
                    } else {
                        in[u][j] = ld_partial<ES>(r, off, mn_valid - mn0);
                    }
                }
            }
        }
    }

    __device__ inline void store(char *s, int tid) const {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int q = tid + u * THREADS;
            if (kBlocks % THREADS != 0 && q >= kBlocks) break;
            const int mb = q % NMB, kb = q / NMB;
            if constexpr (ES == 4) {
                // 4 k rows x 4 values: column e is word e of each row.
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    u32x4 o = {in[u][0][e], in[u][1][e], in[u][2][e], in[u][3][e]};
                    *reinterpret_cast<u32x4 *>(s + lds_off(mb * 4 + e, kb)) = o;
                }
            } else if constexpr (ES == 2) {
                // 8 k rows x 8 halves: column e takes half (e & 1) of word e/2
                // of rows 2p and 2p+1 into word p.
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    u32x4 o;
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const u32 x0 = in[u][2 * p][e >> 1], x1 = in[u][2 * p + 1][e >> 1];
                        o[p] = (e & 1) ? ((x0 >> 16) | (x1 & 0xFFFF0000u))
                                       : ((x0 & 0xFFFFu) | (x1 << 16));
                    }
                    *reinterpret_cast<u32x4 *>(s + lds_off(mb * 8 + e, kb)) = o;
                }
            } else {
                // 8 k rows x 16 bytes: column c gathers byte c of each row,
                // rows 0-3 into the low word and rows 4-7 into the high word;
                // the 8 bytes go to byte offset 8*kb of the 128-byte row.
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    const int w = c >> 2, sh = (c & 3) * 8;
                    u32 lo = 0, hi = 0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        lo |= ((in[u][j][w] >> sh) & 0xFFu) << (8 * j);
                        hi |= ((in[u][j + 4][w] >> sh) & 0xFFu) << (8 * j);
                    }
                    *reinterpret_cast<u32x2 *>(s + lds_off(mb * 16 + c, kb >> 1) +
                                               ((kb & 1) << 3)) = u32x2{lo, hi};
                }
            }
        }
    }
};

// ---------------------------------------------------------------------------
// MFMA step: one 16x16 output block, one 16-byte K chunk per lane.
// Lane l supplies row (l % 16) of its operand and chunk (l / 16) of the
// current 64-byte half of the LDS row; both operands use the same lane -> k
// mapping, so the instruction contracts matching k.
// ---------------------------------------------------------------------------
template <int DT>
struct Mma;

template <>
struct Mma<DT_BF16> {
    using Acc = f32x4;
    __device__ static inline void run(Acc &acc, u32x4 b, u32x4 a) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b),
                                                      __builtin_bit_cast(bf16x8, a), acc, 0, 0, 0);
    }
};

template <>
struct Mma<DT_F16> {
    using Acc = f32x4;
    __device__ static inline void run(Acc &acc, u32x4 b, u32x4 a) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, b),
                                                     __builtin_bit_cast(f16x8, a), acc, 0, 0, 0);
    }
};

template <>
struct Mma<DT_I8> {
    using Acc = i32x4;
    __device__ static inline void run(Acc &acc, u32x4 b, u32x4 a) {
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, b),
                                                    __builtin_bit_cast(i32x4, a), acc, 0, 0, 0);
    }
};

// fp32: a 16-byte chunk holds 4 k values; element e of every lane's chunk
// feeds the e-th 16x16x4 instruction, which therefore contracts the k set
// {4g + e : g = 0..3} -- the four instructions together cover all 16.
template <>
struct Mma<DT_F32> {
    using Acc = f32x4;
    __device__ static inline void run(Acc &acc, u32x4 b, u32x4 a) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32(b[e]), as_f32(a[e]), acc,
                                                       0, 0, 0);
    }
};

// ---------------------------------------------------------------------------
// Output conversion and the shared epilogue of the GEMM and reduce kernels.
// ---------------------------------------------------------------------------
__device__ inline u32 to_bf16_bits(float x) {
    return (u32)__builtin_bit_cast(unsigned short, static_cast<__bf16>(x));
}
__device__ inline u32 to_f16_bits(float x) {
    return (u32)__builtin_bit_cast(unsigned short, static_cast<_Float16>(x));
}
// Two values rounded to the 16-bit type in one packed conversion; the first
// in the low half.
template <int CDT>
__device__ inline u32 pack2_16(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t x = {lo, hi};
    if constexpr (CDT == DT_BF16) return __builtin_bit_cast(u32, __builtin_convertvector(x, bf16x2_t));
    else return __builtin_bit_cast(u32, __builtin_convertvector(x, f16x2_t));
}
__device__ inline float from_bf16_bits(u32 h) { return as_f32(h << 16); }
__device__ inline float from_f16_bits(u32 h) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)h);
}

// Read up to 4 consecutive C values (n < nvalid) as float.
template <int CDT>
__device__ inline void load_c4(__amdgpu_buffer_rsrc_t r, int off, int nvalid, bool vec,
                               float (&o)[4]) {
    if constexpr (CDT == DT_F32) {
        if (vec && nvalid >= 4) {
            u32x4 w = ld128(r, off);
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = as_f32(w[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = e < nvalid ? as_f32(__builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * e, 0, 0))
                                  : 0.f;
        }
    } else {
        u32 h[4];
        if (vec && nvalid >= 4) {
            u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
            h[0] = w[0] & 0xFFFFu; h[1] = w[0] >> 16; h[2] = w[1] & 0xFFFFu; h[3] = w[1] >> 16;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                h[e] = e < nvalid ? (u32)__builtin_amdgcn_raw_buffer_load_b16(r, off + 2 * e, 0, 0)
                                  : 0u;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o[e] = (CDT == DT_BF16) ? from_bf16_bits(h[e]) : from_f16_bits(h[e]);
    }
}

// Store up to 4 consecutive values (n < nvalid) converted to CDT.
template <int CDT>
__device__ inline void store_c4(__amdgpu_buffer_rsrc_t r, int off, int nvalid, bool vec,
                                const float (&v)[4]) {
    if constexpr (CDT == DT_F32) {
        if (vec && nvalid >= 4) {
            u32x4 w = {as_u32(v[0]), as_u32(v[1]), as_u32(v[2]), as_u32(v[3])};
            __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, 0);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (e < nvalid)
                    __builtin_amdgcn_raw_buffer_store_b32(as_u32(v[e]), r,
                                                          off + 4 * e, 0, 0);
        }
    } else {
        if (vec && nvalid >= 4) {
            u32x2 w = {pack2_16<CDT>(v[0], v[1]), pack2_16<CDT>(v[2], v[3])};
            __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, 0);
        } else {
            u32 h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                h[e] = (CDT == DT_BF16) ? to_bf16_bits(v[e]) : to_f16_bits(v[e]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (e < nvalid)
                    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)h[e], r, off + 2 * e, 0, 0);
        }
    }
}

__device__ inline void store_i4(__amdgpu_buffer_rsrc_t r, int off, int nvalid, bool vec,
                                const int (&v)[4]) {
    if (vec && nvalid >= 4) {
        u32x4 w = {(u32)v[0], (u32)v[1], (u32)v[2], (u32)v[3]};
        __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, 0);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e < nvalid) __builtin_amdgcn_raw_buffer_store_b32((u32)v[e], r, off + 4 * e, 0, 0);
    }
}

// Fused epilogue of one problem (tessl "Architecture", "Fused Epilogue" and
// "Integer GEMM"): the accumulator times the column's dequantization scale
// (fp32, one vector per problem; 1 without), then alpha * . + beta * C_old,
// plus the column's bias (stored in C's element type) and the activation,
// still in fp32 registers, before the single rounding to the output type.
struct EpiState {
    __amdgpu_buffer_rsrc_t rb;   // this problem's bias vector (empty range without one)
    __amdgpu_buffer_rsrc_t rs;   // this problem's scale vector (likewise)
    int act;
    bool bias, scale;
    bool on;
};

template <int CDT>
__device__ inline EpiState make_epi(const void *bias, int64_t bias_stride, const float *scale,
                                    int64_t scale_stride, int act, int epi, int z, int N) {
    constexpr int CES = dt_size(CDT);
    EpiState e;
    e.on = epi != 0;
    e.act = act;
    e.bias = bias != nullptr;
    e.scale = scale != nullptr;
    const char *b = e.bias ? static_cast<const char *>(bias) + z * bias_stride * CES : nullptr;
    e.rb = make_rsrc(b, e.bias ? (int64_t)N * CES : 0);
    const float *s = e.scale ? scale + z * scale_stride : nullptr;
    e.rs = make_rsrc(s, e.scale ? (int64_t)N * 4 : 0);
    return e;
}

template <int CDT, typename Args>
__device__ inline EpiState make_epi(const Args &a, int z, int N) {
    return make_epi<CDT>(a.bias, a.bias_stride, a.scale, a.scale_stride, a.act, a.epi, z, N);
}

// GELU, tanh form: 0.5 y (1 + tanh(u)) with u = sqrt(2/pi) (y + 0.044715 y^3).
// Since 1 + tanh(u) = 2 / (1 + exp(-2u)), this is y / (1 + exp(-2u)): one
// hardware exp2 and one reciprocal.  The exponent -2u log2(e) is
// y (g1 + g3 y^2) with the constants folded (g1 = -2 log2(e) sqrt(2/pi),
// g3 = 0.044715 g1): three VALU operations.  Large negative u gives exp =
// inf and the value 0 (-0 for y < 0); large positive u gives y.
__device__ inline float gelu_tanh(float y) {
    constexpr float g1 = -2.3022082f;      // -2 * 1.4426950409 * 0.7978845608
    constexpr float g3 = -0.10294324f;     // g1 * 0.044715
    const float t = y * __builtin_fmaf(g3, y * y, g1);
    return y * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(t));
}

// The activation of one value.
template <int ACT>
__device__ inline float act1(float v) {
    if constexpr (ACT == ACT_RELU) return v > 0.f ? v : 0.f;
    else if constexpr (ACT == ACT_GELU_TANH) return gelu_tanh(v);
    else return v;
}

// The bias of columns n .. n + nvalid - 1 (zero past them or without a bias)
// and their scales (one without a scale).
template <int CDT>
__device__ inline void load_bias4(const EpiState &e, int n, int nvalid, float (&b)[4]) {
    if (e.bias) {
        load_c4<CDT>(e.rb, n * dt_size(CDT), nvalid, true, b);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) b[q] = 0.f;
    }
}
__device__ inline void load_scale4(const EpiState &e, int n, int nvalid, float (&s)[4]) {
    if (e.scale) {
        load_c4<DT_F32>(e.rs, n * 4, nvalid, true, s);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) s[q] = 1.f;
    }
}

// Column n's bias (zero past N or without a bias) and scale (one without).
template <int CDT>
__device__ inline void load_epi1(const EpiState &e, int n, int N, float &b, float &s) {
    constexpr int CES = dt_size(CDT);
    b = 0.f;
    s = 1.f;
    if (n < N) {
        if (e.bias) {
            const int off = n * CES;
            if constexpr (CDT == DT_F32) b = as_f32(__builtin_amdgcn_raw_buffer_load_b32(e.rb, off, 0, 0));
            else if constexpr (CDT == DT_BF16) b = from_bf16_bits(__builtin_amdgcn_raw_buffer_load_b16(e.rb, off, 0, 0));
            else b = from_f16_bits(__builtin_amdgcn_raw_buffer_load_b16(e.rb, off, 0, 0));
        }
        if (e.scale) s = as_f32(__builtin_amdgcn_raw_buffer_load_b32(e.rs, n * 4, 0, 0));
    }
}

// The bn bias values of the tile starting at column n0 (lds[0 .. bn), zero
// past N or without a bias) and its scales (lds[bn .. 2 bn), one without a
// scale), as fp32 in LDS: staged once per workgroup, so the epilogue reads
// each lane's four columns from LDS instead of from memory behind its own C
// stores.  The caller makes the LDS free before and synchronizes after.
template <int CDT>
__device__ inline void stage_epi(const EpiState &e, int n0, int N, int bn, float *lds, int tid,
                                 int nthreads) {
    for (int t = tid; t < bn; t += nthreads) {
        float b, s;
        load_epi1<CDT>(e, n0 + t, N, b, s);
        lds[t] = b;
        lds[bn + t] = s;
    }
}

// Four staged bias values and scales from tile column nl (a multiple of 4).
__device__ inline void read_epi4(const float *lds, int bn, int nl, float (&b)[4], float (&s)[4]) {
    const f32x4 wb = *reinterpret_cast<const f32x4 *>(lds + nl);
    const f32x4 ws = *reinterpret_cast<const f32x4 *>(lds + bn + nl);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        b[q] = wb[q];
        s[q] = ws[q];
    }
}

// v + b (when there is a bias), then the activation.
__device__ inline void act4(const EpiState &e, const float (&b)[4], float (&v)[4]) {
    if (e.bias) {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] += b[q];
    }
    if (e.act == ACT_RELU) {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = v[q] > 0.f ? v[q] : 0.f;
    } else if (e.act == ACT_GELU_TANH) {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = gelu_tanh(v[q]);
    }
}



// alpha * acc + beta * C_old for 4 values, C_old read only when beta != 0.
template <int CDT>
__device__ inline void scale4(__amdgpu_buffer_rsrc_t rc, int off, int nvalid, bool vec, float alpha,
                              float beta, float (&v)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] *= alpha;
    if (beta != 0.f) {
        float old[4];
        load_c4<CDT>(rc, off, nvalid, vec, old);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(beta, old[e], v[e]);
    }
}

// scale4, then the store.
template <int CDT>
__device__ inline void finish4(__amdgpu_buffer_rsrc_t rc, int off, int nvalid, bool vec,
                               float alpha, float beta, float (&v)[4]) {
    scale4<CDT>(rc, off, nvalid, vec, alpha, beta, v);
    store_c4<CDT>(rc, off, nvalid, vec, v);
}

// The fused epilogue with the four columns' bias b and scale s at hand:
// v * s, then scale4, then bias and activation, then the store.
template <int CDT>
__device__ inline void finish4(__amdgpu_buffer_rsrc_t rc, int off, int nvalid, bool vec,
                               float alpha, float beta, float (&v)[4], const EpiState &ep,
                               const float (&b)[4], const float (&s)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] *= s[q];
    scale4<CDT>(rc, off, nvalid, vec, alpha, beta, v);
    act4(ep, b, v);
    store_c4<CDT>(rc, off, nvalid, vec, v);
}

// The fused epilogue with sa = alpha * scale of the four columns folded:
// v * sa + beta * C_old (C read only when beta != 0), bias, activation,
// store.
template <int CDT>
__device__ inline void finish4_fused(__amdgpu_buffer_rsrc_t rc, int off, int nvalid, bool vec,
                                     float beta, float (&v)[4], const EpiState &ep,
                                     const float (&b)[4], const float (&sa)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] *= sa[q];
    if (beta != 0.f) {
        float old[4];
        load_c4<CDT>(rc, off, nvalid, vec, old);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = __builtin_fmaf(beta, old[q], v[q]);
    }
    act4(ep, b, v);
    store_c4<CDT>(rc, off, nvalid, vec, v);
}

// The same with bias and scale loaded here (n: column of v[0]); without a
// fused epilogue the plain finish4.
template <int CDT>
__device__ inline void finish4(__amdgpu_buffer_rsrc_t rc, int off, int nvalid, bool vec,
                               float alpha, float beta, float (&v)[4], const EpiState &ep, int n) {
    if (!ep.on) {
        finish4<CDT>(rc, off, nvalid, vec, alpha, beta, v);
        return;
    }
    float b[4], s[4];
    load_bias4<CDT>(ep, n, nvalid, b);
    load_scale4(ep, n, nvalid, s);
    finish4<CDT>(rc, off, nvalid, vec, alpha, beta, v, ep, b, s);
}

// ---------------------------------------------------------------------------
// The GEMM kernel.
// ---------------------------------------------------------------------------
template <int CLS>
struct Occupancy {
    // waves per SIMD (= workgroups per CU) the tile class is sized for.
    // LDS per workgroup: 2 stages x (BM + BN) x 128 B = 128 / 64 / 32 KiB.
    // 2 waves per SIMD leave 256 VGPRs per lane for the staging registers
    // of both operands.
    static constexpr int value = CLS == TILE_256 ? 1 : 2;
};

// OUT is the output element type (DT_F32 / DT_F16 / DT_BF16 / DT_I32), or
// OUT_PARTIAL to write raw split-K partial sums to the workspace.
template <int DT, bool TA, bool TB, int CLS, int OUT>
__global__ __launch_bounds__(256, Occupancy<CLS>::value) void gemm_kernel(const GemmArgs args) {
    constexpr TileShape TS = tile_shape(CLS);
    constexpr int BM = TS.bm, BN = TS.bn, WM = TS.wm, WN = TS.wn;
    constexpr int THREADS = WM * WN * 64;
    static_assert(THREADS == 256, "launch uses 256 threads");
    constexpr int ES = dt_size(DT);
    constexpr int BK = kLdsRowBytes / ES;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int STAGE = (BM + BN) * kLdsRowBytes;
    using Acc = typename Mma<DT>::Acc;

    __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    int32_t tm, tn, g;
    tile_of_workgroup(args.tiles_m, args.tiles_n, args.band, blockIdx.x, gridDim.x, &tm, &tn, &g);
    const int z = g / args.splits, sidx = g % args.splits;
    const int M = args.M, N = args.N, K = args.K;
    const int m0 = tm * BM, n0 = tn * BN;
    const int k_lo = sidx * args.k_per_split;
    const int k_hi = min(K, k_lo + args.k_per_split);
    const int nkt = (k_hi - k_lo + BK - 1) / BK;

    const char *Ab = static_cast<const char *>(args.A) + z * args.stride_a * ES;
    const char *Bb = static_cast<const char *>(args.B) + z * args.stride_b * ES;
    const int lda_b = args.lda * ES, ldb_b = args.ldb * ES;
    const bool mn_interior = (m0 + BM <= M) && (n0 + BN <= N);

    using LoadA = std::conditional_t<TA, ColLoader<ES, BM, THREADS>, RowLoader<ES, BM, THREADS>>;
    using LoadB = std::conditional_t<TB, RowLoader<ES, BN, THREADS>, ColLoader<ES, BN, THREADS>>;
    // The 64x64 class (small outputs, short per-tile work) stages two tiles
    // ahead in registers: tile t+2 loads while tile t+1 waits in the other
    // set, so two tiles' latency overlap; the larger classes stage one.
    constexpr bool PF2 = CLS == TILE_64;
    LoadA la, la2;
    LoadB lb, lb2;

    auto load_tile = [&](int k0, LoadA &la, LoadB &lb) {
        const int64_t a_org = TA ? ((int64_t)k0 * args.lda + m0) * ES
                                 : ((int64_t)m0 * args.lda + k0) * ES;
        const int64_t b_org = TB ? ((int64_t)n0 * args.ldb + k0) * ES
                                 : ((int64_t)k0 * args.ldb + n0) * ES;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab + a_org, args.a_extent - a_org);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb + b_org, args.b_extent - b_org);
        if (mn_interior && k0 + BK <= K) {
            la.template load<false>(ra, tid, lda_b, BM, BK);
            lb.template load<false>(rb, tid, ldb_b, BN, BK);
        } else {
            la.template load<true>(ra, tid, lda_b, M - m0, K - k0);
            lb.template load<true>(rb, tid, ldb_b, N - n0, K - k0);
        }
    };

    Acc acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = Acc{0, 0, 0, 0};

    if (nkt > 0) {
        load_tile(k_lo, la, lb);
        la.store(smem, tid);
        lb.store(smem + BM * kLdsRowBytes, tid);
        if (PF2 && nkt > 1) load_tile(k_lo + BK, la2, lb2);
        __syncthreads();
    }

    const int frag_row = lane & 15, frag_chunk = lane >> 4;
    // K-tile kt from LDS stage kt & 1.  One set: tile kt+1 loads into it
    // now and goes to LDS after the MFMAs.  Two sets (PF2): tile kt+1 is
    // already in set nxt; tile kt+2 loads into set ld (stored to LDS one
    // iteration ago), then set nxt goes to LDS after the MFMAs.
    auto k_step = [&](int kt, LoadA &la_ld, LoadB &lb_ld, LoadA &la_nxt, LoadB &lb_nxt) {
        char *sa = smem + (kt & 1) * STAGE;
        char *sb = sa + BM * kLdsRowBytes;
        if constexpr (PF2) {
            if (kt + 2 < nkt) load_tile(k_lo + (kt + 2) * BK, la_ld, lb_ld);
        } else {
            if (kt + 1 < nkt) load_tile(k_lo + (kt + 1) * BK, la_nxt, lb_nxt);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            u32x4 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const u32x4 *>(
                    sa + lds_off(wm * WTM + i * 16 + frag_row, ks * 4 + frag_chunk));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[j] = *reinterpret_cast<const u32x4 *>(
                    sb + lds_off(wn * WTN + j * 16 + frag_row, ks * 4 + frag_chunk));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) Mma<DT>::run(acc[i][j], bf[j], af[i]);
        }
        if (kt + 1 < nkt) {
            char *na = smem + ((kt + 1) & 1) * STAGE;
            la_nxt.store(na, tid);
            lb_nxt.store(na + BM * kLdsRowBytes, tid);
        }
        __syncthreads();
    };
    if constexpr (PF2) {
        // tile t sits in set t & 1 (la/lb even, la2/lb2 odd)
        for (int kt = 0; kt < nkt; kt += 2) {
            k_step(kt, la, lb, la2, lb2);
            if (kt + 1 < nkt) k_step(kt + 1, la2, lb2, la, lb);
        }
    } else {
        for (int kt = 0; kt < nkt; ++kt) k_step(kt, la, lb, la, lb);
    }

    // ---- epilogue: lane holds C[m][n .. n+3] of each 16x16 block
    const int ml0 = wm * WTM + (lane & 15);
    const int nl0 = wn * WTN + 4 * (lane >> 4);
    if constexpr (OUT == OUT_PARTIAL) {
        // raw fp32 / int32 partial sums of this K slice: workspace plane g
        char *wsb = static_cast<char *>(args.ws) +
                    ((int64_t)g * M * N + (int64_t)m0 * N + n0) * 4;
        const int64_t ws_ext = (int64_t)(M - m0) * N * 4 - (int64_t)n0 * 4;
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(wsb, ws_ext);
        const bool vec = (N % 4) == 0;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int ml = ml0 + i * 16;
            if (m0 + ml >= M) continue;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int nl = nl0 + j * 16;
                const int nvalid = N - (n0 + nl);
                if (nvalid <= 0) continue;
                int v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (DT == DT_I8) v[e] = acc[i][j][e];
                    else v[e] = as_i32(acc[i][j][e]);
                }
                store_i4(rw, (ml * N + nl) * 4, nvalid, vec, v);
            }
        }
    } else {
        constexpr int CES = dt_size(OUT);
        const int64_t c_org = ((int64_t)m0 * args.ldc + n0) * CES;
        char *Cb = static_cast<char *>(args.C) + z * args.stride_c * CES + c_org;
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cb, args.c_extent - c_org);
        const bool vec = args.c_vec_ok != 0;
        const int ldc = args.ldc;
        const float alpha = args.alpha, beta = args.beta;
        const EpiState ep = make_epi<OUT == DT_I32 ? DT_F32 : OUT>(args, z, N);
        // fused epilogue: the tile's bias and scales into the (free) LDS
        float *lds_epi = reinterpret_cast<float *>(smem);
        if constexpr (OUT != DT_I32) {
            if (ep.on) {
                stage_epi<OUT>(ep, n0, N, BN, lds_epi, tid, 256);
                __syncthreads();
            }
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int ml = ml0 + i * 16;
            if (m0 + ml >= M) continue;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int nl = nl0 + j * 16;
                const int nvalid = N - (n0 + nl);
                if (nvalid <= 0) continue;
                const int off = (ml * ldc + nl) * CES;
                if constexpr (OUT == DT_I32) {
                    int v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[i][j][e];
                    store_i4(rc, off, nvalid, vec, v);
                } else {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[i][j][e];
                    if (ep.on) {
                        float b[4], s[4];
                        read_epi4(lds_epi, BN, nl, b, s);
                        finish4<OUT>(rc, off, nvalid, vec, alpha, beta, v, ep, b, s);
                    } else {
                        finish4<OUT>(rc, off, nvalid, vec, alpha, beta, v);
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Small problems: a BT x BT tile (BT = 64, 32 or 16) whose 4 waves split K
// among themselves.
//
// With few tiles and a short K (fp32 256^3: 16 tiles of 64 x 64 with 8
// K-tiles each) the loop above runs on a handful of CUs and waits out one
// memory round trip per K-tile.  Here every wave owns the whole tile and
// takes every 4th K-tile (wave w: tiles w, w+4, ...), staging them through
// its own two LDS stages with no workgroup barrier in the loop; the loads of
// its next tile are in flight while it multiplies the current one, and the
// four waves' round trips overlap.  Smaller tiles put the work on more CUs
// (256^3 on 16 x 16 tiles: 256 workgroups).  After the loop the four partial
// tiles meet in LDS and are added in wave order (a fixed order, so every run
// gives the same bits), then stored once with the usual epilogue.  No
// workspace, one launch.
// ---------------------------------------------------------------------------
template <int BT>
struct KsOccupancy {
    // LDS: 4 waves x 2 stages x 2 BT rows x 128 B = 128 / 64 / 32 KiB
    static constexpr int value = BT == 64 ? 1 : 2;
};

template <int DT, bool TA, bool TB, int OUT, int BT>
__global__ __launch_bounds__(256, KsOccupancy<BT>::value) void gemm_ks_kernel(const GemmArgs args) {
    static_assert(BT == 64 || BT == 32 || BT == 16, "tile edge 64, 32 or 16");
    constexpr int BM = BT, BN = BT, NWAVE = 4;
    constexpr int ES = dt_size(DT);
    constexpr int BK = kLdsRowBytes / ES;
    constexpr int FM = BM / 16, FN = BN / 16;
    constexpr int STAGE = (BM + BN) * kLdsRowBytes;
    constexpr int PITCH = BN + 4;                      // partial-tile row, 32-bit words (bank offset)
    static_assert(NWAVE * BM * PITCH * 4 <= NWAVE * 2 * STAGE, "partials fit the stages");
    using Acc = typename Mma<DT>::Acc;

    __shared__ __attribute__((aligned(16))) char smem[NWAVE * 2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    int32_t tm, tn, g;
    tile_of_workgroup(args.tiles_m, args.tiles_n, args.band, blockIdx.x, gridDim.x, &tm, &tn, &g);
    const int z = g;
    const int M = args.M, N = args.N, K = args.K;
    const int m0 = tm * BM, n0 = tn * BN;
    const int nkt = (K + BK - 1) / BK;

    const char *Ab = static_cast<const char *>(args.A) + z * args.stride_a * ES;
    const char *Bb = static_cast<const char *>(args.B) + z * args.stride_b * ES;
    const int lda_b = args.lda * ES, ldb_b = args.ldb * ES;
    const bool mn_interior = (m0 + BM <= M) && (n0 + BN <= N);

    // one wave loads a whole tile (64 threads)
    using LoadA = std::conditional_t<TA, ColLoader<ES, BM, 64>, RowLoader<ES, BM, 64>>;
    using LoadB = std::conditional_t<TB, RowLoader<ES, BN, 64>, ColLoader<ES, BN, 64>>;
    LoadA la;
    LoadB lb;
    auto load_tile = [&](int k0) {
        const int64_t a_org = TA ? ((int64_t)k0 * args.lda + m0) * ES
                                 : ((int64_t)m0 * args.lda + k0) * ES;
        const int64_t b_org = TB ? ((int64_t)n0 * args.ldb + k0) * ES
                                 : ((int64_t)k0 * args.ldb + n0) * ES;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab + a_org, args.a_extent - a_org);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb + b_org, args.b_extent - b_org);
        if (mn_interior && k0 + BK <= K) {
            la.template load<false>(ra, lane, lda_b, BM, BK);
            lb.template load<false>(rb, lane, ldb_b, BN, BK);
        } else {
            la.template load<true>(ra, lane, lda_b, M - m0, K - k0);
            lb.template load<true>(rb, lane, ldb_b, N - n0, K - k0);
        }
    };

    Acc acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = Acc{0, 0, 0, 0};

    char *const wl = smem + wave * 2 * STAGE;     // this wave's two stages
    const int frag_row = lane & 15, frag_chunk = lane >> 4;
    if (wave < nkt) {
        load_tile(wave * BK);
        la.store(wl, lane);
        lb.store(wl + BM * kLdsRowBytes, lane);
    }
    for (int kt = wave, j = 0; kt < nkt; kt += NWAVE, ++j) {
        const char *sa = wl + (j & 1) * STAGE;
        const char *sb = sa + BM * kLdsRowBytes;
        const bool more = kt + NWAVE < nkt;
        if (more) load_tile((kt + NWAVE) * BK);
        // this wave's LDS writes of the tile are done before any lane reads
        // them (a wave's LDS operations complete in order; the clobber keeps
        // the compiler from moving the reads above the writes)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            u32x4 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const u32x4 *>(sa + lds_off(i * 16 + frag_row, ks * 4 + frag_chunk));
#pragma unroll
            for (int jj = 0; jj < FN; ++jj)
                bf[jj] = *reinterpret_cast<const u32x4 *>(sb + lds_off(jj * 16 + frag_row, ks * 4 + frag_chunk));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int jj = 0; jj < FN; ++jj) Mma<DT>::run(acc[i][jj], bf[jj], af[i]);
        }
        if (more) {
            // the other stage: its reads (the previous tile) were consumed by
            // this wave's MFMAs above, so they are complete
            char *na = wl + ((j + 1) & 1) * STAGE;
            asm volatile("" ::: "memory");
            la.store(na, lane);
            lb.store(na + BM * kLdsRowBytes, lane);
        }
    }

    // ---- the four partial tiles into LDS (raw 32-bit values), then summed in
    // wave order; lane l of block (i, j) holds row i*16 + l%16, columns
    // j*16 + 4(l/16) .. +3
    __syncthreads();
    u32 *part = reinterpret_cast<u32 *>(smem);
    {
        u32 *mine = part + wave * BM * PITCH;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int jj = 0; jj < FN; ++jj) {
                const int r = i * 16 + frag_row, c = jj * 16 + 4 * frag_chunk;
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (DT == DT_I8) w[e] = (u32)acc[i][jj][e];
                    else w[e] = as_u32(acc[i][jj][e]);
                }
                *reinterpret_cast<u32x4 *>(mine + r * PITCH + c) = w;
            }
    }
    __syncthreads();

    constexpr int CES = dt_size(OUT == DT_I32 ? DT_I32 : OUT);
    const int64_t c_org = ((int64_t)m0 * args.ldc + n0) * CES;
    char *Cb = static_cast<char *>(args.C) + z * args.stride_c * CES + c_org;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cb, args.c_extent - c_org);
    const bool vec = args.c_vec_ok != 0;
    const int ldc = args.ldc;
    const float alpha = args.alpha, beta = args.beta;
    [[maybe_unused]] const EpiState ep = make_epi<OUT == DT_I32 ? DT_F32 : OUT>(args, z, N);
    // BM rows x BN / 4 column quads, spread over the threads
    constexpr int QPR = BN / 4;
    for (int q = tid; q < BM * QPR; q += 256) {
        const int r = q / QPR, c = (q % QPR) * 4;
        const int nvalid = N - (n0 + c);
        if (m0 + r >= M || nvalid <= 0) continue;
        const int off = (r * ldc + c) * CES;
        if constexpr (DT == DT_I8) {
            int s[4] = {0, 0, 0, 0};
#pragma unroll
            for (int w = 0; w < NWAVE; ++w) {
                const u32x4 p = *reinterpret_cast<const u32x4 *>(part + w * BM * PITCH + r * PITCH + c);
#pragma unroll
                for (int e = 0; e < 4; ++e) s[e] += (int)p[e];
            }
            if constexpr (OUT == DT_I32) {
                store_i4(rc, off, nvalid, vec, s);
            } else {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (float)s[e];
                finish4<OUT>(rc, off, nvalid, vec, alpha, beta, v, ep, n0 + c);
            }
        } else {
            float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < NWAVE; ++w) {
                const u32x4 p = *reinterpret_cast<const u32x4 *>(part + w * BM * PITCH + r * PITCH + c);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] += as_f32(p[e]);
            }
            finish4<OUT>(rc, off, nvalid, vec, alpha, beta, v, ep, n0 + c);
        }
    }
}

}  // namespace
}  // namespace tcg
