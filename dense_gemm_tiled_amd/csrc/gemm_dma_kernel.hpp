// gemm_dma_kernel.hpp -- the GEMM kernel for gfx950 whose operand tiles go
// from HBM straight into LDS (buffer loads with the LDS flag), for 16-bit and
// int8 inputs whose rows start on 16-byte boundaries.
//
// Same computation and epilogue as gemm_kernel (C = alpha*op(A)op(B) +
// beta*C, accumulator in registers for the whole K loop of a slice, C or the
// slice's partial sums written once; tessl "Architecture", "Cooperative
// Destination Accumulation"), with a static schedule.  Tile shapes:
//
//   256 x 256, 4 waves of 128 x 128 (256 AGPRs per lane), one workgroup per
//     CU; or 8 waves of 128 x 64, two per SIMD;
//   128 x 128, 4 waves of 64 x 64, two workgroups per CU (mid-size outputs
//     and split-K).
//
//   * per K-tile (128 bytes of K: 64 bf16/f16 or 128 int8) the operand tiles
//     arrive as direct-to-LDS loads of 1 KiB, issued by 4 waves; NST LDS
//     stages (2, or 4 where one workgroup per CU has the LDS to spare) hold
//     tiles t .. t+NST-1;
//   * the MFMAs of a K-tile run in two sub-steps.  While one sub-step runs,
//     the fragments of the next are read from LDS into a second register
//     set, one read between every few MFMAs;
//   * one barrier per K-tile, between the sub-steps: after it, tile t+1 is
//     visible to every wave and the stage of tile t is free, so the loads of
//     tile t+NST are issued into it during the second sub-step;
//   * K-contiguous operands are read with ds_read_b128; M/N-contiguous ones
//     with the gfx950 transposing LDS reads (ds_read_b64_tr_b16 / _b8),
//     which hand every lane the K-run of one column -- no transpose pass and
//     no register shuffles (tensorcore "GEMM", "Transposes": a transpose is a
//     choice of strides);
//   * few instructions besides the MFMAs: a wave issues one instruction per 4
//     cycles and an MFMA block takes 16, so a run of more than three other
//     instructions holds up the matrix core.  The loads go four to an M0
//     write (their immediate offset moves the LDS address and the buffer
//     offset alike), and the next tile's buffer resources advance by one
//     K-tile with scalar adds;
//   * interior tiles are stored through LDS, 16 bytes per lane along the
//     rows (32-bit outputs where C's rows are whole 16-byte chunks);
//   * with beta != 0 and a 16-bit C, an interior tile of the 256 x 256 ring
//     loads its C tile into LDS during the last two K-tiles (which load no
//     operands), into slots those K-tiles free, and stages its results in
//     the one slot left over.
//
// The MFMAs, the LDS-bound loads and the barrier are inline assembly.  The
// accumulators are pinned to AGPRs (operand constraint "+a", destination =
// source C), the loads are invisible to the compiler (so it cannot order the
// LDS reads of one stage behind the loads into the other), and every
// assembly statement is volatile, so the interleave below is the issue order.
// The waits the compiler cannot see are written out: before each barrier a
// vmcnt that leaves only the newer tiles' loads in flight, vmcnt(0) at the
// end of the loop, and wait states between the last MFMA
// and the first read of the accumulators.
//
// LDS layouts (bytes; chosen so that the reads below hit every bank once per
// 256 bytes and the DMA writes stay contiguous).  R is the tile extent along
// M (A) or N (B):
//   K-contiguous tile: R rows x 128 B; 16-byte chunk c of row r at position
//     c ^ ((r & 7) ^ ((r >> 3) & 1)).
//   M/N-contiguous tile, 16-bit: 64 k-rows x 2R B; 32-byte segment s (16
//     columns) of row k at position s ^ ((k & 3) | ((k >> 3) & 1) << 2).
//   M/N-contiguous tile, int8, R = 256: 128 k-rows x 256 B; 16-byte segment s
//     of row k at position s ^ ((k & 7) | ((k >> 4) & 1) << 3); R = 128:
//     128 k-rows x 128 B, segment s at s ^ (((k >> 1) & 3) | ((k >> 4) & 1) << 2)
//     (two rows share 256 bytes of banks, so the row parity picks the half).
//
// Ragged edges (tessl "Architecture", "Edge-Slice Support"): rows past M or
// N only feed outputs that are never stored, and buffer range checks return
// zero past the operand; k past K is zeroed per 16-byte chunk (the planner
// sends this kernel only shapes whose K is a whole number of chunks).

#pragma once

#include "gemm_kernel.hpp"

namespace tcg {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
#define TCG_LDS __attribute__((address_space(3)))

// An offset past every buffer range (ranges are < 2^31 bytes; the offset plus
// the 16-byte access does not wrap 32 bits): such a load reads zeros.
constexpr int kOobOffset = INT32_MIN;

// K-contiguous rows: position of chunk c of row r is c ^ swz_kc(r).  (A
// swizzle whose 32-lane groups hit 32 distinct 16-byte slots of a 512-byte
// window left SQ_LDS_BANK_CONFLICT exactly where it was: the counter books
// about 4 cycles on every 64-lane ds_read_b128, whatever the addresses.)
__device__ inline int swz_kc(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// M/N-contiguous swizzle for LDS rows of RB bytes (16-bit: 32-byte segments;
// int8: 16-byte segments).
template <int ES, int RB>
__device__ inline int swz_mc(int k) {
    if constexpr (ES == 2) return (k & 3) | (((k >> 3) & 1) << 2);
    else if constexpr (RB == 256) return (k & 7) | (((k >> 4) & 1) << 3);
    else return ((k >> 1) & 3) | (((k >> 4) & 1) << 2);
}

// The row bits each swizzle reads.
template <int ES, bool MC, int RB>
constexpr int swz_bits() {
    if constexpr (!MC) return 0xF;
    else if constexpr (ES == 2) return 0xB;
    else if constexpr (RB == 256) return 0x17;
    else return 0x16;
}

constexpr int bit_count(int v) { return v == 0 ? 0 : (v & 1) + bit_count(v >> 1); }

// The bits of u selected by mask, packed to the bottom (and the reverse).
constexpr int bits_extract(int u, int mask) {
    int r = 0, o = 0;
    for (int b = 0; b < 8; ++b)
        if ((mask >> b) & 1) r |= ((u >> b) & 1) << o++;
    return r;
}
constexpr int bits_deposit(int c, int mask) {
    int r = 0, o = 0;
    for (int b = 0; b < 8; ++b)
        if ((mask >> b) & 1) r |= ((c >> o++) & 1) << b;
    return r;
}

// Raw buffer resource as four SGPRs (same fields as make_rsrc).
__device__ inline i32x4 rsrc4(const void *base, int64_t bytes) {
    const int32_t n = bytes <= 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)bytes);
    const uint64_t a = (uint64_t)base;
    return i32x4{(int)(uint32_t)a, (int)((a >> 32) & 0xFFFF), n, kRsrcWord3};
}

// 16 bytes per lane from buffer offset `voff` to LDS byte address
// lds + 16 * lane.  M0 holds the LDS address; a load with the LDS flag needs
// one wait state after an SALU write of M0.  (M0 is listed as clobbered; the
// compiler reserves it and sets it itself wherever it needs it.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void dma16(i32x4 rsrc, uint32_t lds, int voff) {
    asm volatile("s_mov_b32 m0, %0\n\t"
                 "s_nop 0\n\t"
                 "buffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

// The same loads in groups of kLoadGroup sharing one M0 write: the
// instruction's immediate offset is added to both the buffer offset and the
// LDS address, so load j of a group (M0 = the group's first 1 KiB) takes
// offset j KiB and a buffer offset j KiB lower.  set_m0 writes M0 with an
// SALU add; the caller issues another instruction (an MFMA) before the first
// load of the group, the one wait state such a load needs after an SALU
// write of M0.  (The add writes SCC, so SCC is listed as clobbered: the
// compiler must not keep a comparison in it across the statement.)
constexpr int kLoadGroup = 4;
__device__ inline void set_m0(uint32_t lds, uint32_t off) {
    asm volatile("s_add_u32 m0, %0, %1"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "s"(__builtin_amdgcn_readfirstlane(off))
                 : "m0", "scc");
}
__device__ inline void dma16_m0(i32x4 rsrc, int voff, int j) {
    switch (j) {
    case 0: asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc) : "memory"); break;
    case 1: asm volatile("buffer_load_dwordx4 %0, %1, 0 offen offset:1024 lds" ::"v"(voff), "s"(rsrc) : "memory"); break;
    case 2: asm volatile("buffer_load_dwordx4 %0, %1, 0 offen offset:2048 lds" ::"v"(voff), "s"(rsrc) : "memory"); break;
    default: asm volatile("buffer_load_dwordx4 %0, %1, 0 offen offset:3072 lds" ::"v"(voff), "s"(rsrc) : "memory"); break;
    }
}
#pragma clang diagnostic pop

// Wait for this wave's LDS reads and all but its newest VM loads, then for
// the other waves.
template <int VM>
__device__ inline void wait_barrier_vm() {
    static_assert(VM >= 0 && VM <= 63, "vmcnt is a 6-bit count");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VM) : "memory");
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// One MFMA on a 16-byte fragment of each operand per lane: MS = 16 is the
// 16 x 16 output block (16x16x32 for 16-bit inputs, 16x16x64 for int8; 4
// accumulators per lane), MS = 32 the 32 x 32 block (32x32x16, 32x32x32; 16
// accumulators per lane, twice the cycles per instruction).
template <int DT, int MS>
struct MmaAsm;

template <>
struct MmaAsm<DT_BF16, 16> {
    using Acc = f32x4;
    __device__ static inline void run(Acc &acc, const u32x4 &b, const u32x4 &a) {
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
    }
};

template <>
struct MmaAsm<DT_F16, 16> {
    using Acc = f32x4;
    __device__ static inline void run(Acc &acc, const u32x4 &b, const u32x4 &a) {
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
    }
};

template <>
struct MmaAsm<DT_I8, 16> {
    using Acc = i32x4;
    __device__ static inline void run(Acc &acc, const u32x4 &b, const u32x4 &a) {
        asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
    }
};

template <>
struct MmaAsm<DT_BF16, 32> {
    using Acc = f32x16;
    __device__ static inline void run(Acc &acc, const u32x4 &b, const u32x4 &a) {
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
    }
};

template <>
struct MmaAsm<DT_F16, 32> {
    using Acc = f32x16;
    __device__ static inline void run(Acc &acc, const u32x4 &b, const u32x4 &a) {
        asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
    }
};

template <>
struct MmaAsm<DT_I8, 32> {
    using Acc = i32x16;
    __device__ static inline void run(Acc &acc, const u32x4 &b, const u32x4 &a) {
        asm volatile("v_mfma_i32_32x32x32_i8 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
    }
};

// One operand's share of the DMA of a tile of R rows (M or N indices) x 128
// bytes of K: R / 8 loads of 1 KiB, LPW = R / (8 NDW) per loading wave (NDW
// loading waves).  MC: the operand is M/N-contiguous in memory (global row =
// one k).  Load u of wave w fills tile rows (LPW w + u) * RPI + lane / LPR.
// A lane's byte offset is a lane part, which depends on u only through the
// swizzle (the u bits in UMASK: NCLS variants), plus u * RPI rows, which is
// wave-uniform.
template <int ES, bool MC, int R, int NDW>
struct DmaLoader {
    static constexpr int RB = MC ? R * ES : kLdsRowBytes;          // LDS row bytes
    static constexpr int LPR = RB / 16;                            // lanes per row
    static constexpr int RPI = 64 / LPR;                           // rows per load
    static constexpr int LPW = R / 8 / NDW;                        // loads per wave
    static_assert(LPW >= 2 && (LPW & (LPW - 1)) == 0, "loads per wave: a power of two");
    static constexpr int UMASK = (swz_bits<ES, MC, RB>() / RPI) & (LPW - 1);
    static constexpr int NCLS = 1 << bit_count(UMASK);
    int lane_off[NCLS];  // [bits_extract(u, UMASK)]: lane part of the byte offset
    int row0;            // MC: tile row (k) of this lane for u = 0
    int kfirst[NCLS];    // KC: first k (elements) of this lane's chunk
    int ld_bytes;

    __device__ static inline int row_of(int wave, int lane, int u) {
        return (wave * LPW + u) * RPI + lane / LPR;
    }
    __device__ static inline int col_of(int r, int q) {
        if constexpr (MC) {
            if constexpr (ES == 2) return (((q >> 1) ^ swz_mc<2, RB>(r)) << 5) + ((q & 1) << 4);
            else return (q ^ swz_mc<1, RB>(r)) << 4;
        } else {
            return (q ^ swz_kc(r)) << 4;
        }
    }

    __device__ inline void init(int wave, int lane, int ldb) {
        ld_bytes = ldb;
        row0 = row_of(wave, lane, 0);
#pragma unroll
        for (int c = 0; c < NCLS; ++c) {
            const int r = row_of(wave, lane, bits_deposit(c, UMASK));
            lane_off[c] = row0 * ldb + col_of(r, lane % LPR);
            kfirst[c] = (col_of(r, lane % LPR) >> 4) * (16 / ES);
        }
    }

    // Byte offset of load u for a tile with k_valid valid k (<= tile depth).
    // KMASK: chunks past K get an offset outside the buffer, which loads
    // zeros; without it (K a whole number of tiles) every tile the loop reads
    // is full, and a tile past the end has an empty buffer range anyway.
    template <bool KMASK>
    __device__ inline int offset(int u, int k_valid) const {
        const int c = bits_extract(u, UMASK);
        const int off = lane_off[c] + u * RPI * ld_bytes;
        if constexpr (!KMASK) return off;
        const bool in = MC ? (row0 < k_valid - u * RPI) : (kfirst[c] < k_valid);
        return in ? off : kOobOffset;
    }
};

// LDS fragment reads.  KC: ds_read_b128 of a K-contiguous tile; MC: two
// transposing reads of an M/N-contiguous tile of extent R.  A K-tile (128
// bytes of K) holds NKS k-steps of one MFMA each.  MS = 16: lane l gets the
// K-run {8*(l/16) .. +7} (16-bit) or {16*(l/16) .. +15} (int8) of k-step ks
// for row/column (l % 16) of 16-block i -- the operand layout of the
// 16x16x32 and 16x16x64 MFMAs.  MS = 32: lane l gets the K-run
// {8*(l/32) .. +7} / {16*(l/32) .. +15} for row/column (l % 32) of 32-block
// i (32x32x16, 32x32x32).  NB: blocks per wave.
template <int ES, bool MC, int R, int NB, int MS>
struct FragReader {
    static constexpr int RB = R * ES;   // MC: LDS row bytes
    static constexpr int NKS = MS == 16 ? 2 : 4;   // k-steps per K-tile
    int base[MC ? NB : NKS];            // lane byte offsets inside an operand tile

    __device__ inline void init(int lane, int blk0) {
        const int l16 = lane & 15, g = lane >> 4;
        if constexpr (MC) {
            // the transposing reads serve 16 lanes each: with MS = 32 lane
            // group g covers k-half g / 2 and column half g % 2 of the block
            const int kg = MS == 16 ? g : g >> 1;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int seg = blk0 / 16 + (MS == 16 ? j : 2 * j + (g & 1));
                if constexpr (ES == 2) {
                    const int k = 8 * kg + (l16 >> 2);
                    base[j] = k * RB + ((seg ^ swz_mc<2, RB>(k)) << 5) + ((lane & 3) << 3);
                } else {
                    const int k = 16 * kg + (l16 >> 1);
                    base[j] = k * RB + ((seg ^ swz_mc<1, RB>(k)) << 4) + ((lane & 1) << 3);
                }
            }
        } else {
            const int row = MS == 16 ? l16 : (lane & 31);
            const int part = MS == 16 ? g : lane >> 5;      // 16-byte chunk of the k-step
            constexpr int CPS = MS == 16 ? 4 : 2;           // chunks per k-step
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                base[ks] = (blk0 + row) * kLdsRowBytes + (((ks * CPS + part) ^ swz_kc(row)) << 4);
        }
    }

    // tile: LDS byte address of the operand tile.
    __device__ inline void read(uint32_t tile, int ks, int i, u32x4 &out) const {
        if constexpr (MC) {
            // rows advance by the k of one k-step per step, by 4 / 8 for the
            // second half of the K-run (the swizzles read none of those bits)
            constexpr int KS_ROWS = (ES == 2 ? 32 : 64) * 16 / MS, H_ROWS = ES == 2 ? 4 : 8;
            const uint32_t p = tile + base[i] + ks * KS_ROWS * RB;
            i32x2 lo, hi;
            if constexpr (ES == 2) {
                lo = __builtin_bit_cast(
                    i32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((TCG_LDS s16x4 *)(size_t)p));
                hi = __builtin_bit_cast(i32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                   (TCG_LDS s16x4 *)(size_t)(p + H_ROWS * RB)));
            } else {
                lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((TCG_LDS i32x2 *)(size_t)p);
                hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (TCG_LDS i32x2 *)(size_t)(p + H_ROWS * RB));
            }
            out = u32x4{(u32)lo[0], (u32)lo[1], (u32)hi[0], (u32)hi[1]};
        } else {
            // the block offset as a constant pointer step, so that it becomes
            // the instruction's immediate offset
            const TCG_LDS char *p = (const TCG_LDS char *)(size_t)(tile + base[ks]);
            out = *(const TCG_LDS u32x4 *)(p + i * MS * kLdsRowBytes);
        }
    }
};

// The static interleave of a sub-step: QN MFMAs; in sub-step 0 the NR
// fragment reads of sub-step 1, in sub-step 1 the ND loads of tile t+NST and
// the NR fragment reads of tile t+1 alternating (load first).  Operation o of
// n goes after MFMA (o * QN) / n, so MFMA q is followed by operations
// op_begin(q) .. op_begin(q + 1) - 1.
constexpr int op_begin(int q, int n, int qn) { return (q * n + qn - 1) / qn; }

// The ring's sub-steps interleave reads and loads, alternating (load first)
// while both remain, then the rest of the longer kind: op o is load
// ring_op_load(o) or read ring_op_read(o) (-1: the other kind).
constexpr int ring_op_load(int o, int nl, int nr) {
    const int pair = 2 * (nl < nr ? nl : nr);
    if (o < pair) return (o & 1) == 0 ? o >> 1 : -1;
    return nl > nr ? o - pair + nr : -1;
}
constexpr int ring_op_read(int o, int nl, int nr) {
    const int pair = 2 * (nl < nr ? nl : nr);
    if (o < pair) return (o & 1) == 1 ? o >> 1 : -1;
    return nl > nr ? -1 : o - pair + nl;
}
// M0 moves to a load group before the MFMA that precedes the group's first
// load, so no other load may sit between that MFMA and the group's first
// load.
constexpr bool ring_groups_ok(int nl, int nr, int qn) {
    for (int q = 0; q < qn; ++q) {
        bool load_seen = false;
        for (int o = op_begin(q, nl + nr, qn); o < op_begin(q + 1, nl + nr, qn); ++o) {
            const int d = ring_op_load(o, nl, nr);
            if (d < 0) continue;
            if (d % kLoadGroup == 0 && load_seen) return false;
            load_seen = true;
        }
    }
    return nl % kLoadGroup == 0;
}

// Buffer source of one operand's K-tiles: the resource of the next tile to
// load (based at the tile's origin, ranging to the end of the operand, at
// most 2^31 - 1 bytes), advanced one K-tile at a time with scalar adds.  A
// tile inside the K slice has its origin inside the operand, so its range is
// never empty.  Device addresses have 48 bits, so the base's high word fits
// the resource's 16-bit field as it is.
struct RingSrc {
    uint64_t base, rem, step;   // tile address, bytes left to the end, bytes per K-tile
    // inside: the tile lies inside the K slice (else an empty range: its
    // loads fetch nothing and fill their LDS with zeros)
    __device__ inline i32x4 rsrc(bool inside = true) const {
        const uint32_t n = !inside ? 0u : (rem >> 31) != 0 ? 0x7FFFFFFFu : (uint32_t)rem;
        return i32x4{(int)(uint32_t)base, (int)(uint32_t)(base >> 32), (int)n, kRsrcWord3};
    }
    __device__ inline void advance() {
        base += step;
        rem -= step;
    }
};

// Buffer offset of load j of a group, whose immediate offset adds j KiB
// (unsigned arithmetic: an out-of-range offset stays out of range).
__device__ inline int group_voff(int off, int j) { return (int)((uint32_t)off - (uint32_t)(j * 1024)); }

// Epilogue variants of the kernel: beta == 0 and no fused epilogue; beta != 0
// (16-bit C tiles staged through LDS); the fused epilogue (bias and
// activation, any beta, C_old read per block).  The last one is a separate
// instantiation so that its code does not weigh on the other two.
constexpr int EPI_PLAIN = 0, EPI_BETA = 1, EPI_FUSED = 2;

// BM x BN tile, NW waves (2 along M, NW/2 along N), OCC workgroups per CU;
// EPI: one of the epilogue variants above; NST LDS stages (2, 4 or 5): tiles
// kt+1 .. kt+NST-1 are in flight while tile kt is computed -- except that
// NST = 5 where five stages do not fit (the 256 x 256 tile) means a ring of
// five slots of one operand tile each (BM == BN; 160 KiB), see below; MS:
// the MFMA output block (16 or 32).
//
// The ring.  Operand tiles are items: item 2t is A of K-tile t, item 2t+1
// its B, held in slot item % 5.  At the barrier in the middle of K-tile t
// (after sub-step 0, whose reads fetch the rest of tile t into registers)
// the slots of items 2t and 2t+1 are free.  Sub-step 0 of tile t loads item
// 2t+4 (A of tile t+2, into the slot item 2t-1 left at the previous
// barrier); sub-step 1 loads item 2t+5 (B of tile t+2, into the slot item 2t
// just left).  So both sub-steps issue half of a tile's loads -- with two
// stages all of them go out in sub-step 1 -- still with one barrier per
// K-tile, and tile t+2 has from then to the middle of tile t+1 to land.
template <int DT, bool TA, bool TB, int OUT, int BM, int BN, int NW, int OCC, bool KMASK,
          int EPI, int NST, int MS>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                          amdgpu_waves_per_eu(NW / 4 * OCC, NW / 4 * OCC)))
void gemm_dma_kernel(const GemmArgs args) {
    constexpr int ES = dt_size(DT);
    static_assert(ES == 2 || ES == 1, "direct-to-LDS kernel: 16-bit and int8 inputs");
    static_assert(NW == 4 || NW == 8, "4 or 8 waves");
    constexpr int BK = kLdsRowBytes / ES;
    constexpr bool A_MC = TA, B_MC = !TB;
    // waves: 2 along M, NW/2 along N; each owns WTM x WTN of C
    constexpr int WNW = NW / 2, WTM = BM / 2, WTN = BN / WNW;
    static_assert(MS == 16 || MS == 32, "16x16 or 32x32 MFMA blocks");
    constexpr int FM = WTM / MS, FN = WTN / MS;
    static_assert(FM >= 1 && FN >= 1, "the wave tile holds whole MFMA blocks");
    // a K-tile is two sub-steps (one barrier between them) of KSUB k-steps
    constexpr int KSUB = MS == 16 ? 1 : 2;
    constexpr int QN = KSUB * FM * FN;  // MFMAs per wave and sub-step
    constexpr int NR = KSUB * (FM + FN);   // fragment reads per sub-step
    // The loads are issued by 4 waves: all of them with 4 waves; with 8, the
    // second four only, so that while a loading wave waits to issue a load
    // the other wave on its SIMD keeps the matrix core busy.
    constexpr int NDW = 4;
    using LoadA = DmaLoader<ES, A_MC, BM, NDW>;
    using LoadB = DmaLoader<ES, B_MC, BN, NDW>;
    constexpr int LPA = LoadA::LPW, LPB = LoadB::LPW;   // loads per loading wave
    constexpr int ND = LPA + LPB;                       // ... and tile
    constexpr int A_BYTES = BM * kLdsRowBytes;          // [A tile | B tile]
    constexpr int STAGE = (BM + BN) * kLdsRowBytes;
    using Mma = MmaAsm<DT, MS>;
    using Acc = typename Mma::Acc;

    static_assert(NST == 2 || NST == 4 || NST == 5, "2, 4 or 5 stages, or the ring of 5 slots");
    constexpr int kLdsMax = 160 * 1024;
    constexpr bool RING = NST == 5 && 5 * STAGE > kLdsMax;
    static_assert(!RING || BM == BN, "the ring's slots hold either operand tile");
    constexpr int SLOT = A_BYTES;                        // ring: one operand tile
    constexpr int LDS_BYTES = RING ? 5 * SLOT : NST * STAGE;
    static_assert(RING || (NST - 1) * ND <= 63, "loads in flight fit vmcnt");
    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
    const uint32_t lds = (uint32_t)(size_t)(TCG_LDS char *)smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wm = wave / WNW, wn = wave % WNW;

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

    const int dwave = wave % NDW;                 // index among the loading waves
    const bool loads = wave >= NW - NDW;          // wave-uniform
    LoadA la;
    LoadB lb;
    la.init(dwave, lane, args.lda * ES);
    lb.init(dwave, lane, args.ldb * ES);
    FragReader<ES, A_MC, BM, FM, MS> fa;
    FragReader<ES, B_MC, BN, FN, MS> fb;
    fa.init(lane, wm * WTM);
    fb.init(lane, wn * WTN);

    // Buffer resources of tile kt, based at its origin; a tile past the end
    // of the K slice gets empty ranges (its loads fetch nothing and read
    // zeros, into a stage nobody reads).
    struct TileSrc {
        i32x4 ra, rb;
        int kv;
    };
    auto tile_src = [&](int kt) {
        TileSrc s;
        const int k0 = k_lo + kt * BK;
        const int64_t a_org = A_MC ? ((int64_t)k0 * args.lda + m0) * ES
                                   : ((int64_t)m0 * args.lda + k0) * ES;
        const int64_t b_org = B_MC ? ((int64_t)k0 * args.ldb + n0) * ES
                                   : ((int64_t)n0 * args.ldb + k0) * ES;
        const bool past = k0 >= k_hi;
        s.ra = rsrc4(Ab + a_org, past ? 0 : args.a_extent - a_org);
        s.rb = rsrc4(Bb + b_org, past ? 0 : args.b_extent - b_org);
        s.kv = min(BK, k_hi - k0);
        return s;
    };
    // the source of an operand's tile t0 (origin k_lo + t0 BK), from which the
    // loop advances one K-tile at a time
    [[maybe_unused]] auto ring_src = [&](int t0, const char *base, int64_t extent, bool mc,
                                         int64_t ld, int mn0) {
        const int64_t k0 = k_lo + (int64_t)t0 * BK;
        const int64_t org = mc ? (k0 * ld + mn0) * ES : ((int64_t)mn0 * ld + k0) * ES;
        RingSrc r;
        r.base = (uint64_t)(base + org);
        r.rem = (uint64_t)(extent - org);
        r.step = (uint64_t)(mc ? (int64_t)BK * ld * ES : (int64_t)BK * ES);
        return r;
    };
    // ring: load d of an A item (0 .. LPA-1) or a B item (0 .. LPB-1) into
    // slot address `slot`
    [[maybe_unused]] auto dma_a = [&](const TileSrc &s, uint32_t slot, int d) {
        if (loads) dma16(s.ra, slot + (dwave * LPA + d) * 1024, la.template offset<KMASK>(d, s.kv));
    };
    [[maybe_unused]] auto dma_b = [&](const TileSrc &s, uint32_t slot, int d) {
        if (loads) dma16(s.rb, slot + (dwave * LPB + d) * 1024, lb.template offset<KMASK>(d, s.kv));
    };
    // DMA load number d (0 .. ND-1) of a tile: A first, then B.
    auto dma = [&](const TileSrc &s, uint32_t stage, int d) {
        if (!loads) return;
        if (d < LPA)
            dma16(s.ra, stage + (dwave * LPA + d) * 1024, la.template offset<KMASK>(d, s.kv));
        else
            dma16(s.rb, stage + A_BYTES + (dwave * LPB + d - LPA) * 1024,
                  lb.template offset<KMASK>(d - LPA, s.kv));
    };

    Acc acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = Acc{};

    // fragments of one sub-step: [k-step of the sub-step][block]
    u32x4 a0[KSUB][FM], b0[KSUB][FN], a1[KSUB][FM], b1[KSUB][FN];

    // fragment read number r (0 .. NR-1) of sub-step sub: per k-step, B
    // blocks, then A
    // (A tile at a_at, B tile at b_at)
    auto read2 = [&](uint32_t a_at, uint32_t b_at, int sub, int r, u32x4 (&af)[KSUB][FM],
                     u32x4 (&bf)[KSUB][FN]) {
        const int kk = r / (FM + FN), rr = r % (FM + FN), ks = sub * KSUB + kk;
        if (rr < FN) fb.read(b_at, ks, rr, bf[kk][rr]);
        else fa.read(a_at, ks, rr - FN, af[kk][rr - FN]);
    };
    auto read = [&](uint32_t stage, int sub, int r, u32x4 (&af)[KSUB][FM],
                    u32x4 (&bf)[KSUB][FN]) { read2(stage, stage + A_BYTES, sub, r, af, bf); };
    // MFMA number q (0 .. QN-1) of a sub-step: k-step major
    auto mma = [&](int q, const u32x4 (&af)[KSUB][FM], const u32x4 (&bf)[KSUB][FN]) {
        const int kk = q / (FM * FN), qq = q % (FM * FN);
        Mma::run(acc[qq / FN][qq % FN], bf[kk][qq % FN], af[kk][qq / FN]);
    };

    // Sub-step 0 of the tile in `cur`: MFMAs on (a0, b0) and the reads of
    // sub-step 1.
    auto sub0 = [&](uint32_t cur) {
#pragma unroll
        for (int q = 0; q < QN; ++q) {
            mma(q, a0, b0);
#pragma unroll
            for (int r = op_begin(q, NR, QN); r < op_begin(q + 1, NR, QN); ++r)
                read(cur, 1, r, a1, b1);
        }
    };
    // The ring's sub-steps: MFMAs on one register set, NR fragment reads into
    // the other, and NL loads, the reads and loads alternating while both
    // remain (loads first).  rd(r) and ld(d) issue read r and load d; grp(g)
    // points M0 at load group g, before the MFMA that precedes the group's
    // first load.
    [[maybe_unused]] auto ring_sub = [&](auto nl_tag, const u32x4 (&af)[KSUB][FM],
                                         const u32x4 (&bf)[KSUB][FN], auto &&rd, auto &&ld,
                                         auto &&grp) {
        constexpr int NL = decltype(nl_tag)::value;
        static_assert(ring_groups_ok(NL, NR, QN), "a load group starts first in its MFMA gap");
#pragma unroll
        for (int q = 0; q < QN; ++q) {
#pragma unroll
            for (int o = op_begin(q, NL + NR, QN); o < op_begin(q + 1, NL + NR, QN); ++o) {
                const int d = ring_op_load(o, NL, NR);
                if (d >= 0 && d % kLoadGroup == 0) grp(d / kLoadGroup);
            }
            mma(q, af, bf);
#pragma unroll
            for (int o = op_begin(q, NL + NR, QN); o < op_begin(q + 1, NL + NR, QN); ++o) {
                const int d = ring_op_load(o, NL, NR);
                if (d >= 0) ld(d);
                else rd(ring_op_read(o, NL, NR));
            }
        }
    };

    // fused epilogue: the tile's bias and alpha * scale go into LDS of their
    // own at the start, their loads issued ahead of the first tiles' (the
    // epilogue then reads them with no wait; the loop's barriers publish them)
    constexpr int EPI_LDS = EPI == EPI_FUSED && OUT != DT_I32 && OUT != OUT_PARTIAL ? 2 * BN : 1;
    // (declared only where used; where the stages take all 160 KiB of LDS --
    // the ring, five 128 x 128 stages -- the bias and scales wait in
    // registers and go into the first stage once the loop is done)
    constexpr bool EPI_AFTER = EPI_LDS > 1 && LDS_BYTES + EPI_LDS * 4 > kLdsMax;
    float *epi_smem = nullptr;
    if constexpr (EPI_AFTER) {
        epi_smem = reinterpret_cast<float *>(smem);
    } else if constexpr (EPI_LDS > 1) {
        __shared__ __attribute__((aligned(16))) float epi_buf[EPI_LDS];
        epi_smem = epi_buf;
    }
    [[maybe_unused]] float epi_b = 0.f, epi_s = 1.f;
    if constexpr (EPI_LDS > 1) {
        if (tid < BN)
            load_epi1<OUT>(make_epi<OUT>(args, z, N), n0 + tid, N, epi_b, epi_s);
    }
    // beta != 0 with a 16-bit C tile inside C: the epilogue reads C_old from
    // an LDS image of the tile (below).  On the ring with at least two
    // K-tiles the image's four 64-row quarters load during the last two
    // iterations, which load no operands, into slots free by then (c_pf);
    // cq0 .. cq3: LDS addresses of the quarters, cfree: the fifth slot, free
    // once the loop is done.
    constexpr bool C16 = EPI == EPI_BETA && (OUT == DT_F16 || OUT == DT_BF16);
    [[maybe_unused]] const bool c_pf = C16 && RING && args.beta != 0.f && args.c_dma_ok != 0 &&
                                       m0 + BM <= M && n0 + BN <= N && nkt >= 2;
    [[maybe_unused]] uint32_t cq0 = lds, cq1 = lds, cq2 = lds, cq3 = lds, cfree = lds;
    if constexpr (RING) {
      if (nkt > 0) {
        // items 0 .. 3 (tiles 0 and 1) into slots 0 .. 3
        const TileSrc s0 = tile_src(0), s1 = tile_src(1);
#pragma unroll
        for (int d = 0; d < LPA; ++d) dma_a(s0, lds, d);
#pragma unroll
        for (int d = 0; d < LPB; ++d) dma_b(s0, lds + SLOT, d);
#pragma unroll
        for (int d = 0; d < LPA; ++d) dma_a(s1, lds + 2 * SLOT, d);
#pragma unroll
        for (int d = 0; d < LPB; ++d) dma_b(s1, lds + 3 * SLOT, d);
        // tile 0 landed (tile 1 may still be in flight)
        wait_barrier_vm<LPA + LPB>();
#pragma unroll
        for (int r = 0; r < NR; ++r) read2(lds, lds + SLOT, 0, r, a0, b0);
        // Sources of the loaded tiles from tile 2 on, advanced one K-tile per
        // iteration; only tiles inside the K slice are loaded (the last two
        // iterations load nothing).
        RingSrc ga = ring_src(2, Ab, args.a_extent, A_MC, args.lda, m0);
        RingSrc gb = ring_src(2, Bb, args.b_extent, B_MC, args.ldb, n0);
        // M0 offsets of this wave's load groups inside a slot
        const uint32_t wofs_a = dwave * LPA * 1024, wofs_b = dwave * LPB * 1024;
        // slot addresses of items 2kt .. 2kt+4, advanced by 2 (mod 5) per tile
        uint32_t s_a = lds, s_b = lds + SLOT, s_an = lds + 2 * SLOT, s_bn = lds + 3 * SLOT,
                 s_ld = lds + 4 * SLOT;
        // C quarters (c_pf): load u (0 .. 7) of this wave for quarter q brings
        // rows 64 q + 2 (8 wave + u) + {0, 1}, row r's 16-byte chunk c at
        // position c ^ ((r & 15) * 2) of its 512 bytes (the image's layout,
        // below); the C tile's resource is based at its origin
        // (without c_pf the resource holds no bytes: the loads bring zeros and
        // touch no memory, and the tail's code and wait counts stay the same)
        [[maybe_unused]] i32x4 rcq{};
        if constexpr (C16) {
            const int64_t c_org0 = ((int64_t)m0 * args.ldc + n0) * 2;
            rcq = rsrc4(static_cast<char *>(args.C) + z * args.stride_c * 2 + c_org0,
                        c_pf ? args.c_extent - c_org0 : 0);
        }
        [[maybe_unused]] auto cq_load = [&](int q, int u) {
            const int r = 64 * q + (dwave * 8 + u) * 2 + lane / 32;
            const int c = (lane % 32) ^ ((r & 15) * 2);
            dma16_m0(rcq, group_voff(r * args.ldc * 2 + c * 16, u % kLoadGroup), u % kLoadGroup);
        };
        // CPH: 0, or the C quarter loads of the last two iterations (1: quarter
        // 0 in sub-step 0, quarters 1 and 2 in sub-step 1; 2: quarter 3)
        auto iter = [&](int kt, auto with_loads, auto cph_tag) {
            constexpr bool WL = decltype(with_loads)::value;
            constexpr int CPH = decltype(cph_tag)::value;
            static_assert(CPH == 0 || (!WL && NW == 4 && NDW == NW && LPA == 8 && LPB == 8 && BN == 256),
                          "C quarters: 8 loads per wave, every wave loading");
            const uint32_t a_at = s_a, b_at = s_b, an_at = s_an, bn_at = s_bn, ld_at = s_ld;
            const int kv = min(BK, k_hi - (k_lo + (kt + 2) * BK));
            // sub-step 0: reads of sub-step 1 from tile kt, A of tile kt+2 (or C
            // quarter 0 into the slot tile kt+2's A would have taken)
            {
                const i32x4 ra = ga.rsrc();
                ring_sub(std::integral_constant<int, WL ? LPA : CPH == 1 ? 8 : 0>{}, a0, b0,
                         [&](int r) { read2(a_at, b_at, 1, r, a1, b1); },
                         [&](int d) {
                             if constexpr (CPH == 1) cq_load(0, d);
                             else if (loads)
                                 dma16_m0(ra, group_voff(la.template offset<KMASK>(d, kv), d % kLoadGroup),
                                          d % kLoadGroup);
                         },
                         [&](int g) {
                             if (CPH == 1 || loads) set_m0(ld_at, wofs_a + g * kLoadGroup * 1024);
                         });
            }
            if constexpr (WL) ga.advance();
            // tile kt+1 landed (only A of tile kt+2, or the C quarters, may be
            // in flight); every wave is done with the slots of tile kt
            wait_barrier_vm<WL ? LPA : CPH == 1 ? 8 : CPH == 2 ? 24 : 0>();
            // sub-step 1: reads of tile kt+1's sub-step 0, B of tile kt+2 into
            // the slot of tile kt's A (or C quarters 1 and 2 into tile kt's two
            // slots, or quarter 3 into tile kt's A slot)
            {
                const i32x4 rb = gb.rsrc();
                ring_sub(std::integral_constant<int, WL ? LPB : CPH == 1 ? 16 : CPH == 2 ? 8 : 0>{}, a1, b1,
                         [&](int r) { read2(an_at, bn_at, 0, r, a0, b0); },
                         [&](int d) {
                             if constexpr (CPH == 1) cq_load(1 + d / 8, d % 8);
                             else if constexpr (CPH == 2) cq_load(3, d);
                             else if (loads)
                                 dma16_m0(rb, group_voff(lb.template offset<KMASK>(d, kv), d % kLoadGroup),
                                          d % kLoadGroup);
                         },
                         [&](int g) {
                             if constexpr (CPH == 1)
                                 set_m0(g < 2 ? a_at : b_at, wofs_a + (g % 2) * kLoadGroup * 1024);
                             else if (loads)
                                 set_m0(a_at, wofs_b + g * kLoadGroup * 1024);
                         });
            }
            if constexpr (WL) gb.advance();
            if constexpr (CPH == 1) {
                cq0 = ld_at;
                cq1 = a_at;
                cq2 = b_at;
            } else if constexpr (CPH == 2) {
                cq3 = a_at;
                cfree = b_at;
            }
            // items 2kt+2 .. 2kt+6 are in slots s_an, s_bn, s_ld, s_a, s_b
            s_a = an_at;
            s_b = bn_at;
            s_an = ld_at;
            s_bn = a_at;
            s_ld = b_at;
        };
        using C0 = std::integral_constant<int, 0>;
        int kt = 0;
        for (; kt < nkt - 2; ++kt) iter(kt, std::true_type{}, C0{});
        if constexpr (C16) {
            // kt == max(nkt - 2, 0)
            iter(kt, std::false_type{}, std::integral_constant<int, 1>{});
            if (kt + 1 < nkt) iter(kt + 1, std::false_type{}, std::integral_constant<int, 2>{});
        } else {
            for (; kt < nkt; ++kt) iter(kt, std::false_type{}, C0{});
        }
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" :::
                         "memory");
      }
    } else if (nkt > 0) {
#pragma unroll
        for (int t = 0; t < NST; ++t) {
            const TileSrc st = tile_src(t);
#pragma unroll
            for (int d = 0; d < ND; ++d) dma(st, lds + t * STAGE, d);
        }
        // tile 0 landed (tiles 1 .. NST-1 may still be in flight: the loop
        // barriers wait for them); the waves without loads have none in flight
        wait_barrier_vm<(NST - 1) * ND>();
        if constexpr (EPI_LDS > 1 && !EPI_AFTER) {
            if (tid < BN) {
                epi_smem[tid] = epi_b;
                epi_smem[BN + tid] = args.alpha * epi_s;
            }
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) read(lds, 0, r, a0, b0);
        // sources of tile NST on, advanced one K-tile per iteration (tiles
        // past the K slice: empty ranges)
        RingSrc ga = ring_src(NST, Ab, args.a_extent, A_MC, args.lda, m0);
        RingSrc gb = ring_src(NST, Bb, args.b_extent, B_MC, args.ldb, n0);
        // M0 offsets of this wave's load groups inside a stage
        static_assert(LPA % kLoadGroup == 0 && LPB % kLoadGroup == 0, "whole load groups per operand");
        const uint32_t wofs_a = dwave * LPA * 1024, wofs_b = A_BYTES + dwave * LPB * 1024;
        for (int kt = 0; kt < nkt; ++kt) {
            const uint32_t cur = lds + (kt % NST) * STAGE;
            const uint32_t nxt = lds + ((kt + 1) % NST) * STAGE;
            sub0(cur);
            // tile kt+1 landed for every wave (tiles up to kt+NST-1 may still
            // be in flight); every wave is done with `cur`
            wait_barrier_vm<(NST - 2) * ND>();
            // sub-step 1: MFMAs on (a1, b1), the reads of tile kt+1's
            // sub-step 0 and the loads of tile kt+NST into `cur` (A, then B),
            // a group of loads per M0 write
            const bool inside = kt + NST < nkt;
            const int kv = min(BK, k_hi - (k_lo + (kt + NST) * BK));
            const i32x4 ra = ga.rsrc(inside), rb = gb.rsrc(inside);
            ring_sub(std::integral_constant<int, ND>{}, a1, b1,
                     [&](int r) { read(nxt, 0, r, a0, b0); },
                     [&](int d) {
                         if (!loads) return;
                         if (d < LPA)
                             dma16_m0(ra, group_voff(la.template offset<KMASK>(d, kv), d % kLoadGroup),
                                      d % kLoadGroup);
                         else
                             dma16_m0(rb, group_voff(lb.template offset<KMASK>(d - LPA, kv), d % kLoadGroup),
                                      d % kLoadGroup);
                     },
                     [&](int g) {
                         if (!loads) return;
                         if (g * kLoadGroup < LPA) set_m0(cur, wofs_a + g * kLoadGroup * 1024);
                         else set_m0(cur, wofs_b + (g * kLoadGroup - LPA) * 1024);
                     });
            ga.advance();
            gb.advance();
        }
        // no load may still be writing LDS when the workgroup ends, and the
        // last MFMA results need wait states before the accumulators are read
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" :::
                         "memory");
    }
    if constexpr (EPI_AFTER) {
        // every wave is done with the stages: the bias and alpha * scale
        // (held in registers through the loop) go into the first one (also
        // with no K-tile at all, so the epilogue reads what it expects)
        asm volatile("s_barrier" ::: "memory");
        if (tid < BN) {
            epi_smem[tid] = epi_b;
            epi_smem[BN + tid] = args.alpha * epi_s;
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) asm volatile("" : "+a"(acc[i][j]));

    // ---- epilogue: the lane holds NG groups of 4 consecutive columns of one
    // C row per block (the B block is the MFMA's first operand): with MS = 16
    // row l % 16, columns 4 (l / 16) + 0..3; with MS = 32 row l % 32,
    // columns 8 q + 4 (l / 32) + 0..3 for group q -- accumulators 4q .. 4q+3
    constexpr int NG = MS == 16 ? 1 : 4;
    auto ml_of = [&](int i) { return wm * WTM + i * MS + (lane & (MS - 1)); };
    auto nl_of = [&](int j, int q) {
        return wn * WTN + j * MS + (MS == 16 ? 4 * (lane >> 4) : 8 * q + 4 * (lane >> 5));
    };
    constexpr int CES = dt_size(OUT == OUT_PARTIAL ? DT_F32 : OUT);
    // Interior tiles whose output rows are whole 16-byte chunks store through
    // LDS (C, or the split-K partial sums, rows ld values apart, at r):
    // each wave writes its tile, SCH rows at a time, into a region of its own
    // (rows padded by 16 values, so the writes of 16 rows spread over the
    // banks), then reads it back 16 bytes per lane along the rows and stores
    // whole row pieces (measured on the 256 x 256 tile, bf16 4096^3: the
    // 16 x 32-byte pieces of a block per store took 3.6 us longer per call
    // than 16-byte pieces along rows).  col(j, q) runs before the values of
    // column group (j, q) are packed; pack(i, j, q, w): the CES words of the 4
    // values of block (i, j), group q, in the output's type.  Rows past M
    // start past the store range of r, so their stores are dropped.  The
    // regions start past the bias and scales that the fused epilogue keeps at
    // the start of the stages.  16-bit outputs take this path also where C's
    // rows do not start on 16-byte boundaries (the stores are unaligned then,
    // which the GPU allows; int8 4093 x 4099 x 4096 dequantized into bf16 at
    // ldc = 4099: 78.2 -> 71.7 us per call); 32-bit ones only where they do
    // (int32 out at ldc = 4099: no gain, the main kernel 1 % slower).
    constexpr int SROW = WTN * CES, SPITCH = SROW + 16 * CES;
    constexpr int SBASE = EPI_AFTER ? (EPI_LDS * 4 + 1023) / 1024 * 1024 : 0;
    constexpr int SREGION = (LDS_BYTES - SBASE) / NW / 16 * 16;
    constexpr int SCH = (WTM * SPITCH <= SREGION) ? WTM : (WTM / 2 * SPITCH <= SREGION) ? WTM / 2
                      : (WTM / 4 * SPITCH <= SREGION) ? WTM / 4 : WTM / 8;
    static_assert(SCH >= MS && SCH * SPITCH <= SREGION && WTM % SCH == 0, "staging band fits");
    constexpr int SLPR = SROW / 16, SRPI = 64 / SLPR;   // lanes per row, rows per read
    // (staged_in: the same into the region at `region`, SCHX rows at a time,
    // band(c0) first in the band of rows c0 ..)
    [[maybe_unused]] auto staged_in = [&](auto sch_tag, uint32_t region, __amdgpu_buffer_rsrc_t r, int ld,
                                          auto &&band, auto &&col, auto &&pack) {
        constexpr int SCHX = decltype(sch_tag)::value;
        static_assert(SCHX >= MS && WTM % SCHX == 0, "staging band");
        TCG_LDS char *reg = (TCG_LDS char *)(size_t)region;
#pragma unroll
        for (int c0 = 0; c0 < WTM; c0 += SCHX) {
            band(c0);
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < NG; ++q) {
                    col(j, q);
#pragma unroll
                    for (int i = c0 / MS; i < (c0 + SCHX) / MS; ++i) {
                        u32 w[CES];
                        pack(i, j, q, w);
                        TCG_LDS char *at =
                            reg + (ml_of(i) - wm * WTM - c0) * SPITCH + (nl_of(j, q) - wn * WTN) * CES;
                        if constexpr (CES == 2) *(TCG_LDS u32x2 *)at = u32x2{w[0], w[1]};
                        else *(TCG_LDS u32x4 *)at = u32x4{w[0], w[1], w[2], w[3]};
                    }
                }
            // the LDS runs one wave's accesses in order: the reads below see
            // the writes above, and the next band's writes follow these reads
#pragma unroll
            for (int t = 0; t < SCHX / SRPI; ++t) {
                const int row = t * SRPI + lane / SLPR, ch = lane % SLPR;
                const u32x4 d = *(const TCG_LDS u32x4 *)(reg + row * SPITCH + ch * 16);
                __builtin_amdgcn_raw_buffer_store_b128(
                    d, r, (wm * WTM + c0 + row) * ld * CES + wn * WTN * CES + ch * 16, 0, 0);
            }
        }
    };
    [[maybe_unused]] auto staged_store = [&](__amdgpu_buffer_rsrc_t r, int ld, auto &&col, auto &&pack) {
        // every wave is done with the stages and no load is still writing them
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        staged_in(std::integral_constant<int, SCH>{}, lds + SBASE + wave * SREGION, r, ld, [](int) {}, col,
                  pack);
    };
    if constexpr (OUT == OUT_PARTIAL) {
        // raw fp32 / int32 partial sums of this K slice: workspace plane g
        char *wsb = static_cast<char *>(args.ws) +
                    ((int64_t)g * M * N + (int64_t)m0 * N + n0) * 4;
        const int64_t ws_ext = (int64_t)(M - m0) * N * 4 - (int64_t)n0 * 4;
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(wsb, ws_ext);
        const bool vec = (N % 4) == 0;
        if (vec && n0 + BN <= N) {
            staged_store(rw, N, [](int, int) {}, [&](int i, int j, int q, u32 (&w)[CES]) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (DT == DT_I8) w[e] = (u32)acc[i][j][4 * q + e];
                    else w[e] = as_u32(acc[i][j][4 * q + e]);
                }
            });
            return;
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int ml = ml_of(i);
            if (m0 + ml >= M) continue;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < NG; ++q) {
                    const int nl = nl_of(j, q);
                    const int nvalid = N - (n0 + nl);
                    if (nvalid <= 0) continue;
                    int v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if constexpr (DT == DT_I8) v[e] = acc[i][j][4 * q + e];
                        else v[e] = as_i32(acc[i][j][4 * q + e]);
                    }
                    store_i4(rw, (ml * N + nl) * 4, nvalid, vec, v);
                }
        }
        return;
    }
    const int64_t c_org = ((int64_t)m0 * args.ldc + n0) * CES;
    char *Cb = static_cast<char *>(args.C) + z * args.stride_c * CES + c_org;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cb, args.c_extent - c_org);
    const bool vec = args.c_vec_ok != 0;
    const int ldc = args.ldc;
    const float alpha = args.alpha, beta = EPI != EPI_PLAIN ? args.beta : 0.f;

    // beta != 0 with a 16-bit C tile that lies wholly inside C and whose
    // rows are whole 16-byte chunks: the tile (BM x BN x 2 bytes, the size of
    // the two operand stages) comes into LDS with direct-to-LDS loads, all of
    // it in flight at once, instead of one round trip per 16x16 block from
    // the registers' side.  Row r of the LDS image holds 16-byte chunk q at
    // position q ^ ((r & 15) * CSW), so the epilogue's reads of 16 rows at
    // one column hit distinct banks.
    constexpr int CRB = BN * 2;                    // C tile row bytes (16-bit)
    constexpr int CSW = CRB >= 512 ? 2 : 1;
    static_assert(BM * CRB <= LDS_BYTES, "the C tile fits the operand stages");
    bool c_lds = false;
    // v = beta * C_old + alpha * acc for the 4 values of tile row ml, columns
    // nl .. nl+3, C_old from the tile's LDS image, the row at LDS address
    // row_at (its 16-byte chunks swizzled by the row's low bits)
    // (c_old4: the 8 bytes of C_old; beta4: v from them)
    [[maybe_unused]] auto c_old4 = [&](uint32_t row_at, int ml, int nl) {
        const int cq = (nl * 2) / 16;
        const uint32_t a = row_at + ((cq ^ ((ml & 15) * CSW)) << 4) + ((nl * 2) & 15);
        return *(const TCG_LDS u32x2 *)(size_t)a;
    };
    [[maybe_unused]] auto beta4 = [&](u32x2 w, float (&v)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const u32 h = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
            const float old = OUT == DT_BF16 ? from_bf16_bits(h) : from_f16_bits(h);
            v[e] = __builtin_fmaf(beta, old, v[e] * alpha);
        }
    };
    [[maybe_unused]] auto beta_lds4 = [&](uint32_t row_at, int ml, int nl, float (&v)[4]) {
        beta4(c_old4(row_at, ml, nl), v);
    };
    if constexpr (EPI == EPI_BETA && (OUT == DT_F16 || OUT == DT_BF16) && RING) {
        if (c_pf) {
            // the quarters loaded during the last iterations: every wave's
            // loads have landed.  The results go out along rows through the
            // fifth slot, a quarter of it per wave (the quarters hold C_old
            // meanwhile).  The ring's other tiles read C_old from C itself.
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            constexpr int SREG_C = SLOT / NW / 16 * 16;
            constexpr int SCH_C = (WTM / 4 * SPITCH <= SREG_C) ? WTM / 4
                                : (WTM / 8 * SPITCH <= SREG_C) ? WTM / 8 : MS;
            static_assert(SCH_C * SPITCH <= SREG_C, "staging band fits a quarter slot");
            // the wave's rows span two quarters: the first and second, or the
            // third and fourth
            static_assert(BM == 256 && WTM == 128, "two C quarters per wave");
            const uint32_t qw0 = wm == 0 ? cq0 : cq2, qw1 = wm == 0 ? cq1 : cq3;
            // a band's C_old is read before its first write to the staging
            // region, so that the reads go out together
            constexpr int BI = SCH_C / MS;
            u32x2 cold[BI][FN][NG];
            staged_in(std::integral_constant<int, SCH_C>{}, cfree + wave * SREG_C, rc, ldc,
                      [&](int c0) {
#pragma unroll
                          for (int ib = 0; ib < BI; ++ib) {
                              const int i = c0 / MS + ib, ml = ml_of(i);
                              const uint32_t row_at = (i * MS < 64 ? qw0 : qw1) + (ml % 64) * CRB;
#pragma unroll
                              for (int j = 0; j < FN; ++j)
#pragma unroll
                                  for (int q = 0; q < NG; ++q) cold[ib][j][q] = c_old4(row_at, ml, nl_of(j, q));
                          }
                      },
                      [](int, int) {}, [&](int i, int j, int q, u32 (&w)[CES]) {
                          float v[4];
#pragma unroll
                          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
                          beta4(cold[i % BI][j][q], v);
                          w[0] = pack2_16<OUT>(v[0], v[1]);
                          w[1] = pack2_16<OUT>(v[2], v[3]);
                      });
            return;
        }
    } else if constexpr (EPI == EPI_BETA && (OUT == DT_F16 || OUT == DT_BF16)) {
        c_lds = beta != 0.f && args.c_dma_ok != 0 && m0 + BM <= M && n0 + BN <= N;
        if (c_lds) {
            // every wave is done with the operand stages
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            const i32x4 rcc = rsrc4(Cb, args.c_extent - c_org);
            constexpr int LOADS = BM * CRB / 1024 / NW;   // per wave
            constexpr int LPR_C = CRB / 16, RPI_C = 64 / LPR_C;
#pragma unroll
            for (int u = 0; u < LOADS; ++u) {
                const int r = (wave * LOADS + u) * RPI_C + lane / LPR_C;
                const int q = (lane % LPR_C) ^ ((r & 15) * CSW);
                dma16(rcc, lds + (wave * LOADS + u) * 1024, r * ldc * CES + q * 16);
            }
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        }
    }
    [[maybe_unused]] const EpiState ep = make_epi<OUT == DT_I32 ? DT_F32 : OUT>(args, z, N);
    // A tile whose columns lie inside C, with vector-aligned rows, and no
    // C_old to read: every block is stored whole, so the store sequence is
    // straight-line code with no per-block bounds or alignment branches
    // (short code: the epilogue runs once per workgroup, from a cold
    // instruction cache).  Rows past M need no test: they start at or past
    // M * ldc >= (M - 1) * ldc + N elements, the end of the store range of
    // `rc`, so the buffer unit drops their stores.
    const bool interior = vec && n0 + BN <= N;
    // fused epilogue: act(acc * (alpha * scale) + bias), with bias and
    // alpha * scale of the lane's columns read from LDS
    // (MS = 32: a lane has 16 column groups; the loops run column groups
    // outside so that only one group's bias and scales are live)
    [[maybe_unused]] auto fused_interior = [&](auto act_tag) {
        constexpr int ACT = decltype(act_tag)::value;
        auto one = [&](int i, int j, int q, const float (&b)[4], const float (&sa)[4]) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = act1<ACT>(__builtin_fmaf((float)acc[i][j][4 * q + e], sa[e], b[e]));
            store_c4<OUT>(rc, (ml_of(i) * ldc + nl_of(j, q)) * CES, 4, true, v);
        };
        if constexpr (MS == 16) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    float b[4], sa[4];
                    read_epi4(epi_smem, BN, nl_of(j, 0), b, sa);
                    one(i, j, 0, b, sa);
                }
        } else {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < NG; ++q) {
                    float b[4], sa[4];
                    read_epi4(epi_smem, BN, nl_of(j, q), b, sa);
#pragma unroll
                    for (int i = 0; i < FM; ++i) one(i, j, q, b, sa);
                }
        }
    };
    // the same through LDS for 16-byte C rows: act(acc * (alpha * scale) + bias)
    [[maybe_unused]] auto fused_staged = [&](auto act_tag) {
        constexpr int ACT = decltype(act_tag)::value;
        float b[4], sa[4];
        staged_store(rc, ldc, [&](int j, int q) { read_epi4(epi_smem, BN, nl_of(j, q), b, sa); },
                     [&](int i, int j, int q, u32 (&w)[CES]) {
                         float v[4];
#pragma unroll
                         for (int e = 0; e < 4; ++e)
                             v[e] = act1<ACT>(__builtin_fmaf((float)acc[i][j][4 * q + e], sa[e], b[e]));
                         if constexpr (CES == 4) {
#pragma unroll
                             for (int e = 0; e < 4; ++e) w[e] = as_u32(v[e]);
                         } else {
                             w[0] = pack2_16<OUT>(v[0], v[1]);
                             w[1] = pack2_16<OUT>(v[2], v[3]);
                         }
                     });
    };
    if constexpr (EPI_LDS > 1) {
        if (interior && beta == 0.f && (CES == 2 || args.c_dma_ok)) {
            if (ep.act == ACT_GELU_TANH) fused_staged(std::integral_constant<int, ACT_GELU_TANH>{});
            else if (ep.act == ACT_RELU) fused_staged(std::integral_constant<int, ACT_RELU>{});
            else fused_staged(std::integral_constant<int, ACT_NONE>{});
            return;
        }
        if (interior && beta == 0.f) {
            if (ep.act == ACT_GELU_TANH) fused_interior(std::integral_constant<int, ACT_GELU_TANH>{});
            else if (ep.act == ACT_RELU) fused_interior(std::integral_constant<int, ACT_RELU>{});
            else fused_interior(std::integral_constant<int, ACT_NONE>{});
            return;
        }
    }
    if constexpr (EPI == EPI_PLAIN && OUT != OUT_PARTIAL) {
        if (interior && (CES == 2 || args.c_dma_ok)) {
            staged_store(rc, ldc, [](int, int) {}, [&](int i, int j, int q, u32 (&w)[CES]) {
                if constexpr (OUT == DT_I32) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = (u32)acc[i][j][4 * q + e];
                } else if constexpr (OUT == DT_F32) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = as_u32(alpha * (float)acc[i][j][4 * q + e]);
                } else {
                    w[0] = pack2_16<OUT>(alpha * (float)acc[i][j][4 * q], alpha * (float)acc[i][j][4 * q + 1]);
                    w[1] = pack2_16<OUT>(alpha * (float)acc[i][j][4 * q + 2],
                                         alpha * (float)acc[i][j][4 * q + 3]);
                }
            });
            return;
        }
        if (interior) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int ml = ml_of(i);
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int q = 0; q < NG; ++q) {
                        const int off = (ml * ldc + nl_of(j, q)) * CES;
                        if constexpr (OUT == DT_I32) {
                            int v[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
                            store_i4(rc, off, 4, true, v);
                        } else {
                            float v[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) v[e] = alpha * (float)acc[i][j][4 * q + e];
                            store_c4<OUT>(rc, off, 4, true, v);
                        }
                    }
            }
            return;
        }
    }
    // fused epilogue, general case: rows and columns past C skipped, C_old
    // read per block when beta != 0
    if constexpr (EPI_LDS > 1) {
        const float *lds_epi = epi_smem;
        // row blocks outside, as in the plain epilogue, so the stores of one
        // row's column blocks follow each other and complete whole lines
        auto one = [&](int i, int j, int q, const float (&b)[4], const float (&sa)[4]) {
            const int ml = ml_of(i), nl = nl_of(j, q);
            const int nvalid = N - (n0 + nl);
            if (m0 + ml >= M || nvalid <= 0) return;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
            finish4_fused<OUT>(rc, (ml * ldc + nl) * CES, nvalid, vec, beta, v, ep, b, sa);
        };
        if constexpr (MS == 16) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    float b[4], sa[4];
                    read_epi4(lds_epi, BN, nl_of(j, 0), b, sa);
                    one(i, j, 0, b, sa);
                }
        } else {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < NG; ++q) {
                    float b[4], sa[4];
                    read_epi4(lds_epi, BN, nl_of(j, q), b, sa);
#pragma unroll
                    for (int i = 0; i < FM; ++i) one(i, j, q, b, sa);
                }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int ml = ml_of(i);
        if (m0 + ml >= M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < NG; ++q) {
                const int nl = nl_of(j, q);
                const int nvalid = N - (n0 + nl);
                if (nvalid <= 0) continue;
                const int off = (ml * ldc + nl) * CES;
                if constexpr (OUT == DT_I32) {
                    int v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
                    store_i4(rc, off, nvalid, vec, v);
                } else if constexpr (OUT != OUT_PARTIAL) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
                    if constexpr (EPI == EPI_BETA && (OUT == DT_F16 || OUT == DT_BF16)) {
                        if (c_lds) {
                            // C_old from the LDS image (8 bytes: 4 values)
                            beta_lds4(lds + ml * CRB, ml, nl, v);
                            store_c4<OUT>(rc, off, 4, true, v);
                            continue;
                        }
                    }
                    finish4<OUT>(rc, off, nvalid, vec, alpha, beta, v);
                }
            }
    }
}

}  // namespace
}  // namespace tcg
