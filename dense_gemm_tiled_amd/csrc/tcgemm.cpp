// tcgemm.cpp -- host side of libtcgemm.so: the C ABI declared in
// include/tcgemm.h.
//
// Call path (tessl "Architecture", "GEMM Pipeline & Kernel Selection"):
// normalize leading dims -> validate everything with checked 64-bit
// arithmetic -> plan (kernel by dtype x layout, tile class by shape, split-K
// when the output has too few tiles to fill the GPU) -> enqueue.  Validation
// returns before anything is enqueued, so a refused call leaves the dispatch
// count unchanged (same page, "The Kernel Library and the nn Boundary").

#include "tcgemm.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <map>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include <unistd.h>   // environ

#include "tc_internal.h"

using namespace tcg;

struct tc_stream {
    tc_context *ctx = nullptr;
    hipStream_t stream = nullptr;
    bool owned = false;
    void *ws = nullptr;          // split-K workspace (device memory)
    int64_t ws_bytes = 0;
};

// A tuned (or forced) choice the planner follows instead of its own rules.
struct Choice {
    int cls = -1;          // tile class, -1: the planner's
    int64_t splits = 0;    // split-K slices with a forced class (0: none)
    int gemv = -1;         // small-M route: 0 off, 1 on where eligible, -1: the planner's
};

struct tc_context {
    int device = -1;             // bound at the first launch
    tc_stream *internal = nullptr;
    uint64_t dispatches = 0;
    std::string last_kernel;
    std::string last_error;
    hipEvent_t time_ev[2] = {nullptr, nullptr};   // armed by tc_time_next_gemm
    bool autotune = false;                        // tc_set_autotune
    std::map<std::string, Choice> tuned;          // problem key -> measured best choice
};

namespace {

constexpr int64_t kMaxIndex = 0x7FFFFFFF;          // every element index fits int32
constexpr int64_t kMaxTileSpanBytes = 0x7FFFFFFF;  // byte offsets inside one tile fit int32
constexpr int32_t kMaxInt8K = 131071;              // 16384 * 131072 = 2^31 would wrap
constexpr int kMaxTileRows = 256;

std::string g_plan_error;   // error text of tc_gemm_plan(NULL, ...)

// The fused epilogue of a call (none: act == ACT_NONE and no bias).
struct Epilogue {
    const void *bias = nullptr;   // N values of c_dtype per problem
    int64_t bias_stride = 0;      // elements between problems' vectors
    const float *scale = nullptr; // N per-column fp32 scales per problem
    int64_t scale_stride = 0;
    int act = ACT_NONE;
    bool on() const { return bias != nullptr || scale != nullptr || act != ACT_NONE; }
};

// Everything validation derives from a descriptor.
struct Problem {
    int32_t M, N, K, batch;
    int dt, cdt;
    bool ta, tb;
    float alpha, beta;
    int64_t lda, ldb, ldc;
    int64_t stride_a, stride_b, stride_c;
    int64_t a_ext, b_ext, c_ext;          // elements spanned by one problem
    int64_t a_total, b_total, c_total;    // bytes spanned by all problems
    // the transposed form of a small-M GEMM: this problem's output (r, c) is
    // C[c*ldc + r] of the caller's
    bool c_trans = false;
};

struct Plan {
    int cls;
    int bm, bn, bk;
    int32_t tiles_m, tiles_n;
    int32_t splits, k_per_split;
    int64_t grid;
    int64_t ws_bytes;           // whole workspace: split-K partials, then packed operands
    int32_t band;
    // Operand repacking for the direct-to-LDS classes ([0] = A, [1] = B):
    // byte pitch, batch stride and workspace offset of the packed copy.
    bool pack[2];
    int64_t pack_pitch[2], pack_stride[2], pack_off[2];
    // Edge split: 1 = the columns from edge_at on, 2 = the rows from edge_at
    // on, run as a second GEMM after the whole tiles (0: no split).
    int edge;
    int32_t edge_at;
    // small-M GEMM run as its transposed product (the plan fields describe
    // that product): see transposed_problem
    bool swap;
};

tc_status_t fail(std::string *err, tc_status_t st, const char *fmt, ...) {
    if (err) {
        char buf[512];
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(buf, sizeof buf, fmt, ap);
        va_end(ap);
        *err = buf;
    }
    return st;
}

bool mul_ok(int64_t a, int64_t b, int64_t *out) { return !__builtin_mul_overflow(a, b, out); }
bool add_ok(int64_t a, int64_t b, int64_t *out) { return !__builtin_add_overflow(a, b, out); }

// Elements spanned by a rows x cols matrix with leading dim ld; -1 on overflow.
int64_t span(int64_t rows, int64_t cols, int64_t ld) {
    int64_t t, r;
    if (!mul_ok(rows - 1, ld, &t) || !add_ok(t, cols, &r)) return -1;
    return r;
}

// Bytes spanned by `batch` problems of `ext` elements at `stride`; -1 on overflow.
int64_t total_bytes(int64_t batch, int64_t stride, int64_t ext, int es) {
    int64_t t, r, b;
    if (!mul_ok(batch - 1, stride, &t) || !add_ok(t, ext, &r) || !mul_ok(r, es, &b)) return -1;
    return b;
}

const char *dt_name(int dt) {
    switch (dt) {
    case TC_F32: return "f32";
    case TC_F16: return "f16";
    case TC_BF16: return "bf16";
    case TC_I8: return "i8";
    case TC_I32: return "i32";
    default: return "?";
    }
}

// dequant: the call carries a per-column scale, so int8 inputs may have a
// float output (tessl "Architecture", "Integer GEMM": gemm_i8_dequant).
tc_status_t validate(const tc_gemm_batched_desc *bd, Problem *p, std::string *err,
                     bool dequant = false) {
    if (!bd) return fail(err, TC_ERR_INVALID_ARGUMENT, "descriptor is NULL");
    const tc_gemm_desc &d = bd->base;
    if (d.M < 1 || d.N < 1 || d.K < 1)
        return fail(err, TC_ERR_INVALID_ARGUMENT, "dims must be >= 1 (M=%d N=%d K=%d)", d.M, d.N, d.K);
    if (bd->batch < 1) return fail(err, TC_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", bd->batch);

    // supported (a, b, c, accum) tuples
    const int a = d.a_dtype, b = d.b_dtype, c = d.c_dtype, acc = d.accum_dtype;
    bool ok = false;
    if (a != b) {
        ok = false;
    } else if (a == TC_F32) {
        ok = c == TC_F32 && acc == TC_F32;
    } else if (a == TC_F16 || a == TC_BF16) {
        ok = (c == a || c == TC_F32) && acc == TC_F32;
    } else if (a == TC_I8) {
        ok = acc == TC_I32 &&
             (c == TC_I32 || (dequant && (c == TC_F32 || c == TC_F16 || c == TC_BF16)));
    }
    if (!ok)
        return fail(err, TC_ERR_UNSUPPORTED, "unsupported dtypes a=%s b=%s c=%s accum=%s", dt_name(a),
                    dt_name(b), dt_name(c), dt_name(acc));

    p->M = d.M; p->N = d.N; p->K = d.K; p->batch = bd->batch;
    p->dt = a; p->cdt = c;
    p->ta = d.transpose_a; p->tb = d.transpose_b;
    p->alpha = d.alpha; p->beta = d.beta;

    // leading dims: 0 means contiguous (tensorcore "GEMM", "Surface")
    const int64_t a_rows = p->ta ? d.K : d.M, a_cols = p->ta ? d.M : d.K;
    const int64_t b_rows = p->tb ? d.N : d.K, b_cols = p->tb ? d.K : d.N;
    p->lda = d.lda == 0 ? a_cols : d.lda;
    p->ldb = d.ldb == 0 ? b_cols : d.ldb;
    p->ldc = d.ldc == 0 ? d.N : d.ldc;
    if (p->lda < a_cols)
        return fail(err, TC_ERR_INVALID_ARGUMENT, "lda=%lld < %lld", (long long)p->lda, (long long)a_cols);
    if (p->ldb < b_cols)
        return fail(err, TC_ERR_INVALID_ARGUMENT, "ldb=%lld < %lld", (long long)p->ldb, (long long)b_cols);
    if (p->ldc < d.N)
        return fail(err, TC_ERR_INVALID_ARGUMENT, "ldc=%lld < N=%d", (long long)p->ldc, d.N);

    if (!std::isfinite(d.alpha) || !std::isfinite(d.beta))
        return fail(err, TC_ERR_INVALID_ARGUMENT, "alpha and beta must be finite");

    if (a == TC_I8) {
        if (c == TC_I32 && (d.alpha != 1.0f || d.beta != 0.0f))
            return fail(err, TC_ERR_UNSUPPORTED, "int8 GEMM needs alpha = 1 and beta = 0");
        if (d.K > kMaxInt8K)
            return fail(err, TC_ERR_OVERFLOW, "int8 K=%d > %d: an int32 sum could wrap", d.K, kMaxInt8K);
    }

    const int es = dt_size(a), ces = dt_size(c);
    p->a_ext = span(a_rows, a_cols, p->lda);
    p->b_ext = span(b_rows, b_cols, p->ldb);
    p->c_ext = span(d.M, d.N, p->ldc);
    if (p->a_ext < 0 || p->a_ext > kMaxIndex) return fail(err, TC_ERR_OVERFLOW, "A spans more than 2^31-1 elements");
    if (p->b_ext < 0 || p->b_ext > kMaxIndex) return fail(err, TC_ERR_OVERFLOW, "B spans more than 2^31-1 elements");
    if (p->c_ext < 0 || p->c_ext > kMaxIndex) return fail(err, TC_ERR_OVERFLOW, "C spans more than 2^31-1 elements");
    // byte offsets inside one tile are 32-bit
    if ((int64_t)kMaxTileRows * p->lda * es + 256 > kMaxTileSpanBytes ||
        (int64_t)kMaxTileRows * p->ldb * es + 256 > kMaxTileSpanBytes ||
        (int64_t)kMaxTileRows * p->ldc * ces + 256 > kMaxTileSpanBytes)
        return fail(err, TC_ERR_OVERFLOW, "a leading dimension exceeds 8 MiB per row");

    p->stride_a = bd->batch > 1 ? bd->stride_a : 0;
    p->stride_b = bd->batch > 1 ? bd->stride_b : 0;
    p->stride_c = bd->batch > 1 ? bd->stride_c : 0;
    if (p->stride_a < 0 || p->stride_b < 0 || p->stride_c < 0)
        return fail(err, TC_ERR_INVALID_ARGUMENT, "batch strides must be >= 0");
    if (bd->batch > 1 && p->stride_c < p->c_ext)
        return fail(err, TC_ERR_ALIASING, "stride_c=%lld < C extent %lld: batch outputs overlap",
                    (long long)p->stride_c, (long long)p->c_ext);
    p->a_total = total_bytes(bd->batch, p->stride_a, p->a_ext, es);
    p->b_total = total_bytes(bd->batch, p->stride_b, p->b_ext, es);
    p->c_total = total_bytes(bd->batch, p->stride_c, p->c_ext, ces);
    if (p->a_total < 0 || p->b_total < 0 || p->c_total < 0)
        return fail(err, TC_ERR_OVERFLOW, "batched extent overflows 64 bits");
    return TC_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The direct-to-LDS kernel takes 16-bit and int8 inputs.  It moves 16-byte
// chunks, so an operand feeds it as it is when its row pitch, its batch
// stride, its base pointer and its rows themselves are whole chunks: the
// loads zero whole chunks past K, and no chunk may straddle the end of the
// operand, where a range-checked load would not return the valid part.  Any
// other operand is first copied into a packed layout in the workspace (rows
// padded to 16 bytes with zeros; pack_rows_kernel).  The loads do take
// unaligned addresses, so rows of whole chunks at an odd pitch or base could
// be read in place -- but measured on the int8 ragged shape (B rows of 4096
// bytes at a pitch of 4099) the GEMM kernel then ran 13.7 us longer than
// the 10.5 us packing pass it saves.  Tuning knob: TCGEMM_PACK_UNALIGNED=0
// reads such operands in place.
bool dma_types(const Problem &p) { return p.dt == TC_F16 || p.dt == TC_BF16 || p.dt == TC_I8; }

// Tile classes whose kernel can write split-K partial sums.
bool splits_ok(int cls) {
    return cls == TILE_64 || cls == TILE_128 || cls == TILE_128_DMA || cls == TILE_128_DMA4 ||
           cls == TILE_256_DMA;
}

// Rows and columns (elements) of operand w (0 = A, 1 = B) as stored.
void operand_shape(const Problem &p, int w, int64_t *rows, int64_t *cols) {
    const int64_t mn = w == 0 ? p.M : p.N;
    const bool mc = w == 0 ? p.ta : !p.tb;   // M/N-contiguous: rows are k
    *rows = mc ? p.K : mn;
    *cols = mc ? mn : p.K;
}

// Tuning knobs (environment variables TCGEMM_*, unset in normal use).  An
// entry point reads them all in one pass over the environment when it starts
// (KnobScope); the planner then looks them up here instead of calling getenv
// for each (a getenv walks the whole environment).  Outside a scope the
// lookup falls back to getenv.
enum Knob { K_TILE, K_SPLITS, K_BAND, K_EDGE, K_GEMV, K_PACK_UNALIGNED, NUM_KNOBS };
const char *const kKnobName[NUM_KNOBS] = {"TCGEMM_TILE", "TCGEMM_SPLITS", "TCGEMM_BAND",
                                          "TCGEMM_EDGE", "TCGEMM_GEMV", "TCGEMM_PACK_UNALIGNED"};
thread_local const char *t_knob[NUM_KNOBS];
thread_local int t_knob_depth = 0;

struct KnobScope {
    KnobScope() {
        if (t_knob_depth++ > 0) return;
        for (int k = 0; k < NUM_KNOBS; ++k) t_knob[k] = nullptr;
        for (char **e = environ; e && *e; ++e) {
            if (strncmp(*e, "TCGEMM_", 7) != 0) continue;
            for (int k = 0; k < NUM_KNOBS; ++k) {
                const size_t n = strlen(kKnobName[k]);
                if (strncmp(*e, kKnobName[k], n) == 0 && (*e)[n] == '=') t_knob[k] = *e + n + 1;
            }
        }
    }
    ~KnobScope() { --t_knob_depth; }
    KnobScope(const KnobScope &) = delete;
    KnobScope &operator=(const KnobScope &) = delete;
};

const char *knob(Knob k) { return t_knob_depth > 0 ? t_knob[k] : getenv(kKnobName[k]); }

bool pack_unaligned() {
    const char *env = knob(K_PACK_UNALIGNED);
    return !env || atoi(env) != 0;
}

// aligned: the operand's base pointer is 16-byte aligned.
bool operand_dma_ready(const Problem &p, int w, bool aligned) {
    const int es = dt_size(p.dt);
    const int64_t ld = w == 0 ? p.lda : p.ldb, stride = w == 0 ? p.stride_a : p.stride_b;
    int64_t rows, cols;
    operand_shape(p, w, &rows, &cols);
    if ((cols * es) % 16 != 0) return false;
    return !pack_unaligned() || ((ld * es) % 16 == 0 && (stride * es) % 16 == 0 && aligned);
}

int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// The thin kernel reads B as N rows of K values: a B stored [K, N] (not
// transposed) is gathered into a transposed copy first, once, rather than
// by every workgroup (read from a wide matrix, each row of B is a cache
// line of its own).
bool thin_transposes_b(const Problem &p, const Plan &pl) { return pl.cls == TILE_THIN && !p.tb; }

// Workspace layout of a plan: split-K partials at offset 0, then the packed
// copies of the operands that need one (aligned: whether the operand's base
// pointer is 16-byte aligned).
void layout_workspace(const Problem &p, Plan *pl, const bool aligned[2]) {
    const int es = dt_size(p.dt);
    int64_t off = pl->splits > 1 ? align_up(pl->splits * p.batch * (int64_t)p.M * p.N * 4, 256) : 0;
    for (int w = 0; w < 2; ++w) {
        pl->pack[w] = is_dma_class(pl->cls) && !operand_dma_ready(p, w, aligned[w]);
        pl->pack_pitch[w] = pl->pack_stride[w] = pl->pack_off[w] = 0;
        if (w == 1 && thin_transposes_b(p, *pl)) {
            // thin kernel: B^T, N rows of K values
            const int64_t stride = p.stride_b;
            pl->pack[1] = true;
            pl->pack_pitch[1] = align_up((int64_t)p.K * es, 16);
            pl->pack_stride[1] = stride == 0 ? 0 : p.N * pl->pack_pitch[1];
            pl->pack_off[1] = off;
            off += align_up((stride == 0 ? 1 : p.batch) * p.N * pl->pack_pitch[1], 256);
            continue;
        }
        if (!pl->pack[w]) continue;
        int64_t rows, cols;
        operand_shape(p, w, &rows, &cols);
        const int64_t stride = w == 0 ? p.stride_a : p.stride_b;
        pl->pack_pitch[w] = align_up(cols * es, 16);
        pl->pack_stride[w] = stride == 0 ? 0 : rows * pl->pack_pitch[w];
        pl->pack_off[w] = off;
        off += align_up((stride == 0 ? 1 : p.batch) * rows * pl->pack_pitch[w], 256);
    }
    pl->ws_bytes = off;
}

// Tile class and split-K choice.  MI355X has 256 CUs; a launch wants at least
// about one workgroup per CU.  The big tile is used when it alone fills the
// chip; otherwise the smaller classes, then split-K for tall-K outputs with
// few tiles (the case tessl "Architecture" routes to split-K: K >= 2048 with
// small M and N).
//
// For 16-bit and int8 inputs the 256x256 and 128x128 classes run as the
// direct-to-LDS kernel (an operand it cannot read as it is gets packed
// first), and split-K runs on its 4-stage 128x128 tile, one workgroup per
// CU, in one round of workgroups: the slices stream the operands from HBM and
// write fp32 partial sums that one more kernel adds up in a fixed order.
//
// Tuning overrides (environment, read at every call; unset in normal use):
// TCGEMM_TILE=dma|dma8|dma128|dma128x4|thin|256|128|64|64ks|32ks|16ks forces a tile class
// (dma* only for 16-bit and int8 inputs, thin only for N <= 16 with A not
// transposed) without split-K, TCGEMM_SPLITS=S forces split-K
// with S slices (on a class with a partial-sum output: 64x64 or 128x128,
// else 64x64), TCGEMM_BAND=h sets the band height of the tile order (0:
// row-major).
// C = op(A) @ B^T with few rows (M <= 16, B stored [N, K]: a linear layer
// applied to a few vectors) is the transposed product C^T = B @ op(A)^T, an
// output of N rows and at most 16 columns with K-contiguous rows on the left:
// the thin-output kernel's shape, reading B (the large operand) once.  The
// returned problem is that product: A' = B, B' = A (stored [M, K], or [K, M]
// when transposed), C written transposed.
Problem transposed_problem(const Problem &p) {
    Problem q = p;
    q.M = p.N;
    q.N = p.M;
    q.ta = false;
    q.tb = !p.ta;
    q.lda = p.ldb;
    q.ldb = p.lda;
    q.stride_a = p.stride_b;
    q.stride_b = p.stride_a;
    q.a_ext = p.b_ext;
    q.b_ext = p.a_ext;
    q.a_total = p.b_total;
    q.b_total = p.a_total;
    q.c_trans = true;
    return q;
}

bool gemv_eligible(const Problem &p) {
    return !p.c_trans && p.M <= 16 && p.tb && p.alpha != 0.0f &&
           ceil_div(p.N, kThinRows) * p.batch >= 256;
}

bool gemv_route(const Problem &p, const Choice *ch) {
    if (!gemv_eligible(p)) return false;
    if (ch && ch->gemv >= 0) return ch->gemv == 1;
    if (ch && ch->cls >= 0) return false;                       // a chosen class
    if (knob(K_TILE)) return false;                    // a forced class
    if (const char *env = knob(K_GEMV))                // tuning knob: 0 disables
        if (atoi(env) == 0) return false;
    return true;
}

void make_plan(const Problem &p, Plan *pl, bool allow_edge = true, const Choice *ch = nullptr) {
    if (gemv_route(p, ch)) {
        make_plan(transposed_problem(p), pl, false);
        pl->swap = true;
        return;
    }
    pl->swap = false;
    const int es = dt_size(p.dt);
    const int bk = kLdsRowBytes / es;
    const bool dma = dma_types(p);
    const int64_t ktiles = ceil_div(p.K, bk);
    auto tile_count = [&](int c) {
        const TileShape ts = tile_shape(c);
        return ceil_div(p.M, ts.bm) * ceil_div(p.N, ts.bn) * p.batch;
    };
    // the largest tile class that alone fills the chip (at least 192 tiles)
    // and whose tile is less than half empty along M and N (a batch of
    // 128 x 128 problems on 256 x 256 tiles would be three quarters padding:
    // fp32 128^3 x 256 ran 60.9 us there against 18.0 on 128 x 128 tiles)
    int cls = TILE_64;
    for (int c = TILE_256; c <= TILE_64; ++c) {
        const TileShape ts = tile_shape(c);
        if (c == TILE_64 || (tile_count(c) >= 192 && ts.bm < 2 * p.M && ts.bn < 2 * p.N)) {
            cls = c;
            break;
        }
    }
    // 16-bit and int8 outputs just past one round of 256 x 256 tiles whose
    // extra tiles are whole (no thin strip for the edge split below): the
    // 128 x 128 tile, two workgroups per CU, when its rounds cost less.  A
    // round of 128 x 128 tiles covers half the outputs of a 256 x 256 round
    // at about 0.8 of its rate, i.e. 0.625 of its time.  Measured on bf16
    // 4096 x 4352 x 4096 (272 tiles of 256 x 256): 157.1 us against 186.3.
    if (dma && cls == TILE_256 && tile_count(TILE_256) > 256) {
        const int64_t rn = p.N % 256, rm = p.M % 256;
        const bool strip = (rn != 0 && rn <= 128 && p.N > 256) || (rm != 0 && rm <= 128 && p.M > 256);
        const double r256 = (double)ceil_div(tile_count(TILE_256), 256);
        const double r128 = 0.625 * (double)ceil_div(tile_count(TILE_128), 512);
        if (!strip && r128 < r256) cls = TILE_128;
    }
    // The same comparison the other way: too few 256 x 256 tiles to be taken
    // by count (under 192, M and N at least 256) but more 128 x 128 tiles
    // than two workgroups per CU hold (over 512): one partly filled round of
    // 256 x 256 tiles costs less than two rounds of 128 x 128.  Measured,
    // bf16 NN, us per call (256 / 128): 3072^2 x 8192 155.5 / 186.3, 3328 x
    // 3072 x 8192 141.6 / 177.9, 3072^2 x 4096 82.9 / 98.2; and where 128 x
    // 128 stays (484 and 400 tiles): 2816^2 x 8192 148.5 / 120.1, 2560^2 x
    // 8192 141.1 / 101.5.
    if (dma && cls == TILE_128 && p.M >= 256 && p.N >= 256 && tile_count(TILE_256) <= 256) {
        const double r256 = (double)ceil_div(tile_count(TILE_256), 256);
        const double r128 = 0.625 * (double)ceil_div(tile_count(TILE_128), 512);
        if (r256 < r128) cls = TILE_256;
    }
    int64_t splits = 1;
    // 16-bit and int8 outputs of 129 to 191 tiles of 128 x 128 (M and N at
    // least 256) and a long K: too many of those tiles for a K split of them
    // to fit one round of workgroups, too few to fill the chip unsplit.  The
    // 256 x 256 ring takes them with as many K slices as fit one round, at
    // least 16 K-tiles per slice and at least 192 workgroups.
    // The same for 192 to 256 tiles of 128 x 128 (one workgroup per CU
    // unsplit, each streaming all of K) when K is long enough that the
    // partial sums stay a small part of the traffic: at least 25 K-tiles
    // per slice (8 bytes of partial sums written and read per output and
    // slice, against 2 K multiply-adds).
    const int64_t t256 = tile_count(TILE_256), t128 = tile_count(TILE_128);
    const bool few128 = cls == TILE_64 && t128 > 128;
    const bool one128 = cls == TILE_128 && t128 <= 256;
    int64_t s256 = t256 > 0 ? 256 / t256 : 0;
    if (s256 > ktiles / (few128 ? 16 : 25)) s256 = ktiles / (few128 ? 16 : 25);
    if (s256 > 32) s256 = 32;
    // Both only from 160 K-tiles on: below that the unsplit 128 x 128 tile
    // with 4 stages (one workgroup per CU, see below) is ahead.  Measured,
    // bf16 NN, us per call (ring split / 4-stage unsplit): 2048^2 x 16384
    // (256 K-tiles) 130.9 / 143.4, 1536^2 x 12288 (192) 67.5 / 79.9;
    // 2048^2 x 8192 (128) 82.9 / 74.2, 4096 x 1024 x 8192 75.3 / 63.5,
    // 1664 x 1544 x 6144 (96) 51.8 / 45.3.
    const bool wide_split = dma && (few128 || one128) && p.M >= 256 && p.N >= 256 &&
                            p.alpha != 0.0f && ktiles >= 160 && s256 >= 2 && t256 * s256 >= 192;
    // Few tiles (under 128 of 64 x 64) and a short K: the 4 waves of a
    // workgroup take every 4th K-tile each and add their partial tiles in
    // LDS (each K-tile of the register-staged loop would wait out a memory
    // round trip), on the largest tile that still gives 128 workgroups, else
    // on 16 x 16 tiles; one launch, no workspace.  Short K: under 16 K-tiles,
    // or for fp32 up to 32 when the tiles fill a round of workgroups (the
    // split-K alternative there streams fp32 through the register-staged
    // loop; 16-bit and int8 split-K streams through the direct-to-LDS tile).
    // Measured on fp32 256^3 (16 x 16 tiles): 6.8 us per call against 9.7 us
    // for 8 slices of split-K plus the reduction; fp32 256 x 256 x 1024:
    // 8.6 against 10.4 us.
    const int ks_cls = tile_count(TILE_32_KS) >= 128 ? TILE_32_KS : TILE_16_KS;
    const bool ks = !wide_split && cls == TILE_64 && tile_count(TILE_64) < 128 && ktiles >= 4 &&
                    p.alpha != 0.0f &&
                    (ktiles < 16 || (!dma && ktiles <= 32 && tile_count(ks_cls) >= 256));
    // tall K and too few tiles to fill the chip: split K
    const bool split =
        !wide_split && !ks && cls == TILE_64 && tile_count(TILE_64) < 128 && ktiles >= 16 && p.alpha != 0.0f;
    // 16-bit and int8 outputs of 32 to 191 tiles of 128 x 128 (too few for
    // that class by the count above; M and N at least 128) run on 128 x 128
    // direct-to-LDS tiles, not on 64 x 64 tiles of the register-staged loop:
    // with a long K (32 K-tiles or more) on the 4-stage tile with as many K
    // slices as fill one round of workgroups, else on the 2-workgroup-per-CU
    // tile as it is.
    // Measured, bf16 NN, us per call: 4096 x 512 x 4096 30.3 (2 slices)
    // against 68.5 on 64 x 64 and 41.0 unsliced; 1024 x 768 x 2048 19.6
    // against 31.3 and 22.7; 1024^3 12.4 unsliced against 16.1 on 64 x 64
    // and 19.1 with slices; int8 2048 x 512 x 2048 12.3 unsliced against 21.6.
    const bool mid = !wide_split && !ks && !split && dma && cls == TILE_64 && tile_count(TILE_128) >= 32 &&
                     p.M >= 128 && p.N >= 128 && p.alpha != 0.0f;
    if (wide_split) {
        cls = TILE_256;                                          // TILE_256 -> TILE_256_DMA below
        splits = s256;
    } else if (ks) {
        cls = ks_cls;
    } else if (mid) {
        splits = ktiles >= 32 ? 256 / tile_count(TILE_128_DMA4) : 1;
        if (splits > ktiles / 4) splits = ktiles / 4;          // keep >= 4 K-tiles per slice
        if (splits > 32) splits = 32;
        cls = splits >= 2 ? TILE_128_DMA4 : TILE_128;          // TILE_128 -> TILE_128_DMA below
        if (splits < 2) splits = 1;
    } else if (split && dma) {
        // the 4-stage 128x128 tile, one workgroup per CU: as many slices as
        // fit one round of workgroups (a second, partial round costs more
        // than the extra slices gain; measured on the batched 128 x 384 x
        // 16384 shape: 10 slices, 240 workgroups)
        cls = TILE_128_DMA4;
        splits = 256 / tile_count(TILE_128_DMA4);
        if (splits > ktiles / 4) splits = ktiles / 4;          // keep >= 4 K-tiles per slice
        if (splits > 32) splits = 32;
    } else if (split) {
        // the register-staged loop waits out a memory round trip per K-tile:
        // short slices (about two K-tiles) on up to 512 workgroups
        splits = ceil_div(ktiles, 2);
        const int64_t cap = 512 / tile_count(TILE_64);
        if (splits > cap) splits = cap;
        if (splits > 64) splits = 64;
    }
    if (splits < 1) splits = 1;
    // at most 16 output columns and K-contiguous A rows: the vector-ALU
    // dot-product kernel, when its 8-row workgroups give every CU at least
    // one (a matrix-core tile would be at least 16 / N padding, and the
    // work is bound by reading A once)
    const bool thin_ok = p.N <= 16 && !p.ta && p.alpha != 0.0f;
    if (thin_ok && ceil_div(p.M, kThinRows) * p.batch >= 256) {
        cls = TILE_THIN;
        splits = 1;
    }
    if (dma && cls == TILE_256) cls = TILE_256_DMA;
    if (dma && cls == TILE_128) cls = TILE_128_DMA;
    // 128 x 128 tiles that leave every CU at most one workgroup: the 4-stage
    // variant, three K-tiles in flight instead of one (the room the 2-stage
    // variant leaves for a second workgroup per CU has nothing to run).
    // Measured, bf16 NN, us per call (4 stages / 2): 4096 x 1024 x 4096 37.9
    // / 47.4, 3072 x 1024 x 3072 27.5 / 34.7, 2048^3 21.8 / 26.4, 2048^2 x
    // 4096 37.2 / 46.8, 1024^3 11.5 / 13.7, fp16 3072 x 512 x 1024 12.0 /
    // 14.0, int8 2048 x 512 x 2048 12.3 / 14.5.  With 288 tiles (3072 x 1536
    // x 2048) the 2-stage tile, two per CU, stays ahead (28.5 against 36.1),
    // and so it does with under 16 K-tiles, where the deeper pipeline has
    // little to overlap (fp16 1024^2 x 512 7.7 against 8.2, int8 1024^3 8.5
    // against 9.1, a batch of 256 bf16 128^3 7.7 against 8.0).
    if (cls == TILE_128_DMA && splits == 1 && tile_count(TILE_128) <= 256 && ktiles >= 16)
        cls = TILE_128_DMA4;
    if (const char *env = knob(K_TILE)) {
        const int v = atoi(env);
        if (strcmp(env, "dma") == 0) cls = dma ? TILE_256_DMA : cls;
        else if (strcmp(env, "dma8") == 0) cls = dma ? TILE_256_DMA8 : cls;
        else if (strcmp(env, "dma128") == 0) cls = dma ? TILE_128_DMA : cls;
        else if (strcmp(env, "dma128x4") == 0) cls = dma ? TILE_128_DMA4 : cls;
        else if (strcmp(env, "thin") == 0) cls = thin_ok ? TILE_THIN : cls;
        else if (strcmp(env, "64ks") == 0) cls = TILE_64_KS;
        else if (strcmp(env, "32ks") == 0) cls = TILE_32_KS;
        else if (strcmp(env, "16ks") == 0) cls = TILE_16_KS;
        else cls = v == 256 ? TILE_256 : v == 128 ? TILE_128 : v == 64 ? TILE_64 : cls;
        splits = 1;   // a forced class splits only when TCGEMM_SPLITS says so
    }
    if (const char *env = knob(K_SPLITS)) {
        const int64_t forced = atoi(env);
        if (forced > 0 && p.alpha != 0.0f) splits = forced > ktiles ? ktiles : forced;
    }
    if (ch && ch->cls >= 0) {
        // a chosen class (validated by the caller for this problem)
        cls = ch->cls;
        splits = ch->splits > 0 && p.alpha != 0.0f ? (ch->splits > ktiles ? ktiles : ch->splits) : 1;
    }
    if (splits > 1 && !splits_ok(cls)) cls = TILE_64;
    if (cls == TILE_THIN) splits = 1;
    const TileShape ts = tile_shape(cls);
    pl->cls = cls;
    pl->bm = ts.bm; pl->bn = ts.bn; pl->bk = bk;
    pl->tiles_m = (int32_t)ceil_div(p.M, ts.bm);
    pl->tiles_n = (int32_t)ceil_div(p.N, ts.bn);
    const int64_t tiles = (int64_t)pl->tiles_m * pl->tiles_n * p.batch;

    int64_t kps = ceil_div(ceil_div(p.K, splits), bk) * bk;
    splits = ceil_div(p.K, kps);                            // every slice non-empty
    if (splits > 1 && (int64_t)splits * p.M * p.N * 4 > 0x7FFFFFFF) {  // reduce offsets are 32-bit
        splits = 1;
        kps = ceil_div(p.K, bk) * bk;
    }
    pl->splits = (int32_t)splits;
    pl->k_per_split = (int32_t)kps;
    pl->grid = tiles * splits;
    pl->band = 8;
    if (const char *env = knob(K_BAND)) pl->band = atoi(env);   // tuning knob
    const bool aligned[2] = {true, true};
    layout_workspace(p, pl, aligned);

    // Edge split.  A 256x256 launch whose last tile column (or row) holds
    // only a thin ragged strip can cost a whole extra round of workgroups
    // (272 tiles on 256 CUs take two rounds).  Such a strip runs as a
    // second, split-K GEMM of its own when dropping it from the main launch
    // saves a round.
    pl->edge = 0;
    pl->edge_at = 0;
    const char *env_edge = knob(K_EDGE);   // tuning knob: 0 disables
    if (allow_edge && p.alpha != 0.0f && (cls == TILE_256_DMA || cls == TILE_256_DMA8) && splits == 1 &&
        !(env_edge && atoi(env_edge) == 0)) {
        auto rounds = [](int64_t t) { return (t + 255) / 256; };
        const int64_t rn = p.N % ts.bn, rm = p.M % ts.bm;
        const int64_t tmn = (int64_t)pl->tiles_m * pl->tiles_n;
        // (a strip only when whole tiles remain beside it)
        if (rn != 0 && rn <= ts.bn / 2 && pl->tiles_n > 1 &&
            rounds((tmn - pl->tiles_m) * p.batch) < rounds(tmn * p.batch)) {
            pl->edge = 1;
            pl->edge_at = (int32_t)(p.N - rn);
        } else if (rm != 0 && rm <= ts.bm / 2 && pl->tiles_m > 1 &&
                   rounds((tmn - pl->tiles_n) * p.batch) < rounds(tmn * p.batch)) {
            pl->edge = 2;
            pl->edge_at = (int32_t)(p.M - rm);
        }
    }
    // Round split.  Past one round of 256 x 256 tiles, the tiles of the last
    // partial round can cost more than they are worth to the whole launch:
    // the rows (or columns) of tiles that fill whole rounds then run as one
    // launch of 256 x 256 tiles and the rest as a second GEMM with a plan of
    // its own, when the two cost less by the round count used above (a
    // round of 256 x 256 tiles = 1, of 128 x 128 two per CU = 0.625; 0.05
    // for the second launch).  Measured, bf16 NN, us per call (whole /
    // split): 6144 x 4096 x 4096 199.2 / 171.3, 6144^3 379.0 / 358.0, 5120 x
    // 4096 x 4096 158.6 / 144.9, 4096 x 4352 x 4096 150.7 / 140.7, 6144 x
    // 4096 x 2048 100.7 / 92.0; 7168 x 4096 x 4096 (no gain by the count)
    // 189.9 / 188.8.
    if (pl->edge == 0 && allow_edge && dma && p.alpha != 0.0f && splits == 1 && p.batch == 1 &&
        (cls == TILE_256_DMA || cls == TILE_128_DMA) && !knob(K_TILE) && !(ch && ch->cls >= 0) &&
        !(env_edge && atoi(env_edge) == 0)) {
        auto cost = [](int64_t m, int64_t n) {
            const int64_t t2 = ceil_div(m, 256) * ceil_div(n, 256), t1 = ceil_div(m, 128) * ceil_div(n, 128);
            const double r2 = (double)ceil_div(t2, 256), r1 = 0.625 * (double)ceil_div(t1, 512);
            return r2 < r1 ? r2 : r1;
        };
        const int64_t tm = ceil_div(p.M, 256), tn = ceil_div(p.N, 256), t2 = tm * tn;
        if (t2 > 256 && t2 % 256 != 0) {
            const int64_t full = t2 / 256 * 256;   // tiles of the whole rounds
            double best = cost(p.M, p.N) - 0.05;
            const int64_t rows = full / tn, cols = full / tm;
            if (rows >= 1 && rows < tm) {
                const double c = (double)ceil_div(rows * tn, 256) + cost(p.M - rows * 256, p.N);
                if (c < best) {
                    best = c;
                    pl->edge = 2;
                    pl->edge_at = (int32_t)(rows * 256);
                }
            }
            if (cols >= 1 && cols < tn) {
                const double c = (double)ceil_div(cols * tm, 256) + cost(p.M, p.N - cols * 256);
                if (c < best) {
                    best = c;
                    pl->edge = 1;
                    pl->edge_at = (int32_t)(cols * 256);
                }
            }
        }
    }
}

// The part [lo, lo + n) of problem p along N (axis 1) or M (axis 2), and the
// element offsets of its A, B and C origins.
Problem sub_problem(const Problem &p, int axis, int64_t lo, int64_t n, int64_t off[3]) {
    Problem q = p;
    off[0] = off[1] = off[2] = 0;
    if (axis == 1) {
        q.N = (int32_t)n;
        off[1] = p.tb ? lo * p.ldb : lo;
        off[2] = lo;
        q.b_ext = p.tb ? span(n, p.K, p.ldb) : span(p.K, n, p.ldb);
    } else {
        q.M = (int32_t)n;
        off[0] = p.ta ? lo : lo * p.lda;
        off[2] = lo * p.ldc;
        q.a_ext = p.ta ? span(p.K, n, p.lda) : span(n, p.K, p.lda);
    }
    q.c_ext = span(q.M, q.N, p.ldc);
    const int es = dt_size(p.dt), ces = dt_size(p.cdt);
    q.a_total = total_bytes(p.batch, p.stride_a, q.a_ext, es);
    q.b_total = total_bytes(p.batch, p.stride_b, q.b_ext, es);
    q.c_total = total_bytes(p.batch, p.stride_c, q.c_ext, ces);
    return q;
}

// The two parts of an edge-split problem with their plans.
struct Parts {
    int n;
    int axis;           // 1: the second part is a column strip, 2: a row strip
    Problem p[2];
    Plan pl[2];
    int64_t off[2][3];  // element offsets of the part's A, B, C origins (caller's operands)
    bool swap[2];       // the part runs as its transposed product (A and B exchanged)
};

Parts split_parts(const Problem &p, const Plan &pl) {
    Parts r;
    r.swap[0] = r.swap[1] = false;
    r.axis = pl.swap ? 0 : pl.edge;
    if (pl.swap) {
        r.n = 1;
        r.p[0] = transposed_problem(p);
        r.pl[0] = pl;
        r.off[0][0] = r.off[0][1] = r.off[0][2] = 0;
        r.swap[0] = true;
        return r;
    }
    if (pl.edge == 0) {
        r.n = 1;
        r.p[0] = p;
        r.pl[0] = pl;
        r.off[0][0] = r.off[0][1] = r.off[0][2] = 0;
        return r;
    }
    r.n = 2;
    const int64_t ext = pl.edge == 1 ? p.N : p.M;
    r.p[0] = sub_problem(p, pl.edge, 0, pl.edge_at, r.off[0]);
    r.p[1] = sub_problem(p, pl.edge, pl.edge_at, ext - pl.edge_at, r.off[1]);
    for (int i = 0; i < 2; ++i) {
        make_plan(r.p[i], &r.pl[i], false);
        // a strip of at most 16 rows can take the small-M route itself
        if (r.pl[i].swap) {
            r.p[i] = transposed_problem(r.p[i]);
            r.swap[i] = true;
        }
    }
    return r;
}

// The kernels a plan launches, in order, joined by '+'.
std::string kernel_chain(const Problem &p, const Plan &pl) {
    if (p.alpha == 0.0f) return "scale_c";
    std::string name;
    if (p.c_trans) {
        // the transposed product of a small-M GEMM, named by the caller's
        // layout: its A is the product's B (gathered when stored [K, M])
        if (pl.pack[1]) name += "transpose_a+";
        name += std::string("gemv_") + dt_name(p.dt) + (p.tb ? "_nt" : "_tt") + "_thin";
        return name;
    }
    if (pl.pack[0]) name += "pack_a+";
    if (pl.pack[1]) name += thin_transposes_b(p, pl) ? "transpose_b+" : "pack_b+";
    name += tcg_kernel_name(p.dt, p.ta, p.tb, pl.cls);
    if (pl.splits > 1) name += "+splitk_reduce";
    return name;
}

int plan_launches(const Problem &p, const Plan &pl) {
    if (p.alpha == 0.0f) return 1;
    return 1 + (pl.splits > 1) + pl.pack[0] + pl.pack[1];
}

// A column strip whose B^T comes out of the main part's row packing of B:
// when the main part packs B stored [K, N] row by row and the strip runs on
// the thin kernel (which reads B^T), the packing kernel also writes the
// strip's columns, which follow the main part's in every row, transposed,
// and the strip needs no gather pass.  The B^T goes after the main part's
// workspace.  main and strip: the parts' plans as laid out for the call.
struct StripBt {
    bool on = false;
    int64_t off = 0;             // workspace byte offset of the B^T
    int64_t pitch = 0, stride = 0, bytes = 0;
    int32_t cols = 0;            // the strip's columns
};

StripBt strip_bt(const Parts &r, const Plan &main, const Plan &strip) {
    StripBt b;
    if (r.n != 2 || r.axis != 1 || r.swap[0] || r.swap[1] || r.p[0].alpha == 0.0f) return b;
    const Problem &m = r.p[0], &st = r.p[1];
    if (!main.pack[1] || m.tb || thin_transposes_b(m, main) || !thin_transposes_b(st, strip))
        return b;
    b.on = true;
    b.cols = st.N;
    b.pitch = strip.pack_pitch[1];
    b.stride = strip.pack_stride[1];
    b.off = align_up(main.ws_bytes, 256);
    b.bytes = align_up((st.stride_b == 0 ? 1 : st.batch) * st.N * b.pitch, 256);
    return b;
}

// The strip's plan as it runs when its B^T comes from the main part.
Plan without_bt_pass(const Plan &pl) {
    Plan q = pl;
    q.pack[1] = false;
    return q;
}

// Kernel chains of the parts, joined by '|'.
std::string parts_chain(const Parts &r) {
    const bool fused = strip_bt(r, r.pl[0], r.pl[1]).on;
    std::string name = kernel_chain(r.p[0], r.pl[0]);
    for (int i = 1; i < r.n; ++i)
        name += "|" + kernel_chain(r.p[i], fused ? without_bt_pass(r.pl[i]) : r.pl[i]);
    return name;
}

void fill_info(const Problem &p, const Plan &pl, tc_plan_info *info) {
    if (!info) return;
    memset(info, 0, sizeof *info);
    const Parts parts = split_parts(p, pl);
    snprintf(info->kernel, sizeof info->kernel, "%s", parts_chain(parts).c_str());
    const StripBt sb = strip_bt(parts, parts.pl[0], parts.pl[1]);
    const Plan &m = parts.pl[0];   // tile fields: the main (whole-tile) part
    info->tile_m = m.bm; info->tile_n = m.bn; info->tile_k = m.bk;
    info->threads = tile_threads(m.cls);
    info->tiles_m = m.tiles_m; info->tiles_n = m.tiles_n;
    info->splits = m.splits; info->k_per_split = m.k_per_split;
    info->grid = 0;
    info->workspace_bytes = 0;
    info->launches = 0;
    for (int i = 0; i < parts.n; ++i) {
        if (p.alpha != 0.0f) info->grid += parts.pl[i].grid;
        if (p.alpha != 0.0f && parts.pl[i].ws_bytes > info->workspace_bytes)
            info->workspace_bytes = parts.pl[i].ws_bytes;
        info->launches += plan_launches(parts.p[i], i == 1 && sb.on ? without_bt_pass(parts.pl[i])
                                                                     : parts.pl[i]);
    }
    if (sb.on && sb.off + sb.bytes > info->workspace_bytes) info->workspace_bytes = sb.off + sb.bytes;
    info->band = pl.band;
}

bool ranges_overlap(const void *a, int64_t an, const void *b, int64_t bn) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)bn && b0 < a0 + (uintptr_t)an;
}

tc_status_t check_allocation(const char *name, const void *ptr, int64_t bytes, std::string *err) {
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    hipError_t e = hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)ptr);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(err, TC_ERR_INVALID_ARGUMENT, "%s=%p is not device memory (%s)", name, ptr,
                    hipGetErrorString(e));
    }
    const uintptr_t b0 = (uintptr_t)base, p0 = (uintptr_t)ptr;
    if (p0 < b0 || p0 + (uintptr_t)bytes > b0 + size)
        return fail(err, TC_ERR_INVALID_ARGUMENT,
                    "%s needs %lld bytes from %p but its allocation ends %lld bytes after it", name,
                    (long long)bytes, ptr, (long long)(b0 + size - p0));
    return TC_OK;
}

tc_status_t bind_device(tc_context *ctx) {
    if (ctx->device >= 0) return hipSetDevice(ctx->device) == hipSuccess ? TC_OK : TC_ERR_DEVICE;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        ctx->last_error = std::string("no HIP device: ") + hipGetErrorString(e);
        return TC_ERR_DEVICE;
    }
    ctx->device = dev;
    return TC_OK;
}

tc_status_t ensure_workspace(tc_stream *s, int64_t bytes, std::string *err) {
    if (bytes <= s->ws_bytes) return TC_OK;
    if (s->ws) {
        // the old buffer may still be in use by work queued on this stream
        if (hipStreamSynchronize(s->stream) != hipSuccess)
            return fail(err, TC_ERR_DEVICE, "hipStreamSynchronize failed while growing the workspace");
        (void)hipFree(s->ws);
        s->ws = nullptr;
        s->ws_bytes = 0;
    }
    const int64_t want = ((bytes + (1 << 20) - 1) >> 20) << 20;
    hipError_t e = hipMalloc(&s->ws, (size_t)want);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        s->ws = nullptr;
        return fail(err, TC_ERR_OUT_OF_MEMORY, "split-K workspace of %lld bytes: %s", (long long)want,
                    hipGetErrorString(e));
    }
    s->ws_bytes = want;
    return TC_OK;
}

tc_status_t create_stream(tc_context *ctx, tc_stream **out, hipStream_t existing) {
    tc_stream *s = new (std::nothrow) tc_stream();
    if (!s) return TC_ERR_OUT_OF_MEMORY;
    s->ctx = ctx;
    if (existing) {
        s->stream = existing;
        s->owned = false;
    } else {
        hipError_t e = hipStreamCreate(&s->stream);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            ctx->last_error = std::string("hipStreamCreate: ") + hipGetErrorString(e);
            delete s;
            return TC_ERR_DEVICE;
        }
        s->owned = true;
    }
    *out = s;
    return TC_OK;
}

// Enqueue the launches of one planned problem (packs, GEMM, reduction) on
// stream s; their names are appended to *names.
// sb: a column strip's B^T made by the main part's B packing (null: none);
// sb_writes: this part is the main part (its B packing writes the B^T), else
// the strip (its thin kernel reads the B^T, with no gather pass).
// fixed_ws: the allocation-free call's scratch (null: the stream's
// workspace, grown here on demand); its size was checked by the caller.
tc_status_t enqueue(tc_context *ctx, tc_stream *s, const Problem &p, const Plan &plan,
                    const void *A, const void *B, void *C, const Epilogue &epi, bool main_part,
                    std::string *names, std::string *err, const StripBt *sb = nullptr,
                    bool sb_writes = false, void *fixed_ws = nullptr) {
    Plan pl = plan;
    const bool aligned[2] = {(uintptr_t)A % 16 == 0, (uintptr_t)B % 16 == 0};
    layout_workspace(p, &pl, aligned);   // a misaligned base pointer is packed too
    const bool bt_ready = sb && !sb_writes;
    *names += kernel_chain(p, bt_ready ? without_bt_pass(pl) : pl);
    tc_status_t st;
    const bool use_splitk = p.alpha != 0.0f && pl.splits > 1;
    const bool use_ws = p.alpha != 0.0f && pl.ws_bytes > 0;
    if (use_ws && !fixed_ws && (st = ensure_workspace(s, pl.ws_bytes, err)) != TC_OK) return st;
    char *const wsb = static_cast<char *>(fixed_ws ? fixed_ws : s->ws);

    const int ces = dt_size(p.cdt);
    // Four complete C values of a row go as one vector access (16 bytes for
    // 32-bit types, 8 for 16-bit) at any alignment: the GPU runs with
    // unaligned memory access enabled, and one unaligned vector access costs
    // less than four element accesses (odd ldc included).
    const bool c_vec_ok = true;
    EpilogueArgs ea;
    memset(&ea, 0, sizeof ea);
    ea.C = C;
    ea.stride_c = p.stride_c;
    ea.c_extent = p.c_ext * ces;
    ea.M = p.M; ea.N = p.N; ea.ldc = (int32_t)p.ldc;
    ea.batch = p.batch;
    ea.c_dtype = p.cdt;
    ea.acc_is_int = p.dt == TC_I8;
    ea.alpha = p.alpha; ea.beta = p.beta;
    ea.c_vec_ok = c_vec_ok;
    ea.bias = epi.bias;
    ea.bias_stride = epi.bias_stride;
    ea.scale = epi.scale;
    ea.scale_stride = epi.scale_stride;
    ea.act = epi.act;
    ea.epi = epi.on();

    hipError_t e = hipSuccess;
    if (p.alpha == 0.0f) {
        e = tcg_launch_scale_c(ea, s->stream);
        if (e == hipSuccess) ctx->dispatches += 1;
    } else {
        const int es = dt_size(p.dt);
        const void *src[2] = {A, B};
        int64_t ld[2] = {p.lda, p.ldb}, stride[2] = {p.stride_a, p.stride_b};
        int64_t extent[2] = {p.a_ext * es, p.b_ext * es};
        bool tb = p.tb;
        for (int w = 0; w < 2 && e == hipSuccess; ++w) {
            if (!pl.pack[w]) continue;
            if (w == 1 && thin_transposes_b(p, pl) && bt_ready) {
                // the main part's B packing wrote this strip's B^T
                src[1] = wsb + sb->off;
                ld[1] = sb->pitch / es;
                stride[1] = sb->stride / es;
                extent[1] = (int64_t)p.N * sb->pitch;
                tb = true;
                continue;
            }
            if (w == 1 && thin_transposes_b(p, pl)) {
                PackArgs pa;
                memset(&pa, 0, sizeof pa);
                pa.src = src[1];
                pa.dst = wsb + pl.pack_off[1];
                pa.src_stride = stride[1] * es;
                pa.dst_stride = pl.pack_stride[1];
                pa.src_pitch = ld[1] * es;
                pa.dst_pitch = pl.pack_pitch[1];
                pa.rows = p.K;
                pa.row_bytes = p.N * es;
                pa.batch = stride[1] == 0 ? 1 : p.batch;
                e = tcg_launch_thin_pack_bt(pa, es, s->stream);
                if (e != hipSuccess) break;
                ctx->dispatches += 1;
                // the thin kernel reads B^T: N rows of K values
                src[1] = pa.dst;
                ld[1] = pl.pack_pitch[1] / es;
                stride[1] = pl.pack_stride[1] / es;
                extent[1] = (int64_t)p.N * pl.pack_pitch[1];
                tb = true;
                continue;
            }
            int64_t rows, cols;
            operand_shape(p, w, &rows, &cols);
            PackArgs pa;
            memset(&pa, 0, sizeof pa);
            pa.src = src[w];
            pa.dst = wsb + pl.pack_off[w];
            pa.src_stride = stride[w] * es;
            pa.dst_stride = pl.pack_stride[w];
            pa.src_pitch = ld[w] * es;
            pa.dst_pitch = pl.pack_pitch[w];
            pa.rows = (int32_t)rows;
            pa.row_bytes = (int32_t)(cols * es);
            pa.batch = stride[w] == 0 ? 1 : p.batch;
            if (w == 1 && sb && sb_writes) {
                pa.bt = wsb + sb->off;
                pa.bt_stride = sb->stride;
                pa.bt_pitch = (int32_t)sb->pitch;
                pa.bt_cols = sb->cols;
                pa.bt_es = es;
            }
            e = tcg_launch_pack_rows(pa, s->stream);
            if (e != hipSuccess) break;
            ctx->dispatches += 1;
            // the GEMM reads the packed copy
            src[w] = pa.dst;
            ld[w] = pl.pack_pitch[w] / es;
            stride[w] = pl.pack_stride[w] / es;
            extent[w] = rows * pl.pack_pitch[w];   // whole padded rows
        }
        GemmArgs ga;
        memset(&ga, 0, sizeof ga);
        ga.A = src[0]; ga.B = src[1]; ga.C = C;
        ga.ws = use_splitk ? wsb : nullptr;
        ga.stride_a = stride[0]; ga.stride_b = stride[1]; ga.stride_c = p.stride_c;
        ga.a_extent = extent[0];
        ga.b_extent = extent[1];
        ga.c_extent = p.c_ext * ces;
        ga.M = p.M; ga.N = p.N; ga.K = p.K;
        ga.lda = (int32_t)ld[0]; ga.ldb = (int32_t)ld[1]; ga.ldc = (int32_t)p.ldc;
        ga.c_dtype = p.cdt;
        ga.alpha = p.alpha; ga.beta = p.beta;
        ga.tiles_m = pl.tiles_m; ga.tiles_n = pl.tiles_n;
        ga.splits = pl.splits; ga.k_per_split = pl.k_per_split;
        ga.groups = p.batch * pl.splits;
        ga.band = pl.band;
        ga.c_vec_ok = c_vec_ok;
        ga.c_dma_ok = (p.ldc * ces) % 16 == 0 && (p.stride_c * ces) % 16 == 0 &&
                      (uintptr_t)C % 16 == 0;
        ga.bias = epi.bias;
        ga.bias_stride = epi.bias_stride;
        ga.scale = epi.scale;
        ga.scale_stride = epi.scale_stride;
        ga.c_trans = p.c_trans;
        ga.act = epi.act;
        ga.epi = epi.on();
        // an armed measurement brackets the GEMM kernel alone (one call only)
        hipEvent_t ev_start = nullptr, ev_end = nullptr;
        if (main_part) {
            ev_start = ctx->time_ev[0];
            ev_end = ctx->time_ev[1];
            ctx->time_ev[0] = ctx->time_ev[1] = nullptr;
        }
        if (ev_start && e == hipSuccess) e = hipEventRecord(ev_start, s->stream);
        if (e == hipSuccess && pl.cls == TILE_THIN)
            e = tb ? tcg_launch_thin(p.dt, p.cdt, ga, pl.grid, s->stream) : hipErrorInvalidValue;
        else if (e == hipSuccess)
            e = tcg_launch_gemm(p.dt, p.ta, p.tb, pl.cls, use_splitk ? OUT_PARTIAL : p.cdt, ga,
                                pl.grid, s->stream);
        if (ev_end && e == hipSuccess) e = hipEventRecord(ev_end, s->stream);
        if (e == hipSuccess) {
            ctx->dispatches += 1;
            if (use_splitk) {
                ea.ws = wsb;
                ea.splits = pl.splits;
                e = tcg_launch_splitk_reduce(ea, s->stream);
                if (e == hipSuccess) ctx->dispatches += 1;
            }
        }
    }
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(err, TC_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    }
    return TC_OK;
}

// Bytes the bias (w = 0) or scale (w = 1) vectors of all problems span.
int64_t epilogue_vec_bytes(const Problem &p, const Epilogue &e, int w) {
    return ((int64_t)(p.batch - 1) * (w ? e.scale_stride : e.bias_stride) + p.N) *
           (w ? 4 : dt_size(p.cdt));
}

// The fused epilogue (tessl "Architecture", "Fused Epilogue"): it needs the
// register accumulator of a float GEMM, so int8 (exact int32 results) is
// refused rather than run as separate passes; the bias is read while C is
// written, so it may not overlap C.
tc_status_t validate_epilogue(const Problem &p, const tc_epilogue *ep, const void *C, Epilogue *out,
                              std::string *err) {
    if (ep->activation != TC_ACT_NONE && ep->activation != TC_ACT_RELU &&
        ep->activation != TC_ACT_GELU_TANH)
        return fail(err, TC_ERR_INVALID_ARGUMENT, "unknown activation %d", (int)ep->activation);
    if (p.dt == TC_I8 && p.cdt == TC_I32)
        return fail(err, TC_ERR_UNSUPPORTED,
                    "the fused epilogue needs a float result; int8 into int32 is the exact sum "
                    "(give a per-column scale and a float C to dequantize)");
    if (ep->bias_stride < 0 || ep->scale_stride < 0)
        return fail(err, TC_ERR_INVALID_ARGUMENT, "bias_stride and scale_stride must be >= 0");
    out->bias = ep->bias;
    out->bias_stride = p.batch > 1 ? ep->bias_stride : 0;
    out->scale = ep->col_scale;
    out->scale_stride = p.batch > 1 ? ep->scale_stride : 0;
    out->act = ep->activation == TC_ACT_RELU ? ACT_RELU
             : ep->activation == TC_ACT_GELU_TANH ? ACT_GELU_TANH : ACT_NONE;
    const void *vec[2] = {out->bias, out->scale};
    const int64_t stride[2] = {out->bias_stride, out->scale_stride};
    const int64_t es[2] = {dt_size(p.cdt), 4};
    const char *name[2] = {"bias", "col_scale"};
    for (int w = 0; w < 2; ++w) {
        if (!vec[w]) continue;
        int64_t t, bytes;
        if (__builtin_mul_overflow((int64_t)(p.batch - 1), stride[w], &t) ||
            __builtin_add_overflow(t, (int64_t)p.N, &t) || __builtin_mul_overflow(t, es[w], &bytes))
            return fail(err, TC_ERR_OVERFLOW, "%s extent overflows 64 bits", name[w]);
        if (ranges_overlap(C, p.c_total, vec[w], bytes))
            return fail(err, TC_ERR_ALIASING, "the %s overlaps C", name[w]);
    }
    return TC_OK;
}

// Validate, plan and enqueue one (batched) GEMM on stream s.
// Enqueue every part of a planned call (the whole tiles, then the edge strip
// if the plan splits one off); their kernel names go to *name.
// The operand pointers of part i of a call (the parts of an edge split,
// or the transposed product of a small-M GEMM, which exchanges A and B).
const void *part_operand(const Parts &parts, int i, int w, const void *A, const void *B, int es) {
    const bool from_b = (w == 1) != parts.swap[i];
    return static_cast<const char *>(from_b ? B : A) + parts.off[i][from_b ? 1 : 0] * es;
}

// Workspace a call uses with these operand pointers: the largest part's
// (split-K partials and packed copies, laid out for the pointers' 16-byte
// alignment), and the strip's B^T when the main part's packing writes it.
// *sb receives that B^T's placement.
int64_t call_workspace(const Problem &p, const Plan &pl, const void *A, const void *B,
                       StripBt *sb) {
    *sb = StripBt{};
    if (p.alpha == 0.0f) return 0;
    const Parts parts = split_parts(p, pl);
    const int es = dt_size(p.dt);
    Plan lp[2];
    int64_t need = 0;
    for (int i = 0; i < parts.n; ++i) {
        lp[i] = parts.pl[i];
        const bool aligned[2] = {(uintptr_t)part_operand(parts, i, 0, A, B, es) % 16 == 0,
                                 (uintptr_t)part_operand(parts, i, 1, A, B, es) % 16 == 0};
        layout_workspace(parts.p[i], &lp[i], aligned);
        if (lp[i].ws_bytes > need) need = lp[i].ws_bytes;
    }
    if (parts.n == 2) {
        *sb = strip_bt(parts, lp[0], lp[1]);
        if (sb->on && sb->off + sb->bytes > need) need = sb->off + sb->bytes;
    }
    return need;
}

tc_status_t enqueue_call(tc_context *ctx, tc_stream *s, const Problem &p, const Plan &pl,
                         const void *A, const void *B, void *C, const Epilogue &epi,
                         std::string *name, std::string *err, void *fixed_ws = nullptr) {
    const Parts parts = split_parts(p, pl);
    const int es = dt_size(p.dt);
    // the strip's B^T from the main part's packing, laid out for these
    // pointers (a misaligned base pointer changes what is packed)
    StripBt sb;
    const int64_t need = call_workspace(p, pl, A, B, &sb);
    tc_status_t st;
    if (sb.on && !fixed_ws && (st = ensure_workspace(s, need, err)) != TC_OK) return st;
    for (int i = 0; i < parts.n; ++i) {
        const int ces = dt_size(p.cdt);
        const void *Ai = part_operand(parts, i, 0, A, B, es);
        const void *Bi = part_operand(parts, i, 1, A, B, es);
        void *Ci = static_cast<char *>(C) + parts.off[i][2] * ces;
        // a column strip's bias and scales start at its first column
        Epilogue epi_i = epi;
        if (pl.edge == 1 && i == 1) {
            if (epi.bias) epi_i.bias = static_cast<const char *>(epi.bias) + (int64_t)pl.edge_at * ces;
            if (epi.scale) epi_i.scale = epi.scale + pl.edge_at;
        }
        if (i) *name += "|";
        st = enqueue(ctx, s, parts.p[i], parts.pl[i], Ai, Bi, Ci, epi_i, i == 0, name, err,
                     sb.on ? &sb : nullptr, i == 0, fixed_ws);
        if (st != TC_OK) return st;
    }
    return TC_OK;
}

// Autotuning key: everything the plan or the kernels' speed depends on.
std::string tune_key(const Problem &p, const Epilogue &epi, const void *A, const void *B) {
    char k[320];
    snprintf(k, sizeof k, "%d:%d:%d%d:%d:%d:%d:%d:%lld:%lld:%lld:%lld:%lld:%lld:%d:%d:%d",
             p.dt, p.cdt, (int)p.ta, (int)p.tb, p.M, p.N, p.K, p.batch, (long long)p.lda,
             (long long)p.ldb, (long long)p.ldc, (long long)p.stride_a, (long long)p.stride_b,
             (long long)p.stride_c, (int)(p.beta != 0.0f), (int)epi.on(),
             (int)((uintptr_t)A % 16 == 0) * 2 + (int)((uintptr_t)B % 16 == 0));
    return k;
}

// The candidates a first call measures: the planner's own choice, every tile
// class that fits the input type (with and without the planner's split
// count, halved and doubled, for the classes that split), the thin kernel
// and the small-M route where they apply.
std::vector<Choice> tune_candidates(const Problem &p) {
    std::vector<Choice> c;
    c.push_back(Choice{});
    Plan base;
    make_plan(p, &base);
    const int64_t s0 = base.swap ? 1 : base.splits;
    const bool dma = dma_types(p);
    const int classes_dma[] = {TILE_256_DMA, TILE_256_DMA8, TILE_128_DMA, TILE_128_DMA4, TILE_64,
                               TILE_64_KS, TILE_32_KS, TILE_16_KS};
    const int classes_f32[] = {TILE_256, TILE_128, TILE_64, TILE_64_KS, TILE_32_KS, TILE_16_KS};
    const int *cl = dma ? classes_dma : classes_f32;
    const int ncl = dma ? 8 : 6;
    for (int i = 0; i < ncl; ++i) {
        c.push_back(Choice{cl[i], 1, 0});
        if (splits_ok(cl[i]) && s0 > 1)
            for (int64_t s : {s0 / 2, s0, s0 * 2})
                if (s > 1) c.push_back(Choice{cl[i], s, 0});
    }
    if (p.N <= 16 && !p.ta && p.alpha != 0.0f) c.push_back(Choice{TILE_THIN, 1, 0});
    if (gemv_eligible(p)) c.push_back(Choice{-1, 0, 1});
    return c;
}

// Time each candidate on this stream (C replaced by a scratch buffer and
// beta by 0, so C is untouched; one warm-up and three timed runs each, the
// fastest counted) and return the best.  Candidates with identical launch
// chains are measured once.
tc_status_t autotune(tc_context *ctx, tc_stream *s, const Problem &p, const void *A, const void *B,
                     const Epilogue &epi, Choice *best, std::string *err) {
    Problem q = p;
    q.beta = 0.0f;
    void *scratch = nullptr;
    hipEvent_t ev[2] = {nullptr, nullptr};
    hipError_t e = hipMalloc(&scratch, (size_t)p.c_total);
    if (e == hipSuccess) e = hipEventCreate(&ev[0]);
    if (e == hipSuccess) e = hipEventCreate(&ev[1]);
    tc_status_t st = TC_OK;
    float best_ms = 1e30f;
    *best = Choice{};
    std::vector<std::string> seen;
    for (const Choice &ch : tune_candidates(q)) {
        if (e != hipSuccess || st != TC_OK) break;
        Plan pl;
        make_plan(q, &pl, true, &ch);
        const std::string chain = parts_chain(split_parts(q, pl));
        bool dup = false;
        for (const std::string &x : seen) dup = dup || x == chain;
        if (dup) continue;
        seen.push_back(chain);
        float ms = 1e30f;
        for (int rep = 0; rep < 4 && st == TC_OK && e == hipSuccess; ++rep) {
            std::string name;
            if (rep) e = hipEventRecord(ev[0], s->stream);
            if (e != hipSuccess) break;
            st = enqueue_call(ctx, s, q, pl, A, B, scratch, epi, &name, err);
            if (st != TC_OK) break;
            if (rep) {
                float t = 0.f;
                if ((e = hipEventRecord(ev[1], s->stream)) != hipSuccess) break;
                if ((e = hipEventSynchronize(ev[1])) != hipSuccess) break;
                if ((e = hipEventElapsedTime(&t, ev[0], ev[1])) != hipSuccess) break;
                if (t < ms) ms = t;
            }
        }
        if (st == TC_OK && e == hipSuccess && ms < best_ms) {
            best_ms = ms;
            *best = ch;
        }
    }
    if (e == hipSuccess && st == TC_OK) e = hipStreamSynchronize(s->stream);
    for (hipEvent_t x : ev)
        if (x) (void)hipEventDestroy(x);
    if (scratch) (void)hipFree(scratch);
    if (st != TC_OK) return st;
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(err, TC_ERR_DEVICE, "autotuning: %s", hipGetErrorString(e));
    }
    return TC_OK;
}

// Validate, plan and enqueue one (batched) GEMM on stream s.  noalloc: the
// allocation-free form -- the workspace is the static scratch array of the
// current device (a plan that needs more is refused before anything is
// enqueued), no autotuning, no allocation of any kind.
tc_status_t run(tc_context *ctx, const tc_gemm_batched_desc *bd, const void *A, const void *B,
                void *C, tc_stream *s, bool sync, const tc_epilogue *ep = nullptr,
                bool noalloc = false) {
    if (!ctx) return TC_ERR_INVALID_ARGUMENT;
    const KnobScope knobs;
    ctx->last_error.clear();
    std::string *err = &ctx->last_error;
    if (!A || !B || !C) return fail(err, TC_ERR_INVALID_ARGUMENT, "A, B and C must be non-NULL");
    Problem p;
    tc_status_t st = validate(bd, &p, err, ep && ep->col_scale);
    if (st != TC_OK) return st;
    Epilogue epi;
    if (ep && (st = validate_epilogue(p, ep, C, &epi, err)) != TC_OK) return st;
    if (ranges_overlap(C, p.c_total, A, p.a_total) || ranges_overlap(C, p.c_total, B, p.b_total))
        return fail(err, TC_ERR_ALIASING, "C overlaps A or B");

    st = bind_device(ctx);
    if (st != TC_OK) return st;
    if ((st = check_allocation("A", A, p.a_total, err)) != TC_OK) return st;
    if ((st = check_allocation("B", B, p.b_total, err)) != TC_OK) return st;
    if ((st = check_allocation("C", C, p.c_total, err)) != TC_OK) return st;
    if (epi.bias && (st = check_allocation("bias", epi.bias, epilogue_vec_bytes(p, epi, 0), err)) != TC_OK)
        return st;
    if (epi.scale &&
        (st = check_allocation("col_scale", epi.scale, epilogue_vec_bytes(p, epi, 1), err)) != TC_OK)
        return st;

    if (!s) {
        if (!ctx->internal && (st = create_stream(ctx, &ctx->internal, nullptr)) != TC_OK) return st;
        s = ctx->internal;
    }
    Plan pl;
    if (noalloc) {
        make_plan(p, &pl);
        StripBt sb;
        const int64_t need = call_workspace(p, pl, A, B, &sb);
        void *fixed = nullptr;
        if (need > 0) {
            if (need > kStaticScratchBytes)
                return fail(err, TC_ERR_OUT_OF_MEMORY,
                            "this call needs %lld bytes of scratch (split-K partials and packed "
                            "operands); the allocation-free entry point has %lld",
                            (long long)need, (long long)kStaticScratchBytes);
            const hipError_t e = tcg_static_scratch(ctx->device, &fixed);
            if (e != hipSuccess) {
                (void)hipGetLastError();
                return fail(err, TC_ERR_DEVICE, "static scratch address: %s", hipGetErrorString(e));
            }
        }
        std::string name;
        if ((st = enqueue_call(ctx, s, p, pl, A, B, C, Epilogue{}, &name, err,
                               need > 0 ? fixed : nullptr)) != TC_OK)
            return st;
        ctx->last_kernel = name;
        return TC_OK;
    }
    if (ctx->autotune && p.alpha != 0.0f) {
        // first call of this problem: measure the candidates, then keep the
        // fastest for every later call
        const std::string key = tune_key(p, epi, A, B);
        auto it = ctx->tuned.find(key);
        if (it == ctx->tuned.end()) {
            Choice best;
            if ((st = autotune(ctx, s, p, A, B, epi, &best, err)) != TC_OK) return st;
            it = ctx->tuned.emplace(key, best).first;
        }
        make_plan(p, &pl, true, &it->second);
    } else {
        make_plan(p, &pl);
    }
    std::string name;
    if ((st = enqueue_call(ctx, s, p, pl, A, B, C, epi, &name, err)) != TC_OK) return st;
    ctx->last_kernel = name;
    if (sync) {
        const hipError_t e = hipStreamSynchronize(s->stream);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(err, TC_ERR_DEVICE, "hipStreamSynchronize: %s", hipGetErrorString(e));
        }
    }
    return TC_OK;
}

tc_gemm_batched_desc single(const tc_gemm_desc *d) {
    tc_gemm_batched_desc bd;
    memset(&bd, 0, sizeof bd);
    if (d) bd.base = *d;
    bd.batch = 1;
    return bd;
}

}  // namespace

extern "C" {

tc_status_t tc_context_create(tc_context **out) {
    if (!out) return TC_ERR_INVALID_ARGUMENT;
    *out = new (std::nothrow) tc_context();
    if (!*out) return TC_ERR_OUT_OF_MEMORY;
    const char *env = getenv("TCGEMM_AUTOTUNE");
    (*out)->autotune = env && atoi(env) != 0;
    return TC_OK;
}

void tc_context_destroy(tc_context *ctx) {
    if (!ctx) return;
    if (ctx->internal) tc_stream_destroy(ctx->internal);
    delete ctx;
}

tc_status_t tc_stream_create(tc_context *ctx, tc_stream **out) {
    if (!ctx || !out) return TC_ERR_INVALID_ARGUMENT;
    tc_status_t st = bind_device(ctx);
    if (st != TC_OK) return st;
    return create_stream(ctx, out, nullptr);
}

tc_status_t tc_stream_wrap(tc_context *ctx, void *hip_stream, tc_stream **out) {
    if (!ctx || !out) return TC_ERR_INVALID_ARGUMENT;
    tc_status_t st = bind_device(ctx);
    if (st != TC_OK) return st;
    tc_stream *s = new (std::nothrow) tc_stream();
    if (!s) return TC_ERR_OUT_OF_MEMORY;
    s->ctx = ctx;
    s->stream = static_cast<hipStream_t>(hip_stream);   // NULL: the default stream
    s->owned = false;
    *out = s;
    return TC_OK;
}

tc_status_t tc_stream_sync(tc_stream *s) {
    if (!s) return TC_ERR_INVALID_ARGUMENT;
    hipError_t e = hipStreamSynchronize(s->stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        if (s->ctx) s->ctx->last_error = std::string("hipStreamSynchronize: ") + hipGetErrorString(e);
        return TC_ERR_DEVICE;
    }
    return TC_OK;
}

void tc_stream_destroy(tc_stream *s) {
    if (!s) return;
    if (s->ws) {
        (void)hipStreamSynchronize(s->stream);
        (void)hipFree(s->ws);
    }
    if (s->owned && s->stream) (void)hipStreamDestroy(s->stream);
    delete s;
}

tc_status_t tc_gemm(tc_context *ctx, const tc_gemm_desc *d, const void *A, const void *B, void *C) {
    if (!d) {
        if (ctx) ctx->last_error = "descriptor is NULL";
        return TC_ERR_INVALID_ARGUMENT;
    }
    tc_gemm_batched_desc bd = single(d);
    return run(ctx, &bd, A, B, C, nullptr, true);
}

tc_status_t tc_gemm_async(tc_context *ctx, const tc_gemm_desc *d, const void *A, const void *B,
                          void *C, tc_stream *s) {
    if (!d || !s) {
        if (ctx) ctx->last_error = !d ? "descriptor is NULL" : "stream is NULL";
        return TC_ERR_INVALID_ARGUMENT;
    }
    tc_gemm_batched_desc bd = single(d);
    return run(ctx, &bd, A, B, C, s, false);
}

tc_status_t tc_gemm_batched(tc_context *ctx, const tc_gemm_batched_desc *bd, const void *A,
                            const void *B, void *C) {
    return run(ctx, bd, A, B, C, nullptr, true);
}

tc_status_t tc_gemm_batched_async(tc_context *ctx, const tc_gemm_batched_desc *bd, const void *A,
                                  const void *B, void *C, tc_stream *s) {
    if (!s) {
        if (ctx) ctx->last_error = "stream is NULL";
        return TC_ERR_INVALID_ARGUMENT;
    }
    return run(ctx, bd, A, B, C, s, false);
}

tc_status_t tc_gemm_batched_async_noalloc(tc_context *ctx, const tc_gemm_batched_desc *bd,
                                          const void *A, const void *B, void *C, tc_stream *s) {
    if (!s) {
        if (ctx) ctx->last_error = "stream is NULL";
        return TC_ERR_INVALID_ARGUMENT;
    }
    return run(ctx, bd, A, B, C, s, false, nullptr, true);
}

tc_status_t tc_gemm_epilogue(tc_context *ctx, const tc_gemm_batched_desc *bd, const tc_epilogue *ep,
                             const void *A, const void *B, void *C) {
    if (!ep) {
        if (ctx) ctx->last_error = "epilogue is NULL";
        return TC_ERR_INVALID_ARGUMENT;
    }
    return run(ctx, bd, A, B, C, nullptr, true, ep);
}

tc_status_t tc_gemm_epilogue_async(tc_context *ctx, const tc_gemm_batched_desc *bd,
                                   const tc_epilogue *ep, const void *A, const void *B, void *C,
                                   tc_stream *s) {
    if (!ep || !s) {
        if (ctx) ctx->last_error = !ep ? "epilogue is NULL" : "stream is NULL";
        return TC_ERR_INVALID_ARGUMENT;
    }
    return run(ctx, bd, A, B, C, s, false, ep);
}

tc_status_t tc_set_autotune(tc_context *ctx, int enable) {
    if (!ctx) return TC_ERR_INVALID_ARGUMENT;
    ctx->autotune = enable != 0;
    return TC_OK;
}

int64_t tc_autotune_entries(const tc_context *ctx) { return ctx ? (int64_t)ctx->tuned.size() : 0; }

tc_status_t tc_gemm_plan(tc_context *ctx, const tc_gemm_batched_desc *bd, tc_plan_info *info) {
    const KnobScope knobs;
    std::string *err = ctx ? &ctx->last_error : &g_plan_error;
    err->clear();
    Problem p;
    tc_status_t st = validate(bd, &p, err);
    if (st != TC_OK) return st;
    Plan pl;
    make_plan(p, &pl);
    fill_info(p, pl, info);
    return TC_OK;
}

const char *tc_last_kernel(const tc_context *ctx) { return ctx ? ctx->last_kernel.c_str() : ""; }

uint64_t tc_dispatch_count(const tc_context *ctx) { return ctx ? ctx->dispatches : 0; }

tc_status_t tc_time_next_gemm(tc_context *ctx, void *start_event, void *end_event) {
    if (!ctx || (!start_event) != (!end_event)) return TC_ERR_INVALID_ARGUMENT;
    ctx->time_ev[0] = static_cast<hipEvent_t>(start_event);
    ctx->time_ev[1] = static_cast<hipEvent_t>(end_event);
    return TC_OK;
}

const char *tc_status_string(tc_status_t status) {
    switch (status) {
    case TC_OK: return "TC_OK";
    case TC_ERR_INVALID_ARGUMENT: return "TC_ERR_INVALID_ARGUMENT";
    case TC_ERR_UNSUPPORTED: return "TC_ERR_UNSUPPORTED";
    case TC_ERR_OVERFLOW: return "TC_ERR_OVERFLOW";
    case TC_ERR_ALIASING: return "TC_ERR_ALIASING";
    case TC_ERR_OUT_OF_MEMORY: return "TC_ERR_OUT_OF_MEMORY";
    case TC_ERR_DEVICE: return "TC_ERR_DEVICE";
    default: return "TC_ERR_UNKNOWN";
    }
}

const char *tc_last_error(const tc_context *ctx) {
    return ctx ? ctx->last_error.c_str() : g_plan_error.c_str();
}

tc_status_t tc_tile_of_workgroup(int32_t tiles_m, int32_t tiles_n, int32_t groups, int32_t band,
                                 int64_t wg, int32_t *tm, int32_t *tn, int32_t *g) {
    if (tiles_m < 1 || tiles_n < 1 || groups < 1 || !tm || !tn || !g) return TC_ERR_INVALID_ARGUMENT;
    const int64_t n_wg = (int64_t)tiles_m * tiles_n * groups;
    if (wg < 0 || wg >= n_wg) return TC_ERR_INVALID_ARGUMENT;
    tile_of_workgroup(tiles_m, tiles_n, band, wg, n_wg, tm, tn, g);
    return TC_OK;
}

const char *tc_version(void) { return "tcgemm 0.1.0 (gfx950)"; }

}  // extern "C"
