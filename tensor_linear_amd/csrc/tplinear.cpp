// Host side of libtplinear: argument checks, the placement -> view map and
// the choice of kernel for each shard GEMM.  Declarations and the meaning of
// every argument are in include/tplinear.h.
#include "tplinear.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "kernels.h"

namespace {

using namespace tpl;

constexpr size_t WS_ALIGN = 256;

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline bool valid_dtype(int32_t d) { return d == TP_F32 || d == TP_BF16; }

inline tp_status hip_status(hipError_t e) { return e == hipSuccess ? TP_OK : TP_ERR_HIP; }

// Largest element (or byte) count the library accepts for one buffer: every
// offset and size it derives then fits in int64 / size_t without wrapping.
constexpr int64_t MAX_EXTENT = (int64_t)1 << 60;

// a * b * c <= MAX_EXTENT for non-negative a, b, c, without overflow.
inline bool extent_ok(int64_t a, int64_t b, int64_t c = 1) {
    int64_t ab, abc;
    return !__builtin_mul_overflow(a, b, &ab) && !__builtin_mul_overflow(ab, c, &abc) &&
           abc <= MAX_EXTENT;
}

// Common size checks of the two Linear entry points.
tp_status check_gemm_shape(int64_t M, int64_t N, int64_t K, int32_t P, int64_t ldx,
                           int64_t ldw) {
    if (M < 0 || N < 0 || K < 0) return TP_ERR_SHAPE;
    if (P < 1 || P > TP_MAX_SHARDS) return TP_ERR_SHAPE;
    if (ldx < K || ldw < K || ldx < 1 || ldw < 1) return TP_ERR_SHAPE;
    if (!extent_ok(M, ldx) || !extent_ok(N, ldw)) return TP_ERR_SHAPE;
    return TP_OK;
}

// A reduce-scatter's slice stride: 0 (the slices are the row blocks of Y)
// or at least the extent of one slice, (rows - 1) * ldy + N elements, so that
// no two slices share an element (shared elements would be written by two
// workgroups in no fixed order).
inline bool slice_stride_ok(int64_t stride, int64_t rows, int64_t N, int64_t ldy) {
    if (stride == 0 || rows == 0 || N == 0) return true;
    return stride >= (rows - 1) * ldy + N;
}

// Element distance between consecutive shard views of a placement over a
// [rows, cols] tensor with row stride ld.  The launch path addresses shard i
// at base + i * stride, so the stride is read off tp_shard_layout's own views
// (and checked to be uniform): the views the kernels touch are exactly the
// ones the layout entry point reports.  -1 if the layout rejects the shape.
int64_t view_stride(int64_t rows, int64_t cols, int64_t ld, int32_t kind, int32_t dim,
                    int32_t P) {
    tp_view v[TP_MAX_SHARDS];
    if (tp_shard_layout(rows, cols, ld, tp_placement{kind, dim}, P, v) != TP_OK) return -1;
    const int64_t stride = P > 1 ? v[1].elem_offset - v[0].elem_offset : 0;
    for (int32_t i = 0; i < P; ++i)
        if (v[i].elem_offset != i * stride) return -1;
    return stride;
}

// Whether a bf16 shard GEMM takes the skinny kernel: up to 32 tokens, and up
// to 48 where the tile kernels do no better -- a shard K above 4096 (the
// skinny kernel's longer runs per workgroup pay off) or so few 128-row tiles
// over all P shards that they would fill at most half of the CUs.  Same box,
// 8 shards, us after a read-only flush / warm, 33-48 tokens, skinny vs tiles:
// column 4096 -> 28672 66.4-68.3 / 56.1-57.4 vs 59.4-62.3 / 38.6-39.2, 8192
// -> 28672 106.0-109.9 / 105.5-108.5 vs 115.4-119.6 / 114.8-118.5; row
// partials + fold 14336 -> 4096 41.2-42.7 / 37.2-37.3 vs 31.2-31.4 / 26.4-26.6,
// 28672 -> 8192 118.2-136.7 / 113.3-117.5 vs 100.9-114.1 / 101.0-104.0.  The
// tile count uses all shards' columns together, so a column layer takes the
// same kernel family whatever P is (and the same bits).
bool skinny_takes(const GemmArgs &g, const GemmExtra *ex) {
    if (!gemm_skinny_supported(g, ex)) return false;
    if (g.M <= 32 || g.K > 4096 || !gemm_tile_supported(g, ex)) return true;
    const int64_t cols = ex && ex->act == ACT_SWIGLU ? 64 : 128;   // outputs per 128 W rows
    const int64_t t128 = ((g.M + 127) / 128) * ((g.N * g.P + cols - 1) / cols);
    return 2 * t128 <= device_cu_count();
}

// Run one grouped shard GEMM with the best kernel that takes it.
// Decode-shaped bf16 problems (up to 32 or 48 tokens, see skinny_takes)
// stream W with the skinny kernel;
// aligned bf16 problems use the 256x256 MFMA tile kernel, or its narrow
// forms (128x128, or 256x128 with two waves per SIMD) when the 256x256
// tiles would fill at most half of the CUs; everything else (fp32, odd K,
// unaligned views) uses the generic kernel.
hipError_t run_gemm(const GemmArgs &g, int32_t dtype, int out_type, const GemmExtra *ex,
                    hipStream_t s) {
    if (dtype == TP_BF16) {
        if (skinny_takes(g, ex)) return launch_gemm_skinny(g, out_type, nullptr, ex, s);
        if (gemm_tile_supported(g, ex)) {
            // Few 256 x 256 tiles (short prompts): the narrow kernel.  Its
            // 256 x 128 form against the 256 x 256 tiles, same-box times, 8
            // shards, after a 1 GiB write / warm: M = 128, 4096 -> 28672:
            // 93.9 / 53.5 vs 106.3 / 78.0 us; M = 128, 8192 -> 10240: 123.5 /
            // 82.9 vs 168.9 / 133.3 us; M = 256, 4096 -> 28672: 114.7 / 53.1
            // vs 123.7 / 74.9 us (its 128 x 128 form is faster again where
            // those tiles fit in one pass).
            const bool sw = ex && ex->act == ACT_SWIGLU;
            const bool plain = !ex || (ex->x_rows == 0 && (out_type == OUT_BF16 || (!ex->bias && !sw)));
            // the tile kernel's tiles: 256 W rows, 128 outputs with the gated unit
            const int64_t t256 = ((g.M + 255) / 256) * ((g.N + (sw ? 127 : 255)) / (sw ? 128 : 256)) * g.P;
            if (plain && 2 * t256 <= device_cu_count()) return launch_gemm_narrow(g, out_type, ex, s);
            return launch_gemm_tile(g, out_type, ex, s);
        }
        return launch_gemm_generic(g, IN_BF16, out_type, ex, s);
    }
    return launch_gemm_generic(g, IN_F32, out_type, ex, s);
}

inline size_t dtype_bytes(int32_t d) { return d == TP_BF16 ? 2 : 4; }

// Fill the slice table of r from a host array (nullptr: the strided layout).
void set_out_slices(ReduceArgs &r, void *const *y_slices, int32_t P) {
    r.use_slices = y_slices ? 1 : 0;
    for (int j = 0; j < MAX_SLICES; ++j) r.y_slice[j] = (y_slices && j < P) ? y_slices[j] : nullptr;
}

// Bytes of P fp32 [M, N] partials, rounded up; 0 when the count would pass
// MAX_EXTENT (the callers reject those sizes).
size_t partials_bytes(int64_t M, int64_t N, int32_t P) {
    if (!extent_ok(M, N, (int64_t)P * (int64_t)sizeof(float))) return 0;
    return round_up((size_t)P * (size_t)M * (size_t)N * sizeof(float), WS_ALIGN);
}

}  // namespace

extern "C" {

int32_t tp_version(void) { return 100; }

const char *tp_status_str(int32_t s) {
    switch (s) {
        case TP_OK: return "TP_OK";
        case TP_ERR_NULL: return "TP_ERR_NULL: a required pointer is NULL";
        case TP_ERR_SHAPE: return "TP_ERR_SHAPE: invalid size, leading dimension or shard count";
        case TP_ERR_INDIVISIBLE: return "TP_ERR_INDIVISIBLE: the split dimension is not a multiple of P";
        case TP_ERR_PLACEMENT: return "TP_ERR_PLACEMENT: invalid placement kind or dim";
        case TP_ERR_DTYPE: return "TP_ERR_DTYPE: invalid dtype";
        case TP_ERR_MODE: return "TP_ERR_MODE: invalid mode";
        case TP_ERR_WORKSPACE: return "TP_ERR_WORKSPACE: workspace missing or too small";
        case TP_ERR_HIP: return "TP_ERR_HIP: a HIP call or kernel launch failed";
        default: return "unknown tp_status";
    }
}

tp_status tp_shard_layout(int64_t rows, int64_t cols, int64_t ld, tp_placement pl, int32_t P,
                          tp_view *views) {
    if (!views) return TP_ERR_NULL;
    if (rows < 0 || cols < 0 || ld < cols || P < 1 || P > TP_MAX_SHARDS) return TP_ERR_SHAPE;
    if (!extent_ok(rows, ld, pl.kind == TP_PARTIAL ? P : 1)) return TP_ERR_SHAPE;
    if (pl.kind == TP_SHARD) {
        int d = pl.dim;
        if (d < 0) d += 2;
        if (d != 0 && d != 1) return TP_ERR_PLACEMENT;
        const int64_t L = d == 0 ? rows : cols;
        if (L % P != 0) return TP_ERR_INDIVISIBLE;
        const int64_t s = L / P;
        for (int32_t i = 0; i < P; ++i) {
            tp_view v;
            v.ld = ld;
            if (d == 0) {
                v.row0 = i * s; v.col0 = 0; v.rows = s; v.cols = cols;
            } else {
                v.row0 = 0; v.col0 = i * s; v.rows = rows; v.cols = s;
            }
            v.elem_offset = v.row0 * ld + v.col0;
            views[i] = v;
        }
        return TP_OK;
    }
    if (pl.kind == TP_REPLICATE || pl.kind == TP_PARTIAL) {
        for (int32_t i = 0; i < P; ++i) {
            tp_view v;
            v.ld = ld; v.rows = rows; v.cols = cols; v.row0 = 0; v.col0 = 0;
            v.elem_offset = pl.kind == TP_PARTIAL ? (int64_t)i * rows * ld : 0;
            views[i] = v;
        }
        return TP_OK;
    }
    return TP_ERR_PLACEMENT;
}

tp_status tp_linear_column_ex(const void *X, const void *const *x_slices, int64_t ldx,
                              const void *W, int64_t ldw, const void *bias, void *Y, int64_t ldy,
                              int32_t y_mode, int32_t act, int64_t M, int64_t N, int64_t K,
                              int32_t P, int32_t dtype, void *stream) {
    tp_status st = check_gemm_shape(M, N, K, P, ldx, ldw);
    if (st != TP_OK) return st;
    if (!valid_dtype(dtype)) return TP_ERR_DTYPE;
    if (y_mode != TP_Y_CONCAT && y_mode != TP_Y_SHARDS) return TP_ERR_MODE;
    if (act != TP_ACT_NONE && act != TP_ACT_SWIGLU) return TP_ERR_MODE;
    if (N % P != 0) return TP_ERR_INDIVISIBLE;
    const int64_t Ns = N / P;                                   // W rows per shard
    const bool swiglu = act == TP_ACT_SWIGLU;
    if (swiglu && Ns % 2 != 0) return TP_ERR_INDIVISIBLE;
    const int64_t On = swiglu ? Ns / 2 : Ns;                     // outputs per shard
    if (x_slices && M % P != 0) return TP_ERR_INDIVISIBLE;
    if (y_mode == TP_Y_CONCAT ? ldy < On * P : ldy < On) return TP_ERR_SHAPE;
    if (ldy < 1) return TP_ERR_SHAPE;
    if (!extent_ok(M, ldy, y_mode == TP_Y_SHARDS ? P : 1)) return TP_ERR_SHAPE;
    if (M == 0 || N == 0) return TP_OK;
    if (!Y) return TP_ERR_NULL;
    if (K > 0) {
        if (!W || (X != nullptr) == (x_slices != nullptr)) return TP_ERR_NULL;
        if (x_slices)
            for (int32_t j = 0; j < P; ++j)
                if (!x_slices[j]) return TP_ERR_NULL;
    }

    // Shard strides from the placements: W [N, K] Shard(0) (row blocks); Y
    // concatenated = [M, P*On] Shard(1) (column blocks), or P shard buffers
    // stacked = [P*M, On] Shard(0); the bias [N] Shard(0).  X is Replicate.
    const int64_t w_stride = view_stride(N, K, ldw, TP_SHARD, 0, P);
    const int64_t y_stride = y_mode == TP_Y_CONCAT ? view_stride(M, P * On, ldy, TP_SHARD, 1, P)
                                                   : view_stride(P * M, On, ldy, TP_SHARD, 0, P);
    const int64_t b_stride = view_stride(N, 1, 1, TP_SHARD, 0, P);
    if (w_stride < 0 || y_stride < 0 || b_stride < 0) return TP_ERR_SHAPE;
    GemmArgs g;
    g.A = X; g.lda = ldx; g.a_shard = 0;
    g.B = W; g.ldb = ldw; g.b_shard = w_stride;
    g.C = Y; g.ldc = ldy; g.c_shard = y_stride;
    g.M = M; g.N = On; g.K = K; g.P = P;
    GemmExtra ex{};
    ex.bias = bias; ex.bias_shard = b_stride;
    ex.act = swiglu ? ACT_SWIGLU : ACT_NONE; ex.up_off = swiglu ? On : 0;
    ex.x_rows = 0;
    if (x_slices && K > 0) {
        ex.x_rows = M / P;
        for (int32_t j = 0; j < P; ++j) ex.x_slice[j] = x_slices[j];
        g.A = x_slices[0];
    }
    const bool plain = !bias && !swiglu && ex.x_rows == 0;
    const int out = dtype == TP_BF16 ? OUT_BF16 : OUT_F32;
    return hip_status(run_gemm(g, dtype, out, plain ? nullptr : &ex, (hipStream_t)stream));
}

tp_status tp_linear_column(const void *X, int64_t ldx, const void *W, int64_t ldw, void *Y,
                           int64_t ldy, int32_t y_mode, int64_t M, int64_t N, int64_t K,
                           int32_t P, int32_t dtype, void *stream) {
    return tp_linear_column_ex(X, nullptr, ldx, W, ldw, nullptr, Y, ldy, y_mode, TP_ACT_NONE,
                               M, N, K, P, dtype, stream);
}

size_t tp_row_workspace_bytes(int32_t mode, int64_t M, int64_t N, int32_t P) {
    if (M < 0 || N < 0 || P < 1 || P > TP_MAX_SHARDS) return 0;
    switch (mode) {
        case TP_ROW_SUM:
        case TP_ROW_FUSED:
        case TP_ROW_SCATTER: return partials_bytes(M, N, P);
        default: return 0;
    }
}

}  // extern "C"

namespace tpl {

tp_status row_args_status(const void *X, int64_t ldx, const void *W, int64_t ldw,
                          const void *bias, void *Y, void *const *y_slices, int64_t ldy,
                          int64_t y_slice_stride, int32_t mode, int64_t M, int64_t N, int64_t K,
                          int32_t P, int32_t dtype) {
    tp_status st = check_gemm_shape(M, N, K, P, ldx, ldw);
    if (st != TP_OK) return st;
    if (!valid_dtype(dtype)) return TP_ERR_DTYPE;
    if (mode < TP_ROW_PARTIAL || mode > TP_ROW_SCATTER) return TP_ERR_MODE;
    if (bias && mode == TP_ROW_PARTIAL) return TP_ERR_MODE;
    if (y_slices && mode != TP_ROW_SCATTER) return TP_ERR_MODE;
    if (K % P != 0) return TP_ERR_INDIVISIBLE;
    if (mode == TP_ROW_SCATTER && M % P != 0) return TP_ERR_INDIVISIBLE;
    if (ldy < N || ldy < 1) return TP_ERR_SHAPE;
    if (y_slice_stride < 0) return TP_ERR_SHAPE;
    if (!extent_ok(M, ldy, mode == TP_ROW_PARTIAL ? P : 1) ||
        !extent_ok(M, N, (int64_t)P * (int64_t)sizeof(float)) || !extent_ok(P, y_slice_stride))
        return TP_ERR_SHAPE;
    if (mode == TP_ROW_SCATTER && !y_slices && !slice_stride_ok(y_slice_stride, M / P, N, ldy))
        return TP_ERR_SHAPE;
    if (M == 0 || N == 0) return TP_OK;
    if (y_slices) {
        for (int32_t j = 0; j < P; ++j)
            if (!y_slices[j]) return TP_ERR_NULL;
    } else if (!Y) {
        return TP_ERR_NULL;
    }
    if (K > 0 && (!X || !W)) return TP_ERR_NULL;
    return TP_OK;
}

// TPLINEAR_ROW_FOLD=gemm: TP_ROW_FUSED and TP_ROW_SCATTER fold inside the
// GEMM wherever a kernel takes the shape, not only where that measured
// faster (the result is the same, bit for bit).
bool row_fold_in_gemm_forced() {
    const char *e = getenv("TPLINEAR_ROW_FOLD");
    return e && strcmp(e, "gemm") == 0;
}

// The two ways to fold give the same bits, so the choice is by speed alone.
// Same-box times, 8 shards, bf16, us after a read-only 1 GiB flush (warm in
// brackets), partials + fold vs the fold inside the GEMM:
// Decode (M <= 48, the skinny kernel): above 16 tokens the fused form loses
// everywhere (M = 32: 14336 -> 4096 33.5 vs 83.1, 8192 -> 8192 38.2 vs 51.8,
// 28672 -> 8192 100.2 vs 179.7; M = 48: 41.9 vs 93.1, 49.6 vs 59.7, 122.7
// vs 177.7).  Up to 16 tokens it wins where its grid fills the CUs
// with 32 output columns per workgroup and the shard's K is long (28672 ->
// 8192, M = 16: 91.3 vs 95.5; 57344 -> 8192: 155.8 vs 178.3), or where 16
// columns per workgroup fill them and the layer is small (4096 -> 4096:
// 13.8 vs 17.1; 8192 -> 4096: 21.2 vs 22.4), and loses otherwise (8192 ->
// 8192, K/P = 1024: 34.1-35.1 vs 31.5-33.8; 14336 -> 4096, K/P = 1792:
// 31.8-32.2 vs 29.4-33.0 [26.0-26.4 vs 31.8-32.0]).
bool skinny_fold_faster(int64_t M, int64_t N, int64_t Ks) {
    if (M > 16) return false;
    return N >= 32 * (int64_t)device_cu_count() ? Ks >= 2048 : Ks <= 1024;
}

// Prefill (M > 64, the 256 x 128 fold-in-registers kernel): it walks the P
// shards of each output tile in turn, so it needs enough tiles; the shorter
// the shard's K, the fewer.  Crossovers (tiles: fused vs unfused): K/P = 512,
// 4096 -> 4096: 64 tiles 60.5 vs 41.8, 96 59.0 vs 61.0, 128 59.5 vs 75.7;
// K/P = 1024, 8192 -> 8192: 128 110.3 vs 98.1 [91.0 vs 93.5], 192 111.6 vs
// 143.7; 8192 -> 4096: 128 110.2 vs 96.4, 192 109.5 vs 141.1; K/P = 1792,
// 14336 -> 4096: 128 193.5 vs 131.6, 192 197.1 vs 189.9 [157.9 vs 178.7],
// 256 201.7 vs 242.0; K/P = 2048, 16384 -> 8192: 192 241.3 vs 212.1, 256
// 228.9 vs 282.3.  So: tiles >= CUs * min(1, (K/P + 512) / 2048).
bool rowfold_faster(int64_t M, int64_t N, int64_t Ks) {
    if (M <= 64) return false;   // its 256-row tile would be three-quarters empty
    const int64_t tiles = ((M + 255) / 256) * ((N + 127) / 128);
    return tiles * 2048 >= (int64_t)device_cu_count() * std::min<int64_t>(2048, Ks + 512);
}

// The kernels tp_linear_row_ex runs for a call that passed
// row_args_status (non-empty), and whether they use the workspace.
tp_status plan_row(const void *X, int64_t ldx, const void *W, int64_t ldw, const void *bias,
                   void *Y, void *const *y_slices, int64_t ldy, int64_t y_slice_stride,
                   int32_t mode, int64_t M, int64_t N, int64_t K, int32_t P, int32_t dtype,
                   size_t ws_cap, RowPlan &p) {
    const int64_t Ks = K / P;
    // Shard strides from the placements: X [M, K] and W [N, K] Shard(1)
    // (column blocks); the partials Partial() (P [M, N] buffers back to
    // back, row stride ldy in Y or N in the workspace); the reduce-scatter's
    // slices Shard(0) of Y (row blocks) unless a slice stride is given.
    const int64_t x_stride = view_stride(M, K, ldx, TP_SHARD, 1, P);
    const int64_t w_stride = view_stride(N, K, ldw, TP_SHARD, 1, P);
    if (x_stride < 0 || w_stride < 0) return TP_ERR_SHAPE;
    GemmArgs &g = p.g;
    g.A = X; g.lda = ldx; g.a_shard = x_stride;
    g.B = W; g.ldb = ldw; g.b_shard = w_stride;
    g.M = M; g.N = N; g.K = Ks; g.P = P;
    p.dtype = dtype;
    p.out = dtype == TP_BF16 ? OUT_BF16 : OUT_F32;
    p.ex = GemmExtra{};
    p.ex.bias = bias;

    if (mode == TP_ROW_PARTIAL) {
        const int64_t p_stride = view_stride(M, N, ldy, TP_PARTIAL, 0, P);
        if (p_stride < 0) return TP_ERR_SHAPE;
        g.C = Y; g.ldc = ldy; g.c_shard = p_stride;
        p.path = RowPlan::PARTIAL;
        return TP_OK;
    }

    const int64_t p_stride = view_stride(M, N, N, TP_PARTIAL, 0, P);
    if (p_stride < 0) return TP_ERR_SHAPE;
    g.C = nullptr; g.ldc = N; g.c_shard = p_stride;   // the workspace, set by run_row

    // Fold inside the GEMM where a kernel takes the shape and that is the
    // faster way, or the override asks for it, or the partials would not fit.
    const bool any_fold = row_fold_in_gemm_forced() || partials_bytes(M, N, P) > ws_cap;
    if (mode == TP_ROW_FUSED && dtype == TP_BF16 && skinny_takes(g, nullptr) &&
        (any_fold || skinny_fold_faster(M, N, Ks))) {
        p.f.Y = Y; p.f.ldy = ldy; p.f.out_type = p.out;
        p.path = RowPlan::SKINNY_FOLD;
        return TP_OK;
    }

    ReduceArgs &r = p.r;
    r.partials = nullptr; r.shard_stride = p_stride; r.ldp = N;
    r.Y = Y; r.ldy = ldy; r.M = M; r.N = N; r.P = P;
    r.bias = bias;
    set_out_slices(r, y_slices, P);
    if (mode == TP_ROW_SCATTER) {
        const int64_t s_stride = view_stride(M, N, ldy, TP_SHARD, 0, P);
        if (s_stride < 0) return TP_ERR_SHAPE;
        r.slice_rows = M / P;
        r.slice_stride = y_slice_stride ? y_slice_stride : s_stride;
    } else {
        r.slice_rows = M;
        r.slice_stride = 0;
    }
    // Prefill shapes: the fold in registers (256x128 tiles walking the P
    // shards) saves writing and re-reading the P fp32 partials, but its
    // narrower tile moves 1.5x the operand bytes per flop, so it wins only
    // while the shard's K is short enough -- the shorter, the smaller the
    // output.  Fused / unfused time measured on one box with cold caches (a
    // 1 GiB write before each call), P = 8: M x N = 2048 x 4096: K/P = 1024
    // 0.73, 2048 0.93; 4096 x 4096: 1024 0.74, 1792 0.86, 2560 0.93, 3584
    // 0.97, 5120 1.03; 8192 x 8192: 1024 0.64, 1280 0.71, 1792 0.75, 3584
    // 0.93, 7168 1.04; 16384 x 8192: 3584 0.92, 7168 1.02.
    const bool fold_in_gemm = Ks <= 2048 || (Ks <= 3584 && M * N >= (int64_t)4096 * 4096);
    if ((mode == TP_ROW_FUSED || mode == TP_ROW_SCATTER) && dtype == TP_BF16 && fold_in_gemm &&
        gemm_rowfold_supported(g, r) && (any_fold || rowfold_faster(M, N, Ks))) {
        p.path = RowPlan::ROWFOLD;
        return TP_OK;
    }
    p.path = RowPlan::PARTIALS_AND_FOLD;
    return TP_OK;
}

tp_status run_row(RowPlan &p, float *workspace, hipStream_t s) {
    switch (p.path) {
        case RowPlan::PARTIAL:
            return hip_status(run_gemm(p.g, p.dtype, OUT_F32, nullptr, s));
        case RowPlan::SKINNY_FOLD:
            return hip_status(launch_gemm_skinny(p.g, p.out, &p.f, p.ex.bias ? &p.ex : nullptr, s));
        case RowPlan::ROWFOLD:
            return hip_status(launch_gemm_rowfold(p.g, p.r, s));
        case RowPlan::PARTIALS_AND_FOLD:
        default: {
            if (!workspace) return TP_ERR_WORKSPACE;
            p.g.C = workspace;
            p.r.partials = workspace;
            const hipError_t e = run_gemm(p.g, p.dtype, OUT_F32, nullptr, s);
            if (e != hipSuccess) return TP_ERR_HIP;
            return hip_status(launch_shard_fold(p.r, p.out, s));
        }
    }
}

}  // namespace tpl

extern "C" {

tp_status tp_linear_row_ex(const void *X, int64_t ldx, const void *W, int64_t ldw,
                           const void *bias, void *Y, void *const *y_slices, int64_t ldy,
                           int64_t y_slice_stride, int32_t mode, void *workspace,
                           size_t ws_bytes, int64_t M, int64_t N, int64_t K, int32_t P,
                           int32_t dtype, void *stream) {
    const tp_status st = row_args_status(X, ldx, W, ldw, bias, Y, y_slices, ldy, y_slice_stride,
                                         mode, M, N, K, P, dtype);
    if (st != TP_OK) return st;
    if (M == 0 || N == 0) return TP_OK;
    const size_t need = tp_row_workspace_bytes(mode, M, N, P);
    if (need > 0 && (!workspace || ws_bytes < need || ((uintptr_t)workspace % WS_ALIGN) != 0))
        return TP_ERR_WORKSPACE;
    RowPlan plan;
    const tp_status pst = plan_row(X, ldx, W, ldw, bias, Y, y_slices, ldy, y_slice_stride, mode,
                                   M, N, K, P, dtype, SIZE_MAX, plan);
    if (pst != TP_OK) return pst;
    return run_row(plan, (float *)workspace, (hipStream_t)stream);
}

tp_status tp_linear_row(const void *X, int64_t ldx, const void *W, int64_t ldw, void *Y,
                        int64_t ldy, int64_t y_slice_stride, int32_t mode, void *workspace,
                        size_t ws_bytes, int64_t M, int64_t N, int64_t K, int32_t P,
                        int32_t dtype, void *stream) {
    return tp_linear_row_ex(X, ldx, W, ldw, nullptr, Y, nullptr, ldy, y_slice_stride, mode,
                            workspace, ws_bytes, M, N, K, P, dtype, stream);
}

tp_status tp_shard_reduce_ex(const float *partials, int64_t shard_stride, int64_t ldp,
                             const void *bias, void *Y, void *const *y_slices, int64_t ldy,
                             int64_t y_slice_stride, int32_t scatter, int64_t M, int64_t N,
                             int32_t P, int32_t out_dtype, void *stream) {
    if (M < 0 || N < 0 || P < 1 || P > TP_MAX_SHARDS) return TP_ERR_SHAPE;
    if (ldp < N || ldy < N || ldp < 1 || ldy < 1 || shard_stride < 0 || y_slice_stride < 0)
        return TP_ERR_SHAPE;
    if (!extent_ok(M, ldp) || !extent_ok(M, ldy) || !extent_ok(P, shard_stride) ||
        !extent_ok(P, y_slice_stride))
        return TP_ERR_SHAPE;
    if (!valid_dtype(out_dtype)) return TP_ERR_DTYPE;
    if (scatter != 0 && scatter != 1) return TP_ERR_MODE;
    if (y_slices && !scatter) return TP_ERR_MODE;
    if (scatter && M % P != 0) return TP_ERR_INDIVISIBLE;
    if (scatter && !y_slices && !slice_stride_ok(y_slice_stride, M / P, N, ldy))
        return TP_ERR_SHAPE;
    if (M == 0 || N == 0) return TP_OK;
    if (!partials) return TP_ERR_NULL;
    if (y_slices) {
        for (int32_t j = 0; j < P; ++j)
            if (!y_slices[j]) return TP_ERR_NULL;
    } else if (!Y) {
        return TP_ERR_NULL;
    }
    ReduceArgs r;
    r.partials = partials; r.shard_stride = shard_stride; r.ldp = ldp;
    r.Y = Y; r.ldy = ldy; r.M = M; r.N = N; r.P = P;
    r.bias = bias;
    set_out_slices(r, y_slices, P);
    if (scatter) {
        // the slices: Shard(0) of Y (row blocks) unless a stride is given
        const int64_t s_stride = view_stride(M, N, ldy, TP_SHARD, 0, P);
        if (s_stride < 0) return TP_ERR_SHAPE;
        r.slice_rows = M / P;
        r.slice_stride = y_slice_stride ? y_slice_stride : s_stride;
    } else {
        r.slice_rows = M;
        r.slice_stride = 0;
    }
    return hip_status(launch_shard_fold(r, out_dtype == TP_BF16 ? OUT_BF16 : OUT_F32,
                                        (hipStream_t)stream));
}

tp_status tp_shard_reduce(const float *partials, int64_t shard_stride, int64_t ldp, void *Y,
                          int64_t ldy, int64_t y_slice_stride, int32_t scatter, int64_t M,
                          int64_t N, int32_t P, int32_t out_dtype, void *stream) {
    return tp_shard_reduce_ex(partials, shard_stride, ldp, nullptr, Y, nullptr, ldy,
                              y_slice_stride, scatter, M, N, P, out_dtype, stream);
}

tp_status tp_embedding(const int64_t *ids, int64_t T, const void *E, const void *const *e_shards,
                       int64_t lde, int64_t V, int64_t D, void *Y, int64_t ldy, int32_t y_mode,
                       int32_t P, int32_t dtype, int32_t *bad_flag, void *stream) {
    if (T < 0 || V < 0 || D < 0 || P < 1 || P > TP_MAX_SHARDS) return TP_ERR_SHAPE;
    if (!valid_dtype(dtype)) return TP_ERR_DTYPE;
    if (y_mode != TP_Y_CONCAT && y_mode != TP_Y_SHARDS) return TP_ERR_MODE;
    if (D % P != 0) return TP_ERR_INDIVISIBLE;
    const int64_t Ds = D / P;
    if (E ? lde < D : lde < Ds) return TP_ERR_SHAPE;
    if (lde < 1) return TP_ERR_SHAPE;
    if (y_mode == TP_Y_CONCAT ? ldy < D : ldy < Ds) return TP_ERR_SHAPE;
    if (ldy < 1) return TP_ERR_SHAPE;
    if (!extent_ok(V, lde) || !extent_ok(T, ldy, y_mode == TP_Y_SHARDS ? P : 1))
        return TP_ERR_SHAPE;
    if (T == 0 || D == 0) return TP_OK;
    if (!ids || !Y || (E != nullptr) == (e_shards != nullptr)) return TP_ERR_NULL;
    // Shard strides from the placements: the table [V, D] Shard(1) (column
    // blocks of the embedding dim); the output concatenated = [T, D]
    // Shard(1), or P shard buffers stacked = [P*T, Ds] Shard(0).
    const int64_t e_stride = E ? view_stride(V, D, lde, TP_SHARD, 1, P) : 0;
    const int64_t y_stride = y_mode == TP_Y_CONCAT ? view_stride(T, D, ldy, TP_SHARD, 1, P)
                                                   : view_stride(P * T, Ds, ldy, TP_SHARD, 0, P);
    if (e_stride < 0 || y_stride < 0) return TP_ERR_SHAPE;
    EmbedArgs e;
    e.ids = ids; e.T = T; e.V = V; e.Ds = Ds; e.P = P;
    e.lde = lde; e.Y = Y; e.ldy = ldy;
    e.y_shard = y_stride;
    e.bad = bad_flag;
    const size_t es = dtype_bytes(dtype);
    for (int j = 0; j < MAX_SLICES; ++j) e.e_shard[j] = nullptr;
    for (int32_t i = 0; i < P; ++i) {
        if (e_shards) {
            if (!e_shards[i]) return TP_ERR_NULL;
            e.e_shard[i] = e_shards[i];
        } else {
            e.e_shard[i] = (const char *)E + (size_t)(i * e_stride) * es;
        }
    }
    return hip_status(launch_embedding(e, (int)es, (hipStream_t)stream));
}

tp_status tp_workspace_zero(void *ptr, size_t bytes, void *stream) {
    if (bytes == 0) return TP_OK;
    if (!ptr) return TP_ERR_NULL;
    if (bytes % 4 != 0 || ((uintptr_t)ptr % 4) != 0) return TP_ERR_SHAPE;
    return hip_status(launch_fill_zero(ptr, bytes / 4, (hipStream_t)stream));
}

}  // extern "C"
