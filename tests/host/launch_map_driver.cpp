// Host-only driver: the shard offsets every compute entry point hands to its
// kernels are the views tp_shard_layout reports for the placements of the
// layer ("DTensor API 文档", sections "distribute_tensor" and "放置策略类型":
// Shard(d) gives shard i the i-th equal block of dim d, Replicate() the whole
// tensor, Partial() a full-shape part).  Links the host side of the C ABI
// (tplinear.cpp) against launchers that record their arguments instead of
// launching, calls each entry point in each mode with fake (never
// dereferenced) addresses, and checks base + i * stride of every recorded
// operand against base + views[i].elem_offset.  Built and run by
// tests/test_host_sanitizers.py.
#include <cstdio>
#include <cstdlib>
#include <cstdint>
#include <vector>

#include "tplinear.h"
#include "kernels.h"

namespace {
struct Rec {
    int gemms = 0, folds = 0, embeds = 0;
    tpl::GemmArgs g{};
    tpl::GemmExtra ex{};
    bool has_ex = false;
    tpl::ReduceArgs r{};
    tpl::EmbedArgs e{};
} rec;
}  // namespace

namespace tpl {
// Every GEMM takes the generic kernel (the kernel choice does not change the
// arguments), every fold the fold kernel.
bool gemm_tile_supported(const GemmArgs &, const GemmExtra *) { return false; }
bool gemm_skinny_supported(const GemmArgs &, const GemmExtra *) { return false; }
bool gemm_rowfold_supported(const GemmArgs &, const ReduceArgs &) { return false; }
hipError_t launch_gemm_tile(const GemmArgs &, int, const GemmExtra *, hipStream_t) { std::abort(); }
hipError_t launch_gemm_narrow(const GemmArgs &, int, const GemmExtra *, hipStream_t) { std::abort(); }
hipError_t launch_gemm_skinny(const GemmArgs &, int, const FoldArgs *, const GemmExtra *, hipStream_t) {
    std::abort();
}
hipError_t launch_gemm_rowfold(const GemmArgs &, const ReduceArgs &, hipStream_t) { std::abort(); }
hipError_t launch_gemm_generic(const GemmArgs &g, int, int, const GemmExtra *ex, hipStream_t) {
    ++rec.gemms;
    rec.g = g;
    rec.has_ex = ex != nullptr;
    if (ex) rec.ex = *ex;
    return hipSuccess;
}
hipError_t launch_shard_fold(const ReduceArgs &r, int, hipStream_t) {
    ++rec.folds;
    rec.r = r;
    return hipSuccess;
}
hipError_t launch_embedding(const EmbedArgs &e, int, hipStream_t) {
    ++rec.embeds;
    rec.e = e;
    return hipSuccess;
}
hipError_t launch_fill_zero(void *, size_t, hipStream_t) { std::abort(); }
int device_cu_count() { return 256; }
}  // namespace tpl

static int failures = 0;
#define CHECK(c) do { if (!(c)) { std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); ++failures; } } while (0)

// Views of a placement over [rows, cols] with row stride ld.
static std::vector<tp_view> views(int64_t rows, int64_t cols, int64_t ld, int32_t kind, int32_t dim,
                                  int32_t P) {
    std::vector<tp_view> v(P);
    CHECK(tp_shard_layout(rows, cols, ld, tp_placement{kind, dim}, P, v.data()) == TP_OK);
    return v;
}

// base + i * stride == base + v[i].elem_offset for every shard i.
static void same_offsets(int64_t stride, const std::vector<tp_view> &v, const char *what) {
    for (size_t i = 0; i < v.size(); ++i)
        if ((int64_t)i * stride != v[i].elem_offset) {
            std::fprintf(stderr, "%s: shard %zu at %lld, view at %lld\n", what, i, (long long)(i * stride),
                         (long long)v[i].elem_offset);
            ++failures;
        }
}

static char *const BASE = reinterpret_cast<char *>(0x10000000);

int main() {
    // Shapes with distinct leading dims so that a swapped stride shows.
    struct Shape { int64_t M, N, K; int32_t P; int64_t pad; };
    const Shape shapes[] = {{6, 12, 8, 4, 3}, {16, 24, 48, 8, 5}, {5, 7, 9, 1, 2}, {64, 128, 64, 64, 1}};
    for (const Shape &sh : shapes) {
        const int64_t M = sh.M, N = sh.N, K = sh.K, pad = sh.pad;
        const int32_t P = sh.P;
        const int64_t ldx = K + pad, ldw = K + 2 * pad;
        void *X = BASE, *W = BASE + (1 << 24), *Y = BASE + (2 << 24), *WS = BASE + (3 << 24);
        void *b = BASE + (4 << 24);

        // ---- column: X Replicate, W [N, K] Shard(0), bias Shard(0); Y
        // concatenated [M, N] Shard(1) or P shard buffers stacked [P*M, N/P].
        for (int y_mode : {TP_Y_CONCAT, TP_Y_SHARDS}) {
            const int64_t ldy = (y_mode == TP_Y_CONCAT ? N : N / P) + pad;
            rec = Rec{};
            CHECK(tp_linear_column_ex(X, nullptr, ldx, W, ldw, b, Y, ldy, y_mode, TP_ACT_NONE, M, N, K, P, TP_BF16,
                                      nullptr) == TP_OK);
            CHECK(rec.gemms == 1 && rec.g.A == X && rec.g.B == W && rec.g.C == Y && rec.has_ex);
            same_offsets(rec.g.a_shard, views(M, K, ldx, TP_REPLICATE, 0, P), "column X");
            same_offsets(rec.g.b_shard, views(N, K, ldw, TP_SHARD, 0, P), "column W");
            same_offsets(rec.ex.bias_shard, views(N, 1, 1, TP_SHARD, 0, P), "column bias");
            if (y_mode == TP_Y_CONCAT)
                same_offsets(rec.g.c_shard, views(M, N, ldy, TP_SHARD, 1, P), "column Y concat");
            else
                same_offsets(rec.g.c_shard, views(P * M, N / P, ldy, TP_SHARD, 0, P), "column Y shards");
            CHECK(rec.g.lda == ldx && rec.g.ldb == ldw && rec.g.ldc == ldy);
            CHECK(rec.g.M == M && rec.g.N == N / P && rec.g.K == K && rec.g.P == P);
        }

        // ---- row: X [M, K] and W [N, K] Shard(1); partials Partial().
        if (K % P == 0) {
            const int64_t Ks = K / P;
            // Partial() output in Y, row stride ldy.
            const int64_t ldp = N + pad;
            rec = Rec{};
            CHECK(tp_linear_row(X, ldx, W, ldw, Y, ldp, 0, TP_ROW_PARTIAL, nullptr, 0, M, N, K, P, TP_BF16,
                                nullptr) == TP_OK);
            CHECK(rec.gemms == 1 && rec.folds == 0 && rec.g.C == Y && rec.g.K == Ks);
            same_offsets(rec.g.a_shard, views(M, K, ldx, TP_SHARD, 1, P), "row X");
            same_offsets(rec.g.b_shard, views(N, K, ldw, TP_SHARD, 1, P), "row W");
            same_offsets(rec.g.c_shard, views(M, N, ldp, TP_PARTIAL, 0, P), "row partials in Y");
            // Partial() in the workspace, folded into Y (all-reduce) or
            // scattered into its Shard(0) row blocks (reduce-scatter).
            const size_t ws = tp_row_workspace_bytes(TP_ROW_SUM, M, N, P);
            for (int mode : {TP_ROW_SUM, TP_ROW_FUSED, TP_ROW_SCATTER}) {
                if (mode == TP_ROW_SCATTER && M % P) continue;
                const int64_t ldy = N + 2 * pad;
                rec = Rec{};
                CHECK(tp_linear_row(X, ldx, W, ldw, Y, ldy, 0, mode, WS, ws, M, N, K, P, TP_BF16, nullptr) ==
                      TP_OK);
                CHECK(rec.gemms == 1 && rec.folds == 1 && rec.g.C == WS && rec.r.partials == WS);
                same_offsets(rec.g.a_shard, views(M, K, ldx, TP_SHARD, 1, P), "row X");
                same_offsets(rec.g.b_shard, views(N, K, ldw, TP_SHARD, 1, P), "row W");
                same_offsets(rec.g.c_shard, views(M, N, N, TP_PARTIAL, 0, P), "row partials in workspace");
                same_offsets(rec.r.shard_stride, views(M, N, N, TP_PARTIAL, 0, P), "fold partials");
                CHECK(rec.r.Y == Y && rec.r.ldy == ldy && rec.r.ldp == N);
                if (mode == TP_ROW_SCATTER) {
                    CHECK(rec.r.slice_rows == M / P);
                    same_offsets(rec.r.slice_stride, views(M, N, ldy, TP_SHARD, 0, P), "scatter slices");
                } else {
                    CHECK(rec.r.slice_rows == M);
                }
            }
            // tp_shard_reduce's reduce-scatter: slices are Shard(0) of Y.
            if (M % P == 0) {
                const int64_t ldy = N + pad;
                rec = Rec{};
                CHECK(tp_shard_reduce(static_cast<const float *>(WS), M * N, N, Y, ldy, 0, 1, M, N, P, TP_BF16,
                                      nullptr) == TP_OK);
                CHECK(rec.folds == 1 && rec.r.slice_rows == M / P);
                same_offsets(rec.r.slice_stride, views(M, N, ldy, TP_SHARD, 0, P), "reduce slices");
            }
        }

        // ---- embedding: table [V, D] Shard(1); output concatenated [T, D]
        // Shard(1) or P shard buffers stacked [P*T, D/P] Shard(0).
        const int64_t T = M, V = K + 3, D = N, lde = D + pad;
        for (int y_mode : {TP_Y_CONCAT, TP_Y_SHARDS}) {
            const int64_t ldy = (y_mode == TP_Y_CONCAT ? D : D / P) + pad;
            rec = Rec{};
            CHECK(tp_embedding(static_cast<const int64_t *>(X), T, W, nullptr, lde, V, D, Y, ldy, y_mode, P,
                               TP_BF16, nullptr, nullptr) == TP_OK);
            CHECK(rec.embeds == 1 && rec.e.Ds == D / P && rec.e.lde == lde);
            const std::vector<tp_view> ev = views(V, D, lde, TP_SHARD, 1, P);
            for (int32_t i = 0; i < P; ++i)
                CHECK(static_cast<const char *>(rec.e.e_shard[i]) ==
                      static_cast<const char *>(W) + 2 * ev[i].elem_offset);
            if (y_mode == TP_Y_CONCAT)
                same_offsets(rec.e.y_shard, views(T, D, ldy, TP_SHARD, 1, P), "embedding Y concat");
            else
                same_offsets(rec.e.y_shard, views(P * T, D / P, ldy, TP_SHARD, 0, P), "embedding Y shards");
        }
    }

    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("launch map driver ok\n");
    return 0;
}
