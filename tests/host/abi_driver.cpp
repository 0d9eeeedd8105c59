// Host-only driver for the sanitizer test: links the host side of the C ABI
// (tplinear.cpp) against stub launchers that abort, and exercises every path
// that returns before a launch -- tp_shard_layout over a brute-force grid
// (checked against the closed form of an even split) and every argument
// error of the compute entry points.  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py.
#include <cstdio>
#include <cstdlib>
#include <cstdint>

#include "tplinear.h"
#include "kernels.h"

namespace tpl {
// Reaching any of these means an argument check let a bad call through.
hipError_t launch_gemm_tile(const GemmArgs &, int, const GemmExtra *, hipStream_t) { std::abort(); }
hipError_t launch_gemm_narrow(const GemmArgs &, int, const GemmExtra *, hipStream_t) { std::abort(); }
bool gemm_tile_supported(const GemmArgs &, const GemmExtra *) { std::abort(); }
hipError_t launch_gemm_skinny(const GemmArgs &, int, const FoldArgs *, const GemmExtra *, hipStream_t) { std::abort(); }
bool gemm_skinny_supported(const GemmArgs &, const GemmExtra *) { std::abort(); }
hipError_t launch_gemm_generic(const GemmArgs &, int, int, const GemmExtra *, hipStream_t) { std::abort(); }
hipError_t launch_shard_fold(const ReduceArgs &, int, hipStream_t) { std::abort(); }
hipError_t launch_gemm_rowfold(const GemmArgs &, const ReduceArgs &, hipStream_t) { std::abort(); }
bool gemm_rowfold_supported(const GemmArgs &, const ReduceArgs &) { std::abort(); }
hipError_t launch_embedding(const EmbedArgs &, int, hipStream_t) { std::abort(); }
hipError_t launch_fill_zero(void *, size_t, hipStream_t) { std::abort(); }
int device_cu_count() { std::abort(); }
}  // namespace tpl

static int failures = 0;
#define CHECK(c) do { if (!(c)) { std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); ++failures; } } while (0)

int main() {
    // Layouts: every view of Shard(0/1), Replicate, Partial over a grid.
    tp_view views[TP_MAX_SHARDS];
    for (int64_t R = 0; R <= 12; ++R)
        for (int64_t C = 0; C <= 12; ++C)
            for (int64_t extra = 0; extra <= 2; ++extra)
                for (int32_t P = 1; P <= 13; ++P)
                    for (int kind = 0; kind <= 2; ++kind)
                        for (int dim = -2; dim <= 1; ++dim) {
                            const int64_t ld = C + extra;
                            tp_placement pl{kind, dim};
                            const tp_status st = tp_shard_layout(R, C, ld, pl, P, views);
                            if (kind == TP_SHARD) {
                                const int d = dim < 0 ? dim + 2 : dim;
                                const int64_t L = d == 0 ? R : C;
                                if (L % P) { CHECK(st == TP_ERR_INDIVISIBLE); continue; }
                                CHECK(st == TP_OK);
                                for (int32_t i = 0; i < P; ++i) {
                                    const tp_view &v = views[i];
                                    const int64_t s = L / P;
                                    CHECK(v.ld == ld);
                                    CHECK(d == 0 ? (v.row0 == i * s && v.col0 == 0 && v.rows == s && v.cols == C)
                                                 : (v.row0 == 0 && v.col0 == i * s && v.rows == R && v.cols == s));
                                    CHECK(v.elem_offset == v.row0 * ld + v.col0);
                                }
                            } else {
                                CHECK(st == TP_OK);
                                for (int32_t i = 0; i < P; ++i)
                                    CHECK(views[i].elem_offset == (kind == TP_PARTIAL ? i * R * ld : 0));
                                if (dim != 0) break;
                            }
                        }
    CHECK(tp_shard_layout(4, 4, 4, tp_placement{TP_SHARD, 0}, TP_MAX_SHARDS + 1, views) == TP_ERR_SHAPE);
    CHECK(tp_shard_layout(4, 4, 4, tp_placement{TP_SHARD, 0}, 2, nullptr) == TP_ERR_NULL);

    // Compute entry points: every error returns before a launch.
    void *F = reinterpret_cast<void *>(0x1000);
    const void *slices4[4] = {F, F, nullptr, F};
    CHECK(tp_linear_column(nullptr, 8, F, 8, F, 12, TP_Y_CONCAT, 3, 12, 8, 4, TP_BF16, nullptr) == TP_ERR_NULL);
    CHECK(tp_linear_column(F, 8, F, 8, F, 12, TP_Y_CONCAT, 3, 10, 8, 4, TP_BF16, nullptr) == TP_ERR_INDIVISIBLE);
    CHECK(tp_linear_column(F, 7, F, 8, F, 12, TP_Y_CONCAT, 3, 12, 8, 4, TP_BF16, nullptr) == TP_ERR_SHAPE);
    CHECK(tp_linear_column(F, 8, F, 8, F, 12, 9, 3, 12, 8, 4, TP_BF16, nullptr) == TP_ERR_MODE);
    CHECK(tp_linear_column(F, 8, F, 8, F, 12, TP_Y_CONCAT, 3, 12, 8, 4, 7, nullptr) == TP_ERR_DTYPE);
    CHECK(tp_linear_column(F, 8, F, 8, F, 12, TP_Y_CONCAT, 0, 12, 8, 4, TP_BF16, nullptr) == TP_OK);
    CHECK(tp_linear_column_ex(nullptr, slices4, 8, F, 8, nullptr, F, 12, TP_Y_CONCAT, TP_ACT_NONE, 4, 12, 8, 4,
                              TP_BF16, nullptr) == TP_ERR_NULL);
    CHECK(tp_linear_column_ex(F, nullptr, 8, F, 8, nullptr, F, 12, TP_Y_CONCAT, TP_ACT_SWIGLU, 4, 12, 8, 4,
                              TP_BF16, nullptr) == TP_ERR_INDIVISIBLE);
    CHECK(tp_linear_row(F, 8, F, 8, F, 12, 0, TP_ROW_SUM, nullptr, 0, 4, 12, 8, 4, TP_BF16, nullptr) ==
          TP_ERR_WORKSPACE);
    CHECK(tp_linear_row(F, 8, F, 8, F, 12, 0, TP_ROW_SCATTER, F, 1 << 20, 6, 12, 8, 4, TP_BF16, nullptr) ==
          TP_ERR_INDIVISIBLE);
    CHECK(tp_linear_row_ex(F, 8, F, 8, F, F, nullptr, 12, 0, TP_ROW_PARTIAL, nullptr, 0, 4, 12, 8, 4, TP_BF16,
                           nullptr) == TP_ERR_MODE);
    // Overlapping reduce-scatter slices (stride below (M/P - 1)*ldy + N).
    CHECK(tp_linear_row(F, 8, F, 8, F, 12, 23, TP_ROW_SCATTER, F, 1 << 20, 8, 12, 8, 4, TP_BF16, nullptr) ==
          TP_ERR_SHAPE);
    CHECK(tp_shard_reduce(static_cast<const float *>(F), 96, 12, F, 12, 11, 1, 4, 12, 4, TP_BF16, nullptr) ==
          TP_ERR_SHAPE);
    void *yslices[4] = {F, F, F, nullptr};
    CHECK(tp_linear_row_ex(F, 8, F, 8, nullptr, nullptr, yslices, 12, 0, TP_ROW_SCATTER, F, 1 << 20, 4, 12, 8, 4,
                           TP_BF16, nullptr) == TP_ERR_NULL);
    CHECK(tp_shard_reduce(nullptr, 48, 12, F, 12, 0, 0, 4, 12, 4, TP_BF16, nullptr) == TP_ERR_NULL);
    CHECK(tp_shard_reduce(static_cast<const float *>(F), 48, 12, F, 12, 0, 2, 4, 12, 4, TP_BF16, nullptr) ==
          TP_ERR_MODE);
    CHECK(tp_shard_reduce_ex(static_cast<const float *>(F), 48, 12, nullptr, F, yslices, 12, 0, 0, 4, 12, 4,
                             TP_BF16, nullptr) == TP_ERR_MODE);
    const void *eslices[2] = {F, nullptr};
    CHECK(tp_embedding(static_cast<const int64_t *>(F), 5, nullptr, eslices, 4, 10, 8, F, 8, TP_Y_CONCAT, 2,
                       TP_BF16, nullptr, nullptr) == TP_ERR_NULL);
    CHECK(tp_embedding(static_cast<const int64_t *>(F), 5, F, nullptr, 8, 10, 9, F, 9, TP_Y_CONCAT, 2, TP_BF16,
                       nullptr, nullptr) == TP_ERR_INDIVISIBLE);
    CHECK(tp_workspace_zero(F, 6, nullptr) == TP_ERR_SHAPE);
    CHECK(tp_row_workspace_bytes(TP_ROW_SUM, 4, 12, 4) >= 4 * 4 * 12 * 4);
    for (int s = 0; s <= 9; ++s) CHECK(tp_status_str(s) != nullptr);

    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("abi driver ok\n");
    return 0;
}
