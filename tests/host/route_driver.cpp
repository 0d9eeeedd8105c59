// Host-only driver: which kernel a column layer takes, and which way the
// row modes fold (tpl::plan_row), for a GPU of 256 CUs.  TP_ROW_FUSED and TP_ROW_SCATTER give the bits of TP_ROW_SUM
// whichever way they fold, so the choice is by speed: the fused decode
// kernel for M <= 16 where its grid fills the CUs with 32 output columns
// per workgroup and K/P >= 2048, or where it does not and K/P <= 1024; the
// fold-in-registers kernel for M > 64 when the output has at least
// 256 * min(1, (K/P + 512) / 2048) tiles of 256 x 128; partials + fold
// otherwise.  TPLINEAR_ROW_FOLD=gemm, or partials that would not fit the
// caller's workspace, send every shape a fused kernel takes to it.  Links
// the host side of the C ABI (tplinear.cpp) against stubs; built and run by
// tests/test_host_sanitizers.py.
#include <cstdio>
#include <cstdlib>
#include <cstdint>
#include <cstring>

#include "tplinear.h"
#include "kernels.h"

namespace tpl {
// The shapes the fused kernels take (the real checks also look at alignment
// and leading dims, which every call below satisfies).
bool gemm_skinny_supported(const GemmArgs &g, const GemmExtra *) { return g.M >= 1 && g.M <= 48; }
bool gemm_rowfold_supported(const GemmArgs &g, const ReduceArgs &r) {
    return g.K % 64 == 0 && !(r.slice_rows < g.M && r.slice_rows % 256 != 0);
}
bool gemm_tile_supported(const GemmArgs &g, const GemmExtra *) { return g.K % 64 == 0; }
// The column GEMM's launches are recorded, not run.
const char *last_launch = "";
hipError_t launch_gemm_tile(const GemmArgs &, int, const GemmExtra *, hipStream_t) {
    last_launch = "tile";
    return hipSuccess;
}
hipError_t launch_gemm_narrow(const GemmArgs &, int, const GemmExtra *, hipStream_t) {
    last_launch = "narrow";
    return hipSuccess;
}
hipError_t launch_gemm_skinny(const GemmArgs &, int, const FoldArgs *, const GemmExtra *, hipStream_t) {
    last_launch = "skinny";
    return hipSuccess;
}
hipError_t launch_gemm_rowfold(const GemmArgs &, const ReduceArgs &, hipStream_t) { std::abort(); }
hipError_t launch_gemm_generic(const GemmArgs &, int, int, const GemmExtra *, hipStream_t) { std::abort(); }
hipError_t launch_shard_fold(const ReduceArgs &, int, hipStream_t) { std::abort(); }
hipError_t launch_embedding(const EmbedArgs &, int, hipStream_t) { std::abort(); }
hipError_t launch_fill_zero(void *, size_t, hipStream_t) { std::abort(); }
int device_cu_count() { return 256; }
}  // namespace tpl

static int failures = 0;

using Path = tpl::RowPlan::Path;
static const char *name(Path p) {
    switch (p) {
        case tpl::RowPlan::PARTIAL: return "PARTIAL";
        case tpl::RowPlan::SKINNY_FOLD: return "SKINNY_FOLD";
        case tpl::RowPlan::ROWFOLD: return "ROWFOLD";
        default: return "PARTIALS_AND_FOLD";
    }
}

static void expect(int line, int32_t mode, int64_t M, int64_t N, int64_t Ks, int32_t P, Path want,
                   size_t ws_cap = SIZE_MAX) {
    void *F = reinterpret_cast<void *>(0x1000);
    const int64_t K = Ks * P;
    tpl::RowPlan plan;
    const tp_status st = tpl::plan_row(F, K, F, K, nullptr, F, nullptr, N, 0, mode, M, N, K, P, TP_BF16,
                                       ws_cap, plan);
    if (st != TP_OK || plan.path != want) {
        std::fprintf(stderr, "line %d: mode %d M=%lld N=%lld K/P=%lld P=%d: status %d path %s, want %s\n",
                     line, mode, (long long)M, (long long)N, (long long)Ks, P, (int)st,
                     st == TP_OK ? name(plan.path) : "-", name(want));
        ++failures;
    }
}
#define EXPECT(...) expect(__LINE__, __VA_ARGS__)

// Which kernel a bf16 column layer [M, K] x [N, K]^T over P shards takes.
static void expect_col(int line, int64_t M, int64_t N, int64_t K, int32_t P, const char *want,
                       int32_t act = TP_ACT_NONE) {
    void *F = reinterpret_cast<void *>(0x1000);
    tpl::last_launch = "";
    const int64_t On = act == TP_ACT_SWIGLU ? N / 2 : N;
    const tp_status st = tp_linear_column_ex(F, nullptr, K, F, K, nullptr, F, On, TP_Y_CONCAT, act,
                                             M, N, K, P, TP_BF16, nullptr);
    if (st != TP_OK || std::strcmp(tpl::last_launch, want) != 0) {
        std::fprintf(stderr, "line %d: column M=%lld N=%lld K=%lld P=%d act %d: status %d kernel %s, want %s\n",
                     line, (long long)M, (long long)N, (long long)K, P, act, (int)st, tpl::last_launch, want);
        ++failures;
    }
}
#define EXPECT_COL(...) expect_col(__LINE__, __VA_ARGS__)

int main() {
    const Path PART = tpl::RowPlan::PARTIAL, SK = tpl::RowPlan::SKINNY_FOLD, RF = tpl::RowPlan::ROWFOLD,
               PF = tpl::RowPlan::PARTIALS_AND_FOLD;
    unsetenv("TPLINEAR_ROW_FOLD");
    // TP_ROW_PARTIAL and TP_ROW_SUM never fold inside the GEMM.
    EXPECT(TP_ROW_PARTIAL, 16, 8192, 3584, 8, PART);
    EXPECT(TP_ROW_SUM, 16, 8192, 3584, 8, PF);
    EXPECT(TP_ROW_SUM, 4096, 4096, 1792, 8, PF);
    // Decode: 32 columns per workgroup fill 256 CUs from N = 8192 on.
    EXPECT(TP_ROW_FUSED, 16, 8192, 3584, 8, SK);
    EXPECT(TP_ROW_FUSED, 1, 8192, 2048, 8, SK);
    EXPECT(TP_ROW_FUSED, 16, 8192, 1984, 8, PF);
    EXPECT(TP_ROW_FUSED, 16, 8192, 1024, 8, PF);
    EXPECT(TP_ROW_FUSED, 16, 8191, 512, 8, SK);    // 16 columns per workgroup
    EXPECT(TP_ROW_FUSED, 16, 4096, 512, 8, SK);
    EXPECT(TP_ROW_FUSED, 16, 4096, 1024, 8, SK);
    EXPECT(TP_ROW_FUSED, 16, 4096, 1088, 8, PF);
    EXPECT(TP_ROW_FUSED, 16, 4096, 1792, 8, PF);
    EXPECT(TP_ROW_FUSED, 17, 8192, 3584, 8, PF);   // above 16 tokens: partials + fold
    EXPECT(TP_ROW_FUSED, 48, 4096, 512, 8, PF);
    EXPECT(TP_ROW_FUSED, 64, 4096, 512, 8, PF);    // past the skinny kernel's 48 tokens
    EXPECT(TP_ROW_FUSED, 16, 65536, 1024, 8, PF);  // never the 256-row kernel for M <= 64
    EXPECT(TP_ROW_FUSED, 64, 65536, 1024, 8, PF);
    // Prefill: tiles = ceil(M / 256) * ceil(N / 128) against 256 * min(1, (K/P + 512) / 2048).
    EXPECT(TP_ROW_FUSED, 4096, 4096, 1792, 8, RF);   // 512 tiles
    EXPECT(TP_ROW_FUSED, 2048, 4096, 1792, 8, RF);   // 256
    EXPECT(TP_ROW_FUSED, 1792, 4096, 1792, 8, PF);   // 224
    EXPECT(TP_ROW_FUSED, 1024, 4096, 512, 8, RF);    // 128 against 128
    EXPECT(TP_ROW_FUSED, 768, 4096, 512, 8, PF);     // 96
    EXPECT(TP_ROW_FUSED, 1536, 4096, 1024, 8, RF);   // 192 against 192
    EXPECT(TP_ROW_FUSED, 1024, 4096, 1024, 8, PF);   // 128
    EXPECT(TP_ROW_FUSED, 768, 8192, 1024, 8, RF);    // 192
    EXPECT(TP_ROW_FUSED, 512, 8192, 1024, 8, PF);    // 128
    EXPECT(TP_ROW_FUSED, 65, 32768, 64, 8, RF);      // 256 tiles, K/P = 64: 72 needed
    EXPECT(TP_ROW_FUSED, 65, 4096, 64, 8, PF);       // 32
    EXPECT(TP_ROW_FUSED, 4096, 4096, 3584, 8, RF);   // K/P 3584 with a 4096 x 4096 output
    EXPECT(TP_ROW_FUSED, 4096, 4095, 3584, 8, PF);   // ... and one column short of it
    EXPECT(TP_ROW_FUSED, 8192, 8192, 4096, 8, PF);   // too long a shard K for the kernel
    EXPECT(TP_ROW_FUSED, 4096, 4096, 1800, 8, PF);   // K/P not a multiple of 64
    // The reduce-scatter folds in registers under the same rule, with
    // 256-row token slices.
    EXPECT(TP_ROW_SCATTER, 16384, 8192, 3584, 8, RF);
    EXPECT(TP_ROW_SCATTER, 2048, 4096, 1792, 8, RF);
    EXPECT(TP_ROW_SCATTER, 2048, 2048, 1792, 8, PF);   // 128 tiles
    EXPECT(TP_ROW_SCATTER, 1024, 4096, 1792, 8, PF);   // 128-row slices
    EXPECT(TP_ROW_SCATTER, 16, 8192, 3584, 8, PF);     // the decode kernel has no scatter form
    // Partials that would not fit the caller's workspace: every shape a
    // fused kernel takes folds inside the GEMM.
    EXPECT(TP_ROW_FUSED, 48, 32768, 4160, 8, SK, (size_t)32 << 20);   // K/P > 4096: skinny
    EXPECT(TP_ROW_FUSED, 64, 32768, 64, 8, RF, (size_t)32 << 20);
    EXPECT(TP_ROW_FUSED, 2048, 1024, 1024, 8, RF, (size_t)32 << 20);
    EXPECT(TP_ROW_FUSED, 2048, 1024, 1024, 8, PF, (size_t)64 << 20);   // they fit
    EXPECT(TP_ROW_FUSED, 4096, 4096, 8192, 8, PF, (size_t)32 << 20);   // no kernel takes it
    EXPECT(TP_ROW_SUM, 2048, 1024, 1024, 8, PF, (size_t)32 << 20);     // TP_ROW_SUM never folds inside
    // TPLINEAR_ROW_FOLD=gemm: the same, whatever the sizes.
    setenv("TPLINEAR_ROW_FOLD", "gemm", 1);
    EXPECT(TP_ROW_FUSED, 48, 512, 512, 8, SK);      // few tiles: skinny
    EXPECT(TP_ROW_FUSED, 32, 4096, 512, 8, SK);
    EXPECT(TP_ROW_FUSED, 48, 4096, 512, 8, RF);     // 256 tiles of 128 rows: the tile order
    EXPECT(TP_ROW_FUSED, 64, 4096, 512, 8, RF);
    EXPECT(TP_ROW_FUSED, 16, 8192, 1024, 8, SK);
    EXPECT(TP_ROW_FUSED, 65, 4096, 64, 8, RF);
    EXPECT(TP_ROW_FUSED, 1024, 4096, 1792, 8, RF);
    EXPECT(TP_ROW_SCATTER, 2048, 2048, 1792, 8, RF);
    EXPECT(TP_ROW_SCATTER, 1024, 4096, 1792, 8, PF);
    EXPECT(TP_ROW_FUSED, 8192, 8192, 4096, 8, PF);
    EXPECT(TP_ROW_SUM, 16, 8192, 3584, 8, PF);
    setenv("TPLINEAR_ROW_FOLD", "auto", 1);          // any other value: the library's choice
    EXPECT(TP_ROW_FUSED, 64, 4096, 512, 8, PF);
    unsetenv("TPLINEAR_ROW_FOLD");

    // The column GEMM: skinny up to 32 tokens, and up to 48 for K > 4096 or
    // when 128-row tiles over all shards would fill at most half of the CUs;
    // the narrow kernel when 256 x 256 tiles would fill at most half of them.
    EXPECT_COL(16, 28672, 8192, 8, "skinny");
    EXPECT_COL(32, 28672, 4096, 8, "skinny");
    EXPECT_COL(33, 28672, 4096, 8, "narrow");     // 224 tiles of 128 rows
    EXPECT_COL(48, 28672, 4096, 8, "narrow");
    EXPECT_COL(48, 28672, 4096, 1, "narrow");     // the same family whatever P is
    EXPECT_COL(48, 28672, 8192, 8, "skinny");     // K > 4096
    EXPECT_COL(48, 10240, 4096, 8, "skinny");     // 80 tiles of 128 rows
    EXPECT_COL(49, 10240, 8192, 8, "narrow");
    EXPECT_COL(48, 65536, 4096, 8, "tile");       // 256 tiles of 256 x 256
    EXPECT_COL(256, 28672, 4096, 8, "narrow");    // 112 tiles of 256 x 256
    EXPECT_COL(512, 28672, 4096, 8, "tile");      // 224
    EXPECT_COL(4096, 28672, 4096, 8, "tile");
    EXPECT_COL(40, 28672, 4096, 8, "narrow", TP_ACT_SWIGLU);   // gated unit: 64 outputs per 128 W rows
    EXPECT_COL(40, 8192, 4096, 8, "skinny", TP_ACT_SWIGLU);
    EXPECT_COL(256, 28672, 4096, 8, "narrow", TP_ACT_SWIGLU);  // 112 tiles of 256 rows x 128 outputs
    EXPECT_COL(512, 28672, 4096, 8, "tile", TP_ACT_SWIGLU);    // 224
    if (failures) {
        std::fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    std::printf("route driver ok\n");
    return 0;
}
