// Internal launch interface between the C ABI (tplinear.cpp) and the HIP
// kernels.  Not installed, not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tplinear.h"

namespace tpl {

// One grouped GEMM over P shards: for i in [0, P)
//   C_i[M, N] = A_i[M, K] * B_i[N, K]^T
// with A_i = A + i*a_shard, B_i = B + i*b_shard, C_i = C + i*c_shard
// (element offsets), row-major with leading dims lda, ldb, ldc.
// Column parallel: A = X (a_shard 0), B = W row block i, C = Y column block i.
// Row parallel:    A = X column block i, B = W column block i, C = part i.
struct GemmArgs {
    const void *A; int64_t lda; int64_t a_shard;
    const void *B; int64_t ldb; int64_t b_shard;
    void *C;       int64_t ldc; int64_t c_shard;
    int64_t M, N, K;
    int32_t P;
};

enum InType { IN_F32 = 0, IN_BF16 = 1 };

constexpr int MAX_SLICES = 64;  // = TP_MAX_SHARDS

// What a column GEMM does besides C_i = A_i B_i^T (all optional).
//   bias:  per output feature, of the output type; shard i's bias starts at
//          bias + i*bias_shard (elements).  Added in fp32 before rounding.
//   swiglu: the gated unit.  Output column c of shard i is
//          silu(g + bg) * (u + bu) with g from B row c and u from B row
//          up_off + c of the shard (and the bias at the same offsets), so
//          g.N counts output columns, not B rows.
//   x_rows: > 0 when A is given as token slices: row m of A is row
//          m % x_rows of slice m / x_rows, at x_slice[m / x_rows] with row
//          stride lda (a_shard then only offsets the column).
enum ActType { ACT_NONE = 0, ACT_SWIGLU = 1 };
struct GemmExtra {
    const void *bias; int64_t bias_shard;
    int32_t act; int64_t up_off;
    int64_t x_rows;
    const void *x_slice[MAX_SLICES];
};

// silu(v) = v * sigmoid(v) = v / (1 + e^-v), fp32, shared by every kernel
// that applies the gated unit.  For v below about -88 the exponential is
// +inf and the quotient a signed zero, the function's limit.
__device__ __forceinline__ float silu_f32(float v) { return v / (1.0f + __expf(-v)); }
enum OutType { OUT_F32 = 0, OUT_BF16 = 1 };

// Fused fold for the skinny row GEMM: each workgroup walks all P shards of
// its output tile in ascending order and adds the shard partials into a
// running fp32 sum, written once to Y.
struct FoldArgs {
    void *Y; int64_t ldy; int32_t out_type;
};

// 256x256x64 bf16 MFMA tile kernel.  Requires K > 0, K % 64 == 0, lda, ldb,
// a_shard, b_shard multiples of 8 and A, B 16-byte aligned; with x slices,
// x_rows a multiple of 256 and every slice 16-byte aligned.
hipError_t launch_gemm_tile(const GemmArgs &g, int out_type, const GemmExtra *ex,
                            hipStream_t s);
bool gemm_tile_supported(const GemmArgs &g, const GemmExtra *ex);
// Narrow tiles for launches whose 256 x 256 tiles would fill at most half of
// the CUs: 128 x 128 (four waves) when those fit in one pass over the CUs,
// 128 x 64 when they would fill at most half of it, else 256 x 128 (eight
// waves, two per SIMD); no token slices, and the bias and the gated unit
// (on 128 W rows: 64 outputs per tile) only with bf16 output.  Bitwise the
// same results as the tile kernel.
hipError_t launch_gemm_narrow(const GemmArgs &g, int out_type, const GemmExtra *ex,
                              hipStream_t s);

// Skinny (M <= 48) bf16 kernel that streams W.  Requires K > 0, K % 8 == 0,
// lda, ldb, a_shard, b_shard multiples of 8 and A, B 16-byte aligned.
// fold == nullptr: C_i written as out_type.  fold != nullptr: C is unused
// and the fold of the P shard products is written to fold->Y.
// ex: bias and the gated unit (column form), or the bias added after the
// fold (fused form); x slices are not taken here.
hipError_t launch_gemm_skinny(const GemmArgs &g, int out_type, const FoldArgs *fold,
                              const GemmExtra *ex, hipStream_t s);
bool gemm_skinny_supported(const GemmArgs &g, const GemmExtra *ex);
constexpr int SKINNY_MAX_M = 48;

// Any shape, stride or alignment; fp32 or bf16 inputs; every GemmExtra option.
hipError_t launch_gemm_generic(const GemmArgs &g, int in_type, int out_type,
                               const GemmExtra *ex, hipStream_t s);

// Ascending-shard fold of P fp32 parts into Y (optionally scattered into
// token slices: output row m goes to slice m / slice_rows at
// Y + (m / slice_rows)*slice_stride + (m % slice_rows)*ldy).
// With use_slices, slice j is at y_slice[j] instead (slice_stride unused).
// bias (optional, of the output type, [N]) is added once after the fold.
struct ReduceArgs {
    const float *partials; int64_t shard_stride; int64_t ldp;
    void *Y; int64_t ldy; int64_t slice_rows; int64_t slice_stride;
    int64_t M, N; int32_t P;
    const void *bias;
    int32_t use_slices;
    void *y_slice[MAX_SLICES];
};
hipError_t launch_shard_fold(const ReduceArgs &r, int out_type, hipStream_t s);

// Row GEMM with the fold of the P shard partials in registers (bf16 in and
// out; 256x128 tiles): writes the fold (+ r.bias) of the products
// A_i B_i^T, i ascending, where r places the output (Y, ldy, token slices);
// the partials fields of r are unused.  Same requirements as the tile
// kernel; for a reduce-scatter, slice_rows a multiple of 256.
hipError_t launch_gemm_rowfold(const GemmArgs &g, const ReduceArgs &r, hipStream_t s);
bool gemm_rowfold_supported(const GemmArgs &g, const ReduceArgs &r);

// Feature-sharded embedding lookup: for token t and shard i,
//   Y row t, columns [i*Ds, (i+1)*Ds)  (CONCAT), or block i row t (SHARDS)
//   = row ids[t] of shard i (e_shard[i], row stride lde), Ds = D / P;
// an id outside [0, V) writes zeros and sets *bad to 1 when bad != nullptr.
struct EmbedArgs {
    const int64_t *ids; int64_t T, V, Ds; int32_t P;
    int64_t lde; void *Y; int64_t ldy; int64_t y_shard;
    int32_t *bad;
    const void *e_shard[MAX_SLICES];
};
hipError_t launch_embedding(const EmbedArgs &e, int elem_bytes, hipStream_t s);

hipError_t launch_fill_zero(void *ptr, size_t words, hipStream_t s);

// Every argument check of tp_linear_row_ex except the workspace's (TP_OK
// also for empty problems, which queue nothing).  Shared by the entry points
// so that they reject the same calls with the same status.
tp_status row_args_status(const void *X, int64_t ldx, const void *W, int64_t ldw,
                          const void *bias, void *Y, void *const *y_slices, int64_t ldy,
                          int64_t y_slice_stride, int32_t mode, int64_t M, int64_t N, int64_t K,
                          int32_t P, int32_t dtype);

// The launch plan of a row-parallel call that passed row_args_status and is
// not empty: the kernels tp_linear_row_ex runs for it (which depend on the
// mode, dtype and shape), built without touching any memory.  Only
// PARTIALS_AND_FOLD uses the workspace (P fp32 [M, N] partials, row stride
// N); the other paths write the output directly.
struct RowPlan {
    enum Path { PARTIAL, SKINNY_FOLD, ROWFOLD, PARTIALS_AND_FOLD } path;
    GemmArgs g; ReduceArgs r; FoldArgs f; GemmExtra ex;
    int out; int32_t dtype;
};
// ws_cap: the workspace bytes the caller can give; where the P fp32 partials
// would not fit it, TP_ROW_FUSED / TP_ROW_SCATTER fold inside the GEMM
// wherever a kernel takes the shape.
tp_status plan_row(const void *X, int64_t ldx, const void *W, int64_t ldw, const void *bias,
                   void *Y, void *const *y_slices, int64_t ldy, int64_t y_slice_stride,
                   int32_t mode, int64_t M, int64_t N, int64_t K, int32_t P, int32_t dtype,
                   size_t ws_cap, RowPlan &plan);
// Queue the plan's kernels; `workspace` is read only by PARTIALS_AND_FOLD
// (TP_ERR_WORKSPACE if it is null there).
tp_status run_row(RowPlan &plan, float *workspace, hipStream_t s);

// Compute units of the current device (cached per device; 256 if the query
// fails).  Sizes the persistent grids of the tile kernels.
int device_cu_count();

}  // namespace tpl
