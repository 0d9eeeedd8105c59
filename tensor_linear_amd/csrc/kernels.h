// Internal launch interface between the C ABI (tplinear.cpp) and the HIP
// kernels.  Not installed, not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
enum OutType { OUT_F32 = 0, OUT_BF16 = 1 };

// Fused fold for the skinny row GEMM: each workgroup walks all P shards of
// its output tile in ascending order and adds the shard partials into a
// running fp32 sum, written once to Y.
struct FoldArgs {
    void *Y; int64_t ldy; int32_t out_type;
};

// 256x256x64 bf16 MFMA tile kernel.  Requires K > 0, K % 64 == 0, lda, ldb,
// a_shard, b_shard multiples of 8 and A, B 16-byte aligned.
hipError_t launch_gemm_tile(const GemmArgs &g, int out_type, hipStream_t s);
bool gemm_tile_supported(const GemmArgs &g);

// Skinny (M <= 64) bf16 kernel that streams W.  Requires K > 0, K % 8 == 0,
// lda, ldb, a_shard, b_shard multiples of 8 and A, B 16-byte aligned.
// fold == nullptr: C_i written as out_type.  fold != nullptr: C is unused
// and the fold of the P shard products is written to fold->Y.
hipError_t launch_gemm_skinny(const GemmArgs &g, int out_type, const FoldArgs *fold,
                              hipStream_t s);
bool gemm_skinny_supported(const GemmArgs &g);
constexpr int SKINNY_MAX_M = 64;

// Any shape, stride or alignment; fp32 or bf16 inputs.
hipError_t launch_gemm_generic(const GemmArgs &g, int in_type, int out_type, hipStream_t s);

// Ascending-shard fold of P fp32 parts into Y (optionally scattered into
// token slices: output row m goes to slice m / slice_rows at
// Y + (m / slice_rows)*slice_stride + (m % slice_rows)*ldy).
struct ReduceArgs {
    const float *partials; int64_t shard_stride; int64_t ldp;
    void *Y; int64_t ldy; int64_t slice_rows; int64_t slice_stride;
    int64_t M, N; int32_t P;
};
hipError_t launch_shard_fold(const ReduceArgs &r, int out_type, hipStream_t s);

hipError_t launch_fill_zero(void *ptr, size_t words, hipStream_t s);

}  // namespace tpl
