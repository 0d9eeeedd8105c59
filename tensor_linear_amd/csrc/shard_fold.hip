// Shard fold: Y = ((p_0 + p_1) + p_2) + ... + p_{P-1} over P fp32 partial
// results, the on-device replacement of the row-parallel all-reduce
// ("模型并行", "Row parallel": the local results are summed; "DTensor API 文档",
// "reduce_partial").  The scatter form writes token slice j to its own place,
// the reduce-scatter over tokens (nanotron "5.1 TP", REDUCE_SCATTER mode).
//
// HBM-bound: every partial is read once and Y written once.  Each lane folds
// 8 consecutive columns of one row over the P shards in registers (the
// lanes of a wavefront cover 512 consecutive columns, 16-byte loads), so
// there is no LDS, no atomic and no cross-lane step, and the order of the
// adds is fixed by the code, not by scheduling.
#include "kernels.h"

namespace tpl {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int FOLD_THREADS = 256;
constexpr int FOLD_BATCH = 8;  // shards loaded before their adds are issued

__device__ __forceinline__ int64_t out_offset(const ReduceArgs &r, int64_t m, int64_t n) {
    const int64_t j = m / r.slice_rows;
    return j * r.slice_stride + (m - j * r.slice_rows) * r.ldy + n;
}

template <int OUT>
__global__ __launch_bounds__(FOLD_THREADS)
void shard_fold_vec(ReduceArgs r) {
    const int64_t gpr = r.N >> 3;  // 8-column groups per row
    const int64_t idx = (int64_t)blockIdx.x * FOLD_THREADS + threadIdx.x;
    if (idx >= r.M * gpr) return;
    const int64_t m = idx / gpr;
    const int64_t n = (idx - m * gpr) << 3;
    const float *p = r.partials + m * r.ldp + n;

    f32x4 a0 = __builtin_nontemporal_load((const f32x4 *)p);
    f32x4 a1 = __builtin_nontemporal_load((const f32x4 *)(p + 4));
    for (int i0 = 1; i0 < r.P; i0 += FOLD_BATCH) {
        f32x4 v0[FOLD_BATCH], v1[FOLD_BATCH];
        const int cnt = min(FOLD_BATCH, r.P - i0);
#pragma unroll
        for (int u = 0; u < FOLD_BATCH; ++u) {
            if (u < cnt) {
                const float *q = p + (int64_t)(i0 + u) * r.shard_stride;
                v0[u] = __builtin_nontemporal_load((const f32x4 *)q);
                v1[u] = __builtin_nontemporal_load((const f32x4 *)(q + 4));
            }
        }
#pragma unroll
        for (int u = 0; u < FOLD_BATCH; ++u) {
            if (u < cnt) {
                a0 = a0 + v0[u];
                a1 = a1 + v1[u];
            }
        }
    }
    const int64_t o = out_offset(r, m, n);
    if (OUT == OUT_BF16) {
        bf16x8 h;
        h[0] = (__bf16)a0[0]; h[1] = (__bf16)a0[1]; h[2] = (__bf16)a0[2]; h[3] = (__bf16)a0[3];
        h[4] = (__bf16)a1[0]; h[5] = (__bf16)a1[1]; h[6] = (__bf16)a1[2]; h[7] = (__bf16)a1[3];
        __builtin_nontemporal_store(h, (bf16x8 *)((__bf16 *)r.Y + o));
    } else {
        float *y = (float *)r.Y + o;
        __builtin_nontemporal_store(a0, (f32x4 *)y);
        __builtin_nontemporal_store(a1, (f32x4 *)(y + 4));
    }
}

template <int OUT>
__global__ __launch_bounds__(FOLD_THREADS)
void shard_fold_scalar(ReduceArgs r) {
    const int64_t idx = (int64_t)blockIdx.x * FOLD_THREADS + threadIdx.x;
    if (idx >= r.M * r.N) return;
    const int64_t m = idx / r.N;
    const int64_t n = idx - m * r.N;
    const float *p = r.partials + m * r.ldp + n;
    float a = p[0];
    for (int i = 1; i < r.P; ++i) a = a + p[(int64_t)i * r.shard_stride];
    const int64_t o = out_offset(r, m, n);
    if (OUT == OUT_BF16)
        ((__bf16 *)r.Y)[o] = (__bf16)a;
    else
        ((float *)r.Y)[o] = a;
}

__global__ __launch_bounds__(256)
void fill_zero_kernel(uint32_t *p, size_t words) {
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * 256;
    for (; i < words; i += stride) p[i] = 0u;
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

hipError_t launch_shard_fold(const ReduceArgs &r, int out_type, hipStream_t s) {
    if (r.M == 0 || r.N == 0) return hipSuccess;
    const int64_t oel = out_type == OUT_BF16 ? 8 : 4;  // elements per 16 bytes
    const bool vec = (r.N % 8 == 0) && (r.ldp % 4 == 0) && (r.shard_stride % 4 == 0) &&
                     aligned16(r.partials) && aligned16(r.Y) && (r.ldy % oel == 0) &&
                     (r.slice_stride % oel == 0);
    const int64_t work = vec ? r.M * (r.N / 8) : r.M * r.N;
    const int64_t blocks = (work + FOLD_THREADS - 1) / FOLD_THREADS;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)blocks), block(FOLD_THREADS);
    if (vec) {
        if (out_type == OUT_BF16) shard_fold_vec<OUT_BF16><<<grid, block, 0, s>>>(r);
        else shard_fold_vec<OUT_F32><<<grid, block, 0, s>>>(r);
    } else {
        if (out_type == OUT_BF16) shard_fold_scalar<OUT_BF16><<<grid, block, 0, s>>>(r);
        else shard_fold_scalar<OUT_F32><<<grid, block, 0, s>>>(r);
    }
    return hipGetLastError();
}

hipError_t launch_fill_zero(void *ptr, size_t words, hipStream_t s) {
    if (words == 0) return hipSuccess;
    size_t blocks = (words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    fill_zero_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>((uint32_t *)ptr, words);
    return hipGetLastError();
}

}  // namespace tpl
