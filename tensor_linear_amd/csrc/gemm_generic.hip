// Generic grouped shard GEMM: C_i = A_i * B_i^T for any M, N, K, leading
// dimensions and alignment, fp32 or bf16 inputs ("模型并行", "Tensor
// Parallel": the per-shard products Y_i = X W_i and X_i W_i).
//
// It serves the shapes the bf16 tile kernels do not take (fp32 inputs, K not
// a multiple of 8, unaligned views).  Operands are staged through LDS as
// fp32 (a bf16 value widens to fp32 exactly, and the product of two bf16
// values is exact in fp32), and multiplied on the fp32 matrix cores with
// v_mfma_f32_16x16x4_f32, accumulating in fp32.
//
// Tile 64 (M) x 64 (N) x 16 (K); 4 waves in a 2x2 grid, 32x32 outputs each.
#include "kernels.h"

namespace tpl {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int GB = 64;   // tile edge in M and N
constexpr int GK = 16;   // K per stage
constexpr int GPAD = 4;  // LDS row padding (floats)

template <int IN>
__device__ __forceinline__ float load_in(const void *p, int64_t i) {
    if (IN == IN_BF16) return (float)((const __bf16 *)p)[i];
    return ((const float *)p)[i];
}

template <int IN, int OUT>
__global__ __launch_bounds__(256)
void gemm_generic_kernel(GemmArgs g, int tiles_m, int tiles_n) {
    __shared__ float Xs[GK][GB + GPAD];  // [k][m]
    __shared__ float Ws[GK][GB + GPAD];  // [k][n]

    const int per_shard = tiles_m * tiles_n;
    const int shard = blockIdx.x / per_shard;
    const int t = blockIdx.x - shard * per_shard;
    const int64_t m0 = (int64_t)(t / tiles_n) * GB;
    const int64_t n0 = (int64_t)(t % tiles_n) * GB;

    const int esz = IN == IN_BF16 ? 2 : 4;
    const char *A = (const char *)g.A + (int64_t)shard * g.a_shard * esz;
    const char *B = (const char *)g.B + (int64_t)shard * g.b_shard * esz;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    f32x4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int64_t k0 = 0; k0 < g.K; k0 += GK) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int idx = tid + e * 256;
            const int r = idx / GK, kk = idx % GK;
            const int64_t k = k0 + kk;
            float xv = 0.f, wv = 0.f;
            if (k < g.K) {
                if (m0 + r < g.M) xv = load_in<IN>(A, (m0 + r) * g.lda + k);
                if (n0 + r < g.N) wv = load_in<IN>(B, (n0 + r) * g.ldb + k);
            }
            Xs[kk][r] = xv;
            Ws[kk][r] = wv;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < GK; kk += 4) {
            const int kr = kk + (lane >> 4);
            float a[2], b[2];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) a[nb] = Ws[kr][wn * 32 + nb * 16 + (lane & 15)];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) b[mb] = Xs[kr][wm * 32 + mb * 16 + (lane & 15)];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
                    acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[nb], b[mb], acc[nb][mb], 0, 0, 0);
        }
        __syncthreads();
    }

    // D[n][m] layout of the 16x16 block: lane holds m = lane % 16 and
    // n = 4*(lane / 16) + r for r = 0..3.
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int64_t m = m0 + wm * 32 + mb * 16 + (lane & 15);
            if (m >= g.M) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t n = n0 + wn * 32 + nb * 16 + 4 * (lane >> 4) + r;
                if (n >= g.N) continue;
                const int64_t o = (int64_t)shard * g.c_shard + m * g.ldc + n;
                if (OUT == OUT_BF16)
                    ((__bf16 *)g.C)[o] = (__bf16)acc[nb][mb][r];
                else
                    ((float *)g.C)[o] = acc[nb][mb][r];
            }
        }
}

}  // namespace

hipError_t launch_gemm_generic(const GemmArgs &g, int in_type, int out_type, hipStream_t s) {
    if (g.M == 0 || g.N == 0 || g.P == 0) return hipSuccess;
    const int64_t tm = (g.M + GB - 1) / GB, tn = (g.N + GB - 1) / GB;
    const int64_t blocks = tm * tn * g.P;
    if (tm * tn > 0x7FFFFFFFll || blocks > 0x7FFFFFFFll) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)blocks), block(256);
    const int a = (int)tm, b = (int)tn;
    if (in_type == IN_BF16) {
        if (out_type == OUT_BF16) gemm_generic_kernel<IN_BF16, OUT_BF16><<<grid, block, 0, s>>>(g, a, b);
        else gemm_generic_kernel<IN_BF16, OUT_F32><<<grid, block, 0, s>>>(g, a, b);
    } else {
        if (out_type == OUT_BF16) gemm_generic_kernel<IN_F32, OUT_BF16><<<grid, block, 0, s>>>(g, a, b);
        else gemm_generic_kernel<IN_F32, OUT_F32><<<grid, block, 0, s>>>(g, a, b);
    }
    return hipGetLastError();
}

}  // namespace tpl
