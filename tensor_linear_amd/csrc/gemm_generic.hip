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
//
// Every epilogue option of the column layer is taken here too: the bias (of
// the output type) added in fp32 before rounding; the gated unit, for which
// the tile's 64 W rows are 32 gate rows and the 32 up rows of the same hidden
// units (each wave's 16-row blocks 0 and 1), giving 64 x 32 outputs of
// silu(g + bg) * (u + bu); and X given as token slices, row m read from
// slice m / x_rows.
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

template <int OUT>
__device__ __forceinline__ float load_bias(const void *b, int64_t i) {
    if (OUT == OUT_BF16) return (float)((const __bf16 *)b)[i];
    return ((const float *)b)[i];
}

template <int IN, int OUT, bool SWIGLU, bool XG>
__global__ __launch_bounds__(256)
void gemm_generic_kernel(GemmArgs g, int tiles_m, int tiles_n, GemmExtra ex) {
    constexpr int ON = SWIGLU ? GB / 2 : GB;   // output columns per tile
    __shared__ float Xs[GK][GB + GPAD];  // [k][m]
    __shared__ float Ws[GK][GB + GPAD];  // [k][n]

    const int per_shard = tiles_m * tiles_n;
    const int shard = blockIdx.x / per_shard;
    const int t = blockIdx.x - shard * per_shard;
    const int64_t m0 = (int64_t)(t / tiles_n) * GB;
    const int64_t n0 = (int64_t)(t % tiles_n) * ON;

    const int esz = IN == IN_BF16 ? 2 : 4;
    const char *A = (const char *)g.A + (int64_t)shard * g.a_shard * esz;
    const char *B = (const char *)g.B + (int64_t)shard * g.b_shard * esz;
    // Row m of this shard's A.
    auto a_row = [&](int64_t m) -> const char * {
        if (XG) {
            const int64_t sl = m / ex.x_rows;
            return (const char *)ex.x_slice[sl] + ((int64_t)shard * g.a_shard + (m - sl * ex.x_rows) * g.lda) * esz;
        }
        return A + m * g.lda * esz;
    };
    // Tile row r of B: for the gated unit rows 16-31 of each 32 are the up
    // rows of the units in rows 0-15.
    auto b_index = [&](int r, bool &ok) -> int64_t {
        if (SWIGLU) {
            const int64_t h = n0 + (r >> 5) * 16 + (r & 15);
            ok = h < g.N;
            return h + ((r >> 4) & 1 ? ex.up_off : 0);
        }
        ok = n0 + r < g.N;
        return n0 + r;
    };

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
                if (m0 + r < g.M) xv = load_in<IN>(a_row(m0 + r), k);
                bool ok;
                const int64_t br = b_index(r, ok);
                if (ok) wv = load_in<IN>(B, br * g.ldb + k);
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
    auto store = [&](int64_t m, int64_t n, float v) {
        const int64_t o = (int64_t)shard * g.c_shard + m * g.ldc + n;
        if (OUT == OUT_BF16)
            ((__bf16 *)g.C)[o] = (__bf16)v;
        else
            ((float *)g.C)[o] = v;
    };
    const int64_t bsh = (int64_t)shard * ex.bias_shard;
    if (SWIGLU) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int64_t m = m0 + wm * 32 + mb * 16 + (lane & 15);
            if (m >= g.M) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t n = n0 + wn * 16 + 4 * (lane >> 4) + r;
                if (n >= g.N) continue;
                float gv = acc[0][mb][r], uv = acc[1][mb][r];
                if (ex.bias) {
                    gv = gv + load_bias<OUT>(ex.bias, bsh + n);
                    uv = uv + load_bias<OUT>(ex.bias, bsh + ex.up_off + n);
                }
                store(m, n, silu_f32(gv) * uv);
            }
        }
        return;
    }
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
                float v = acc[nb][mb][r];
                if (ex.bias) v = v + load_bias<OUT>(ex.bias, bsh + n);
                store(m, n, v);
            }
        }
}

}  // namespace

namespace {

template <int IN, int OUT>
hipError_t launch_generic_t(const GemmArgs &g, const GemmExtra &ex, dim3 grid, int a, int b,
                            hipStream_t s) {
    const bool sw = ex.act == ACT_SWIGLU, xg = ex.x_rows > 0;
    if (sw && xg) gemm_generic_kernel<IN, OUT, true, true><<<grid, dim3(256), 0, s>>>(g, a, b, ex);
    else if (sw) gemm_generic_kernel<IN, OUT, true, false><<<grid, dim3(256), 0, s>>>(g, a, b, ex);
    else if (xg) gemm_generic_kernel<IN, OUT, false, true><<<grid, dim3(256), 0, s>>>(g, a, b, ex);
    else gemm_generic_kernel<IN, OUT, false, false><<<grid, dim3(256), 0, s>>>(g, a, b, ex);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_generic(const GemmArgs &g, int in_type, int out_type,
                               const GemmExtra *exp, hipStream_t s) {
    if (g.M == 0 || g.N == 0 || g.P == 0) return hipSuccess;
    GemmExtra ex{};
    if (exp) ex = *exp;
    const int on = ex.act == ACT_SWIGLU ? GB / 2 : GB;
    const int64_t tm = (g.M + GB - 1) / GB, tn = (g.N + on - 1) / on;
    const int64_t blocks = tm * tn * g.P;
    if (tm * tn > 0x7FFFFFFFll || blocks > 0x7FFFFFFFll) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)blocks);
    const int a = (int)tm, b = (int)tn;
    if (in_type == IN_BF16) {
        if (out_type == OUT_BF16) return launch_generic_t<IN_BF16, OUT_BF16>(g, ex, grid, a, b, s);
        return launch_generic_t<IN_BF16, OUT_F32>(g, ex, grid, a, b, s);
    }
    if (out_type == OUT_BF16) return launch_generic_t<IN_F32, OUT_BF16>(g, ex, grid, a, b, s);
    return launch_generic_t<IN_F32, OUT_F32>(g, ex, grid, a, b, s);
}

}  // namespace tpl
