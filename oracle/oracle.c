/*
 * CPU oracle for the tensor-parallel Linear Y = X W.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the bench's CPU
 * baseline leg use it.  It shares no source, header or table with the HIP
 * library under tensor_linear_amd/.
 *
 * Written from:
 *   - "模型并行" (wineandchord.com), section "Tensor Parallel": the Linear
 *     Y = X W, column parallel W = [W_1..W_P], Y_i = X W_i, row parallel
 *     Y = sum_i X_i W_i; section "Tensor-parallel 线性层": weight in the
 *     [in,out] orientation, results compared with the dense product.
 *   - "DTensor API 文档" (MindSpore hyper-parallel), section "reduce_partial":
 *     a Partial value is turned into the reduced value by summing the parts.
 *
 * Build: gcc -O3 -fopenmp -ffp-contract=off -fPIC -shared (no -ffast-math),
 * so every add and multiply below is one IEEE operation in the written order.
 *
 * Precision: products of two fp32 (or bf16) numbers are exact in fp64 and
 * the fp64 sum over k carries a relative error of about K * 2^-53, so
 * orc_dense is the exact product up to that bound.
 */
#include <stdint.h>
#include <string.h>

/*
 * Dense product, the plain definition ("模型并行", "Tensor Parallel", Y = XW):
 *   Y[m][n] = sum_{k=0}^{K-1} X[m][k] * W[k][n]
 * with W in the [in,out] orientation the page uses for its formula.
 * k runs in ascending order into one fp64 accumulator per (m, n).
 * Row-major, leading dimensions ldx, ldw, ldy in elements.
 */
void orc_dense(const double *X, int64_t ldx, const double *W, int64_t ldw,
               double *Y, int64_t ldy, int64_t M, int64_t K, int64_t N)
{
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        double *y = Y + m * ldy;
        for (int64_t n = 0; n < N; ++n)
            y[n] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double x = X[m * ldx + k];
            const double *w = W + k * ldw;
            for (int64_t n = 0; n < N; ++n) {
                const double p = x * w[n];
                y[n] = y[n] + p;
            }
        }
    }
}

/*
 * Sum of P partial results in fp32, the Partial -> reduced step
 * ("DTensor API 文档", "reduce_partial"; "模型并行", "Row parallel": the
 * local results are summed).  The pages fix no order for the sum; this
 * oracle takes the ascending-shard left fold
 *   out = ((p_0 + p_1) + p_2) + ... + p_{P-1}
 * one fp32 add at a time.
 *   partials: shard i at partials + i * shard_stride, row stride ldp.
 * bias (may be NULL): the row-parallel bias, whose placement is Partial()
 * ("Linear 实现解析", tp_shard_type table, row "row").  Its value is the
 * bias of the whole layer, so it is added once, to the reduced sum, as one
 * more fp32 add after the last shard: out = fold + bias[n].
 */
void orc_fold_f32(const float *partials, int64_t shard_stride, int64_t ldp,
                  int64_t M, int64_t N, int32_t P, const float *bias,
                  float *out, int64_t ldo)
{
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            float acc = partials[m * ldp + n];
            for (int32_t i = 1; i < P; ++i) {
                const float v = partials[(int64_t)i * shard_stride + m * ldp + n];
                acc = acc + v;
            }
            if (bias)
                acc = acc + bias[n];
            out[m * ldo + n] = acc;
        }
    }
}

/*
 * fp32 -> bf16, round to nearest, ties to even, on the bit pattern.
 * bf16 keeps the upper 16 bits of the fp32 pattern.  The discarded lower
 * 16 bits are compared with one half (0x8000); on a tie the kept part is
 * rounded to the even neighbour.  Adding 0x7FFF plus the lowest kept bit
 * and shifting right by 16 does exactly that, and carries into the exponent
 * (up to infinity) where the mantissa overflows.  NaN inputs give a quiet
 * NaN with the same sign and upper payload bits.  Subnormals are kept.
 */
static uint16_t bf16_rne_bits(uint32_t u)
{
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    const uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

void orc_round_bf16(const float *in, uint16_t *out, int64_t n)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, &in[i], sizeof u);
        out[i] = bf16_rne_bits(u);
    }
}

/* Number of OpenMP threads the oracle runs on (reported with its timings). */
int orc_num_threads(void)
{
    int t = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            t = omp_get_num_threads();
#endif
        }
    }
    return t;
}
