/* Host driver for the sanitizer test of the CPU oracle (oracle.c): runs its
 * dense product, fp32 fold (with and without bias) and bf16 rounding on
 * small inputs, including empty and one-element cases, and checks a few
 * exact results.  Built with AddressSanitizer and UndefinedBehaviorSanitizer
 * by tests/test_host_sanitizers.py. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void orc_dense(const double *X, int64_t ldx, const double *W, int64_t ldw, double *Y, int64_t ldy,
               int64_t M, int64_t K, int64_t N);
void orc_fold_f32(const float *partials, int64_t shard_stride, int64_t ldp, int64_t M, int64_t N,
                  int32_t P, const float *bias, float *out, int64_t ldo);
void orc_round_bf16(const float *in, uint16_t *out, int64_t n);
int orc_num_threads(void);

int main(void) {
    int fail = 0;
    for (int64_t M = 0; M <= 5; ++M)
        for (int64_t K = 0; K <= 6; ++K)
            for (int64_t N = 0; N <= 7; ++N) {
                double *X = malloc(sizeof(double) * (size_t)(M * K + 1));
                double *W = malloc(sizeof(double) * (size_t)(K * N + 1));
                double *Y = malloc(sizeof(double) * (size_t)(M * N + 1));
                for (int64_t i = 0; i < M * K; ++i) X[i] = (double)(i % 5) - 2.0;
                for (int64_t i = 0; i < K * N; ++i) W[i] = (double)(i % 3) - 1.0;
                orc_dense(X, K, W, N, Y, N, M, K, N);
                for (int64_t m = 0; m < M; ++m)
                    for (int64_t n = 0; n < N; ++n) {
                        double s = 0.0;
                        for (int64_t k = 0; k < K; ++k) s += X[m * K + k] * W[k * N + n];
                        if (Y[m * N + n] != s) fail = 1;
                    }
                free(X); free(W); free(Y);
            }
    for (int32_t P = 1; P <= 9; ++P)
        for (int64_t M = 0; M <= 3; ++M)
            for (int64_t N = 0; N <= 5; ++N) {
                float *p = malloc(sizeof(float) * (size_t)(P * M * N + 1));
                float *b = malloc(sizeof(float) * (size_t)(N + 1));
                float *o = malloc(sizeof(float) * (size_t)(M * N + 1));
                for (int64_t i = 0; i < P * M * N; ++i) p[i] = (float)(i % 7);
                for (int64_t i = 0; i < N; ++i) b[i] = (float)i;
                orc_fold_f32(p, M * N, N, M, N, P, NULL, o, N);
                orc_fold_f32(p, M * N, N, M, N, P, b, o, N);
                for (int64_t m = 0; m < M; ++m)
                    for (int64_t n = 0; n < N; ++n) {
                        float s = p[m * N + n];
                        for (int32_t i = 1; i < P; ++i) s += p[(int64_t)i * M * N + m * N + n];
                        if (o[m * N + n] != s + b[n]) fail = 1;
                    }
                free(p); free(b); free(o);
            }
    {
        float in[5] = {1.0f, -2.5f, 3.0e38f, 1.0e-40f, 0.0f};
        uint16_t out[5];
        orc_round_bf16(in, out, 5);
        if (out[0] != 0x3f80 || out[1] != 0xc020 || out[4] != 0) fail = 1;
        orc_round_bf16(in, out, 0);
    }
    if (orc_num_threads() < 1) fail = 1;
    if (fail) {
        fprintf(stderr, "oracle driver: wrong result\n");
        return 1;
    }
    printf("oracle driver ok\n");
    return 0;
}
