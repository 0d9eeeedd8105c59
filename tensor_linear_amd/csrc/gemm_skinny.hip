// Skinny shard GEMM for decode-shaped inputs (M <= 64 tokens): C_i = A_i B_i^T
// where the weight dominates the bytes, so the kernel is bound by how fast
// it streams W from HBM ("模型并行", "Tensor Parallel": Y_i = X W_i for the
// column form, the partials X_i W_i for the row form).
//
// Work unit: one workgroup = one shard i and one 64-column tile of the output
// (64 rows of W_i), over the shard's whole K range.  Four waves split that K
// range into four contiguous quarters; each wave loads its W rows and the
// matching X rows straight from global memory into MFMA fragments
// (16-byte loads, several k-steps in flight) and multiplies on
// v_mfma_f32_16x16x32_bf16 with W as the 16-row operand and X as the
// 16-column operand.  The four wave partials are added through LDS in
// fixed order (w0 + w1) + w2 + w3.
//
// Fused fold (row form, decode): each workgroup stores its fp32 partial tile,
// then bumps the tile's counter with an agent-scope release/acquire atomic.
// The workgroup that sees the count reach P-1 is the last one for that tile:
// it folds the P partial tiles in ascending shard order, one fp32 add at a
// time, rounds once, writes Y and puts the counter back to zero.  The order
// of the adds does not depend on which workgroup arrives last, so the result
// equals the unfused partial + fold sequence bit for bit.  No workgroup ever
// waits for another.
#include "kernels.h"

namespace tpl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int SK_THREADS = 256;
constexpr int SK_WAVES = 4;
constexpr int SK_NB = SKINNY_BN / 16;  // 16-row W blocks per workgroup

template <int OUT>
__device__ __forceinline__ void store_out(void *Y, int64_t o, float v) {
    if (OUT == OUT_BF16) ((__bf16 *)Y)[o] = (__bf16)v;
    else ((float *)Y)[o] = v;
}

template <int MB, int U, int OUT, bool FUSED>
__global__ __launch_bounds__(SK_THREADS)
void gemm_skinny_kernel(GemmArgs g, FoldArgs f, int tiles_n) {
    __shared__ f32x4 red[SK_WAVES][SK_NB * MB][64];

    const int tn = blockIdx.x / g.P;
    const int shard = blockIdx.x - tn * g.P;
    const int64_t n0 = (int64_t)tn * SKINNY_BN;

    const __bf16 *A = (const __bf16 *)g.A + (int64_t)shard * g.a_shard;
    const __bf16 *B = (const __bf16 *)g.B + (int64_t)shard * g.b_shard;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kl = 8 * (lane >> 4);  // this lane's 8-element slice of a k32 step

    // Row pointers; rows past the edge are clamped (their results are never
    // stored), so every load stays inside the operands.
    const __bf16 *wrow[SK_NB];
#pragma unroll
    for (int nb = 0; nb < SK_NB; ++nb) {
        int64_t n = n0 + nb * 16 + (lane & 15);
        if (n > g.N - 1) n = g.N - 1;
        wrow[nb] = B + n * g.ldb + kl;
    }
    const __bf16 *xrow[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        int64_t m = mb * 16 + (lane & 15);
        if (m > g.M - 1) m = g.M - 1;
        xrow[mb] = A + m * g.lda + kl;
    }

    f32x4 acc[SK_NB][MB];
#pragma unroll
    for (int nb = 0; nb < SK_NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t nsteps = (g.K + 31) / 32;
    const int64_t s0 = nsteps * wave / SK_WAVES;
    const int64_t s1 = nsteps * (wave + 1) / SK_WAVES;
    const int64_t full = g.K / 32;  // steps with all 32 k inside K
    const int64_t s_full_end = s1 < full ? s1 : full;

    int64_t s = s0;
    for (; s + U <= s_full_end; s += U) {
        bf16x8 wv[U][SK_NB], xv[U][MB];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int nb = 0; nb < SK_NB; ++nb)
                wv[u][nb] = __builtin_nontemporal_load((const bf16x8 *)(wrow[nb] + (s + u) * 32));
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                xv[u][mb] = *(const bf16x8 *)(xrow[mb] + (s + u) * 32);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int nb = 0; nb < SK_NB; ++nb)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[u][nb], xv[u][mb],
                                                                          acc[nb][mb], 0, 0, 0);
    }
    for (; s < s1; ++s) {
        // K % 8 == 0, so a lane's 8-element slice is either all inside K or
        // all outside; outside slices contribute zero.
        const bool valid = s * 32 + kl < g.K;
        bf16x8 wv[SK_NB], xv[MB];
#pragma unroll
        for (int nb = 0; nb < SK_NB; ++nb) {
            wv[nb] = bf16x8{};
            if (valid) wv[nb] = *(const bf16x8 *)(wrow[nb] + s * 32);
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            xv[mb] = bf16x8{};
            if (valid) xv[mb] = *(const bf16x8 *)(xrow[mb] + s * 32);
        }
#pragma unroll
        for (int nb = 0; nb < SK_NB; ++nb)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[nb], xv[mb], acc[nb][mb], 0, 0, 0);
    }

#pragma unroll
    for (int nb = 0; nb < SK_NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) red[wave][nb * MB + mb][lane] = acc[nb][mb];
    __syncthreads();

    // Output element (m, n) of the tile sits in block (n/16, m/16) at lane
    // 16*((n%16)/4) + m%16, register n%4 (16x16 MFMA D layout with W rows as
    // the row operand).  Threads take consecutive n for coalesced stores.
    constexpr int OUTS = 64 * 16 * MB / SK_THREADS;
    float val[OUTS];
    int64_t mm[OUTS], nn[OUTS];
#pragma unroll
    for (int e = 0; e < OUTS; ++e) {
        const int idx = tid + e * SK_THREADS;
        const int n = idx & 63, m = idx >> 6;
        const int blk = (n >> 4) * MB + (m >> 4);
        const int ln = 16 * ((n & 15) >> 2) + (m & 15);
        const int r = n & 3;
        float v = red[0][blk][ln][r];
        v = v + red[1][blk][ln][r];
        v = v + red[2][blk][ln][r];
        v = v + red[3][blk][ln][r];
        val[e] = v;
        mm[e] = m;
        nn[e] = n0 + n;
    }

    if (!FUSED) {
#pragma unroll
        for (int e = 0; e < OUTS; ++e)
            if (mm[e] < g.M && nn[e] < g.N)
                store_out<OUT>(g.C, (int64_t)shard * g.c_shard + mm[e] * g.ldc + nn[e], val[e]);
        return;
    }

    // Fused: publish this shard's partial tile, then count arrivals.
    const int64_t part_stride = g.M * g.N;
#pragma unroll
    for (int e = 0; e < OUTS; ++e)
        if (mm[e] < g.M && nn[e] < g.N)
            f.partials[(int64_t)shard * part_stride + mm[e] * g.N + nn[e]] = val[e];
    __threadfence();
    __syncthreads();
    __shared__ uint32_t s_last;
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&f.counters[tn], 1u, __ATOMIC_ACQ_REL,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        s_last = (old == (uint32_t)(g.P - 1)) ? 1u : 0u;
    }
    __syncthreads();
    if (s_last == 0u) return;
    __threadfence();
#pragma unroll
    for (int e = 0; e < OUTS; ++e) {
        if (mm[e] < g.M && nn[e] < g.N) {
            const float *p = f.partials + mm[e] * g.N + nn[e];
            float a = __builtin_nontemporal_load(p);
            for (int i = 1; i < g.P; ++i) a = a + __builtin_nontemporal_load(p + (int64_t)i * part_stride);
            store_out<OUT>(f.Y, mm[e] * f.ldy + nn[e], a);
        }
    }
    if (tid == 0)
        __hip_atomic_store(&f.counters[tn], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MB, int U>
hipError_t launch_mb(const GemmArgs &g, int out_type, const FoldArgs *fold, hipStream_t s) {
    const int64_t tn = (g.N + SKINNY_BN - 1) / SKINNY_BN;
    const int64_t blocks = tn * g.P;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)blocks), block(SK_THREADS);
    FoldArgs f = fold ? *fold : FoldArgs{nullptr, 0, 0, nullptr, nullptr};
    if (fold) {
        if (out_type == OUT_BF16) gemm_skinny_kernel<MB, U, OUT_BF16, true><<<grid, block, 0, s>>>(g, f, (int)tn);
        else gemm_skinny_kernel<MB, U, OUT_F32, true><<<grid, block, 0, s>>>(g, f, (int)tn);
    } else {
        if (out_type == OUT_BF16) gemm_skinny_kernel<MB, U, OUT_BF16, false><<<grid, block, 0, s>>>(g, f, (int)tn);
        else gemm_skinny_kernel<MB, U, OUT_F32, false><<<grid, block, 0, s>>>(g, f, (int)tn);
    }
    return hipGetLastError();
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

bool gemm_skinny_supported(const GemmArgs &g) {
    return g.M >= 1 && g.M <= SKINNY_MAX_M && g.K % 8 == 0 && g.lda % 8 == 0 &&
           g.ldb % 8 == 0 && g.a_shard % 8 == 0 && g.b_shard % 8 == 0 &&
           aligned16(g.A) && aligned16(g.B);
}

hipError_t launch_gemm_skinny(const GemmArgs &g, int out_type, const FoldArgs *fold,
                              hipStream_t s) {
    if (g.M == 0 || g.N == 0 || g.P == 0) return hipSuccess;
    if (g.M <= 16) return launch_mb<1, 4>(g, out_type, fold, s);
    if (g.M <= 32) return launch_mb<2, 4>(g, out_type, fold, s);
    return launch_mb<4, 2>(g, out_type, fold, s);
}

}  // namespace tpl
