// Skinny shard GEMM for decode-shaped inputs (M <= 48 tokens): C_i = A_i B_i^T
// where the weight dominates the bytes, so the kernel is bound by how fast
// it streams W from HBM ("模型并行", "Tensor Parallel": Y_i = X W_i for the
// column form, the partials X_i W_i for the row form).
//
// Work unit: one workgroup owns BN = 16*NB rows of W (NB blocks of 16 output
// columns) and one shard -- or, in the fused row form, all P shards in
// ascending order; the NB blocks share the staged X rows.
// W and X move global -> LDS with global_load_lds_dwordx4 in NST stages of
// KB columns of K; each 1 KB load instruction covers one contiguous KB*2-byte
// run of one row, so HBM sees long sequential runs rather than 64-byte
// pieces of many rows.  In LDS, 16-byte chunk c of row r sits at slot
// c ^ (r % 16), so the 16 rows of an MFMA fragment read hit 16 different
// bank groups.  The shard's K is cut into 32-column blocks; wave w takes the
// blocks whose index is w mod 4, in ascending order, and multiplies on
// v_mfma_f32_16x16x32_bf16 (W rows as the row operand).  The four wave sums
// are added through LDS in the fixed order ((w0 + w1) + w2) + w3 when a
// shard ends.  Since a stage holds a multiple of four blocks, which blocks
// each wave adds, and in which order, does not depend on the stage size:
// every instantiation gives the same fp32 result for the same shard.
//
// Fused fold (row form, decode): the shard partials are added into a
// running fp32 sum in ascending shard order, one add at a time, and the sum
// is rounded once -- the same operations, in the same order, as writing the
// partials and running the fold kernel, so the result is bitwise equal to
// that unfused sequence.  No workspace, counter or cross-workgroup signal is
// needed.
//
// Epilogue options: the column bias (Shard(0)) is added to each output in
// fp32 before rounding; the row bias (Partial(), the whole layer's bias) is
// added once to the fused sum after the last shard.  The gated unit of a
// fused gate+up column layer (SWIGLU) takes 16 gate rows and the 16 up rows
// of the same hidden units per workgroup (NB = 2), so both products of an
// output land in the same thread's reduction: silu(g + bg) * (u + bu).
#include "kernels.h"

namespace tpl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T) __attribute__((address_space(3))) T *

constexpr int SK_THREADS = 256;

template <int OUT>
__device__ __forceinline__ void store_out(void *Y, int64_t o, float v) {
    if (OUT == OUT_BF16) ((__bf16 *)Y)[o] = (__bf16)v;
    else ((float *)Y)[o] = v;
}

// NB: 16-row blocks of W.  MB: 16-row blocks of M.  KB: K columns per stage.
// NST: stages.
template <int NB, int MB, int KB, int NST, int OUT, bool FOLD, bool SWIGLU>
__global__ __launch_bounds__(SK_THREADS)
void gemm_skinny_kernel(GemmArgs g, FoldArgs f, GemmExtra ex) {
    static_assert(!SWIGLU || (NB == 2 && !FOLD), "gated unit: 16 gate + 16 up rows, column form");
    constexpr int BN = 16 * NB;            // W rows per workgroup
    constexpr int ON = SWIGLU ? 16 : BN;   // output columns per workgroup
    constexpr int XR = 16 * MB;            // X rows staged
    constexpr int ROWB = KB * 2;           // bytes per staged row
    constexpr int CPR = ROWB / 16;         // 16-byte chunks per row
    static_assert(CPR >= 16, "rows of at least 256 bytes");
    constexpr int STB = (BN + XR) * ROWB;  // bytes per stage (rows back to back)
    constexpr int NI = STB / 1024;         // 1 KB load instructions per stage
    static_assert(STB % 4096 == 0, "loads split over 4 waves");
    constexpr int LPW = NI / 4;            // per wave
    constexpr int SUBS = KB / 32 / 4;      // k32 sub-steps per wave per stage
    static_assert(SUBS >= 1, "KB >= 128");
    __shared__ __attribute__((aligned(1024))) char smem[NST * STB];
    __shared__ f32x4 red[4][NB][MB][64];
    LDS_PTR(char) lds = (LDS_PTR(char))smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    int tn, s_begin, s_count;
    if (FOLD) {
        tn = blockIdx.x; s_begin = 0; s_count = g.P;
    } else {
        tn = blockIdx.x / g.P; s_begin = blockIdx.x - tn * g.P; s_count = 1;
    }
    const int64_t n0 = (int64_t)tn * ON;
    const int64_t Ks = g.K;
    const int nks = (int)((Ks + KB - 1) / KB);  // stages per shard
    const int total = s_count * nks;

    // ---- load cursor: stage t -> (shard, k stage).  Load instruction q
    // (= j*4 + wave) fills bytes [q KB, (q+1) KB) of the stage; lane takes
    // 16-byte unit idx = 64q + lane: row idx / CPR (W rows first, then X
    // rows), slot idx % CPR, which holds chunk slot ^ (row % 16).
    int ls = 0, lk = 0;
    auto issue = [&](int t) {
        if (t >= total) return;  // uniform
        const int shard = s_begin + ls;
        const int64_t kb = (int64_t)lk * KB;
        LDS_PTR(char) dst = lds + (t % NST) * STB;
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const int q = j * 4 + wave;
            const int idx = q * 64 + lane;
            const int row = idx / CPR, slot = idx % CPR;
            const int chunk = slot ^ (row & 15);
            int64_t k = kb + chunk * 8;
            // K tail: chunks past the shard's K are loaded from column 0 of
            // the row (in bounds) and zeroed after the fragment read.
            if (k >= Ks) k = 0;
            const __bf16 *src;
            if (row < BN) {
                int64_t n = n0 + (SWIGLU ? (row & 15) : row);
                if (n > g.N - 1) n = g.N - 1;
                if (SWIGLU && row >= 16) n += ex.up_off;   // the up row of the same unit
                src = (const __bf16 *)g.B + (int64_t)shard * g.b_shard + n * g.ldb + k;
            } else {
                int64_t m = row - BN;
                if (m > g.M - 1) m = g.M - 1;
                src = (const __bf16 *)g.A + (int64_t)shard * g.a_shard + m * g.lda + k;
            }
            // Written as an instruction the compiler does not track: its own
            // wait analysis would drain every load in flight before the next
            // LDS read (it cannot tell which stage a load writes), which
            // leaves no stage of lead; the waits the pipeline needs are the
            // explicit ones at the top of each stage.
            const uint32_t m0v = (uint32_t)(uintptr_t)(dst + q * 1024);
            asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                         :: "v"(src), "s"(m0v) : "memory", "m0");
        }
        if (++lk == nks) { lk = 0; ++ls; }
    };

#pragma unroll
    for (int t = 0; t < NST - 1; ++t) issue(t);

    f32x4 acc[NB][MB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float run[NB][MB];  // running fused sum, output mapping (see below)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) run[nb][mb] = 0.f;

    const int frow = lane & 15;   // fragment row
    const int fk = lane >> 4;     // fragment 8-column group
    int cs = 0, ck = 0;           // compute cursor (shard index, k stage)
    for (int t = 0; t < total; ++t) {
        // Stage t's loads were issued NST-1 stages ago; the loads of the
        // later stages issued since (NST-2 of them, fewer in the last stages,
        // where nothing is issued past the end) may stay in flight.
        const int later = total - 1 - t;
        if (later >= NST - 2) {
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPW * (NST - 2)) : "memory");
        } else {
#pragma unroll
            for (int r = 0; r < NST - 2; ++r)
                if (later == r) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPW * r) : "memory");
        }
        __syncthreads();
        issue(t + NST - 1);
        LDS_PTR(char) st = lds + (t % NST) * STB;
        const int64_t kb = (int64_t)ck * KB;
#pragma unroll
        for (int sub = 0; sub < SUBS; ++sub) {
            const int c = (sub * 4 + wave) * 4 + fk;  // chunk within the stage
            const bool valid = kb + c * 8 < Ks;
            bf16x8 wv[NB], xv[MB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                wv[nb] = *(LDS_PTR(bf16x8))(st + (nb * 16 + frow) * ROWB + ((c ^ frow) << 4));
                if (!valid) wv[nb] = bf16x8{};
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int xr = BN + mb * 16 + frow;
                xv[mb] = *(LDS_PTR(bf16x8))(st + xr * ROWB + ((c ^ (xr & 15)) << 4));
                if (!valid) xv[mb] = bf16x8{};
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[nb], xv[mb], acc[nb][mb], 0, 0, 0);
        }
        if (++ck < nks) continue;

        // ---- shard finished: add the four waves' partials in fixed order.
        // Output (n, m) of the tile sits in lane 16*(n/4) + m%16, register
        // n%4, block m/16 (16x16 D layout, W rows as the row operand).
        // Thread tid takes n = tid % 16, m = tid / 16 + 16*mb.
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            red[wave][nb][mb][lane] = acc[nb][mb];
            acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        __syncthreads();
        const int on = tid & 15, om = tid >> 4;
        const int src_lane = 16 * (on >> 2) + om, src_r = on & 3;
        const int shard = s_begin + cs;
        const __bf16 *bb = (const __bf16 *)ex.bias;
        if (SWIGLU) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                float gv = red[0][0][mb][src_lane][src_r];
                gv = gv + red[1][0][mb][src_lane][src_r];
                gv = gv + red[2][0][mb][src_lane][src_r];
                gv = gv + red[3][0][mb][src_lane][src_r];
                float uv = red[0][1][mb][src_lane][src_r];
                uv = uv + red[1][1][mb][src_lane][src_r];
                uv = uv + red[2][1][mb][src_lane][src_r];
                uv = uv + red[3][1][mb][src_lane][src_r];
                const int64_t m = om + 16 * mb, n = n0 + on;
                if (m < g.M && n < g.N) {
                    if (bb) {
                        const __bf16 *bs = bb + (int64_t)shard * ex.bias_shard;
                        gv = gv + (float)bs[n];
                        uv = uv + (float)bs[ex.up_off + n];
                    }
                    store_out<OUT>(g.C, (int64_t)shard * g.c_shard + m * g.ldc + n, silu_f32(gv) * uv);
                }
            }
        } else {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                float v = red[0][nb][mb][src_lane][src_r];
                v = v + red[1][nb][mb][src_lane][src_r];
                v = v + red[2][nb][mb][src_lane][src_r];
                v = v + red[3][nb][mb][src_lane][src_r];
                const int64_t m = om + 16 * mb, n = n0 + nb * 16 + on;
                if (FOLD) {
                    run[nb][mb] = cs == 0 ? v : run[nb][mb] + v;
                    if (cs == s_count - 1 && m < g.M && n < g.N) {
                        float y = run[nb][mb];
                        if (bb) y = y + (float)bb[n];     // row bias: once, after the fold
                        store_out<OUT>(f.Y, m * f.ldy + n, y);
                    }
                } else if (m < g.M && n < g.N) {
                    if (bb) v = v + (float)bb[(int64_t)shard * ex.bias_shard + n];
                    store_out<OUT>(g.C, (int64_t)shard * g.c_shard + m * g.ldc + n, v);
                }
            }
        }
        ck = 0;
        ++cs;
        // `red` is written again only after at least one more barrier.
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int NB, int MB, int KB, int NST, bool SWIGLU = false>
hipError_t launch_mb(const GemmArgs &g, int out_type, const FoldArgs *fold, const GemmExtra &ex,
                     hipStream_t s) {
    constexpr int ON = SWIGLU ? 16 : 16 * NB;
    const int64_t tn = (g.N + ON - 1) / ON;
    const int64_t blocks = fold ? tn : tn * g.P;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)blocks), block(SK_THREADS);
    FoldArgs f = fold ? *fold : FoldArgs{nullptr, 0, 0};
    if (SWIGLU) {
        if (fold) return hipErrorInvalidValue;
        if (out_type == OUT_BF16) gemm_skinny_kernel<NB, MB, KB, NST, OUT_BF16, false, SWIGLU><<<grid, block, 0, s>>>(g, f, ex);
        else gemm_skinny_kernel<NB, MB, KB, NST, OUT_F32, false, SWIGLU><<<grid, block, 0, s>>>(g, f, ex);
    } else if (fold) {
        if (out_type == OUT_BF16) gemm_skinny_kernel<NB, MB, KB, NST, OUT_BF16, true, false><<<grid, block, 0, s>>>(g, f, ex);
        else gemm_skinny_kernel<NB, MB, KB, NST, OUT_F32, true, false><<<grid, block, 0, s>>>(g, f, ex);
    } else {
        if (out_type == OUT_BF16) gemm_skinny_kernel<NB, MB, KB, NST, OUT_BF16, false, false><<<grid, block, 0, s>>>(g, f, ex);
        else gemm_skinny_kernel<NB, MB, KB, NST, OUT_F32, false, false><<<grid, block, 0, s>>>(g, f, ex);
    }
    return hipGetLastError();
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

bool gemm_skinny_supported(const GemmArgs &g, const GemmExtra *ex) {
    if (ex && ex->x_rows > 0) return false;
    return g.M >= 1 && g.M <= SKINNY_MAX_M && g.K > 0 && g.K % 8 == 0 && g.lda % 8 == 0 &&
           g.ldb % 8 == 0 && g.a_shard % 8 == 0 && g.b_shard % 8 == 0 &&
           aligned16(g.A) && aligned16(g.B);
}

hipError_t launch_gemm_skinny(const GemmArgs &g, int out_type, const FoldArgs *fold,
                              const GemmExtra *exp, hipStream_t s) {
    if (g.M == 0 || g.N == 0 || g.P == 0) return hipSuccess;
    GemmExtra ex{};
    if (exp) ex = *exp;
    if (ex.x_rows > 0) return hipErrorInvalidValue;
    // LDS per workgroup: NST * (16*NB + 16*MB) * KB * 2 bytes, plus the
    // cross-wave sums (4 * NB * MB KB).  Small stages let several workgroups share a CU, which
    // keeps more loads in flight when the grid is large (one workgroup per
    // 16 output columns and shard: three 16 KB stages, two in flight).  The
    // fused fold has a P times smaller grid: one workgroup per CU with 32
    // output columns and four 24 KB stages, three in flight (16 columns and
    // four 16 KB stages where 32 would leave CUs without one).  Measured with
    // M = 16, K = 8192, N = 28672 over 8 shards: column 82-83 us with 3 or 4
    // stages of 256 columns against 88-89 with 2; fused fold of 8 shards of
    // K = 3584, N = 8192: 82-83 us with 32 columns and 3-6 stages, 86-87 with
    // 16 columns and two 512-column stages; a later same-box sweep gave 86.6
    // us for this choice against 85.9 (32 columns, 3 stages), 89.6-90.8 (16
    // columns: 3 or 4 stages of 256, 2 of 512), 97.6 (32 columns, 2 stages of
    // 512) and 147.7 (64 columns: half the CUs idle); three later same-box
    // runs of 2-6 stages of 256 put 4 stages 2-7% ahead of 5 (6 stages 5% and
    // 2 stages 25% behind).  The gated unit streams 32 W rows (16 gate, 16
    // up) per workgroup with the column form's stages.
    if (ex.act == ACT_SWIGLU) {
        if (fold) return hipErrorInvalidValue;
        if (g.M <= 16) return launch_mb<2, 1, 256, 3, true>(g, out_type, fold, ex, s);   // 72 KB
        if (g.M <= 32) return launch_mb<2, 2, 256, 2, true>(g, out_type, fold, ex, s);   // 64 KB
        return launch_mb<2, 4, 256, 2, true>(g, out_type, fold, ex, s);                  // 96 KB
    }
    if (g.M <= 16) {
        // Fused fold: 32 output columns per workgroup where that still gives
        // every CU one, else 16.  Same box, 8 shards, us after a read-only
        // 1 GiB flush, 16 vs 32 columns: 4096 -> 4096 13.8 vs 16.3-16.8,
        // 8192 -> 4096 21.2-21.6 vs 26.0-26.1, 14336 -> 4096 31.8-32.2 vs
        // 38.6-39.4; bitwise equal.
        if (fold && g.N >= 32 * (int64_t)device_cu_count())
            return launch_mb<2, 1, 256, 4>(g, out_type, fold, ex, s);         // 96 KB
        if (fold) return launch_mb<1, 1, 256, 4>(g, out_type, fold, ex, s);   // 64 KB
        return launch_mb<1, 1, 256, 3>(g, out_type, fold, ex, s);             // 48 KB
    }
    // Above 16 tokens every workgroup re-reads its X rows from L2 with each
    // stage, so more W rows per workgroup share them (and no more 16-row X
    // blocks than M needs).  Same-box sweep, 8 shards, us for M = 24 / 32 /
    // 48 / 64, against 16 W rows per workgroup and 2 or 4 X blocks: column
    // 4096 -> 28672: 39.9 / 39.1 / 55.9 / 72.2 vs 53.1 / 51.9 / 108.1 / 116.0;
    // 8192 -> 10240: 33.8 / 35.2 / 43.0 / 67.8 vs 45.3 / 45.8 / 84.0 / 86.5;
    // 8192 -> 28672: 88.4 / 88.4 / 103.2 / 145.6 vs 124.4 / 125.5 / 216.2 /
    // 217.2; fused fold of 28672 -> 8192: 93.0 / 94.1 / 171.6 / 171.5 vs 119.8 /
    // 123.5 / 228.7 / 230.5.  All bitwise equal (each output's K blocks and
    // their order do not depend on the workgroup's shape).
    if (g.M <= 32) {
        if (fold) return launch_mb<4, 2, 256, 2>(g, out_type, fold, ex, s);   // 128 KB
        return launch_mb<2, 2, 256, 2>(g, out_type, fold, ex, s);             // 80 KB
    }
    if (fold) return launch_mb<2, 4, 128, 3>(g, out_type, fold, ex, s);       // 104 KB
    // Above 48 tokens the tile kernels' order of work is faster (same box, 8
    // shards, us after a read-only flush / warm, 64 tokens, skinny vs 128 x
    // 128 tiles: column 4096 -> 28672 79.8 / 75.1 vs 59.3 / 39.0, 8192 ->
    // 28672 146.1 / 146.9 vs 106.0 / 106.3; row partials + fold 14336 ->
    // 4096 50.7 / 45.8 vs 31.9 / 27.1), so no call reaches here with more.
    return launch_mb<4, 3, 256, 2>(g, out_type, fold, ex, s);                 // 160 KB
}

}  // namespace tpl
