// Row-parallel GEMM with the shard fold in registers, for prefill shapes
// ("模型并行", "Row parallel": Y = sum_i X_i W_i; the all-reduce of
// RowParallelLinearWithReplicateOutput done on device, in ascending shard
// order, as one fp32 add per shard).
//
// A workgroup owns one 256 (tokens) x 128 (output features) tile and walks
// the P shards in ascending order.  Shard i's partial X_i W_i^T is computed
// in 128 accumulator registers (2 x 4 v_mfma_f32_32x32x16_bf16 blocks per
// wave, the same instruction and the same K order as the partial GEMM), then
// added into a running fp32 sum held in another 128 registers:
//   run = p_0;  run = run + p_i  (i = 1 .. P-1);  Y = rne(run [+ bias]).
// These are the operations, in the order, of writing the P fp32 partials and
// folding them, so the result is bitwise equal to that unfused sequence; no
// partial reaches memory and no workspace is needed.  The tile is half as
// wide as the partial GEMM's (the running sum takes the other half of the
// register budget), so each K step moves 1.5x the operand bytes per flop;
// the gain is the 2 P M N x 4 bytes of partials that are neither written nor
// read back.
//
// Pipeline, as in the partial GEMM: global -> LDS with global_load_lds_dwordx4
// (16 bytes per lane), two stages of 64 K columns (48 KB each), 128-byte LDS
// rows with 16-byte chunk c of row r at slot c ^ ((r / 2) % 8); per K step
// four phases of 8 MFMAs with the next sub-step's 6 fragment reads and the
// global loads interleaved, the W part of the next step issued in phase 0,
// the X part of the step after it in phase 3 behind the step's one barrier.
// Persistent: one workgroup per CU walks an XCD-contiguous range of tiles,
// and the K pipeline runs across shard and tile boundaries.
#include "kernels.h"
#include <type_traits>

namespace tpl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T) __attribute__((address_space(3))) T *

constexpr int FM = 256;   // tile rows (tokens)
constexpr int FN = 128;   // tile columns (output features)
constexpr int FT = 256;   // threads
constexpr int FBK = 64;   // K columns per stage
constexpr int FGROUP = 4; // tile rows visited as a group

struct FoldSched {
    int tiles_m, tiles_n;
    int T;
    int xcd_split, per_xcd;
};

__device__ __forceinline__ void fold_decode(const FoldSched &ts, int t, int &tm, int &tn) {
    const int in_group = FGROUP * ts.tiles_n;
    const int first_m = (t / in_group) * FGROUP;
    const int gsz = min(ts.tiles_m - first_m, FGROUP);
    const int tr = t - (t / in_group) * in_group;
    tm = first_m + tr % gsz;
    tn = tr / gsz;
}

__device__ __forceinline__ int fold_tile_of(const FoldSched &ts, int q) {
    const int b = blockIdx.x;
    if (ts.xcd_split) {
        const int x = b & 7, lb = b >> 3;
        const int per = (ts.T + 7) >> 3;
        const int lo = x * per, hi = min(lo + per, ts.T);
        const int t = lo + lb + q * ts.per_xcd;
        return t < hi ? t : -1;
    }
    const int t = b + q * (int)gridDim.x;
    return t < ts.T ? t : -1;
}

// ro: where the folded tile goes (Y, ldy, the token slices of a
// reduce-scatter, the bias); its partials fields are unused.
template <bool SCAT>
__global__ __attribute__((amdgpu_flat_work_group_size(FT, FT), amdgpu_waves_per_eu(1, 1)))
void gemm_rowfold_kernel(GemmArgs g, FoldSched ts, ReduceArgs ro, int vec_store) {
    constexpr int ROWB = FBK * 2;          // 128 bytes per LDS row
    constexpr int CPR = FBK / 8;           // 16-byte chunks per row
    constexpr int RP = 256 / ROWB;         // rows per 256 bytes
    constexpr int OPX = FM * ROWB;         // X tile, 32 KB
    constexpr int OPW = FN * ROWB;         // W tile, 16 KB
    constexpr int STAGE = OPX + OPW;
    constexpr int RPI = 1024 / ROWB;       // rows per 1 KB load instruction
    constexpr int LX = OPX / 1024 / 4;     // X loads per wave per step
    constexpr int LW = OPW / 1024 / 4;     // W loads per wave per step
    constexpr int KS = FBK / 16;           // MFMA k-steps per stage
    constexpr int EPI_ROWB = 32 * 4 + 16;
    constexpr int EPI_WAVE = 32 * EPI_ROWB;
    static_assert(2 * STAGE + 4 * EPI_WAVE <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE + 4 * EPI_WAVE];
    LDS_PTR(char) lds = (LDS_PTR(char))smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    int ntiles = 0;
    while (fold_tile_of(ts, ntiles) >= 0) ++ntiles;
    if (ntiles == 0) return;
    const int nk = (int)(g.K / FBK);       // K steps per shard
    const int P = g.P;
    const int total = ntiles * P * nk;

    // ---- prefetch cursor: (tile pq, shard psh, step pkt), NST-1 = 1 step
    // ahead of the compute cursor; past the last step it stays there.
    int pq = 0, psh = 0, pkt = 0, pstep = 0;
    int64_t pm0 = 0, pn0 = 0;
    const char *pa = nullptr, *pb = nullptr;
    uint32_t aoff[LX], boff[LW];
    auto enter_tile = [&](int q) {
        int tm, tn;
        fold_decode(ts, fold_tile_of(ts, q), tm, tn);
        pm0 = (int64_t)tm * FM;
        pn0 = (int64_t)tn * FN;
        const int a_rows = (int)min<int64_t>(g.M - pm0, FM);
        const int b_rows = (int)min<int64_t>(g.N - pn0, FN);
#pragma unroll
        for (int j = 0; j < LX; ++j) {
            const int r = (j * 4 + wave) * RPI + lane / CPR;
            const int chunk = (lane % CPR) ^ ((r / RP) % CPR);
            const int ra = r < a_rows ? r : a_rows - 1;
            aoff[j] = (uint32_t)(((int64_t)ra * g.lda + chunk * 8) * 2);
        }
#pragma unroll
        for (int j = 0; j < LW; ++j) {
            const int r = (j * 4 + wave) * RPI + lane / CPR;
            const int chunk = (lane % CPR) ^ ((r / RP) % CPR);
            const int rb = r < b_rows ? r : b_rows - 1;
            boff[j] = (uint32_t)(((int64_t)rb * g.ldb + chunk * 8) * 2);
        }
    };
    auto set_bases = [&]() {
        pa = (const char *)((const __bf16 *)g.A + (int64_t)psh * g.a_shard + pm0 * g.lda);
        pb = (const char *)((const __bf16 *)g.B + (int64_t)psh * g.b_shard + pn0 * g.ldb);
    };
    // Loads [j0, j1) of the cursor's step into `stage`: 0..LX-1 fill the X
    // tile, LX..LX+LW-1 the W tile.
    auto issue_part = [&](int stage, int j0, int j1) {
        LDS_PTR(char) dst = lds + stage * STAGE;
        const int64_t kb = (int64_t)pkt * FBK * 2;
#pragma unroll
        for (int j = 0; j < LX + LW; ++j) {
            if (j < j0 || j >= j1) continue;
            if (j < LX)
                __builtin_amdgcn_global_load_lds((const void *)(pa + kb + aoff[j]),
                                                 (LDS_PTR(void))(dst + (j * 4 + wave) * 1024), 16, 0, 0);
            else
                __builtin_amdgcn_global_load_lds(
                    (const void *)(pb + kb + boff[j - LX]),
                    (LDS_PTR(void))(dst + OPX + ((j - LX) * 4 + wave) * 1024), 16, 0, 0);
        }
    };
    auto advance = [&]() {
        if (pstep + 1 < total) {
            ++pstep;
            if (++pkt == nk) {
                pkt = 0;
                if (++psh == P) {
                    psh = 0;
                    ++pq;
                    enter_tile(pq);
                }
                set_bases();
            }
        }
    };

    enter_tile(0);
    set_bases();
    issue_part(0, 0, LX + LW);
    advance();
    issue_part(1, 0, LX);

    // Fragment addressing (32x32x16 operands: lane reads row lane%32,
    // k-chunk 2*ks + lane/32).
    const int frow = lane & 31;
    const int fhalf = lane >> 5;
    const int fx = (frow / RP) % CPR;
    const int wrow_off = (wn * 64 + frow) * ROWB;
    const int xrow_off = (wm * 128 + frow) * ROWB;

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    bf16x8 wf[2][2], xf[2][4];
    {
        const int slot = ((0 + fhalf) ^ fx) << 4;
#pragma unroll
        for (int i = 0; i < 2; ++i) wf[0][i] = *(LDS_PTR(bf16x8))(lds + OPX + wrow_off + i * 32 * ROWB + slot);
#pragma unroll
        for (int j = 0; j < 4; ++j) xf[0][j] = *(LDS_PTR(bf16x8))(lds + xrow_off + j * 32 * ROWB + slot);
    }

    int it = 0;
    f32x16 acc[2][4], run[2][4];
    for (int q = 0; q < ntiles; ++q) {
        for (int sh = 0; sh < P; ++sh) {
            // One K step: KS phases of 8 MFMAs; the next sub-step's 6
            // fragment reads in slots 0-5; the W loads of the step after
            // this one in phase 0 (slots 4-7), the X loads of the step two
            // ahead in the last phase (one per slot), behind the barrier
            // that frees their stage.
            auto kstep = [&](auto first) __attribute__((always_inline)) {
                constexpr bool FIRST = decltype(first)::value;
                LDS_PTR(char) st = lds + (it & 1) * STAGE;
                LDS_PTR(char) st_next = lds + ((it + 1) & 1) * STAGE;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int cur = ks & 1, nx = cur ^ 1;
                    if (ks == KS - 1) {
                        __builtin_amdgcn_sched_barrier(0);
                        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                        __syncthreads();
                    }
                    LDS_PTR(char) rd = ks + 1 < KS ? st : st_next;
                    const int rks = ks + 1 < KS ? ks + 1 : 0;
                    const int slot = ((2 * rks + fhalf) ^ fx) << 4;
                    int j0 = LX + LW, j1 = LX + LW, s0 = 0;
                    if (ks == 0) { j0 = LX; j1 = LX + LW; s0 = 4; }     // W of step it+1
                    if (ks == KS - 1) { j0 = 0; j1 = LX; s0 = 0; }      // X of step it+2
                    const int lstage = ks == 0 ? (it + 1) & 1 : it & 1;
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        __builtin_amdgcn_sched_barrier(0);
                        // Order (i, j): the first four MFMAs touch all six
                        // fragments.
                        const int i = u & 1, j = (u + (u >> 2)) & 3;
                        if (FIRST && ks == 0)   // the shard's first product of each block: C = 0
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cur][i], xf[cur][j],
                                                                                f32x16{}, 0, 0, 0);
                        else
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cur][i], xf[cur][j],
                                                                                acc[i][j], 0, 0, 0);
                        if (u < 6) {
                            if (u < 2)
                                wf[nx][u] = *(LDS_PTR(bf16x8))(rd + OPX + wrow_off + u * 32 * ROWB + slot);
                            else
                                xf[nx][u - 2] = *(LDS_PTR(bf16x8))(rd + xrow_off + (u - 2) * 32 * ROWB + slot);
                        }
                        const int la = j0 + (u - s0);
                        const bool ld = u >= s0 && la < j1;
                        if (ld) issue_part(lstage, la, la + 1);
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // MFMA
                        if (u < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
                        if (ld) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // VMEM
                    }
                    if (ks == 0) {
                        __builtin_amdgcn_sched_barrier(0);
                        advance();
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            };
            kstep(std::true_type{});
            ++it;
            for (int kt = 1; kt < nk; ++kt, ++it) kstep(std::false_type{});
            // The fold: one fp32 add per shard, ascending.
            if (sh == 0) {
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) run[i][j] = acc[i][j];
            } else {
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) run[i][j] = run[i][j] + acc[i][j];
            }
        }

        // ---- epilogue: run (+ bias) -> bf16.  Each 32x32 block goes
        // through this wave's LDS area, written in its MFMA layout (lane:
        // token lane%32, four consecutive features per register group) and
        // read back row-contiguous: lane holds 8 consecutive features of one
        // token row, 16-byte stores.
        int tm, tn;
        fold_decode(ts, fold_tile_of(ts, q), tm, tn);
        const int64_t tm_w = (int64_t)tm * FM + wm * 128, tn_w = (int64_t)tn * FN + wn * 64;
        LDS_PTR(char) ep = lds + 2 * STAGE + wave * EPI_WAVE;
        const int lr = lane >> 2, lc = 8 * (lane & 3);
        const __bf16 *bias = (const __bf16 *)ro.bias;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            float bv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int64_t n = tn_w + i * 32 + lc + e;
                bv[e] = bias && n < g.N ? (float)bias[n] : 0.0f;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const f32x4 v = {run[i][j][4 * r4], run[i][j][4 * r4 + 1],
                                     run[i][j][4 * r4 + 2], run[i][j][4 * r4 + 3]};
                    *(LDS_PTR(f32x4))(ep + frow * EPI_ROWB + (8 * r4 + 4 * fhalf) * 4) = v;
                }
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    LDS_PTR(char) rp = ep + (pp * 16 + lr) * EPI_ROWB + lc * 4;
                    const f32x4 a0 = *(LDS_PTR(f32x4))rp, a1 = *(LDS_PTR(f32x4))(rp + 16);
                    float v[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                    const int64_t m = tm_w + j * 32 + pp * 16 + lr, n = tn_w + i * 32 + lc;
                    if (m >= g.M) continue;
                    bf16x8 hv;
#pragma unroll
                    for (int e = 0; e < 8; ++e) hv[e] = (__bf16)(bias ? v[e] + bv[e] : v[e]);
                    __bf16 *row;
                    if (SCAT) {
                        const int64_t sl = m / ro.slice_rows, rr = m - sl * ro.slice_rows;
                        row = ro.use_slices ? (__bf16 *)ro.y_slice[sl] + rr * ro.ldy
                                            : (__bf16 *)ro.Y + sl * ro.slice_stride + rr * ro.ldy;
                    } else {
                        row = (__bf16 *)ro.Y + m * ro.ldy;
                    }
                    if (vec_store && n + 8 <= g.N) {
                        __builtin_nontemporal_store(hv, (bf16x8 *)(row + n));
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (n + e < g.N) row[n + e] = hv[e];
                    }
                }
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }


}  // namespace

bool gemm_rowfold_supported(const GemmArgs &g, const ReduceArgs &ro) {
    const bool small_rows = (int64_t)FM * g.lda * 2 < (1ll << 31) &&
                            (int64_t)FN * g.ldb * 2 < (1ll << 31);
    if (!(g.K > 0 && g.K % FBK == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 && g.a_shard % 8 == 0 &&
          g.b_shard % 8 == 0 && aligned16(g.A) && aligned16(g.B) && small_rows))
        return false;
    // A reduce-scatter tile must not span two token slices.
    if (ro.slice_rows < g.M && ro.slice_rows % FM != 0) return false;
    return true;
}

hipError_t launch_gemm_rowfold(const GemmArgs &g, const ReduceArgs &ro, hipStream_t s) {
    if (g.M == 0 || g.N == 0 || g.P == 0) return hipSuccess;
    const int64_t tm = (g.M + FM - 1) / FM, tn = (g.N + FN - 1) / FN;
    const int64_t T = tm * tn;
    if (T > 0x7FFFFFFFll) return hipErrorInvalidConfiguration;
    FoldSched ts;
    ts.tiles_m = (int)tm;
    ts.tiles_n = (int)tn;
    ts.T = (int)T;
    const int cus = device_cu_count();
    const int grid = (int)(T < cus ? T : cus);
    ts.xcd_split = (grid == cus && cus % 8 == 0 && T >= cus) ? 1 : 0;
    ts.per_xcd = grid / 8;
    bool vec = ro.ldy % 8 == 0;
    // Slice addressing whenever the output is split into slices or given as
    // slice allocations (with one slice, P = 1, slice 0 is the whole output
    // and ro.Y is not set).
    const bool scat = ro.use_slices || ro.slice_rows < g.M;
    if (scat && ro.use_slices) {
        for (int64_t j = 0; j * ro.slice_rows < g.M; ++j) vec = vec && aligned16(ro.y_slice[j]);
    } else {
        vec = vec && aligned16(ro.Y) && (!scat || ro.slice_stride % 8 == 0);
    }
    if (scat)
        gemm_rowfold_kernel<true><<<dim3(grid), dim3(FT), 0, s>>>(g, ts, ro, vec ? 1 : 0);
    else
        gemm_rowfold_kernel<false><<<dim3(grid), dim3(FT), 0, s>>>(g, ts, ro, vec ? 1 : 0);
    return hipGetLastError();
}

}  // namespace tpl
