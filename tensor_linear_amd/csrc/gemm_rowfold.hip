// Row-parallel GEMM with the shard fold in registers, for prefill shapes
// ("模型并行", "Row parallel": Y = sum_i X_i W_i; the all-reduce of
// RowParallelLinearWithReplicateOutput done on device, in ascending shard
// order, as one fp32 add per shard).
//
// A workgroup owns one 256 (tokens) x 128 (output features) tile and walks
// the P shards in ascending order.  Shard i's partial X_i W_i^T is computed
// in 128 accumulator registers per lane (4 waves in a 2x2 grid, each a
// 128 x 64 block of 8 x 4 v_mfma_f32_16x16x32_bf16 blocks, the instruction
// and K order of the partial GEMM), then added into a running fp32 sum held
// in another 128 registers:
//   run = p_0;  run = run + p_i  (i = 1 .. P-1);  Y = rne(run [+ bias]).
// These are the operations, in the order, of writing the P fp32 partials and
// folding them, so the result is bitwise equal to that unfused sequence; no
// partial reaches memory and no workspace is needed.  The tile is half as
// wide as the partial GEMM's (the running sum takes the registers the other
// half of the accumulators would), so each K step moves 1.5x the operand
// bytes per flop; the gain is the 2 P M N x 4 bytes of partials that are
// neither written nor read back.
//
// Pipeline: global -> LDS with global_load_lds_dwordx4 (1 KB per wave
// instruction), three stages of 64 K columns for both operands (3 x (32 +
// 16) KB = 144 KB), 128-byte LDS rows with 16-byte chunk c of row r at slot
// c ^ ((r / 2) % 8).  Step it+2's 12 loads per wave go out in the first
// three quarters of step it, one every 4th MFMA, into the stage step it-1
// freed.  Per K step 4 quarters of 16 MFMAs (a 4 x 4 group of W x X blocks):
//   q0 W0-3 x X0-3, q1 W0-3 x X4-7 on substep 0, q2, q3 the same on
//   substep 1;
// fragment reads: q0 X4-7 (substep 0) and W0-1 (1), q1 W2-3 and X0-3 (1),
// q2 X4-7 (1); then the step's one barrier; q3 the next step's substep-0
// W0-3 and X0-3, interleaved so that q0 can start on the first pair.
// Persistent: one workgroup per CU walks an XCD-contiguous range of tiles,
// and the K pipeline runs across shard and tile boundaries.
//
// Launches with fewer tiles than CUs take an eight-wave form of the same
// tile (gemm_rowfold8_kernel below): two waves per SIMD, so one issues its
// MFMAs while the other waits on its reads and loads.
#include "kernels.h"
#include <type_traits>

namespace tpl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T) __attribute__((address_space(3))) T *

constexpr int FM = 256;   // tile rows (tokens)
constexpr int FN = 128;   // tile columns (output features)
constexpr int FT = 256;   // threads
constexpr int FT8 = 512;  // threads of the eight-wave form
constexpr int FW8 = FT8 / 64;
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

// q0's MFMA order: the next step's fragments arrive X0, W0, X1, W1, ...;
// (W block, X block) pairs in the order they become ready.
__device__ __forceinline__ constexpr int q0_w(int u) {
    return u < 4 ? (u >> 1) : (u < 9 ? (u < 6 ? u - 4 : 2) : (u < 12 ? u - 9 : 3));
}
__device__ __forceinline__ constexpr int q0_x(int u) {
    return u < 4 ? (u & 1) : (u < 9 ? (u < 6 ? 2 : u - 6) : (u < 12 ? 3 : u - 12));
}

// ro: where the folded tile goes (Y, ldy, the token slices of a
// reduce-scatter, the bias); its partials fields are unused.
template <bool SCAT>
__global__ __attribute__((amdgpu_flat_work_group_size(FT, FT), amdgpu_waves_per_eu(1, 1)))
void gemm_rowfold_kernel(GemmArgs g, FoldSched ts, ReduceArgs ro, int vec_store) {
    constexpr int ROWB = FBK * 2;          // 128 bytes per LDS row
    constexpr int OPX = FM * ROWB;         // X stage, 32 KB
    constexpr int OPW = FN * ROWB;         // W stage, 16 KB
    constexpr int W_BASE = 3 * OPX;        // three X stages, then three W stages
    constexpr int LX = OPX / 1024 / 4;     // X loads per wave per step (8)
    constexpr int LW = OPW / 1024 / 4;     // W loads per wave per step (4)
    __shared__ __attribute__((aligned(1024))) char smem[3 * OPX + 3 * OPW];
    LDS_PTR(char) lds = (LDS_PTR(char))smem;
    const uint32_t lds_u = (uint32_t)(uintptr_t)lds;

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

    // ---- load cursor: (tile pq, shard psh, step pkt), two steps ahead of
    // the compute; past the last step it stays there, so later issues reload
    // the last step into stages that are not read again.
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
            const int r = (j * 4 + wave) * 8 + lane / 8;
            const int chunk = (lane % 8) ^ ((r / 2) % 8);
            const int ra = r < a_rows ? r : a_rows - 1;
            aoff[j] = (uint32_t)(((int64_t)ra * g.lda + chunk * 8) * 2);
        }
#pragma unroll
        for (int j = 0; j < LW; ++j) {
            const int r = (j * 4 + wave) * 8 + lane / 8;
            const int chunk = (lane % 8) ^ ((r / 2) % 8);
            const int rb = r < b_rows ? r : b_rows - 1;
            boff[j] = (uint32_t)(((int64_t)rb * g.ldb + chunk * 8) * 2);
        }
    };
    auto set_bases = [&]() {
        pa = (const char *)((const __bf16 *)g.A + (int64_t)psh * g.a_shard + pm0 * g.lda);
        pb = (const char *)((const __bf16 *)g.B + (int64_t)psh * g.b_shard + pn0 * g.ldb);
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
    // One 1 KB DMA load, issued as an instruction the compiler does not
    // track (its own wait analysis cannot tell which stage a DMA writes);
    // the waits the pipeline needs are written out below.
    auto dma = [&](const char *base, uint32_t voff, uint32_t lds_addr) __attribute__((always_inline)) {
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                     :: "v"(voff), "s"(base), "s"(lds_addr) : "memory", "m0");
    };
    // Load l (0..11) of the cursor's step into stage `slot`: 0..7 the X
    // tile, 8..11 the W tile.
    auto load = [&](int slot, int l) __attribute__((always_inline)) {
        if (l < LX)
            dma(pa + (int64_t)pkt * 128, aoff[l], lds_u + slot * OPX + (l * 4 + wave) * 1024);
        else
            dma(pb + (int64_t)pkt * 128, boff[l - LX],
                lds_u + W_BASE + slot * OPW + ((l - LX) * 4 + wave) * 1024);
    };

    // Prologue: steps 0 and 1 into stages 0 and 1.
    enter_tile(0);
    set_bases();
#pragma unroll
    for (int l = 0; l < LX + LW; ++l) load(0, l);
    advance();
#pragma unroll
    for (int l = 0; l < LX + LW; ++l) load(1, l);
    advance();
    asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    asm volatile("s_barrier" ::: "memory");

    // Fragments (16 rows x 32 k): lane reads row lane%16 of its block,
    // 16-byte k-chunk 4*h + lane/16 of substep h.  fr[h][0..3] W blocks
    // (output features 16i.. of the wave's 64), fr[h][4..11] X blocks
    // (tokens 16j.. of the wave's 128).
    const int frow = lane & 15;
    const int fq = lane >> 4;
    const int fx = (frow / 2) % 8;
    const uint32_t wrow_off = (wn * 64 + frow) * ROWB;
    const uint32_t xrow_off = (wm * 128 + frow) * ROWB;
    auto frag_addr = [&](int stage, int f, int h) -> uint32_t {
        const uint32_t slot = (uint32_t)(((4 * h + fq) ^ fx) << 4);
        if (f < 4) return W_BASE + stage * OPW + wrow_off + f * 16 * ROWB + slot;
        return stage * OPX + xrow_off + (f - 4) * 16 * ROWB + slot;
    };
    bf16x8 fr[2][12];
    auto read_frag = [&](int h, int f, uint32_t addr) __attribute__((always_inline)) {
        fr[h][f] = *(LDS_PTR(bf16x8))(lds + addr);
    };
#pragma unroll
    for (int f = 0; f < 8; ++f) read_frag(0, f, frag_addr(0, f, 0));

    int s0 = 0;                 // stage of the current step (step index % 3)
    bool drained = true;        // no epilogue store is in flight
    f32x4 acc[4][8], run[4][8];
    for (int q = 0; q < ntiles; ++q) {
        for (int sh = 0; sh < P; ++sh) {
            auto kstep = [&](auto first) __attribute__((always_inline)) {
                constexpr bool FIRST = decltype(first)::value;
                const int s1 = s0 == 2 ? 0 : s0 + 1;   // stage of step it+1
                const int s2 = s1 == 2 ? 0 : s1 + 1;   // stage of step it+2 (= it-1's)
#pragma unroll
                for (int qr = 0; qr < 4; ++qr) {
                    if (qr == 3) {
                        __builtin_amdgcn_sched_barrier(0);
                        // Step it+1's loads (issued in step it-1) have
                        // landed; step it+2's 12 may stay in flight.  This
                        // wave's reads of step it's stage are done before
                        // anyone's loads may overwrite it (two steps on).
                        // After an epilogue its stores are in flight too,
                        // and a store may complete before an older load:
                        // then wait for all.
                        if (drained)
                            asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)" ::: "memory");
                        else
                            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
                        drained = true;
                        asm volatile("s_barrier" ::: "memory");
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    const int h = qr >> 1;
#pragma unroll
                    for (int u = 0; u < 16; ++u) {
                        __builtin_amdgcn_sched_barrier(0);
                        int i, j;
                        if (qr == 0) {
                            i = q0_w(u);
                            j = q0_x(u);
                        } else {
                            i = u & 3;
                            j = (qr & 1) * 4 + (u >> 2);
                        }
                        if (FIRST && h == 0)   // the shard's first product of each block: C = 0
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[0][i], fr[0][4 + j], f32x4{}, 0, 0, 0);
                        else
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[h][i], fr[h][4 + j], acc[i][j], 0, 0, 0);
                        // fragment reads
                        bool rd = false;
                        if (qr == 0 && (u & 1) == 0 && u < 12) {
                            const int k = u >> 1;   // 0..5
                            if (k < 4) read_frag(0, 8 + k, frag_addr(s0, 8 + k, 0));   // X4-7 substep 0
                            else read_frag(1, k - 4, frag_addr(s0, k - 4, 1));         // W0-1 substep 1
                            rd = true;
                        } else if (qr == 1 && (u & 1) == 0 && u < 12) {
                            const int k = u >> 1;
                            if (k < 2) read_frag(1, 2 + k, frag_addr(s0, 2 + k, 1));   // W2-3 substep 1
                            else read_frag(1, 4 + (k - 2), frag_addr(s0, 4 + (k - 2), 1));   // X0-3
                            rd = true;
                        } else if (qr == 2 && (u & 3) == 0) {
                            const int k = u >> 2;
                            read_frag(1, 8 + k, frag_addr(s0, 8 + k, 1));             // X4-7 substep 1
                            rd = true;
                        } else if (qr == 3 && (u & 1) == 0) {
                            const int k = u >> 1;   // X0, W0, X1, W1, ... of step it+1
                            const int f = (k & 1) ? (k >> 1) : 4 + (k >> 1);
                            read_frag(0, f, frag_addr(s1, f, 0));
                            rd = true;
                        }
                        // step it+2's loads, one every 4th MFMA in q0-q2
                        const bool ld = qr < 3 && (u & 3) == 1;
                        if (ld) load(s2, qr * 4 + (u >> 2));
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                        if (rd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    if (qr == 2) advance();
                }
                __builtin_amdgcn_sched_barrier(0);
                s0 = s1;
            };
            kstep(std::true_type{});
            for (int kt = 1; kt < nk; ++kt) kstep(std::false_type{});
            // The fold: one fp32 add per shard, ascending.
            if (sh == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 8; ++j) run[i][j] = acc[i][j];
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 8; ++j) run[i][j] = run[i][j] + acc[i][j];
            }
        }

        // ---- epilogue: run (+ bias) -> bf16.  run[i][j][r] = Y[m = 16j +
        // lane%16][n = 16i + 4*(lane/16) + r] of the wave's block.  32 rows x
        // 64 columns at a time go through this wave's 1 KB chunks w + 4c
        // (c = 0..7) of the X stage of the tile's last step (read by everyone
        // before that step's barrier; only this wave's own later loads write
        // these chunks): staging row r of 256 bytes at chunk r/4, offset
        // (r%4)*256, 16-byte slot s at s ^ (r % 16).  Each lane then holds 8
        // consecutive features of one row: a row of 64 features leaves as one
        // 128-byte line.
        __builtin_amdgcn_sched_barrier(0);
        int tm, tn;
        fold_decode(ts, fold_tile_of(ts, q), tm, tn);
        const int es = s0 == 0 ? 2 : s0 - 1;
        LDS_PTR(char) ep = lds + es * OPX + wave * 1024;
        auto st_addr = [&](int r, int s) -> LDS_PTR(char) {
            return ep + (r >> 2) * 4096 + (r & 3) * 256 + ((s ^ (r & 15)) << 4);
        };
        const int64_t m_t = (int64_t)tm * FM, tm_w = m_t + wm * 128, tn_w = (int64_t)tn * FN + wn * 64;
        __bf16 *ybase;   // row m_t of the output (tile rows never span two slices)
        if (SCAT) {
            const int64_t sl = m_t / ro.slice_rows, rr = m_t - sl * ro.slice_rows;
            ybase = ro.use_slices ? (__bf16 *)ro.y_slice[sl] + rr * ro.ldy
                                  : (__bf16 *)ro.Y + sl * ro.slice_stride + rr * ro.ldy;
        } else {
            ybase = (__bf16 *)ro.Y + m_t * ro.ldy;
        }
        const __bf16 *bias = (const __bf16 *)ro.bias;
        const int c8 = lane & 7;
        const int64_t ncol = tn_w + c8 * 8;
        float bv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) bv[e] = bias && ncol + e < g.N ? (float)bias[ncol + e] : 0.0f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {        // rows 32jj.. of the wave
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int bj = 0; bj < 2; ++bj)
#pragma unroll
                for (int bi = 0; bi < 4; ++bi)
                    *(LDS_PTR(f32x4))st_addr(bj * 16 + frow, bi * 4 + fq) = run[bi][2 * jj + bj];
            f32x4 a0[4], a1[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int rr = p * 8 + (lane >> 3);
                a0[p] = *(LDS_PTR(f32x4))st_addr(rr, 2 * c8);
                a1[p] = *(LDS_PTR(f32x4))st_addr(rr, 2 * c8 + 1);
            }
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int rr = p * 8 + (lane >> 3);
                const int64_t m = tm_w + jj * 32 + rr;
                if (m >= g.M) continue;
                float v[8] = {a0[p][0], a0[p][1], a0[p][2], a0[p][3], a1[p][0], a1[p][1], a1[p][2], a1[p][3]};
                bf16x8 hv;
#pragma unroll
                for (int e = 0; e < 8; ++e) hv[e] = (__bf16)(bias ? v[e] + bv[e] : v[e]);
                __bf16 *row = ybase + (m - m_t) * ro.ldy;
                if (vec_store && ncol + 8 <= g.N) {
                    __builtin_nontemporal_store(hv, (bf16x8 *)(row + ncol));
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (ncol + e < g.N) row[ncol + e] = hv[e];
                }
            }
        }
        drained = false;
    }
    // No DMA load may still be writing LDS when the workgroup ends.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// The eight-wave form, for launches with fewer tiles than CUs: two waves per
// SIMD, each a 64 x 64 block of 4 x 4 MFMA blocks (64 accumulator and 64
// running-sum registers, within the 256 that two waves per SIMD leave each).
// The same products, in the same K order per output, and the same fold as
// the four-wave form.  Per K step each wave issues 32 MFMAs in two substeps
// of 32 K: during substep 0 it reads its substep-1 fragments and issues all 6
// of step it+2's loads (4 of the X tile, then 2 of the W tile) into the stage
// step it-1 freed; then the step's one barrier; during substep 1 it reads the
// next step's substep-0 fragments.  The epilogue stages 16 rows x 64 columns
// at a time through the wave's 4 chunks of the last step's X stage.
template <bool SCAT>
__global__ __attribute__((amdgpu_flat_work_group_size(FT8, FT8), amdgpu_waves_per_eu(2, 2)))
void gemm_rowfold8_kernel(GemmArgs g, FoldSched ts, ReduceArgs ro, int vec_store) {
    constexpr int ROWB = FBK * 2;          // 128 bytes per LDS row
    constexpr int OPX = FM * ROWB;         // X stage, 32 KB
    constexpr int OPW = FN * ROWB;         // W stage, 16 KB
    constexpr int W_BASE = 3 * OPX;        // three X stages, then three W stages
    constexpr int LX = OPX / 1024 / FW8;    // X loads per wave per step (4)
    constexpr int LW = OPW / 1024 / FW8;    // W loads per wave per step (2)
    __shared__ __attribute__((aligned(1024))) char smem[3 * OPX + 3 * OPW];
    LDS_PTR(char) lds = (LDS_PTR(char))smem;
    const uint32_t lds_u = (uint32_t)(uintptr_t)lds;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;   // 64 tokens x 64 features each

    int ntiles = 0;
    while (fold_tile_of(ts, ntiles) >= 0) ++ntiles;
    if (ntiles == 0) return;
    const int nk = (int)(g.K / FBK);       // K steps per shard
    const int P = g.P;
    const int total = ntiles * P * nk;

    // ---- load cursor: (tile pq, shard psh, step pkt), two steps ahead of
    // the compute; past the last step it stays there, so later issues reload
    // the last step into stages that are not read again.
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
            const int r = (j * FW8 + wave) * 8 + lane / 8;
            const int chunk = (lane % 8) ^ ((r / 2) % 8);
            const int ra = r < a_rows ? r : a_rows - 1;
            aoff[j] = (uint32_t)(((int64_t)ra * g.lda + chunk * 8) * 2);
        }
#pragma unroll
        for (int j = 0; j < LW; ++j) {
            const int r = (j * FW8 + wave) * 8 + lane / 8;
            const int chunk = (lane % 8) ^ ((r / 2) % 8);
            const int rb = r < b_rows ? r : b_rows - 1;
            boff[j] = (uint32_t)(((int64_t)rb * g.ldb + chunk * 8) * 2);
        }
    };
    auto set_bases = [&]() {
        pa = (const char *)((const __bf16 *)g.A + (int64_t)psh * g.a_shard + pm0 * g.lda);
        pb = (const char *)((const __bf16 *)g.B + (int64_t)psh * g.b_shard + pn0 * g.ldb);
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
    // One 1 KB DMA load, issued as an instruction the compiler does not
    // track (its own wait analysis cannot tell which stage a DMA writes);
    // the waits the pipeline needs are written out below.
    auto dma = [&](const char *base, uint32_t voff, uint32_t lds_addr) __attribute__((always_inline)) {
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                     :: "v"(voff), "s"(base), "s"(lds_addr) : "memory", "m0");
    };
    // Load l (0..5) of the cursor's step into stage `slot`: 0..3 the X tile
    // (1 KB chunks 8l + wave), 4..5 the W tile.
    auto load = [&](int slot, int l) __attribute__((always_inline)) {
        if (l < LX)
            dma(pa + (int64_t)pkt * 128, aoff[l], lds_u + slot * OPX + (l * FW8 + wave) * 1024);
        else
            dma(pb + (int64_t)pkt * 128, boff[l - LX],
                lds_u + W_BASE + slot * OPW + ((l - LX) * FW8 + wave) * 1024);
    };

    // Prologue: steps 0 and 1 into stages 0 and 1.
    enter_tile(0);
    set_bases();
#pragma unroll
    for (int l = 0; l < LX + LW; ++l) load(0, l);
    advance();
#pragma unroll
    for (int l = 0; l < LX + LW; ++l) load(1, l);
    advance();
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(LX + LW) : "memory");
    asm volatile("s_barrier" ::: "memory");

    // Fragments (16 rows x 32 k): lane reads row lane%16 of its block,
    // 16-byte k-chunk 4*h + lane/16 of substep h.  fr[h][0..3] W blocks
    // (output features 16i.. of the wave's 64), fr[h][4..7] X blocks
    // (tokens 16j.. of the wave's 64).
    const int frow = lane & 15;
    const int fq = lane >> 4;
    const int fx = (frow / 2) % 8;
    const uint32_t wrow_off = (wn * 64 + frow) * ROWB;
    const uint32_t xrow_off = (wm * 64 + frow) * ROWB;
    auto frag_addr = [&](int stage, int f, int h) -> uint32_t {
        const uint32_t slot = (uint32_t)(((4 * h + fq) ^ fx) << 4);
        if (f < 4) return W_BASE + stage * OPW + wrow_off + f * 16 * ROWB + slot;
        return stage * OPX + xrow_off + (f - 4) * 16 * ROWB + slot;
    };
    bf16x8 fr[2][8];
    auto read_frag = [&](int h, int f, uint32_t addr) __attribute__((always_inline)) {
        fr[h][f] = *(LDS_PTR(bf16x8))(lds + addr);
    };
#pragma unroll
    for (int f = 0; f < 8; ++f) read_frag(0, f, frag_addr(0, f, 0));

    int s0 = 0;                 // stage of the current step (step index % 3)
    bool drained = true;        // no epilogue store is in flight
    f32x4 acc[4][4], run[4][4];
    for (int q = 0; q < ntiles; ++q) {
        for (int sh = 0; sh < P; ++sh) {
            auto kstep = [&](auto first) __attribute__((always_inline)) {
                constexpr bool FIRST = decltype(first)::value;
                const int s1 = s0 == 2 ? 0 : s0 + 1;   // stage of step it+1
                const int s2 = s1 == 2 ? 0 : s1 + 1;   // stage of step it+2 (= it-1's)
                // substep 0: the substep-1 fragments, step it+2's loads
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    __builtin_amdgcn_sched_barrier(0);
                    const int i = u & 3, j = u >> 2;
                    if (FIRST)   // the shard's first product of each block: C = 0
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[0][i], fr[0][4 + j], f32x4{}, 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[0][i], fr[0][4 + j], acc[i][j], 0, 0, 0);
                    const bool rd = (u & 1) == 0;
                    if (rd) read_frag(1, u >> 1, frag_addr(s0, u >> 1, 1));
                    // step it+2's six loads, X then W, at MFMAs 1, 3, 6, 9, 11, 14
                    const int li = u == 1 ? 0 : u == 3 ? 1 : u == 6 ? 2 : u == 9 ? 3 : u == 11 ? 4 : u == 14 ? 5 : -1;
                    if (li >= 0) load(s2, li);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    if (rd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
                }
                __builtin_amdgcn_sched_barrier(0);
                // Step it+1's loads (issued in step it-1) have landed; step
                // it+2's 6 may stay in flight.  This wave's reads of
                // step it's stage are done before anyone's loads may
                // overwrite it (two steps on).  After an epilogue its stores
                // are in flight too, and a store may complete before an
                // older load: then wait for all.
                if (drained)
                    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" :: "n"(LX + LW) : "memory");
                else
                    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
                drained = true;
                asm volatile("s_barrier" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                // substep 1: the next step's substep-0 fragments (W0-3, then
                // X0-3, the order its first MFMAs use them)
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    __builtin_amdgcn_sched_barrier(0);
                    const int i = u & 3, j = u >> 2;
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[1][i], fr[1][4 + j], acc[i][j], 0, 0, 0);
                    const bool rd = (u & 1) == 0;
                    if (rd) read_frag(0, u >> 1, frag_addr(s1, u >> 1, 0));
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    if (rd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
                }
                __builtin_amdgcn_sched_barrier(0);
                advance();
                s0 = s1;
            };
            kstep(std::true_type{});
            for (int kt = 1; kt < nk; ++kt) kstep(std::false_type{});
            // The fold: one fp32 add per shard, ascending.
            if (sh == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) run[i][j] = acc[i][j];
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) run[i][j] = run[i][j] + acc[i][j];
            }
        }

        // ---- epilogue: run (+ bias) -> bf16.  run[i][j][r] = Y[m = 16j +
        // lane%16][n = 16i + 4*(lane/16) + r] of the wave's block.  16 rows x
        // 64 columns at a time go through this wave's 1 KB chunks w + 8c
        // (c = 0..3) of the X stage of the tile's last step (read by everyone
        // before that step's barrier; only this wave's own later loads write
        // these chunks): staging row r of 256 bytes at chunk r/4, offset
        // (r%4)*256, 16-byte slot s at s ^ (r % 16).  Each lane then holds 8
        // consecutive features of one row: a row of 64 features leaves as one
        // 128-byte line.
        __builtin_amdgcn_sched_barrier(0);
        int tm, tn;
        fold_decode(ts, fold_tile_of(ts, q), tm, tn);
        const int es = s0 == 0 ? 2 : s0 - 1;
        LDS_PTR(char) ep = lds + es * OPX + wave * 1024;
        auto st_addr = [&](int r, int s) -> LDS_PTR(char) {
            return ep + (r >> 2) * (FW8 * 1024) + (r & 3) * 256 + ((s ^ (r & 15)) << 4);
        };
        const int64_t m_t = (int64_t)tm * FM, tm_w = m_t + wm * 64, tn_w = (int64_t)tn * FN + wn * 64;
        __bf16 *ybase;   // row m_t of the output (tile rows never span two slices)
        if (SCAT) {
            const int64_t sl = m_t / ro.slice_rows, rr = m_t - sl * ro.slice_rows;
            ybase = ro.use_slices ? (__bf16 *)ro.y_slice[sl] + rr * ro.ldy
                                  : (__bf16 *)ro.Y + sl * ro.slice_stride + rr * ro.ldy;
        } else {
            ybase = (__bf16 *)ro.Y + m_t * ro.ldy;
        }
        const __bf16 *bias = (const __bf16 *)ro.bias;
        const int c8 = lane & 7;
        const int64_t ncol = tn_w + c8 * 8;
        float bv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) bv[e] = bias && ncol + e < g.N ? (float)bias[ncol + e] : 0.0f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {        // rows 16jj.. of the wave
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int bi = 0; bi < 4; ++bi)
                *(LDS_PTR(f32x4))st_addr(frow, bi * 4 + fq) = run[bi][jj];
            f32x4 a0[2], a1[2];
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int rr = p * 8 + (lane >> 3);
                a0[p] = *(LDS_PTR(f32x4))st_addr(rr, 2 * c8);
                a1[p] = *(LDS_PTR(f32x4))st_addr(rr, 2 * c8 + 1);
            }
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int rr = p * 8 + (lane >> 3);
                const int64_t m = tm_w + jj * 16 + rr;
                if (m >= g.M) continue;
                float v[8] = {a0[p][0], a0[p][1], a0[p][2], a0[p][3], a1[p][0], a1[p][1], a1[p][2], a1[p][3]};
                bf16x8 hv;
#pragma unroll
                for (int e = 0; e < 8; ++e) hv[e] = (__bf16)(bias ? v[e] + bv[e] : v[e]);
                __bf16 *row = ybase + (m - m_t) * ro.ldy;
                if (vec_store && ncol + 8 <= g.N) {
                    __builtin_nontemporal_store(hv, (bf16x8 *)(row + ncol));
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (ncol + e < g.N) row[ncol + e] = hv[e];
                }
            }
        }
        drained = false;
    }
    // No DMA load may still be writing LDS when the workgroup ends.
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
    // Fewer tiles than CUs: the chip is not at its power limit, and the
    // second wave per SIMD, issuing MFMAs while the other waits on its reads
    // and loads, shows as wall time (measured on one box, cold / warm: M x N
    // = 520 x 4136, K/P = 512, 99 tiles, 63.1 / 48.8 vs 69.4 / 57.4 us; 300 x
    // 1000, K/P = 1024, 16 tiles, 107.4 / 82.5 vs 111.7 / 90.5 us).  From 256
    // tiles on the four-wave form holds its own (2048 x 4096, K/P = 2048:
    // 260.3 / 220.8 vs 262.6 / 220.2 us; larger shapes 2-3% behind).
    if (T < cus) {
        if (scat)
            gemm_rowfold8_kernel<true><<<dim3(grid), dim3(FT8), 0, s>>>(g, ts, ro, vec ? 1 : 0);
        else
            gemm_rowfold8_kernel<false><<<dim3(grid), dim3(FT8), 0, s>>>(g, ts, ro, vec ? 1 : 0);
    } else if (scat) {
        gemm_rowfold_kernel<true><<<dim3(grid), dim3(FT), 0, s>>>(g, ts, ro, vec ? 1 : 0);
    } else {
        gemm_rowfold_kernel<false><<<dim3(grid), dim3(FT), 0, s>>>(g, ts, ro, vec ? 1 : 0);
    }
    return hipGetLastError();
}

}  // namespace tpl
