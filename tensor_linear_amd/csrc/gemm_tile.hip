// Grouped bf16 shard GEMM on the gfx950 matrix cores: C_i = A_i B_i^T for all
// P shards in one launch ("模型并行", "Tensor Parallel": the column products
// Y_i = X W_i and the row partials X_i W_i; both operands are K-contiguous in
// the [N, K] weight storage, so no transpose is needed).
//
// Output tile 256 (M) x 256 (N); 256 threads = 4 waves in a 2x2 grid, each
// wave owning a 128x128 block = 4x4 v_mfma_f32_32x32x16_bf16 accumulators
// (256 fp32 registers per lane).  The W tile is the MFMA row operand and the
// X tile the column operand, so each lane holds 4 consecutive output columns
// of one row: 16-byte fp32 / 8-byte bf16 stores.
//
// Persistent: one workgroup per CU walks a list of tiles, and the K pipeline
// runs straight across tile boundaries -- the first K steps of the next tile
// are loaded while the current tile finishes and writes its outputs -- so no
// CU sits idle between tiles.  Workgroup b runs on XCD b % 8; the tiles are
// split into 8 contiguous ranges, one per XCD, and inside a range the 32
// workgroups of the XCD take consecutive tiles (visited in groups of 8
// tile-rows, 4 for fp32 partials), so the panels of X and W they share stay
// in that XCD's L2.
//
// Global -> LDS: global_load_lds_dwordx4 (16 bytes per lane straight into
// LDS, no register staging), NST stages of BK columns of K.  One wave
// instruction fills 1 KB of LDS.  Rows are BK*2 bytes; 16-byte chunk c of row
// r sits at slot c ^ ((r / RP) % CPR) (RP rows per 256 bytes, CPR chunks per
// row), so the 16 rows read by one 16-lane group of ds_read_b128 hit 16
// different 16-byte bank groups.
//
// Each tile's first MFMA of every accumulator block takes a zero C operand,
// so no accumulator registers are cleared between tiles.
//
// Edges: rows past M or N are clamped to the last valid row (their results
// are not stored).  K must be a positive multiple of BK.  Tiles entirely
// inside M x N store without per-store bounds tests.
//
// Epilogue options (template EPI): EPI_BIAS adds the column bias (Shard(0),
// "Module 并行：实现 DP/TP/CP/PP 组合", "Linear 实现解析") to the fp32
// accumulators before rounding; EPI_SWIGLU is the gated unit of a fused
// gate+up column layer: the W tile's 256 rows are 128 gate rows and the 128
// up rows of the same hidden units, placed so that each wave's MFMA blocks
// 0-1 hold gate and blocks 2-3 the matching up features in the same lanes;
// the output tile is 256 tokens x 128 hidden units, silu(g + bg) * (u + bu).
// XG: the X rows come from token slices in separate allocations (the
// all-gather of the sequence-parallel layout read in place); a tile never
// spans two slices, so only its base pointer changes.
#include "kernels.h"
#include <type_traits>

namespace tpl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T) __attribute__((address_space(3))) T *

constexpr int TB = 256;  // tile edge in M and N (W rows)
constexpr int TT = 256;  // threads

enum { EPI_NONE = 0, EPI_BIAS = 1, EPI_SWIGLU = 2 };

struct TileSched {
    int tiles_m, tiles_n;  // per shard
    int group_m;           // tile rows visited as a group inside a shard
    int T;                 // tiles over all shards
    int xcd_split;         // 1: XCD-contiguous ranges (grid == 8 * per_xcd)
    int per_xcd;           // workgroups per XCD when xcd_split
};

// Logical tile index -> (shard, tile row, tile column), tile rows grouped by
// group_m inside a shard.
__device__ __forceinline__ void decode_tile(const TileSched &ts, int logical, int &shard,
                                           int &tm, int &tn) {
    const int per_shard = ts.tiles_m * ts.tiles_n;
    shard = logical / per_shard;
    const int t = logical - shard * per_shard;
    const int in_group = ts.group_m * ts.tiles_n;
    const int first_m = (t / in_group) * ts.group_m;
    const int gsz = min(ts.tiles_m - first_m, ts.group_m);
    const int tr = t - (t / in_group) * in_group;
    tm = first_m + tr % gsz;
    tn = tr / gsz;
}

// The q-th tile of this workgroup, or -1 when it has no q-th tile.
__device__ __forceinline__ int tile_of(const TileSched &ts, int q) {
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

template <int BK, int NST, int OUT, int EPI, bool XG>
__global__ __attribute__((amdgpu_flat_work_group_size(TT, TT), amdgpu_waves_per_eu(1, 1)))
void gemm_tile_kernel(GemmArgs g, TileSched ts, int vec_store, GemmExtra ex) {
    constexpr bool SWIGLU = EPI == EPI_SWIGLU;
    constexpr int TBN = SWIGLU ? TB / 2 : TB;   // output columns per tile
    constexpr int ROWB = BK * 2;          // LDS bytes per tile row
    constexpr int CPR = BK / 8;           // 16-byte chunks per row
    constexpr int RP = 256 / ROWB;        // rows per 256 bytes
    constexpr int OPB = TB * ROWB;        // one operand tile
    constexpr int STAGE = 2 * OPB;        // X tile + W tile
    constexpr int RPI = 1024 / ROWB;      // rows per 1 KB load instruction
    constexpr int LPW = OPB / 1024 / 4;   // load instructions per operand per wave
    constexpr int KS = BK / 16;           // MFMA k-steps per stage
    constexpr int EPI_ROWB = 32 * 4 + 16;   // one fp32 row of a 32x32 block, padded
    constexpr int EPI_WAVE = 32 * EPI_ROWB; // per-wave staging area
    static_assert(NST * STAGE + 4 * EPI_WAVE <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE + 4 * EPI_WAVE];
    LDS_PTR(char) lds = (LDS_PTR(char))smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // Number of tiles this workgroup owns.
    int ntiles = 0;
    while (tile_of(ts, ntiles) >= 0) ++ntiles;
    const int nk = (int)(g.K / BK);
    if (ntiles == 0) return;
    const int total = ntiles * nk;

    // ---- prefetch cursor (runs NST-1 steps ahead of the compute cursor).
    // Per-lane load offsets depend on the tile (row clamping), so they are
    // rebuilt whenever the cursor enters a new tile.
    int pq = 0, pkt = 0;
    const char *pa = nullptr, *pb = nullptr;
    uint32_t aoff[LPW], boff[LPW];
    auto enter_tile = [&](int q) {
        int shard, tm, tn;
        decode_tile(ts, tile_of(ts, q), shard, tm, tn);
        const int64_t m0 = (int64_t)tm * TB, n0 = (int64_t)tn * TBN;
        if (XG) {
            const int64_t sl = m0 / ex.x_rows;
            pa = (const char *)((const __bf16 *)ex.x_slice[sl] + (int64_t)shard * g.a_shard +
                                (m0 - sl * ex.x_rows) * g.lda);
        } else {
            pa = (const char *)((const __bf16 *)g.A + (int64_t)shard * g.a_shard + m0 * g.lda);
        }
        pb = (const char *)((const __bf16 *)g.B + (int64_t)shard * g.b_shard + n0 * g.ldb);
        const int a_rows = (int)min<int64_t>(g.M - m0, TB);
        const int b_rows = (int)min<int64_t>(g.N - n0, TBN);
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const int r = (j * 4 + wave) * RPI + lane / CPR;
            const int chunk = (lane % CPR) ^ ((r / RP) % CPR);
            const int ra = r < a_rows ? r : a_rows - 1;
            int64_t wrow;
            if (SWIGLU) {
                // LDS row r feeds wave r / 128, MFMA block (r / 32) % 4:
                // blocks 0-1 gate rows, blocks 2-3 the up rows of the same
                // 64 hidden units.
                const int blk = (r >> 5) & 3;
                int h = ((r >> 7) << 6) + ((blk & 1) << 5) + (r & 31);
                h = h < b_rows ? h : b_rows - 1;
                wrow = h + (blk >= 2 ? ex.up_off : 0);
            } else {
                wrow = r < b_rows ? r : b_rows - 1;
            }
            aoff[j] = (uint32_t)(((int64_t)ra * g.lda + chunk * 8) * 2);
            boff[j] = (uint32_t)((wrow * g.ldb + chunk * 8) * 2);
        }
    };
    // Issue loads [j0, j1) of the cursor's step into `stage` (branch-free;
    // loads 0..LPW-1 fill the X tile, LPW..2*LPW-1 the W tile).
    auto issue_part = [&](int stage, int j0, int j1) {
        LDS_PTR(char) dst = lds + stage * STAGE;
        const int64_t kb = (int64_t)pkt * BK * 2;
#pragma unroll
        for (int j = 0; j < 2 * LPW; ++j) {
            if (j < j0 || j >= j1) continue;
            if (j < LPW)
                __builtin_amdgcn_global_load_lds((const void *)(pa + kb + aoff[j]),
                                                 (LDS_PTR(void))(dst + (j * 4 + wave) * 1024), 16, 0, 0);
            else
                __builtin_amdgcn_global_load_lds(
                    (const void *)(pb + kb + boff[j - LPW]),
                    (LDS_PTR(void))(dst + OPB + ((j - LPW) * 4 + wave) * 1024), 16, 0, 0);
        }
    };
    auto issue_step = [&](int stage) { issue_part(stage, 0, 2 * LPW); };
    // Advance the cursor one step.  Past the last step it stays there, so
    // later issues reload the last step into stages that are not read again.
    auto advance = [&]() {
        if (pq * nk + pkt + 1 < total) {
            if (++pkt == nk) {
                pkt = 0;
                ++pq;
                enter_tile(pq);
            }
        }
    };

    // With two stages the loads of a step are split in halves: the X half is
    // issued in the last phase of the step two before it (its stage is free
    // once that step's barrier has passed), the W half in phase 0 of the step
    // before it.  Spreading them over two phases keeps the vector memory
    // queue from backing up into the MFMA issue.  With more stages a whole
    // step is issued in phase 0, NST-1 steps ahead.
    enter_tile(0);
    if (NST == 2) {
        issue_step(0);
        advance();
        issue_part(1, 0, LPW);
    } else {
#pragma unroll
        for (int s = 0; s < NST - 1; ++s) {
            issue_step(s);
            advance();
        }
    }

    // Fragment addressing: a 32x32x16 operand fragment is 32 rows x 16 k;
    // lane reads row lane%32, k-chunk 2*ks + lane/32.
    const int frow = lane & 31;
    const int fhalf = lane >> 5;
    const int fx = (frow / RP) % CPR;
    const int wrow_off = (wn * 128 + frow) * ROWB;
    const int xrow_off = (wm * 128 + frow) * ROWB;
    auto read_frags = [&](bf16x8 (&wd)[4], bf16x8 (&xd)[4], LDS_PTR(char) st, int ks) {
        const int slot = ((2 * ks + fhalf) ^ fx) << 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) wd[i] = *(LDS_PTR(bf16x8))(st + OPB + wrow_off + i * 32 * ROWB + slot);
#pragma unroll
        for (int j = 0; j < 4; ++j) xd[j] = *(LDS_PTR(bf16x8))(st + xrow_off + j * 32 * ROWB + slot);
    };

    // Step 0's data, then its first fragments.
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LPW * (NST - 2)) : "memory");
    __syncthreads();
    bf16x8 wf[2][4], xf[2][4];
    read_frags(wf[0], xf[0], lds, 0);

    // Per K step (KS phases of 16 MFMAs, with the 8 fragment reads after the
    // first 8 MFMAs and the phase's global->LDS loads after every other MFMA
    // -- one wave per SIMD issues in order, so memory instructions issued back
    // to back would stall the wave while its MFMA pipe runs dry):
    //   phase 0       MFMAs of k-step 0; reads of k-step 1; the loads of the
    //                 step NST-1 ahead (into the stage freed last step);
    //   phase ks      MFMAs of k-step ks; reads of k-step ks+1;
    //   (barrier)     the next step's stage has landed and every wave is done
    //                 reading this step's stage;
    //   phase KS-1    MFMAs of the last k-step; reads of the next step's
    //                 k-step 0, so its LDS latency is hidden too.
    int it = 0;
    bool drained = true;  // no epilogue store is in flight
    for (int q = 0; q < ntiles; ++q) {
        f32x16 acc[4][4];

        auto kstep = [&](auto first) __attribute__((always_inline)) {
            constexpr bool FIRST = decltype(first)::value;
            LDS_PTR(char) st = lds + (it % NST) * STAGE;
            LDS_PTR(char) st_next = lds + ((it + 1) % NST) * STAGE;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int cur = ks & 1, nx = cur ^ 1;
                if (ks == KS - 1) {
                    // The next step's loads were issued NST-1 steps ago; the
                    // NST-2 later groups may stay in flight.  After an epilogue
                    // its stores are in flight too; then wait for everything.
                    __builtin_amdgcn_sched_barrier(0);
                    if (NST == 2 || !drained)
                        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    else
                        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LPW * (NST - 2)) : "memory");
                    drained = true;
                    __syncthreads();
                }
                LDS_PTR(char) rd = ks + 1 < KS ? st : st_next;
                const int rks = ks + 1 < KS ? ks + 1 : 0;
                const int slot = ((2 * rks + fhalf) ^ fx) << 4;
                // Loads of this phase: [j0, j1) of the cursor's step.
                int j0 = 2 * LPW, j1 = 2 * LPW;
                if (NST == 2) {
                    if (ks == 0) { j0 = LPW; j1 = 2 * LPW; }      // W half of step it+1
                    if (ks == KS - 1) { j0 = 0; j1 = LPW; }       // X half of step it+2
                } else if (ks == 0) {
                    j0 = 0; j1 = 2 * LPW;                         // all of step it+NST-1
                }
                const int lstage = NST == 2 ? (ks == 0 ? (it + 1) % 2 : it % 2) : (it + NST - 1) % NST;
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    __builtin_amdgcn_sched_barrier(0);
                    // Diagonal order: MFMAs 0..3 touch all 8 fragments, so no
                    // wait on an LDS read comes after the first global->LDS
                    // load of the phase (the compiler drains every LDS read at
                    // such a wait once an LDS-writing load is in flight).
                    const int i = u & 3, j = ((u & 3) + (u >> 2)) & 3;
                    if (FIRST && ks == 0)   // the tile's first product of each block: C = 0
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cur][i], xf[cur][j],
                                                                            f32x16{}, 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cur][i], xf[cur][j],
                                                                            acc[i][j], 0, 0, 0);
                    if (u < 8) {
                        if (u < 4)
                            wf[nx][u] = *(LDS_PTR(bf16x8))(rd + OPB + wrow_off + u * 32 * ROWB + slot);
                        else
                            xf[nx][u - 4] = *(LDS_PTR(bf16x8))(rd + xrow_off + (u - 4) * 32 * ROWB + slot);
                    }
                    // Global->LDS loads after every other MFMA (slots 1, 3,
                    // ..., 15; two per slot when a phase has more than 8), so
                    // each wave leaves the CU's load path a slot between its
                    // loads: 1.5-2% faster on every GEMM shape measured than
                    // the same loads in 8 consecutive slots.
                    const int per = j1 - j0 > 8 ? 2 : 1;
                    const int ls = (u >> 1) * per;
                    const int lc = (u & 1) ? per : 0;
                    const int la = j0 + ls < j1 ? j0 + ls : j1;
                    const int lb = j0 + ls + lc < j1 ? j0 + ls + lc : j1;
                    if (la < lb) issue_part(lstage, la, lb);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA
                    if (u < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);       // DS read
                    if (lb - la >= 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); // VMEM
                    if (lb - la >= 2) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
                if (NST == 2 && ks == 0) {
                    __builtin_amdgcn_sched_barrier(0);
                    advance();
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (NST != 2) advance();
        };
        kstep(std::true_type{});
        ++it;
        for (int kt = 1; kt < nk; ++kt, ++it) kstep(std::false_type{});

        // ---- epilogue.  32x32 D layout with W rows as the row operand:
        // lane holds m = lane%32 and, for r4 = 0..3, the 4 columns
        // n = 8*r4 + 4*(lane/32) + 0..3 in registers 4*r4..4*r4+3.
        int shard, tm, tn;
        decode_tile(ts, tile_of(ts, q), shard, tm, tn);
        const int64_t tm0 = (int64_t)tm * TB, tn0 = (int64_t)tn * TBN;
        const int64_t cbase = (int64_t)shard * g.c_shard;
        if constexpr (EPI == EPI_NONE) {
            // Each 32x32 block goes through this wave's LDS area: written in its
            // MFMA layout (lane: row m, four consecutive n), read back
            // row-contiguous, so a store covers whole 64-byte (bf16) or 128-byte
            // (fp32) row segments.  One path for all tiles: only stores that
            // cross M or N fall back to element stores.  The stores are
            // non-temporal: every CU reaches its epilogue at about the same time,
            // and streaming the burst past L2 keeps it from filling the L2 with
            // dirty lines the next loads would have to wait behind.
            {
                LDS_PTR(char) ep = lds + NST * STAGE + wave * EPI_WAVE;
                const int64_t tm_w = tm0 + wm * 128, tn_w = tn0 + wn * 128;
                constexpr int VW = OUT == OUT_BF16 ? 8 : 4;   // values per lane store
                constexpr int RPP = 64 * VW / 32;              // rows per pass
                constexpr int ES = OUT == OUT_BF16 ? 2 : 4;    // bytes per value
                // Tiles inside M x N (all but the last tile row and column) take a
                // path without per-store bounds tests: one per-lane byte offset
                // and a uniform base per store.
                const bool interior = vec_store && tm0 + TB <= g.M && tn0 + TB <= g.N &&
                                      (int64_t)RPP * g.ldc * ES < (1ll << 31);
                if (interior) {
                    const uint32_t lane_off =
                        (uint32_t)(((int64_t)(lane / (32 / VW)) * g.ldc + VW * (lane % (32 / VW))) * ES);
                    char *wbase = (char *)g.C + (cbase + tm_w * g.ldc + tn_w) * ES;
    #pragma unroll
                    for (int j = 0; j < 4; ++j) {
    #pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                            for (int r4 = 0; r4 < 4; ++r4) {
                                const f32x4 v = {acc[i][j][4 * r4], acc[i][j][4 * r4 + 1],
                                                 acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]};
                                *(LDS_PTR(f32x4))(ep + frow * EPI_ROWB + (8 * r4 + 4 * fhalf) * 4) = v;
                            }
    #pragma unroll
                            for (int pp = 0; pp < 32 / RPP; ++pp) {
                                const int r = pp * RPP + lane / (32 / VW), c = VW * (lane % (32 / VW));
                                float vv[VW];
    #pragma unroll
                                for (int h = 0; h < VW / 4; ++h) {
                                    const f32x4 a4 = *(LDS_PTR(f32x4))(ep + r * EPI_ROWB + (c + 4 * h) * 4);
                                    vv[4 * h] = a4[0]; vv[4 * h + 1] = a4[1]; vv[4 * h + 2] = a4[2]; vv[4 * h + 3] = a4[3];
                                }
                                char *bp = wbase + ((int64_t)(j * 32 + pp * RPP) * g.ldc + i * 32) * ES + lane_off;
                                if (OUT == OUT_BF16) {
                                    bf16x8 hv;
    #pragma unroll
                                    for (int e = 0; e < 8; ++e) hv[e] = (__bf16)vv[e];
                                    __builtin_nontemporal_store(hv, (bf16x8 *)bp);
                                } else {
                                    __builtin_nontemporal_store(f32x4{vv[0], vv[1], vv[2], vv[3]}, (f32x4 *)bp);
                                }
                            }
                        }
                    }
                } else {
    #pragma unroll
                    for (int j = 0; j < 4; ++j) {
    #pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                            for (int r4 = 0; r4 < 4; ++r4) {
                                const f32x4 v = {acc[i][j][4 * r4], acc[i][j][4 * r4 + 1],
                                                 acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]};
                                *(LDS_PTR(f32x4))(ep + frow * EPI_ROWB + (8 * r4 + 4 * fhalf) * 4) = v;
                            }
                            const int64_t bm = tm_w + j * 32, bn = tn_w + i * 32;
    #pragma unroll
                            for (int pp = 0; pp < 32 / RPP; ++pp) {
                                const int r = pp * RPP + lane / (32 / VW), c = VW * (lane % (32 / VW));
                                const int64_t m = bm + r, n = bn + c;
                                float vv[VW];
    #pragma unroll
                                for (int h = 0; h < VW / 4; ++h) {
                                    const f32x4 a4 = *(LDS_PTR(f32x4))(ep + r * EPI_ROWB + (c + 4 * h) * 4);
                                    vv[4 * h] = a4[0]; vv[4 * h + 1] = a4[1]; vv[4 * h + 2] = a4[2]; vv[4 * h + 3] = a4[3];
                                }
                                if (m < g.M) {
                                    const int64_t o = cbase + m * g.ldc + n;
                                    if (vec_store && n + VW <= g.N) {
                                        if (OUT == OUT_BF16) {
                                            bf16x8 hv;
    #pragma unroll
                                            for (int e = 0; e < 8; ++e) hv[e] = (__bf16)vv[e];
                                            __builtin_nontemporal_store(hv, (bf16x8 *)((__bf16 *)g.C + o));
                                        } else {
                                            __builtin_nontemporal_store(f32x4{vv[0], vv[1], vv[2], vv[3]},
                                                                        (f32x4 *)((float *)g.C + o));
                                        }
                                    } else {
    #pragma unroll
                                        for (int e = 0; e < VW; ++e) {
                                            if (n + e < g.N) {
                                                if (OUT == OUT_BF16) ((__bf16 *)g.C)[o + e] = (__bf16)vv[e];
                                                else ((float *)g.C)[o + e] = vv[e];
                                            }
                                        }
                                    }
                                }
                            }
                        }
                    }
                }
            }
        } else {
            // With a bias or the gated unit (bf16 output): each 32x32 block
            // is staged through LDS as above and read back row-contiguous, a
            // lane holding 8 consecutive columns of a row; the bias and the
            // activation are applied there, in VGPRs.  For the gated unit the
            // gate block and then its up block go through the staging area,
            // so both values of an output meet in the same lane.
            static_assert(OUT == OUT_BF16, "epilogue options write bf16");
            LDS_PTR(char) ep = lds + NST * STAGE + wave * EPI_WAVE;
            constexpr int NI = SWIGLU ? 2 : 4;      // output column blocks per wave
            constexpr int NH = SWIGLU ? 2 : 1;      // bias vectors per block (gate, up)
            const int64_t tm_w = tm0 + wm * 128, tn_w = tn0 + wn * (TBN / 2);
            const int lr = lane >> 2, lc = 8 * (lane & 3);  // row within a 16-row pass, first column
            const bool has_bias = ex.bias != nullptr;
            bf16x8 bvec[NI][NH];
            if (has_bias) {
                const __bf16 *bb = (const __bf16 *)ex.bias + (int64_t)shard * ex.bias_shard;
#pragma unroll
                for (int i = 0; i < NI; ++i) {
#pragma unroll
                    for (int h = 0; h < NH; ++h) {
                        const int64_t c = tn_w + i * 32 + lc;
                        const __bf16 *src = bb + (h ? ex.up_off : 0) + c;
                        if (c + 7 < g.N) {
                            bvec[i][h] = *(const bf16x8 *)src;
                        } else {
#pragma unroll
                            for (int e = 0; e < 8; ++e) bvec[i][h][e] = c + e < g.N ? src[e] : (__bf16)0.0f;
                        }
                    }
                }
            }
            auto stage = [&](const f32x16 &a) __attribute__((always_inline)) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const f32x4 v = {a[4 * r4], a[4 * r4 + 1], a[4 * r4 + 2], a[4 * r4 + 3]};
                    *(LDS_PTR(f32x4))(ep + frow * EPI_ROWB + (8 * r4 + 4 * fhalf) * 4) = v;
                }
            };
            auto readback = [&](float (&v)[2][8]) __attribute__((always_inline)) {
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    LDS_PTR(char) rp = ep + (pp * 16 + lr) * EPI_ROWB + lc * 4;
                    const f32x4 a0 = *(LDS_PTR(f32x4))rp, a1 = *(LDS_PTR(f32x4))(rp + 16);
#pragma unroll
                    for (int e = 0; e < 4; ++e) { v[pp][e] = a0[e]; v[pp][4 + e] = a1[e]; }
                }
            };
            const bool interior = vec_store && tm0 + TB <= g.M && tn0 + TBN <= g.N;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    __builtin_amdgcn_sched_barrier(0);
                    float v[2][8];
                    stage(acc[i][j]);
                    readback(v);
                    if (SWIGLU) {
                        float u[2][8];
                        stage(acc[i + 2][j]);
                        readback(u);
#pragma unroll
                        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                float gv = v[pp][e], uv = u[pp][e];
                                if (has_bias) {
                                    gv = gv + (float)bvec[i][0][e];
                                    uv = uv + (float)bvec[i][NH - 1][e];
                                }
                                v[pp][e] = silu_f32(gv) * uv;
                            }
                    } else if (has_bias) {
#pragma unroll
                        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
                            for (int e = 0; e < 8; ++e) v[pp][e] = v[pp][e] + (float)bvec[i][0][e];
                    }
#pragma unroll
                    for (int pp = 0; pp < 2; ++pp) {
                        const int64_t m = tm_w + j * 32 + pp * 16 + lr, n = tn_w + i * 32 + lc;
                        bf16x8 hv;
#pragma unroll
                        for (int e = 0; e < 8; ++e) hv[e] = (__bf16)v[pp][e];
                        __bf16 *dst = (__bf16 *)g.C + cbase + m * g.ldc + n;
                        if (interior) {
                            __builtin_nontemporal_store(hv, (bf16x8 *)dst);
                        } else if (m < g.M) {
                            if (vec_store && n + 8 <= g.N) {
                                __builtin_nontemporal_store(hv, (bf16x8 *)dst);
                            } else {
#pragma unroll
                                for (int e = 0; e < 8; ++e)
                                    if (n + e < g.N) dst[e] = hv[e];
                            }
                        }
                    }
                }
            }
        }
        drained = false;
    }
    // No global->LDS load may still be writing when the workgroup ends.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }


// K per stage and number of stages (tuning parameters; 2 x 64 and 4 x 32 both
// use 128 KB of LDS).
#ifndef TPL_TILE_BK
#define TPL_TILE_BK 64
#endif
#ifndef TPL_TILE_NST
#define TPL_TILE_NST 2
#endif
constexpr int KERNEL_BK = TPL_TILE_BK;
constexpr int KERNEL_NST = TPL_TILE_NST;

}  // namespace

bool gemm_tile_supported(const GemmArgs &g, const GemmExtra *ex) {
    // 32-bit per-lane offsets: one tile's rows must span < 2 GiB (for the
    // gated unit, up to the up rows of the tile).
    const int64_t wspan = TB + (ex && ex->act == ACT_SWIGLU ? ex->up_off : 0);
    const bool small_rows = (int64_t)TB * g.lda * 2 < (1ll << 31) &&
                            wspan * g.ldb * 2 < (1ll << 31);
    bool ok = g.K > 0 && g.K % KERNEL_BK == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 &&
              g.a_shard % 8 == 0 && g.b_shard % 8 == 0 && aligned16(g.B) && small_rows;
    if (!ex) return ok && aligned16(g.A);
    // Bias: 16-byte loads of 8 values per lane.
    if (ex->bias && (((uintptr_t)ex->bias % 16) != 0 || ex->bias_shard % 8 != 0)) return false;
    if (ex->act == ACT_SWIGLU && ex->up_off % 8 != 0) return false;
    if (ex->x_rows > 0) {
        if (ex->x_rows % TB != 0) return false;
        const int64_t ns = (g.M + ex->x_rows - 1) / ex->x_rows;
        for (int64_t j = 0; j < ns; ++j)
            if (!aligned16(ex->x_slice[j])) return false;
        return ok;
    }
    return ok && aligned16(g.A);
}

namespace {

template <int OUT, int EPI, bool XG>
hipError_t launch_tile_t(const GemmArgs &g, const TileSched &ts, int vec, const GemmExtra &ex,
                         int grid, hipStream_t s) {
    gemm_tile_kernel<KERNEL_BK, KERNEL_NST, OUT, EPI, XG><<<dim3(grid), dim3(TT), 0, s>>>(g, ts, vec, ex);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_tile(const GemmArgs &g, int out_type, const GemmExtra *exp, hipStream_t s) {
    if (g.M == 0 || g.N == 0 || g.P == 0) return hipSuccess;
    GemmExtra ex{};
    if (exp) ex = *exp;
    const bool swiglu = ex.act == ACT_SWIGLU;
    const int tbn = swiglu ? TB / 2 : TB;
    const int64_t tm = (g.M + TB - 1) / TB, tn = (g.N + tbn - 1) / tbn;
    const int64_t T = tm * tn * g.P;
    if (T > 0x7FFFFFFFll) return hipErrorInvalidConfiguration;
    TileSched ts;
    ts.tiles_m = (int)tm;
    ts.tiles_n = (int)tn;
    // Groups of 8 tile rows for the bf16 column products, 4 for the fp32
    // row partials (measured on one box: fc2 +1.2-1.4%, Llama-70B O row
    // +1.7-2.2% with 4; column products equal or better with 8).
    ts.group_m = out_type == OUT_BF16 ? 8 : 4;
    ts.T = (int)T;
    const int cus = device_cu_count();
    int grid = (int)(T < cus ? T : cus);
    ts.xcd_split = (grid == cus && cus % 8 == 0 && T >= cus) ? 1 : 0;
    ts.per_xcd = grid / 8;
    // 16-byte stores of 8 bf16 or 4 fp32 values: row starts and shard offsets
    // must keep that alignment.
    const int vw = out_type == OUT_BF16 ? 8 : 4;
    const int vec = (g.ldc % vw == 0) && (g.c_shard % vw == 0) && (((uintptr_t)g.C) % 16 == 0);
    const bool xg = ex.x_rows > 0;
    if (out_type != OUT_BF16) {
        // fp32 output (row partials): no epilogue options.
        if (xg || swiglu || ex.bias) return hipErrorInvalidValue;
        return launch_tile_t<OUT_F32, EPI_NONE, false>(g, ts, vec, ex, grid, s);
    }
    const int epi = swiglu ? EPI_SWIGLU : ex.bias ? EPI_BIAS : EPI_NONE;
    if (xg) {
        if (epi == EPI_SWIGLU) return launch_tile_t<OUT_BF16, EPI_SWIGLU, true>(g, ts, vec, ex, grid, s);
        if (epi == EPI_BIAS) return launch_tile_t<OUT_BF16, EPI_BIAS, true>(g, ts, vec, ex, grid, s);
        return launch_tile_t<OUT_BF16, EPI_NONE, true>(g, ts, vec, ex, grid, s);
    }
    if (epi == EPI_SWIGLU) return launch_tile_t<OUT_BF16, EPI_SWIGLU, false>(g, ts, vec, ex, grid, s);
    if (epi == EPI_BIAS) return launch_tile_t<OUT_BF16, EPI_BIAS, false>(g, ts, vec, ex, grid, s);
    return launch_tile_t<OUT_BF16, EPI_NONE, false>(g, ts, vec, ex, grid, s);
}

}  // namespace tpl
