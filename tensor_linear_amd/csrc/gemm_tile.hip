// Grouped bf16 shard GEMM on the gfx950 matrix cores: C_i = A_i B_i^T for all
// P shards in one launch ("模型并行", "Tensor Parallel": the column products
// Y_i = X W_i and the row partials X_i W_i; both operands are K-contiguous in
// the [N, K] weight storage, so no transpose is needed).
//
// Output tile 256 (M) x 256 (N); 256 threads = 4 waves in a 2x2 grid, each
// wave owning a 128x128 block = 8x8 v_mfma_f32_16x16x32_bf16 accumulators
// (256 fp32 registers per lane).  The 16x16x32 form and not 32x32x16: at
// full issue rate with random operands the chip holds about 2.0 GHz under
// the former and about 1.66 GHz under the latter (the same flops per
// instruction-cycle; the clock is power-limited), and the results are the
// same bit for bit.  The W tile is the MFMA row operand and the X tile the
// column operand, so each lane holds 4 consecutive output columns of one
// output row.
//
// Persistent: one workgroup per CU walks a list of tiles and the K pipeline
// runs straight across tile boundaries.  Workgroup b runs on XCD b % 8; the
// tiles are split into 8 contiguous ranges, one per XCD, and inside a range
// the 32 workgroups of the XCD take consecutive tiles (visited in groups of 8
// tile-rows, 4 for fp32 partials), so the panels of X and W they share stay in
// that XCD's L2.
//
// LDS: three X stages and two W stages of K = 64 (5 x 32 KB = 160 KB), rows
// of 128 bytes (one cache line); 16-byte chunk c of row r at slot
// c ^ ((r / 2) % 8), so the 16 rows a 16-lane group of ds_read_b128 reads hit
// 16 different bank groups.  Global -> LDS with global_load_lds_dwordx4 (one
// 1 KB wave instruction = 8 rows, no register staging).  Each step's 16 loads
// per wave are spread evenly, one every 8th MFMA: the W half loaded one step
// ahead has 4-6 quarter-steps of lead before the barrier that needs it, the
// other W half 7-8, the X loaded two steps ahead (the third X stage makes room
// for it) 9-12 -- with two stages of each, a whole step had to be loaded in
// the quarter of the step after the stage came free.
//
// Per step (K = 64 = two 32-wide substeps), 8 quarters of 16 MFMAs (16 cycles
// each), each one 4 x 4 group of the wave's W blocks against its X blocks:
// q0 W0-3 x X0-3, q1 W0-3 x X4-7, q2 W4-7 x X0-3, q3 W4-7 x X4-7 on substep 0,
// q4-q7 the same on substep 1.  The quarters read four fragments each, one
// every 4th MFMA, except q4 (eight) and q5 (none), so that no read is still in
// flight when the wave reaches the barrier:
//   q0 X4-7 (substep 0)  q1 W4-7 (0)  q2 W0-3 (1)  q3 X0-3 (1)
//   q4 X4-7 and W4-7 (1) q5 -
//   (barrier: step it+1 has landed; every wave is done with step it's stages)
//   q6 W0-3, q7 X0-3 of step it+1's substep 0.
// A fragment replaces the same block's fragment of the step before, whose
// last use is at least a quarter earlier.  Inside a quarter the block
// group read most recently is the slow index, so each of its fragments is
// first used 16 MFMAs after its read.  One barrier per step, before q6.
// DMA loads: q0-q1 the second W half of step it+1, q2-q5 X of step it+2,
// q6-q7 the first W half of step it+2.  (Measured against four 32-MFMA
// phases with 8, 8, 4 and 12 reads: the same results bit for bit, 0.3-2%
// faster on every GEMM shape; moving q5's reads into q4 another ~0.5%.)
//
// Each tile's first MFMA of every accumulator block takes a zero C operand,
// so no accumulator registers are cleared between tiles.
//
// Epilogue: 32 output rows x 64 columns at a time go through this wave's part
// of the X stage the tile's last barrier freed (its own 1 KB DMA chunks, which
// only its own later loads overwrite): written in the MFMA layout, read back
// row-contiguous (a group's reads all issued before its stores), so a bf16
// row leaves as one full 128-byte line and an fp32 row as two.  Stores are non-temporal (measured faster than cached stores
// for every shape: the burst of all CUs' tiles would fill the L2 with dirty
// lines the next loads wait behind).
//
// Edges: rows past M or N are clamped to the last valid row (their results are
// not stored).  K must be a positive multiple of 64.  Tiles entirely inside
// M x N store without per-store bounds tests.
//
// Epilogue options (template EPI): EPI_BIAS adds the column bias (Shard(0),
// "Module 并行：实现 DP/TP/CP/PP 组合", "Linear 实现解析") to the fp32
// accumulators before rounding; EPI_SWIGLU is the gated unit of a fused
// gate+up column layer: the W tile's 256 rows are 128 gate rows and the 128
// up rows of the same hidden units, placed so that each wave's W blocks 0-3
// hold gate and blocks 4-7 the matching up features in the same lanes; the
// output tile is 256 tokens x 128 hidden units, silu(g + bg) * (u + bu).
// XG: the X rows come from token slices in separate allocations (the
// all-gather of the sequence-parallel layout read in place); a tile never
// spans two slices, so only its base pointer changes.
#include "kernels.h"
#include <type_traits>

namespace tpl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T) __attribute__((address_space(3))) T *

constexpr int TB = 256;   // tile edge in M and N (W rows)
constexpr int TT = 256;   // threads

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

template <int OUT, int EPI, bool XG>
__global__ __attribute__((amdgpu_flat_work_group_size(TT, TT), amdgpu_waves_per_eu(1, 1)))
void gemm_tile_kernel(GemmArgs g, TileSched ts, int vec_store, GemmExtra ex) {
    constexpr bool SWIGLU = EPI == EPI_SWIGLU;
    constexpr int TBN = SWIGLU ? TB / 2 : TB;   // output columns per tile
    constexpr int ROWB = 128;                   // LDS bytes per tile row (K = 64)
    constexpr int OPB = TB * ROWB;              // one operand stage, 32 KB
    constexpr int LPW = 8;                      // 1 KB loads per operand per wave per step
    constexpr int W_BASE = 3 * OPB;             // three X stages, then two W stages
    __shared__ __attribute__((aligned(1024))) char smem[5 * OPB];
    LDS_PTR(char) lds = (LDS_PTR(char))smem;
    const uint32_t lds_u = (uint32_t)(uintptr_t)lds;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    int ntiles = 0;
    while (tile_of(ts, ntiles) >= 0) ++ntiles;
    const int nk = (int)(g.K / 64);
    if (ntiles == 0) return;
    const int total = ntiles * nk;

    // ---- load cursor: the step whose operands are being loaded.  Per-lane
    // load offsets depend on the tile (row clamping), so they are rebuilt
    // whenever the cursor enters a new tile.
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
            const int r = (j * 4 + wave) * 8 + lane / 8;
            const int chunk = (lane % 8) ^ ((r / 2) % 8);
            const int ra = r < a_rows ? r : a_rows - 1;
            int64_t wrow;
            if (SWIGLU) {
                // LDS row r feeds wave half r / 128, W block (r / 16) % 8:
                // blocks 0-3 gate rows, blocks 4-7 the up rows of the same
                // 64 hidden units.
                const int blk = (r >> 4) & 7;
                int h = ((r >> 7) << 6) + ((blk & 3) << 4) + (r & 15);
                h = h < b_rows ? h : b_rows - 1;
                wrow = h + (blk >= 4 ? ex.up_off : 0);
            } else {
                wrow = r < b_rows ? r : b_rows - 1;
            }
            aoff[j] = (uint32_t)(((int64_t)ra * g.lda + chunk * 8) * 2);
            boff[j] = (uint32_t)((wrow * g.ldb + chunk * 8) * 2);
        }
    };
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
    // One 1 KB DMA load: 16 bytes per lane from base + voff into LDS at
    // lds_addr + 16 * lane.  Issued as an instruction the compiler does not
    // track: its own wait analysis cannot tell which stage a DMA writes and
    // would drain every load in flight before the next LDS read; the waits
    // this pipeline needs are written out below.
    auto dma = [&](const char *base, uint32_t voff, uint32_t lds_addr) __attribute__((always_inline)) {
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                     :: "v"(voff), "s"(base), "s"(lds_addr) : "memory", "m0");
    };
    auto load_x = [&](int slot, int j) __attribute__((always_inline)) {
        dma(pa + (int64_t)pkt * 128, aoff[j], lds_u + slot * OPB + (j * 4 + wave) * 1024);
    };
    auto load_w = [&](int slot, int j) __attribute__((always_inline)) {
        dma(pb + (int64_t)pkt * 128, boff[j], lds_u + W_BASE + slot * OPB + (j * 4 + wave) * 1024);
    };

    // Prologue: X and W of step 0, X of step 1, the first W half of step 1.
    enter_tile(0);
#pragma unroll
    for (int j = 0; j < LPW; ++j) load_x(0, j);
#pragma unroll
    for (int j = 0; j < LPW; ++j) load_w(0, j);
    advance();
#pragma unroll
    for (int j = 0; j < LPW; ++j) load_x(1, j);
#pragma unroll
    for (int j = 0; j < 4; ++j) load_w(1, j);
    asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    asm volatile("s_barrier" ::: "memory");

    // Fragments: a 16x16x32 operand fragment is 16 rows x 32 k; lane reads
    // row lane%16 of its block, 16-byte k-chunk 4*h + lane/16 of substep h.
    // acc[i][j]: W block i (output columns 16i..), X block j (output rows
    // 16j..) of the wave's 128x128 block.
    const int frow = lane & 15;
    const int fq = lane >> 4;
    const int fx = (frow / 2) % 8;
    const uint32_t wrow_off = (wn * 128 + frow) * ROWB;
    const uint32_t xrow_off = (wm * 128 + frow) * ROWB;
    // fragment f: 0..7 W blocks, 8..15 X blocks; substep h
    auto frag_addr = [&](uint32_t xbase, uint32_t wbase, int f, int h) -> uint32_t {
        const uint32_t slot = (uint32_t)(((4 * h + fq) ^ fx) << 4);
        if (f < 8) return wbase + wrow_off + f * 16 * ROWB + slot;
        return xbase + xrow_off + (f - 8) * 16 * ROWB + slot;
    };
    bf16x8 fr[2][16];   // [substep][fragment]
    auto read_frag = [&](int h, int f, uint32_t addr) __attribute__((always_inline)) {
        fr[h][f] = *(LDS_PTR(bf16x8))(lds + addr);
    };
    // Step 0's substep-0 W0-3 and X0-3, which its first quarter uses.
#pragma unroll
    for (int f = 0; f < 4; ++f) read_frag(0, f, frag_addr(0, W_BASE, f, 0));
#pragma unroll
    for (int f = 8; f < 12; ++f) read_frag(0, f, frag_addr(0, W_BASE, f, 0));

    int it = 0;
    int xs = 0, ws = 0;       // X stage it % 3, W stage it % 2
    bool drained = true;      // no epilogue store is in flight
    for (int q = 0; q < ntiles; ++q) {
        f32x4 acc[8][8];
        auto kstep = [&](auto first) __attribute__((always_inline)) {
            constexpr bool FIRST = decltype(first)::value;
            const int xs1 = xs == 2 ? 0 : xs + 1, ws1 = ws ^ 1;     // stages of step it+1
            const int xs2 = xs1 == 2 ? 0 : xs1 + 1;                 // X stage of step it+2
            const uint32_t xb = xs * OPB, wb = W_BASE + ws * OPB;
            const uint32_t xb1 = xs1 * OPB, wb1 = W_BASE + ws1 * OPB;
#pragma unroll
            for (int qr = 0; qr < 8; ++qr) {
                if (qr == 6) {
                    __builtin_amdgcn_sched_barrier(0);
                    // Step it+1's operands have landed (X issued in q2-q5 of
                    // step it-1, W in q6-q7 of it-1 and q0-q1 of it); the 8 X
                    // loads of step it+2 may stay in flight.  After an
                    // epilogue its stores are in flight too, and a store may
                    // complete before an older load: wait for all.
                    // lgkmcnt(0): this wave's reads of step it's stages are
                    // done before anyone's DMA may overwrite them.
                    if (drained)
                        asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory");
                    else
                        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
                    asm volatile("s_barrier" ::: "memory");
                    drained = true;
                    __builtin_amdgcn_sched_barrier(0);
                }
                const int h = qr >> 2;                       // substep
                const int wg = (qr >> 1) & 1, xg = qr & 1;   // W blocks 4wg.., X blocks 4xg..
                const bool x_outer = (qr & 3) != 2;          // X blocks the slow index
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    __builtin_amdgcn_sched_barrier(0);
                    const int a = u >> 2, b = u & 3;
                    const int i = wg * 4 + (x_outer ? b : a), j = xg * 4 + (x_outer ? a : b);
                    if (FIRST && h == 0)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[0][i], fr[0][8 + j], f32x4{}, 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[h][i], fr[h][8 + j], acc[i][j], 0, 0, 0);
                    // q4 also reads W4-7 of substep 1 (slots 1, 5, 9, 13) and q5
                    // reads nothing, so that no read is in flight at the barrier
                    const bool rd2 = qr == 4 && (u & 3) == 1;
                    if (rd2) read_frag(1, 4 + (u >> 2), frag_addr(xb, wb, 4 + (u >> 2), 1));
                    const bool rd = (u & 3) == 0 && qr != 5;
                    if (rd) {
                        const int k = u >> 2;
                        switch (qr) {
                            case 0: read_frag(0, 12 + k, frag_addr(xb, wb, 12 + k, 0)); break;  // X4-7 sub 0
                            case 1: read_frag(0, 4 + k, frag_addr(xb, wb, 4 + k, 0)); break;    // W4-7 sub 0
                            case 2: read_frag(1, k, frag_addr(xb, wb, k, 1)); break;            // W0-3 sub 1
                            case 3: read_frag(1, 8 + k, frag_addr(xb, wb, 8 + k, 1)); break;    // X0-3 sub 1
                            case 4: read_frag(1, 12 + k, frag_addr(xb, wb, 12 + k, 1)); break;  // X4-7 sub 1
                            case 6: read_frag(0, k, frag_addr(xb1, wb1, k, 0)); break;          // next W0-3
                            default: read_frag(0, 8 + k, frag_addr(xb1, wb1, 8 + k, 0)); break; // next X0-3
                        }
                    }
                    const bool ld = (u & 7) == 2;
                    if (ld) {
                        const int l = (qr & 1) * 2 + (u >> 3);   // 0..3 within a pair of quarters
                        if (qr < 2) load_w(ws1, 4 + l);                     // second W half of step it+1
                        else if (qr < 6) load_x(xs2, ((qr - 2) >> 1) * 4 + l);  // X of step it+2
                        else load_w(ws, l);                                 // first W half of step it+2
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    if (rd || rd2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
                }
                __builtin_amdgcn_sched_barrier(0);
                if (qr == 1) advance();
            }
            __builtin_amdgcn_sched_barrier(0);
            xs = xs1;
            ws = ws1;
        };
        kstep(std::true_type{});
        ++it;
        for (int kt = 1; kt < nk; ++kt, ++it) kstep(std::false_type{});

        // ---- epilogue.  acc[i][j][r] = C[m = 16j + lane%16][n = 16i +
        // 4*(lane/16) + r] of the wave's block.  Staging: this wave's 1 KB
        // chunks w + 4c (c = 0..7) of the X stage step it-1 (the tile's last)
        // read; staging row r of 256 bytes at chunk r/4, offset (r%4)*256,
        // 16-byte slot s at s ^ (r % 16): conflict-free for the MFMA-layout
        // writes (16 rows, one slot) and the row-contiguous reads.
        __builtin_amdgcn_sched_barrier(0);
        int shard, tm, tn;
        decode_tile(ts, tile_of(ts, q), shard, tm, tn);
        const int64_t cbase = (int64_t)shard * g.c_shard;
        const int es = xs == 0 ? 2 : xs - 1;
        LDS_PTR(char) ep = lds + es * OPB + wave * 1024;
        auto st_addr = [&](int r, int s) -> LDS_PTR(char) {
            return ep + (r >> 2) * 4096 + (r & 3) * 256 + ((s ^ (r & 15)) << 4);
        };
        if constexpr (!SWIGLU) {
            constexpr int ES = OUT == OUT_BF16 ? 2 : 4;
            const int64_t tm_w = (int64_t)tm * TB + wm * 128, tn_w = (int64_t)tn * TB + wn * 128;
            const bool interior = vec_store && (int64_t)tm * TB + TB <= g.M &&
                                  (int64_t)tn * TB + TB <= g.N && (int64_t)32 * g.ldc * ES < (1ll << 31);
            // interior stores: uniform row base + one per-lane offset; LPR
            // lanes of 16 bytes per row (8 for bf16: one 128-byte line)
            constexpr int LPR = OUT == OUT_BF16 ? 8 : 16;
            const uint32_t lane_off = (uint32_t)((lane / LPR) * g.ldc * ES + (lane % LPR) * 16);
            const bool has_bias = EPI == EPI_BIAS && ex.bias != nullptr;
            const __bf16 *bias = has_bias ? (const __bf16 *)ex.bias + (int64_t)shard * ex.bias_shard : nullptr;
#pragma unroll
            for (int j = 0; j < 4; ++j) {          // output rows 32j.. of the wave
#pragma unroll
                for (int ip = 0; ip < 2; ++ip) {   // output columns 64ip.. of the wave
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
                        for (int bi = 0; bi < 4; ++bi)
                            *(LDS_PTR(f32x4))st_addr(bj * 16 + frow, bi * 4 + fq) = acc[4 * ip + bi][2 * j + bj];
                    const int64_t ncol = tn_w + ip * 64;
                    if (OUT == OUT_BF16) {
                        // lane: row p*8 + lane/8, 8 columns from 8*(lane%8)
                        const int c8 = lane & 7;
                        float bv[8];
                        if (has_bias) {
                            const int64_t n = ncol + c8 * 8;
                            if (n + 7 < g.N) {
                                const bf16x8 b8 = *(const bf16x8 *)(bias + n);
#pragma unroll
                                for (int e = 0; e < 8; ++e) bv[e] = (float)b8[e];
                            } else {
#pragma unroll
                                for (int e = 0; e < 8; ++e) bv[e] = n + e < g.N ? (float)bias[n + e] : 0.0f;
                            }
                        }
                        // All of the group's LDS reads first, so that they
                        // overlap each other rather than each waiting on
                        // its own store.
                        f32x4 a0[4], a1[4];
#pragma unroll
                        for (int p = 0; p < 4; ++p) {
                            const int rr = p * 8 + (lane >> 3);
                            a0[p] = *(LDS_PTR(f32x4))st_addr(rr, 2 * c8);
                            a1[p] = *(LDS_PTR(f32x4))st_addr(rr, 2 * c8 + 1);
                        }
#pragma unroll
                        for (int p = 0; p < 4; ++p) {
                            float v[8] = {a0[p][0], a0[p][1], a0[p][2], a0[p][3],
                                          a1[p][0], a1[p][1], a1[p][2], a1[p][3]};
                            if (has_bias) {
#pragma unroll
                                for (int e = 0; e < 8; ++e) v[e] = v[e] + bv[e];
                            }
                            bf16x8 hv;
#pragma unroll
                            for (int e = 0; e < 8; ++e) hv[e] = (__bf16)v[e];
                            const int64_t mrow = tm_w + j * 32 + p * 8;
                            if (interior) {
                                char *rb = (char *)g.C + (cbase + mrow * g.ldc + ncol) * 2;
                                __builtin_nontemporal_store(hv, (bf16x8 *)(rb + lane_off));
                            } else {
                                const int64_t m = mrow + (lane >> 3), n = ncol + c8 * 8;
                                if (m < g.M) {
                                    __bf16 *dst = (__bf16 *)g.C + cbase + m * g.ldc + n;
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
                    } else {
                        // lane: row p*4 + lane/16, 4 columns from 4*(lane%16);
                        // the reads first, as above
                        const int sl = lane & 15;
                        f32x4 a[8];
#pragma unroll
                        for (int p = 0; p < 8; ++p) a[p] = *(LDS_PTR(f32x4))st_addr(p * 4 + (lane >> 4), sl);
                        if (interior) {
#pragma unroll
                            for (int p = 0; p < 8; ++p) {
                                const int64_t mrow = tm_w + j * 32 + p * 4;
                                char *rb = (char *)g.C + (cbase + mrow * g.ldc + ncol) * 4;
                                __builtin_nontemporal_store(a[p], (f32x4 *)(rb + lane_off));
                            }
                        } else {
#pragma unroll
                            for (int p = 0; p < 8; ++p) {
                                const int64_t m = tm_w + j * 32 + p * 4 + (lane >> 4), n = ncol + sl * 4;
                                if (m < g.M) {
                                    float *dst = (float *)g.C + cbase + m * g.ldc + n;
                                    if (vec_store && n + 4 <= g.N) {
                                        __builtin_nontemporal_store(a[p], (f32x4 *)dst);
                                    } else {
#pragma unroll
                                        for (int e = 0; e < 4; ++e)
                                            if (n + e < g.N) dst[e] = a[p][e];
                                    }
                                }
                            }
                        }
                    }
                }
            }
        } else {
            // Gated unit: per X block j (16 output rows), the wave's 4 gate
            // blocks (hidden units 16i..) and 4 up blocks (the same units)
            // go through the staging area as one 16-row x 128-column fp32
            // block (gate in slots 0-15, up in 16-31 of 512-byte rows; row r
            // at chunk r/2, offset (r%2)*512, slot s at s ^ (r % 16)); each
            // lane then reads 8 gate and 8 up values of one row.
            static_assert(OUT == OUT_BF16, "the gated unit writes bf16");
            auto sw_addr = [&](int r, int s) -> LDS_PTR(char) {
                return ep + (r >> 1) * 4096 + (r & 1) * 512 + ((s ^ (r & 15)) << 4);
            };
            const int64_t tm_w = (int64_t)tm * TB + wm * 128, tn_w = (int64_t)tn * TBN + wn * 64;
            const bool interior = vec_store && (int64_t)tm * TB + TB <= g.M && (int64_t)tn * TBN + TBN <= g.N;
            const bool has_bias = ex.bias != nullptr;
            const int c8 = lane & 7;                       // 8 hidden units from 8*c8
            float bg[8], bu[8];
            if (has_bias) {
                const __bf16 *bb = (const __bf16 *)ex.bias + (int64_t)shard * ex.bias_shard;
                const int64_t n = tn_w + c8 * 8;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    bg[e] = n + e < g.N ? (float)bb[n + e] : 0.0f;
                    bu[e] = n + e < g.N ? (float)bb[ex.up_off + n + e] : 0.0f;
                }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < 8; ++i) *(LDS_PTR(f32x4))sw_addr(frow, i * 4 + fq) = acc[i][j];
                // both row groups' LDS reads first, then the unit and the stores
                f32x4 gq[2][2], uq[2][2];
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const int rr = p * 8 + (lane >> 3);
                    gq[p][0] = *(LDS_PTR(f32x4))sw_addr(rr, 2 * c8);
                    gq[p][1] = *(LDS_PTR(f32x4))sw_addr(rr, 2 * c8 + 1);
                    uq[p][0] = *(LDS_PTR(f32x4))sw_addr(rr, 16 + 2 * c8);
                    uq[p][1] = *(LDS_PTR(f32x4))sw_addr(rr, 16 + 2 * c8 + 1);
                }
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const int rr = p * 8 + (lane >> 3);
                    bf16x8 hv;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float gg = gq[p][e >> 2][e & 3], uu = uq[p][e >> 2][e & 3];
                        if (has_bias) {
                            gg = gg + bg[e];
                            uu = uu + bu[e];
                        }
                        hv[e] = (__bf16)(silu_f32(gg) * uu);
                    }
                    const int64_t m = tm_w + j * 16 + rr, n = tn_w + c8 * 8;
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
        __builtin_amdgcn_sched_barrier(0);
        drained = false;
    }
    // No DMA load may still be writing LDS when the workgroup ends.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

bool gemm_tile_supported(const GemmArgs &g, const GemmExtra *ex) {
    // 32-bit per-lane offsets: one tile's rows must span < 2 GiB (for the
    // gated unit, up to the up rows of the tile).
    const int64_t wspan = TB + (ex && ex->act == ACT_SWIGLU ? ex->up_off : 0);
    const bool small_rows = (int64_t)TB * g.lda * 2 < (1ll << 31) &&
                            wspan * g.ldb * 2 < (1ll << 31);
    bool ok = g.K > 0 && g.K % 64 == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 &&
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
    gemm_tile_kernel<OUT, EPI, XG><<<dim3(grid), dim3(TT), 0, s>>>(g, ts, vec, ex);
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
