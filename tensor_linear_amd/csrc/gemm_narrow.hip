// Column shard GEMM (and row partials) on narrow output tiles, for launches
// whose 256 x 256 tiles would fill at most half of the CUs ("模型并行",
// "Tensor Parallel": the per-shard products Y_i = X W_i and X_i W_i).  Each
// wave owns a 64 x 64 block of 4 x 4 v_mfma_f32_16x16x32_bf16 blocks (64 x
// 32 in the 64-column tiles), with the instruction and the K order of the
// 256 x 256 tile kernel, so every output is bitwise the same.  Three tile
// shapes:
//  - 128 x 128 tiles, four waves in a 2 x 2 grid, when they fit in one pass
//    over the CUs (up to 128 tokens, and up to 256 when the N side is short):
//    no MFMA work on rows past M, twice the workgroups of 256-row tiles
//    where M > 128;
//  - 128 x 64 tiles where 128 x 128 ones would fill at most half of the CUs:
//    each wave a 64 x 32 block (4 x 2 MFMA blocks), twice the workgroups
//    again;
//  - else 256 x 128 tiles, eight waves in a 4 x 2 grid, two per SIMD: the
//    second wave on each SIMD issues its MFMAs while the first waits on its
//    LDS reads and loads.
// Epilogues: bf16 (+ the column bias), fp32 partials, or the gated unit of a
// fused gate+up layer (128-column W tiles: half gate rows, half the up rows
// of the same hidden units, the tile kernel's arithmetic).
//
// Pipeline (the fold-in-registers kernel's eight-wave form, without the
// fold): three stages of 64 K columns for both operands (3 x (32 + 16) KB,
// 3 x (16 + 16) KB or 3 x (16 + 8) KB), 128-byte LDS rows with 16-byte chunk c
// of row r at slot c ^ ((r / 2) % 8), global -> LDS with
// global_load_lds_dwordx4.  Per K step each wave issues 32 MFMAs (16 with
// 64 columns) in two substeps of 32 K: during substep 0 it reads its
// substep-1 fragments and issues all of step it+2's loads (6 per wave with
// 256 rows, 8 with 128, 6 with 64 columns) into the stage step it-1 freed;
// then the step's one barrier; during substep 1 it reads the next step's
// substep-0 fragments.  Persistent workgroups walk an XCD-contiguous range
// of (shard, tile) pairs; the K pipeline runs across tiles.
#include "kernels.h"

namespace tpl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T) __attribute__((address_space(3))) T *

constexpr int FBK = 64;   // K columns per stage
constexpr int FGROUP = 4; // tile rows visited as a group

struct NarrowSched {
    int tiles_m, tiles_n;  // per shard
    int T;                 // tiles over all shards
    int xcd_split, per_xcd;
};

// Tile index -> (shard, tile row, tile column), tile rows grouped by FGROUP.
__device__ __forceinline__ void narrow_decode(const NarrowSched &ts, int t, int &shard, int &tm,
                                              int &tn) {
    const int per_shard = ts.tiles_m * ts.tiles_n;
    shard = t / per_shard;
    t -= shard * per_shard;
    const int in_group = FGROUP * ts.tiles_n;
    const int first_m = (t / in_group) * FGROUP;
    const int gsz = min(ts.tiles_m - first_m, FGROUP);
    const int tr = t - (t / in_group) * in_group;
    tm = first_m + tr % gsz;
    tn = tr / gsz;
}

// The q-th tile of this workgroup, or -1 when it has none.
__device__ __forceinline__ int narrow_tile_of(const NarrowSched &ts, int q) {
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

// FM: tile rows, 256 (eight waves, two per SIMD) or 128 (four waves).
// TN: tile columns (W rows), 128 or (with 128 rows) 64.
// SW: the gated unit of a fused gate+up layer: of each wave's four W blocks
// two are gate rows and two the up rows (up_off further on) of the same 32
// hidden units, so a tile gives TN / 2 outputs silu(g + bg) * (u + bu).
template <int OUT, int FM, int TN, bool SW = false>
__global__ __attribute__((amdgpu_flat_work_group_size(FM * 2, FM * 2),
                          amdgpu_waves_per_eu(FM / 128, FM / 128)))
void gemm_narrow_kernel(GemmArgs g, NarrowSched ts, const __bf16 *bias_all, int64_t bias_shard,
                        int vec_store, int64_t up_off) {
    static_assert(TN == 128 || (TN == 64 && FM == 128), "tile shapes");
    static_assert(!SW || (TN == 128 && OUT == OUT_BF16), "the gated unit: 128 W rows, bf16 out");
    constexpr int TBN = SW ? TN / 2 : TN;  // output columns per tile
    constexpr int NW = FM / 32;            // waves
    constexpr int WI = TN / 32;            // 16-column W blocks per wave
    constexpr int NF = WI + 4;             // fragments per substep
    constexpr int NU = 4 * WI;             // MFMAs per substep
    constexpr int ROWB = FBK * 2;          // 128 bytes per LDS row
    constexpr int OPX = FM * ROWB;         // X stage, 32 or 16 KB
    constexpr int OPW = TN * ROWB;         // W stage, 16 or 8 KB
    constexpr int W_BASE = 3 * OPX;        // three X stages, then three W stages
    constexpr int LX = OPX / 1024 / NW;    // X loads per wave per step (4)
    constexpr int LW = OPW / 1024 / NW;    // W loads per wave per step (2 or 4)
    __shared__ __attribute__((aligned(1024))) char smem[3 * OPX + 3 * OPW];
    LDS_PTR(char) lds = (LDS_PTR(char))smem;
    const uint32_t lds_u = (uint32_t)(uintptr_t)lds;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;   // 64 tokens x 64 features each

    int ntiles = 0;
    while (narrow_tile_of(ts, ntiles) >= 0) ++ntiles;
    if (ntiles == 0) return;
    const int nk = (int)(g.K / FBK);       // K steps per tile
    const int total = ntiles * nk;

    // ---- load cursor: (tile pq of shard psh, step pkt), two steps ahead of
    // the compute; past the last step it stays there, so later issues reload
    // the last step into stages that are not read again.
    int pq = 0, psh = 0, pkt = 0, pstep = 0;
    int64_t pm0 = 0, pn0 = 0;
    const char *pa = nullptr, *pb = nullptr;
    uint32_t aoff[LX], boff[LW];
    auto enter_tile = [&](int q) {
        int tm, tn;
        narrow_decode(ts, narrow_tile_of(ts, q), psh, tm, tn);
        pm0 = (int64_t)tm * FM;
        pn0 = (int64_t)tn * TBN;
        const int a_rows = (int)min<int64_t>(g.M - pm0, FM);
        const int b_rows = (int)min<int64_t>(g.N - pn0, TBN);
#pragma unroll
        for (int j = 0; j < LX; ++j) {
            const int r = (j * NW + wave) * 8 + lane / 8;
            const int chunk = (lane % 8) ^ ((r / 2) % 8);
            const int ra = r < a_rows ? r : a_rows - 1;
            aoff[j] = (uint32_t)(((int64_t)ra * g.lda + chunk * 8) * 2);
        }
#pragma unroll
        for (int j = 0; j < LW; ++j) {
            const int r = (j * NW + wave) * 8 + lane / 8;
            const int chunk = (lane % 8) ^ ((r / 2) % 8);
            int64_t rb;
            if constexpr (SW) {
                // LDS row r feeds wave column r / 64, W block (r / 16) % 4:
                // blocks 0-1 gate rows, 2-3 the up rows of the same 32 units.
                int h = ((r >> 6) << 5) + (((r >> 4) & 1) << 4) + (r & 15);
                h = h < b_rows ? h : b_rows - 1;
                rb = h + (((r >> 4) & 2) ? up_off : 0);
            } else {
                rb = r < b_rows ? r : b_rows - 1;
            }
            boff[j] = (uint32_t)((rb * g.ldb + chunk * 8) * 2);
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
                ++pq;
                enter_tile(pq);
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
    // Load l (0 .. LX+LW-1) of the cursor's step into stage `slot`: the
    // first LX the X tile (1 KB chunks NW*l + wave), then the W tile.
    auto load = [&](int slot, int l) __attribute__((always_inline)) {
        if (l < LX)
            dma(pa + (int64_t)pkt * 128, aoff[l], lds_u + slot * OPX + (l * NW + wave) * 1024);
        else
            dma(pb + (int64_t)pkt * 128, boff[l - LX],
                lds_u + W_BASE + slot * OPW + ((l - LX) * NW + wave) * 1024);
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
    const uint32_t wrow_off = (wn * (TN / 2) + frow) * ROWB;
    const uint32_t xrow_off = (wm * 64 + frow) * ROWB;
    auto frag_addr = [&](int stage, int f, int h) -> uint32_t {
        const uint32_t slot = (uint32_t)(((4 * h + fq) ^ fx) << 4);
        if (f < WI) return W_BASE + stage * OPW + wrow_off + f * 16 * ROWB + slot;
        return stage * OPX + xrow_off + (f - WI) * 16 * ROWB + slot;
    };
    bf16x8 fr[2][NF];
    auto read_frag = [&](int h, int f, uint32_t addr) __attribute__((always_inline)) {
        fr[h][f] = *(LDS_PTR(bf16x8))(lds + addr);
    };
#pragma unroll
    for (int f = 0; f < NF; ++f) read_frag(0, f, frag_addr(0, f, 0));

    int s0 = 0;                 // stage of the current step (step index % 3)
    bool drained = true;        // no epilogue store is in flight
    f32x4 acc[WI][4];
    for (int q = 0; q < ntiles; ++q) {
        {
            auto kstep = [&](auto first) __attribute__((always_inline)) {
                constexpr bool FIRST = decltype(first)::value;
                const int s1 = s0 == 2 ? 0 : s0 + 1;   // stage of step it+1
                const int s2 = s1 == 2 ? 0 : s1 + 1;   // stage of step it+2 (= it-1's)
                // substep 0: the substep-1 fragments, step it+2's loads
#pragma unroll
                for (int u = 0; u < NU; ++u) {
                    __builtin_amdgcn_sched_barrier(0);
                    const int i = u % WI, j = u / WI;
                    if (FIRST)   // the shard's first product of each block: C = 0
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[0][i], fr[0][WI + j], f32x4{}, 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[0][i], fr[0][WI + j], acc[i][j], 0, 0, 0);
                    const bool rd = NU >= 2 * NF ? (u & 1) == 0 : u < NF;
                    const int ri = NU >= 2 * NF ? u >> 1 : u;
                    if (rd) read_frag(1, ri, frag_addr(s0, ri, 1));
                    // step it+2's loads, X then W: six at MFMAs 1, 3, 6, 9,
                    // 11, 14 (256 rows), eight at the odd MFMAs (128 rows)
                    // or six at MFMAs 1-6 (64 columns)
                    const int li = NU == 8 ? (u >= 1 && u <= LX + LW ? u - 1 : -1)
                                 : LX + LW == 8 ? ((u & 1) ? (u >> 1) : -1)
                                 : u == 1 ? 0 : u == 3 ? 1 : u == 6 ? 2 : u == 9 ? 3 : u == 11 ? 4 : u == 14 ? 5 : -1;
                    if (li >= 0) load(s2, li);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    if (rd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
                }
                __builtin_amdgcn_sched_barrier(0);
                // Step it+1's loads (issued in step it-1) have landed; step
                // it+2's may stay in flight.  This wave's reads of
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
                for (int u = 0; u < NU; ++u) {
                    __builtin_amdgcn_sched_barrier(0);
                    const int i = u % WI, j = u / WI;
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[1][i], fr[1][WI + j], acc[i][j], 0, 0, 0);
                    const bool rd = NU >= 2 * NF ? (u & 1) == 0 : u < NF;
                    const int ri = NU >= 2 * NF ? u >> 1 : u;
                    if (rd) read_frag(0, ri, frag_addr(s1, ri, 0));
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    if (rd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
                }
                __builtin_amdgcn_sched_barrier(0);
                advance();
                s0 = s1;
            };
            kstep(std::true_type{});
            for (int kt = 1; kt < nk; ++kt) kstep(std::false_type{});
        }

        // ---- epilogue: acc (+ bias) -> the output type.  acc[i][j][r] =
        // C[m = 16j + lane%16][n = 16i + 4*(lane/16) + r] of the wave's block.
        // 16 rows x 64 (or 32) columns at a time go through this wave's 1 KB chunks
        // w + NW*c (c = 0..3) of the X stage of the tile's last step (read by
        // everyone before that step's barrier; only this wave's own later
        // loads write these chunks): staging row r of 256 bytes at chunk r/4,
        // offset (r%4)*256, 16-byte slot s at s ^ (r % 16).  Then each lane
        // holds 8 consecutive bf16 outputs of a row (a 64-column row leaves as
        // one 128-byte line, a 32-column one as half of one) or 4
        // consecutive fp32 ones (two lines, or one).
        __builtin_amdgcn_sched_barrier(0);
        int shard, tm, tn;
        narrow_decode(ts, narrow_tile_of(ts, q), shard, tm, tn);
        const int es = s0 == 0 ? 2 : s0 - 1;
        LDS_PTR(char) ep = lds + es * OPX + wave * 1024;
        auto st_addr = [&](int r, int s) -> LDS_PTR(char) {
            return ep + (r >> 2) * (NW * 1024) + (r & 3) * 256 + ((s ^ (r & 15)) << 4);
        };
        const int64_t m_t = (int64_t)tm * FM, tm_w = m_t + wm * 64, tn_w = (int64_t)tn * TBN + wn * (TBN / 2);
        const int64_t cbase = (int64_t)shard * g.c_shard;
        const __bf16 *bias = bias_all ? bias_all + (int64_t)shard * bias_shard : nullptr;
        constexpr int LPR8 = 2 * WI;            // lanes per staged row, 8 bf16 each
        constexpr int RPP8 = 64 / LPR8;         // rows per pass
        const int c8 = lane % LPR8;
        const int64_t ncol = tn_w + c8 * 8;
        float bv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) bv[e] = bias && ncol + e < g.N ? (float)bias[ncol + e] : 0.0f;
        // gated unit: lane takes 8 hidden units from 8 * (lane % 4) of row lane / 4
        const int64_t nsw = tn_w + (lane & 3) * 8;
        float bg[8], bu[8];
        if constexpr (SW) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bg[e] = bias && nsw + e < g.N ? (float)bias[nsw + e] : 0.0f;
                bu[e] = bias && nsw + e < g.N ? (float)bias[up_off + nsw + e] : 0.0f;
            }
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {        // rows 16jj.. of the wave
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int bi = 0; bi < WI; ++bi)
                *(LDS_PTR(f32x4))st_addr(frow, bi * 4 + fq) = acc[bi][jj];
            if constexpr (SW) {
                // gate units 0-31 in slots 0-7, the up units in slots 8-15
                const int rr = lane >> 2, c4 = lane & 3;
                const f32x4 g0 = *(LDS_PTR(f32x4))st_addr(rr, 2 * c4);
                const f32x4 g1 = *(LDS_PTR(f32x4))st_addr(rr, 2 * c4 + 1);
                const f32x4 u0 = *(LDS_PTR(f32x4))st_addr(rr, 8 + 2 * c4);
                const f32x4 u1 = *(LDS_PTR(f32x4))st_addr(rr, 8 + 2 * c4 + 1);
                const int64_t m = tm_w + jj * 16 + rr;
                if (m >= g.M) continue;
                bf16x8 hv;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float gg = e < 4 ? g0[e] : g1[e - 4], uu = e < 4 ? u0[e] : u1[e - 4];
                    if (bias) {
                        gg = gg + bg[e];
                        uu = uu + bu[e];
                    }
                    hv[e] = (__bf16)(silu_f32(gg) * uu);
                }
                __bf16 *row = (__bf16 *)g.C + cbase + m * g.ldc;
                if (vec_store && nsw + 8 <= g.N) {
                    __builtin_nontemporal_store(hv, (bf16x8 *)(row + nsw));
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (nsw + e < g.N) row[nsw + e] = hv[e];
                }
                continue;
            }
            if constexpr (OUT == OUT_F32) {
                constexpr int LPR4 = 4 * WI;        // lanes per staged row, 4 fp32 each
                constexpr int RPP4 = 64 / LPR4;     // rows per pass
                const int c16 = lane % LPR4;
                f32x4 a[16 / RPP4];
#pragma unroll
                for (int p = 0; p < 16 / RPP4; ++p) a[p] = *(LDS_PTR(f32x4))st_addr(p * RPP4 + lane / LPR4, c16);
#pragma unroll
                for (int p = 0; p < 16 / RPP4; ++p) {
                    const int64_t m = tm_w + jj * 16 + p * RPP4 + lane / LPR4, n = tn_w + c16 * 4;
                    if (m >= g.M) continue;
                    float *dst = (float *)g.C + cbase + m * g.ldc + n;
                    if (vec_store && n + 4 <= g.N) {
                        __builtin_nontemporal_store(a[p], (f32x4 *)dst);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < g.N) dst[e] = a[p][e];
                    }
                }
                continue;
            }
            f32x4 a0[16 / RPP8], a1[16 / RPP8];
#pragma unroll
            for (int p = 0; p < 16 / RPP8; ++p) {
                const int rr = p * RPP8 + lane / LPR8;
                a0[p] = *(LDS_PTR(f32x4))st_addr(rr, 2 * c8);
                a1[p] = *(LDS_PTR(f32x4))st_addr(rr, 2 * c8 + 1);
            }
#pragma unroll
            for (int p = 0; p < 16 / RPP8; ++p) {
                const int rr = p * RPP8 + lane / LPR8;
                const int64_t m = tm_w + jj * 16 + rr;
                if (m >= g.M) continue;
                float v[8] = {a0[p][0], a0[p][1], a0[p][2], a0[p][3], a1[p][0], a1[p][1], a1[p][2], a1[p][3]};
                bf16x8 hv;
#pragma unroll
                for (int e = 0; e < 8; ++e) hv[e] = (__bf16)(bias ? v[e] + bv[e] : v[e]);
                __bf16 *row = (__bf16 *)g.C + cbase + m * g.ldc;
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

hipError_t launch_gemm_narrow(const GemmArgs &g, int out_type, const GemmExtra *exp,
                              hipStream_t s) {
    if (g.M == 0 || g.N == 0 || g.P == 0) return hipSuccess;
    GemmExtra ex{};
    if (exp) ex = *exp;
    const bool sw = ex.act == ACT_SWIGLU;
    if ((ex.act != ACT_NONE && !sw) || ex.x_rows > 0 || (out_type != OUT_BF16 && (ex.bias || sw)))
        return hipErrorInvalidValue;
    // 128-row tiles when they fit in one pass over the CUs, else 256-row.
    // Same-box A/B, 8 shards, us after a read-only 1 GiB cache flush / warm,
    // 128-row vs 256-row tiles: M = 128, 4096 -> 28672: 61.6 / 41.0 vs
    // 65.5 / 56.9; M = 65, 8192 -> 10240: 74.2 / 54.6 vs 91.7 / 88.3;
    // M = 256, 8192 -> 10240: 83.9 / 62.0 vs 110.7 / 88.6; M = 200,
    // 4096 -> 14336: 49.0 / 41.6 vs 57.6 / 49.4.  Bitwise equal.
    const int cus = device_cu_count();
    const int64_t tn128 = sw ? (g.N + 63) / 64 : (g.N + 127) / 128;   // tiles of 128 W rows
    const int FM = ((g.M + 127) / 128) * tn128 * g.P <= cus ? 128 : 256;
    const int64_t tm = (g.M + FM - 1) / FM;
    // 64-column tiles where 128 x 128 ones would fill at most half of the
    // CUs.  Same box, 8 shards, us after a read-only 1 GiB flush / warm, 64-
    // vs 128-column tiles: M = 65, 8192 -> 10240 65.6 / 48.4 vs 74.5 / 55.6;
    // M = 128 70.1 / 51.6 vs 81.5 / 55.8; M = 128, 4096 -> 4096 36.9 / 27.3
    // vs 43.3 / 30.9; row partials M = 128, 8192 -> 2048 15.0 / 12.2 vs
    // 17.7 / 14.4.  Bitwise equal.
    const int TN = (!sw && FM == 128 && 2 * tm * tn128 * g.P <= cus) ? 64 : 128;
    const int64_t tn = sw ? tn128 : (g.N + TN - 1) / TN;
    const int64_t T = tm * tn * g.P;
    if (T > 0x7FFFFFFFll) return hipErrorInvalidConfiguration;
    NarrowSched ts;
    ts.tiles_m = (int)tm;
    ts.tiles_n = (int)tn;
    ts.T = (int)T;
    const int grid = (int)(T < cus ? T : cus);
    ts.xcd_split = (grid == cus && cus % 8 == 0 && T >= cus) ? 1 : 0;
    ts.per_xcd = grid / 8;
    const int vw = out_type == OUT_BF16 ? 8 : 4;
    const int vec = g.ldc % vw == 0 && g.c_shard % vw == 0 && aligned16(g.C);
    const __bf16 *bias = (const __bf16 *)ex.bias;
    const int64_t uo = ex.up_off;
    if (sw) {
        if (FM == 128)
            gemm_narrow_kernel<OUT_BF16, 128, 128, true><<<dim3(grid), dim3(256), 0, s>>>(g, ts, bias, ex.bias_shard, vec, uo);
        else
            gemm_narrow_kernel<OUT_BF16, 256, 128, true><<<dim3(grid), dim3(512), 0, s>>>(g, ts, bias, ex.bias_shard, vec, uo);
    } else if (TN == 64) {
        if (out_type == OUT_BF16)
            gemm_narrow_kernel<OUT_BF16, 128, 64><<<dim3(grid), dim3(256), 0, s>>>(g, ts, bias, ex.bias_shard, vec, 0);
        else
            gemm_narrow_kernel<OUT_F32, 128, 64><<<dim3(grid), dim3(256), 0, s>>>(g, ts, nullptr, 0, vec, 0);
    } else if (FM == 128) {
        if (out_type == OUT_BF16)
            gemm_narrow_kernel<OUT_BF16, 128, 128><<<dim3(grid), dim3(256), 0, s>>>(g, ts, bias, ex.bias_shard, vec, 0);
        else
            gemm_narrow_kernel<OUT_F32, 128, 128><<<dim3(grid), dim3(256), 0, s>>>(g, ts, nullptr, 0, vec, 0);
    } else if (out_type == OUT_BF16) {
        gemm_narrow_kernel<OUT_BF16, 256, 128><<<dim3(grid), dim3(512), 0, s>>>(g, ts, bias, ex.bias_shard, vec, 0);
    } else {
        gemm_narrow_kernel<OUT_F32, 256, 128><<<dim3(grid), dim3(512), 0, s>>>(g, ts, nullptr, 0, vec, 0);
    }
    return hipGetLastError();
}

}  // namespace tpl
