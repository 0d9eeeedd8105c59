// Grouped bf16 shard GEMM on the gfx950 matrix cores: C_i = A_i B_i^T for all
// P shards in one launch ("模型并行", "Tensor Parallel": the column products
// Y_i = X W_i and the row partials X_i W_i; both operands are K-contiguous in
// the [N, K] weight storage, so no transpose is needed).
//
// Workgroup tile 256 (M) x 256 (N), K step 64, 256 threads = 4 waves in a
// 2x2 grid, each wave owning a 128x128 block = 4x4 v_mfma_f32_32x32x16_bf16
// accumulators (256 fp32 registers per lane).  The W tile is the MFMA row
// operand and the X tile the column operand, so each lane ends up holding
// 4 consecutive output columns of one row: 16-byte fp32 / 8-byte bf16 stores.
//
// Global -> LDS: global_load_lds_dwordx4 (16 bytes per lane straight into LDS,
// no register staging).  One wave instruction fills 1 KB = 8 LDS rows of
// 128 bytes (64 bf16 of K).  Within a row the 16-byte chunk holding k-chunk c
// sits at slot c ^ (row & 7); the lanes choose their global addresses to
// produce that swizzle, so the 32 lanes of a fragment read (32 rows, one
// chunk each) hit 8 different 16-byte slots per group of 8 rows.
// Two LDS stages (2 x 64 KB): the loads for step k+1 are in flight while
// step k is multiplied; one barrier per step.
//
// Edges: rows past M or N are clamped to the last valid row (their results
// are not stored).  K must be a multiple of 64; other K go to the generic
// kernel.
//
// Tile order: workgroup b runs on XCD b % 8, so b is remapped to give each
// XCD a contiguous range of tiles, and tiles inside a shard are visited in
// groups of 8 tile-rows so the workgroups resident on one XCD share X and W
// panels in that XCD's L2.
#include "kernels.h"

namespace tpl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T) __attribute__((address_space(3))) T *

constexpr int TB = 256;          // tile edge in M and N
constexpr int TK = 64;           // K per stage
constexpr int TT = 256;          // threads
constexpr int OPB = TB * TK * 2; // bytes of one operand tile (32 KB)
constexpr int STAGE = 2 * OPB;   // A tile + B tile
constexpr int GROUP_M = 8;

// Issue the 8 direct-to-LDS loads of this wave for one operand tile.
// base: the operand's row 0 of this tile at k = k0 (uniform).
// off[j]: this lane's byte offset for load j (row clamp and swizzle applied).
__device__ __forceinline__ void issue_tile(const char *base, const uint32_t (&off)[8],
                                           LDS_PTR(char) dst, int wave) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        __builtin_amdgcn_global_load_lds((const void *)(base + off[j]),
                                         (LDS_PTR(void))(dst + (j * 4 + wave) * 1024), 16, 0, 0);
    }
}

template <int OUT>
__global__ __attribute__((amdgpu_flat_work_group_size(TT, TT), amdgpu_waves_per_eu(1, 1)))
void gemm_tile_kernel(GemmArgs g, int tiles_m, int tiles_n, int vec_store) {
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

    // ---- tile index: XCD-contiguous ranges, then grouped order in a shard.
    const int T = gridDim.x;
    const int b = blockIdx.x;
    const int logical = (T % 8 == 0) ? (b % 8) * (T / 8) + (b / 8) : b;
    const int per_shard = tiles_m * tiles_n;
    const int shard = logical / per_shard;
    const int t = logical - shard * per_shard;
    const int in_group = GROUP_M * tiles_n;
    const int first_m = (t / in_group) * GROUP_M;
    const int gsz = min(tiles_m - first_m, GROUP_M);
    const int tr = t % in_group;
    const int tile_m = first_m + tr % gsz;
    const int tile_n = tr / gsz;
    const int64_t m0 = (int64_t)tile_m * TB;
    const int64_t n0 = (int64_t)tile_n * TB;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    const char *Abase = (const char *)((const __bf16 *)g.A + (int64_t)shard * g.a_shard + m0 * g.lda);
    const char *Bbase = (const char *)((const __bf16 *)g.B + (int64_t)shard * g.b_shard + n0 * g.ldb);
    const int a_rows = (int)min<int64_t>(g.M - m0, TB);
    const int b_rows = (int)min<int64_t>(g.N - n0, TB);

    // Per-lane byte offsets of the 8 loads per operand: load j of wave w fills
    // LDS rows (4j + w)*8 .. +7; lane takes row +lane/8, LDS slot lane%8,
    // which must hold k-chunk slot ^ (row & 7) = (lane%8) ^ (lane/8).
    uint32_t aoff[8], boff[8];
    {
        const int sub = lane >> 3;
        const int chunk = (lane & 7) ^ sub;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = (j * 4 + wave) * 8 + sub;
            const int ra = r < a_rows ? r : a_rows - 1;
            const int rb = r < b_rows ? r : b_rows - 1;
            aoff[j] = (uint32_t)(((int64_t)ra * g.lda + chunk * 8) * 2);
            boff[j] = (uint32_t)(((int64_t)rb * g.ldb + chunk * 8) * 2);
        }
    }

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    LDS_PTR(char) lds = (LDS_PTR(char))smem;
    const int nk = (int)(g.K / TK);

    if (nk > 0) {
        issue_tile(Abase, aoff, lds, wave);
        issue_tile(Bbase, boff, lds + OPB, wave);
    }

    // Fragment addressing: a 32x32x16 operand fragment is 32 rows x 16 k;
    // lane reads row lane%32, k-chunk 2*ks + lane/32 (8 bf16 = 16 bytes),
    // stored at slot chunk ^ (row & 7) = chunk ^ (lane & 7).
    const int frow = lane & 31;
    const int fhalf = lane >> 5;
    const int fx = lane & 7;
    const int wrow_off = (wn * 128 + frow) * 128;
    const int xrow_off = (wm * 128 + frow) * 128;

    for (int kt = 0; kt < nk; ++kt) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        LDS_PTR(char) As = lds + (kt & 1) * STAGE;
        LDS_PTR(char) Bs = As + OPB;

        bf16x8 wf[2][4], xf[2][4];
        {
            const int slot = (fhalf ^ fx) << 4;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                wf[0][i] = *(LDS_PTR(bf16x8))(Bs + wrow_off + i * 4096 + slot);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                xf[0][j] = *(LDS_PTR(bf16x8))(As + xrow_off + j * 4096 + slot);
        }
        // Phase ks: issue the fragment reads of step ks+1, then the 16
        // independent MFMAs of step ks, whose operands were read one phase
        // earlier.  The fences keep the compiler from mixing phases (which
        // would put dependent MFMAs back to back).
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            __builtin_amdgcn_sched_barrier(0);
            const int cur = ks & 1, nx = cur ^ 1;
            if (ks == 0) {
                // Prefetch the next K step into the idle stage.  The last
                // step reloads its own K range there instead, so the body
                // has no branch; that stage is not read again.
                const int kn = kt + 1 < nk ? kt + 1 : kt;
                const int64_t kb = (int64_t)kn * TK * 2;
                LDS_PTR(char) nxt = lds + ((kt + 1) & 1) * STAGE;
                issue_tile(Abase + kb, aoff, nxt, wave);
                issue_tile(Bbase + kb, boff, nxt + OPB, wave);
            }
            if (ks < 3) {
                const int slot = ((2 * (ks + 1) + fhalf) ^ fx) << 4;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    wf[nx][i] = *(LDS_PTR(bf16x8))(Bs + wrow_off + i * 4096 + slot);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    xf[nx][j] = *(LDS_PTR(bf16x8))(As + xrow_off + j * 4096 + slot);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cur][i], xf[cur][j],
                                                                        acc[i][j], 0, 0, 0);
            // One MFMA first (it consumes the reads of the previous phase, so
            // the wait for them never also covers the new ones: at most 8
            // LDS reads are in flight, within what lgkmcnt can count), then
            // the next step's 8 reads, then the other 15 MFMAs.  Phase 0
            // first issues the 16 global->LDS loads of the next K step.
            if (ks == 0) __builtin_amdgcn_sched_group_barrier(0x020, 16, 0);  // VMEM read
            if (ks < 3) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // DS read
                __builtin_amdgcn_sched_group_barrier(0x008, 15, 0);
            } else {
                __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    // No global->LDS load may still be writing when the workgroup ends.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- epilogue.  32x32 D layout with W rows as the row operand:
    // lane holds m = lane%32 and, for q = 0..3, the 4 columns
    // n = 8q + 4*(lane/32) + 0..3 in registers 4q..4q+3.
    const int64_t cbase = (int64_t)shard * g.c_shard;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t m = m0 + wm * 128 + j * 32 + frow;
        if (m >= g.M) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = n0 + wn * 128 + i * 32 + 8 * q + 4 * fhalf;
                const int64_t o = cbase + m * g.ldc + n;
                f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                           acc[i][j][4 * q + 3]};
                if (vec_store && n + 3 < g.N) {
                    if (OUT == OUT_BF16) {
                        bf16x4 h = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
                        *(bf16x4 *)((__bf16 *)g.C + o) = h;
                    } else {
                        *(f32x4 *)((float *)g.C + o) = v;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (n + e < g.N) {
                            if (OUT == OUT_BF16) ((__bf16 *)g.C)[o + e] = (__bf16)v[e];
                            else ((float *)g.C)[o + e] = v[e];
                        }
                    }
                }
            }
        }
    }
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

bool gemm_tile_supported(const GemmArgs &g) {
    // 32-bit per-lane offsets: one tile's rows must span < 4 GiB.
    const bool small_rows = (int64_t)TB * (g.lda > g.ldb ? g.lda : g.ldb) * 2 < (1ll << 31);
    return g.K % TK == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 && g.a_shard % 8 == 0 &&
           g.b_shard % 8 == 0 && aligned16(g.A) && aligned16(g.B) && small_rows;
}

hipError_t launch_gemm_tile(const GemmArgs &g, int out_type, hipStream_t s) {
    if (g.M == 0 || g.N == 0 || g.P == 0) return hipSuccess;
    const int64_t tm = (g.M + TB - 1) / TB, tn = (g.N + TB - 1) / TB;
    const int64_t blocks = tm * tn * g.P;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidConfiguration;
    const int esz = out_type == OUT_BF16 ? 2 : 4;
    const int vec = (g.ldc % 4 == 0) && (g.c_shard % 4 == 0) &&
                    (((uintptr_t)g.C) % (uintptr_t)(4 * esz) == 0);
    dim3 grid((unsigned)blocks), block(TT);
    if (out_type == OUT_BF16)
        gemm_tile_kernel<OUT_BF16><<<grid, block, 0, s>>>(g, (int)tm, (int)tn, vec);
    else
        gemm_tile_kernel<OUT_F32><<<grid, block, 0, s>>>(g, (int)tm, (int)tn, vec);
    return hipGetLastError();
}

}  // namespace tpl
