/*
 * tplinear.h -- C ABI of libtplinear, the tensor-parallel Linear Y = X W with
 * all P shards resident on one MI355X (gfx950).
 *
 * The operation ("模型并行", wineandchord.com, section "Tensor Parallel"):
 *   column parallel: W = [W_1 .. W_P] split along the output dim, Y_i = X W_i,
 *                    the Y_i concatenated (or kept as P shards);
 *   row parallel:    X = [X_1 .. X_P] and W split along the input dim,
 *                    Y = sum_i X_i W_i.
 * The reduction that would be an all-reduce or a reduce-scatter across ranks
 * ("3D 并行的实现：TP / PP / DP 各占几行", nanotron, section "5.1 TP") is an
 * on-device fold over the P shards in ascending shard order.
 *
 * Conventions used by every entry point:
 *   - Matrices are row-major with a leading dimension (row stride) given in
 *     elements.  X is [M, K], W is stored [N, K] (the [out, in] orientation
 *     of nn.Linear used by the DTorch "Linear 实现解析" section: column
 *     parallel = Shard(0) of that storage, row parallel = Shard(1)), Y is
 *     [M, N].  In the [in, out] orientation of the formula, W_io = W^T.
 *   - M = tokens, K = input features, N = output features, P = shards.
 *   - Device pointers: X, W, Y, partials and workspace live in GPU memory
 *     (hipMalloc or torch).  The caller allocates and owns every buffer.  The
 *     library never allocates or frees memory and keeps no pointer after a
 *     call returns.
 *   - Work is queued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without waiting.  Buffers must stay valid until the
 *     stream has reached the work.  Calls on one stream run in order.
 *   - Outputs must not overlap inputs.
 *   - Every argument check runs on the host before anything is queued; a
 *     failed check returns an error and queues nothing.  TP_ERR_HIP reports a
 *     failed kernel launch.
 *   - Arithmetic: bf16 inputs are multiplied and accumulated in fp32; results
 *     written as bf16 are rounded to nearest even once, at the end.  fp32
 *     inputs are multiplied and accumulated in fp32.  Row partial results are
 *     kept in fp32.
 *   - A size of 0 for M or N is valid and queues nothing.  K = 0 gives Y = 0.
 */
#ifndef TPLINEAR_H
#define TPLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TP_OK = 0,
    TP_ERR_NULL = 1,         /* a required pointer is NULL                          */
    TP_ERR_SHAPE = 2,        /* negative size, leading dim too small, P out of range,
                                a buffer of more than 2^60 elements (or workspace bytes) */
    TP_ERR_INDIVISIBLE = 3,  /* the split dim is not a multiple of P                 */
    TP_ERR_PLACEMENT = 4,    /* unknown placement kind, or dim out of range          */
    TP_ERR_DTYPE = 5,        /* unknown dtype                                        */
    TP_ERR_MODE = 6,         /* unknown y_mode / row mode                            */
    TP_ERR_WORKSPACE = 7,    /* workspace NULL or smaller than required              */
    TP_ERR_HIP = 8           /* a HIP call or kernel launch failed                   */
} tp_status;

typedef enum { TP_F32 = 0, TP_BF16 = 1 } tp_dtype;

/* Placements ("DTensor API 文档", MindSpore hyper-parallel, section
 * "放置策略类型"): Shard(dim) splits the tensor along dim, Replicate() gives
 * every shard the full tensor, Partial() gives every shard a full-shape part
 * whose sum over the shards is the value. */
typedef enum { TP_REPLICATE = 0, TP_SHARD = 1, TP_PARTIAL = 2 } tp_placement_kind;

typedef struct {
    int32_t kind;  /* tp_placement_kind                                          */
    int32_t dim;   /* for TP_SHARD: 0 or 1, or -1 / -2 counted from the end      */
} tp_placement;

/* One shard's view of a row-major [rows, cols] tensor of leading dim ld. */
typedef struct {
    int64_t elem_offset;  /* offset of view[0,0] from the tensor base, elements */
    int64_t rows, cols;   /* extent of the view                                 */
    int64_t ld;           /* row stride of the view in elements (= tensor ld)   */
    int64_t row0, col0;   /* global index of view[0,0]                          */
} tp_view;

#define TP_MAX_SHARDS 64

/* Column output modes. */
enum {
    TP_Y_CONCAT = 0,  /* Y is [M, N]; shard i writes columns [i*N/P, (i+1)*N/P)     */
    TP_Y_SHARDS = 1   /* Y is P blocks [M, N/P] at Y + i*M*ldy (block row stride ldy) */
};

/* Row modes. */
enum {
    TP_ROW_PARTIAL = 0,  /* Y = P fp32 partials, part i at (float*)Y + i*M*ldy        */
    TP_ROW_SUM = 1,      /* Y [M, N] = fold of the partials (partials in workspace)   */
    TP_ROW_FUSED = 2,    /* as TP_ROW_SUM, the fold done inside the GEMM's epilogue   */
    TP_ROW_SCATTER = 3   /* Y = P token slices of the fold (reduce-scatter over dim 0) */
};

/*
 * tp_shard_layout -- the P shard views of a row-major [rows, cols] tensor of
 * leading dimension ld under one placement.  Host only; touches no GPU.
 *
 * Follows "DTensor API 文档", sections "distribute_tensor" (every device holds
 * the global tensor and keeps the slice its placement gives it; the printed
 * 4x4 example gives the first two rows to the first shard along the mesh dim
 * and the last two to the second) and "shape"/"local_shape", with the
 * even-split rule of "模型并行", "Tensor-parallel 线性层" (the split dim must
 * divide by P; every shard covers each global index exactly once):
 *   TP_SHARD, dim 0:  views[i] = rows [i*rows/P, (i+1)*rows/P), all columns,
 *                     elem_offset = row0*ld;
 *   TP_SHARD, dim 1:  views[i] = all rows, columns [i*cols/P, (i+1)*cols/P),
 *                     elem_offset = col0;
 *   TP_REPLICATE:     views[i] = the whole tensor (elem_offset 0);
 *   TP_PARTIAL:       views[i] = a whole-shape part stored after the first i
 *                     parts: elem_offset = i*rows*ld, row0 = col0 = 0.
 * Every view keeps the tensor's ld.  The views alias the tensor; no data
 * moves (the DTensor page's to_local returns the local part with no
 * communication).
 *
 * views: caller array of P entries, written on success.
 * Errors: TP_ERR_NULL (views NULL), TP_ERR_SHAPE (rows or cols < 0,
 * ld < cols, P < 1 or P > TP_MAX_SHARDS), TP_ERR_PLACEMENT,
 * TP_ERR_INDIVISIBLE (the sharded dim is not a multiple of P).
 */
tp_status tp_shard_layout(int64_t rows, int64_t cols, int64_t ld,
                          tp_placement placement, int32_t P, tp_view *views);

/*
 * tp_linear_column -- column-parallel Linear ("模型并行", "Column parallel":
 * Y_i = X W_i; DTorch "Linear 实现解析": tp_shard_type "col", weight
 * Shard(0), input Replicate()).
 *
 * X [M, K] (ldx >= K), the same full input for every shard.  W [N, K]
 * (ldw >= K); shard i is the row block W[i*N/P : (i+1)*N/P, :].
 * y_mode TP_Y_CONCAT: Y [M, N] (ldy >= N), shard i's result written at
 *   columns [i*N/P, (i+1)*N/P) -- the concatenated, replicated output
 *   (ColumnParallelLinearWithReplicateOutput).
 * y_mode TP_Y_SHARDS: shard i's result [M, N/P] at Y + i*M*ldy with row
 *   stride ldy >= N/P -- the Shard(-1) output (ColumnParallelLinear).
 * dtype: X, W and Y all TP_BF16 or all TP_F32.  All P shards run in one
 * launch.
 * Errors: TP_ERR_NULL, TP_ERR_SHAPE, TP_ERR_INDIVISIBLE (N % P != 0),
 * TP_ERR_DTYPE, TP_ERR_MODE, TP_ERR_HIP.
 */
tp_status tp_linear_column(const void *X, int64_t ldx, const void *W, int64_t ldw,
                           void *Y, int64_t ldy, int32_t y_mode,
                           int64_t M, int64_t N, int64_t K, int32_t P,
                           int32_t dtype, void *stream);

/*
 * tp_linear_row -- row-parallel Linear ("模型并行", "Row parallel":
 * Y = sum_i X_i W_i; DTorch: tp_shard_type "row", weight Shard(1), input
 * Shard(-1); nanotron "5.1 TP": the row output is all-reduced or
 * reduce-scattered).
 *
 * X [M, K] (ldx >= K); shard i reads columns [i*K/P, (i+1)*K/P).
 * W [N, K] (ldw >= K); shard i reads the same column range.
 * Partial products X_i W_i are fp32 [M, N].
 * mode TP_ROW_PARTIAL: Y is float; part i at (float*)Y + i*M*ldy, ldy >= N
 *   (the Partial() output of RowParallelLinear).  workspace unused.
 * mode TP_ROW_SUM: Y [M, N] of dtype, ldy >= N, Y = ((p_0 + p_1) + ...) +
 *   p_{P-1} in fp32, ascending shard order, then rounded once
 *   (RowParallelLinearWithReplicateOutput; the all-reduce).  The partials are
 *   kept in the workspace.
 * mode TP_ROW_FUSED: the same result, bit for bit, as TP_ROW_SUM, with the
 *   fold inside the GEMM where that is faster: each workgroup computes all P
 *   shard partials of its output tile in ascending order and adds them into
 *   a running fp32 sum, so no partial reaches memory and the workspace is
 *   not touched.  Kernels exist for bf16 operands (16-byte aligned, leading
 *   dims and shard offsets multiples of 8) with 1 <= M <= 32 (up to 48 when
 *   K/P > 4096 or the P partials span at most CUs/2 tiles of 128 x 128), or
 *   with K/P a multiple of 64 and at most 2048 (at most 3584 when M*N >=
 *   4096*4096); they are used where they measured faster: for M <= 16 when
 *   N >= 32 x the GPU's CU count and K/P >= 2048, or N is smaller and
 *   K/P <= 1024; for
 *   M > 64 when the output has at least CUs * min(1, (K/P + 512) / 2048)
 *   tiles of 256 x 128.  Other shapes run the TP_ROW_SUM sequence in the
 *   workspace, which is therefore always required.  With the environment
 *   variable TPLINEAR_ROW_FOLD=gemm every shape a fused kernel takes runs
 *   it (same result).
 * mode TP_ROW_SCATTER: requires M % P == 0.  Token slice j = rows
 *   [j*M/P, (j+1)*M/P) of the fold is written to Y + j*y_slice_stride with
 *   row stride ldy (y_slice_stride = 0 means (M/P)*ldy, the contiguous layout
 *   whose Shard(0) views are the slices; a nonzero stride must be at least
 *   (M/P - 1)*ldy + N, so that slices do not overlap, else TP_ERR_SHAPE).
 *   The reduce-scatter over tokens.
 *   Bit for bit the rows of TP_ROW_SUM; for bf16 with K/P and the tile
 *   count as for TP_ROW_FUSED with M > 64, and M/P a multiple of 256, the
 *   fold runs inside the GEMM and the workspace is not touched.
 * y_slice_stride is ignored by the other modes.
 * workspace: device memory of ws_bytes >= tp_row_workspace_bytes(mode, M, N, P),
 *   256-byte aligned.  May be NULL when that size is 0.  Calls that share a
 *   workspace must be ordered (same stream, or synchronised).
 * dtype: X and W (and Y for SUM/FUSED/SCATTER) TP_BF16 or TP_F32.
 * Errors: TP_ERR_NULL, TP_ERR_SHAPE, TP_ERR_INDIVISIBLE (K % P, or M % P for
 * SCATTER), TP_ERR_DTYPE, TP_ERR_MODE, TP_ERR_WORKSPACE, TP_ERR_HIP.
 */
tp_status tp_linear_row(const void *X, int64_t ldx, const void *W, int64_t ldw,
                        void *Y, int64_t ldy, int64_t y_slice_stride, int32_t mode,
                        void *workspace, size_t ws_bytes,
                        int64_t M, int64_t N, int64_t K, int32_t P,
                        int32_t dtype, void *stream);

/*
 * tp_shard_reduce -- fold P fp32 partial results into one (the Partial ->
 * Replicate step of "DTensor API 文档", "reduce_partial", done on device in
 * ascending shard order; scatter = 1 is the Partial -> Shard(0) step, the
 * reduce-scatter over tokens of nanotron's REDUCE_SCATTER mode).
 *
 * partials: part i at partials + i*shard_stride (elements), [M, N] with row
 *   stride ldp >= N.
 * scatter = 0: Y [M, N] of out_dtype, row stride ldy >= N.
 * scatter = 1: requires M % P == 0; slice j (rows [j*M/P, (j+1)*M/P)) at
 *   Y + j*y_slice_stride, row stride ldy (y_slice_stride = 0 means
 *   (M/P)*ldy; a nonzero stride below (M/P - 1)*ldy + N, which would make
 *   slices overlap, is TP_ERR_SHAPE).
 * Y = ((p_0 + p_1) + p_2) + ... + p_{P-1}, fp32 adds, then one rounding to
 *   bf16 (round to nearest even) for out_dtype TP_BF16.
 * Errors: TP_ERR_NULL, TP_ERR_SHAPE, TP_ERR_INDIVISIBLE, TP_ERR_DTYPE,
 * TP_ERR_MODE (scatter not 0 or 1), TP_ERR_HIP.
 */
tp_status tp_shard_reduce(const float *partials, int64_t shard_stride, int64_t ldp,
                          void *Y, int64_t ldy, int64_t y_slice_stride, int32_t scatter,
                          int64_t M, int64_t N, int32_t P, int32_t out_dtype,
                          void *stream);

/* Column activations. */
enum {
    TP_ACT_NONE = 0,    /* Y = X W_i^T (+ bias)                                   */
    TP_ACT_SWIGLU = 1   /* the gated unit of a fused gate+up layer, see below      */
};

/*
 * tp_linear_column_ex -- tp_linear_column with a bias, the gated activation
 * of a fused gate+up layer, and an input given as token slices.
 *
 * Input: exactly one of X and x_slices is non-NULL.
 *   X: [M, K] row stride ldx, the full input (as tp_linear_column);
 *   x_slices: host array of P device pointers; slice j holds rows
 *     [j*M/P, (j+1)*M/P) of X with row stride ldx, each in its own
 *     allocation -- the Shard(0) token slices of the sequence-parallel layout
 *     ("模型并行", "Sequence Parallel": the layout is converted before a
 *     column layer; nanotron "5.1 TP": the column layer all-gathers x in
 *     REDUCE_SCATTER mode).  The slices are read in place, so the all-gather
 *     moves no bytes.  Requires M % P == 0.  The host array is read during
 *     the call and not kept.
 * bias: NULL or device [N] of dtype.  The column bias is Shard(0) ("Module
 *   并行：实现 DP/TP/CP/PP 组合", "Linear 实现解析", tp_shard_type table): shard
 *   i adds bias[i*N/P + c] to its output feature c, in fp32, before the one
 *   rounding.
 * act TP_ACT_NONE: Y as tp_linear_column, plus the bias.
 * act TP_ACT_SWIGLU: N = 2*I counts the gate and up features, N/P even.
 *   Shard i's W row block [i*N/P, (i+1)*N/P) holds its I/P gate rows first,
 *   then the I/P up rows of the same hidden units (the bias likewise).  The
 *   output is H [M, I]: y_mode TP_Y_CONCAT: ldy >= I, shard i at columns
 *   [i*I/P, (i+1)*I/P); TP_Y_SHARDS: P blocks [M, I/P] at Y + i*M*ldy,
 *   ldy >= I/P.  H = silu(G) * U with G, U the fp32 gate and up products
 *   (plus bias) and silu(g) = g / (1 + e^-g) in fp32; one rounding.
 * Other arguments and errors as tp_linear_column; also TP_ERR_NULL when both
 * or neither of X and x_slices are given (K > 0), TP_ERR_INDIVISIBLE when
 * M % P != 0 with x_slices or (N/P) % 2 != 0 with TP_ACT_SWIGLU, TP_ERR_MODE
 * for an unknown act.
 */
tp_status tp_linear_column_ex(const void *X, const void *const *x_slices, int64_t ldx,
                              const void *W, int64_t ldw, const void *bias,
                              void *Y, int64_t ldy, int32_t y_mode, int32_t act,
                              int64_t M, int64_t N, int64_t K, int32_t P,
                              int32_t dtype, void *stream);

/*
 * tp_linear_row_ex -- tp_linear_row with a bias and token slices in separate
 * allocations.
 *
 * bias: NULL or device [N] of dtype.  The row bias is Partial() ("Module
 *   并行：实现 DP/TP/CP/PP 组合", "Linear 实现解析", tp_shard_type table): its
 *   parts sum to the layer's bias, so it enters the reduced output once, as
 *   one fp32 add after the last shard and before the rounding.  Not allowed
 *   with TP_ROW_PARTIAL (TP_ERR_MODE): there it is the caller's to add.
 * y_slices: NULL, or for TP_ROW_SCATTER a host array of P device pointers;
 *   token slice j is written at y_slices[j] with row stride ldy
 *   (y_slice_stride is then ignored).  TP_ERR_MODE with another mode.
 * Other arguments and errors as tp_linear_row.
 */
tp_status tp_linear_row_ex(const void *X, int64_t ldx, const void *W, int64_t ldw,
                           const void *bias, void *Y, void *const *y_slices, int64_t ldy,
                           int64_t y_slice_stride, int32_t mode,
                           void *workspace, size_t ws_bytes,
                           int64_t M, int64_t N, int64_t K, int32_t P,
                           int32_t dtype, void *stream);

/*
 * tp_shard_reduce_ex -- tp_shard_reduce with the row bias (out_dtype, [N],
 * added once after the fold; NULL for none) and, for scatter = 1, token
 * slices in separate allocations (y_slices: NULL, or a host array of P
 * device pointers, slice j at y_slices[j] with row stride ldy; Y and
 * y_slice_stride are then ignored and Y may be NULL).  TP_ERR_MODE when
 * y_slices is given with scatter = 0.
 */
tp_status tp_shard_reduce_ex(const float *partials, int64_t shard_stride, int64_t ldp,
                             const void *bias, void *Y, void *const *y_slices, int64_t ldy,
                             int64_t y_slice_stride, int32_t scatter,
                             int64_t M, int64_t N, int32_t P, int32_t out_dtype,
                             void *stream);

/*
 * tp_embedding -- EmbeddingWithReplicateOutput ("Module 并行：实现 DP/TP/CP/PP
 * 组合", "DP / TP / CP / PP 并行实现", "Tensor Parallel": the embedding weight
 * is Shard(1) on embedding_dim, the token ids are Replicate, and the output
 * is all-gathered back to Replicate).
 *
 * ids: device int64 [T].
 * Table: exactly one of E and e_shards is non-NULL.
 *   E: device [V, D] with row stride lde >= D; shard i is its column block
 *     [i*D/P, (i+1)*D/P) (the Shard(1) views of one allocation);
 *   e_shards: host array of P device pointers, shard i a [V, D/P] table with
 *     row stride lde >= D/P in its own allocation (as P ranks would hold it).
 * Y: y_mode TP_Y_CONCAT: [T, D], ldy >= D, shard i's features at columns
 *   [i*D/P, (i+1)*D/P) -- the all-gathered, replicated output;
 *   TP_Y_SHARDS: P blocks [T, D/P] at Y + i*T*ldy, ldy >= D/P -- the Shard(-1)
 *   output before the all-gather.
 * Y[t] = row ids[t] of the table, copied bit for bit.  An id outside [0, V)
 *   gives a zero row and, when bad_flag (device int32) is not NULL, stores 1
 *   there (the library never clears it).
 * dtype: TP_BF16 or TP_F32 (table and output).
 * Errors: TP_ERR_NULL, TP_ERR_SHAPE (negative size, leading dim too small, P
 * out of range), TP_ERR_INDIVISIBLE (D % P != 0), TP_ERR_DTYPE, TP_ERR_MODE,
 * TP_ERR_HIP.
 */
tp_status tp_embedding(const int64_t *ids, int64_t T, const void *E,
                       const void *const *e_shards, int64_t lde, int64_t V, int64_t D,
                       void *Y, int64_t ldy, int32_t y_mode, int32_t P, int32_t dtype,
                       int32_t *bad_flag, void *stream);

/*
 * tp_linear_row_noalloc -- tp_linear_row for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same computation, modes, arguments and errors,
 * without the workspace arguments.
 *
 * The workspace is a fixed array of TP_NOALLOC_SCRATCH_BYTES that the library
 * holds on each GPU it runs on (reserved when the library is loaded on that
 * GPU, kept until the process ends).  The call allocates nothing and calls no
 * allocating routine; the array's device address on the current device is
 * looked up once per device, on its first call there.
 * Limit: the calls that fold fp32 partials in a separate kernel need
 *   tp_row_workspace_bytes(mode, M, N, P) <= TP_NOALLOC_SCRATCH_BYTES, else
 *   TP_ERR_WORKSPACE before anything is queued: TP_ROW_SUM, and TP_ROW_FUSED
 *   / TP_ROW_SCATTER at the shapes no fused kernel takes (see TP_ROW_FUSED;
 *   where the partials would not fit the array, these two modes fold inside
 *   the GEMM at every shape a fused kernel takes, as with
 *   TPLINEAR_ROW_FOLD=gemm).  TP_ROW_PARTIAL and the calls whose fold runs
 *   inside the GEMM use no workspace and have no such limit.  No part of the
 *   array has to start at zero: every partial is written before the fold
 *   reads it.
 * Concurrency: all calls on one GPU share that GPU's array and it keeps the
 *   last call's contents, so calls that may overlap on one GPU (on different
 *   streams without ordering, or from several threads) race on it and must
 *   be ordered by the caller.
 */
#define TP_NOALLOC_SCRATCH_BYTES (32u << 20)
tp_status tp_linear_row_noalloc(const void *X, int64_t ldx, const void *W, int64_t ldw,
                                void *Y, int64_t ldy, int64_t y_slice_stride, int32_t mode,
                                int64_t M, int64_t N, int64_t K, int32_t P,
                                int32_t dtype, void *stream);

/* Bytes of workspace tp_linear_row needs for (mode, M, N, P); 0 for
 * TP_ROW_PARTIAL, and for invalid arguments (including P*M*N*4 > 2^60,
 * which tp_linear_row rejects with TP_ERR_SHAPE). */
size_t tp_row_workspace_bytes(int32_t mode, int64_t M, int64_t N, int32_t P);

/* Queue a fill of `bytes` bytes (a multiple of 4) at `ptr` with zero, with a
 * kernel (no hipMemset node, so it may be captured in a graph). */
tp_status tp_workspace_zero(void *ptr, size_t bytes, void *stream);

/* A static string naming a status code. */
const char *tp_status_str(int32_t status);

/* Library version, major*10000 + minor*100 + patch. */
int32_t tp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TPLINEAR_H */
