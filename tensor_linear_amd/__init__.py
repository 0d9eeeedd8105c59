"""Python binding of libtplinear (include/tplinear.h), the tensor-parallel
Linear Y = X W on one MI355X with all P shards resident.

Argument marshalling only: every function passes device pointers, sizes and
leading dimensions taken from torch tensors to the C entry point of the same
name and turns a non-zero status into an exception (ValueError for argument
errors, RuntimeError for TP_ERR_HIP).  All arithmetic runs in the HIP
kernels of the library; there is no fallback.  The first call raises
ImportError if libtplinear.so has not been built
(python -m tensor_linear_amd.build).

Tensors: 2-D row-major views with unit column stride; the row stride is the
leading dimension.  X is [M, K], W is stored [N, K] ([out, in]), Y is [M, N].
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtplinear.so")

_lib = None


def _get_lib():
    """Load libtplinear.so once; fail loudly if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m tensor_linear_amd.build` "
            "(hipcc, gfx950)")
    _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def __getattr__(name):
    if name == "lib":
        return _get_lib()
    raise AttributeError(name)


# ---- constants (mirror include/tplinear.h) --------------------------------
TP_OK, TP_ERR_NULL, TP_ERR_SHAPE, TP_ERR_INDIVISIBLE, TP_ERR_PLACEMENT, \
    TP_ERR_DTYPE, TP_ERR_MODE, TP_ERR_WORKSPACE, TP_ERR_HIP = range(9)
TP_F32, TP_BF16 = 0, 1
TP_REPLICATE, TP_SHARD, TP_PARTIAL = 0, 1, 2
TP_Y_CONCAT, TP_Y_SHARDS = 0, 1
TP_ROW_PARTIAL, TP_ROW_SUM, TP_ROW_FUSED, TP_ROW_SCATTER = 0, 1, 2, 3
TP_ACT_NONE, TP_ACT_SWIGLU = 0, 1
TP_MAX_SHARDS = 64

EXPORTS = ("tp_shard_layout", "tp_linear_column", "tp_linear_row", "tp_shard_reduce",
           "tp_linear_column_ex", "tp_linear_row_ex", "tp_shard_reduce_ex", "tp_embedding",
           "tp_row_workspace_bytes", "tp_workspace_zero", "tp_status_str", "tp_version",
           "tp_linear_row_noalloc")
TP_NOALLOC_SCRATCH_BYTES = 32 << 20


class tp_placement(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("dim", ctypes.c_int32)]


class tp_view(ctypes.Structure):
    _fields_ = [("elem_offset", ctypes.c_int64), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("ld", ctypes.c_int64),
                ("row0", ctypes.c_int64), ("col0", ctypes.c_int64)]


_i32, _i64, _ptr, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t


def _declare(lib):
    lib.tp_shard_layout.argtypes = [_i64, _i64, _i64, tp_placement, _i32, ctypes.POINTER(tp_view)]
    lib.tp_shard_layout.restype = _i32
    lib.tp_linear_column.argtypes = [_ptr, _i64, _ptr, _i64, _ptr, _i64, _i32, _i64, _i64, _i64,
                                     _i32, _i32, _ptr]
    lib.tp_linear_column.restype = _i32
    lib.tp_linear_row.argtypes = [_ptr, _i64, _ptr, _i64, _ptr, _i64, _i64, _i32, _ptr, _sz,
                                  _i64, _i64, _i64, _i32, _i32, _ptr]
    lib.tp_linear_row.restype = _i32
    lib.tp_shard_reduce.argtypes = [_ptr, _i64, _i64, _ptr, _i64, _i64, _i32, _i64, _i64, _i32,
                                    _i32, _ptr]
    lib.tp_shard_reduce.restype = _i32
    lib.tp_linear_column_ex.argtypes = [_ptr, _ptr, _i64, _ptr, _i64, _ptr, _ptr, _i64, _i32,
                                        _i32, _i64, _i64, _i64, _i32, _i32, _ptr]
    lib.tp_linear_column_ex.restype = _i32
    lib.tp_linear_row_ex.argtypes = [_ptr, _i64, _ptr, _i64, _ptr, _ptr, _ptr, _i64, _i64, _i32,
                                     _ptr, _sz, _i64, _i64, _i64, _i32, _i32, _ptr]
    lib.tp_linear_row_ex.restype = _i32
    lib.tp_shard_reduce_ex.argtypes = [_ptr, _i64, _i64, _ptr, _ptr, _ptr, _i64, _i64, _i32,
                                       _i64, _i64, _i32, _i32, _ptr]
    lib.tp_shard_reduce_ex.restype = _i32
    lib.tp_embedding.argtypes = [_ptr, _i64, _ptr, _ptr, _i64, _i64, _i64, _ptr, _i64, _i32,
                                 _i32, _i32, _ptr, _ptr]
    lib.tp_embedding.restype = _i32
    lib.tp_linear_row_noalloc.argtypes = [_ptr, _i64, _ptr, _i64, _ptr, _i64, _i64, _i32,
                                          _i64, _i64, _i64, _i32, _i32, _ptr]
    lib.tp_linear_row_noalloc.restype = _i32
    lib.tp_row_workspace_bytes.argtypes = [_i32, _i64, _i64, _i32]
    lib.tp_row_workspace_bytes.restype = _sz
    lib.tp_workspace_zero.argtypes = [_ptr, _sz, _ptr]
    lib.tp_workspace_zero.restype = _i32
    lib.tp_status_str.argtypes = [_i32]
    lib.tp_status_str.restype = ctypes.c_char_p
    lib.tp_version.argtypes = []
    lib.tp_version.restype = _i32
    return lib


class TPError(ValueError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(_get_lib().tp_status_str(status).decode())


class TPHipError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(_get_lib().tp_status_str(status).decode())


def check(status: int) -> None:
    if status == TP_OK:
        return
    if status == TP_ERR_HIP:
        raise TPHipError(status)
    raise TPError(status)


def tp_status_str(status: int) -> str:
    return _get_lib().tp_status_str(status).decode()


def tp_version() -> int:
    return int(_get_lib().tp_version())


# ---- marshalling helpers --------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return TP_BF16
    if t.dtype == torch.float32:
        return TP_F32
    raise TypeError(f"unsupported dtype {t.dtype}: bfloat16 or float32")


def _mat(t, name):
    """(data pointer, rows, cols, leading dim) of a 2-D unit-column-stride view."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    # A one-row view keeps the row stride of the buffer it was cut from when
    # that stride is a valid leading dim (it places the blocks of a [P, 1, N]
    # output); otherwise its leading dim is its width.
    ld = t.stride(0) if t.shape[0] > 1 or t.stride(0) >= t.shape[1] else t.shape[1]
    return t.data_ptr(), t.shape[0], t.shape[1], max(ld, t.shape[1], 1)


def _same_gpu(*items):
    """Every tensor given (lists of tensors included, None skipped) must live
    on one GPU: the kernels dereference the data pointers on that device, so
    a host tensor or a second device is rejected here, before any launch."""
    dev = None
    for it in items:
        for t in (it if isinstance(it, (list, tuple)) else (it,)):
            if t is None:
                continue
            if not t.is_cuda:
                raise ValueError("every tensor must be a GPU tensor (got one on "
                                 f"{t.device})")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"tensors on {dev} and {t.device}: all must share one GPU")


def _ptr_array(ts, name):
    """Host array of the data pointers of a list of tensors (or None)."""
    if ts is None:
        return None
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def _check_p(P):
    if not 1 <= P <= TP_MAX_SHARDS:
        check(TP_ERR_SHAPE)


def _expect_shape(t, shape, name):
    """The library writes exactly `shape`; a smaller or differently shaped
    output would be written out of bounds, so it is refused here."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _expect_room(t, elems, name):
    """t's storage must hold `elems` elements from t's first element."""
    have = t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()
    if elems > have:
        raise ValueError(f"{name}: the output needs {elems} elements from its first one, "
                         f"its storage holds {have}")


def _scatter_out(Y, M, N, P, scatter, y_slice_stride, name="Y"):
    """Row stride of a fold / reduce-scatter output Y: [M, N], or for a
    reduce-scatter with a nonzero slice stride the [M/P, N] view of slice 0
    inside a buffer that holds all P slices."""
    if scatter and M % P:
        check(TP_ERR_INDIVISIBLE)
    yp, _, _, ldy = _mat(Y, name)
    if scatter and y_slice_stride:
        s = M // P
        _expect_shape(Y, (s, N), name)
        if s and N:
            _expect_room(Y, (P - 1) * y_slice_stride + (s - 1) * ldy + N, name)
    else:
        _expect_shape(Y, (M, N), name)
    return yp, ldy


def _block_out(Y, P, rows, cols, name="Y"):
    """Pointer and row stride of a [P, rows, cols] output whose blocks are
    rows*ldy elements apart."""
    _expect_shape(Y, (P, rows, cols), name)
    _, _, _, ldy = _mat(Y[0], f"{name}[0]")
    if P > 1 and Y.stride(0) != rows * ldy:
        raise ValueError(f"{name} blocks must be rows*ldy elements apart")
    return Y.data_ptr(), ldy


def _bias_ptr(bias, dt):
    if bias is None:
        return None
    if bias.dim() != 1 or (bias.numel() > 1 and bias.stride(0) != 1):
        raise ValueError("bias must be a contiguous 1-D tensor")
    if _dtype_code(bias) != dt:
        raise TypeError("bias must have the output dtype")
    return bias.data_ptr()


def _stream(t, stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    if t.is_cuda:
        return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    return ctypes.c_void_p(0)


# ---- entry points ---------------------------------------------------------

def tp_shard_layout(rows: int, cols: int, ld: int, kind: int, dim: int, P: int) -> list:
    """Views of the P shards as (elem_offset, rows, cols, ld, row0, col0)."""
    if not 1 <= P <= TP_MAX_SHARDS:
        check(TP_ERR_SHAPE)
    views = (tp_view * P)()
    check(_get_lib().tp_shard_layout(rows, cols, ld, tp_placement(kind, dim), P, views))
    return [(v.elem_offset, v.rows, v.cols, v.ld, v.row0, v.col0) for v in views]


def tp_linear_column(X, W, Y, P: int, y_mode: int = TP_Y_CONCAT, stream=None) -> None:
    """Column-parallel Linear.  X [M, K], W [N, K]; Y [M, N] for TP_Y_CONCAT
    or [P, M, N/P] (block stride M*ldy) for TP_Y_SHARDS."""
    xp, M, K, ldx = _mat(X, "X")
    wp, N, Kw, ldw = _mat(W, "W")
    if Kw != K:
        raise ValueError(f"X has K={K} but W has K={Kw}")
    dt = _dtype_code(X)
    if _dtype_code(W) != dt or _dtype_code(Y) != dt:
        raise TypeError("X, W and Y must share one dtype")
    _check_p(P)
    if N % P:
        check(TP_ERR_INDIVISIBLE)
    if y_mode == TP_Y_SHARDS:
        yp, ldy = _block_out(Y, P, M, N // P)
    else:
        yp, _, _, ldy = _mat(Y, "Y")
        _expect_shape(Y, (M, N), "Y")
    _same_gpu(X, W, Y)
    check(_get_lib().tp_linear_column(xp, ldx, wp, ldw, yp, ldy, y_mode, M, N, K, P, dt,
                               _stream(X, stream)))


def tp_row_workspace_bytes(mode: int, M: int, N: int, P: int) -> int:
    return int(_get_lib().tp_row_workspace_bytes(mode, M, N, P))


def tp_workspace_zero(buf, stream=None) -> None:
    _same_gpu(buf)
    check(_get_lib().tp_workspace_zero(buf.data_ptr(), buf.numel() * buf.element_size(),
                                _stream(buf, stream)))


def tp_linear_row(X, W, Y, P: int, mode: int = TP_ROW_SUM, workspace=None,
                  y_slice_stride: int = 0, stream=None) -> None:
    """Row-parallel Linear.  X [M, K], W [N, K].  Y: TP_ROW_PARTIAL ->
    float32 [P, M, N]; TP_ROW_SUM / TP_ROW_FUSED -> [M, N]; TP_ROW_SCATTER ->
    [M, N] whose row blocks are the slices (y_slice_stride = 0), or a buffer
    with slice j at element offset j*y_slice_stride and rows [:M/P] of its
    2-D view Y."""
    xp, M, K, ldx = _mat(X, "X")
    wp, N, Kw, ldw = _mat(W, "W")
    if Kw != K:
        raise ValueError(f"X has K={K} but W has K={Kw}")
    dt = _dtype_code(X)
    if _dtype_code(W) != dt:
        raise TypeError("X and W must share one dtype")
    _check_p(P)
    if mode == TP_ROW_PARTIAL:
        import torch
        if Y.dtype != torch.float32:
            raise ValueError("Y must be float32 [P, M, N] for TP_ROW_PARTIAL")
        yp, ldy = _block_out(Y, P, M, N)
    else:
        if _dtype_code(Y) != dt:
            raise TypeError("Y must have the dtype of X")
        yp, ldy = _scatter_out(Y, M, N, P, mode == TP_ROW_SCATTER, y_slice_stride)
    if workspace is not None:
        wsp, wsb = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    else:
        wsp, wsb = None, 0
    _same_gpu(X, W, Y, workspace)
    check(_get_lib().tp_linear_row(xp, ldx, wp, ldw, yp, ldy, y_slice_stride, mode, wsp, wsb,
                            M, N, K, P, dt, _stream(X, stream)))


def tp_linear_row_noalloc(X, W, Y, P: int, mode: int = TP_ROW_SUM, y_slice_stride: int = 0,
                          stream=None) -> None:
    """tp_linear_row without a workspace argument: the library's fixed
    per-GPU array of TP_NOALLOC_SCRATCH_BYTES serves as the workspace, so
    nothing is allocated (calls that may overlap on one GPU race on it).
    Shapes whose workspace would exceed it raise TPError(TP_ERR_WORKSPACE)."""
    xp, M, K, ldx = _mat(X, "X")
    wp, N, Kw, ldw = _mat(W, "W")
    if Kw != K:
        raise ValueError(f"X has K={K} but W has K={Kw}")
    dt = _dtype_code(X)
    if _dtype_code(W) != dt:
        raise TypeError("X and W must share one dtype")
    _check_p(P)
    if mode == TP_ROW_PARTIAL:
        import torch
        if Y.dtype != torch.float32:
            raise ValueError("Y must be float32 [P, M, N] for TP_ROW_PARTIAL")
        yp, ldy = _block_out(Y, P, M, N)
    else:
        if _dtype_code(Y) != dt:
            raise TypeError("Y must have the dtype of X")
        yp, ldy = _scatter_out(Y, M, N, P, mode == TP_ROW_SCATTER, y_slice_stride)
    _same_gpu(X, W, Y)
    check(_get_lib().tp_linear_row_noalloc(xp, ldx, wp, ldw, yp, ldy, y_slice_stride, mode,
                                           M, N, K, P, dt, _stream(X, stream)))


def tp_shard_reduce(partials, Y, P: int, scatter: int = 0, y_slice_stride: int = 0,
                    stream=None) -> None:
    """Fold float32 partials [P, M, N] (or any [P, M, ldp] view) into Y [M, N]
    (scatter=0) or into P token slices (scatter=1)."""
    import torch
    _check_p(P)
    if partials.dtype != torch.float32 or partials.dim() != 3 or partials.shape[0] != P:
        raise ValueError("partials must be float32 [P, M, N]")
    _, M, N, ldp = _mat(partials[0], "partials[0]")
    ss = partials.stride(0) if P > 1 else M * ldp
    yp, ldy = _scatter_out(Y, M, N, P, scatter, y_slice_stride)
    _same_gpu(partials, Y)
    check(_get_lib().tp_shard_reduce(partials.data_ptr(), ss, ldp, yp, ldy, y_slice_stride, scatter,
                              M, N, P, _dtype_code(Y), _stream(partials, stream)))


def tp_linear_column_ex(X, W, Y, P: int, y_mode: int = TP_Y_CONCAT, bias=None,
                        act: int = TP_ACT_NONE, x_slices=None, stream=None) -> None:
    """Column-parallel Linear with a bias, the gated unit and token-slice
    input.  Exactly one of X ([M, K]) and x_slices (P tensors [M/P, K] with
    one row stride) is given.  W [N, K]; bias [N] or None.  Output columns per
    shard On = N/P, or N/(2P) with TP_ACT_SWIGLU; Y [M, P*On] for TP_Y_CONCAT
    or [P, M, On] for TP_Y_SHARDS."""
    _check_p(P)
    if (X is None) == (x_slices is None):
        raise ValueError("give exactly one of X and x_slices")
    if X is not None:
        xp, M, K, ldx = _mat(X, "X")
        ref = X
        sl = None
    else:
        if len(x_slices) != P:
            raise ValueError(f"x_slices must hold P={P} tensors")
        _, ms, K, ldx = _mat(x_slices[0], "x_slices[0]")
        for j, t in enumerate(x_slices):
            _, mj, kj, lj = _mat(t, f"x_slices[{j}]")
            if (mj, kj) != (ms, K) or (mj > 1 and lj != ldx):
                raise ValueError("token slices must share shape and row stride")
            if _dtype_code(t) != _dtype_code(x_slices[0]):
                raise TypeError("token slices must share one dtype")
        M, xp, ref = ms * P, None, x_slices[0]
        sl = _ptr_array(x_slices, "x_slices")
    wp, N, Kw, ldw = _mat(W, "W")
    if Kw != K:
        raise ValueError(f"X has K={K} but W has K={Kw}")
    dt = _dtype_code(ref)
    if _dtype_code(W) != dt or _dtype_code(Y) != dt:
        raise TypeError("X, W and Y must share one dtype")
    if N % P or (act == TP_ACT_SWIGLU and (N // P) % 2):
        check(TP_ERR_INDIVISIBLE)
    On = N // P // 2 if act == TP_ACT_SWIGLU else N // P
    if bias is not None:
        _expect_shape(bias, (N,), "bias")
    if y_mode == TP_Y_SHARDS:
        yp, ldy = _block_out(Y, P, M, On)
    else:
        yp, _, _, ldy = _mat(Y, "Y")
        _expect_shape(Y, (M, P * On), "Y")
    _same_gpu(X, W, Y, bias, x_slices)
    check(_get_lib().tp_linear_column_ex(xp, sl, ldx, wp, ldw, _bias_ptr(bias, dt), yp, ldy,
                                         y_mode, act, M, N, K, P, dt, _stream(ref, stream)))


def tp_linear_row_ex(X, W, Y, P: int, mode: int = TP_ROW_SUM, workspace=None, bias=None,
                     y_slices=None, y_slice_stride: int = 0, stream=None) -> None:
    """Row-parallel Linear with the row bias (added once after the fold) and,
    for TP_ROW_SCATTER, token slices in separate tensors (y_slices: P tensors
    [M/P, N] with one row stride; Y is then None).  Otherwise as
    tp_linear_row."""
    _check_p(P)
    xp, M, K, ldx = _mat(X, "X")
    wp, N, Kw, ldw = _mat(W, "W")
    if Kw != K:
        raise ValueError(f"X has K={K} but W has K={Kw}")
    dt = _dtype_code(X)
    if _dtype_code(W) != dt:
        raise TypeError("X and W must share one dtype")
    if bias is not None:
        _expect_shape(bias, (N,), "bias")
    ys = None
    if y_slices is not None:
        if Y is not None:
            raise ValueError("give Y or y_slices, not both")
        if len(y_slices) != P:
            raise ValueError(f"y_slices must hold P={P} tensors")
        if M % P:
            check(TP_ERR_INDIVISIBLE)
        _, _, _, ldy = _mat(y_slices[0], "y_slices[0]")
        for j, t in enumerate(y_slices):
            _, mj, nj, lj = _mat(t, f"y_slices[{j}]")
            if (mj, nj) != (M // P, N) or (mj > 1 and lj != ldy) or _dtype_code(t) != dt:
                raise ValueError("y_slices must be [M/P, N] of the input dtype, one row stride")
        yp, ys = None, _ptr_array(y_slices, "y_slices")
    elif mode == TP_ROW_PARTIAL:
        import torch
        if Y.dtype != torch.float32:
            raise ValueError("Y must be float32 [P, M, N] for TP_ROW_PARTIAL")
        yp, ldy = _block_out(Y, P, M, N)
    else:
        if _dtype_code(Y) != dt:
            raise TypeError("Y must have the dtype of X")
        yp, ldy = _scatter_out(Y, M, N, P, mode == TP_ROW_SCATTER, y_slice_stride)
    if workspace is not None:
        wsp, wsb = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    else:
        wsp, wsb = None, 0
    _same_gpu(X, W, Y, workspace, bias, y_slices)
    check(_get_lib().tp_linear_row_ex(xp, ldx, wp, ldw, _bias_ptr(bias, dt), yp, ys, ldy,
                                      y_slice_stride, mode, wsp, wsb, M, N, K, P, dt,
                                      _stream(X, stream)))


def tp_shard_reduce_ex(partials, Y, P: int, scatter: int = 0, bias=None, y_slices=None,
                       y_slice_stride: int = 0, stream=None) -> None:
    """tp_shard_reduce with the row bias and, for scatter=1, token slices in
    separate tensors (y_slices: P tensors [M/P, N], one row stride; Y None)."""
    import torch
    _check_p(P)
    if partials.dtype != torch.float32 or partials.dim() != 3 or partials.shape[0] != P:
        raise ValueError("partials must be float32 [P, M, N]")
    _, M, N, ldp = _mat(partials[0], "partials[0]")
    ss = partials.stride(0) if P > 1 else M * ldp
    if bias is not None:
        _expect_shape(bias, (N,), "bias")
    if y_slices is not None:
        if Y is not None:
            raise ValueError("give Y or y_slices, not both")
        if len(y_slices) != P:
            raise ValueError(f"y_slices must hold P={P} tensors")
        if M % P:
            check(TP_ERR_INDIVISIBLE)
        _, _, _, ldy = _mat(y_slices[0], "y_slices[0]")
        odt = _dtype_code(y_slices[0])
        for j, t in enumerate(y_slices):
            _, mj, nj, lj = _mat(t, f"y_slices[{j}]")
            if (mj, nj) != (M // P, N) or (mj > 1 and lj != ldy) or _dtype_code(t) != odt:
                raise ValueError("y_slices must be [M/P, N] of one dtype and row stride")
        yp, ys = None, _ptr_array(y_slices, "y_slices")
    else:
        yp, ldy = _scatter_out(Y, M, N, P, scatter, y_slice_stride)
        odt, ys = _dtype_code(Y), None
    _same_gpu(partials, Y, bias, y_slices)
    check(_get_lib().tp_shard_reduce_ex(partials.data_ptr(), ss, ldp, _bias_ptr(bias, odt), yp,
                                        ys, ldy, y_slice_stride, scatter, M, N, P, odt,
                                        _stream(partials, stream)))


def tp_embedding(ids, Y, P: int, E=None, e_shards=None, y_mode: int = TP_Y_CONCAT, bad=None,
                 stream=None) -> None:
    """Feature-sharded embedding lookup (EmbeddingWithReplicateOutput).
    ids: int64 [T].  Exactly one of E ([V, D]) and e_shards (P tensors
    [V, D/P], one row stride).  Y: [T, D] (TP_Y_CONCAT) or [P, T, D/P]
    (TP_Y_SHARDS).  bad: None or an int32 tensor set to 1 when an id is
    outside [0, V) (its output row is zero)."""
    import torch
    _check_p(P)
    if ids.dtype != torch.int64 or ids.dim() != 1 or (ids.numel() > 1 and ids.stride(0) != 1):
        raise ValueError("ids must be a contiguous int64 [T] tensor")
    T = ids.shape[0]
    if (E is None) == (e_shards is None):
        raise ValueError("give exactly one of E and e_shards")
    if E is not None:
        ep, V, D, lde = _mat(E, "E")
        dt, es = _dtype_code(E), None
    else:
        if len(e_shards) != P:
            raise ValueError(f"e_shards must hold P={P} tensors")
        _, V, Ds, lde = _mat(e_shards[0], "e_shards[0]")
        dt = _dtype_code(e_shards[0])
        for i, t in enumerate(e_shards):
            _, vi, di, li = _mat(t, f"e_shards[{i}]")
            if (vi, di) != (V, Ds) or (vi > 1 and li != lde) or _dtype_code(t) != dt:
                raise ValueError("e_shards must share shape, dtype and row stride")
        ep, D, es = None, Ds * P, _ptr_array(e_shards, "e_shards")
    if _dtype_code(Y) != dt:
        raise TypeError("Y must have the table's dtype")
    if D % P:
        check(TP_ERR_INDIVISIBLE)
    if y_mode == TP_Y_SHARDS:
        yp, ldy = _block_out(Y, P, T, D // P)
    else:
        yp, _, _, ldy = _mat(Y, "Y")
        _expect_shape(Y, (T, D), "Y")
    if bad is not None and (bad.dtype != torch.int32 or bad.numel() < 1):
        raise ValueError("bad must be an int32 tensor")
    _same_gpu(ids, Y, E, e_shards, bad)
    check(_get_lib().tp_embedding(ids.data_ptr(), T, ep, es, lde, V, D, yp, ldy, y_mode, P, dt,
                                  None if bad is None else bad.data_ptr(), _stream(ids, stream)))
