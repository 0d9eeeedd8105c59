"""CPU tests of the host-side argument checks of the entry points for the
steps next to the Linear (bias, gated unit, token slices, embedding).  Every
call is rejected, or is an empty problem, before anything is queued: fake
non-null addresses are never dereferenced and no kernel runs."""
import ctypes

import tensor_linear_amd as tl

FX, FW, FY, FWS, FB, FI = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000


def _arr(ptrs):
    return (ctypes.c_void_p * len(ptrs))(*ptrs)


def colx(**kw):
    a = dict(X=FX, xs=None, ldx=8, W=FW, ldw=8, b=None, Y=FY, ldy=12, y_mode=tl.TP_Y_CONCAT,
             act=tl.TP_ACT_NONE, M=4, N=12, K=8, P=4, dtype=tl.TP_BF16)
    a.update(kw)
    return tl.lib.tp_linear_column_ex(a["X"], a["xs"], a["ldx"], a["W"], a["ldw"], a["b"], a["Y"],
                                      a["ldy"], a["y_mode"], a["act"], a["M"], a["N"], a["K"],
                                      a["P"], a["dtype"], None)


def rowx(**kw):
    a = dict(X=FX, ldx=8, W=FW, ldw=8, b=None, Y=FY, ys=None, ldy=12, ss=0,
             mode=tl.TP_ROW_SUM, ws=FWS, wsb=1 << 20, M=4, N=12, K=8, P=4, dtype=tl.TP_BF16)
    a.update(kw)
    return tl.lib.tp_linear_row_ex(a["X"], a["ldx"], a["W"], a["ldw"], a["b"], a["Y"], a["ys"],
                                   a["ldy"], a["ss"], a["mode"], a["ws"], a["wsb"], a["M"],
                                   a["N"], a["K"], a["P"], a["dtype"], None)


def redx(**kw):
    a = dict(p=FWS, ss=48, ldp=12, b=None, Y=FY, ys=None, ldy=12, yss=0, scatter=0, M=4, N=12,
             P=4, dtype=tl.TP_BF16)
    a.update(kw)
    return tl.lib.tp_shard_reduce_ex(a["p"], a["ss"], a["ldp"], a["b"], a["Y"], a["ys"], a["ldy"],
                                     a["yss"], a["scatter"], a["M"], a["N"], a["P"], a["dtype"],
                                     None)


def emb(**kw):
    a = dict(ids=FI, T=5, E=FW, es=None, lde=16, V=10, D=16, Y=FY, ldy=16,
             y_mode=tl.TP_Y_CONCAT, P=4, dtype=tl.TP_BF16, bad=None)
    a.update(kw)
    return tl.lib.tp_embedding(a["ids"], a["T"], a["E"], a["es"], a["lde"], a["V"], a["D"], a["Y"],
                               a["ldy"], a["y_mode"], a["P"], a["dtype"], a["bad"], None)


def test_column_ex_errors():
    slices = _arr([FX, FX + 256, FX + 512, FX + 768])
    assert colx(X=None) == tl.TP_ERR_NULL                      # neither input
    assert colx(xs=slices) == tl.TP_ERR_NULL                   # both inputs
    assert colx(X=None, xs=_arr([FX, None, FX, FX])) == tl.TP_ERR_NULL
    assert colx(X=None, xs=slices, M=6) == tl.TP_ERR_INDIVISIBLE   # slices need M % P == 0
    assert colx(act=7) == tl.TP_ERR_MODE
    assert colx(act=tl.TP_ACT_SWIGLU, N=4, ldy=4) == tl.TP_ERR_INDIVISIBLE  # N/P = 1 is odd
    # gated unit: the output is [M, N/2]; concat needs ldy >= N/2, shards ldy >= N/(2P)
    assert colx(act=tl.TP_ACT_SWIGLU, N=16, ldy=7) == tl.TP_ERR_SHAPE
    assert colx(act=tl.TP_ACT_SWIGLU, N=16, ldy=1, y_mode=tl.TP_Y_SHARDS) == tl.TP_ERR_SHAPE
    assert colx(ldy=11) == tl.TP_ERR_SHAPE
    assert colx(N=10) == tl.TP_ERR_INDIVISIBLE
    assert colx(dtype=2) == tl.TP_ERR_DTYPE
    assert colx(y_mode=3) == tl.TP_ERR_MODE
    assert colx(M=0) == tl.TP_OK
    assert colx(M=0, X=None, xs=None, W=None, Y=None, b=FB) == tl.TP_OK


def test_row_ex_errors():
    ys = _arr([FY, FY + 256, FY + 512, FY + 768])
    assert rowx(b=FB, mode=tl.TP_ROW_PARTIAL) == tl.TP_ERR_MODE   # bias after the fold only
    assert rowx(ys=ys, mode=tl.TP_ROW_SUM) == tl.TP_ERR_MODE      # slices only for SCATTER
    assert rowx(ys=_arr([FY, FY, None, FY]), mode=tl.TP_ROW_SCATTER) == tl.TP_ERR_NULL
    assert rowx(Y=None) == tl.TP_ERR_NULL
    assert rowx(ys=ys, mode=tl.TP_ROW_SCATTER, M=6) == tl.TP_ERR_INDIVISIBLE
    assert rowx(ws=None, b=FB) == tl.TP_ERR_WORKSPACE
    assert rowx(M=0, b=FB) == tl.TP_OK


def test_reduce_ex_errors():
    ys = _arr([FY, FY + 256, FY + 512, FY + 768])
    assert redx(ys=ys, scatter=0) == tl.TP_ERR_MODE
    assert redx(ys=_arr([FY, None, FY, FY]), scatter=1) == tl.TP_ERR_NULL
    assert redx(Y=None) == tl.TP_ERR_NULL
    assert redx(ys=ys, scatter=1, M=6) == tl.TP_ERR_INDIVISIBLE
    assert redx(p=None, b=FB) == tl.TP_ERR_NULL
    assert redx(M=0, b=FB) == tl.TP_OK


def test_embedding_errors():
    shards = _arr([FW, FW + 1024, FW + 2048, FW + 4096])
    assert emb(ids=None) == tl.TP_ERR_NULL
    assert emb(Y=None) == tl.TP_ERR_NULL
    assert emb(E=None) == tl.TP_ERR_NULL                       # neither table
    assert emb(es=shards) == tl.TP_ERR_NULL                    # both tables
    assert emb(E=None, es=_arr([FW, None, FW, FW]), lde=4) == tl.TP_ERR_NULL
    assert emb(P=0) == tl.TP_ERR_SHAPE
    assert emb(P=65) == tl.TP_ERR_SHAPE
    assert emb(T=-1) == tl.TP_ERR_SHAPE
    assert emb(D=18, lde=18, ldy=18) == tl.TP_ERR_INDIVISIBLE
    assert emb(lde=15) == tl.TP_ERR_SHAPE                      # one table: lde >= D
    assert emb(E=None, es=shards, lde=3) == tl.TP_ERR_SHAPE    # shard tables: lde >= D/P
    assert emb(ldy=15) == tl.TP_ERR_SHAPE
    assert emb(ldy=3, y_mode=tl.TP_Y_SHARDS) == tl.TP_ERR_SHAPE
    assert emb(dtype=5) == tl.TP_ERR_DTYPE
    assert emb(y_mode=2) == tl.TP_ERR_MODE
    assert emb(T=0, ids=None, Y=None) == tl.TP_OK
