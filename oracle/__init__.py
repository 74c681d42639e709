"""fp64 CPU oracle for row-wise softmax cross-entropy -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never imports, links or
calls it, and the two share no code.

The arithmetic lives in ``ce_oracle.c`` (plain C, fp64); this module only moves
numpy arrays in and out of it.  What each function computes, and the passages
of the pages it follows, is documented in ``ce_oracle.c``:

* loss of a row = log-sum-exp of the row minus the target logit (POPCORNBENCH
  "Kimi-K2.6 l1_p95" trace, problem statement; Triton issue "Cross Entropy Loss
  performance issue", loss_kernel's output line);
* mean / sum over rows (same trace: mean reduction of ``F.cross_entropy``);
* gradient (softmax - onehot) * c written in the storage type ("9 Triton
  kernels in 9 weeks", week 7), optionally times a per-row upstream gradient;
* row softmax and log-softmax (same page, week 1; the trace's log_softmax);
* linear + cross-entropy: logits H W^T of bf16 H, W, then the loss, and the
  gradients of H and W (same page, week 8).

Storage types are passed as raw bits: float32 arrays for fp32, uint16 arrays of
the bit patterns for fp16 and bf16.
"""
import ctypes
import os

import numpy as np

F32, F16, BF16 = 0, 1, 2
NONE, MEAN, SUM = 0, 1, 2
_DTYPE_CODE = {"f32": F32, "fp32": F32, "float32": F32,
               "f16": F16, "fp16": F16, "float16": F16,
               "bf16": BF16, "bfloat16": BF16}
_RED_CODE = {"none": NONE, "mean": MEAN, "sum": SUM}

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIBRARY: another build of ce_oracle.c (the host-sanitizer test's)
_LIB_OVERRIDE = os.environ.get("ORACLE_LIBRARY")
_LIB_PATH = _LIB_OVERRIDE or os.path.join(_HERE, "libce_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    src = os.path.join(_HERE, "ce_oracle.c")
    if not _LIB_OVERRIDE and (not os.path.exists(_LIB_PATH)
                              or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src)):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.oracle_widen_f16.argtypes = [ctypes.c_uint16]
    lib.oracle_widen_f16.restype = ctypes.c_double
    lib.oracle_widen_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_widen_bf16.restype = ctypes.c_double
    lib.oracle_round_f16.argtypes = [ctypes.c_double]
    lib.oracle_round_f16.restype = ctypes.c_uint16
    lib.oracle_round_bf16.argtypes = [ctypes.c_double]
    lib.oracle_round_bf16.restype = ctypes.c_uint16
    lib.oracle_round_f32.argtypes = [ctypes.c_double]
    lib.oracle_round_f32.restype = ctypes.c_float
    lib.oracle_ce_loss_rows.argtypes = [vp, i32, _i64p, i64, i64, i64, i64, _dp, _dp]
    lib.oracle_ce_loss_rows.restype = i32
    lib.oracle_ce_reduce.argtypes = [_dp, i64, i32]
    lib.oracle_ce_reduce.restype = ctypes.c_double
    lib.oracle_ce_fwd.argtypes = [vp, i32, _i64p, i64, i64, i32, _dp, _dp]
    lib.oracle_ce_fwd.restype = i32
    lib.oracle_ce_grad_rows.argtypes = [vp, i32, _i64p, i64, i64, i64, i64,
                                        ctypes.c_double, _dp, i32, vp, _dp]
    lib.oracle_ce_grad_rows.restype = i32
    lib.oracle_softmax_rows.argtypes = [vp, i32, i64, i64, i64, i64, i32, i32, vp, _dp, _dp]
    lib.oracle_softmax_rows.restype = i32
    lib.oracle_at_elements.argtypes = [vp, i32, _i64p, i64, i64, _dp, i64, _i64p, _i64p, i32,
                                       ctypes.c_double, _dp, i32, vp, _dp]
    lib.oracle_at_elements.restype = i32
    u16p = ctypes.POINTER(ctypes.c_uint16)
    lib.oracle_linear_ce.argtypes = [u16p, u16p, _i64p, i64, i64, i64, i32, _dp, _dp, _dp, _dp, _dp]
    lib.oracle_linear_ce.restype = i32
    lib.oracle_set_num_threads.argtypes = [i32]
    lib.oracle_set_num_threads.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i32
    _lib = lib
    return lib


def dtype_code(dtype):
    if isinstance(dtype, int):
        return dtype
    return _DTYPE_CODE[str(dtype).replace("torch.", "")]


def _prep(x, dtype):
    code = dtype_code(dtype)
    x = np.ascontiguousarray(x)
    if code == F32:
        if x.dtype != np.float32:
            raise TypeError("fp32 logits must be a float32 array")
    elif x.dtype != np.uint16:
        raise TypeError("fp16/bf16 logits must be passed as uint16 bit patterns")
    if x.ndim != 2:
        raise ValueError("logits must be [M, V]")
    return x, code


def _targets(t, M):
    t = np.ascontiguousarray(t, dtype=np.int64)
    if t.shape != (M,):
        raise ValueError("targets must be [M] int64")
    return t


def loss_rows(x, targets, dtype="f32", row0=0, nrows=None, with_lse=False):
    """Per-row fp64 losses (and log-sum-exps) of rows [row0, row0 + nrows)."""
    lib = _load()
    x, code = _prep(x, dtype)
    M, V = x.shape
    t = _targets(targets, M)
    if nrows is None:
        nrows = M - row0
    loss = np.empty(nrows, dtype=np.float64)
    lse = np.empty(nrows, dtype=np.float64)
    rc = lib.oracle_ce_loss_rows(x.ctypes.data, code, t.ctypes.data_as(_i64p), M, V,
                                 row0, nrows, loss.ctypes.data_as(_dp),
                                 lse.ctypes.data_as(_dp))
    if rc:
        raise ValueError("oracle_ce_loss_rows: bad arguments")
    return (loss, lse) if with_lse else loss


def reduce(losses, reduction):
    """Compensated mean or sum of fp64 row losses."""
    lib = _load()
    losses = np.ascontiguousarray(losses, dtype=np.float64)
    return float(lib.oracle_ce_reduce(losses.ctypes.data_as(_dp), losses.size,
                                      _RED_CODE[reduction]))


def fwd(x, targets, dtype="f32", reduction="mean"):
    """Whole forward: fp64 [M] losses for 'none', else a Python float."""
    lib = _load()
    x, code = _prep(x, dtype)
    M, V = x.shape
    t = _targets(targets, M)
    red = _RED_CODE[reduction]
    out = np.empty(max(M, 1) if red == NONE else 1, dtype=np.float64)
    scratch = np.empty(max(M, 1), dtype=np.float64)
    rc = lib.oracle_ce_fwd(x.ctypes.data, code, t.ctypes.data_as(_i64p), M, V, red,
                           out.ctypes.data_as(_dp), scratch.ctypes.data_as(_dp))
    if rc:
        raise ValueError("oracle_ce_fwd: bad arguments")
    return out[:M] if red == NONE else float(out[0])


def grad_rows(x, targets, dtype="f32", c=1.0, row0=0, nrows=None, out_dtype=None,
              want64=False, d=None):
    """Gradient rows [row0, row0 + nrows) scaled by c (and by d[i], the
    upstream gradient of row i's loss, when d is given: [M] values).

    Returns the gradient rounded once to the storage type (float32 array, or
    uint16 bit patterns for fp16/bf16), and also the fp64 values if want64.
    """
    lib = _load()
    x, code = _prep(x, dtype)
    M, V = x.shape
    t = _targets(targets, M)
    if nrows is None:
        nrows = M - row0
    ocode = code if out_dtype is None else dtype_code(out_dtype)
    g = np.empty((nrows, V), dtype=np.float32 if ocode == F32 else np.uint16)
    g64 = np.empty((nrows, V), dtype=np.float64) if want64 else None
    if d is not None:
        d = np.ascontiguousarray(d, dtype=np.float64)
        if d.shape != (M,):
            raise ValueError("d must hold one upstream gradient per row")
    rc = lib.oracle_ce_grad_rows(x.ctypes.data, code, t.ctypes.data_as(_i64p), M, V,
                                 row0, nrows, float(c),
                                 d.ctypes.data_as(_dp) if d is not None else None, ocode,
                                 g.ctypes.data, g64.ctypes.data_as(_dp) if want64 else None)
    if rc:
        raise ValueError("oracle_ce_grad_rows: bad arguments")
    return (g, g64) if want64 else g


def softmax_rows(x, dtype="f32", log=False, row0=0, nrows=None, out_dtype=None,
                 want64=False, with_lse=False):
    """Row softmax (or log-softmax) of rows [row0, row0 + nrows), rounded once
    to the storage type; optionally also the fp64 values and the fp64 lse."""
    lib = _load()
    x, code = _prep(x, dtype)
    M, V = x.shape
    if nrows is None:
        nrows = M - row0
    ocode = code if out_dtype is None else dtype_code(out_dtype)
    y = np.empty((nrows, V), dtype=np.float32 if ocode == F32 else np.uint16)
    y64 = np.empty((nrows, V), dtype=np.float64) if want64 else None
    lse = np.empty(nrows, dtype=np.float64)
    rc = lib.oracle_softmax_rows(x.ctypes.data, code, M, V, row0, nrows, int(bool(log)), ocode,
                                 y.ctypes.data, y64.ctypes.data_as(_dp) if want64 else None,
                                 lse.ctypes.data_as(_dp))
    if rc:
        raise ValueError("oracle_softmax_rows: bad arguments")
    res = (y,)
    if want64:
        res += (y64,)
    if with_lse:
        res += (lse,)
    return res[0] if len(res) == 1 else res


_AT_OPS = {"grad": 0, "softmax": 1, "log_softmax": 2}


def at_elements(x, lse, rows, cols, op="grad", dtype="f32", targets=None, c=1.0, d=None,
                out_dtype=None, want64=False):
    """The gradient (op "grad", scaled by c and d[i] as in grad_rows),
    softmax or log-softmax at elements (rows[k], cols[k]) of x, from the fp64
    row log-sum-exps lse [M] (as loss_rows(..., with_lse=True) gives them).
    Returns values rounded once to the storage type (and the fp64 values if
    want64)."""
    lib = _load()
    x, code = _prep(x, dtype)
    M, V = x.shape
    lse = np.ascontiguousarray(lse, dtype=np.float64)
    rows = np.ascontiguousarray(np.broadcast_to(rows, np.shape(cols)), dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if lse.shape != (M,) or rows.shape != cols.shape or cols.ndim != 1:
        raise ValueError("lse must be [M]; rows and cols 1-D of one length")
    t = _targets(targets, M) if targets is not None else None
    if op == "grad" and t is None:
        raise ValueError("the gradient needs the targets")
    if d is not None:
        d = np.ascontiguousarray(d, dtype=np.float64)
        if d.shape != (M,):
            raise ValueError("d must hold one upstream gradient per row")
    ocode = code if out_dtype is None else dtype_code(out_dtype)
    n = cols.size
    y = np.empty(n, dtype=np.float32 if ocode == F32 else np.uint16)
    y64 = np.empty(n, dtype=np.float64) if want64 else None
    rc = lib.oracle_at_elements(x.ctypes.data, code,
                                t.ctypes.data_as(_i64p) if t is not None else None, M, V,
                                lse.ctypes.data_as(_dp), n, rows.ctypes.data_as(_i64p),
                                cols.ctypes.data_as(_i64p), _AT_OPS[op], float(c),
                                d.ctypes.data_as(_dp) if d is not None else None, ocode,
                                y.ctypes.data, y64.ctypes.data_as(_dp) if want64 else None)
    if rc:
        raise ValueError("oracle_at_elements: bad arguments")
    return (y, y64) if want64 else y


def linear_ce(h_bits, w_bits, targets, reduction="mean", grads=False):
    """Linear + cross-entropy on bf16 bit patterns H [M, D], W [V, D].

    Returns (loss, lse) -- loss as fp64 [M] for 'none', else a float -- and,
    with grads, also (G, dH, dW) in fp64: the logits' gradient [M, V] and the
    gradients of the hidden states [M, D] and the weight [V, D].
    """
    lib = _load()
    h = np.ascontiguousarray(h_bits, dtype=np.uint16)
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    if h.ndim != 2 or w.ndim != 2 or h.shape[1] != w.shape[1]:
        raise ValueError("H must be [M, D] and W [V, D]")
    M, D = h.shape
    V = w.shape[0]
    t = _targets(targets, M)
    red = _RED_CODE[reduction]
    out = np.empty(max(M, 1) if red == NONE else 1, dtype=np.float64)
    lse = np.empty(max(M, 1), dtype=np.float64)
    G = np.empty((M, V), dtype=np.float64) if grads else None
    dH = np.empty((M, D), dtype=np.float64) if grads else None
    dW = np.empty((V, D), dtype=np.float64) if grads else None
    u16p = ctypes.POINTER(ctypes.c_uint16)
    rc = lib.oracle_linear_ce(h.ctypes.data_as(u16p), w.ctypes.data_as(u16p),
                              t.ctypes.data_as(_i64p), M, D, V, red, out.ctypes.data_as(_dp),
                              lse.ctypes.data_as(_dp),
                              G.ctypes.data_as(_dp) if grads else None,
                              dH.ctypes.data_as(_dp) if grads else None,
                              dW.ctypes.data_as(_dp) if grads else None)
    if rc:
        raise ValueError("oracle_linear_ce: bad arguments")
    loss = out[:M] if red == NONE else float(out[0])
    if grads:
        return loss, lse[:M], G, dH, dW
    return loss, lse[:M]


def widen(bits, dtype):
    """fp16/bf16 bit patterns -> fp64, by the oracle's own decoder."""
    lib = _load()
    f = lib.oracle_widen_f16 if dtype_code(dtype) == F16 else lib.oracle_widen_bf16
    bits = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([f(int(b)) for b in bits], dtype=np.float64)


def round_to(values, dtype):
    """fp64 -> storage bits (uint16 for fp16/bf16, float32 for fp32), one RNE step."""
    lib = _load()
    code = dtype_code(dtype)
    values = np.asarray(values, dtype=np.float64).ravel()
    if code == F32:
        return np.array([lib.oracle_round_f32(float(v)) for v in values], dtype=np.float32)
    f = lib.oracle_round_f16 if code == F16 else lib.oracle_round_bf16
    return np.array([f(float(v)) for v in values], dtype=np.uint16)


def num_threads():
    return int(_load().oracle_num_threads())


def set_num_threads(n):
    """Threads of the oracle's row loops from now on (for timing)."""
    _load().oracle_set_num_threads(int(n))
