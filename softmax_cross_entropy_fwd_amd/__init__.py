"""Row-wise softmax cross-entropy on MI355X (gfx950).

A thin ctypes binding over the C ABI in ``include/ce.h`` (``libce.so``, built
from ``csrc/`` by ``python -m softmax_cross_entropy_fwd_amd.build``).  The
functions keep the C names; they only marshal torch tensors into pointers and
sizes and pass torch's current HIP stream.  Every step of the computation runs
in the library's HIP kernels; if the library is missing, every call raises.

    loss = ce_fwd(logits, targets, reduction="mean")
    loss = ce_fwd_noalloc(logits, targets, reduction="mean", out=out)   # no workspace
    loss = ce_fwd_bwd_inplace(logits, targets, reduction="mean")   # logits <- grad
    loss, lse = ce_fwd_lse(logits, targets, reduction="mean")
    grad = ce_bwd(logits, targets, lse, reduction="mean", dloss=None)
    probs = ce_softmax(logits)                    # or log_softmax=True
    loss, lse = ce_linear_fwd(hidden, weight, targets)            # logits = hidden @ weight.T
    loss, dhidden, dweight = ce_linear_fwd_bwd(hidden, weight, targets)
"""
import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
# CE_LIBRARY: another build of the library (the host-sanitizer test's)
LIB_PATH = os.environ.get("CE_LIBRARY") or os.path.join(_PKG, "libce.so")

CE_F32, CE_F16, CE_BF16 = 0, 1, 2
CE_NONE, CE_MEAN, CE_SUM = 0, 1, 2
CE_OK = 0
CE_ERR_NULL, CE_ERR_SHAPE, CE_ERR_DTYPE, CE_ERR_REDUCTION = -1, -2, -3, -4
CE_ERR_WORKSPACE, CE_ERR_HIP, CE_ERR_ALIGNMENT, CE_ERR_ALIAS = -5, -6, -7, -8
CE_ERR_SCRATCH = -9
CE_NOALLOC_SCRATCH_BYTES = 229888
CE_OP_FWD, CE_OP_FWD_BWD, CE_OP_SOFTMAX, CE_OP_LOG_SOFTMAX, CE_OP_BWD = 0, 1, 2, 3, 4
REDUCTIONS = {"none": CE_NONE, "mean": CE_MEAN, "sum": CE_SUM}

_lib = None
_lock = threading.Lock()
_workspaces = {}
_codes = None          # torch dtype -> CE_* code
_raw_stream = None     # torch's accessor of the current raw stream handle
_get_device = None     # torch's accessor of the current device index


class CEError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, ce_status_string(status), status))


def load_library(path=None):
    """Load libce.so (after torch, so the library binds to torch's HIP runtime)."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        import torch  # noqa: F401  -- loads the HIP runtime libce.so must share
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError("%s is not built; run `python -m softmax_cross_entropy_fwd_amd.build`" % p)
        lib = ctypes.CDLL(p)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        lib.ce_workspace_bytes.argtypes = [i64, i64, i32, i32]
        lib.ce_workspace_bytes.restype = sz
        lib.ce_fwd.argtypes = [vp, vp, i64, i64, i32, i32, vp, vp, sz, vp]
        lib.ce_fwd.restype = i32
        lib.ce_fwd_noalloc.argtypes = [vp, vp, i64, i64, i32, i32, vp, vp]
        lib.ce_fwd_noalloc.restype = i32
        lib.ce_fwd_bwd_inplace.argtypes = [vp, vp, i64, i64, i32, i32, vp, vp, sz, vp]
        lib.ce_fwd_bwd_inplace.restype = i32
        lib.ce_fwd_lse.argtypes = [vp, vp, i64, i64, i32, i32, vp, vp, vp, sz, vp]
        lib.ce_fwd_lse.restype = i32
        lib.ce_bwd.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, vp, vp, sz, vp]
        lib.ce_bwd.restype = i32
        lib.ce_softmax.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, sz, vp]
        lib.ce_softmax.restype = i32
        lib.ce_linear_chunk.argtypes = [i64, i64, i64, i64]
        lib.ce_linear_chunk.restype = i64
        lib.ce_linear_workspace_bytes.argtypes = [i64, i64, i64, i64]
        lib.ce_linear_workspace_bytes.restype = sz
        lib.ce_linear_fwd.argtypes = [vp, vp, vp, i64, i64, i64, i32, vp, vp, i64, vp, sz, vp]
        lib.ce_linear_fwd.restype = i32
        lib.ce_linear_fwd_bwd.argtypes = [vp, vp, vp, i64, i64, i64, i32, vp, vp, vp, vp, i64, vp,
                                          sz, vp]
        lib.ce_linear_fwd_bwd.restype = i32
        lib.ce_status_string.argtypes = [i32]
        lib.ce_status_string.restype = ctypes.c_char_p
        lib.ce_plan_describe.argtypes = [i64, i64, i32, i32, i32, ctypes.c_char_p, sz]
        lib.ce_plan_describe.restype = i32
        lib.ce_tuning_reload.argtypes = []
        lib.ce_tuning_reload.restype = None
        if path is None:
            _lib = lib
        return lib


def reload_tuning():
    """Make the library read its tuning environment variables again (it reads
    them once, at its first call); for tuning and tests, not while other
    threads call the library."""
    load_library().ce_tuning_reload()
    _ws_bytes.clear()


def _dtype_code(t):
    global _codes
    if _codes is None:
        import torch
        _codes = {torch.float32: CE_F32, torch.float16: CE_F16, torch.bfloat16: CE_BF16}
    code = _codes.get(t.dtype)
    if code is None:
        raise TypeError("logits must be float32, float16 or bfloat16, got %s" % t.dtype)
    return code


def ce_status_string(status):
    return load_library().ce_status_string(int(status)).decode()


def ce_workspace_bytes(M, V, dtype, reduction):
    """Workspace bytes a call needs (dtype: CE_* code, reduction: name or code)."""
    red = REDUCTIONS.get(reduction, reduction)
    return int(load_library().ce_workspace_bytes(int(M), int(V), int(dtype), int(red)))


def ce_plan_describe(M, V, dtype, reduction="mean", fwd_bwd=False, op=None):
    """The launch plan the library picks on the current device (op: CE_OP_*;
    by default the forward, or the fused backward when fwd_bwd)."""
    red = REDUCTIONS.get(reduction, reduction)
    if op is None:
        op = CE_OP_FWD_BWD if fwd_bwd else CE_OP_FWD
    buf = ctypes.create_string_buffer(256)
    rc = load_library().ce_plan_describe(int(M), int(V), int(dtype), int(red), int(op), buf, 256)
    if rc:
        raise CEError(rc, "ce_plan_describe")
    return buf.value.decode()


def workspace_for(device, stream, nbytes):
    """A workspace cached per (device, stream) (its contents need no initialization)."""
    return _cached_workspace(device, int(stream.cuda_stream), nbytes, stream)


def _cached_workspace(device, handle, nbytes, stream=None):
    import torch
    key = (device.index, handle)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        if stream is None:
            stream = torch.cuda.current_stream(device)
        with torch.cuda.stream(stream):
            ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _stream_handle(dev):
    """The raw hipStream_t of torch's current stream on dev (torch's own
    accessor when it has one: the Stream object costs ~2 us per call)."""
    global _raw_stream
    if _raw_stream is None:
        import torch
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _raw_stream = raw if raw is not None else (
            lambda i: torch.cuda.current_stream(i).cuda_stream)
    return int(_raw_stream(dev.index))


# sizes from ce_workspace_bytes, which also depend on the split and plan
# overrides the library read (cleared by reload_tuning)
_ws_bytes = {}


def _workspace_bytes(lib, M, V, code, red):
    key = (M, V, code, red)
    n = _ws_bytes.get(key)
    if n is None:
        n = int(lib.ce_workspace_bytes(M, V, code, red))
        if len(_ws_bytes) < 4096:
            _ws_bytes[key] = n
    return n


def _check_logits(logits):
    if not logits.is_cuda:
        raise ValueError("logits must be a device tensor")
    if logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous [M, V] tensor")


def _check_rows(t, M, dev, what):
    import torch
    if t.dtype != torch.float32 or not t.is_contiguous() or t.device != dev or t.numel() != M:
        raise ValueError("%s must be a contiguous float32 tensor of %d entries on %s" % (what, M, dev))


def _check_like(out, logits, what):
    if (out.dtype != logits.dtype or out.shape != logits.shape or not out.is_contiguous()
            or out.device != logits.device):
        raise ValueError("%s must be a contiguous tensor shaped and typed like the logits" % what)


def _check(logits, targets):
    import torch
    _check_logits(logits)
    if targets.dtype != torch.int64 or targets.dim() != 1 or not targets.is_contiguous():
        raise ValueError("targets must be a contiguous int64 [M] tensor")
    if targets.get_device() != logits.get_device() or targets.numel() != logits.shape[0]:
        raise ValueError("targets must be on the logits' device with M entries")


def _invoke(fn, dev, args):
    """Calls a library entry point with dev current (switching only if needed)."""
    global _get_device
    import torch
    if _get_device is None:
        _get_device = getattr(torch._C, "_cuda_getDevice", torch.cuda.current_device)
    if _get_device() == dev.index:
        return fn(*args)
    with torch.cuda.device(dev):
        return fn(*args)


def _call(fn_name, logits, targets, reduction, out, workspace, lse=None):
    import torch
    lib = _lib or load_library()
    _check(logits, targets)
    red = REDUCTIONS[reduction]
    M, V = logits.shape
    dev = logits.device
    if out is None:
        out = torch.empty((M,) if red == CE_NONE else (), dtype=torch.float32, device=dev)
    else:
        _check_rows(out, M if red == CE_NONE else 1, dev, "out")
    stream = _stream_handle(dev)
    code = _dtype_code(logits)
    nbytes = _workspace_bytes(lib, M, V, code, red)
    if nbytes and workspace is None:
        workspace = _cached_workspace(dev, stream, nbytes)
    ws_ptr = workspace.data_ptr() if nbytes else None
    ws_len = workspace.numel() * workspace.element_size() if nbytes else 0
    args = [logits.data_ptr(), targets.data_ptr(), M, V, code, red,
            out.data_ptr() if out.numel() else None]
    if fn_name == "ce_fwd_lse":
        _check_rows(lse, M, dev, "lse")
        args.append(lse.data_ptr() if M else None)
    rc = _invoke(getattr(lib, fn_name), dev, args + [ws_ptr, ws_len, stream])
    if rc:
        raise CEError(rc, fn_name)
    return out


def ce_fwd(logits, targets, reduction="mean", out=None, workspace=None):
    """Cross-entropy of each row of logits [M, V] against targets [M].

    Returns a 0-d fp32 tensor (mean, sum) or the [M] fp32 row losses (none).
    """
    return _call("ce_fwd", logits, targets, reduction, out, workspace)


def ce_fwd_noalloc(logits, targets, reduction="mean", out=None):
    """ce_fwd with the library's static per-device scratch in place of a
    workspace: the C call allocates no device memory (pass out to allocate
    nothing here either).  Calls that overlap on one GPU race on the scratch."""
    import torch
    lib = load_library()
    _check(logits, targets)
    red = REDUCTIONS[reduction]
    M, V = logits.shape
    dev = logits.device
    if out is None:
        out = torch.empty((M,) if red == CE_NONE else (), dtype=torch.float32, device=dev)
    else:
        _check_rows(out, M if red == CE_NONE else 1, dev, "out")
    rc = _invoke(lib.ce_fwd_noalloc, dev,
                 [logits.data_ptr(), targets.data_ptr(), M, V, _dtype_code(logits), red,
                  out.data_ptr() if out.numel() else None, _stream_handle(dev)])
    if rc:
        raise CEError(rc, "ce_fwd_noalloc")
    return out


def ce_fwd_bwd_inplace(logits, targets, reduction="mean", out=None, workspace=None):
    """Loss as ce_fwd, and logits overwritten with d(loss)/d(logits)."""
    return _call("ce_fwd_bwd_inplace", logits, targets, reduction, out, workspace)


def ce_fwd_lse(logits, targets, reduction="mean", out=None, lse=None, workspace=None):
    """Loss as ce_fwd, plus the [M] fp32 row log-sum-exps; returns (loss, lse)."""
    import torch
    if lse is None:
        lse = torch.empty(logits.shape[0], dtype=torch.float32, device=logits.device)
    return _call("ce_fwd_lse", logits, targets, reduction, out, workspace, lse=lse), lse


def _workspace(lib, logits, red, workspace):
    """(pointer, bytes) of the workspace a call can use, cached per stream
    unless one is given; (None, 0) when the call uses none."""
    import torch
    M, V = logits.shape
    nbytes = _workspace_bytes(lib, M, V, _dtype_code(logits), red)
    if not nbytes:
        return None, 0
    if workspace is None:
        workspace = _cached_workspace(logits.device, _stream_handle(logits.device), nbytes)
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def ce_bwd(logits, targets, lse, reduction="mean", dloss=None, grad=None, workspace=None):
    """Gradient of the loss from saved row log-sum-exps, into grad (a new
    tensor by default; grad=logits overwrites the logits).  dloss: the
    upstream gradient, [M] for 'none', one element otherwise, or None for 1."""
    import torch
    lib = load_library()
    _check(logits, targets)
    red = REDUCTIONS[reduction]
    M, V = logits.shape
    dev = logits.device
    _check_rows(lse, M, dev, "lse")
    if dloss is not None:
        _check_rows(dloss, M if red == CE_NONE else 1, dev, "dloss")
    if grad is None:
        grad = torch.empty_like(logits)
    _check_like(grad, logits, "grad")
    stream = _stream_handle(dev)
    ws_ptr, ws_len = _workspace(lib, logits, red, workspace)
    rc = _invoke(lib.ce_bwd, dev,
                 [logits.data_ptr(), targets.data_ptr(), lse.data_ptr() if M else None,
                  dloss.data_ptr() if dloss is not None else None, M, V, _dtype_code(logits),
                  red, grad.data_ptr() if M else None, ws_ptr, ws_len, stream])
    if rc:
        raise CEError(rc, "ce_bwd")
    return grad


def ce_softmax(logits, log_softmax=False, out=None, lse=None, workspace=None):
    """Row softmax (or log-softmax) of logits [M, V] in their dtype, into out
    (a new tensor by default; out=logits works in place).  lse: optional [M]
    fp32 tensor that receives the row log-sum-exps."""
    import torch
    lib = load_library()
    _check_logits(logits)
    M, V = logits.shape
    dev = logits.device
    if out is None:
        out = torch.empty_like(logits)
    _check_like(out, logits, "out")
    if lse is not None:
        _check_rows(lse, M, dev, "lse")
    stream = _stream_handle(dev)
    ws_ptr, ws_len = _workspace(lib, logits, CE_NONE, workspace)
    rc = _invoke(lib.ce_softmax, dev,
                 [logits.data_ptr(), M, V, _dtype_code(logits), int(bool(log_softmax)),
                  out.data_ptr() if M else None,
                  lse.data_ptr() if (lse is not None and M) else None,
                  ws_ptr, ws_len, stream])
    if rc:
        raise CEError(rc, "ce_softmax")
    return out


def _linear(fn_name, hidden, weight, targets, reduction, chunk, workspace, bwd):
    import torch
    lib = load_library()
    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("hidden and weight must be bfloat16")
    for t, name in ((hidden, "hidden"), (weight, "weight")):
        if not t.is_cuda or t.dim() != 2 or not t.is_contiguous():
            raise ValueError("%s must be a contiguous 2-D device tensor" % name)
    M, D = hidden.shape
    V = weight.shape[0]
    if weight.shape[1] != D or weight.device != hidden.device:
        raise ValueError("weight must be [V, D] on the hidden states' device")
    if (targets.dtype != torch.int64 or targets.dim() != 1 or not targets.is_contiguous()
            or targets.numel() != M or targets.device != hidden.device):
        raise ValueError("targets must be a contiguous int64 [M] tensor on the same device")
    red = REDUCTIONS[reduction]
    dev = hidden.device
    out = torch.empty((M,) if red == CE_NONE else (), dtype=torch.float32, device=dev)
    lse = torch.empty(M, dtype=torch.float32, device=dev)
    nbytes = int(lib.ce_linear_workspace_bytes(M, D, V, int(chunk)))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    ws_len = workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(dev)
    args = [hidden.data_ptr(), weight.data_ptr(), targets.data_ptr(), M, D, V, red,
            out.data_ptr() if out.numel() else None, lse.data_ptr() if M else None]
    if bwd:
        dh = torch.empty((M, D), dtype=torch.float32, device=dev)
        dw = torch.empty((V, D), dtype=torch.float32, device=dev)
        args += [dh.data_ptr() if M else None, dw.data_ptr()]
    rc = _invoke(getattr(lib, fn_name), dev,
                 args + [int(chunk), workspace.data_ptr(), ws_len, stream.cuda_stream])
    if rc:
        raise CEError(rc, fn_name)
    return (out, lse, dh, dw) if bwd else (out, lse)


def ce_linear_fwd(hidden, weight, targets, reduction="mean", chunk=0, workspace=None):
    """Cross-entropy of the logits hidden @ weight.T (bf16 [M, D] and [V, D]),
    taken over vocabulary chunks; returns (loss, lse)."""
    return _linear("ce_linear_fwd", hidden, weight, targets, reduction, chunk, workspace, False)


def ce_linear_fwd_bwd(hidden, weight, targets, reduction="mean", chunk=0, workspace=None):
    """Loss as ce_linear_fwd and its gradients; returns (loss, lse, dhidden,
    dweight), the gradients in fp32."""
    return _linear("ce_linear_fwd_bwd", hidden, weight, targets, reduction, chunk, workspace,
                   True)


__all__ = ["ce_fwd", "ce_fwd_noalloc", "ce_fwd_lse", "ce_fwd_bwd_inplace", "ce_bwd", "ce_softmax",
           "ce_linear_fwd", "ce_linear_fwd_bwd",
           "ce_workspace_bytes", "ce_status_string", "ce_plan_describe", "load_library",
           "CEError", "LIB_PATH"]
