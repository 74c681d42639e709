"""The C ABI without a GPU: the library loads, exports every symbol include/ce.h
declares, and rejects bad arguments with the documented status before any HIP
call (argument checks come first in every entry point)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("ce.h", "ce_linear.h")]


@pytest.fixture(scope="module")
def lib():
    import softmax_cross_entropy_fwd_amd as ce
    if not os.path.exists(ce.LIB_PATH):
        from softmax_cross_entropy_fwd_amd import build
        build.build()
    return ce.load_library()


def declared_functions():
    names = set()
    for header in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
        names.update(re.findall(r"\b(ce_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("ce_fwd", "ce_fwd_lse", "ce_fwd_bwd_inplace", "ce_bwd", "ce_softmax",
              "ce_workspace_bytes", "ce_status_string", "ce_plan_describe", "ce_linear_chunk",
              "ce_linear_workspace_bytes", "ce_linear_fwd", "ce_linear_fwd_bwd"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    import softmax_cross_entropy_fwd_amd as ce
    out = subprocess.run(["nm", "-D", "--defined-only", ce.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)


def test_library_links_no_oracle_code(lib):
    import softmax_cross_entropy_fwd_amd as ce
    out = subprocess.run(["nm", "-D", ce.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    assert "oracle" not in out


FAKE = 0x100000          # never dereferenced: every case fails its checks first
VP = ctypes.c_void_p


def call(lib, fn, logits=FAKE, targets=FAKE, M=4, V=8, dtype=0, red=1, out=FAKE + 4096,
         ws=FAKE + 8192, ws_bytes=1 << 20, stream=None):
    f = getattr(lib, fn)
    return f(VP(logits) if logits else None, VP(targets) if targets else None, M, V, dtype, red,
             VP(out) if out else None, VP(ws) if ws else None, ws_bytes, stream)


@pytest.mark.parametrize("fn", ["ce_fwd", "ce_fwd_bwd_inplace"])
def test_argument_errors(lib, fn):
    import softmax_cross_entropy_fwd_amd as ce
    assert call(lib, fn, dtype=3) == ce.CE_ERR_DTYPE
    assert call(lib, fn, dtype=-1) == ce.CE_ERR_DTYPE
    assert call(lib, fn, red=3) == ce.CE_ERR_REDUCTION
    assert call(lib, fn, M=-1) == ce.CE_ERR_SHAPE
    assert call(lib, fn, V=0) == ce.CE_ERR_SHAPE
    assert call(lib, fn, V=1 << 31) == ce.CE_ERR_SHAPE
    assert call(lib, fn, M=1 << 62, V=1 << 20) == ce.CE_ERR_SHAPE
    assert call(lib, fn, logits=0) == ce.CE_ERR_NULL
    assert call(lib, fn, targets=0) == ce.CE_ERR_NULL
    assert call(lib, fn, out=0) == ce.CE_ERR_NULL
    assert call(lib, fn, logits=FAKE + 2, dtype=0) == ce.CE_ERR_ALIGNMENT
    assert call(lib, fn, logits=FAKE + 1, dtype=2) == ce.CE_ERR_ALIGNMENT
    assert call(lib, fn, ws=0) == ce.CE_ERR_WORKSPACE
    assert call(lib, fn, ws_bytes=100) == ce.CE_ERR_WORKSPACE
    assert call(lib, fn, ws=FAKE + 8196) == ce.CE_ERR_WORKSPACE
    # M == 0 with no reduction has nothing to do and touches nothing
    assert call(lib, fn, M=0, red=0, logits=0, targets=0, out=0, ws=0, ws_bytes=0) == ce.CE_OK
    # M == 0 with a reduction still needs somewhere to write the scalar
    assert call(lib, fn, M=0, red=1, logits=0, targets=0, out=0, ws=0, ws_bytes=0) == ce.CE_ERR_NULL


def test_inplace_alias_checks(lib):
    import softmax_cross_entropy_fwd_amd as ce
    M, V = 4, 8
    xb = M * V * 4
    # targets inside the logits
    assert call(lib, "ce_fwd_bwd_inplace", targets=FAKE + 16) == ce.CE_ERR_ALIAS
    # output inside the logits
    assert call(lib, "ce_fwd_bwd_inplace", out=FAKE + xb - 4) == ce.CE_ERR_ALIAS
    # workspace overlapping the logits' end
    assert call(lib, "ce_fwd_bwd_inplace", ws=FAKE + xb - 8) == ce.CE_ERR_ALIAS


def test_forward_output_may_not_overlap_inputs(lib):
    import softmax_cross_entropy_fwd_amd as ce
    xb = 4 * 8 * 4
    assert call(lib, "ce_fwd", out=FAKE + xb - 4) == ce.CE_ERR_ALIAS
    assert call(lib, "ce_fwd", red=0, ws=0, ws_bytes=0, out=FAKE + 8) == ce.CE_ERR_ALIAS


def call_lse(lib, lse=FAKE + 12288, **kw):
    kw.setdefault("logits", FAKE)
    kw.setdefault("targets", FAKE + 2048)
    kw.setdefault("M", 4)
    kw.setdefault("V", 8)
    kw.setdefault("dtype", 0)
    kw.setdefault("red", 1)
    kw.setdefault("out", FAKE + 4096)
    kw.setdefault("ws", FAKE + 8192 * 4)
    kw.setdefault("ws_bytes", 1 << 20)
    return lib.ce_fwd_lse(VP(kw["logits"]) if kw["logits"] else None,
                          VP(kw["targets"]) if kw["targets"] else None, kw["M"], kw["V"],
                          kw["dtype"], kw["red"], VP(kw["out"]) if kw["out"] else None,
                          VP(lse) if lse else None, VP(kw["ws"]) if kw["ws"] else None,
                          kw["ws_bytes"], None)


def test_fwd_lse_argument_errors(lib):
    import softmax_cross_entropy_fwd_amd as ce
    assert call_lse(lib, lse=0) == ce.CE_ERR_NULL
    assert call_lse(lib, lse=FAKE + 12290) == ce.CE_ERR_ALIGNMENT
    assert call_lse(lib, lse=FAKE + 4096) == ce.CE_ERR_ALIAS            # on the loss output
    assert call_lse(lib, lse=FAKE + 64) == ce.CE_ERR_ALIAS              # inside the logits
    assert call_lse(lib, lse=FAKE + 2048 + 16) == ce.CE_ERR_ALIAS       # on the targets
    assert call_lse(lib, dtype=7) == ce.CE_ERR_DTYPE
    assert call_lse(lib, M=0, red=0, lse=0, logits=0, targets=0, out=0, ws=0,
                    ws_bytes=0) == ce.CE_OK


def call_bwd(lib, logits=FAKE, targets=FAKE + 2048, lse=FAKE + 3072, dloss=None, M=4, V=8,
             dtype=0, red=1, grad=FAKE + 65536, ws=None, ws_bytes=0):
    return lib.ce_bwd(VP(logits) if logits else None, VP(targets) if targets else None,
                      VP(lse) if lse else None, VP(dloss) if dloss else None, M, V, dtype, red,
                      VP(grad) if grad else None, VP(ws) if ws else None, ws_bytes, None)


def test_bwd_argument_errors(lib):
    import softmax_cross_entropy_fwd_amd as ce
    assert call_bwd(lib, dtype=3) == ce.CE_ERR_DTYPE
    assert call_bwd(lib, red=9) == ce.CE_ERR_REDUCTION
    assert call_bwd(lib, M=-2) == ce.CE_ERR_SHAPE
    assert call_bwd(lib, V=0) == ce.CE_ERR_SHAPE
    assert call_bwd(lib, logits=0) == ce.CE_ERR_NULL
    assert call_bwd(lib, targets=0) == ce.CE_ERR_NULL
    assert call_bwd(lib, lse=0) == ce.CE_ERR_NULL
    assert call_bwd(lib, grad=0) == ce.CE_ERR_NULL
    assert call_bwd(lib, lse=FAKE + 3073) == ce.CE_ERR_ALIGNMENT
    assert call_bwd(lib, dloss=FAKE + 4098) == ce.CE_ERR_ALIGNMENT
    # the gradient is written with the logits' 16-byte vectors
    assert call_bwd(lib, grad=FAKE + 65536 + 4) == ce.CE_ERR_ALIGNMENT
    assert call_bwd(lib, dtype=2, grad=FAKE + 65536 + 2) == ce.CE_ERR_ALIGNMENT
    # a gradient that overlaps the logits without being them
    assert call_bwd(lib, grad=FAKE + 16) == ce.CE_ERR_ALIAS
    # a gradient over the targets, the lse or the upstream gradient
    assert call_bwd(lib, grad=FAKE + 2048) == ce.CE_ERR_ALIAS
    assert call_bwd(lib, grad=FAKE + 3072 - 64) == ce.CE_ERR_ALIAS
    assert call_bwd(lib, dloss=FAKE + 65536 + 32) == ce.CE_ERR_ALIAS
    # nothing to do for M == 0
    assert call_bwd(lib, M=0, logits=0, targets=0, lse=0, grad=0) == ce.CE_OK


def call_softmax(lib, logits=FAKE, M=4, V=8, dtype=0, log=0, out=FAKE + 65536, lse=None,
                 ws=None, ws_bytes=0):
    return lib.ce_softmax(VP(logits) if logits else None, M, V, dtype, log,
                          VP(out) if out else None, VP(lse) if lse else None,
                          VP(ws) if ws else None, ws_bytes, None)


def test_softmax_argument_errors(lib):
    import softmax_cross_entropy_fwd_amd as ce
    assert call_softmax(lib, dtype=3) == ce.CE_ERR_DTYPE
    assert call_softmax(lib, V=0) == ce.CE_ERR_SHAPE
    assert call_softmax(lib, logits=0) == ce.CE_ERR_NULL
    assert call_softmax(lib, out=0) == ce.CE_ERR_NULL
    assert call_softmax(lib, out=FAKE + 65536 + 8) == ce.CE_ERR_ALIGNMENT
    assert call_softmax(lib, out=FAKE + 32) == ce.CE_ERR_ALIAS
    assert call_softmax(lib, lse=FAKE + 65536 + 16) == ce.CE_ERR_ALIAS
    assert call_softmax(lib, lse=FAKE + 16) == ce.CE_ERR_ALIAS
    assert call_softmax(lib, out=FAKE, lse=FAKE + 64) == ce.CE_ERR_ALIAS   # in place
    assert call_softmax(lib, M=0, logits=0, out=0) == ce.CE_OK


def test_plan_describe_rejects_unknown_op(lib):
    import softmax_cross_entropy_fwd_amd as ce
    buf = ctypes.create_string_buffer(64)
    assert lib.ce_plan_describe(4, 8, 0, 1, 5, buf, 64) == ce.CE_ERR_SHAPE
    assert lib.ce_plan_describe(4, 8, 0, 1, -1, buf, 64) == ce.CE_ERR_SHAPE


def test_split_workspace_checks(lib):
    import softmax_cross_entropy_fwd_amd as ce
    # few long rows: the workspace also holds the split scratch, for every
    # reduction; a misaligned workspace is refused, an overlapping one too
    M, V = 8, 1 << 17
    n = lib.ce_workspace_bytes(M, V, 2, 0)
    assert n >= (128 << 10) + M * 64 * 12
    assert lib.ce_workspace_bytes(M, V, 2, 1) == n
    assert lib.ce_workspace_bytes(4096, V, 2, 0) == 0            # many rows: no split
    assert lib.ce_workspace_bytes(8, 1000, 0, 0) == 0            # short rows: no split
    big = 1 << 40
    assert call_softmax(lib, M=M, V=V, dtype=2, out=FAKE + big, ws=FAKE + 2 * big + 4,
                        ws_bytes=n) == ce.CE_ERR_WORKSPACE
    assert call_softmax(lib, M=M, V=V, dtype=2, out=FAKE + big, ws=FAKE + big + 64,
                        ws_bytes=n) == ce.CE_ERR_ALIAS
    assert call_bwd(lib, M=M, V=V, dtype=2, lse=FAKE + 3 * big, targets=FAKE + 3 * big + 4096,
                    grad=FAKE + big, ws=FAKE + 64, ws_bytes=n) == ce.CE_ERR_ALIAS


def call_noalloc(lib, logits=FAKE, targets=FAKE, M=4, V=8, dtype=0, red=1, out=FAKE + 4096):
    return lib.ce_fwd_noalloc(VP(logits) if logits else None, VP(targets) if targets else None,
                              M, V, dtype, red, VP(out) if out else None, None)


def test_noalloc_argument_errors(lib, tuning):
    import softmax_cross_entropy_fwd_amd as ce
    assert call_noalloc(lib, dtype=3) == ce.CE_ERR_DTYPE
    assert call_noalloc(lib, red=3) == ce.CE_ERR_REDUCTION
    assert call_noalloc(lib, M=-1) == ce.CE_ERR_SHAPE
    assert call_noalloc(lib, V=0) == ce.CE_ERR_SHAPE
    assert call_noalloc(lib, logits=0) == ce.CE_ERR_NULL
    assert call_noalloc(lib, targets=0) == ce.CE_ERR_NULL
    assert call_noalloc(lib, out=0) == ce.CE_ERR_NULL
    assert call_noalloc(lib, logits=FAKE + 1) == ce.CE_ERR_ALIGNMENT
    assert call_noalloc(lib, out=FAKE + 16) == ce.CE_ERR_ALIAS       # inside the logits
    # Beyond the scratch: 512 rows of 131072 bf16 split 16 ways (forced) would
    # need 128 KiB + 512 * (16 * 12 + 4) bytes, more than it holds; refused
    # before any HIP call.  Unforced, 512 rows are not split and need only the
    # partial sums (such a call would run; it is not made here, without a GPU).
    big = 1 << 40
    tuning.setenv("CE_FORCE_SPLIT", "64")
    assert (128 << 10) + 512 * (16 * 12 + 4) > ce.CE_NOALLOC_SCRATCH_BYTES
    assert call_noalloc(lib, logits=FAKE, targets=FAKE + big, M=512, V=1 << 17, dtype=2,
                        out=FAKE + 2 * big) == ce.CE_ERR_SCRATCH
    assert call_noalloc(lib, logits=FAKE, targets=FAKE + big, M=512, V=1 << 17, dtype=2, red=0,
                        out=FAKE + 2 * big) == ce.CE_ERR_SCRATCH
    assert "scratch" in ce.ce_status_string(ce.CE_ERR_SCRATCH)


def test_noalloc_scratch_size_is_stated_in_the_header():
    import re
    import softmax_cross_entropy_fwd_amd as ce
    text = open(HEADERS[0]).read()
    m = re.search(r"#define CE_NOALLOC_SCRATCH_BYTES (\d+)", text)
    assert m and int(m.group(1)) == ce.CE_NOALLOC_SCRATCH_BYTES == (128 << 10) + 128 * (64 * 12 + 4)


def test_workspace_bytes(lib):
    assert lib.ce_workspace_bytes(100, 1000, 0, 0) == 0         # none
    mean = lib.ce_workspace_bytes(100, 1000, 0, 1)
    assert mean >= 256 + 8 * 4096
    assert lib.ce_workspace_bytes(100, 1000, 2, 2) == mean      # sum
    assert lib.ce_workspace_bytes(0, 1000, 0, 1) == 0
    assert lib.ce_workspace_bytes(10, 0, 0, 1) == 0
    assert lib.ce_workspace_bytes(10, 10, 5, 1) == 0


def test_status_strings(lib):
    import softmax_cross_entropy_fwd_amd as ce
    seen = set()
    for code in range(-9, 1):
        s = lib.ce_status_string(code).decode()
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 10
    assert lib.ce_status_string(-99).decode() == "unknown status"
    assert "overlaps" in ce.ce_status_string(ce.CE_ERR_ALIAS)


def test_binding_rejects_host_tensors():
    import torch
    import softmax_cross_entropy_fwd_amd as ce
    x = torch.zeros(2, 3)
    t = torch.zeros(2, dtype=torch.int64)
    with pytest.raises(ValueError):
        ce.ce_fwd(x, t)


def call_linear(lib, fn="ce_linear_fwd_bwd", H=FAKE, W=FAKE + (1 << 30), t=FAKE + (2 << 30),
                M=4, D=8, V=300, red=1, out=FAKE + (3 << 30), lse=None, dH=FAKE + (4 << 30),
                dW=FAKE + (5 << 30), chunk=0, ws=FAKE + (6 << 30), ws_bytes=1 << 30):
    vp = lambda a: VP(a) if a else None
    args = [vp(H), vp(W), vp(t), M, D, V, red, vp(out), vp(lse)]
    if fn == "ce_linear_fwd_bwd":
        args += [vp(dH), vp(dW)]
    return getattr(lib, fn)(*args, chunk, vp(ws), ws_bytes, None)


def test_linear_chunk_and_workspace(lib):
    assert lib.ce_linear_chunk(4096, 4096, 131072, 0) == 8192
    assert lib.ce_linear_chunk(1 << 20, 64, 131072, 0) == 1024   # at least 1024 columns
    assert lib.ce_linear_chunk(4, 8, 300, 0) == 512            # the whole vocabulary, rounded
    assert lib.ce_linear_chunk(4, 8, 3000, 100) == 256         # rounded up to 256 columns
    assert lib.ce_linear_chunk(-1, 8, 300, 0) == 0
    n = lib.ce_linear_workspace_bytes(64, 128, 5000, 1024)
    assert n >= 64 * 1024 * 6 + 64 * 5 * 8
    # the matrix-core path: (max, sum) per token and 128 vocabulary rows, and
    # the bf16 gradient chunk
    assert n >= 64 * 2 * ((5000 + 255) // 256) * 8 + 1024 * 64 * 2
    assert lib.ce_linear_workspace_bytes(64, 0, 5000, 0) == 0


@pytest.mark.parametrize("fn", ["ce_linear_fwd", "ce_linear_fwd_bwd"])
def test_linear_argument_errors(lib, fn):
    import softmax_cross_entropy_fwd_amd as ce
    assert call_linear(lib, fn, red=5) == ce.CE_ERR_REDUCTION
    assert call_linear(lib, fn, M=-1) == ce.CE_ERR_SHAPE
    assert call_linear(lib, fn, D=0) == ce.CE_ERR_SHAPE
    assert call_linear(lib, fn, V=1 << 31) == ce.CE_ERR_SHAPE
    assert call_linear(lib, fn, H=0) == ce.CE_ERR_NULL
    assert call_linear(lib, fn, W=0) == ce.CE_ERR_NULL
    assert call_linear(lib, fn, t=0) == ce.CE_ERR_NULL
    assert call_linear(lib, fn, out=0) == ce.CE_ERR_NULL
    assert call_linear(lib, fn, H=FAKE + 1) == ce.CE_ERR_ALIGNMENT
    assert call_linear(lib, fn, t=FAKE + (2 << 30) + 4) == ce.CE_ERR_ALIGNMENT
    assert call_linear(lib, fn, ws=0) == ce.CE_ERR_WORKSPACE
    assert call_linear(lib, fn, ws_bytes=1000) == ce.CE_ERR_WORKSPACE
    assert call_linear(lib, fn, ws=FAKE + (6 << 30) + 8) == ce.CE_ERR_WORKSPACE
    assert call_linear(lib, fn, out=FAKE + 8) == ce.CE_ERR_ALIAS          # inside H
    assert call_linear(lib, fn, lse=FAKE + (2 << 30)) == ce.CE_ERR_ALIAS  # on the targets
    assert call_linear(lib, fn, ws=FAKE + (3 << 30) - 256) == ce.CE_ERR_ALIAS
    if fn == "ce_linear_fwd_bwd":
        assert call_linear(lib, fn, dH=0) == ce.CE_ERR_NULL
        assert call_linear(lib, fn, dW=0) == ce.CE_ERR_NULL
        assert call_linear(lib, fn, dW=FAKE + (1 << 30) + 64) == ce.CE_ERR_ALIAS   # on W
        assert call_linear(lib, fn, dH=FAKE + (5 << 30)) == ce.CE_ERR_ALIAS        # on dW
