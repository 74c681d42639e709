"""The C ABI without a GPU: the library loads, exports every symbol include/ce.h
declares, and rejects bad arguments with the documented status before any HIP
call (argument checks come first in every entry point)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ce.h")


@pytest.fixture(scope="module")
def lib():
    import softmax_cross_entropy_fwd_amd as ce
    if not os.path.exists(ce.LIB_PATH):
        from softmax_cross_entropy_fwd_amd import build
        build.build()
    return ce.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ce_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("ce_fwd", "ce_fwd_bwd_inplace", "ce_workspace_bytes", "ce_status_string",
              "ce_plan_describe"):
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
    for code in range(-8, 1):
        s = lib.ce_status_string(code).decode()
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 9
    assert lib.ce_status_string(-99).decode() == "unknown status"
    assert ce.ce_status_string(ce.CE_ERR_ALIAS).startswith("in-place")


def test_binding_rejects_host_tensors():
    import torch
    import softmax_cross_entropy_fwd_amd as ce
    x = torch.zeros(2, 3)
    t = torch.zeros(2, dtype=torch.int64)
    with pytest.raises(ValueError):
        ce.ce_fwd(x, t)
