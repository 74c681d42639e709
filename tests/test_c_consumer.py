"""The C ABI from a plain C99 program (tests/c_consumer/ce_consumer.c): no
Python or torch between the caller and the library.

CPU: the program compiles as C99 with -Wall -Wextra -Werror against the
headers and links against libce.so and the HIP runtime alone.
GPU: the program runs every entry point (forward none / mean, forward with
lse, backward from that lse, softmax, log-softmax, fused in-place forward +
backward, linear + cross-entropy) and four calls that must fail before any
launch, on inputs it draws itself and writes out; its outputs are checked
against the fp64 oracle with the tolerances of the other parity tests.
"""
import importlib.util
import os
import subprocess

import numpy as np
import pytest

from gpu_util import (check_grads, check_log_softmax, check_lse, check_row_losses, check_scalar,
                      check_softmax, oracle, say, widen)

HERE = os.path.dirname(os.path.abspath(__file__))
DCODE = {"f32": 0, "f16": 1, "bf16": 2}


def consumer_build():
    spec = importlib.util.spec_from_file_location(
        "ce_consumer_build", os.path.join(HERE, "c_consumer", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_consumer_compiles_as_c99(tmp_path):
    b = consumer_build()
    import softmax_cross_entropy_fwd_amd as ce
    if not os.path.exists(ce.LIB_PATH):
        from softmax_cross_entropy_fwd_amd import build
        build.build()
    out = str(tmp_path / "ce_consumer")
    r = subprocess.run(b.command(out), capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    nm = subprocess.run(["nm", "-u", out], capture_output=True, text=True).stdout
    # the program calls the library's entry points and nothing of torch
    for sym in ("ce_fwd", "ce_fwd_lse", "ce_bwd", "ce_softmax", "ce_fwd_bwd_inplace",
                "ce_linear_fwd", "ce_workspace_bytes", "ce_status_string"):
        assert " %s\n" % sym in nm or nm.endswith(" " + sym), sym
    assert "torch" not in nm and "c10" not in nm


def read(d, name, dtype, shape=None):
    a = np.fromfile(os.path.join(d, name), dtype=dtype)
    return a.reshape(shape) if shape is not None else a


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_consumer_matches_oracle(dtype, tmp_path):
    exe = consumer_build().EXE
    assert os.path.exists(exe), "the C consumer is not built (run __graft_entry__.build())"
    M, V = 300, 1003
    d = str(tmp_path)
    say("c consumer", dtype, M, V)
    r = subprocess.run([exe, d, str(DCODE[dtype]), str(M), str(V), "20261202"],
                       capture_output=True, text=True, timeout=120)
    say(r.stdout.strip())
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")

    st = np.float32 if dtype == "f32" else np.uint16
    xb = read(d, "x.bin", st, (M, V))
    tn = read(d, "t.bin", np.int64)
    loss_o, lse_o = oracle.loss_rows(xb, tn, dtype=dtype, with_lse=True)
    mean_o = oracle.reduce(loss_o, "mean")

    check_row_losses(read(d, "loss_none.bin", np.float32), loss_o, xb, tn, dtype)
    check_scalar(read(d, "loss_mean.bin", np.float32)[0], mean_o)
    check_scalar(read(d, "loss_sum.bin", np.float32)[0], oracle.reduce(loss_o, "sum"))
    check_lse(read(d, "lse.bin", np.float32), lse_o, xb, dtype)

    grad_o = oracle.grad_rows(xb, tn, dtype=dtype, c=1.0 / M, want64=dtype == "f32")
    g_bits, g64 = grad_o if dtype == "f32" else (grad_o, None)
    check_grads(read(d, "grad.bin", st, (M, V)), g_bits, dtype, 1.0 / M, g64)
    check_grads(read(d, "grad_fused.bin", st, (M, V)), g_bits, dtype, 1.0 / M, g64)
    check_scalar(read(d, "loss_fused.bin", np.float32)[0], mean_o)

    p_bits, p64 = oracle.softmax_rows(xb, dtype=dtype, want64=True)
    check_softmax(read(d, "softmax.bin", st, (M, V)), p_bits, p64, dtype)
    _, lp64 = oracle.softmax_rows(xb, dtype=dtype, log=True, want64=True)
    check_log_softmax(read(d, "log_softmax.bin", st, (M, V)), lp64, xb, dtype)

    # linear + cross-entropy: products of these bf16 values (multiples of
    # 1/16 in [-1, 1)) and their sums over D = 96 are exact in fp32, so the
    # logits carry no rounding and the cross-entropy bounds apply as they are
    h = read(d, "linear_h.bin", np.uint16, (64, 96))
    w = read(d, "linear_w.bin", np.uint16, (1000, 96))
    lt = read(d, "linear_t.bin", np.int64)
    per_row, llse = oracle.linear_ce(h, w, lt, "none")
    zmax = (widen(h, "bf16") @ widen(w, "bf16").T).max(axis=1)   # tolerance scale only
    check_lse(read(d, "linear_lse.bin", np.float32), llse, None, "f32", m=zmax)
    check_scalar(read(d, "linear_loss.bin", np.float32)[0], oracle.reduce(per_row, "mean"))
    say("ok")
