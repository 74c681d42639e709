"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on a host copy of the same inputs, and compare with the
tolerances the tests state."""
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from softmax_cross_entropy_fwd_amd import inputs  # noqa: E402

# Loss tolerances: relative 1e-5 on the mean/sum for every storage type (the
# arithmetic is fp32 on exactly widened inputs; the stated bar for 16-bit
# inputs is 2e-3), and per row  rtol*|loss| + 4 ulp_fp32(max(|m|, |x_t|, 1)),
# the floor covering the cancellation in lse - x_t.
LOSS_RTOL = 1e-5
# Gradients: at most 2 units in the last place of the storage type (+-0 equal);
# fp32 storage: |d| <= 1e-5 |g| + 1e-7 c.
GRAD_ULP = 2


def say(*a):
    print(*a, flush=True)


def ulp32(x):
    x = np.abs(np.asarray(x, dtype=np.float64))
    x = np.maximum(x, 1.0)
    return np.spacing(x.astype(np.float32)).astype(np.float64)


def row_stats(xb, dtype):
    """fp64 row max of the stored values (for the per-row loss floor)."""
    w = widen(xb, dtype)
    with np.errstate(invalid="ignore"):
        return np.max(w, axis=1)


def widen(xb, dtype):
    if dtype == "f32":
        return xb.astype(np.float64)
    if dtype == "f16":
        return xb.view(np.float16).astype(np.float64)
    u = xb.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def check_row_losses(got, want, xb, targets, dtype, rtol=LOSS_RTOL, m=None, xt=None):
    """m, xt: the rows' max and target logit when given (for inputs too large
    to widen on the host); else taken from xb."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape
    nan_w = np.isnan(want)
    np.testing.assert_array_equal(np.isnan(got), nan_w)
    ok = ~nan_w
    if not ok.any():
        return 0.0
    if m is None:
        w = widen(xb[ok], dtype)
        m = np.max(w, axis=1)
        t = np.asarray(targets)[ok]
        xt = w[np.arange(w.shape[0]), t]
    else:
        m = np.asarray(m, dtype=np.float64)[ok]
        xt = np.asarray(xt, dtype=np.float64)[ok]
    inf = np.isinf(want[ok])
    np.testing.assert_array_equal(got[ok][inf], want[ok][inf])
    fin = ~inf
    floor = 4 * ulp32(np.maximum(np.abs(m), np.abs(xt)))
    err = np.abs(got[ok] - want[ok])
    bound = rtol * np.abs(want[ok]) + floor
    bad = fin & (err > bound)
    assert not bad.any(), "row loss mismatch at rows %s: got %s want %s" % (
        np.nonzero(ok)[0][bad][:5], got[ok][bad][:5], want[ok][bad][:5])
    return float(np.max(err[fin] / np.maximum(bound[fin], 1e-300))) if fin.any() else 0.0


def check_scalar(got, want, rtol=LOSS_RTOL):
    got, want = float(got), float(want)
    if math.isnan(want):
        assert math.isnan(got)
        return
    assert abs(got - want) <= rtol * abs(want) + 1e-30, (got, want)


def ordered16(bits):
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def check_grads(got_bits, want_bits, dtype, c, want64=None):
    """got/want: uint16 bit patterns (fp16/bf16) or float32 arrays."""
    if dtype == "f32":
        g = np.asarray(got_bits, dtype=np.float64)
        w = np.asarray(want64 if want64 is not None else want_bits, dtype=np.float64)
        assert not np.isnan(g).any()
        err = np.abs(g - w)
        bound = 1e-5 * np.abs(w) + 1e-7 * c
        bad = err > bound
        assert not bad.any(), "fp32 grad mismatch at %s: got %s want %s" % (
            np.argwhere(bad)[:5].tolist(), g[bad][:5], w[bad][:5])
        return
    gb = np.asarray(got_bits, dtype=np.uint16)
    wb = np.asarray(want_bits, dtype=np.uint16)
    nan_mask = 0x7C00 if dtype == "f16" else 0x7F80
    frac_mask = 0x03FF if dtype == "f16" else 0x007F
    gnan = ((gb & nan_mask) == nan_mask) & ((gb & frac_mask) != 0)
    wnan = ((wb & nan_mask) == nan_mask) & ((wb & frac_mask) != 0)
    np.testing.assert_array_equal(gnan, wnan)
    d = np.abs(ordered16(gb) - ordered16(wb))
    d[wnan] = 0
    bad = d > GRAD_ULP
    assert not bad.any(), "grad ulp mismatch (max %d) at %s: got %s want %s" % (
        d.max(), np.argwhere(bad)[:5].tolist(), [hex(v) for v in gb[bad][:5]],
        [hex(v) for v in wb[bad][:5]])
    return int(d.max())


def host_grad_bits(t):
    return inputs.host_bits(t)


# Row softmax: 16-bit outputs within GRAD_ULP units in the last place; fp32
# outputs |d| <= 1e-5 |p| + 2^-125 (the floor is where the hardware exp2 may
# flush a result below the normal range).
# Log-softmax: the per-row loss bound (it is minus a row loss),
# 1e-5 |y| + 4 ulp_fp32(max(|m|, |x|, 1)), plus one unit of the storage type
# for 16-bit outputs.  Row log-sum-exps: 1e-5 (lse - m) + 4 ulp_fp32(max(|m|,
# |lse|, 1)).


def check_softmax(got_bits, want_bits, want64, dtype):
    if dtype != "f32":
        return check_grads(got_bits, want_bits, dtype, 1.0)
    g = np.asarray(got_bits, dtype=np.float64)
    w = np.asarray(want64, dtype=np.float64)
    nan_w = np.isnan(w)
    np.testing.assert_array_equal(np.isnan(g), nan_w)
    err = np.abs(g - w)
    err[nan_w] = 0
    bound = 1e-5 * np.abs(np.where(nan_w, 0, w)) + 2.0 ** -125
    bad = err > bound
    assert not bad.any(), "fp32 softmax mismatch at %s: got %s want %s" % (
        np.argwhere(bad)[:5].tolist(), g[bad][:5], w[bad][:5])


def storage_ulp(values, dtype):
    v = np.abs(np.asarray(values, dtype=np.float64))
    v = np.where(np.isfinite(v), v, 0.0)
    if dtype == "f32":
        return np.spacing(v.astype(np.float32)).astype(np.float64)
    if dtype == "f16":
        return np.spacing(np.minimum(v, 65504).astype(np.float16)).astype(np.float64)
    # bf16: 8 significant bits
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_log_softmax(got_bits, want64, xb, dtype, m=None):
    """m: the rows' max ([rows, 1]) when xb holds only some of each row's
    columns; else taken from xb."""
    g = widen(np.asarray(got_bits), dtype)
    w = np.asarray(want64, dtype=np.float64)
    x = widen(np.asarray(xb), dtype)
    nan_w = np.isnan(w)
    np.testing.assert_array_equal(np.isnan(g), nan_w)
    inf_w = np.isinf(w)
    np.testing.assert_array_equal(g[inf_w], w[inf_w])
    fin = ~nan_w & ~inf_w
    if m is None:
        with np.errstate(invalid="ignore"):
            m = np.max(x, axis=1, keepdims=True)
    scale = np.maximum(np.abs(np.broadcast_to(m, x.shape)), np.abs(np.where(np.isfinite(x), x, 0)))
    bound = 1e-5 * np.abs(w) + 4 * ulp32(scale)
    if dtype != "f32":
        bound = bound + storage_ulp(w, dtype)
    with np.errstate(invalid="ignore"):
        err = np.abs(np.where(fin, g, 0) - np.where(fin, w, 0))
    bad = fin & (err > bound)
    assert not bad.any(), "log-softmax mismatch at %s: got %s want %s" % (
        np.argwhere(bad)[:5].tolist(), g[bad][:5], w[bad][:5])


def check_lse(got, want, xb, dtype, m=None):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    nan_w = np.isnan(want)
    np.testing.assert_array_equal(np.isnan(got), nan_w)
    ok = ~nan_w & np.isfinite(want)
    np.testing.assert_array_equal(got[~nan_w & ~ok], want[~nan_w & ~ok])
    if not ok.any():
        return
    if m is None:
        with np.errstate(invalid="ignore"):
            m = np.max(widen(np.asarray(xb)[ok], dtype), axis=1)
    else:
        m = np.asarray(m, dtype=np.float64)[ok]
    bound = 1e-5 * np.abs(want[ok] - m) + 4 * ulp32(np.maximum(np.abs(m), np.abs(want[ok])))
    err = np.abs(got[ok] - want[ok])
    bad = err > bound
    assert not bad.any(), "lse mismatch at rows %s: got %s want %s" % (
        np.nonzero(ok)[0][bad][:5], got[ok][bad][:5], want[ok][bad][:5])


def check_grads_on_device(got, want_bits, dtype):
    """Every element of got (a device tensor of fp16/bf16 gradients) within
    GRAD_ULP units in the last place of want_bits (the oracle's uint16 bit
    patterns, computed on the host), with NaN positions equal.  The oracle's
    values are copied to the device and compared there, so that rows of the
    full-size workloads are checked in seconds.  Returns the largest ulp
    distance."""
    import torch
    assert dtype in ("f16", "bf16")
    w = torch.from_numpy(np.ascontiguousarray(want_bits).view(np.int16)).to(got.device)
    g = got.detach().reshape(w.shape).view(torch.int16)
    gi, wi = g.to(torch.int32) & 0xFFFF, w.to(torch.int32) & 0xFFFF
    nan_mask = 0x7C00 if dtype == "f16" else 0x7F80
    frac_mask = 0x03FF if dtype == "f16" else 0x007F

    def is_nan(b):
        return ((b & nan_mask) == nan_mask) & ((b & frac_mask) != 0)

    def ordered(b):
        mag = b & 0x7FFF
        return torch.where((b & 0x8000) != 0, -mag, mag)

    gnan, wnan = is_nan(gi), is_nan(wi)
    assert torch.equal(gnan, wnan), "NaN positions differ"
    d = (ordered(gi) - ordered(wi)).abs()
    d = torch.where(wnan, torch.zeros_like(d), d)
    worst = int(d.max().item()) if d.numel() else 0
    if worst > GRAD_ULP:
        bad = torch.nonzero(d > GRAD_ULP)[:5].cpu().tolist()
        raise AssertionError("grad ulp mismatch (max %d) at %s" % (worst, bad))
    return worst
