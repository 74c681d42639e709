"""GPU parity at the largest sizes the entry points take.

- One row of CE_MAX_V = 2^31 - 1 logits (fp32: 8 GiB, bf16: 4 GiB), the
  longest row the C ABI accepts, split over workgroups: the forward with its
  log-sum-exp, the backward from that log-sum-exp out of place, the fused
  backward in place, and the row softmax and log-softmax, against the fp64
  oracle.  Loss and lse to the bounds of the other parity tests; the
  elementwise outputs on a sample of columns (both ends of the row, both
  sides of every multiple of 2^22 elements, the slice boundaries among them,
  the target and 2^21 random columns), the oracle's values there taken from
  its fp64 row log-sum-exp.
- A batch of more than 2^31 elements with a ragged row length (16500 x
  131075 bf16: rows at every 2-byte phase of a 16-byte vector), so that row
  addresses pass the 32-bit element range: every row's loss and the mean,
  and the split and the fused backward element by element on the first and
  last rows, the rows at the 2^31-element boundary and random rows.

Row maxima and target logits for the loss tolerance are taken on the device
(a max and a gather are exact), since widening these inputs on the host would
take tens of GB.
"""
import numpy as np
import pytest

from gpu_util import (check_grads, check_log_softmax, check_lse, check_row_losses, check_scalar,
                      check_softmax, oracle, inputs, say)

pytestmark = pytest.mark.gpu

DCODE = {"f32": 0, "f16": 1, "bf16": 2}
CE_MAX_V = 2 ** 31 - 1


@pytest.fixture(scope="module")
def ce():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    import softmax_cross_entropy_fwd_amd as ce
    ce.load_library()
    return ce


def sample_cols(V, t, seed):
    rng = np.random.default_rng(seed)
    edge = np.arange(65536)
    parts = [edge, V - 1 - edge, rng.integers(0, V, size=1 << 21), np.array([t])]
    step = 1 << 22
    for b in range(step, V, step):
        parts.append(np.arange(b - 64, min(V, b + 64)))
    return np.unique(np.concatenate(parts)).astype(np.int64)


def longest_row(ce, dtype, seed):
    import torch
    dev = torch.device("cuda:0")
    x, t = inputs.make(dtype, 1, CE_MAX_V, sigma=2.0, seed=seed, device=dev)
    tn = t.cpu().numpy()
    m = np.array([float(x.max())])
    xt = np.array([float(x[0, int(tn[0])])])
    plan = ce.ce_plan_describe(1, CE_MAX_V, DCODE[dtype], "none")
    say("plan", plan)
    assert plan.startswith("split:"), plan
    return x, t, tn, m, xt


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_longest_row(ce, dtype):
    import torch
    say("longest row", dtype, CE_MAX_V)
    x, t, tn, m, xt = longest_row(ce, dtype, seed=2024)
    xb = inputs.host_bits(x)
    loss_o, lse_o = oracle.loss_rows(xb, tn, dtype=dtype, with_lse=True)
    say("oracle loss", loss_o[0], "lse", lse_o[0])
    cols = sample_cols(CE_MAX_V, int(tn[0]), seed=7)
    grad_o = oracle.at_elements(xb, lse_o, 0, cols, "grad", dtype=dtype, targets=tn)
    p_o, p64_o = oracle.at_elements(xb, lse_o, 0, cols, "softmax", dtype=dtype, want64=True)
    _, lp64_o = oracle.at_elements(xb, lse_o, 0, cols, "log_softmax", dtype=dtype, want64=True)
    xs = xb[:, cols]
    del xb
    say(cols.size, "sampled columns")
    cols_d = torch.from_numpy(cols).to(x.device)

    say("ce_fwd_lse")
    loss, lse = ce.ce_fwd_lse(x, t, "none")
    torch.cuda.synchronize()
    check_row_losses(loss.cpu().numpy(), loss_o, None, tn, dtype, m=m, xt=xt)
    check_lse(lse.cpu().numpy(), lse_o, None, dtype, m=m)

    say("ce_bwd")
    y = ce.ce_bwd(x, t, lse, "mean")
    torch.cuda.synchronize()
    check_grads(inputs.host_bits(y[0, cols_d]), grad_o, dtype, 1.0)

    say("ce_softmax")
    lse2 = torch.empty(1, dtype=torch.float32, device=x.device)
    ce.ce_softmax(x, out=y, lse=lse2)
    torch.cuda.synchronize()
    check_lse(lse2.cpu().numpy(), lse_o, None, dtype, m=m)
    check_softmax(inputs.host_bits(y[0, cols_d])[None], p_o[None], p64_o[None], dtype)
    say("ce_softmax log")
    ce.ce_softmax(x, log_softmax=True, out=y)
    torch.cuda.synchronize()
    check_log_softmax(inputs.host_bits(y[0, cols_d])[None], lp64_o[None], xs, dtype,
                      m=m[:, None])
    del y

    say("ce_fwd_bwd_inplace")
    mean = ce.ce_fwd_bwd_inplace(x, t, "mean")
    torch.cuda.synchronize()
    check_scalar(mean.item(), loss_o[0])
    check_grads(inputs.host_bits(x[0, cols_d]), grad_o, dtype, 1.0)
    say("ok")


def test_batch_beyond_2_31_elements(ce):
    import torch
    M, V, dtype = 16500, 131075, "bf16"
    assert M * V > 2 ** 31
    dev = torch.device("cuda:0")
    say("batch", dtype, M, V, "elements", M * V)
    x, t = inputs.make(dtype, M, V, sigma=2.0, seed=2025, device=dev)
    xb, tn = inputs.host_bits(x), t.cpu().numpy()
    m = x.max(dim=1).values.float().cpu().numpy()
    xt = x.gather(1, t[:, None])[:, 0].float().cpu().numpy()
    say("plan", ce.ce_plan_describe(M, V, DCODE[dtype], "mean"))
    loss_o = oracle.loss_rows(xb, tn, dtype=dtype)
    say("oracle losses done")

    got = ce.ce_fwd(x, t, "none")
    torch.cuda.synchronize()
    check_row_losses(got.cpu().numpy(), loss_o, None, tn, dtype, m=m, xt=xt)
    check_scalar(ce.ce_fwd(x, t, "mean").item(), oracle.reduce(loss_o, "mean"))
    say("forward ok")

    boundary = (2 ** 31) // V                     # the row holding element 2^31
    rng = np.random.default_rng(11)
    rows = sorted({0, 1, boundary - 1, boundary, boundary + 1, M - 1}
                  | set(rng.choice(M, size=6, replace=False).tolist()))
    want = {r: oracle.grad_rows(xb, tn, dtype=dtype, c=1.0 / M, row0=r, nrows=1)[0]
            for r in rows}
    del xb

    say("ce_fwd_lse + ce_bwd")
    mean, lse = ce.ce_fwd_lse(x, t, "mean")
    y = ce.ce_bwd(x, t, lse, "mean")
    torch.cuda.synchronize()
    check_scalar(mean.item(), oracle.reduce(loss_o, "mean"))
    for r in rows:
        check_grads(inputs.host_bits(y[r]), want[r], dtype, 1.0 / M)
    del y

    say("ce_fwd_bwd_inplace")
    mean = ce.ce_fwd_bwd_inplace(x, t, "mean")
    torch.cuda.synchronize()
    check_scalar(mean.item(), oracle.reduce(loss_o, "mean"))
    for r in rows:
        check_grads(inputs.host_bits(x[r]), want[r], dtype, 1.0 / M)
    say("ok")


@pytest.mark.parametrize("dtype,V", [("f32", 17), ("f16", 9)])
def test_short_rows_beyond_2_31_elements(ce, dtype, V):
    # many short ragged rows held in the registers of a few lanes each (the
    # rows kernel), past the 32-bit element range
    import torch
    M = (2 ** 31) // V + 4099
    assert M * V > 2 ** 31
    dev = torch.device("cuda:0")
    say("short rows", dtype, M, V, "elements", M * V)
    x, t = inputs.make(dtype, M, V, sigma=3.0, seed=2026, device=dev, chunk_rows=1 << 24)
    xb, tn = inputs.host_bits(x), t.cpu().numpy()
    m = x.max(dim=1).values.float().cpu().numpy()
    xt = x.gather(1, t[:, None])[:, 0].float().cpu().numpy()
    say("plan", ce.ce_plan_describe(M, V, DCODE[dtype], "none"))
    loss_o = oracle.loss_rows(xb, tn, dtype=dtype)
    say("oracle losses done")

    got = ce.ce_fwd(x, t, "none")
    torch.cuda.synchronize()
    check_row_losses(got.cpu().numpy(), loss_o, None, tn, dtype, m=m, xt=xt)
    del got
    check_scalar(ce.ce_fwd(x, t, "sum").item(), oracle.reduce(loss_o, "sum"))
    say("forward ok")

    boundary = (2 ** 31) // V
    rng = np.random.default_rng(12)
    rows = sorted({0, 1, boundary - 1, boundary, boundary + 1, M - 2, M - 1}
                  | set(rng.choice(M, size=64, replace=False).tolist()))
    want = {r: oracle.grad_rows(xb, tn, dtype=dtype, c=1.0 / M, row0=r, nrows=1)[0]
            for r in rows}
    del xb
    mean = ce.ce_fwd_bwd_inplace(x, t, "mean")
    torch.cuda.synchronize()
    check_scalar(mean.item(), oracle.reduce(loss_o, "mean"))
    for r in rows:
        check_grads(inputs.host_bits(x[r]), want[r], dtype, 1.0 / M)
    say("ok")
