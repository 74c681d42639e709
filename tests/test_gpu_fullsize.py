"""The five workloads at full size, in the launch configuration the bench times.

Reduced losses are checked against the oracle over every row; per-row losses
(reduction none) over every row; in-place gradients element by element on a
sample of rows (first, last and random ones), and on every row through a
property that holds at any size (each gradient row sums to zero up to the
storage rounding).
"""
import numpy as np
import pytest

from gpu_util import (check_grads, check_row_losses, check_scalar, host_grad_bits, oracle,
                      inputs, say)

pytestmark = pytest.mark.gpu

NAMES = ["tiny", "classifier", "lmhead", "stress", "skinny"]


@pytest.fixture(scope="module")
def ce():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    import softmax_cross_entropy_fwd_amd as ce
    ce.load_library()
    return ce


def sample_rows(M, n, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(M, size=min(n, M), replace=False).tolist())
    rows.update([0, M - 1])
    return sorted(rows)


@pytest.mark.parametrize("name", NAMES)
def test_full_size(ce, name):
    import torch
    c = inputs.CONFIGS[name]
    M, V, dtype = c["M"], c["V"], c["dtype"]
    say("full size", name, dtype, M, V)
    x, t = inputs.make_config(name, device="cuda:0")
    xb, tn = inputs.host_bits(x), t.cpu().numpy()
    say("plan fwd:", ce.ce_plan_describe(M, V, {"f32": 0, "f16": 1, "bf16": 2}[dtype], "mean"))
    per_row = oracle.loss_rows(xb, tn, dtype=dtype)
    say("oracle done")
    for red in c["reductions"]:
        got = ce.ce_fwd(x, t, red)
        torch.cuda.synchronize()
        if red == "none":
            check_row_losses(got.cpu().numpy(), per_row, xb, tn, dtype)
        else:
            check_scalar(got.item(), oracle.reduce(per_row, red))
    say("fwd ok")
    if "fwd_bwd" not in c["ops"]:
        return
    xg = x.clone()
    del x
    loss = ce.ce_fwd_bwd_inplace(xg, t, "mean")
    torch.cuda.synchronize()
    check_scalar(loss.item(), oracle.reduce(per_row, "mean"))
    cscale = 1.0 / M
    rows = sample_rows(M, 48, seed=M + V)
    # plus the rows whose target dominates (smallest losses) and rows whose
    # loss is ln V (all-equal rows, in the stress structure)
    order = np.argsort(per_row)
    special = set(order[:4].tolist())
    special.update(np.nonzero(np.abs(per_row - np.log(V)) < 1e-9)[0][:4].tolist())
    rows = sorted(set(rows) | special)
    for r in rows:
        want, want64 = oracle.grad_rows(xb, tn, dtype=dtype, c=cscale, row0=r, nrows=1,
                                        want64=True)
        check_grads(host_grad_bits(xg[r:r + 1]), want, dtype, cscale, want64)
    say("sampled grads ok", len(rows))
    # every row: sum_j g_ij = 0 up to rounding each element to the storage type
    eps = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}[dtype]
    tiny = {"f32": 0.0, "f16": 2.0 ** -25, "bf16": 0.0}[dtype]
    sums = torch.empty(M, dtype=torch.float64, device="cuda:0")
    for r0 in range(0, M, 1024):
        sums[r0:r0 + 1024] = xg[r0:r0 + 1024].double().sum(dim=1)
    bound = 2 * cscale * eps * 2 + V * tiny
    worst = sums.abs().max().item()
    say("max |row sum of grad| = %.3g (bound %.3g)" % (worst, bound))
    assert worst <= bound
