"""The five workloads at full size, in the launch configuration the bench times.

Reduced losses are checked against the oracle over every row; per-row losses
(reduction none) over every row; in-place gradients element by element on
every row (the oracle runs over row chunks on the host, the ulp comparison of
its values with the kernel's runs on the device), and through a property that
holds at any size (each gradient row sums to zero up to the storage rounding).
"""
import numpy as np
import pytest

from gpu_util import (check_grads_on_device, check_row_losses, check_scalar, oracle, inputs,
                      say)

pytestmark = pytest.mark.gpu

NAMES = ["tiny", "classifier", "lmhead", "stress", "skinny"]


@pytest.fixture(scope="module")
def ce():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    import softmax_cross_entropy_fwd_amd as ce
    ce.load_library()
    return ce


# the fused backward's plan at full size (the LM head: the exact 16-wave
# register tile, whose every element is compared with the oracle below)
FWD_BWD_PLAN = {"lmhead": "wg:16:16 exact", "stress": "wg2:8:13"}


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
    plan = ce.ce_plan_describe(M, V, {"f32": 0, "f16": 1, "bf16": 2}[dtype], "mean",
                               fwd_bwd=True)
    say("plan fwd_bwd:", plan)
    assert plan.startswith(FWD_BWD_PLAN[name] + " "), plan
    xg = x.clone()
    del x
    loss = ce.ce_fwd_bwd_inplace(xg, t, "mean")
    torch.cuda.synchronize()
    check_scalar(loss.item(), oracle.reduce(per_row, "mean"))
    cscale = 1.0 / M
    # every row, element by element, in chunks of rows
    chunk = max(1, (1 << 27) // V)
    worst = 0
    for r0 in range(0, M, chunk):
        n = min(chunk, M - r0)
        want = oracle.grad_rows(xb, tn, dtype=dtype, c=cscale, row0=r0, nrows=n)
        worst = max(worst, check_grads_on_device(xg[r0:r0 + n], want, dtype))
    say("grads ok on all %d rows, max %d ulp" % (M, worst))
    # the dominant-target and all-equal rows are among them (stress structure)
    special = int(np.sum(per_row < 1e-6)) + int(np.sum(np.abs(per_row - np.log(V)) < 1e-9))
    say("rows with a dominant target or all-equal values: %d" % special)
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
