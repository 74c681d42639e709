"""GPU parity of split rows (several workgroups per row, for few long rows):
every entry point against the fp64 oracle, with misaligned bases, the stress
structure (dominant targets, -inf entries, all-equal rows), out-of-range
targets, in place and out of place, and the split and one-row paths against
each other.  Tolerances are those of the other parity tests (gpu_util)."""
import numpy as np
import pytest

from gpu_util import (check_grads, check_row_losses, check_scalar, host_grad_bits, oracle,
                      inputs, say)
from test_gpu_epilogues import bwd_case, fwd_lse_case, softmax_case
from test_gpu_parity import DTYPES, run_and_check

pytestmark = pytest.mark.gpu

DCODE = {"f32": 0, "f16": 1, "bf16": 2}
# (dtype, V): rows of 256 KiB and more (split by default for M <= 128),
# aligned and ragged
LONG = [("f32", 65536), ("f32", 100003), ("f16", 131075), ("bf16", 131072), ("bf16", 200003)]


@pytest.fixture(scope="module")
def ce():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    import softmax_cross_entropy_fwd_amd as ce
    ce.load_library()
    return ce


def test_split_is_planned(ce):
    for dtype, V in LONG:
        for M in (1, 5, 64, 128):
            plan = ce.ce_plan_describe(M, V, DCODE[dtype], "mean")
            assert plan.startswith("split:"), (dtype, V, M, plan)
        assert not ce.ce_plan_describe(129, V, DCODE[dtype], "mean").startswith("split:")
    assert not ce.ce_plan_describe(8, 32768, 2, "mean").startswith("split:")   # 64 KiB rows


@pytest.mark.parametrize("dtype,V", LONG)
def test_split_forward_and_fused_backward(ce, dtype, V):
    for M in (1, 3, 40):
        for red in ("none", "mean", "sum"):
            run_and_check(ce, dtype, M, V, 3.0, seed=V + M, reduction=red, offset=M % 3)
        run_and_check(ce, dtype, M, V, 3.0, seed=V + M + 1, reduction="mean", op="fwd_bwd",
                      offset=(M + 1) % 3)
        run_and_check(ce, dtype, M, V, 3.0, seed=V + M + 2, reduction="none", op="fwd_bwd")
        fwd_lse_case(ce, dtype, M, V, 3.0, seed=V + M + 3, reduction="sum", offset=1)


@pytest.mark.parametrize("dtype,V", LONG)
def test_split_backward_from_lse(ce, dtype, V):
    for M in (1, 7, 33):
        bwd_case(ce, dtype, M, V, 3.0, seed=V + M + 4, reduction="none", offset=M % 2)
        bwd_case(ce, dtype, M, V, 3.0, seed=V + M + 5, reduction="mean", inplace=True,
                 lse_from="library")
        bwd_case(ce, dtype, M, V, 3.0, seed=V + M + 6, reduction="sum", upstream=False)


@pytest.mark.parametrize("dtype,V", LONG)
def test_split_softmax(ce, dtype, V):
    for M in (1, 9):
        for log in (False, True):
            softmax_case(ce, dtype, M, V, 3.0, seed=V + M + 7, log=log, offset=M % 3)
            softmax_case(ce, dtype, M, V, 3.0, seed=V + M + 8, log=log, inplace=True,
                         want_lse=False)


def test_split_stress_rows(ce, tuning):
    # the stress structure at a few rows: dominant targets (the sum of the
    # other terms comes from the slices), -inf entries, all-equal rows
    tuning.setenv("CE_FORCE_SPLIT", "4")
    for dtype in DTYPES:
        for M in (100, 300):
            run_and_check(ce, dtype, M, 50257, 8.0, seed=104, structure="stress",
                          reduction="none", offset=1)
            run_and_check(ce, dtype, M, 50257, 8.0, seed=104, structure="stress",
                          reduction="mean", op="fwd_bwd", offset=1)
            bwd_case(ce, dtype, M, 50257, 8.0, seed=104, structure="stress", reduction="mean",
                     lse_from="library", offset=1)
            bwd_case(ce, dtype, M, 50257, 8.0, seed=104, structure="stress", reduction="none",
                     inplace=True, offset=1)
            softmax_case(ce, dtype, M, 50257, 8.0, seed=104, structure="stress", log=True,
                         offset=1)


def test_split_dominant_targets_and_bad_targets(ce, tuning):
    import torch
    tuning.setenv("CE_FORCE_SPLIT", "3")
    for dtype in DTYPES:
        V = 40000
        M = 6
        bwd_case(ce, dtype, M, V, 2.0, seed=11, reduction="none",
                 targets=[0, -1, V, 7, 1 << 40, V - 1])
        run_and_check(ce, dtype, M, V, 2.0, seed=11, reduction="none", op="fwd_bwd",
                      targets=[0, -1, V, 7, 1 << 40, V - 1])
        for gap in (3.0, 12.0):
            x, t = inputs.make(dtype, 8, V, 1.0, seed=int(gap) + V)
            xf = x.float()
            xf[torch.arange(8), t] = xf.max(dim=1).values + gap
            xd = xf.to(x.dtype)
            xb, tn = inputs.host_bits(xd), t.numpy()
            per_row, lse64 = oracle.loss_rows(xb, tn, dtype=dtype, with_lse=True)
            want, want64 = oracle.grad_rows(xb, tn, dtype=dtype, c=1.0, want64=True)
            xg, tg = xd.to("cuda:0"), t.to("cuda:0")
            loss = ce.ce_fwd(xg, tg, "none")
            g = ce.ce_bwd(xg, tg, torch.from_numpy(lse64.astype(np.float32)).to("cuda:0"),
                          "sum")
            y = xg.clone()
            ce.ce_fwd_bwd_inplace(y, tg, "sum")
            torch.cuda.synchronize()
            np.testing.assert_allclose(loss.cpu().numpy(), per_row, rtol=1e-4)
            check_grads(host_grad_bits(g), want, dtype, 1.0, want64)
            check_grads(host_grad_bits(y), want, dtype, 1.0, want64)


def test_split_matches_one_row_path(ce, tuning):
    # The split and the one-row paths agree with each other, and both with the
    # oracle element by element.  For bf16 rows of 131072 the one-row path is
    # the exact 16-wave register tile the full-size LM head runs.
    import torch
    for dtype, V in LONG:
        x, t = inputs.make(dtype, 24, V, 2.0, seed=V + 99, device="cuda:0")
        xb, tn = inputs.host_bits(x), t.cpu().numpy()
        a = ce.ce_fwd(x, t, "none")
        ga = x.clone()
        la = ce.ce_fwd_bwd_inplace(ga, t, "mean")
        tuning.setenv("CE_FORCE_SPLIT", "0")
        plan = ce.ce_plan_describe(24, V, DCODE[dtype], "mean", fwd_bwd=True)
        say("one-row plan", dtype, V, plan)
        if (dtype, V) == ("bf16", 131072):
            assert plan.startswith("wg:16:16 exact "), plan
        b = ce.ce_fwd(x, t, "none")
        gb = x.clone()
        lb = ce.ce_fwd_bwd_inplace(gb, t, "mean")
        tuning.delenv("CE_FORCE_SPLIT")
        torch.cuda.synchronize()
        np.testing.assert_allclose(a.cpu().numpy(), b.cpu().numpy(), rtol=2e-6, atol=2e-6)
        check_scalar(la.item(), lb.item(), rtol=2e-6)
        check_grads(host_grad_bits(ga), host_grad_bits(gb), dtype, 1.0 / 24,
                    inputs.host_bits(gb).astype(np.float64) if dtype == "f32" else None)
        # both against the oracle
        per_row = oracle.loss_rows(xb, tn, dtype=dtype)
        check_row_losses(b.cpu().numpy(), per_row, xb, tn, dtype)
        check_row_losses(a.cpu().numpy(), per_row, xb, tn, dtype)
        check_scalar(lb.item(), oracle.reduce(per_row, "mean"))
        want, want64 = oracle.grad_rows(xb, tn, dtype=dtype, c=1.0 / 24, want64=True)
        check_grads(host_grad_bits(gb), want, dtype, 1.0 / 24, want64)
        check_grads(host_grad_bits(ga), want, dtype, 1.0 / 24, want64)


@pytest.mark.parametrize("M", [129, 160])
def test_lmhead_register_tile_every_element(ce, M):
    # More than 128 rows of 131072 bf16: the default plan is the exact 16-wave
    # register tile (no split), compared with the oracle on every element.
    plan = ce.ce_plan_describe(M, 131072, DCODE["bf16"], "mean", fwd_bwd=True)
    say("plan", M, plan)
    assert plan.startswith("wg:16:16 exact "), plan
    run_and_check(ce, "bf16", M, 131072, 2.0, seed=103 + M, reduction="mean", op="fwd_bwd")
    run_and_check(ce, "bf16", M, 131072, 2.0, seed=104 + M, reduction="none", op="fwd_bwd")
    run_and_check(ce, "bf16", M, 131072, 8.0, seed=105 + M, structure="stress",
                  reduction="sum", op="fwd_bwd")


def test_split_forced_slice_counts(ce, tuning):
    # every slice count the plan can take, including one slice per chunk
    for S in (2, 3, 16, 64):
        tuning.setenv("CE_FORCE_SPLIT", str(S))
        for dtype, V in (("bf16", 131072), ("f32", 70001)):
            say("forced split", S, dtype, V)
            run_and_check(ce, dtype, 5, V, 3.0, seed=S + V, reduction="mean", offset=1)
            run_and_check(ce, dtype, 5, V, 3.0, seed=S + V, reduction="sum", op="fwd_bwd")
            bwd_case(ce, dtype, 5, V, 3.0, seed=S + V, reduction="none", offset=1)
            softmax_case(ce, dtype, 5, V, 3.0, seed=S + V, log=False)
