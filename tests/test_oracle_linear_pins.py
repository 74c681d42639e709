"""Pins for the oracle's linear + cross-entropy (logits H W^T of bf16 H and W,
then the loss, and the gradients of H and W): an independent library (torch
CPU float64 autograd), the identity-weight case that reduces to the plain
cross-entropy oracle (itself pinned), and central differences."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(20261203)


def bf16_bits(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def bf16_values(bits):
    return torch.from_numpy(np.asarray(bits).view(np.int16)).view(torch.bfloat16).double()


@pytest.mark.parametrize("reduction", ["none", "mean", "sum"])
def test_linear_ce_against_torch_float64(reduction):
    M, D, V = 13, 37, 301
    hb = bf16_bits(RNG.normal(size=(M, D)))
    wb = bf16_bits(RNG.normal(size=(V, D)) * 0.3)
    t = RNG.integers(0, V, size=M)
    loss, lse, G, dH, dW = oracle.linear_ce(hb, wb, t, reduction, grads=True)
    H = bf16_values(hb).requires_grad_(True)
    W = bf16_values(wb).requires_grad_(True)
    z = H @ W.T
    ref = F.cross_entropy(z, torch.from_numpy(t), reduction=reduction)
    (ref.sum() if reduction == "none" else ref).backward()
    if reduction == "none":
        np.testing.assert_allclose(loss, ref.detach().numpy(), rtol=1e-12)
    else:
        assert loss == pytest.approx(float(ref), rel=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(z.detach(), dim=1).numpy(), rtol=1e-12)
    np.testing.assert_allclose(dH, H.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(dW, W.grad.numpy(), rtol=1e-10, atol=1e-14)


def test_identity_weight_reduces_to_plain_cross_entropy():
    # W = I (D = V): the logits are H itself, so the loss, lse and the logits'
    # gradient are those of the plain oracle on H, and dH = G, dW = G^T H
    M, V = 9, 64
    hb = bf16_bits(RNG.normal(size=(M, V)) * 3)
    wb = bf16_bits(np.eye(V))
    t = RNG.integers(0, V, size=M)
    for red in ("none", "mean"):
        loss, lse, G, dH, dW = oracle.linear_ce(hb, wb, t, red, grads=True)
        per_row, lse_plain = oracle.loss_rows(hb, t, dtype="bf16", with_lse=True)
        if red == "none":
            np.testing.assert_array_equal(loss, per_row)
        else:
            assert loss == oracle.reduce(per_row, red)
        np.testing.assert_array_equal(lse, lse_plain)
        c = 1.0 / M if red == "mean" else 1.0
        _, g64 = oracle.grad_rows(hb, t, dtype="bf16", c=c, want64=True)
        np.testing.assert_array_equal(G, g64)
        np.testing.assert_array_equal(dH, g64)
        np.testing.assert_allclose(dW, g64.T @ bf16_values(hb).numpy(), rtol=1e-13, atol=1e-16)


def test_linear_ce_central_differences():
    # inputs on a 2^-4 grid below 4 and steps of 2^-6: every perturbed value
    # is a bf16 value, so the differences see exactly the function the oracle
    # evaluates
    M, D, V = 2, 3, 5
    h = np.round(RNG.uniform(-2, 2, size=(M, D)) * 16) / 16
    w = np.round(RNG.uniform(-2, 2, size=(V, D)) * 16) / 16
    t = RNG.integers(0, V, size=M)
    hb, wb = bf16_bits(h), bf16_bits(w)
    np.testing.assert_array_equal(bf16_values(hb).numpy(), h)
    _, _, _, dH, dW = oracle.linear_ce(hb, wb, t, "sum", grads=True)
    step = 2.0 ** -6

    def f(hh, ww):
        return oracle.linear_ce(bf16_bits(hh), bf16_bits(ww), t, "sum")[0]

    for i in range(M):
        for k in range(D):
            hp, hm = h.copy(), h.copy()
            hp[i, k] += step
            hm[i, k] -= step
            assert (f(hp, w) - f(hm, w)) / (2 * step) == pytest.approx(dH[i, k], rel=2e-3, abs=2e-4)
    for j in range(V):
        for k in range(D):
            wp, wm = w.copy(), w.copy()
            wp[j, k] += step
            wm[j, k] -= step
            assert (f(h, wp) - f(h, wm)) / (2 * step) == pytest.approx(dW[j, k], rel=2e-3, abs=2e-4)


def test_linear_ce_empty_batch():
    hb = np.zeros((0, 4), dtype=np.uint16)
    wb = bf16_bits(np.ones((3, 4)))
    t = np.zeros(0, dtype=np.int64)
    assert oracle.linear_ce(hb, wb, t, "sum")[0] == 0.0
    assert np.isnan(oracle.linear_ce(hb, wb, t, "mean")[0])
