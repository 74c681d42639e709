"""GPU parity of linear + cross-entropy (logits hidden @ weight.T: this
library's matrix-core kernels when D % 8 == 0 and the operands sit on 16-byte
boundaries, else library GEMMs over vocabulary chunks, with this library's row
kernels) against the fp64 oracle.

Tolerances, derived from the arithmetic: the GEMMs add exact bf16 products in
fp32, so each logit is within g_D = D 2^-24 times the sum of its products'
magnitudes, and a row's loss within twice the largest such bound over the row
(lse and the target logit each move by at most that), on top of the
cross-entropy bound of the other tests (1e-5 relative + 4 fp32 ulps).  The
logits' gradient is rounded to bf16 (2^-9 relative) before the gradient
GEMMs, so dH and dW are held to (2^-8 + 2 e + n 2^-24) times |G| |W| and
|G|^T |H| (e the row's logit bound, n the GEMM's inner size)."""
import math

import numpy as np
import pytest

from gpu_util import oracle, inputs, say, ulp32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ce():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    import softmax_cross_entropy_fwd_amd as ce
    ce.load_library()
    return ce


def bits(t):
    return inputs.host_bits(t)


def values(t):
    return t.double().cpu().numpy()


def logit_bounds(h, w):
    """Per row: D 2^-24 max_j sum_k |h_ik w_jk|, and the logits' magnitudes."""
    D = h.shape[1]
    a = np.abs(h) @ np.abs(w).T
    return D * 2.0 ** -24 * a.max(axis=1)


def loss_bounds(want, lse_want, e):
    """Per-row loss bound: the cross-entropy bound plus twice the logit bound."""
    return 1e-5 * np.abs(want) + 4 * ulp32(np.abs(lse_want)) + 2 * e


def check_lse(lse_got, lse_want, e):
    lerr = np.abs(np.asarray(lse_got, np.float64) - lse_want)
    lbound = 1e-5 * np.abs(lse_want) + 4 * ulp32(np.abs(lse_want)) + e
    assert np.all(lerr <= lbound), (np.nonzero(lerr > lbound)[0][:5],)


def check_losses(got, want, lse_got, lse_want, e):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    nan = np.isnan(want)
    np.testing.assert_array_equal(np.isnan(got), nan)
    ok = ~nan
    bound = loss_bounds(want, lse_want, e)
    err = np.abs(got - want)
    assert np.all(err[ok] <= bound[ok]), (np.nonzero(ok & (err > bound))[0][:5], got[:5], want[:5])
    check_lse(lse_got, lse_want, e)


def check_grad(got, want, bound):
    got = np.asarray(got, np.float64)
    err = np.abs(got - want)
    bad = err > bound
    assert not bad.any(), "grad mismatch at %s: got %s want %s bound %s" % (
        np.argwhere(bad)[:5].tolist(), got[bad][:5], want[bad][:5], bound[bad][:5])


def run_case(ce, M, D, V, chunk, reduction, seed, sigma=2.0, bwd=True, h=None, w=None, t=None):
    import torch
    say("linear", M, D, V, chunk, reduction, seed, bwd)
    if h is None:
        h, w, t = inputs.make_linear(M, D, V, sigma, seed)
    hg, wg, tg = h.to("cuda:0"), w.to("cuda:0"), t.to("cuda:0")
    if bwd:
        loss, lse, dh, dw = ce.ce_linear_fwd_bwd(hg, wg, tg, reduction, chunk=chunk)
    else:
        loss, lse = ce.ce_linear_fwd(hg, wg, tg, reduction, chunk=chunk)
    torch.cuda.synchronize()
    want = oracle.linear_ce(bits(h), bits(w), t.numpy(), reduction, grads=bwd)
    hv, wv = values(h), values(w)
    e = logit_bounds(hv, wv)
    if reduction == "none":
        check_losses(loss.cpu().numpy(), want[0], lse.cpu().numpy(), want[1], e)
    else:
        per_row = oracle.linear_ce(bits(h), bits(w), t.numpy(), "none")[0]
        check_lse(lse.cpu().numpy(), want[1], e)
        w_loss = want[0]
        # the rows' bounds add up; the result is rounded to fp32 once
        tol = loss_bounds(per_row, want[1], e).sum() / (M if reduction == "mean" else 1)
        tol += 2.0 ** -24 * abs(w_loss)
        if math.isnan(w_loss):
            assert math.isnan(loss.item())
        else:
            assert abs(loss.item() - w_loss) <= tol, (loss.item(), w_loss, tol)
    if bwd:
        G = want[2]
        eb = 2 * e.max() if M else 0.0
        bh = (2.0 ** -8 + eb + V * 2.0 ** -24) * (np.abs(G) @ np.abs(wv)) + 1e-30
        bw = (2.0 ** -8 + eb + M * 2.0 ** -24) * (np.abs(G).T @ np.abs(hv)) + 1e-30
        check_grad(dh.cpu().numpy(), want[3], bh)
        check_grad(dw.cpu().numpy(), want[4], bw)
    return loss


@pytest.mark.parametrize("chunk", [256, 1024, 0])
def test_linear_small(ce, chunk):
    for red in ("none", "mean", "sum"):
        run_case(ce, 37, 96, 3001, chunk, red, seed=chunk + 1)
    run_case(ce, 37, 96, 3001, chunk, "mean", seed=chunk + 2, bwd=False)


def test_linear_ragged_and_larger(ce):
    # odd sizes: M not a multiple of 4, D odd, V not a multiple of the chunk
    run_case(ce, 61, 257, 50257, 4096, "mean", seed=3)
    run_case(ce, 5, 513, 20011, 0, "none", seed=4, sigma=6.0)
    run_case(ce, 1, 64, 300, 0, "sum", seed=5)


def test_linear_matrix_core_mid_size(ce):
    # the matrix-core path: a mid size (M, D and V several tiles and K steps)
    run_case(ce, 256, 1024, 32768, 0, "mean", seed=21)
    run_case(ce, 256, 1024, 32768, 8192, "none", seed=22, bwd=False)


def test_linear_matrix_core_ragged_tiles(ce):
    # tokens and vocabulary rows past a 256 tile, D past a K step of 64, a
    # single K chunk, tiles fewer than the XCDs
    run_case(ce, 300, 200, 5003, 1024, "none", seed=23)
    run_case(ce, 257, 8, 257, 0, "sum", seed=24)
    run_case(ce, 3, 72, 77, 0, "mean", seed=25)


def test_linear_both_gemm_paths(ce, tuning):
    # the same inputs through the matrix-core kernels and the library GEMMs:
    # both within the oracle bounds, and within twice them of each other
    h, w, t = inputs.make_linear(96, 512, 9000, 2.0, 26)
    a = run_case(ce, 96, 512, 9000, 2048, "none", 0, h=h, w=w, t=t)
    tuning.setenv("CE_LINEAR_GEMM", "library")
    b = run_case(ce, 96, 512, 9000, 2048, "none", 0, h=h, w=w, t=t)
    tuning.delenv("CE_LINEAR_GEMM")
    e = logit_bounds(values(h), values(w))
    bound = 2 * loss_bounds(b.cpu().numpy().astype(np.float64), 0.0, e)
    assert np.all(np.abs(a.cpu().numpy() - b.cpu().numpy()) <= bound + 1e-6)


def test_linear_dominant_and_out_of_range_targets(ce):
    import torch
    # W = I (D = V): the logits are the hidden states; rows with a target
    # 20 or 40 above the rest exercise the dominant-target form
    V = 320
    M = 8
    w = torch.eye(V, dtype=torch.float32).to(torch.bfloat16)
    g = torch.Generator().manual_seed(7)
    t = torch.randint(0, V, (M,), generator=g)
    h = torch.randn((M, V), generator=g) * 0.5
    h[torch.arange(M), t] = torch.tensor([20.0, 40.0, 3.0, 20.0, 40.0, 0.0, 9.0, 20.0])
    h = h.to(torch.bfloat16)
    for chunk in (256, 0):
        run_case(ce, M, V, V, chunk, "none", 0, h=h, w=w, t=t)
    t2 = t.clone()
    t2[1] = -1
    t2[5] = V
    loss = run_case(ce, M, V, V, 0, "none", 0, h=h, w=w, t=t2)
    assert math.isnan(loss[1].item()) and math.isnan(loss[5].item())


def test_linear_empty_batch(ce):
    import torch
    h = torch.empty(0, 16, dtype=torch.bfloat16, device="cuda:0")
    w = torch.ones(40, 16, dtype=torch.bfloat16, device="cuda:0")
    t = torch.empty(0, dtype=torch.int64, device="cuda:0")
    loss, lse, dh, dw = ce.ce_linear_fwd_bwd(h, w, t, "mean")
    torch.cuda.synchronize()
    assert math.isnan(loss.item()) and dh.numel() == 0
    assert torch.count_nonzero(dw).item() == 0
    assert ce.ce_linear_fwd(h, w, t, "sum")[0].item() == 0.0


def test_linear_deterministic(ce):
    import torch
    h, w, t = inputs.make_linear(64, 256, 5000, 2.0, 9, device="cuda:0")
    a = ce.ce_linear_fwd_bwd(h, w, t, "mean", chunk=1024)
    b = ce.ce_linear_fwd_bwd(h, w, t, "mean", chunk=1024)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))


def test_linear_full_size_sampled(ce):
    """The bench's workload at full size: every row's loss is finite and the
    mean matches the per-row losses; sampled rows' loss, lse and dH against
    the oracle; dW through a property that holds at any size (each logits'
    gradient row sums to zero, so each column of dW sums to at most the bf16
    rounding of G times |H|)."""
    import torch
    c = inputs.LINEAR_CONFIGS["lmhead_linear"]
    M, D, V = c["M"], c["D"], c["V"]
    h, w, t = inputs.make_linear(M, D, V, c["sigma"], c["seed"], device="cuda:0")
    loss_rows, lse_rows = ce.ce_linear_fwd(h, w, t, "none")
    loss, lse, dh, dw = ce.ce_linear_fwd_bwd(h, w, t, "mean")
    torch.cuda.synchronize()
    per_row = loss_rows.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(per_row))
    assert loss.item() == pytest.approx(per_row.mean(), rel=1e-5)
    rng = np.random.default_rng(11)
    rows = sorted(set(rng.choice(M, size=6, replace=False).tolist()) | {0, M - 1})
    hb, wb = bits(h[rows].cpu()), bits(w.cpu())
    tr = t.cpu().numpy()[rows]
    say("oracle on rows", rows)
    want = oracle.linear_ce(hb, wb, tr, "none", grads=True)
    hv, wv = values(h[rows]), values(w)
    e = logit_bounds(hv, wv)
    check_losses(per_row[rows], want[0], lse_rows.cpu().numpy()[rows], want[1], e)
    # the sampled rows' dH: G_i (scaled 1/M for the mean) times W
    G = want[2] / M
    bh = (2.0 ** -8 + 2 * e.max() + V * 2.0 ** -24) * (np.abs(G) @ np.abs(wv)) + 1e-30
    check_grad(dh.cpu().numpy()[rows], want[3] / M, bh)
    # sum_j dW_jk = sum_i h_ik sum_j G~_ij, and |sum_j G~_ij| <= (2^-9 + 2e +
    # 1e-6) * 2c for the computed, bf16-rounded G~ (sum_j |G_ij| <= 2c); the
    # fp32 GEMM adds at most M 2^-24 * 2c sum_i |h_ik|
    col = dw.double().sum(dim=0).cpu().numpy()
    hsum = h.double().abs().sum(dim=0).cpu().numpy()
    e_all = logit_bounds(values(h[::64]), wv).max()
    bound = (2.0 ** -9 + 2 * e_all + 1e-6 + M * 2.0 ** -24) * (2.0 / M) * hsum
    assert np.all(np.abs(col) <= bound), np.abs(col / bound).max()
