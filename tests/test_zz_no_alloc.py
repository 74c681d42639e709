"""ce_fwd_noalloc (the forward that allocates nothing: its scratch is the
library's static per-device array) against ce_fwd (the same forward with a
caller workspace) and the oracle, through the C ABI.

Two calls in a row, the second on a smaller input, for each case: the second
call finds the first call's contents in the shared scratch and must not
depend on them.  Results must equal ce_fwd's bit for bit (same kernels, same
plan) and meet the oracle tolerances of the other parity tests.
"""
import numpy as np
import pytest

from gpu_util import check_row_losses, check_scalar, oracle, inputs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ce():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    import softmax_cross_entropy_fwd_amd as ce
    ce.load_library()
    return ce


# (dtype, M, V, sigma, structure, element offset of the base): pairs of a
# larger and a smaller call; the classifier rows (rows kernel, 1024 partial
# slots), the stress rows (streamed workgroups, misaligned), few long rows
# (split over workgroups: partials plus split statistics in the scratch).
PAIRS = [
    (("f32", 32768, 4096, 1.0, None, 0), ("f32", 300, 1000, 1.0, None, 0)),
    (("f16", 2048, 50257, 8.0, "stress", 1), ("f16", 77, 50257, 8.0, "stress", 3)),
    (("bf16", 100, 131072, 2.0, None, 0), ("bf16", 6, 131075, 2.0, None, 5)),
    (("f32", 64, 1000, 1.0, None, 0), ("f32", 1, 7, 1.0, None, 1)),
]


def make_case(dtype, M, V, sigma, structure, offset, seed):
    import torch
    x, t = inputs.make(dtype, M, V, sigma, seed, structure, device="cpu")
    buf = torch.empty(offset + M * V, dtype=x.dtype, device="cuda:0")
    xg = buf[offset:].view(M, V)
    xg.copy_(x.to("cuda:0"))
    return x, t, xg, t.to("cuda:0")


@pytest.mark.parametrize("pair", range(len(PAIRS)))
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_noalloc_matches_ce_fwd(ce, pair, reduction):
    import torch
    for i, (dtype, M, V, sigma, structure, offset) in enumerate(PAIRS[pair]):
        say("noalloc case", pair, i, dtype, M, V, structure, offset, reduction)
        x, t, xg, tg = make_case(dtype, M, V, sigma, structure, offset, seed=1000 * pair + i)
        got = ce.ce_fwd_noalloc(xg, tg, reduction)
        ref = ce.ce_fwd(xg, tg, reduction)
        torch.cuda.synchronize()
        g, r = got.cpu().numpy(), ref.cpu().numpy()
        np.testing.assert_array_equal(g.view(np.uint32), r.view(np.uint32))
        xb, tn = inputs.host_bits(x), t.numpy()
        per_row = oracle.loss_rows(xb, tn, dtype=dtype)
        if reduction == "none":
            check_row_losses(g, per_row, xb, tn, dtype)
        else:
            check_scalar(float(g), oracle.reduce(per_row, reduction))


def test_noalloc_back_to_back_on_one_stream(ce):
    # many calls queued without a synchronization in between, alternating
    # sizes, each with its own output: every result equals ce_fwd's
    import torch
    cases = [make_case("f32", 4096, 4096, 1.0, None, 0, seed=7),
             make_case("bf16", 40, 131072, 2.0, None, 0, seed=8),
             make_case("f16", 333, 5000, 4.0, None, 2, seed=9)]
    outs = []
    for rep in range(3):
        for x, t, xg, tg in cases:
            outs.append(ce.ce_fwd_noalloc(xg, tg, "mean"))
    refs = [ce.ce_fwd(xg, tg, "mean") for _, _, xg, tg in cases]
    torch.cuda.synchronize()
    for k, o in enumerate(outs):
        assert o.item() == refs[k % len(cases)].item(), (k, o.item(), refs[k % len(cases)].item())


def test_noalloc_empty_batch(ce):
    import torch
    x = torch.empty((0, 10), dtype=torch.float32, device="cuda:0")
    t = torch.empty((0,), dtype=torch.int64, device="cuda:0")
    assert np.isnan(ce.ce_fwd_noalloc(x, t, "mean").item())
    assert ce.ce_fwd_noalloc(x, t, "sum").item() == 0.0
    assert ce.ce_fwd_noalloc(x, t, "none").numel() == 0
