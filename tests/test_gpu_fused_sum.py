"""The final sum of a mean or sum done in the kernel's own launch (the last
workgroup adds the partials; whole rows, outside graph capture): bit for
bit the two-launch result, which a graph capture keeps, for every kernel
shape (register rows, one row per wavefront, streamed rows, register tiles),
call after call (every launch puts its counter back to zero), and with two
streams running at once (each stream has its own counter)."""
import pytest

from gpu_util import inputs, say

pytestmark = pytest.mark.gpu

CODES = {"f32": 0, "f16": 1, "bf16": 2}


@pytest.fixture(scope="module")
def ce():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    import softmax_cross_entropy_fwd_amd as ce
    ce.load_library()
    return ce


def bits(t):
    import torch
    return t.view(torch.int32 if t.element_size() == 4 else torch.int16).clone()


def two_launch(ce, fn, *args, **kw):
    """fn's result from a captured graph (where the final sum keeps its own
    launch), replayed once."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(*args, **kw)   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        res = fn(*args, **kw)
    graph.replay()
    torch.cuda.synchronize()
    return res


# forward / fused backward kernel shapes: register rows / register rows;
# rows / rows; rows / rows; rows / rows; streamed / streamed; one row per
# wavefront / streamed; streamed / 16-wave tile; streamed / two-part tile;
# streamed / 16-wave tile
@pytest.mark.parametrize("dtype,M,V", [("f32", 64, 1000), ("bf16", 1, 4096), ("f16", 300, 777),
                                      ("f32", 2048, 1000), ("bf16", 129, 16384),
                                      ("f32", 500, 5000), ("f32", 256, 16384),
                                      ("f16", 200, 40000), ("bf16", 300, 131072)])
def test_fused_sum_matches_two_launch_form(ce, dtype, M, V):
    import torch
    say("fused sum", dtype, M, V)
    x, t = inputs.make(dtype, M, V, 4.0, seed=M + V, device="cuda:0")
    for red in ("mean", "sum"):
        nb = ce.ce_workspace_bytes(M, V, CODES[dtype], red)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
        out = torch.empty((), dtype=torch.float32, device="cuda:0")
        ref = bits(two_launch(ce, ce.ce_fwd, x, t, red, out=out, workspace=ws))
        for i in range(50):
            got = ce.ce_fwd(x, t, red, workspace=ws)
            assert torch.equal(bits(got), ref), (red, i, got.item(), out.item())
    # the fused backward's loss and gradients: the graph helper runs it twice
    # over its buffer (warm-up, then the replay), so compare with a second
    # eager pass
    nb = ce.ce_workspace_bytes(M, V, CODES[dtype], "mean")
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
    g_ref = x.clone()
    lfb = torch.empty((), dtype=torch.float32, device="cuda:0")
    ref = bits(two_launch(ce, ce.ce_fwd_bwd_inplace, g_ref, t, "mean", out=lfb, workspace=ws))
    g = x.clone()
    ce.ce_fwd_bwd_inplace(g, t, "mean", workspace=ws)
    got = ce.ce_fwd_bwd_inplace(g, t, "mean", workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(bits(got), ref)
    assert torch.equal(bits(g), bits(g_ref))


def test_fused_sum_on_two_streams(ce):
    import torch
    x1, t1 = inputs.make("f32", 64, 1000, 4.0, seed=1, device="cuda:0")
    x2, t2 = inputs.make("bf16", 40, 3000, 6.0, seed=2, device="cuda:0")
    ws1 = torch.empty(ce.ce_workspace_bytes(64, 1000, 0, "mean"), dtype=torch.uint8,
                      device="cuda:0")
    ws2 = torch.empty(ce.ce_workspace_bytes(40, 3000, 2, "sum"), dtype=torch.uint8,
                      device="cuda:0")
    ref1 = bits(ce.ce_fwd(x1, t1, "mean", workspace=ws1))
    ref2 = bits(ce.ce_fwd(x2, t2, "sum", workspace=ws2))
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs1, outs2 = [], []
    for _ in range(300):
        with torch.cuda.stream(s1):
            outs1.append(ce.ce_fwd(x1, t1, "mean", workspace=ws1))
        with torch.cuda.stream(s2):
            outs2.append(ce.ce_fwd(x2, t2, "sum", workspace=ws2))
    torch.cuda.synchronize()
    assert all(torch.equal(bits(o), ref1) for o in outs1)
    assert all(torch.equal(bits(o), ref2) for o in outs2)


@pytest.mark.parametrize("dtype,M,V", [("f32", 32768, 4096), ("bf16", 2048, 50257)])
def test_fused_sum_threshold_override(ce, tuning, dtype, M, V):
    """CE_FUSE_MAX_BYTES moves the size limit of the in-launch final sum: a
    large input finishes its mean in one launch with the two-launch form's
    bits (about 2048 workgroups adding their partials)."""
    import torch
    say("fused sum, large", dtype, M, V)
    x, t = inputs.make(dtype, M, V, 4.0, seed=M ^ V, device="cuda:0")
    tuning.setenv("CE_FUSE_MAX_BYTES", "0")
    ref = bits(ce.ce_fwd(x, t, "mean"))
    tuning.setenv("CE_FUSE_MAX_BYTES", str(1 << 40))
    outs = [ce.ce_fwd(x, t, "mean") for _ in range(20)]
    torch.cuda.synchronize()
    assert all(torch.equal(bits(o), ref) for o in outs), [o.item() for o in outs]
