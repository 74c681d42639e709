"""The C-ABI calls captured in a HIP graph (torch.cuda.CUDAGraph over the
binding, which launches on torch's current stream): every replay, with the
program's own eager work and synchronizations between replays, matches the
eager result bit for bit.  The calls record no memset (the workspace needs no
initialization) and allocate nothing during capture (the workspace and
outputs are made beforehand)."""
import numpy as np
import pytest

from gpu_util import inputs, say

pytestmark = pytest.mark.gpu


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


@pytest.mark.parametrize("name", ["tiny", "classifier", "stress"])
def test_graph_replays_match_eager(ce, name):
    import torch
    c = inputs.CONFIGS[name]
    M = min(c["M"], 4096)
    x, t = inputs.make(c["dtype"], M, c["V"], c["sigma"], c["seed"], c["structure"],
                       device="cuda:0")
    nb = ce.ce_workspace_bytes(M, c["V"], {"f32": 0, "f16": 1, "bf16": 2}[c["dtype"]], "mean")
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
    # eager references
    loss_ref = ce.ce_fwd(x, t, "mean", workspace=ws).clone()
    rows_ref = ce.ce_fwd(x, t, "none").clone()
    g_ref = x.clone()
    lfb_ref = ce.ce_fwd_bwd_inplace(g_ref, t, "mean", workspace=ws).clone()
    torch.cuda.synchronize()

    out = torch.empty((), dtype=torch.float32, device="cuda:0")
    rows = torch.empty(M, dtype=torch.float32, device="cuda:0")
    lfb = torch.empty((), dtype=torch.float32, device="cuda:0")
    buf = x.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up on the capture stream
        ce.ce_fwd(x, t, "mean", out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ce.ce_fwd(x, t, "mean", out=out, workspace=ws)
        ce.ce_fwd(x, t, "none", out=rows)
        ce.ce_fwd_bwd_inplace(buf, t, "mean", out=lfb, workspace=ws)
    for rep in range(4):
        say("graph", name, "replay", rep)
        buf.copy_(x)                       # eager work between replays
        out.fill_(-1.0)
        rows.fill_(-1.0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(out), bits(loss_ref)), (rep, out.item(), loss_ref.item())
        assert torch.equal(bits(rows), bits(rows_ref)), rep
        assert torch.equal(bits(lfb), bits(lfb_ref)), rep
        assert torch.equal(bits(buf), bits(g_ref)), rep
        _ = ce.ce_fwd(x, t, "sum", workspace=ws).item()   # eager call on the same workspace
