"""Seeded synthetic inputs for row-wise softmax cross-entropy.

This module builds logits and targets only; it holds none of the loss
arithmetic, and both the GPU library's tests and the CPU oracle's tests feed
from it.  Inputs are drawn with ``torch.Generator`` on the requested device:
logits in fp32 as ``sigma * N(0, 1)``, then (for fp16/bf16) cast with
round-to-nearest-even; targets uniform in ``[0, V)`` as int64.

The ``stress`` structure builds the stability workload (fp16, V = 50257):
  * 1 % of rows (round(0.01 M), at least 1) get a dominant target logit: after
    the -inf entries are placed, x[i, t_i] := max over the other finite
    entries of the row + 30;
  * another, disjoint 1 % of rows are all-equal: every entry is the row's
    first sampled value;
  * 0.1 % of the entries (Bernoulli(0.001) per entry) are -inf, never at the
    target column and never inside an all-equal row.
The two row sets come from one seeded permutation of the rows.
"""
import numpy as np
import torch

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}

# The five workloads: tiny, classifier, LM head, stress, skinny.
CONFIGS = {
    "tiny": dict(dtype="f32", M=64, V=1000, sigma=1.0, seed=101, structure=None,
                 ops=("fwd",), reductions=("mean", "none")),
    "classifier": dict(dtype="f32", M=32768, V=4096, sigma=1.0, seed=102, structure=None,
                       ops=("fwd",), reductions=("mean",)),
    "lmhead": dict(dtype="bf16", M=16384, V=131072, sigma=2.0, seed=103, structure=None,
                   ops=("fwd", "fwd_bwd"), reductions=("mean",)),
    "stress": dict(dtype="f16", M=8192, V=50257, sigma=8.0, seed=104, structure="stress",
                   ops=("fwd", "fwd_bwd"), reductions=("mean",)),
    "skinny": dict(dtype="f32", M=1048576, V=128, sigma=1.0, seed=105, structure=None,
                   ops=("fwd",), reductions=("none", "mean")),
}


def _special_rows(M, gen, device):
    n = max(1, int(round(0.01 * M)))
    if 2 * n > M:
        n = M // 2
    perm = torch.randperm(M, generator=gen, device=device)
    return perm[:n], perm[n:2 * n]


def make(dtype="f32", M=64, V=1000, sigma=1.0, seed=0, structure=None,
         device="cpu", chunk_rows=4096):
    """Return (logits [M, V] of `dtype`, targets [M] int64) on `device`.

    Rows are drawn in chunks of `chunk_rows` from one generator, so the values
    do not depend on the chunk size only when it is left at its default; the
    result is reproducible for a fixed (seed, device, chunk_rows).
    """
    if dtype not in TORCH_DTYPE:
        raise ValueError("dtype must be one of %s" % sorted(TORCH_DTYPE))
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    targets = torch.randint(0, V, (M,), generator=gen, device=dev, dtype=torch.int64)
    out = torch.empty((M, V), dtype=TORCH_DTYPE[dtype], device=dev)
    if structure is None:
        for r0 in range(0, M, chunk_rows):
            r1 = min(M, r0 + chunk_rows)
            x = torch.randn((r1 - r0, V), generator=gen, device=dev, dtype=torch.float32)
            if sigma != 1.0:
                x.mul_(sigma)
            out[r0:r1].copy_(x)
        return out, targets
    if structure != "stress":
        raise ValueError("unknown structure %r" % (structure,))
    dominant, equal = _special_rows(M, gen, dev)
    is_equal = torch.zeros(M, dtype=torch.bool, device=dev)
    is_equal[equal] = True
    is_dominant = torch.zeros(M, dtype=torch.bool, device=dev)
    is_dominant[dominant] = True
    for r0 in range(0, M, chunk_rows):
        r1 = min(M, r0 + chunk_rows)
        n = r1 - r0
        x = torch.randn((n, V), generator=gen, device=dev, dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        ninf = torch.rand((n, V), generator=gen, device=dev) < 0.001
        ninf &= ~is_equal[r0:r1, None]
        tcol = targets[r0:r1]
        rows = torch.arange(n, device=dev)
        ninf[rows, tcol] = False
        x.masked_fill_(ninf, float("-inf"))
        dom = is_dominant[r0:r1]
        if bool(dom.any()):
            other = x.clone()
            other[rows, tcol] = float("-inf")
            mx = other.max(dim=1).values
            x[rows[dom], tcol[dom]] = mx[dom] + 30.0
        eq = is_equal[r0:r1]
        if bool(eq.any()):
            x[eq] = x[eq][:, :1].expand(-1, V)
        out[r0:r1].copy_(x)
    return out, targets


def make_config(name, device="cpu", M=None, V=None):
    """Inputs of a named workload, optionally with M and/or V overridden."""
    c = dict(CONFIGS[name])
    return make(c["dtype"], c["M"] if M is None else M, c["V"] if V is None else V,
                c["sigma"], c["seed"], c["structure"], device=device)


def host_bits(t):
    """A host numpy copy of a logits tensor: float32 for fp32, uint16 bit
    patterns for fp16/bf16 (the form the oracle takes)."""
    t = t.detach()
    if t.dtype == torch.float32:
        return t.cpu().numpy()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def dtype_name(t):
    for k, v in TORCH_DTYPE.items():
        if t.dtype == v:
            return k
    raise TypeError("unsupported logits dtype %s" % t.dtype)


# The linear + cross-entropy workload: an LM head with the LM-head workload's
# vocabulary (V = 131072) and logit spread (sigma = 2), hidden size 4096 and
# 4096 tokens, in bf16.  The sizes other than V are this library's choice.
LINEAR_CONFIGS = {
    "lmhead_linear": dict(M=4096, D=4096, V=131072, sigma=2.0, seed=106),
}


def make_linear(M=64, D=256, V=1000, sigma=2.0, seed=0, device="cpu"):
    """Return (hidden [M, D] bf16, weight [V, D] bf16, targets [M] int64):
    hidden ~ N(0, 1) and weight ~ N(0, sigma^2 / D), so the logits hidden @
    weight.T have standard deviation close to sigma; drawn in fp32 and rounded
    to nearest even."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    targets = torch.randint(0, V, (M,), generator=gen, device=dev, dtype=torch.int64)
    hidden = torch.randn((M, D), generator=gen, device=dev, dtype=torch.float32)
    hidden = hidden.to(torch.bfloat16)
    weight = torch.empty((V, D), dtype=torch.bfloat16, device=dev)
    scale = sigma / float(D) ** 0.5
    for r0 in range(0, V, 8192):
        r1 = min(V, r0 + 8192)
        w = torch.randn((r1 - r0, D), generator=gen, device=dev, dtype=torch.float32)
        weight[r0:r1].copy_(w.mul_(scale))
    return hidden, weight, targets
