"""GPU parity: the HIP path through the C ABI against the fp64 oracle, element by
element, on seeded inputs that span several tiles and ragged tails.

Tolerances (stated once in gpu_util): row and reduced losses 1e-5 relative
(+ 4 fp32 ulps of the row's largest magnitude per row); gradients within 2
ulps of the storage type; targets, NaN positions and untouched memory exact.
"""
import math
import os

import numpy as np
import pytest

from gpu_util import (check_grads, check_row_losses, check_scalar, host_grad_bits, oracle,
                      inputs, say)

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "f16", "bf16"]
CANARY = {"f32": 0x7FC0DEAD, "f16": 0x7E5A, "bf16": 0x7FDA}


@pytest.fixture(scope="module")
def ce():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    import softmax_cross_entropy_fwd_amd as ce
    ce.load_library()
    return ce


def place(x, offset, pad=24):
    """Copy host logits into a device buffer at an element offset, with
    canary elements before and after; returns (view, buffer)."""
    import torch
    M, V = x.shape
    n = M * V
    buf = torch.empty(offset + n + pad, dtype=x.dtype, device="cuda:0")
    canary_bits = CANARY[inputs.dtype_name(x)]
    bits_dtype = torch.int32 if x.dtype == torch.float32 else torch.int16
    if bits_dtype == torch.int16 and canary_bits >= 0x8000:
        canary_bits -= 0x10000
    buf.view(bits_dtype).fill_(canary_bits)
    view = buf[offset:offset + n].view(M, V)
    view.copy_(x.to("cuda:0"))
    return view, buf


def canaries_intact(buf, offset, n, dtype):
    import torch
    bits_dtype = torch.int32 if dtype == "f32" else torch.int16
    b = buf.view(bits_dtype).cpu().numpy().astype(np.int64) & (0xFFFFFFFF if dtype == "f32" else 0xFFFF)
    c = CANARY[dtype]
    return bool(np.all(b[:offset] == c) and np.all(b[offset + n:] == c))


def run_and_check(ce, dtype, M, V, sigma=1.0, seed=0, structure=None, reduction="mean",
                  op="fwd", offset=0, targets=None):
    import torch
    say("case", dtype, M, V, sigma, seed, structure, reduction, op, offset)
    x, t = inputs.make(dtype, M, V, sigma, seed, structure, device="cpu")
    if targets is not None:
        t = torch.as_tensor(targets, dtype=torch.int64)
    xb, tn = inputs.host_bits(x), t.numpy()
    xg, buf = place(x, offset)
    tg = t.to("cuda:0")
    if op == "fwd":
        got = ce.ce_fwd(xg, tg, reduction)
    else:
        got = ce.ce_fwd_bwd_inplace(xg, tg, reduction)
    torch.cuda.synchronize()
    assert canaries_intact(buf, offset, M * V, dtype), "wrote outside the logits"
    per_row = oracle.loss_rows(xb, tn, dtype=dtype)
    if reduction == "none":
        check_row_losses(got.cpu().numpy(), per_row, xb, tn, dtype)
    else:
        check_scalar(got.item(), oracle.reduce(per_row, reduction))
    if op == "fwd_bwd":
        c = 1.0 / M if reduction == "mean" else 1.0
        want, want64 = oracle.grad_rows(xb, tn, dtype=dtype, c=c, want64=True)
        check_grads(host_grad_bits(xg), want, dtype, c, want64)
    else:
        np.testing.assert_array_equal(inputs.host_bits(xg), xb)   # fwd leaves logits alone
    return got


# --------------------------------------------------------------- workloads

def test_tiny_mean_and_none(ce):
    c = inputs.CONFIGS["tiny"]
    for red in ("mean", "none", "sum"):
        run_and_check(ce, c["dtype"], c["M"], c["V"], c["sigma"], c["seed"], reduction=red)
        run_and_check(ce, c["dtype"], c["M"], c["V"], c["sigma"], c["seed"], reduction=red,
                      op="fwd_bwd")


@pytest.mark.parametrize("name,M", [("classifier", 96), ("lmhead", 12), ("stress", 300),
                                    ("skinny", 4099)])
def test_workload_shapes_small_m(ce, name, M):
    c = inputs.CONFIGS[name]
    for red in ("none", "mean"):
        for op in ("fwd", "fwd_bwd"):
            run_and_check(ce, c["dtype"], M, c["V"], c["sigma"], c["seed"], c["structure"],
                          reduction=red, op=op)


# ----------------------------------------------------------- V and alignment

V_SWEEP = [1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256,
           257, 511, 512, 513, 1000, 1023, 1024, 1025, 2047, 2048, 2049, 4095, 4096, 4097, 8191,
           8192, 8193, 16383, 16384, 16385, 32768, 50257, 65536, 65537, 131071, 131072, 131073,
           262151]


@pytest.mark.parametrize("dtype", DTYPES)
def test_v_sweep(ce, dtype):
    for V in V_SWEEP:
        M = 7 if V < 100000 else 3
        sigma = 8.0 if dtype == "f16" else 3.0
        run_and_check(ce, dtype, M, V, sigma, seed=V, reduction="none")
        run_and_check(ce, dtype, M, V, sigma, seed=V + 1, reduction="mean", op="fwd_bwd")


@pytest.mark.parametrize("dtype", DTYPES)
def test_alignment_sweep(ce, dtype):
    E = 4 if dtype == "f32" else 8
    for V in (1, 3, 127, 1000, 4097, 50257, 131072):
        for off in range(1, E):
            M = 5 if V < 100000 else 2
            run_and_check(ce, dtype, M, V, 2.0, seed=17 * off + V, reduction="none", offset=off)
            run_and_check(ce, dtype, M, V, 2.0, seed=17 * off + V + 1, reduction="sum",
                          op="fwd_bwd", offset=off)


# --------------------------------------------------------- every kernel shape

SHAPES = ["rows:1:1", "rows:1:2", "rows:1:4", "rows:2:4", "rows:4:4", "rows:8:4", "rows:16:4",
          "rows:32:4", "rows:64:4", "rows:64:8", "rows:64:16", "rows:4:8", "rows:8:2",
          "rows:16:2", "rows:32:1", "rows:32:8", "rows:32:16", "rows:32:32", "rows:2:16",
          "wg:4:8", "wg:8:8", "wg:8:12", "wg:8:16", "wg:16:8", "wg:16:12", "wg:16:16",
          "wg:4:16", "wg:16:4", "wg:16:2", "wg:16:3", "wg:16:5", "wg:16:6", "wg:16:7",
          "wg2:8:9", "wg2:8:11", "wg2:8:13", "stream:4:8", "stream:8:4", "stream:8:8", "stream:16:4",
          "stream:4:16", "stream:1:4", "stream:2:4", "stream:4:4", "stream:1:8", "stream:2:8",
          "stream:1:16", "stream:16:2", "stream:16:1", "stream:8:2",
          "wstream:1:2", "wstream:1:4", "wstream:1:8",
          # forward only: 5 or 6 vectors per lane
          "rows:8:5", "rows:8:6", "rows:16:5", "rows:16:6", "rows:32:5", "rows:32:6"]
# row buffers of the rows kernel: 1 or 2 with 4-wave workgroups, 17 or 18 with
# 16-wave workgroups (64:16 and 4:8 only)
NBUFS = {"rows:64:16": ("1", "2", "17", "18"), "rows:4:8": ("1", "2", "17", "18")}


@pytest.mark.parametrize("shape", SHAPES)
def test_every_kernel_shape(ce, shape, tuning):
    kind, a, b = shape.split(":")
    a, b = int(a), int(b)
    cap = a * b if kind == "rows" else (a * 64 * b if kind in ("wg", "wg2") else 1 << 30)
    tuning.setenv("CE_FORCE_PLAN", shape)
    for nbuf in NBUFS.get(shape, ("1", "2") if kind == "rows" else ("1",)):
        tuning.setenv("CE_FORCE_NBUF", nbuf)
        _check_shape(ce, shape, kind, cap)


# the forward mappings that pick the target's logit from their registers as
# the row is folded (fp32 rows over 8-32 lanes, 16-bit rows over 8 lanes)
@pytest.mark.parametrize("dtype,V,shape", [("f32", 128, "rows:8:4"), ("f32", 100, "rows:8:4"),
                                           ("f32", 37, "rows:8:4"), ("f32", 256, "rows:16:4"),
                                           ("f32", 61, "rows:16:2"), ("f32", 500, "rows:32:4"),
                                           ("bf16", 256, "rows:8:4"), ("f16", 203, "rows:8:4"),
                                           ("f32", 160, "rows:8:5"), ("f32", 188, "rows:8:6"),
                                           ("f16", 250, "rows:8:5"), ("bf16", 384, "rows:8:6"),
                                           ("f32", 320, "rows:16:5"), ("f32", 380, "rows:16:6")])
def test_forward_target_at_every_position(ce, tuning, dtype, V, shape):
    """Row i's target is i mod V, so every element of the row -- every lane,
    register and element slot of the tile -- is the target of some row;
    per-row losses against the oracle, aligned and shifted bases, one and two
    register sets, and a spread wide enough that many targets dominate."""
    tuning.setenv("CE_FORCE_PLAN", shape)
    M = 2 * V + 37
    targets = [i % V for i in range(M)]
    for nbuf in ("1", "2"):
        tuning.setenv("CE_FORCE_NBUF", nbuf)
        for offset, sigma in ((0, 3.0), (1, 3.0), (0, 12.0)):
            plan = ce.ce_plan_describe(M, V, {"f32": 0, "f16": 1, "bf16": 2}[dtype], "none")
            assert plan.startswith(shape), plan
            run_and_check(ce, dtype, M, V, sigma, seed=V + M + offset, reduction="none",
                          offset=offset, targets=targets)
            run_and_check(ce, dtype, M, V, sigma, seed=V + 7, reduction="mean", offset=offset,
                          targets=targets)


def _check_shape(ce, shape, kind, cap):
    for dtype in DTYPES:
        if kind == "wg2" and dtype == "f32":
            continue   # 16-bit storage only
        E = 4 if dtype == "f32" else 8
        for V in (1, 5, 13 * E + 3, 64 * E, 64 * E + 1, 3000, 20000):
            if (V + 2 * E - 2) // E > cap:
                continue
            M = 37 if V < 4000 else 9
            plan = ce.ce_plan_describe(M, V, {"f32": 0, "f16": 1, "bf16": 2}[dtype], "none")
            if V % E == 0:
                assert plan.startswith(shape), (plan, shape)
            run_and_check(ce, dtype, M, V, 4.0, seed=V, reduction="none", offset=V % 3)
            run_and_check(ce, dtype, M, V, 4.0, seed=V + 5, reduction="mean", op="fwd_bwd",
                          offset=(V // 2) % 2)
            run_and_check(ce, dtype, M, V, 4.0, seed=V + 9, reduction="sum", offset=0)


# The fused backward's mapping for rows past 16 KB, one case per branch of the
# plan table (window vectors: 16 bytes each): streamed twice by 8-wave
# workgroups up to 3072 vectors, by 16-wave ones up to 8192 unless the row
# fills a register tile exactly (16-bit rows of 4097-6656 vectors: 8-wave
# register tiles, two workgroups per CU), register tiles of 12 or 16 x 1024
# vectors up to 16384.
EPI_TABLE = [(1500, 0, "stream:8:4", "stream:8:4"), (3072, 0, "stream:8:4", "stream:8:4"),
             (4096, 0, "wg:16:4", "wg:16:4"), (5120, 0, "wg:16:5", "wg:16:5"),
             (5000, 0, "stream:16:4", "wg2:8:10"), (6283, 1, "stream:16:4", "wg2:8:13"),
             (7168, 0, "wg:16:7", "wg:16:7"), (8192, 0, "wg:16:8", "wg:16:8"),
             (8000, 0, "stream:16:4", "stream:16:4"), (10240, 0, "wg:16:12", "wg:16:12"),
             (14336, 0, "wg:16:16", "wg:16:16")]


@pytest.mark.parametrize("dtype", DTYPES)
def test_epilogue_plan_table(ce, dtype):
    E = 4 if dtype == "f32" else 8
    code = {"f32": 0, "f16": 1, "bf16": 2}[dtype]
    for nvec, ragged, shape32, shape16 in EPI_TABLE:
        shape = shape32 if dtype == "f32" else shape16
        V = nvec * E - (E - 1 if ragged else 0)
        M = 300 if nvec <= 3072 else 150
        plan = ce.ce_plan_describe(M, V, code, "mean", op=ce.CE_OP_FWD_BWD)
        assert plan.startswith(shape), (dtype, V, plan, shape)
        run_and_check(ce, dtype, M, V, 4.0, seed=nvec, reduction="mean", op="fwd_bwd")
        run_and_check(ce, dtype, M, V, 4.0, seed=nvec + 1, reduction="none", op="fwd_bwd",
                      offset=1)


# Both row orders of the rows and workgroup kernels (the grid striding over
# the rows, or a contiguous band of rows per workgroup, CE_ROW_MAP), for
# forwards in register rows (one row per wavefront, and narrower rows), the
# fused backward and a workgroup tile.  Batches that leave some workgroups'
# bands empty (M below the grid's rows per pass) and ragged last bands.
@pytest.mark.parametrize("row_map", ["interleaved", "blocked"])
def test_row_maps(ce, tuning, row_map):
    tuning.setenv("CE_ROW_MAP", row_map)
    cases = [("f32", 1000, 500, "fwd"), ("f32", 3, 500, "fwd"), ("bf16", 777, 2000, "fwd"),
             ("f16", 5000, 128, "fwd"), ("f32", 2049, 1000, "fwd_bwd"),
             ("f32", 1000, 4096, "fwd_bwd"), ("bf16", 300, 32768, "fwd_bwd")]
    for dtype, M, V, op in cases:
        code = {"f32": 0, "f16": 1, "bf16": 2}[dtype]
        plan = ce.ce_plan_describe(M, V, code, "mean",
                                   op=ce.CE_OP_FWD if op == "fwd" else ce.CE_OP_FWD_BWD)
        assert (" blocked " in plan) == (row_map == "blocked"), plan
        for red in ("mean", "none"):
            run_and_check(ce, dtype, M, V, 3.0, seed=M + V, reduction=red, op=op,
                          offset=0 if red == "mean" else 1)


# Grids of 8 to 16 wavefronts per CU (the bytes each keeps in flight set the
# count), at batches that take several grid-stride passes: the forward (a
# rows kernel, or for rows of 257-1536 vectors one wavefront per row in
# chunks) and the fused backward, every element against the oracle.
@pytest.mark.parametrize("dtype,M,V", [("bf16", 20000, 2000), ("f32", 12000, 2000),
                                      ("f16", 6000, 4000), ("f32", 9000, 3000)])
def test_rows_kernels_full_grid(ce, dtype, M, V):
    code = {"f32": 0, "f16": 1, "bf16": 2}[dtype]
    for op, cop in (("fwd", ce.CE_OP_FWD), ("fwd_bwd", ce.CE_OP_FWD_BWD)):
        plan = ce.ce_plan_describe(M, V, code, "mean", op=cop)
        say("plan", op, plan)
        grid = int(plan.split("grid=")[1].split()[0])
        kinds = ("rows:", "wstream:") if op == "fwd" else ("rows:",)
        assert plan.startswith(kinds) and grid >= 512, plan
        for red in ("mean", "none"):
            run_and_check(ce, dtype, M, V, 3.0, seed=M + V + len(red), reduction=red, op=op,
                          offset=0 if red == "mean" else 1)


def test_rows_grid_rule(ce):
    # wavefronts per CU of the rows kernels: ~64 KiB in flight per CU (K KiB
    # each), ~128 KiB for 16-bit rows and for softmax / the fused backward,
    # to the nearest whole 4-wave workgroup, 4 to 16 (fp32 forwards over 8+
    # lanes per row: at most 12); two-buffer narrow rows
    # (epilogues of rows of 17-32 vectors) 4.  The forward of rows of 17-32
    # vectors: 8 lanes x 4 vectors; of 33-128 (16-bit: 33-256): 4-6 vectors
    # per lane over a power-of-two number of lanes (every operation).  Of 257-1536
    # vectors: one wavefront per row in chunks, 8 (fp32) or 12 (16-bit) per
    # CU; fp32 rows of 129-256 vectors: one chunk per row, 12 or 16 per CU.
    # (Batches large enough to fill the grids.)
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    cases = [  # (M, V, dtype code, op, mapping, wavefronts per CU)
        (131072, 1000, 0, ce.CE_OP_FWD, "wstream:1:4", 12),   # fp32, one chunk per row
        (196608, 800, 0, ce.CE_OP_FWD, "wstream:1:4", 16),
        (131072, 512, 0, ce.CE_OP_FWD, "rows:32:4", 12),
        (131072, 2000, 2, ce.CE_OP_FWD, "rows:64:4", 16),     # bf16, K = 4
        (1048576, 128, 0, ce.CE_OP_FWD, "rows:8:4", 12),      # whole lines per load
        (1048576, 256, 2, ce.CE_OP_FWD, "rows:8:4", 16),
        (1048576, 128, 0, ce.CE_OP_FWD_BWD, "rows:4:8", 4),   # two buffers
        (32768, 4096, 0, ce.CE_OP_SOFTMAX, "rows:64:16", 8),  # folded epilogue
        (32768, 4096, 0, ce.CE_OP_FWD_BWD, "rows:64:16", 8),
        (32768, 4096, 0, ce.CE_OP_BWD, "rows:64:16", 4),      # epilogue without a fold
        (65536, 2000, 0, ce.CE_OP_SOFTMAX, "rows:64:8", 16),
        (32768, 8000, 2, ce.CE_OP_SOFTMAX, "rows:64:16", 8),  # bf16, K = 16
        (32768, 4096, 0, ce.CE_OP_FWD, "wstream:1:4", 8),
        (65536, 2000, 0, ce.CE_OP_FWD, "wstream:1:8", 8),
        (32768, 8000, 2, ce.CE_OP_FWD, "wstream:1:4", 12),
        (65536, 1500, 2, ce.CE_OP_FWD, "rows:32:6", 16),      # 188 vectors: 32 x 6
        (1048576, 160, 0, ce.CE_OP_FWD, "rows:8:5", 12),      # 40 vectors: 8 x 5
        (524288, 320, 0, ce.CE_OP_FWD, "rows:16:5", 12),      # 80 vectors: 16 x 5
        (524288, 380, 0, ce.CE_OP_FWD, "rows:16:6", 12),      # 95 vectors: 16 x 6
        (262144, 1500, 1, ce.CE_OP_FWD, "rows:32:6", 16),
        (65536, 1500, 2, ce.CE_OP_FWD_BWD, "rows:32:6", 16),  # the epilogues' tiles fit too
        (1048576, 384, 2, ce.CE_OP_SOFTMAX, "rows:8:6", 16),
        (524288, 320, 0, ce.CE_OP_BWD, "rows:16:5", 12),
    ]
    for M, V, code, op, mapping, waves in cases:
        plan = ce.ce_plan_describe(M, V, code, "mean", op=op)
        grid = int(plan.split("grid=")[1].split()[0])
        block = int(plan.split("block=")[1].split()[0])
        assert plan.startswith(mapping + " "), (M, V, code, op, plan)
        assert grid * block // 64 == waves * cus, (M, V, code, op, plan)


def test_default_row_map(ce):
    # by default every grid strides over the rows (bands only on request)
    for M, V, code, op in ((32768, 4096, 0, ce.CE_OP_FWD), (100, 1000, 0, ce.CE_OP_FWD),
                           (65536, 2000, 0, ce.CE_OP_FWD), (100, 2000, 2, ce.CE_OP_FWD),
                           (1048576, 128, 0, ce.CE_OP_FWD), (32768, 4096, 0, ce.CE_OP_FWD_BWD),
                           (16384, 131072, 2, ce.CE_OP_FWD)):
        assert " blocked " not in ce.ce_plan_describe(M, V, code, "mean", op=op)


# ------------------------------------------------------------------ edge cases

def test_empty_batch(ce):
    import torch
    for dtype in DTYPES:
        x = torch.empty(0, 10, dtype=inputs.TORCH_DTYPE[dtype], device="cuda:0")
        t = torch.empty(0, dtype=torch.int64, device="cuda:0")
        assert math.isnan(ce.ce_fwd(x, t, "mean").item())
        assert ce.ce_fwd(x, t, "sum").item() == 0.0
        assert ce.ce_fwd(x, t, "none").numel() == 0
        assert math.isnan(ce.ce_fwd_bwd_inplace(x, t, "mean").item())


def test_out_of_range_targets(ce):
    for dtype in DTYPES:
        M, V = 6, 300
        targets = [0, -1, V, 5, 1 << 40, V - 1]
        run_and_check(ce, dtype, M, V, 2.0, seed=3, reduction="none", targets=targets)
        run_and_check(ce, dtype, M, V, 2.0, seed=3, reduction="sum", op="fwd_bwd",
                      targets=targets)
        got = run_and_check(ce, dtype, M, V, 2.0, seed=3, reduction="mean", targets=targets)
        assert math.isnan(got.item())


def test_stress_structure_rows(ce):
    # dominant targets, all-equal rows and -inf entries at a size the oracle
    # does in a blink; the fractions make sure every kind of row is present
    for dtype in DTYPES:
        for V in (50257, 1000, 96):
            run_and_check(ce, dtype, 200, V, 8.0, seed=104, structure="stress", reduction="none")
            run_and_check(ce, dtype, 200, V, 8.0, seed=104, structure="stress", reduction="mean",
                          op="fwd_bwd")


def test_dominant_target_loss_and_grad_accuracy(ce):
    import torch
    # p_t close to 1: the target's gradient and the small loss keep their
    # relative accuracy (recomputed from the other terms)
    for dtype in DTYPES:
        for V in (7, 1000, 50257):
            for gap in (3.0, 9.0, 15.0):
                M = 8
                x, t = inputs.make(dtype, M, V, 1.0, seed=int(gap) + V)
                xf = x.float()
                xf[torch.arange(M), t] = xf.max(dim=1).values + gap
                xd = xf.to(x.dtype)
                xb, tn = inputs.host_bits(xd), t.numpy()
                xg = xd.to("cuda:0")
                got = ce.ce_fwd_bwd_inplace(xg, t.to("cuda:0"), "none")
                torch.cuda.synchronize()
                check_row_losses(got.cpu().numpy(), oracle.loss_rows(xb, tn, dtype=dtype), xb,
                                 tn, dtype, rtol=1e-4)
                want, want64 = oracle.grad_rows(xb, tn, dtype=dtype, c=1.0, want64=True)
                check_grads(host_grad_bits(xg), want, dtype, 1.0, want64)


@pytest.mark.parametrize("shape", [None, "stream:4:4", "stream:8:4", "stream:16:4"])
def test_dominant_target_small_loss_relative(ce, shape, tuning):
    import torch
    # p_t > 1/2: the loss log1p(sum of the other terms / e_t) keeps its
    # relative accuracy however small it is (no absolute floor here), in the
    # streamed kernels (which leave the target out of their first pass) and
    # in the default mappings (which sum the other terms on a second read)
    if shape:
        tuning.setenv("CE_FORCE_PLAN", shape)
    for dtype in DTYPES:
        for V in (3000, 20000, 50257):
            for gap in (12.0, 30.0):
                M = 6
                x, t = inputs.make(dtype, M, V, 1.0, seed=int(gap) + V)
                xf = x.float()
                xf[torch.arange(M), t] = xf.max(dim=1).values + gap
                xd = xf.to(x.dtype)
                xb, tn = inputs.host_bits(xd), t.numpy()
                want = oracle.loss_rows(xb, tn, dtype=dtype)
                for op in ("fwd", "fwd_bwd"):
                    xg, buf = place(xd, V % 3)
                    tg = t.to("cuda:0")
                    got = (ce.ce_fwd(xg, tg, "none") if op == "fwd"
                           else ce.ce_fwd_bwd_inplace(xg, tg, "none"))
                    got = got.cpu().numpy().astype(np.float64)
                    assert np.all(want > 0) and np.all(want < math.log(2)), want
                    err = np.abs(got - want) / want
                    assert err.max() <= 1e-4, (dtype, V, gap, op, got, want)
                    if op == "fwd_bwd":
                        w, w64 = oracle.grad_rows(xb, tn, dtype=dtype, c=1.0, want64=True)
                        check_grads(host_grad_bits(xg), w, dtype, 1.0, w64)
                    assert canaries_intact(buf, V % 3, M * V, dtype)


def test_uniform_rows_closed_form(ce):
    import torch
    for dtype in DTYPES:
        for V in (1000, 4096, 50257, 131072, 128):
            for L in (0.0, -7.25, 30.5):
                x = torch.full((3, V), L, dtype=inputs.TORCH_DTYPE[dtype], device="cuda:0")
                t = torch.tensor([0, V // 2, V - 1], device="cuda:0")
                got = ce.ce_fwd(x, t, "none").cpu().numpy()
                np.testing.assert_allclose(got, math.log(V), rtol=1e-5,
                                           atol=4 * np.spacing(np.float32(max(abs(L), 1))))


def test_deterministic_bits(ce):
    import torch
    for name, M in (("classifier", 2048), ("skinny", 70000), ("stress", 256)):
        c = inputs.CONFIGS[name]
        x, t = inputs.make(c["dtype"], M, c["V"], c["sigma"], c["seed"], c["structure"],
                           device="cuda:0")
        a = ce.ce_fwd(x, t, "mean").item()
        b = ce.ce_fwd(x, t, "mean").item()
        assert np.float32(a).tobytes() == np.float32(b).tobytes()
        y = x.clone()
        la = ce.ce_fwd_bwd_inplace(x, t, "mean").item()
        lb = ce.ce_fwd_bwd_inplace(y, t, "mean").item()
        torch.cuda.synchronize()
        assert np.float32(la).tobytes() == np.float32(lb).tobytes()
        assert torch.equal(x.view(torch.int16 if x.element_size() == 2 else torch.int32),
                           y.view(torch.int16 if y.element_size() == 2 else torch.int32))


def test_workspace_reuse_and_streams(ce):
    import torch
    x, t = inputs.make("f32", 5000, 333, 1.0, seed=9, device="cuda:0")
    want = oracle.fwd(inputs.host_bits(x), t.cpu().numpy(), reduction="mean")
    s = torch.cuda.Stream()
    for i in range(5):
        check_scalar(ce.ce_fwd(x, t, "mean").item(), want)
        with torch.cuda.stream(s):
            r = ce.ce_fwd(x, t, "mean")
        s.synchronize()
        check_scalar(r.item(), want)


def test_workspace_needs_no_initialization(ce):
    import torch
    # the partial-sum slots are written before they are read: garbage in the
    # workspace (NaN bit patterns) changes nothing
    for name, M in (("classifier", 3000), ("stress", 64), ("skinny", 9000)):
        c = inputs.CONFIGS[name]
        x, t = inputs.make(c["dtype"], M, c["V"], c["sigma"], c["seed"], c["structure"],
                           device="cuda:0")
        nbytes = ce.ce_workspace_bytes(M, c["V"], {"f32": 0, "f16": 1, "bf16": 2}[c["dtype"]],
                                       "mean")
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda:0")
        want = oracle.reduce(oracle.loss_rows(inputs.host_bits(x), t.cpu().numpy(),
                                              dtype=c["dtype"]), "mean")
        for _ in range(2):
            got = ce.ce_fwd(x, t, "mean", workspace=ws)
            check_scalar(got.item(), want)
        y = x.clone()
        got = ce.ce_fwd_bwd_inplace(y, t, "sum", workspace=ws)
        check_scalar(got.item(), oracle.reduce(oracle.loss_rows(
            inputs.host_bits(x), t.cpu().numpy(), dtype=c["dtype"]), "sum"))
