#!/usr/bin/env python3
"""Throughput of row-wise softmax cross-entropy on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--op fwd|fwd_bwd]
                    [--reduction mean|none|sum] [--no-extra] [--no-cpu]

A step is one pass of the whole path (one call of the C-ABI entry point) over
one batch of synthetic logits already resident in HBM.  The headline line is
the classifier workload (fp32 [32768, 4096], forward, mean): algorithmic HBM
GB/s = bytes the method must move / kernel time.  The same line carries:

  roofline      the kernel's achieved GB/s (algorithmic bytes per launch over
                the average launch duration: the K launches run back to back
                between one pair of HIP events on the launch stream) against
                MI355X's 8 TB/s, and the HBM traffic counted by
                rocprofv3 (FETCH_SIZE + WRITE_SIZE, calibrated on a plain copy)
                when a summary taken on the current kernel source is committed
                under profiles/;
  cpu_baseline  the fp64 oracle timed on the host cores over the whole workload;
  also          the LM-head workload (bf16 [16384, 131072]) forward, fused
                forward + in-place backward, split backward from a saved
                log-sum-exp and row softmax; the classifier's split backward
                and softmax; the stress (fp16 [8192, 50257], misaligned rows)
                forward and fused backward; the skinny (fp32 [1048576, 128])
                forward; each timed the same way; and linear + cross-entropy
                (logits = hidden @ weight.T, bf16 [4096, 4096] x [131072, 4096],
                taken in vocabulary chunks) forward and forward + backward in
                TFLOP/s against the bf16 MFMA peak; the tiny workload's
                microseconds per call (eager and from a HIP graph); with
                --extra-shapes, one GPU's share of a row- and a
                vocabulary-sharded LM head.

Inputs rotate over enough buffers (>= 1 GiB in total) that no launch finds its
rows in the 256 MB last-level cache; the in-place backward restores its logits
from a pristine copy between steps, outside the timed launch, so its lines
are timed launch by launch, each between its own pair of events (which adds
about 2 us per launch).  Every line also reports that per-launch spread
(launch_ms_*).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
ELEM = {"f32": 4, "f16": 2, "bf16": 2}


def alg_bytes(M, V, dtype, op, reduction):
    """Bytes the method must move: logits read (and the gradient or softmax
    written), int64 targets read, losses / log-sum-exps written or read."""
    s = ELEM[dtype]
    out = 4 * M if reduction == "none" else 4
    if op == "fwd":
        return M * V * s + 8 * M + out
    if op == "fwd_lse":
        return M * V * s + 8 * M + out + 4 * M
    if op == "fwd_bwd":
        return 2 * M * V * s + 8 * M + out
    if op == "bwd":                       # logits, targets, lse in; gradient out
        return 2 * M * V * s + 8 * M + 4 * M
    if op in ("softmax", "log_softmax"):
        return 2 * M * V * s
    raise ValueError(op)


OPS = ["fwd", "fwd_lse", "fwd_bwd", "bwd", "softmax", "log_softmax"]


def kernel_source_hash():
    """Hash of the sources the cross-entropy kernels are built from (the
    csrc/ce_* units and headers and the public header)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "softmax_cross_entropy_fwd_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.startswith("ce_") and name.endswith((".hip", ".h")):
            h.update(name.encode())
            h.update(open(os.path.join(csrc, name), "rb").read())
    h.update(open(os.path.join(ROOT, "include", "ce.h"), "rb").read())
    return h.hexdigest()[:16]


def traffic_path(workload, op, reduction):
    return os.path.join(ROOT, "profiles", "traffic_%s_%s_%s.txt" % (workload, op, reduction))


def load_traffic(workload, op, reduction):
    """Counter-based HBM bytes per launch from a committed rocprofv3 summary
    (key = value lines), or None when absent or taken on another kernel source."""
    path = traffic_path(workload, op, reduction)
    if not os.path.exists(path):
        return None
    d = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            d[k.strip()] = v.strip()
    if d.get("kernel_source_sha") != kernel_source_hash():
        return None
    try:
        return int(float(d["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


COPY_BYTES = 1 << 30


def calibrate_copy(log):
    """A plain device copy of known size (COPY_BYTES read, COPY_BYTES written;
    the probe library's copy_kernel), run for the counter passes: FETCH_SIZE
    and WRITE_SIZE of the CE kernel are scaled by what the same counters read
    for this copy."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "softmax_cross_entropy_fwd_amd", "libce_probe.so"))
    lib.probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                               ctypes.c_int, ctypes.c_void_p]
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    st = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        rc = lib.probe_copy(dst.data_ptr(), src.data_ptr(), COPY_BYTES, 2048, 4, st)
        assert rc == 0, rc
    torch.cuda.synchronize()
    log("calibration copy: %d bytes read and written, 3 times" % COPY_BYTES)
    del src, dst
    torch.cuda.empty_cache()


def summarize_pmc(fetch_csv, write_csv, workload, op, reduction, kernel_prefix, command):
    """Turns two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE and
    WRITE_SIZE, KiB per dispatch) into the traffic summary bench.py reads."""
    import csv
    import statistics

    def per_kernel(path, counter):
        rows = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            rows.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return rows

    f, w = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")

    def pick(d, pred):
        vals = [v for k, vs in d.items() if pred(k) for v in vs]
        return statistics.median(vals) if vals else None

    ce_kernel = lambda k: kernel_prefix in k
    is_probe_copy = lambda k: "(anonymous namespace)::copy_kernel<" in k and "native" not in k
    f_copy = pick(f, is_probe_copy)
    w_copy = pick(w, is_probe_copy)
    f_ce, w_ce = pick(f, ce_kernel), pick(w, ce_kernel)
    missing = [what for what, v in (("the calibration copy's FETCH_SIZE", f_copy),
                                    ("the calibration copy's WRITE_SIZE", w_copy),
                                    ("FETCH_SIZE of kernel '%s'" % kernel_prefix, f_ce),
                                    ("WRITE_SIZE of kernel '%s'" % kernel_prefix, w_ce))
               if v is None]
    if missing:
        raise ValueError("no counter rows for %s in %s / %s (kernels seen: %s)" % (
            ", ".join(missing), fetch_csv, write_csv, sorted(set(f) | set(w))[:8]))
    f_scale, w_scale = COPY_BYTES / f_copy, COPY_BYTES / w_copy
    hbm = f_ce * f_scale + w_ce * w_scale
    lines = [
        "# HBM traffic of the %s %s (%s) kernel, from rocprofv3 counters" % (workload, op, reduction),
        "# command: %s" % command,
        "kernel = %s" % kernel_prefix,
        "kernel_source_sha = %s" % kernel_source_hash(),
        "fetch_size_bytes_per_launch_raw = %.0f" % f_ce,
        "write_size_bytes_per_launch_raw = %.0f" % w_ce,
        "copy_fetch_raw = %.0f" % f_copy,
        "copy_write_raw = %.0f" % w_copy,
        "fetch_scale = %.4f" % f_scale,
        "write_scale = %.4f" % w_scale,
        "hbm_bytes_per_launch = %.0f" % hbm,
    ]
    return "\n".join(lines) + "\n"


def summarize_util(csv_path, workload, op, reduction, kernel_prefix, command):
    """One rocprofv3 --pmc pass of VALUBusy, TCC_HIT_sum and TCC_MISS_sum
    (counter_collection.csv) as a short summary for the kernel."""
    import csv
    import statistics
    vals = {}
    for r in csv.DictReader(open(csv_path)):
        if kernel_prefix in r["Kernel_Name"]:
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    med = {k: statistics.median(v) for k, v in vals.items()}
    hit, miss = med.get("TCC_HIT_sum", 0.0), med.get("TCC_MISS_sum", 0.0)
    lines = [
        "# VALU busy and L2 hit rate of the %s %s (%s) kernel, from rocprofv3 counters"
        % (workload, op, reduction),
        "# command: %s" % command,
        "kernel = %s" % kernel_prefix,
        "kernel_source_sha = %s" % kernel_source_hash(),
        "dispatches = %d" % len(vals.get("VALUBusy", [])),
        "valu_busy_percent = %.1f" % med.get("VALUBusy", float("nan")),
        "l2_hit_percent = %.1f" % (100.0 * hit / (hit + miss) if hit + miss else float("nan")),
    ]
    return "\n".join(lines) + "\n"


def time_workload(ce, workload, op, reduction, steps, warmup, log, M=None, V=None,
                  cpu_sample=False, min_warm_ms=0.0):
    """One operation on one workload (M and V may override its sizes, e.g. a
    shard's shape), timed with HIP events on the launch stream: around all
    `steps` launches at once, or, for the in-place backward (whose logits are
    restored between launches), around each launch.
    Warm-up: `warmup` calls, continued until they have taken `min_warm_ms`
    (the secondary lines follow seconds of host-side work, after which the
    device takes some milliseconds to come back to its steady rate: measured,
    the stress rows' forward ran 160-180 us per call for its first ~60 calls
    after a 0.5 s pause, 136 us from about the 100th on)."""
    import torch
    from softmax_cross_entropy_fwd_amd import inputs
    c = inputs.CONFIGS[workload]
    M, V, dtype = M or c["M"], V or c["V"], c["dtype"]
    dev = torch.device("cuda:0")
    x0, t = inputs.make_config(workload, device=dev, M=M, V=V)
    nbytes = x0.numel() * x0.element_size()
    # read-only ops rotate over >= 1 GiB of inputs; the others write a buffer
    # as large as the logits, which already exceeds the last-level cache
    nbuf = max(1, -(-(1 << 30) // nbytes)) if op in ("fwd", "fwd_lse") else 1
    xs = [x0] + [x0.clone() for _ in range(nbuf - 1)]
    pristine = x0.clone() if op == "fwd_bwd" else None
    out = torch.empty((M,) if reduction == "none" else (), dtype=torch.float32, device=dev)
    lse = torch.empty(M, dtype=torch.float32, device=dev)
    y = torch.empty_like(x0) if op in ("bwd", "softmax", "log_softmax") else None
    if op == "bwd":
        ce.ce_fwd_lse(x0, t, reduction, lse=lse)
    launch = {
        "fwd": lambda x: ce.ce_fwd(x, t, reduction, out=out),
        "fwd_lse": lambda x: ce.ce_fwd_lse(x, t, reduction, out=out, lse=lse),
        "fwd_bwd": lambda x: ce.ce_fwd_bwd_inplace(x, t, reduction, out=out),
        "bwd": lambda x: ce.ce_bwd(x, t, lse, reduction, grad=y),
        "softmax": lambda x: ce.ce_softmax(x, out=y),
        "log_softmax": lambda x: ce.ce_softmax(x, log_softmax=True, out=y),
    }[op]
    code = {"fwd": ce.CE_OP_FWD, "fwd_lse": ce.CE_OP_FWD, "fwd_bwd": ce.CE_OP_FWD_BWD,
            "bwd": ce.CE_OP_BWD, "softmax": ce.CE_OP_SOFTMAX,
            "log_softmax": ce.CE_OP_LOG_SOFTMAX}[op]
    stream = torch.cuda.current_stream(dev)
    plan = ce.ce_plan_describe(M, V, {"f32": 0, "f16": 1, "bf16": 2}[dtype], reduction, op=code)
    log("workload %s op %s reduction %s plan %s buffers %d" % (workload, op, reduction, plan, nbuf))
    t_warm = time.perf_counter()
    i = 0
    while i < warmup or (time.perf_counter() - t_warm) * 1e3 < min_warm_ms:
        if pristine is not None:
            xs[0].copy_(pristine)
        launch(xs[i % nbuf])
        i += 1
        if min_warm_ms and i % 8 == 0:
            torch.cuda.synchronize()   # so that the host clock follows the device
    torch.cuda.synchronize()
    region_ms = None
    if pristine is None:
        # The timed region: `steps` launches back to back between one pair of
        # HIP events on the launch stream, synchronized on both sides -- the
        # whole job's time per step.
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        r0.record(stream)
        for i in range(steps):
            launch(xs[i % nbuf])
        r1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        region_ms = r0.elapsed_time(r1) / steps
    # The same launches again, each between its own pair of events (the
    # spread per launch; the events' own packets add about 2 us to each).
    # The in-place backward restores its logits before each launch, outside
    # the launch's events: for it this pass is the timed one.
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    w1 = time.perf_counter()
    for i in range(steps):
        if pristine is not None:
            xs[0].copy_(pristine)
        starts[i].record(stream)
        launch(xs[i % nbuf])
        ends[i].record(stream)
    torch.cuda.synchronize()
    if pristine is not None:
        wall = time.perf_counter() - w1
    ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    launch_avg = sum(ms) / len(ms)
    avg_ms = region_ms if region_ms is not None else launch_avg
    med_ms = sorted(ms)[len(ms) // 2]
    ab = alg_bytes(M, V, dtype, op, reduction)
    has_loss = op in ("fwd", "fwd_lse", "fwd_bwd") and reduction != "none"
    res = {
        "workload": workload if (M, V) == (c["M"], c["V"]) else "%s_%dx%d" % (workload, M, V),
        "op": op, "reduction": reduction, "M": M, "V": V,
        "storage": dtype, "plan": plan,
        "kernel_ms_avg": avg_ms,
        "timing": "region" if region_ms is not None else "per launch",
        "launch_ms_avg": launch_avg, "launch_ms_median": med_ms, "launch_ms_min": min(ms),
        "wall_ms_per_step": 1e3 * wall / steps,
        "alg_bytes_per_launch": ab,
        "alg_GBps": ab / (avg_ms * 1e-3) / 1e9,
        "rows_per_s": M / (avg_ms * 1e-3),
        "loss": float(out.float().mean().item()) if has_loss else None,
    }
    if (M, V) == (c["M"], c["V"]):
        # HBM bytes per launch from the committed counter summary (null once
        # the kernels have changed since), and the rate they imply
        res["traffic"] = load_traffic(workload, op, reduction)
        res["counter_GBps"] = (None if res["traffic"] is None
                               else res["traffic"] / (avg_ms * 1e-3) / 1e9)
    if cpu_sample:
        res["cpu_oracle"] = oracle_sample(workload, op, reduction, M, V)
    res["frac_of_peak"] = res["alg_GBps"] / PEAK_GBS
    log("  %.4f ms/launch (min %.4f), %.1f GB/s = %.1f%% of 8 TB/s, %.3g rows/s" % (
        avg_ms, min(ms), res["alg_GBps"], 100 * res["frac_of_peak"], res["rows_per_s"]))
    del xs, pristine, x0, y
    torch.cuda.empty_cache()
    return res


PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
# warm-up of each secondary line, in milliseconds of calls (time_workload)
EXTRA_WARM_MS = 50.0


def time_linear(ce, op, steps, warmup, log, chunk=0):
    """Linear + cross-entropy on the LM-head linear workload: TFLOP/s of the
    algorithmic GEMM work (forward 2MVD; forward + backward 6MVD -- the
    backward's recomputation of the logits is not counted) over the call's
    HIP-event time, against the bf16 MFMA peak; and, for context, one plain
    bf16 GEMM of the logits (torch.matmul, the same library) timed alike."""
    import torch
    from softmax_cross_entropy_fwd_amd import inputs
    c = inputs.LINEAR_CONFIGS["lmhead_linear"]
    M, D, V = c["M"], c["D"], c["V"]
    dev = torch.device("cuda:0")
    h, w, t = inputs.make_linear(M, D, V, c["sigma"], c["seed"], device=dev)
    nbytes = int(ce.load_library().ce_linear_workspace_bytes(M, D, V, chunk))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    fn = {"fwd": lambda: ce.ce_linear_fwd(h, w, t, "mean", chunk=chunk, workspace=ws),
          "fwd_bwd": lambda: ce.ce_linear_fwd_bwd(h, w, t, "mean", chunk=chunk, workspace=ws)}[op]
    stream = torch.cuda.current_stream(dev)

    def timed(f, n, nw):
        for _ in range(nw):
            f()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for a, b in ev:
            a.record(stream)
            f()
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / n

    ms = timed(fn, steps, warmup)
    flops = (2 if op == "fwd" else 6) * M * V * D
    gemm_ms = timed(lambda: torch.matmul(h, w.t()), max(3, steps // 2), 2)
    chunk_cols = int(ce.load_library().ce_linear_chunk(M, D, V, chunk))
    res = {
        "workload": "lmhead_linear", "op": "linear_" + op, "M": M, "D": D, "V": V,
        "storage": "bf16", "chunk": chunk_cols, "workspace_MB": round(nbytes / 1e6, 1),
        "full_logits_MB": round(M * V * 2 / 1e6, 1),
        "kernel_ms_avg": ms, "alg_TFLOPs": flops / (ms * 1e-3) / 1e12,
        "logits_gemm_ms": gemm_ms, "logits_gemm_TFLOPs": 2 * M * V * D / (gemm_ms * 1e-3) / 1e12,
    }
    res["frac_of_peak"] = res["alg_TFLOPs"] / PEAK_BF16_TFLOPS
    log("linear %s: %.3f ms/call, %.1f TFLOP/s = %.1f%% of bf16 peak; one logits GEMM %.3f ms "
        "(%.1f TFLOP/s); chunk %d columns, workspace %.0f MB vs %.0f MB of bf16 logits" % (
            op, ms, res["alg_TFLOPs"], 100 * res["frac_of_peak"], gemm_ms,
            res["logits_gemm_TFLOPs"], chunk_cols, nbytes / 1e6, M * V * 2 / 1e6))
    del h, w, t, ws
    torch.cuda.empty_cache()
    return res


def measure_ceilings(log, size_bytes=None):
    """What plain kernels reach on this machine (the probe library): a read-only
    stream and a copy over 4 GiB, best of a few launch shapes, in GB/s; and,
    given the headline workload's logits size, the read over that many bytes
    (alternating between two buffers, so that each pass misses the caches)."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "softmax_cross_entropy_fwd_amd", "libce_probe.so"))
    lib.probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                               ctypes.c_int, ctypes.c_void_p]
    nb = 4 << 30
    buf = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
    buf.fill_(1)
    out = torch.empty(1 << 16, dtype=torch.float32, device="cuda:0")
    st = torch.cuda.current_stream()

    def best(fn, n=5):
        rc = fn()
        assert not isinstance(rc, int) or rc == 0, "probe launch failed: %d" % rc
        torch.cuda.synchronize()
        t = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            fn()
            b.record(st)
            torch.cuda.synchronize()
            t.append(a.elapsed_time(b))
        return min(t)

    lib.probe_read_tiles.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    tiles_out = torch.empty(2048 * 256, dtype=torch.float32, device="cuda:0")
    # (grid, tile vectors per lane, non-temporal) of the rows-pattern read:
    # persistent grids of 1-8 workgroups of 4 wavefronts per CU
    tile_shapes = [(g, k, nt) for g in (256, 512, 1024, 2048) for k in (8, 16) for nt in (0, 1)]

    def read_tiles(ptr, nbytes, g, k, nt):
        return lib.probe_read_tiles(ptr, nbytes, g, k, nt, tiles_out.data_ptr(), st.cuda_stream)

    read_plain = max(nb / best(lambda: lib.probe_read(buf.data_ptr(), nb, g, u, blk,
                                                      out.data_ptr(), st.cuda_stream)) / 1e6
                     for g, u, blk in ((1024, 8, 256), (512, 4, 1024), (2048, 8, 256)))
    read_tiles_4g = max(nb / best(lambda: read_tiles(buf.data_ptr(), nb, g, k, nt)) / 1e6
                        for g, k, nt in tile_shapes)
    # the streamed forward's pattern: whole 256 KB rows per workgroup, read in
    # chunks, one to four workgroups per CU
    lib.probe_read_rows.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    read_rows_4g = max(nb / best(lambda: lib.probe_read_rows(
        buf.data_ptr(), nb, 256 << 10, w, k, g, tiles_out.data_ptr(), st.cuda_stream)) / 1e6
        for w, k, g in ((16, 4, 256), (16, 4, 512), (8, 4, 512), (8, 4, 1024), (4, 4, 1024),
                        (16, 8, 256), (8, 8, 512)))
    # torch's own reduction over the same bytes (bf16 elements summed)
    xr = buf.view(torch.bfloat16)
    read_torch = nb / best(lambda: xr.sum(dtype=torch.float32)) / 1e6
    del xr
    read = max(read_plain, read_tiles_4g, read_rows_4g, read_torch)
    read_at_size = None
    if size_bytes and size_bytes % 16 == 0 and size_bytes <= nb // 2:
        flip = [0]

        def read_rotating(g, u, blk):
            flip[0] ^= 1
            return lib.probe_read(buf.data_ptr() + flip[0] * (nb // 2), size_bytes, g, u, blk,
                                  out.data_ptr(), st.cuda_stream)

        def tiles_rotating(g, k, nt):
            flip[0] ^= 1
            return read_tiles(buf.data_ptr() + flip[0] * (nb // 2), size_bytes, g, k, nt)
        plain_at_size = max(size_bytes / best(lambda: read_rotating(g, u, blk), n=10) / 1e6
                            for g, u, blk in ((1024, 8, 256), (512, 4, 1024), (2048, 8, 256),
                                              (256, 16, 256)))
        tiles_at_size = {(g, k, nt): size_bytes / best(lambda: tiles_rotating(g, k, nt), n=10) / 1e6
                         for g, k, nt in tile_shapes}
        best_shape = max(tiles_at_size, key=tiles_at_size.get)
        read_at_size = max(plain_at_size, tiles_at_size[best_shape])
        log("read over %d bytes: plain %.0f GB/s, rows pattern %.0f GB/s (grid %d, %d vectors "
            "per lane, non-temporal %d)" % (size_bytes, plain_at_size, tiles_at_size[best_shape],
                                           *best_shape))
    half = nb // 2
    copy = max(2 * half / best(lambda: lib.probe_copy(buf.data_ptr() + half, buf.data_ptr(), half,
                                                       g, u, st.cuda_stream)) / 1e6
               for g, u in ((4096, 104), (2048, 8), (4096, 4)))
    # in place: rows of 256 and 128 KB held in registers between read and
    # write (the fused backward's pattern without its arithmetic), and
    # torch's own in-place elementwise kernel for comparison
    lib.probe_inplace_rows.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    inplace = max(2 * nb / best(lambda: lib.probe_inplace_rows(buf.data_ptr(), nb, 16, k, g,
                                                                st.cuda_stream)) / 1e6
                  for k, g in ((16, 256), (16, 512), (8, 512)))
    xb = buf.view(torch.bfloat16)
    inplace_torch = 2 * nb / best(lambda: xb.mul_(1.0)) / 1e6
    # torch's own copy (out of place) over the same bytes, for the copy ceiling
    half_b = buf.view(torch.bfloat16)[:nb // 4]
    dst_b = buf.view(torch.bfloat16)[nb // 4:nb // 2]
    copy_torch = 2 * (nb // 2) / best(lambda: dst_b.copy_(half_b)) / 1e6
    del buf, out, xb, tiles_out, half_b, dst_b
    torch.cuda.empty_cache()
    log("measured ceilings: read %.0f GB/s (plain %.0f, rows pattern %.0f, streamed rows %.0f, "
        "torch's sum %.0f), copy %.0f GB/s (read + write; torch's copy %.0f), in place %.0f GB/s "
        "(rows in registers; torch's in-place multiply %.0f GB/s)" % (
            read, read_plain, read_tiles_4g, read_rows_4g, read_torch, copy, copy_torch, inplace,
            inplace_torch))
    if read_at_size is not None:
        log("read over the headline workload's %d bytes: %.0f GB/s" % (size_bytes, read_at_size))
    # the best read and the best read + write anything measured here reached:
    # the ceilings each line is held against (a copy, an in-place rewrite and
    # torch's kernels all move one read and one write per element)
    best_rw = max(copy, copy_torch, inplace, inplace_torch)
    return {"read_GBps": round(read, 1), "read_plain_GBps": round(read_plain, 1),
            "read_rows_pattern_GBps": round(read_tiles_4g, 1),
            "read_streamed_rows_GBps": round(read_rows_4g, 1),
            "read_torch_sum_GBps": round(read_torch, 1), "copy_GBps": round(copy, 1),
            "copy_torch_GBps": round(copy_torch, 1),
            "read_at_size_GBps": None if read_at_size is None else round(read_at_size, 1),
            "inplace_rows_GBps": round(inplace, 1), "inplace_torch_GBps": round(inplace_torch, 1),
            "best_read_GBps": round(read, 1), "best_read_write_GBps": round(best_rw, 1),
            "how": "probe/bw_probe.hip over 4 GiB (copy: 2 GiB each way; in place: 4 GiB "
                   "rewritten), best launch shape; the reads also with the rows kernel's tile "
                   "pattern over persistent grids and the streamed kernel's whole-row chunks; "
                   "torch: bf16 sum, mul_(1.0) in place and copy_ over the same bytes"}


def time_tiny(ce, log, calls=1000, cpu_sample=False, reduction="mean"):
    """The tiny workload is launch-bound: 1000 back-to-back calls timed as a
    whole, in microseconds per call."""
    import torch
    from softmax_cross_entropy_fwd_amd import inputs
    x, t = inputs.make_config("tiny", device="cuda:0")
    out = torch.empty((64,) if reduction == "none" else (), dtype=torch.float32, device="cuda:0")
    for _ in range(100):
        ce.ce_fwd(x, t, reduction, out=out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    a.record()
    for _ in range(calls):
        ce.ce_fwd(x, t, reduction, out=out)
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    us = a.elapsed_time(b) * 1e3 / calls
    # the same call captured in a HIP graph (the launch-bound case graphs are for)
    ws = torch.empty(max(1, ce.ce_workspace_bytes(64, 1000, 0, reduction)), dtype=torch.uint8,
                     device="cuda:0")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ce.ce_fwd(x, t, reduction, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(10):
            ce.ce_fwd(x, t, reduction, out=out, workspace=ws)
    for _ in range(10):
        graph.replay()
    torch.cuda.synchronize()
    a.record()
    for _ in range(calls // 10):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    gus = a.elapsed_time(b) * 1e3 / calls
    log("tiny fwd " + reduction + ": %.2f us per call over %d back-to-back calls (wall %.2f us); "
        "%.2f us per call replayed from a HIP graph of 10 calls" % (
            us, calls, wall * 1e6 / calls, gus))
    res = {"workload": "tiny", "op": "fwd", "reduction": reduction, "M": 64, "V": 1000,
           "us_per_call": us, "wall_us_per_call": wall * 1e6 / calls, "calls": calls,
           "graph_us_per_call": gus, "note": "launch-bound; no roofline claim"}
    if cpu_sample:
        # the oracle on the same inputs, on one thread and on all of them
        import oracle
        xb, tn = inputs.host_bits(x), t.cpu().numpy()
        threads = oracle.num_threads()
        for n, key in ((1, "cpu_oracle_1_thread_us"), (threads, "cpu_oracle_all_threads_us")):
            oracle.set_num_threads(n)
            reps, t0 = 0, time.perf_counter()
            while time.perf_counter() - t0 < 0.5:
                oracle.fwd(xb, tn, dtype="f32", reduction=reduction)
                reps += 1
            res[key] = (time.perf_counter() - t0) * 1e6 / reps
        oracle.set_num_threads(threads)
        res["cpu_oracle_threads"] = threads
        log("tiny on the oracle: %.1f us per call on 1 thread, %.1f us on %d" % (
            res["cpu_oracle_1_thread_us"], res["cpu_oracle_all_threads_us"], threads))
    return res


def oracle_sample(workload, op, reduction, M=None, V=None, budget_s=1.0):
    """The oracle for one line's operation on a bounded sample of its rows
    (drawn by the same generator; rows doubled until about budget_s), on all
    host threads: GB/s of the line's algorithmic bytes for those rows."""
    import oracle
    from softmax_cross_entropy_fwd_amd import inputs
    c = inputs.CONFIGS[workload]
    Mf, V, dtype = M or c["M"], V or c["V"], c["dtype"]
    rows = max(1, min(Mf, 2 ** 20 // V))
    while True:
        x, t = inputs.make_config(workload, device="cpu", M=rows, V=V)
        xb, tn = inputs.host_bits(x), t.numpy()
        t0 = time.perf_counter()
        if op in ("fwd", "fwd_lse"):
            oracle.loss_rows(xb, tn, dtype=dtype)
        elif op in ("fwd_bwd", "bwd"):
            oracle.loss_rows(xb, tn, dtype=dtype)
            oracle.grad_rows(xb, tn, dtype=dtype, c=1.0 / rows)
        else:
            oracle.softmax_rows(xb, dtype=dtype, log=op == "log_softmax")
        el = time.perf_counter() - t0
        if el >= budget_s / 4 or rows >= Mf:
            break
        rows = min(Mf, rows * 4)
    return {"value": alg_bytes(rows, V, dtype, op, reduction) / el / 1e9, "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%d rows of the line's workload, %.2f s" % (rows, el)}


def host_env():
    """Versions and the host the run used (the oracle timings depend on it)."""
    import platform
    import torch
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"device": torch.cuda.get_device_name(0), "torch": torch.__version__,
            "hip": torch.version.hip, "python": platform.python_version(),
            "cpu_model": model, "cpu_count": os.cpu_count(), "cpus_usable": usable,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline(workload, op, reduction, log, budget_s=20.0):
    """The fp64 oracle over the whole workload, repeated until ~10 s have passed
    (each pass is bounded by the budget), on every host core OpenMP gives it."""
    import numpy as np
    import torch
    import oracle
    from softmax_cross_entropy_fwd_amd import inputs
    c = inputs.CONFIGS[workload]
    M, V, dtype = c["M"], c["V"], c["dtype"]
    x, t = inputs.make_config(workload, device="cpu")
    xb, tn = inputs.host_bits(x), t.numpy()
    del x
    reps, t0 = 0, time.perf_counter()
    rows = M
    while True:
        if op == "fwd":
            oracle.fwd(xb[:rows], tn[:rows], dtype=dtype, reduction=reduction)
        else:
            oracle.grad_rows(xb[:rows], tn[:rows], dtype=dtype, c=1.0 / rows)
        reps += 1
        el = time.perf_counter() - t0
        if el >= 10.0 or el > budget_s:
            break
        if reps == 1 and el > budget_s / 4:
            break
    ab = alg_bytes(rows, V, dtype, op, reduction)
    val = ab * reps / el / 1e9
    threads = oracle.num_threads()
    log("cpu oracle: %d pass(es) over %d rows in %.2f s = %.3f GB/s on %d threads" % (
        reps, rows, el, val, threads))
    # the same on one thread, over a tenth of the rows
    oracle.set_num_threads(1)
    r1 = max(1, rows // 10)
    t0 = time.perf_counter()
    if op == "fwd":
        oracle.fwd(xb[:r1], tn[:r1], dtype=dtype, reduction=reduction)
    else:
        oracle.grad_rows(xb[:r1], tn[:r1], dtype=dtype, c=1.0 / r1)
    el1 = time.perf_counter() - t0
    oracle.set_num_threads(threads)
    val1 = alg_bytes(r1, V, dtype, op, reduction) / el1 / 1e9
    log("cpu oracle, one thread: %d rows in %.2f s = %.3f GB/s" % (r1, el1, val1))
    return {"value": val, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "the whole %s workload (%d x %d %s, %s %s), %d pass(es), %.1f s; %.3g rows/s"
                      % (workload, rows, V, dtype, op, reduction, reps, el, rows * reps / el),
            "single_thread": {"value": val1, "unit": "GB/s", "rows": r1, "seconds": el1}}


def linear_cpu_baseline(log, rows=2):
    """The oracle's linear + cross-entropy forward on a bounded sample of the
    LM-head linear workload (a few rows: each is V x D = 537M products)."""
    import torch
    import oracle
    from softmax_cross_entropy_fwd_amd import inputs
    c = inputs.LINEAR_CONFIGS["lmhead_linear"]
    M, D, V = c["M"], c["D"], c["V"]
    h, w, t = inputs.make_linear(M, D, V, c["sigma"], c["seed"])
    hb, wb = inputs.host_bits(h[:rows]), inputs.host_bits(w)
    t0 = time.perf_counter()
    oracle.linear_ce(hb, wb, t[:rows].numpy(), "none")
    el = time.perf_counter() - t0
    val = 2.0 * rows * V * D / el / 1e12
    log("cpu oracle (linear): %d rows in %.2f s = %.4f TFLOP/s" % (rows, el, val))
    return {"value": val, "unit": "TFLOP/s", "cores": min(rows, oracle.num_threads()),
            "kind": "oracle",
            "sample": "forward of %d rows of the lmhead_linear workload (%d x %d x %d bf16), %.1f s"
                      % (rows, M, D, V, el)}


def linear_main(ce, args, log):
    op = args.op or "fwd_bwd"
    if op not in ("fwd", "fwd_bwd"):
        print("lmhead_linear takes --op fwd or fwd_bwd", file=sys.stderr)
        sys.exit(2)
    steps = max(1, args.steps // 20) if args.steps == 200 else args.steps
    r = time_linear(ce, op, steps, max(1, min(args.warmup, 3)), log)
    cpu = None if args.no_cpu else linear_cpu_baseline(log)
    line = {
        "metric": "linear + CE %s TFLOP/s (algorithmic GEMM flops / call time), lmhead_linear "
                  "%dx%dx%d bf16" % (op, r["M"], r["D"], r["V"]),
        "value": round(r["alg_TFLOPs"], 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": max(1, min(args.warmup, 3)), "ms_per_step": round(r["kernel_ms_avg"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0, 1) hidden states, N(0, 4/D) weight, uniform targets)",
        "config": {"workload": "lmhead_linear", "M": r["M"], "D": r["D"], "V": r["V"],
                   "op": op, "reduction": "mean", "chunk": r["chunk"]},
        "roofline": {"bound": "mfma", "achieved": round(r["alg_TFLOPs"], 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(r["frac_of_peak"], 4), "traffic": None},
        "cpu_baseline": cpu,
        "env": host_env(),
        "also": [{k: (round(v, 5) if isinstance(v, float) else v) for k, v in r.items()}],
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # The headline's warm-up: about 40 ms of launches.  Measured on MI355X,
    # the classifier forward's region time is 84.5-86 us per launch after 20
    # warm-up launches and 82.6-82.8 us from the second 200-launch region on.
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default="classifier")
    ap.add_argument("--op", default=None, choices=[None] + OPS,
                    help="for --workload lmhead_linear: fwd or fwd_bwd")
    ap.add_argument("--reduction", default=None, choices=[None, "mean", "none", "sum"])
    ap.add_argument("--no-extra", action="store_true", help="skip the extra lines")
    ap.add_argument("--extra-shapes", action="store_true",
                    help="also time one GPU's share of a row- and a vocabulary-sharded LM head "
                         "(these share kernels with the other lines, so they are off in "
                         "profiled runs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a 1 GiB device copy first (for counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "KERNEL"),
                    help="write the traffic summary from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--pmc-command", default="", help="the profiled command, for the summary")
    ap.add_argument("--summarize-util", nargs=2, metavar=("CSV", "KERNEL"),
                    help="write the VALU-busy / L2-hit summary from one rocprofv3 --pmc run and exit")
    args = ap.parse_args()

    if args.summarize_pmc:
        from softmax_cross_entropy_fwd_amd import inputs as _inp
        c = _inp.CONFIGS[args.workload]
        op = args.op or c["ops"][0]
        red = args.reduction or c["reductions"][0]
        text = summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload, op,
                             red, args.summarize_pmc[2], args.pmc_command)
        open(traffic_path(args.workload, op, red), "w").write(text)
        print(text)
        return

    if args.summarize_util:
        from softmax_cross_entropy_fwd_amd import inputs as _inp
        c = _inp.CONFIGS[args.workload]
        op = args.op or c["ops"][0]
        red = args.reduction or c["reductions"][0]
        text = summarize_util(args.summarize_util[0], args.workload, op, red,
                              args.summarize_util[1], args.pmc_command)
        path = os.path.join(ROOT, "profiles", "util_%s_%s_%s.txt" % (args.workload, op, red))
        open(path, "w").write(text)
        print(text)
        return

    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    def log(msg):
        if not args.quiet:
            print(msg, file=sys.stderr, flush=True)

    import torch
    import softmax_cross_entropy_fwd_amd as ce
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    ce.load_library()
    from softmax_cross_entropy_fwd_amd import inputs
    if args.workload in inputs.LINEAR_CONFIGS:
        linear_main(ce, args, log)
        return
    c = inputs.CONFIGS[args.workload]
    op = args.op or c["ops"][0]
    red = args.reduction or c["reductions"][0]
    log("device: %s, torch %s, hip %s" % (torch.cuda.get_device_name(0), torch.__version__,
                                          torch.version.hip))

    if args.calibrate_copy:
        calibrate_copy(log)
    head = time_workload(ce, args.workload, op, red, args.steps, args.warmup, log)
    also = []
    if not args.no_extra and args.workload == "classifier":
        for wl, eop in (("lmhead", "fwd"), ("lmhead", "fwd_bwd"), ("lmhead", "bwd"),
                        ("lmhead", "softmax"), ("classifier", "bwd"), ("classifier", "softmax"),
                        ("stress", "fwd"), ("stress", "fwd_bwd"), ("skinny", "fwd")):
            also.append(time_workload(ce, wl, eop, "mean", max(20, args.steps // 5),
                                      max(3, args.warmup // 5), log, cpu_sample=not args.no_cpu,
                                      min_warm_ms=EXTRA_WARM_MS))
        # the skinny workload's per-row losses (reduction none: one kernel, M
        # fp32 losses written)
        also.append(time_workload(ce, "skinny", "fwd", "none", max(20, args.steps // 5),
                                  max(3, args.warmup // 5), log, cpu_sample=not args.no_cpu,
                                  min_warm_ms=EXTRA_WARM_MS))
        # the tiny workload: launch-bound, microseconds per call
        also.append(time_tiny(ce, log, cpu_sample=not args.no_cpu))
        also.append(time_tiny(ce, log, reduction="none", cpu_sample=not args.no_cpu))
        if args.extra_shapes:
            # one GPU's share of a sharded LM head: rows (M / 8) and vocabulary
            # (V / 8)
            also.append(time_workload(ce, "lmhead", "fwd", "mean", 50, 5, log, M=2048,
                                      min_warm_ms=EXTRA_WARM_MS))
            also.append(time_workload(ce, "lmhead", "fwd_bwd", "mean", 50, 5, log, M=2048,
                                      min_warm_ms=EXTRA_WARM_MS))
            also.append(time_workload(ce, "lmhead", "fwd_lse", "none", 50, 5, log, V=16384,
                                      min_warm_ms=EXTRA_WARM_MS))
        lin_cpu = None if args.no_cpu else linear_cpu_baseline(log, rows=1)
        for lop in ("fwd", "fwd_bwd"):
            also.append(time_linear(ce, lop, max(5, args.steps // 20), 2, log))
            also[-1]["cpu_oracle"] = lin_cpu
    # after the timed lines, so the 4 GiB probe buffers do not precede them
    ceilings = None if args.no_extra else measure_ceilings(
        log, c["M"] * c["V"] * inputs.ELEM_BYTES[c["dtype"]])
    if ceilings:
        # each line against the probe with its own access pattern: a read for
        # the forwards, a copy for the out-of-place writers, an in-place
        # rewrite of rows held in registers for the in-place fused backward
        # each line against the best rate measured on the box for its traffic:
        # the best read for the forwards, the best read + write (copy, in-place
        # probe, torch's copy and in-place multiply) for the writers
        ref = {"fwd": "best_read_GBps", "fwd_lse": "best_read_GBps",
               "bwd": "best_read_write_GBps", "softmax": "best_read_write_GBps",
               "log_softmax": "best_read_write_GBps", "fwd_bwd": "best_read_write_GBps"}
        for a in also:
            key = ref.get(a.get("op"))
            if key and a.get("alg_GBps") and ceilings.get(key):
                a["frac_of_probe"] = {"probe": key, "frac": a["alg_GBps"] / ceilings[key]}
    traffic = load_traffic(args.workload, op, red)
    cpu = None if args.no_cpu else cpu_baseline(args.workload, op, red, log)

    line = {
        "metric": "CE %s HBM GB/s (algorithmic bytes / kernel time), %s %dx%d %s"
                  % ({"fwd": "fwd", "fwd_bwd": "fused fwd+bwd"}.get(op, op), args.workload,
                     c["M"], c["V"], c["dtype"]),
        "value": round(head["alg_GBps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["kernel_ms_avg"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0, sigma) logits, uniform int64 targets)",
        "config": {"workload": args.workload, "M": c["M"], "V": c["V"], "storage": c["dtype"],
                   "op": op, "reduction": red, "plan": head["plan"]},
        "rows_per_s": round(head["rows_per_s"], 1),
        "wall_ms_per_step": round(head["wall_ms_per_step"], 5),
        "roofline": {"bound": "hbm", "achieved": round(head["alg_GBps"], 2), "peak": PEAK_GBS,
                     "unit": "GB/s", "frac": round(head["frac_of_peak"], 4),
                     "traffic": traffic},
        "timing": head["timing"],
        "launch_ms_avg": round(head["launch_ms_avg"], 5),
        "launch_ms_median": round(head["launch_ms_median"], 5),
        "launch_ms_min": round(head["launch_ms_min"], 5),
        "measured_ceiling": None if ceilings is None else dict(
            ceilings, frac_of_read=round(head["alg_GBps"] / ceilings["read_GBps"], 4),
            frac_of_read_at_size=(None if not ceilings.get("read_at_size_GBps") else
                                  round(head["alg_GBps"] / ceilings["read_at_size_GBps"], 4))),
        "cpu_baseline": cpu,
        "env": host_env(),
        "also": [{k: (round(v, 5) if isinstance(v, float) else v) for k, v in a.items()}
                 for a in also],
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
