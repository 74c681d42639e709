"""Build the HIP library libce.so for gfx950, in-tree.

    python -m softmax_cross_entropy_fwd_amd.build [-v]

Each csrc/*.hip unit is compiled to an object in parallel, then linked into
softmax_cross_entropy_fwd_amd/libce.so (with rocBLAS, for the GEMMs of the
linear + cross-entropy path); probe/bw_probe.hip (HBM bandwidth
probes for the bench) goes into libce_probe.so.  Packed-fp32 VALU forms are disabled
for device code; no fast-math, so fp32 rounding and denormals follow IEEE.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libce.so")
PROBE_SRC = os.path.join(PKG, "probe", "bw_probe.hip")
PROBE_LIB = os.path.join(PKG, "libce_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM_LIB = "/opt/rocm/lib"
ARCH = "gfx950"

CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src, verbose, defines=(), build_dir=None):
    obj = os.path.join(build_dir or BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + CFLAGS + ["-D" + d for d in defines] + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
    if out.strip() and verbose:
        print(out)
    return obj


def build(verbose=False, jobs=None, defines=(), out=None):
    """Compile csrc/ into libce.so (or `out`, with extra -D `defines`, for
    experiments; the probes are only built for the default library)."""
    build_dir = BUILD if not defines else BUILD + "_" + "_".join(d.replace("=", "") for d in defines)
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, defines, build_dir), srcs))
    lib = out or LIB
    tmp = lib + ".tmp%d" % os.getpid()
    # rocBLAS serves the plain GEMMs of the linear + cross-entropy path
    cmd = ([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs +
           ["-L" + ROCM_LIB, "-lrocblas", "-o", tmp])
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    if out:
        return out
    # the bandwidth probes the bench measures the ceiling with (own library)
    pobj = _compile(PROBE_SRC, verbose)
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", pobj, "-o", tmp],
                   check=True)
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    args = sys.argv[1:]
    defs = [a[2:] for a in args if a.startswith("-D")]
    outs = [a[6:] for a in args if a.startswith("--out=")]
    print(build(verbose="-v" in args, defines=defs, out=outs[0] if outs else None))
