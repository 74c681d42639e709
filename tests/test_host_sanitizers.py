"""The host side under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only): the fp64 oracle (oracle/ce_oracle.c) and the library's host logic --
argument checks, plans, workspace layout, the linear path's checks
(csrc/ce_api.hip, csrc/lce_api.hip; host code instrumented, device code as
usual, the kernel units unchanged) -- are built with both sanitizers, and
the CPU test suite (the oracle pins, every argument-error path of the C ABI,
the host logic of the bench) runs against them in a child process with the
sanitizer runtime preloaded.  Any report fails the test.

Built with the ROCm clang, whose ASan runtime also carries the UBSan
handlers, so one runtime serves both libraries.  The child sets CE_LIBRARY
and ORACLE_LIBRARY to the sanitized builds and SANITIZED_CHILD so that this
test does not run again inside it."""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = "/opt/rocm/lib/llvm"
CLANG = os.path.join(LLVM, "bin", "clang")
HIPCC = "/opt/rocm/bin/hipcc"
RUNTIME = glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux",
                                 "libclang_rt.asan-x86_64.so"))
# host-side instrumentation only: each sanitizer flag right after -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]
HOST_UNITS = ("ce_api.hip", "lce_api.hip")

pytestmark = pytest.mark.skipif(
    os.environ.get("SANITIZED_CHILD") == "1" or not RUNTIME or not os.path.exists(CLANG),
    reason="inside the sanitized run, or no sanitizer runtime")


def build_oracle(out):
    src = os.path.join(ROOT, "oracle", "ce_oracle.c")
    lib = os.path.join(out, "libce_oracle_san.so")
    cmd = [CLANG, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-shared-libasan", "-Wl,-rpath," + os.path.join(LLVM, "lib"),
           src, "-o", lib, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)
    return lib


def build_library(out):
    from softmax_cross_entropy_fwd_amd import build as b
    if not all(os.path.exists(os.path.join(b.BUILD, os.path.basename(s) + ".o"))
               for s in glob.glob(os.path.join(b.CSRC, "*.hip"))):
        b.build()

    def host_unit(name):
        obj = os.path.join(out, name + ".san.o")
        cmd = [HIPCC] + b.CFLAGS + HOST_SAN + ["-c", os.path.join(b.CSRC, name), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj

    with cf.ThreadPoolExecutor(len(HOST_UNITS)) as ex:
        objs = list(ex.map(host_unit, HOST_UNITS))
    objs += [o for o in glob.glob(os.path.join(b.BUILD, "*.hip.o"))
             if os.path.basename(o)[:-len(".hip.o")] + ".hip" not in HOST_UNITS
             and not os.path.basename(o).startswith("bw_probe")]
    lib = os.path.join(out, "libce_san.so")
    subprocess.run([HIPCC, "--offload-arch=" + b.ARCH, "-shared", "-fPIC"] + objs +
                   ["-L" + b.ROCM_LIB, "-lrocblas", "-o", lib], check=True, capture_output=True)
    return lib


def test_cpu_suite_under_asan_and_ubsan(tmp_path):
    with cf.ThreadPoolExecutor(2) as ex:
        fo = ex.submit(build_oracle, str(tmp_path))
        fl = ex.submit(build_library, str(tmp_path))
        oracle_lib, ce_lib = fo.result(), fl.result()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": RUNTIME[0],
        # Python and torch keep memory to the end by design: leaks are not checked
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "CE_LIBRARY": ce_lib,
        "ORACLE_LIBRARY": oracle_lib,
        "SANITIZED_CHILD": "1",
        "OMP_NUM_THREADS": "2",
    })
    # the child process maps the sanitized builds, not the default ones
    probe = ("import softmax_cross_entropy_fwd_amd as ce, oracle; ce.load_library(); "
             "oracle._load(); print(open('/proc/self/maps').read())")
    m = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert m.returncode == 0, (m.stdout + m.stderr)[-4000:]
    assert ce_lib in m.stdout and oracle_lib in m.stdout and "libclang_rt.asan" in m.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-x", "-q",
                        "-m", "not gpu", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1500)
    log = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in log, log[-6000:]
    assert "runtime error:" not in log, log[-6000:]
    assert r.returncode == 0, log[-6000:]
    assert "passed" in r.stdout
