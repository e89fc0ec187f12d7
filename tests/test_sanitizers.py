"""AddressSanitizer + UndefinedBehaviorSanitizer runs of the host code.

* The oracle's C library, built with gcc -fsanitize=address,undefined, runs
  every one of its functions on small inputs (tests/san_oracle_calls.py).
* The host side of libmoe.so (argument checks, workspace carving, launch-grid
  arithmetic) is rebuilt with the sanitizers on its host pass only
  (-Xarch_host; device code is never instrumented) for the translation units
  that hold host logic, linked with the normal objects of the kernel-only units,
  and the CPU ABI tests (tests/test_abi_cpu.py: every export, workspace sizes,
  capacities, and every invalid-argument path) run against it.

Both run in child processes with the sanitizer runtime preloaded; any report
fails the test (halt_on_error, no recovery from UB). A planted heap overflow in
either library stops its run with a sanitizer report (checked by hand when
this test was written: an off-by-one store in oracle_capacity and in
moe_capacity).
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

import pytest

pytestmark = pytest.mark.slow

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# translation units with host logic; the others only define kernels and their launchers
HOST_TUS = ("moe_abi", "dispatch", "combine", "noise", "route_hier", "bwd_misc")
SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0:detect_odr_violation=0",
    "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
}


def _report(r: subprocess.CompletedProcess) -> str:
    return f"rc={r.returncode}\n--- stdout ---\n{r.stdout[-4000:]}\n--- stderr ---\n{r.stderr[-6000:]}"


def _clean(r: subprocess.CompletedProcess) -> bool:
    text = r.stdout + r.stderr
    return r.returncode == 0 and "AddressSanitizer" not in text and "runtime error" not in text


def test_oracle_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run([gcc, "-std=c11", "-O1", "-g", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "oracle", "moe_oracle.c"), "-o", lib, "-lm"], check=True)
    env = dict(os.environ, LD_PRELOAD=asan, MOE_ORACLE_LIB=lib, OMP_NUM_THREADS="2", **SAN_ENV)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "san_oracle_calls.py")], env=env,
                       capture_output=True, text=True, timeout=600)
    assert _clean(r), _report(r)
    assert f"library {lib}" in r.stdout and r.stdout.rstrip().endswith("OK"), _report(r)


def _hipcc():
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_host_library_under_asan_ubsan(tmp_path):
    hipcc = _hipcc()
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if hipcc is None or not rt:
        pytest.skip("hipcc or clang's AddressSanitizer runtime not found")
    sys.path.insert(0, ROOT)
    from sparsely_gated_mixture_gate_amd import build as libbuild

    others = [os.path.join(libbuild.BUILD_DIR, os.path.basename(s).replace(".hip", ".o")) for s in libbuild.sources()
              if os.path.basename(s)[:-4] not in HOST_TUS]
    if not all(os.path.exists(o) for o in others):
        libbuild.build()
    san = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
                 "-fno-omit-frame-pointer"):
        san += ["-Xarch_host", flag]

    def compile_one(tu):
        obj = str(tmp_path / f"{tu}.o")
        cmd = [hipcc, *libbuild.HIPCC_FLAGS, "-g", *san, f"-I{libbuild.INCLUDE}", "-c",
               os.path.join(libbuild.CSRC, f"{tu}.hip"), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=len(HOST_TUS)) as ex:
        objs = list(ex.map(compile_one, HOST_TUS))
    lib = str(tmp_path / "libmoe_san.so")
    subprocess.run([hipcc, f"--offload-arch={libbuild.ARCH}", "-shared", "-fPIC", *objs, *others, "-o", lib], check=True)
    env = dict(os.environ, LD_PRELOAD=rt[-1], MOE_LIB=lib, **SAN_ENV)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q", "-x",
                        "-s", "-p", "no:cacheprovider", "-m", "not gpu"], env=env, cwd=ROOT, capture_output=True, text=True,
                       timeout=900)
    assert _clean(r), _report(r)
    assert " passed" in r.stdout, _report(r)
