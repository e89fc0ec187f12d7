"""build() from a clean checkout: a copy of the repository's files (what git
tracks, plus new files it does not ignore) with no built library in it. The
build must compile the HIP library and the oracle there and then import the
package and load the fresh library, in a fresh interpreter. No GPU is needed:
hipcc cross-compiles for gfx950 and loading the library runs no kernel."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_build_from_clean_checkout(tmp_path):
    if shutil.which("git") is None or not os.path.isdir(os.path.join(ROOT, ".git")):
        pytest.skip("not a git checkout")
    files = subprocess.run(["git", "ls-files", "--cached", "--others", "--exclude-standard", "-z"], cwd=ROOT,
                           check=True, capture_output=True).stdout.decode().split("\0")
    dst = tmp_path / "repo"
    n = 0
    for f in files:
        if not f or f.startswith("_work/") or not os.path.isfile(os.path.join(ROOT, f)):
            continue
        os.makedirs(dst / os.path.dirname(f), exist_ok=True)
        shutil.copy2(os.path.join(ROOT, f), dst / f)
        n += 1
    assert n > 20
    assert not list(dst.rglob("*.so")), "the copy must start without built libraries"
    code = ("import __graft_entry__ as g; g.build(); "
            "import sparsely_gated_mixture_gate_amd as m, oracle; "
            "print(m.lib()._name); print(oracle.num_threads())")
    r = subprocess.run([sys.executable, "-c", code], cwd=dst, capture_output=True, text=True, timeout=900,
                       env={**os.environ, "PYTHONDONTWRITEBYTECODE": "1"})
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert str(dst / "sparsely_gated_mixture_gate_amd" / "libmoe.so") in r.stdout
    assert (dst / "oracle" / "liboracle.so").exists()
