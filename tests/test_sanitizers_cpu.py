"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
the host grid builder (vbm_build.cpp) and the oracle (oracle/oracle.cpp), both
of which walk caller arrays with plain pointer arithmetic, are compiled with
g++ -fsanitize=address,undefined and driven over coordinate sets from the
shared generators: empty, one voxel, duplicates, a random grid straddling root
tiles, a tiny shell, the decode-stress topology, one voxel per leaf, and
coordinates next to the 2^30 limit (host builder only; the oracle stops at
2^20).  Any report aborts the test program."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from conftest import ROOT
from nanovdb_stencil_filtering_amd import inputs as I

SRC = [os.path.join(ROOT, "tests", "sanitize_driver.cpp"),
       os.path.join(ROOT, "nanovdb_stencil_filtering_amd", "csrc", "vbm_build.cpp"),
       os.path.join(ROOT, "oracle", "oracle.cpp")]


def write(path, coords):
    c = np.ascontiguousarray(coords, np.int32).reshape(-1, 3)
    with open(path, "wb") as f:
        f.write(np.int64(c.shape[0]).tobytes())
        f.write(c.tobytes())
    return str(path)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_builder_and_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "sanitize_driver")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "nanovdb_stencil_filtering_amd", "csrc"),
                    *SRC, "-o", exe], check=True)
    far = (1 << 30) - 2 * 4096
    tiny = I.shell_coords(**I.TINY_SHELL)
    files = [
        write(tmp_path / "empty.bin", np.zeros((0, 3), np.int32)),
        write(tmp_path / "single.bin", np.array([[-5, 1000, 3]], np.int32)),
        write(tmp_path / "dups.bin", np.array([[1, 2, 3]] * 9 + [[-1, -2, -3]] * 4, np.int32)),
        write(tmp_path / "straddle.bin", I.random_sparse_coords(3, (18, 18, 18), 0.9, (4087, -9, -4100))),
        write(tmp_path / "tiny_shell.bin", I.shuffled(tiny, 2)),
        write(tmp_path / "stress.bin", I.leaf_bernoulli_coords(4, 600, 12, (0.02, 0.1, 0.5, 1.0))),
        write(tmp_path / "one_per_leaf.bin", I.one_per_cell_coords(5, 7)),
        write(tmp_path / "extreme.bin", (tiny.astype(np.int64) + [far, -far, far]).astype(np.int32)),
    ]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, *files], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
    assert r.stdout.count("W=") == 4 * len(files)
