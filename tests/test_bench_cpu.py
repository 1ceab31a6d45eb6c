"""bench.py's bookkeeping, checked on the CPU: the refusal of several GPUs, the
algorithmic-byte models behind roofline.achieved, and the rule that HBM counters
are reported only for the kernel sources they were taken on."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# cfg-shell (R = 185, |d| <= 1.5): active voxels, leaves, blocks at BlockWidth 128
N, L, NB128 = 1290538, 11255, 10083


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_several_gpus_are_refused_before_any_device_use():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_filter_bytes_count_each_row_once():
    b = load_bench()
    # per active voxel: its own C-channel fp32 row read once and its output row
    # written once; plus 92 B per leaf record and 4 + W/8 B per block
    own_rows = 2 * 4 * 16 * N
    assert b.alg_bytes_filter(N, L, NB128, 128, 16) == own_rows + 92 * L + (4 + 16) * NB128
    assert b.alg_bytes_filter(N, L, NB128, 128, 16) == 166425984
    # channels scale only the row term
    assert b.alg_bytes_filter(N, L, NB128, 128, 1) == 2 * 4 * N + 92 * L + 20 * NB128


def test_decode_bytes():
    b = load_bench()
    # u32 leaf index + u16 voxel offset per slot (sentinel slots included)
    assert b.alg_bytes_decode(N, L, NB128, 128) == 6 * NB128 * 128 + 80 * L + 20 * NB128 == 8845804


def test_committed_profile_states_the_same_algorithmic_bytes():
    b = load_bench()
    kv = dict(line.split(": ", 1) for line in open(b.PROFILE).read().splitlines() if ": " in line)
    assert int(kv["algorithmic_bytes_per_launch"]) == b.alg_bytes_filter(N, L, NB128, 128, 16)


def test_counters_only_for_the_sources_they_were_taken_on(tmp_path):
    b = load_bench()
    good = tmp_path / "good.txt"
    good.write_text("sources_sha256: %s\ntraffic_bytes_per_launch: 123456\n" % b.kernel_sources_sha256())
    assert b.counted_traffic(str(good)) == 123456
    stale = tmp_path / "stale.txt"
    stale.write_text("sources_sha256: %s\ntraffic_bytes_per_launch: 123456\n" % ("0" * 64))
    assert b.counted_traffic(str(stale)) is None
    assert b.counted_traffic(str(tmp_path / "missing.txt")) is None


def test_headline_kernel_names():
    b = load_bench()
    assert b.headline_kernel(16) == "k_box_cached_split<16, true, Sidecar>"
    assert b.headline_kernel(8) == "k_box_cached_split<8, true, Sidecar>"
    assert b.headline_kernel(1) == "k_box_cached<1, false, true, Sidecar>"
