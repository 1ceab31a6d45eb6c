"""Code-generation guard for the gfx950 kernels (CPU only: compiles to assembly).

Kernels whose hot loops were compiled to VALU 64-bit shifts with a per-lane
shift count (v_lshlrev_b64 / v_lshrrev_b64 vD, vS, ...) returned wrong tap
indices now and then on the MI355X, varying from run to run, while the same
source at -O1, or written with 32-bit operations, was bit-exact in every run.
The device code therefore uses 32-bit bit manipulation (funnel shifts,
bitfield extracts, v_mbcnt) throughout; this test keeps those shifts out.
"""
import os
import re
import subprocess

import pytest

from nanovdb_stencil_filtering_amd import build as B

VAR_SHIFT64 = re.compile(r"v_(?:lshl|lshr|ashr)rev_[bi]64\s+v\[\d+:\d+\],\s*v\d+,")


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    """Assembly of both HIP sources (the pipeline kernels and the device-side build)."""
    d = tmp_path_factory.mktemp("asm")
    flags = [f for f in B.HIP_FLAGS if not f.startswith("-Rpass")]
    text = []
    for src in ("vbm_kernels.hip", "vbm_build_device.hip"):
        out = str(d / (src + ".s"))
        subprocess.run([B.HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", out],
                       check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
        with open(out) as f:
            text.append(f.read())
    return "\n".join(text)


def kernels(asm):
    for name in re.findall(r"\.type\s+(\S+),@function", asm):
        start = asm.index("\n" + name + ":")
        end = asm.index(".Lfunc_end", start)
        yield name, asm[start:end]


def test_no_variable_count_64bit_vector_shifts(device_asm):
    bad = {name: len(VAR_SHIFT64.findall(body)) for name, body in kernels(device_asm)}
    bad = {k: v for k, v in bad.items() if v}
    assert not bad, bad


def test_kernels_present(device_asm):
    names = [n for n, _ in kernels(device_asm)]
    for k in ("k_decode", "k_decode_sweep", "k_taps", "k_box", "k_stencil", "k_weno", "k_meta_scatter",
              "k_build_keys", "k_fill_leaves", "k_fill_blocks"):
        assert any(k in n for n in names), k


def test_vector_sidecar_loads_are_16_bytes(device_asm):
    """The float4 path must load 16 bytes per instruction (an element-wise
    extraction of the buffer-load vector once collapsed into one dword load
    reused for all four channels).  The one dword load the split kernel may
    hold is its L2 prefetch of a later block (one dword per 128-byte line)."""
    for name, body in kernels(device_asm):
        if "k_box" in name and "ILi16ELb1E" in name and "WideSidecar" in name:
            # rows by 64-bit addresses: 16-byte global loads, no buffer resource at all
            assert "global_load_dwordx4" in body, name
            assert "buffer_load" not in body, name
        elif "k_box" in name and "ILi16ELb1E" in name:
            assert "buffer_load_dwordx4" in body, name
            dword = body.replace("buffer_load_dwordx4", "").count("buffer_load_dword ")
            assert dword <= (1 if "k_box_cached_split" in name else 0), (name, dword)
