"""Checks on the gfx950 code the compiler generates for the kernels (CPU only:
hipcc cross-compiles). They guard against silent failure modes:

* register spills to scratch memory in the kernels (a reload's vmcnt wait
  would also wait for every global-to-LDS copy in flight);
* global-to-LDS and buffer-to-LDS copies written as inline asm without
  their M0 set.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_raster_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")

pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not available")


def _device_asm(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _blocks(asm):
    """Basic blocks as lists of instruction lines."""
    out, cur = [], []
    for line in asm.split("\n"):
        if re.match(r"^(\.LBB\w+|; %bb\.\d+):", line) or line.startswith(".Lfunc_end"):
            out.append(cur)
            cur = []
            continue
        t = line.strip()
        if t and not t.startswith(";") and not t.startswith("."):
            cur.append(t)
    out.append(cur)
    return out


def test_lds_copies_set_m0(tmp_path):
    asm = _device_asm("attend.hip", tmp_path)
    checked = {"global": 0, "buffer": 0}
    for blk in _blocks(asm):
        m0_set = False
        for i in blk:
            if re.match(r"s_\w+ m0,", i):
                m0_set = True
            kind = ("global" if i.startswith("global_load_lds_dwordx4") else
                    "buffer" if re.match(r"buffer_load_dwordx4 .* lds$", i) else None)
            if kind:
                assert m0_set, f"{i}: LDS copy without M0 set in its block"
                checked[kind] += 1
    assert checked["global"] > 0 and checked["buffer"] > 0, checked


@pytest.mark.parametrize("src", ["attend.hip", "select.hip", "pool.hip"])
def test_kernels_do_not_spill(src, tmp_path):
    asm = _device_asm(src, tmp_path)
    sizes = re.findall(r"\.amdhsa_private_segment_fixed_size (\d+)", asm)
    assert sizes and all(int(s) == 0 for s in sizes), sizes
