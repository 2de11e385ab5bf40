"""Checks on the gfx950 code the compiler generates for the kernels (CPU only:
hipcc cross-compiles). They guard against two silent failure modes:

* an inline-asm block of transposed LDS reads whose address register is
  also one of its outputs (a read returning early would corrupt the address
  of the reads after it);
* register spills to scratch memory in the kernels.
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


def test_transposed_read_blocks_keep_their_address(tmp_path):
    asm = _device_asm("attend.hip", tmp_path)
    blocks = re.findall(r";;#ASMSTART\n(.*?);;#ASMEND", asm, re.S)
    checked = 0
    for blk in blocks:
        reads = re.findall(r"ds_read_b64_tr_b16 v\[(\d+):(\d+)\], v(\d+)", blk)
        if not reads:
            continue
        addrs = {int(a) for _, _, a in reads}
        assert len(addrs) == 1
        addr = addrs.pop()
        for lo, hi, _ in reads:
            assert not (int(lo) <= addr <= int(hi)), f"output v[{lo}:{hi}] overlaps address v{addr}"
        assert "s_waitcnt lgkmcnt(0)" in blk
        checked += 1
    assert checked > 0


@pytest.mark.parametrize("src", ["attend.hip", "select.hip", "pool.hip"])
def test_kernels_do_not_spill(src, tmp_path):
    asm = _device_asm(src, tmp_path)
    sizes = re.findall(r"\.amdhsa_private_segment_fixed_size (\d+)", asm)
    assert sizes and all(int(s) == 0 for s in sizes), sizes
