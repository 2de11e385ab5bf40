"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every function include/vsa.h declares, its struct layout matches what a C
compiler sees, and vsa_plan / vsa_describe / argument checks behave as the
header documents."""
import ctypes
import json
import os
import re
import subprocess

import numpy as np
import pytest

import block_sparse_attention_raster_amd as vsa
from block_sparse_attention_raster_amd import _lib
from oracle import vsa_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vsa.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(vsa_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_entry_points():
    assert _declared_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_function():
    L = _lib.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_struct_layout_matches_c(tmp_path):
    fields_p = [f[0] for f in _lib.VsaProblem._fields_]
    fields_l = [f[0] for f in _lib.VsaPlan._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "vsa.h"', "int main(void){",
             'printf("%zu %zu\\n", sizeof(vsa_problem), sizeof(vsa_plan_t));']
    lines += [f'printf("p {f} %zu\\n", offsetof(vsa_problem, {f}));' for f in fields_p]
    lines += [f'printf("l {f} %zu\\n", offsetof(vsa_plan_t, {f}));' for f in fields_l]
    consts = [n for n in dir(_lib) if re.fullmatch(r"VSA_(DTYPE|ERR)_\w+|VSA_OK", n)]
    lines += [f'printf("c {n} %d\\n", (int){n});' for n in consts]
    lines.append("return 0;}")
    c = tmp_path / "layout.c"
    c.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.dirname(HEADER), str(c), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    sp, sl = (int(x) for x in out[0].split())
    assert sp == ctypes.sizeof(_lib.VsaProblem) and sl == ctypes.sizeof(_lib.VsaPlan)
    for line in out[1:]:
        if not line:
            continue
        kind, name, off = line.split()
        if kind == "c":
            assert getattr(_lib, name) == int(off), name
            continue
        cls = _lib.VsaProblem if kind == "p" else _lib.VsaPlan
        assert getattr(cls, name).offset == int(off), name


def test_plan_wan_routing_fields():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "wan_routing_log.json")))
    pl = vsa.plan(1, 24, 128, g["dit_seq_shape"], g["block_size"], g["topk"])
    assert pl.num_blocks == g["num_blocks"]
    assert pl.seq_len == g["seq_len"]
    assert pl.nblk == (8, 3, 5)
    assert pl.num_prefix_blocks == 0 and pl.num_q_blocks == 120 and pl.cube_volume == 256
    assert vsa.describe(pl) == (
        "seq_len={seq_len}, dit_seq_shape=({0}, {1}, {2}), block_size=({3}, {4}, {5}), "
        "num_blocks={num_blocks}, topk={topk}, keep_ratio={keep_ratio}".format(
            *g["dit_seq_shape"], *g["block_size"], **g))
    assert pl.scale == pytest.approx(128 ** -0.5, rel=1e-7)
    assert pl.sel_elems == 24 * 120 * 64
    assert pl.workspace_bytes == 4 * 128 * 24 * 240 and pl.kbar_offset == 4 * 128 * 24 * 120


@pytest.mark.parametrize("latent,cube,prefix", [
    ((31, 22, 40), (4, 8, 8), 0), ((16, 46, 80), (4, 4, 4), 0), ((21, 30, 52), (4, 4, 4), 512),
    ((5, 6, 7), (2, 4, 4), 20), ((3, 5, 7), (4, 8, 8), 0), ((8, 8, 8), (4, 4, 4), 0),
])
def test_plan_geometry_matches_oracle(latent, cube, prefix):
    pl = vsa.plan(2, 3, 64, latent, cube, 1, prefix)
    g = O.geometry(latent, cube, prefix)
    assert (pl.num_blocks, pl.num_prefix_blocks, pl.num_q_blocks, pl.seq_len) == \
        (g.num_blocks, g.num_prefix_blocks, g.num_q_blocks, g.seq_len)
    assert np.array_equal(pl.valid_counts(), g.counts)


def _status(**kw):
    base = dict(batch=1, heads=2, head_dim=128, latent=(8, 8, 8), cube=(4, 4, 4), topk=4, prefix_len=0)
    base.update(kw)
    try:
        vsa.plan(**base)
        return _lib.VSA_OK
    except vsa.VsaError as e:
        return e.status


@pytest.mark.parametrize("kw,status", [
    (dict(), _lib.VSA_OK),
    (dict(topk=0), _lib.VSA_ERR_TOPK),
    (dict(topk=-3), _lib.VSA_ERR_TOPK),
    (dict(topk=9), _lib.VSA_ERR_TOPK),
    (dict(topk=8), _lib.VSA_OK),
    (dict(batch=0), _lib.VSA_ERR_INVALID_ARG),
    (dict(heads=-1), _lib.VSA_ERR_INVALID_ARG),
    (dict(latent=(0, 8, 8)), _lib.VSA_ERR_INVALID_ARG),
    (dict(cube=(4, 0, 4)), _lib.VSA_ERR_INVALID_ARG),
    (dict(prefix_len=-1), _lib.VSA_ERR_INVALID_ARG),
    (dict(head_dim=96), _lib.VSA_ERR_UNSUPPORTED),
    (dict(head_dim=64), _lib.VSA_OK),
    (dict(cube=(8, 16, 16)), _lib.VSA_ERR_UNSUPPORTED),
    (dict(latent=(200, 200, 200), cube=(1, 1, 1)), _lib.VSA_ERR_UNSUPPORTED),
    (dict(strides=(64 * 512 * 2, 64 * 512, 60)), _lib.VSA_ERR_ALIGN),
    (dict(o_strides=(64 * 512 * 2, 64 * 512, 64)), _lib.VSA_ERR_INVALID_ARG),
    (dict(strides=(1 << 40, 1 << 33, 1 << 23)), _lib.VSA_ERR_OVERFLOW),
    (dict(strides=(1 << 62, 1 << 33, 1 << 20), batch=4), _lib.VSA_ERR_OVERFLOW),
    (dict(strides=(0, 128, 128)), _lib.VSA_ERR_INVALID_ARG),
])
def test_plan_status_codes(kw, status):
    assert _status(**kw) == status


def test_plan_dtypes_and_null():
    pr = _lib.VsaProblem()
    out = _lib.VsaPlan()
    assert _lib.lib().vsa_plan(None, ctypes.byref(out)) == _lib.VSA_ERR_INVALID_ARG
    assert _lib.lib().vsa_plan(ctypes.byref(pr), None) == _lib.VSA_ERR_INVALID_ARG
    pl = vsa.plan(1, 2, 64, (8, 8, 8), (4, 4, 4), 4)
    assert pl.dtype == _lib.VSA_DTYPE_BF16
    assert vsa.plan(1, 2, 64, (8, 8, 8), (4, 4, 4), 4, dtype="f16").dtype == _lib.VSA_DTYPE_F16
    with pytest.raises(ValueError):
        vsa.plan(1, 2, 64, (8, 8, 8), (4, 4, 4), 4, dtype="f32")
    pr = pl.raw.p
    for dt, want in ((_lib.VSA_DTYPE_F16, _lib.VSA_OK), (7, _lib.VSA_ERR_UNSUPPORTED),
                     (-1, _lib.VSA_ERR_UNSUPPORTED)):
        pr.dtype = dt
        assert _lib.lib().vsa_plan(ctypes.byref(pr), ctypes.byref(out)) == want


def test_entry_points_check_arguments_before_touching_a_device():
    L = _lib.lib()
    pl = vsa.plan(1, 2, 64, (8, 8, 8), (4, 4, 4), 4)
    p = ctypes.byref(pl.raw)
    assert L.vsa_select(None, 16, 16, 256, 16, None) == _lib.VSA_ERR_INVALID_ARG
    assert L.vsa_select(p, None, 16, 256, 16, None) == _lib.VSA_ERR_INVALID_ARG
    assert L.vsa_select(p, 16, 16, 128, 16, None) == _lib.VSA_ERR_ALIGN       # workspace not 256-aligned
    assert L.vsa_attend(p, 16, 16, 16, None, 16, None) == _lib.VSA_ERR_INVALID_ARG
    assert L.vsa_attend(p, 16, 16, 8, 16, 16, None) == _lib.VSA_ERR_ALIGN
    assert L.vsa_forward(p, 16, 16, 16, 256, None, 16, None) == _lib.VSA_ERR_INVALID_ARG
    # an edited plan is refused
    bad = _lib.VsaPlan.from_buffer_copy(pl.raw)
    bad.num_blocks = 3
    assert L.vsa_attend(ctypes.byref(bad), 16, 16, 16, 16, 16, None) == _lib.VSA_ERR_INVALID_ARG
    bad = _lib.VsaPlan.from_buffer_copy(pl.raw)
    bad.p.topk = 99
    assert L.vsa_select(ctypes.byref(bad), 16, 16, 256, 16, None) == _lib.VSA_ERR_TOPK


def test_describe_truncates_and_reports_length():
    pl = vsa.plan(1, 24, 128, (31, 22, 40), (4, 8, 8), 64)
    full = vsa.describe(pl)
    buf = ctypes.create_string_buffer(10)
    n = _lib.lib().vsa_describe(ctypes.byref(pl.raw), buf, 10)
    assert n == len(full) and buf.value.decode() == full[:9]
    assert _lib.lib().vsa_describe(ctypes.byref(pl.raw), None, 0) == len(full)


def test_status_strings():
    for s in range(-7, 1):
        assert _lib.status_str(s) not in ("", "unknown status")
    assert _lib.status_str(-99) == "unknown status"
