"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every function include/vsa.h declares, its struct layout matches what a C
compiler sees, and vsa_plan / vsa_describe / argument checks behave as the
header documents."""
import ctypes
import json
import os
import re
import subprocess
import sys

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
    consts = [n for n in dir(_lib) if re.fullmatch(r"VSA_(DTYPE|ERR|SIDE)_\w+|VSA_OK", n)]
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


@pytest.mark.parametrize("lq,cq,lk,ck,prefix", [
    ((4, 10, 12), (4, 4, 4), (8, 10, 12), (4, 4, 4), 0),
    ((5, 7, 9), (3, 4, 5), (6, 5, 8), (2, 3, 3), 9),
    ((5, 9, 17), (4, 8, 8), (7, 6, 9), (2, 4, 4), 100),
])
def test_block_counts_of_both_grids_match_oracle(lq, cq, lk, ck, prefix):
    pl = vsa.plan(1, 2, 128, lq, cq, 1, prefix, latent_k=lk, cube_k=ck)
    assert np.array_equal(pl.valid_counts("q"), O.geometry(lq, cq, prefix).counts)
    gk = O.geometry(lk, ck, prefix)
    assert np.array_equal(pl.valid_counts("k"), gk.counts)
    assert pl.num_prefix_blocks_k + pl.num_blocks == gk.num_q_blocks


def test_block_counts_argument_handling():
    pl = vsa.plan(1, 2, 128, (5, 6, 7), (2, 4, 4), 3, 20)
    L = _lib.lib()
    n = L.vsa_block_counts(ctypes.byref(pl.raw), _lib.VSA_SIDE_Q, None, 0)
    assert n == pl.num_q_blocks
    buf = (ctypes.c_int32 * 4)(-7, -7, -7, -7)
    assert L.vsa_block_counts(ctypes.byref(pl.raw), _lib.VSA_SIDE_Q, buf, 3) == n   # writes 3
    assert list(buf) == list(O.geometry((5, 6, 7), (2, 4, 4), 20).counts[:3]) + [-7]
    assert L.vsa_block_counts(None, 0, None, 0) == _lib.VSA_ERR_INVALID_ARG
    assert L.vsa_block_counts(ctypes.byref(pl.raw), 2, None, 0) == _lib.VSA_ERR_INVALID_ARG
    assert L.vsa_block_counts(ctypes.byref(pl.raw), 0, None, -1) == _lib.VSA_ERR_INVALID_ARG
    assert L.vsa_block_counts(ctypes.byref(pl.raw), 0, None, 5) == _lib.VSA_ERR_INVALID_ARG


def test_plan_default_strides():
    """All-zero stride groups take the documented defaults: q contiguous,
    o like q, k and v like q on q's grid and contiguous on their own."""
    B, Hh, D, P = 2, 3, 64, 20
    pl = vsa.plan(B, Hh, D, (5, 6, 7), (2, 4, 4), 3, P)
    N = P + 5 * 6 * 7
    assert (pl.stride_b, pl.stride_h, pl.stride_n) == (Hh * N * D, N * D, D)
    assert (pl.o_stride_b, pl.o_stride_h, pl.o_stride_n) == (Hh * N * D, N * D, D)
    assert pl.kv_strides == (Hh * N * D, N * D, D)
    custom = (Hh * N * 2 * D, 2 * D, Hh * 2 * D)          # a [B, N, Hh, 2D] view
    pl = vsa.plan(B, Hh, D, (5, 6, 7), (2, 4, 4), 3, P, strides=custom)
    assert (pl.o_stride_b, pl.o_stride_h, pl.o_stride_n) == custom and pl.kv_strides == custom
    pl = vsa.plan(B, Hh, D, (5, 6, 7), (2, 4, 4), 3, P, strides=custom, latent_k=(8, 6, 7))
    Nk = P + 8 * 6 * 7
    assert pl.kv_strides == (Hh * Nk * D, Nk * D, D) and pl.seq_len_k == Nk
    assert _status(o_strides=(0, 0, 64)) == _lib.VSA_ERR_INVALID_ARG


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
    (dict(latent=(1, 1, 4097), cube=(1, 1, 1)), _lib.VSA_ERR_UNSUPPORTED),   # 4097 cubes
    (dict(latent=(1, 1, 4096), cube=(1, 1, 1)), _lib.VSA_OK),                # 4096 cubes
    (dict(strides=(64 * 512 * 2, 64 * 512, 60)), _lib.VSA_ERR_ALIGN),
    (dict(o_strides=(64 * 512 * 2, 64 * 512, 64)), _lib.VSA_ERR_INVALID_ARG),
    (dict(strides=(1 << 40, 1 << 33, 1 << 23)), _lib.VSA_ERR_OVERFLOW),
    (dict(strides=(1 << 62, 1 << 33, 1 << 20), batch=4), _lib.VSA_ERR_OVERFLOW),
    (dict(strides=(0, 128, 128)), _lib.VSA_ERR_INVALID_ARG),
    # one head's k/v span: (N - 1) * stride_n + D <= 2^31 - 32 elements
    (dict(latent=(1, 1, 2), cube=(1, 1, 1), topk=1, strides=(1 << 33, 1 << 32, 0x7FFFFF60)), _lib.VSA_OK),
    (dict(latent=(1, 1, 2), cube=(1, 1, 1), topk=1, strides=(1 << 33, 1 << 32, 0x7FFFFF68)), _lib.VSA_ERR_OVERFLOW),
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


# ---------------------------------------------------------------------------
# q and k/v on different grids; sparsity -> top-k (fastbsa package page,
# section "Use")
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("lq,cq,lk,ck,prefix", [
    ((8, 30, 52), (4, 4, 4), (16, 30, 52), (4, 4, 4), 0),
    ((4, 6, 5), (2, 2, 3), (3, 5, 7), (2, 4, 4), 0),
    ((2, 4, 4), (1, 2, 2), (4, 4, 4), (2, 2, 2), 6),
    ((31, 22, 40), (4, 8, 8), (31, 22, 40), (4, 4, 4), 64),
])
def test_plan_two_grids_match_oracle(lq, cq, lk, ck, prefix):
    pl = vsa.plan(2, 3, 128, lq, cq, 1, prefix, latent_k=lk, cube_k=ck)
    gq, gk = O.geometry(lq, cq, prefix), O.geometry(lk, ck, prefix)
    assert (pl.num_prefix_blocks, pl.num_q_blocks, pl.seq_len, pl.cube_volume) == \
        (gq.num_prefix_blocks, gq.num_q_blocks, gq.seq_len, gq.cube_volume)
    assert (pl.num_blocks, pl.num_prefix_blocks_k, pl.seq_len_k, pl.cube_volume_k, pl.nblk_k) == \
        (gk.num_blocks, gk.num_prefix_blocks, gk.seq_len, gk.cube_volume, gk.nblk)
    assert np.array_equal(pl.valid_counts("q"), gq.counts)
    assert np.array_equal(pl.valid_counts("k"), gk.counts)
    Nk = gk.seq_len
    assert pl.kv_strides == (3 * Nk * 128, Nk * 128, 128)
    assert pl.workspace_bytes == pl.kbar_offset + 2 * 3 * gk.num_blocks * 128 * 4
    assert pl.kbar_offset >= 2 * 3 * gq.num_q_blocks * 128 * 4
    assert pl.sel_elems == 2 * 3 * gq.num_q_blocks
    d = vsa.describe(pl)
    assert ("kv_seq_shape" in d) == ((lq, cq) != (lk, ck))


def test_plan_two_grids_status_codes():
    base = dict(batch=1, heads=2, head_dim=128, latent=(8, 8, 8), cube=(4, 4, 4), topk=4)
    # top-k is bounded by the key cube count, not the query cube count
    assert _status(**base, latent_k=(8, 8, 4)) == _lib.VSA_OK
    assert _status(**dict(base, topk=5), latent_k=(8, 8, 4)) == _lib.VSA_ERR_TOPK
    assert _status(**base, cube_k=(8, 16, 16)) == _lib.VSA_ERR_UNSUPPORTED
    assert _status(**base, latent_k=(8, 8, 8), kv_strides=(64 * 512, 64 * 128, 60)) == _lib.VSA_ERR_ALIGN
    pl = vsa.plan(**base)
    out = _lib.VsaPlan()
    for field, val in (("latent_k", (0, 8, 8)), ("cube_k", (4, 0, 0))):
        pr = _lib.VsaProblem.from_buffer_copy(pl.raw.p)
        getattr(pr, field)[:] = list(val)
        assert _lib.lib().vsa_plan(ctypes.byref(pr), ctypes.byref(out)) == _lib.VSA_ERR_INVALID_ARG
    pr = _lib.VsaProblem.from_buffer_copy(pl.raw.p)
    pr.kv_stride_b, pr.kv_stride_h, pr.kv_stride_n = 0, 0, 128
    assert _lib.lib().vsa_plan(ctypes.byref(pr), ctypes.byref(out)) == _lib.VSA_ERR_INVALID_ARG
    # all-zero key groups take q's values, and the plan holds them filled in
    pr = _lib.VsaProblem.from_buffer_copy(pl.raw.p)
    pr.latent_k[:], pr.cube_k[:] = [0, 0, 0], [0, 0, 0]
    pr.kv_stride_b = pr.kv_stride_h = pr.kv_stride_n = 0
    assert _lib.lib().vsa_plan(ctypes.byref(pr), ctypes.byref(out)) == _lib.VSA_OK
    assert tuple(out.p.latent_k) == (8, 8, 8) and tuple(out.p.cube_k) == (4, 4, 4)
    assert (out.p.kv_stride_b, out.p.kv_stride_h, out.p.kv_stride_n) == \
        (out.p.stride_b, out.p.stride_h, out.p.stride_n)
    assert out.num_blocks == pl.num_blocks and out.seq_len_k == out.seq_len


def test_topk_for_sparsity_matches_oracle():
    for nb in (1, 2, 7, 8, 120, 624, 960, 4096):
        for s in (0.0, 0.25, 0.5, 0.75, 0.8, 0.9, 0.9375, 0.95, 0.99, 0.999999):
            assert vsa.topk_for_sparsity(nb, s) == O.topk_for_sparsity(nb, s), (nb, s)
    L = _lib.lib()
    for nb, s in ((120, 1.0), (120, -0.01), (120, float("nan")), (0, 0.5), (-3, 0.5)):
        assert L.vsa_topk_for_sparsity(nb, s) == _lib.VSA_ERR_INVALID_ARG


# ---------------------------------------------------------------------------
# routing front end (user guide, "Wan top-k behavior" and "Verify routing
# and fallback")
# ---------------------------------------------------------------------------

def test_route_wan_log_line():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "wan_routing_log.json")))
    r = vsa.route(1, 24, 128, g["dit_seq_shape"], g["block_size"], g["topk"], checkpoint_mode=g["checkpoint_mode"])
    assert r.route == g["route"] and r.reason == _lib.VSA_REASON_NONE and r.sparse
    assert r.log_line() == (
        "FASTVIDEO_VSA routing: seq_len={seq_len}, dit_seq_shape=({0}, {1}, {2}), block_size=({3}, {4}, {5}), "
        "num_blocks={num_blocks}, topk={topk}, keep_ratio={keep_ratio}, checkpoint_mode={checkpoint_mode}, "
        "route={route}".format(*g["dit_seq_shape"], *g["block_size"], **g))
    assert r.plan.num_blocks == g["num_blocks"] and r.plan.topk == g["topk"]


@pytest.mark.parametrize("topk,mode,route,reason", [
    (64, "native", "VSA", _lib.VSA_REASON_NONE),
    (64, "dmd", "VSA", _lib.VSA_REASON_NONE),
    (1, "native", "VSA", _lib.VSA_REASON_NONE),
    (119, "native", "VSA", _lib.VSA_REASON_NONE),
    # topk == num_blocks: dense on a native checkpoint, all blocks on a DMD one
    (120, "native", "SDPA", _lib.VSA_REASON_ALL_BLOCKS_NATIVE),
    (120, "dmd", "VSA_ALL_BLOCKS", _lib.VSA_REASON_NONE),
    # topk > num_blocks: invalid for the runtime shape, dense either way
    (121, "native", "SDPA", _lib.VSA_REASON_TOPK_ABOVE_BLOCKS),
    (500, "dmd", "SDPA", _lib.VSA_REASON_TOPK_ABOVE_BLOCKS),
])
def test_route_policy(topk, mode, route, reason):
    r = vsa.route(1, 24, 128, (31, 22, 40), (4, 8, 8), topk, checkpoint_mode=mode)
    assert (r.route, r.reason) == (route, reason)
    assert r.plan is not None and r.plan.num_blocks == 120
    assert r.plan.topk == min(topk, 120)
    line = r.log_line()
    assert f"topk={topk}," in line and f"checkpoint_mode={mode}, route={route}" in line
    assert ("reason=" in line) == (reason != _lib.VSA_REASON_NONE)


def test_route_unsupported_and_errors():
    r = vsa.route(1, 24, 96, (31, 22, 40), (4, 8, 8), 64)
    assert r.route == "SDPA" and r.reason == _lib.VSA_REASON_UNSUPPORTED
    assert r.status == _lib.VSA_ERR_UNSUPPORTED and r.plan is None
    assert "unsupported" in r.log_line()
    r = vsa.route(1, 2, 128, (8, 8, 8), (4, 4, 4), 4, strides=(64 * 512 * 2, 64 * 512, 60))
    assert r.route == "SDPA" and r.status == _lib.VSA_ERR_ALIGN
    with pytest.raises(vsa.VsaError):
        vsa.route(1, 24, 128, (31, 22, 40), (4, 8, 8), 0)      # top-k must be positive
    with pytest.raises(ValueError):
        vsa.route(1, 24, 128, (31, 22, 40), (4, 8, 8), 4, checkpoint_mode="gated")
    L = _lib.lib()
    pr = vsa.plan(1, 2, 128, (8, 8, 8), (4, 4, 4), 4).raw.p
    out = _lib.VsaRoute()
    assert L.vsa_route(ctypes.byref(pr), 5, ctypes.byref(out)) == _lib.VSA_ERR_INVALID_ARG
    assert L.vsa_route(None, 0, ctypes.byref(out)) == _lib.VSA_ERR_INVALID_ARG
    assert L.vsa_describe_route(None, None, 0) == _lib.VSA_ERR_INVALID_ARG


def test_library_binds_to_the_hip_runtime_torch_uses():
    """Loading the library before torch was ever imported (here in a fresh
    process whose first act is a host-only call) still leaves a single HIP
    runtime in the process: the one torch ships, so that the library sees
    torch's device memory and streams."""
    code = ("import sys; sys.path.insert(0, sys.argv[1])\n"
            "import block_sparse_attention_raster_amd as vsa\n"
            "from block_sparse_attention_raster_amd import _lib\n"
            "vsa.plan(1, 2, 128, (5, 6, 7), (2, 4, 4), 3)\n"
            "import torch, os\n"
            "rt = _lib.hip_runtimes_mapped()\n"
            "assert len(rt) == 1, rt\n"
            "assert os.path.dirname(next(iter(rt))) == os.path.realpath(os.path.join(os.path.dirname(torch.__file__), 'lib')), rt\n"
            "print('one runtime')\n")
    r = subprocess.run([sys.executable, "-c", code, ROOT], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "one runtime" in r.stdout, (r.stdout[-2000:], r.stderr[-2000:])
