"""vsa_forward_noalloc, the allocation-free entry point (for callers that
cannot allocate device memory): through the C ABI it must give what
vsa_forward gives with a caller workspace, bit for bit (the same kernels),
on consecutive calls whose problems shrink (the fixed scratch array keeps
the previous call's contents), and it must refuse a problem whose pooled
means exceed the array before any device work."""
import ctypes

import numpy as np
import pytest

import block_sparse_attention_raster_amd as vsa
from block_sparse_attention_raster_amd import _lib

SCRATCH_BYTES = 32 << 20


def test_noalloc_refuses_problems_beyond_its_scratch():
    """Host-side: 32 heads of the (16, 46, 80) grid in (4, 4, 4) cubes need
    31.5 MB of pooled means (fits in 32 MiB); 35 heads need 34.4 MB."""
    L = _lib.lib()
    fits = vsa.plan(1, 32, 128, (16, 46, 80), (4, 4, 4), 60)
    over = vsa.plan(1, 35, 128, (16, 46, 80), (4, 4, 4), 60)
    assert fits.workspace_bytes <= SCRATCH_BYTES < over.workspace_bytes
    dummy = ctypes.c_void_p(16)   # never dereferenced: the size check comes first
    assert L.vsa_forward_noalloc(ctypes.byref(over.raw), dummy, dummy, dummy, dummy, dummy, None) == \
        _lib.VSA_ERR_SCRATCH
    assert "scratch" in _lib.status_str(_lib.VSA_ERR_SCRATCH)
    assert L.vsa_forward_noalloc(ctypes.byref(fits.raw), None, None, None, None, None, None) == \
        _lib.VSA_ERR_INVALID_ARG


def _problem(seed, B, Hh, latent, cube, topk, prefix):
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    N = prefix + latent[0] * latent[1] * latent[2]
    q, k, v = (torch.randn((B, Hh, N, 128), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
    pl = vsa.plan_for(q, latent, cube, topk, prefix)
    return pl, q, k, v


def _run(entry, pl, q, k, v):
    import torch
    sel = torch.full((pl.sel_elems,), -1, dtype=torch.int32, device="cuda")
    out = torch.zeros_like(q)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    L = _lib.lib()
    if entry == "noalloc":
        rc = L.vsa_forward_noalloc(ctypes.byref(pl.raw), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                   sel.data_ptr(), out.data_ptr(), st)
    else:
        ws = torch.empty(pl.workspace_bytes, dtype=torch.uint8, device="cuda")
        rc = L.vsa_forward(ctypes.byref(pl.raw), q.data_ptr(), k.data_ptr(), v.data_ptr(), ws.data_ptr(),
                           sel.data_ptr(), out.data_ptr(), st)
    assert rc == _lib.VSA_OK, _lib.status_str(rc)
    torch.cuda.synchronize()
    return sel, out


@pytest.mark.gpu
def test_noalloc_matches_forward_on_consecutive_shrinking_calls():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    problems = [
        # nearly the whole array (31.5 MB of pooled means), 64-token cubes
        dict(seed=81, B=1, Hh=32, latent=(16, 46, 80), cube=(4, 4, 4), topk=60, prefix=0),
        # the Wan-shaped call, 256-token cubes
        dict(seed=83, B=1, Hh=24, latent=(31, 22, 40), cube=(4, 8, 8), topk=64, prefix=0),
        # much smaller, 64-token cubes with a prefix: reads only what it wrote
        dict(seed=82, B=2, Hh=3, latent=(6, 7, 9), cube=(4, 4, 4), topk=5, prefix=100),
    ]
    for p in problems:
        pl, q, k, v = _problem(**p)
        assert pl.workspace_bytes <= SCRATCH_BYTES
        print(f"[gpu-case] noalloc: B={p['B']} Hh={p['Hh']} grid={p['latent']} cube={p['cube']} "
              f"topk={p['topk']} P={p['prefix']} workspace={pl.workspace_bytes}", flush=True)
        sel_a, out_a = _run("noalloc", pl, q, k, v)
        sel_b, out_b = _run("forward", pl, q, k, v)
        assert torch.equal(sel_a, sel_b)
        assert torch.equal(out_a, out_b)
        assert bool(torch.isfinite(out_a.float()).all())
        del q, k, v
