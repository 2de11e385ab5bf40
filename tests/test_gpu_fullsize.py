"""GPU parity at full size, every output row: the HIP path (through the C
ABI) against the CPU oracle's dense-masked attention ("fastbsa" package
page, section "How it works": outputs are validated against dense-masked
attention), recomputed under the GPU's own selection for every query block
of the checked (batch, head) pairs, in worker processes (one per host core).
Each query block must meet the tolerance on its own (relative L2 over its
rows), so an error confined to a few blocks, or to the rows of one
workgroup, cannot hide in the average.

Also here: the routing front end's plans run on the kernels ("FastVideo
VSA" user guide, section "Wan top-k behavior"), the two halves of selection
against the whole, and the binding's refusal of host buffers.
"""
import sys

import numpy as np
import pytest

from block_sparse_attention_raster_amd import synthetic
from oracle import parallel as OP
from oracle import vsa_oracle as O
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def _announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _run(w, topk, dtype="bf16"):
    """One forward on cuda:0; returns the input bits, the GPU's selection
    (int64) and its output bits."""
    import torch
    import block_sparse_attention_raster_amd as vsa
    bits = synthetic.make_inputs(w, dtype=dtype)
    q, k, v = (G.to_device(x, dtype) for x in bits)
    pl = vsa.plan_for(q, w.latent, w.cube, topk, w.prefix_len)
    sel, _ = vsa.select(pl, q, k)
    out = vsa.attend(pl, q, k, v, sel)
    torch.cuda.synchronize()
    out_bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return bits, sel.cpu().numpy().astype(np.int64), out_bits


def _every_block(w, topk, pairs, dtype="bf16"):
    _announce(f"{w.name}: every block of {len(pairs)} (batch, head) pairs, topk={topk}, dtype={dtype}")
    bits, sel, out_bits = _run(w, topk, dtype)
    g, _, _, scores = G.oracle_scores(w, bits[0], bits[1], dtype)
    chk = O.check_selection(sel, scores, topk, band=G.TIE_BAND)
    assert chk["mismatch_rows"] == [], f"selection mismatches in rows {chk['mismatch_rows'][:10]}"
    jobs = OP.head_jobs((*bits, out_bits), pairs, sel=sel, dtype=dtype, latent=w.latent, cube=w.cube,
                        prefix_len=w.prefix_len)
    res = OP.map_jobs(OP.check_head, jobs)
    tol = G.TOL[dtype]
    worst_whole = max(r["whole"]["rel_l2"] for r in res)
    worst_max = max(r["whole"]["max_abs"] for r in res)
    worst_block = max(r["per_block"][r["worst_block"]]["rel_l2"] for r in res)
    n_blocks = sum(r["blocks"] for r in res)
    _announce(f"{w.name}/topk{topk}/{dtype}: {n_blocks} blocks, band rows {chk['band_rows']} of {chk['rows']}, "
              f"max_abs {worst_max:.3e}, rel_l2 per head <= {worst_whole:.3e}, per block <= {worst_block:.3e}")
    for (b, h), r in zip(pairs, res):
        assert r["finite"], (b, h)
        assert r["blocks"] == g.num_q_blocks
        assert r["whole"]["max_abs"] <= tol["max_abs"], ((b, h), r["whole"])
        assert r["whole"]["rel_l2"] <= tol["rel_l2"], ((b, h), r["whole"])
        bad = {i: e for i, e in r["per_block"].items() if e["rel_l2"] > tol["rel_l2"]}
        assert not bad, ((b, h), dict(list(bad.items())[:5]))


def test_wan_every_output_row():
    """The 8-wave tiling (256-token cubes): all 24 heads, all 120 blocks."""
    w = synthetic.WORKLOADS["wan"]
    _every_block(w, w.topk, [(0, h) for h in range(w.heads)])


def test_prefix_every_block_of_sixteen_heads():
    """The 2-wave tiling (64-token cubes) with an always-kept prefix: every
    block of 16 of the 48 (batch, head) pairs, both batches."""
    w = synthetic.WORKLOADS["prefix"]
    _every_block(w, w.topk, [(b, h) for b in range(w.batch) for h in range(0, w.heads, 3)])


# ---------------------------------------------------------------------------
# the routing front end's plans on the kernels (user guide, "Wan top-k
# behavior": a DMD checkpoint with top-k equal to the block count stays on
# the all-block path; top-k below it is the VSA route)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("topk,mode,route", [(12, "dmd", "VSA_ALL_BLOCKS"), (5, "native", "VSA"),
                                             (5, "dmd", "VSA")])
def test_route_plans_run_on_the_kernels(topk, mode, route):
    import torch
    import block_sparse_attention_raster_amd as vsa
    w = synthetic.custom_workload(f"route_{mode}_{topk}", seed=61 + topk, batch=1, heads=2, head_dim=128,
                                  latent=(9, 10, 11), cube=(4, 8, 8), topk=topk)
    r = vsa.route(w.batch, w.heads, w.head_dim, w.latent, w.cube, topk, checkpoint_mode=mode)
    _announce(r.log_line())
    assert r.route == route and r.sparse and r.plan is not None
    assert r.plan.num_blocks == 12
    bits = synthetic.make_inputs(w)
    q, k, v = (G.to_device(x) for x in bits)
    sel, _ = vsa.select(r.plan, q, k)
    out = vsa.attend(r.plan, q, k, v, sel)
    torch.cuda.synchronize()
    got, sel = G.from_device(out), sel.cpu().numpy().astype(np.int64)
    g, _, _, scores = G.oracle_scores(w, bits[0], bits[1])
    assert O.check_selection(sel, scores, topk, band=G.TIE_BAND)["mismatch_rows"] == []
    for h in range(w.heads):
        qf, kf, vf = (O.decode_bf16(x[0, h]) for x in bits)
        if route == "VSA_ALL_BLOCKS":   # every block kept: plain dense attention
            assert np.array_equal(sel[0, h], np.tile(np.arange(12), (g.num_q_blocks, 1)))
            L = (qf @ kf.T) / np.sqrt(w.head_dim)
            P = np.exp(L - L.max(axis=1, keepdims=True))
            ref = (P / P.sum(axis=1, keepdims=True)) @ vf
        else:
            ref = O.attend_dense_masked(qf, kf, vf, sel[0, h], g)
        e = O.error_norms(got[0, h], ref)
        assert e["max_abs"] <= G.MAX_ABS and e["rel_l2"] <= G.REL_L2, (h, e)


def test_dense_routes_run_nothing():
    """The dense routes hand the call back to the caller: top-k equal to the
    block count on a native checkpoint, and top-k above it."""
    import block_sparse_attention_raster_amd as vsa
    r = vsa.route(1, 2, 128, (9, 10, 11), (4, 8, 8), 12, checkpoint_mode="native")
    assert r.route == "SDPA" and not r.sparse and "native checkpoint" in r.log_line()
    r = vsa.route(1, 2, 128, (9, 10, 11), (4, 8, 8), 13, checkpoint_mode="dmd")
    assert r.route == "SDPA" and "topk > num_blocks" in r.log_line()


# ---------------------------------------------------------------------------
# the two halves of selection; buffers on the wrong device
# ---------------------------------------------------------------------------

def _small(seed=71):
    import torch
    import block_sparse_attention_raster_amd as vsa
    w = synthetic.custom_workload("halves", seed=seed, batch=2, heads=3, head_dim=128, latent=(5, 9, 17),
                                  cube=(4, 8, 8), topk=3, prefix_len=20)
    q, k, v = (G.to_device(x) for x in synthetic.make_inputs(w))
    pl = vsa.plan_for(q, w.latent, w.cube, 3, 20)
    return vsa, torch, pl, q, k, v


def test_pool_then_score_topk_equals_select():
    vsa, torch, pl, q, k, v = _small()
    # zeroed, so that the alignment gaps between the workspace's sections
    # compare equal too
    ws_a = torch.zeros(pl.workspace_bytes, dtype=torch.uint8, device="cuda")
    ws_b = torch.zeros_like(ws_a)
    sel_a, _ = vsa.select(pl, q, k, workspace=ws_a)
    vsa.pool(pl, q, k, workspace=ws_b)
    sel_b = vsa.score_topk(pl, ws_b)
    torch.cuda.synchronize()
    assert torch.equal(ws_a[:pl.workspace_bytes], ws_b[:pl.workspace_bytes])
    assert torch.equal(sel_a, sel_b)


def test_host_buffers_are_refused_before_any_launch():
    """A host (CPU) sel, workspace or output would put a host pointer in
    front of the kernels: the binding raises before calling the library."""
    vsa, torch, pl, q, k, v = _small()
    sel, ws = vsa.select(pl, q, k)
    torch.cuda.synchronize()
    with pytest.raises(ValueError, match="sel"):
        vsa.attend(pl, q, k, v, sel.cpu())
    with pytest.raises(ValueError, match="workspace"):
        vsa.select(pl, q, k, workspace=ws.cpu())
    with pytest.raises(ValueError, match="sel"):
        vsa.select(pl, q, k, sel=sel.cpu())
    with pytest.raises(ValueError, match="out"):
        vsa.attend(pl, q, k, v, sel, out=torch.empty_like(q, device="cpu"))
    with pytest.raises(ValueError, match="v"):
        vsa.attend(pl, q, k, v.cpu(), sel)
    with pytest.raises(ValueError, match="workspace"):
        vsa.score_topk(pl, ws.cpu())
