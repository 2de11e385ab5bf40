"""Host-side checks of bench.py's bookkeeping (no GPU): the one-GPU guard,
the FLOP count against the oracle's kept blocks, the traffic record lookup
and the CPU-baseline leg on a tiny workload."""
import numpy as np
import pytest

import bench
import block_sparse_attention_raster_amd as vsa
from block_sparse_attention_raster_amd import synthetic
from oracle import vsa_oracle as O


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


@pytest.mark.parametrize("latent,cube,prefix,topk", [
    ((8, 8, 8), (4, 4, 4), 0, 4), ((5, 6, 7), (2, 4, 4), 9, 3), ((21, 30, 52), (4, 4, 4), 512, 96)])
def test_selected_flops_counts_kept_key_tokens(latent, cube, prefix, topk):
    """4 * D * sum over query tokens of the tokens of their kept blocks,
    recounted from the oracle's geometry for a random ascending selection."""
    D = 64
    pl = vsa.plan(2, 3, D, latent, cube, topk, prefix)
    g = O.geometry(latent, cube, prefix)
    rng = np.random.default_rng(0)
    sel = np.sort(np.stack([rng.choice(g.num_blocks, topk, replace=False)
                            for _ in range(2 * 3 * g.num_q_blocks)]), axis=1).reshape(2, 3, g.num_q_blocks, topk)
    counts = g.counts
    want = 0
    for b in range(2):
        for h in range(3):
            for i in range(g.num_q_blocks):
                kept = O.kept_blocks(sel[b, h, i], g)
                want += counts[i] * counts[kept].sum()
    assert bench.selected_flops(pl, sel) == pytest.approx(4.0 * D * want, rel=1e-12)


def test_selected_flops_two_grids():
    """q and k/v on different grids: query sizes from q's grid, key cube
    sizes from the key grid (the key prefix blocks are kept whole)."""
    D, lq, cq, lk, ck, P, topk = 64, (5, 7, 9), (3, 4, 5), (6, 5, 8), (2, 3, 3), 9, 5
    pl = vsa.plan(1, 2, D, lq, cq, topk, P, latent_k=lk, cube_k=ck)
    gq, gk = O.geometry(lq, cq, P), O.geometry(lk, ck, P)
    rng = np.random.default_rng(1)
    sel = np.sort(np.stack([rng.choice(gk.num_blocks, topk, replace=False)
                            for _ in range(2 * gq.num_q_blocks)]), axis=1).reshape(1, 2, gq.num_q_blocks, topk)
    want = 0
    for h in range(2):
        for i in range(gq.num_q_blocks):
            want += gq.counts[i] * gk.counts[O.kept_blocks(sel[0, h, i], gk)].sum()
    assert bench.selected_flops(pl, sel) == pytest.approx(4.0 * D * want, rel=1e-12)


def test_algorithmic_bytes():
    pl = vsa.plan(1, 24, 128, (31, 22, 40), (4, 8, 8), 64)
    N, BH, D = 27280, 24, 128
    assert bench.pool_bytes(pl) == BH * D * (2 * 2 * N + 4 * 240)
    assert bench.select_bytes(pl) == BH * (4 * D * 240 + 4 * 120 * 64)


def test_traffic_record_lookup():
    assert bench.traffic_for("no_such_workload") is None
    assert bench.attend_source_hash() == bench.attend_source_hash()


def test_cpu_baseline_on_tiny_workload():
    w = synthetic.WORKLOADS["tiny"]
    bits = synthetic.make_inputs(w)
    r = bench.cpu_baseline(w, bits, flops_total=1e9, cores=2)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0 and r["cores"] == 2
    assert "scaled by 1 rounds to the whole call" in r["sample"]
    assert r["cpu_model"] and r["blas"] and r["peak_rss_mib_per_worker"] > 0


def test_parallel_oracle_matches_serial():
    """The process-pool driver gives what the oracle gives serially: an
    output equal to the oracle's own (bf16-rounded) checks with zero error
    in every block, and a perturbed block shows up in that block only."""
    from oracle import parallel as OP
    w = synthetic.custom_workload("par", seed=5, batch=1, heads=2, head_dim=64, latent=(5, 6, 7),
                                  cube=(2, 4, 4), topk=3, prefix_len=7)
    q, k, v = synthetic.make_inputs(w)
    g = O.geometry(w.latent, w.cube, w.prefix_len)
    sel = np.zeros((1, 2, g.num_q_blocks, 3), dtype=np.int64)
    outs = np.zeros_like(q)
    for h in range(2):
        qf, kf, vf = (O.decode_bf16(x[0, h]) for x in (q, k, v))
        s, sel[0, h], o = O.forward_head(qf, kf, vf, g, 3)
        outs[0, h] = synthetic.f32_to_bf16_bits(o.astype(np.float32))
    bad = 4
    outs[0, 1, g.members[bad]] ^= np.uint16(0x4000)        # flip an exponent bit in one block of head 1
    jobs = OP.head_jobs((q, k, v, outs), [(0, 0), (0, 1)], sel=sel, dtype="bf16", latent=w.latent,
                        cube=w.cube, prefix_len=w.prefix_len)
    res = OP.map_jobs(OP.check_head, jobs, workers=2)
    assert all(r["finite"] and r["blocks"] == g.num_q_blocks for r in res)
    assert max(e["rel_l2"] for e in res[0]["per_block"].values()) < 4e-3   # bf16 rounding of the output only
    assert res[1]["worst_block"] == bad and res[1]["per_block"][bad]["rel_l2"] > 0.5
