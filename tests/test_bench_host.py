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


def test_traffic_record_lookup():
    assert bench.traffic_for("no_such_workload") is None
    assert bench.attend_source_hash() == bench.attend_source_hash()


def test_cpu_baseline_on_tiny_workload():
    w = synthetic.WORKLOADS["tiny"]
    bits = synthetic.make_inputs(w)
    r = bench.cpu_baseline(w, bits, None, flops_total=1e9, budget_s=0.2)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0 and r["cores"] >= 1
    assert "scaled to the whole call" in r["sample"]
