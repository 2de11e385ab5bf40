"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
(via the package binding) and compare it with the CPU oracle."""
from __future__ import annotations

import numpy as np

import block_sparse_attention_raster_amd as vsa
from block_sparse_attention_raster_amd import synthetic
from oracle import vsa_oracle as O

# Output tolerance versus the float64 oracle, per element type. P is
# rounded to the input type before it multiplies V and the output is rounded
# once more, so the error scales with the type's unit roundoff: 2^-8 for
# bf16, 2^-11 for fp16. The fp16 bounds are the bf16 ones divided by 5
# (the roundoff ratio is 8).
TOL = {"bf16": {"max_abs": 2e-2, "rel_l2": 1e-2},
       "f16": {"max_abs": 4e-3, "rel_l2": 2e-3}}
MAX_ABS = TOL["bf16"]["max_abs"]
REL_L2 = TOL["bf16"]["rel_l2"]
TIE_BAND = 1e-6


def to_device(bits, dtype="bf16"):
    return synthetic.bits_to_torch(bits, dtype=dtype).to("cuda")


def from_device(t, dtype="bf16") -> np.ndarray:
    """bf16 or fp16 torch tensor -> float64 numpy, exactly."""
    import torch
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return O.decode(bits, dtype)


def run_gpu(w: synthetic.Workload, topk: int, qkv_bits=None, dtype="bf16"):
    """Returns dict with the plan, sel (int64 numpy), pooled qbar/kbar
    (float32 numpy) and out (float64 numpy) of one forward on cuda:0."""
    import torch
    q_b, k_b, v_b = qkv_bits if qkv_bits is not None else synthetic.make_inputs(w, dtype=dtype)
    q, k, v = to_device(q_b, dtype), to_device(k_b, dtype), to_device(v_b, dtype)
    pl = vsa.plan_for(q, w.latent, w.cube, topk, w.prefix_len)
    sel, ws = vsa.select(pl, q, k)
    out = vsa.attend(pl, q, k, v, sel)
    torch.cuda.synchronize()
    BH = w.batch * w.heads
    ws_np = ws.cpu().numpy()
    qbar = ws_np[:BH * pl.num_q_blocks * w.head_dim * 4].view(np.float32).reshape(
        w.batch, w.heads, pl.num_q_blocks, w.head_dim)
    kb0 = pl.kbar_offset
    kbar = ws_np[kb0:kb0 + BH * pl.num_blocks * w.head_dim * 4].view(np.float32).reshape(
        w.batch, w.heads, pl.num_blocks, w.head_dim)
    return {"plan": pl, "sel": sel.cpu().numpy().astype(np.int64), "qbar": qbar, "kbar": kbar,
            "out": from_device(out, dtype), "bits": (q_b, k_b, v_b), "dtype": dtype}


def oracle_scores(w: synthetic.Workload, q_b, k_b, dtype="bf16"):
    g = O.geometry(w.latent, w.cube, w.prefix_len)
    qf = O.decode(q_b, dtype)
    qbar = O.pool(qf, g)
    del qf
    kf = O.decode(k_b, dtype)
    kbar = O.pool(kf, g, video_only=True)
    del kf
    return g, qbar, kbar, O.block_scores(qbar, kbar, w.head_dim)


def check_outputs(w, g, res, heads, blocks_per_head=None, rng_seed=0):
    """Recompute the oracle's dense-masked output with the GPU's selection
    for the given (b, h) pairs and query blocks; return worst norms."""
    q_b, k_b, v_b = res["bits"]
    sel = res["sel"]
    worst = {"max_abs": 0.0, "rel_l2": 0.0}
    rng = np.random.default_rng(rng_seed)
    for (b, h) in heads:
        qf, kf, vf = (O.decode(x[b, h], res.get("dtype", "bf16")) for x in (q_b, k_b, v_b))
        if blocks_per_head is None:
            blocks = list(range(g.num_q_blocks))
        else:
            counts = g.counts
            partial = [i for i in range(g.num_q_blocks) if counts[i] < g.cube_volume]
            pick = set(rng.choice(g.num_q_blocks, size=min(blocks_per_head, g.num_q_blocks),
                                  replace=False).tolist())
            pick |= set(partial[:2]) | set(partial[-2:]) | {0, g.num_q_blocks - 1}
            blocks = sorted(pick)
        ref = O.attend_dense_masked(qf, kf, vf, sel[b, h], g, query_blocks=blocks)
        rows = np.concatenate([g.members[i] for i in blocks])
        got = res["out"][b, h][rows]
        assert np.all(np.isfinite(got)), "non-finite GPU output"
        e = O.error_norms(got, ref[rows])
        per = O.error_norms_by_block(res["out"][b, h], ref, g, blocks)
        worst["max_abs"] = max(worst["max_abs"], e["max_abs"])
        worst["rel_l2"] = max(worst["rel_l2"], e["rel_l2"])
        worst["block_rel_l2"] = max(worst.get("block_rel_l2", 0.0), max(x["rel_l2"] for x in per.values()))
    return worst
