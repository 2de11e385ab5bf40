"""Benchmark: one step = one whole attention call (vsa_select + vsa_attend over
every (batch, head)) of the block-sparse path on synthetic inputs resident in
HBM. Prints one JSON line.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--workload wan] [--dtype bf16]

Throughput is selected-block TFLOP/s: 4 * head_dim * sum over query tokens of
the number of key tokens in their kept blocks (QK^T and PV; the selection of
the GPU's own run), divided by the measured time. The roofline object is for
the attention kernel (the dominant one), timed with HIP events on the stream
it runs on. The cpu_baseline object times the CPU oracle (float64,
dense-masked) on a bounded sample of the same workload and scales it to the
whole call.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ms per attention call + selected-block TFLOP/s (% bf16 MFMA peak), 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_MFMA_TFLOPS = {"bf16": PEAK_BF16_TFLOPS, "f16": 2500.0}   # fp16 dense peak equals bf16's
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attend.json")
ATTEND_SOURCES = ["attend.hip", "vsa_device.h", "vsa_limits.h"]


def attend_source_hash() -> str:
    """Hash of the attention kernel's sources with comments and blank lines
    removed, so that the recorded traffic stays valid across comment edits
    and lapses when the code changes."""
    import re
    h = hashlib.sha256()
    for s in ATTEND_SOURCES:
        with open(os.path.join(ROOT, "block_sparse_attention_raster_amd", "csrc", s)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = "\n".join(line.rstrip() for line in text.split("\n") if line.strip())
        h.update(text.encode())
    return h.hexdigest()


def selected_flops(pl, sel_np: np.ndarray) -> float:
    """4 * D * sum_i n_i * (P + sum_{j in S_i} m_j) over every (b, h)."""
    counts = pl.valid_counts()
    m = counts[pl.num_prefix_blocks:]
    kept = pl.prefix_len + m[sel_np].sum(axis=-1)           # [B, Hh, nq]
    return float(4.0 * pl.head_dim * np.sum(kept * counts[None, None, :]))


def traffic_for(workload: str):
    """HBM bytes per attention launch from committed rocprofv3 counter runs,
    or None when they are missing or were taken on a different kernel."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    e = t.get(workload)
    if not e or e.get("kernel_source_sha256") != attend_source_hash():
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(w, bits, sel_np, flops_total, budget_s: float = 12.0, dtype: str = "bf16"):
    """Time the CPU oracle (float64, dense-masked) on whole (batch, head)
    pairs: pool + score + top-k of the head and attention of all its query
    blocks, head after head until about ``budget_s`` seconds have been spent
    (at least one head; for very large heads, a prefix of its query blocks).
    The per-head time is scaled to the whole call."""
    from oracle import vsa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - informational only
        threads = len(os.sched_getaffinity(0))
    g = O.geometry(w.latent, w.cube, w.prefix_len)
    q_b, k_b, v_b = bits
    BH = w.batch * w.heads
    spent, heads_done, partial = 0.0, 0, None
    for bh in range(BH):
        b, h = divmod(bh, w.heads)
        t0 = time.perf_counter()
        qf, kf, vf = (O.decode(x[b, h], dtype) for x in (q_b, k_b, v_b))
        s = O.block_scores(O.pool(qf, g), O.pool(kf, g, video_only=True), w.head_dim)
        sel0 = O.select_topk(s, w.topk)
        t_sel = time.perf_counter() - t0
        t_att, nblk = 0.0, 0
        for i in range(g.num_q_blocks):
            t1 = time.perf_counter()
            O.attend_dense_masked(qf, kf, vf, sel0, g, query_blocks=[i])
            t_att += time.perf_counter() - t1
            nblk += 1
            if heads_done == 0 and t_sel + t_att > budget_s:
                break
        if nblk < g.num_q_blocks:      # one head is more than the budget
            partial = (t_sel, t_att, nblk)
            break
        spent += t_sel + t_att
        heads_done += 1
        if spent > budget_s:
            break
    if partial is not None:
        t_sel, t_att, nblk = partial
        per_head = t_sel + t_att / nblk * g.num_q_blocks
        sample = (f"(batch 0, head 0) of {BH}: float64 pool+score+top-k of the head ({t_sel:.2f} s) and "
                  f"dense-masked attention of {nblk} of {g.num_q_blocks} query blocks ({t_att:.2f} s)")
    else:
        per_head = spent / heads_done
        sample = (f"{heads_done} of {BH} (batch, head) pairs in full: float64 pool+score+top-k and "
                  f"dense-masked attention of all {g.num_q_blocks} query blocks ({spent:.2f} s)")
    est_s = BH * per_head
    return {
        "value": flops_total / est_s / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "ms_per_call_est": est_s * 1e3,
        "sample": sample + ", scaled to the whole call",
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan")
    ap.add_argument("--topk", type=int, default=None)
    ap.add_argument("--dtype", choices=["bf16", "f16"], default="bf16",
                    help="element type of q, k, v and the output")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 512 MiB device-to-device copy three times (the "
                         "reference kernel for scaling HBM byte counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the path shards over (batch, head) with no exchange "
              "inside attention, and multi-GPU runs are not part of this build. Use --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    import block_sparse_attention_raster_amd as vsa
    from block_sparse_attention_raster_amd import synthetic

    if args.calibrate_copy:
        src = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel(), "repeats": 3}), flush=True)
        return 0

    w = synthetic.WORKLOADS[args.workload]
    topk = args.topk if args.topk is not None else w.topk
    if topk != w.topk:
        w = synthetic.Workload(w.name, w.seed, w.batch, w.heads, w.head_dim, w.latent, w.cube,
                               (topk,), w.prefix_len, w.modification)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bits = synthetic.make_inputs(w, dtype=args.dtype)
    q, k, v = (synthetic.bits_to_torch(x, dev, args.dtype) for x in bits)
    pl = vsa.plan_for(q, w.latent, w.cube, topk, w.prefix_len)
    ws = torch.empty(pl.workspace_bytes, dtype=torch.uint8, device=dev)
    sel = torch.empty((pl.batch, pl.heads, pl.num_q_blocks, topk), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        vsa.select(pl, q, k, ws, sel)
        if ev is not None:
            ev[1].record()
        vsa.attend(pl, q, k, v, sel, out)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    sel_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    att_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))

    sel_np = sel.cpu().numpy().astype(np.int64)
    flops = selected_flops(pl, sel_np)
    value = flops / (ms_per_step * 1e-3) / 1e12
    att_tflops = flops / (att_ms * 1e-3) / 1e12
    traffic = traffic_for(w.name if args.dtype == "bf16" else f"{w.name}_{args.dtype}")
    peak = PEAK_MFMA_TFLOPS[args.dtype]
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.batch, "heads": w.heads, "head_dim": w.head_dim,
            "latent": list(w.latent), "cube": list(w.cube), "topk": topk,
            "prefix_len": w.prefix_len, "num_blocks": pl.num_blocks, "seq_len": pl.seq_len,
            "parallelism": "single GPU",
        },
        "ms_per_call": ms_per_step,
        "select_ms": sel_ms,
        "attend_ms": att_ms,
        "selected_flop": flops,
        "pct_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "attend_pct_bf16_peak": 100.0 * att_tflops / PEAK_BF16_TFLOPS,
        "roofline": {
            "bound": "mfma", "achieved": att_tflops, "peak": peak, "unit": "TFLOP/s",
            "frac": att_tflops / peak,
            "traffic": traffic,
            "kernel": "vsa_attend_kernel",
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, bits, sel_np, flops, dtype=args.dtype)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
