"""Benchmark: one step = one whole attention call (pool, score + top-k, and
block-sparse attention over every (batch, head): vsa_select + vsa_attend,
with vsa_select issued as its two halves vsa_pool and vsa_score_topk so that
an event can sit between them) on synthetic inputs resident in HBM. Prints
one JSON line.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--workload wan] [--dtype bf16]

Throughput is selected-block TFLOP/s: 4 * head_dim * sum over query tokens of
the number of key tokens in their kept blocks (QK^T and PV; the selection of
the GPU's own run), divided by the measured time. ``value`` and
``ms_per_step`` are the wall clock of the timed steps run back to back; HIP
events on the stream the kernels run on split every step into pool, score +
top-k and attention (median and mean over the steps). A second pass runs the
same steps with the L2 and the MALL flushed before each (a 1 GiB buffer
read outside the timed region, which leaves the caches holding clean lines
of that buffer; a write would leave dirty lines whose write-back then lands
inside the first kernel of the step), as between the layers of a real model.
The roofline object is for the attention kernel (the dominant one). The
other workloads of the suite (wan_sweep at top-k 16, 32 and 120, long720p,
prefix) are timed in the same run and reported under ``suite``. The
cpu_baseline object times the CPU oracle (float64, dense-masked) on a
sample of whole (batch, head) pairs, one per host core, and scales it to the
whole call.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
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
SUITE = (("wan_sweep", 16), ("wan_sweep", 32), ("wan_sweep", 120), ("wan_whole", None), ("long720p", None),
         ("prefix", None))


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
    """4 * D * sum_i n_i * (P + sum_{j in S_i} m_j) over every (b, h): n_i
    the valid tokens of query block i (q's grid), m_j those of key cube j
    (the key grid), P the prefix tokens every block keeps."""
    nq = pl.valid_counts("q")
    m = pl.valid_counts("k")[pl.num_prefix_blocks_k:]
    kept = pl.prefix_len + m[sel_np].sum(axis=-1)           # [B, Hh, nq]
    return float(4.0 * pl.head_dim * np.sum(kept * nq[None, None, :]))


def pool_bytes(pl) -> float:
    """Algorithmic bytes of the pooling kernel: q and k read once (2-byte
    elements), the float32 means written."""
    BH = pl.batch * pl.heads
    return float(BH * pl.head_dim * (2 * (pl.seq_len + pl.seq_len_k) + 4 * (pl.num_q_blocks + pl.num_blocks)))


def select_bytes(pl) -> float:
    """Algorithmic bytes of score + top-k: the means read, sel written."""
    BH = pl.batch * pl.heads
    return float(BH * (4 * pl.head_dim * (pl.num_q_blocks + pl.num_blocks) + 4 * pl.num_q_blocks * pl.topk))


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


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _blas() -> str:
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        return f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:  # pragma: no cover - informational only
        return "unknown"


def cpu_baseline(w, bits, flops_total, dtype: str = "bf16", cores: int = None):
    """Time the CPU oracle (float64, dense-masked; pool, score, top-k, then
    attention of every query block) on whole (batch, head) pairs, one per
    worker process with one BLAS thread each, as many pairs as cores (at
    most all of them), and scale the wall time to the whole call."""
    from oracle import parallel as OP
    cores = cores or OP.host_cores()
    BH = w.batch * w.heads
    n = min(BH, cores)
    pairs = [divmod(i, w.heads) for i in range(n)]
    jobs = OP.head_jobs(bits, pairs, dtype=dtype, latent=w.latent, cube=w.cube, prefix_len=w.prefix_len,
                        topk=w.topk)
    t0 = time.perf_counter()
    res = OP.map_jobs(OP.time_head, jobs, workers=n)
    wall = time.perf_counter() - t0
    rounds = -(-BH // n)                     # the whole call in rounds of n pairs
    est_s = wall * rounds
    sel_s = float(np.mean([r["select_s"] for r in res]))
    return {
        "value": flops_total / est_s / 1e12,
        "unit": "TFLOP/s",
        "cores": int(n),
        "kind": "oracle",
        "ms_per_call_est": est_s * 1e3,
        "select_ms_per_head": sel_s * 1e3,
        "cpu_model": _cpu_model(),
        "blas": _blas(),
        "peak_rss_mib_per_worker": max(r["peak_rss_mib"] for r in res),
        "host_cores": int(cores),
        "sample": (f"{n} of {BH} (batch, head) pairs in parallel, one process and one BLAS thread each: "
                   f"float64 pool+score+top-k and dense-masked attention of all query blocks "
                   f"({wall:.2f} s wall), scaled by {rounds} rounds to the whole call"),
    }


class Run:
    """One workload on the GPU: inputs, plan, buffers and an event-timed
    step issued as vsa_pool, vsa_score_topk, vsa_attend."""

    def __init__(self, w, topk, dtype, dev, bits=None):
        import torch
        import block_sparse_attention_raster_amd as vsa
        from block_sparse_attention_raster_amd import synthetic
        self.vsa, self.torch, self.w, self.topk, self.dtype = vsa, torch, w, topk, dtype
        self.bits = synthetic.make_inputs(w, dtype=dtype) if bits is None else bits
        self.q, self.k, self.v = (synthetic.bits_to_torch(x, dev, dtype) for x in self.bits)
        self.pl = vsa.plan_for(self.q, w.latent, w.cube, topk, w.prefix_len)
        self.ws = torch.empty(self.pl.workspace_bytes, dtype=torch.uint8, device=dev)
        self.sel = torch.empty((self.pl.batch, self.pl.heads, self.pl.num_q_blocks, topk), dtype=torch.int32,
                               device=dev)
        self.out = torch.empty_like(self.q)

    def step(self, ev=None):
        vsa, pl = self.vsa, self.pl
        if ev is not None:
            ev[0].record()
        vsa.pool(pl, self.q, self.k, self.ws)
        if ev is not None:
            ev[1].record()
        vsa.score_topk(pl, self.ws, self.sel)
        if ev is not None:
            ev[2].record()
        vsa.attend(pl, self.q, self.k, self.v, self.sel, self.out)
        if ev is not None:
            ev[3].record()

    def timed(self, steps, flush=None):
        """Events of `steps` steps; with `flush` (an int64 tensor), a read of
        the whole buffer before each step, outside its events. Returns
        (per-step ms [steps, 4 phases: pool, score, attend, call], wall ms of
        the loop)."""
        torch = self.torch
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            if flush is not None:
                flush.sum()
            self.step(events[i])
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3
        ms = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3]),
                        e[0].elapsed_time(e[3])] for e in events])
        return ms, wall

    def flops(self):
        return selected_flops(self.pl, self.sel.cpu().numpy().astype(np.int64))

    def free(self):
        del self.q, self.k, self.v, self.ws, self.sel, self.out
        self.torch.cuda.empty_cache()


def _phase_stats(ms, flops, pl, peak):
    med = np.median(ms, axis=0)
    return {
        "ms_per_call_median": float(med[3]), "pool_ms": float(med[0]), "select_ms": float(med[1]),
        "attend_ms": float(med[2]),
        "attend_tflops": flops / (med[2] * 1e-3) / 1e12,
        "attend_pct_bf16_peak": 100.0 * flops / (med[2] * 1e-3) / 1e12 / peak,
        "pool_gbs": pool_bytes(pl) / (med[0] * 1e-3) / 1e9,
        "select_gbs": select_bytes(pl) / (med[1] * 1e-3) / 1e9,
    }


def _short_kernel(name: str) -> str:
    """A kernel's plain name (vsa_attend_kernel, ...) from a demangled or
    mangled symbol."""
    import re
    m = re.search(r"(vsa_\w+?_kernel|__amd_\w+)", name)
    return m.group(1) if m else name[:60]


def cache_bandwidth() -> dict:
    """Read bandwidth (GB/s) from windows that fit each XCD's L2 (2 MiB),
    the MALL (16 to 128 MiB) or neither (2 GiB): the in-tree probe
    block_sparse_attention_raster_amd/cache_probe (built with the library),
    run as a child process."""
    import subprocess
    probe = os.path.join(ROOT, "block_sparse_attention_raster_amd", "cache_probe")
    if not os.path.exists(probe):
        raise RuntimeError("cache_probe is not built; run __graft_entry__.build() first")
    r = subprocess.run([probe], capture_output=True, text=True, timeout=120)
    if r.returncode != 0:
        raise RuntimeError("cache_probe failed:\n" + r.stderr)
    return json.loads(r.stdout)


def step_probe() -> dict:
    """Issue rates (cycles per iteration of exp2 / fma / MFMA mixes), LDS read
    rates (bytes per clock per CU) and the MFMA-busy percentage of a synthetic
    attention step with and without a barrier and copies: the in-tree probe
    block_sparse_attention_raster_amd/step_probe (built with the library),
    run as a child process."""
    import subprocess
    probe = os.path.join(ROOT, "block_sparse_attention_raster_amd", "step_probe")
    if not os.path.exists(probe):
        raise RuntimeError("step_probe is not built; run __graft_entry__.build() first")
    r = subprocess.run([probe], capture_output=True, text=True, timeout=120)
    if r.returncode != 0:
        raise RuntimeError("step_probe failed:\n" + r.stderr)
    return json.loads(r.stdout)


def summarize_trace(path: str, skip: int, take: int = 0) -> str:
    """Per-kernel dispatch statistics of the library's kernels (vsa_*) in a
    rocprofv3 kernel-trace CSV, dropping the first ``skip`` dispatches of
    each kernel (the warm-up steps) and keeping the next ``take`` (all when
    0), in microseconds. Other kernels (input copies, the cache flush) are
    left out."""
    import csv
    rows = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if "vsa_" not in r["Kernel_Name"]:
                continue
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            rows.setdefault(r["Kernel_Name"], []).append((int(r["Start_Timestamp"]), dur))
    lines = [f"{'kernel':<28}{'calls':>6}{'avg_us':>11}{'median_us':>11}{'min_us':>11}{'max_us':>11}"]
    total = {}
    for name, xs in rows.items():
        xs.sort()
        kept = xs[skip:skip + take] if take > 0 else xs[skip:]
        d = np.array([x[1] for x in kept])
        if d.size:
            total[name] = d
    grand = sum(d.sum() for d in total.values())
    for name, d in sorted(total.items(), key=lambda kv: -kv[1].sum()):
        lines.append(f"{_short_kernel(name):<28}{d.size:>6}{d.mean():>11.1f}{np.median(d):>11.1f}"
                     f"{d.min():>11.1f}{d.max():>11.1f}   {100.0 * d.sum() / grand:5.2f}%")
    lines.append(f"(first {skip} dispatches of each kernel dropped"
                 + (f", next {take} kept)" if take > 0 else ")"))
    return "\n".join(lines)


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
    ap.add_argument("--no-suite", action="store_true", help="time the headline workload only")
    ap.add_argument("--suite-steps", type=int, default=10)
    ap.add_argument("--flush-mib", type=int, default=1024, help="buffer read before each flushed step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 512 MiB device-to-device copy three times (the "
                         "reference kernel for scaling HBM byte counters)")
    ap.add_argument("--cache-bandwidth", action="store_true",
                    help="only measure read bandwidth from windows that fit the L2, the MALL or neither "
                         "(the rooflines of the small-cube attention)")
    ap.add_argument("--step-probe", action="store_true",
                    help="only measure issue and LDS rates and a synthetic attention step "
                         "(what bounds the attention step's schedule)")
    ap.add_argument("--summarize-trace", metavar="CSV",
                    help="only print per-kernel statistics of a rocprofv3 kernel-trace CSV")
    ap.add_argument("--skip", type=int, default=0, help="with --summarize-trace: warm-up dispatches to drop")
    ap.add_argument("--take", type=int, default=0,
                    help="with --summarize-trace: dispatches to keep after the skipped ones (0: all)")
    args = ap.parse_args(argv)

    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.skip, args.take))
        return 0
    if args.cache_bandwidth:
        print(json.dumps(cache_bandwidth()), flush=True)
        return 0
    if args.step_probe:
        print(json.dumps(step_probe()), flush=True)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the path shards over (batch, head) with no exchange "
              "inside attention, and multi-GPU runs are not part of this build. Use --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    from block_sparse_attention_raster_amd import synthetic

    if args.calibrate_copy:
        src = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel(), "repeats": 3}), flush=True)
        return 0

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    peak = PEAK_MFMA_TFLOPS[args.dtype]
    w = synthetic.WORKLOADS[args.workload]
    topk = args.topk if args.topk is not None else w.topk
    if topk != w.topk:
        w = synthetic.Workload(w.name, w.seed, w.batch, w.heads, w.head_dim, w.latent, w.cube,
                               (topk,), w.prefix_len, w.modification)
    run = Run(w, topk, args.dtype, dev)
    for _ in range(args.warmup):
        run.step()
    # the timed steps, back to back (the metric's wall clock), then the
    # same steps with the caches flushed before each
    ms, wall = run.timed(args.steps)
    flush = torch.zeros((args.flush_mib << 20) // 8, dtype=torch.int64, device=dev)
    ms_flushed, _ = run.timed(args.steps, flush=flush)
    del flush
    torch.cuda.empty_cache()
    ms_per_step = wall / args.steps
    flops = run.flops()
    pl = run.pl
    value = flops / (ms_per_step * 1e-3) / 1e12
    warm = _phase_stats(ms, flops, pl, peak)
    cold = _phase_stats(ms_flushed, flops, pl, peak)
    att_tflops = warm["attend_tflops"]
    traffic = traffic_for(w.name if args.dtype == "bf16" else f"{w.name}_{args.dtype}")
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
        "ms_per_call_median": warm["ms_per_call_median"],
        "ms_per_call_mean": float(np.mean(ms[:, 3])),
        "pool_ms": warm["pool_ms"],
        "select_ms": warm["select_ms"],
        "attend_ms": warm["attend_ms"],
        "attend_ms_mean": float(np.mean(ms[:, 2])),
        "pool_gbs": warm["pool_gbs"],
        "select_gbs": warm["select_gbs"],
        "selected_flop": flops,
        "pct_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "attend_pct_bf16_peak": warm["attend_pct_bf16_peak"],
        "flushed": {k: cold[k] for k in ("ms_per_call_median", "pool_ms", "select_ms", "attend_ms",
                                         "attend_pct_bf16_peak", "pool_gbs", "select_gbs")},
        "flush_bytes": args.flush_mib << 20,
        "roofline": {
            "bound": "mfma", "achieved": att_tflops, "peak": peak, "unit": "TFLOP/s",
            "frac": att_tflops / peak,
            "traffic": traffic,
            "kernel": "vsa_attend_kernel",
        },
    }
    bits, wl = run.bits, run.w
    run.free()
    del run
    if not args.no_suite:
        suite = {}
        cache = {}
        for name, tk in SUITE:
            ws = synthetic.WORKLOADS[name]
            tk = tk or ws.topk
            key = f"{name}_{tk}" if name == "wan_sweep" else name
            if name not in cache:
                cache.clear()
                cache[name] = synthetic.make_inputs(ws, dtype=args.dtype)
            r = Run(ws, tk, args.dtype, dev, bits=cache[name])
            for _ in range(2):
                r.step()
            sms, swall = r.timed(args.suite_steps)
            sf = r.flops()
            st = _phase_stats(sms, sf, r.pl, peak)
            st.update({"ms_per_call": swall / args.suite_steps, "steps": args.suite_steps, "selected_flop": sf,
                       "topk": tk, "num_blocks": r.pl.num_blocks,
                       "pct_bf16_peak": 100.0 * sf / (swall / args.suite_steps * 1e-3) / 1e12 / PEAK_BF16_TFLOPS})
            suite[key] = st
            r.free()
        line["suite"] = suite
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, bits, flops, dtype=args.dtype)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
