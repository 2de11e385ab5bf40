"""Runs the oracle over (batch, head) pairs in worker processes.

TEST INFRASTRUCTURE ONLY, like ``vsa_oracle``: only ``tests/`` and the
benchmark's CPU-baseline leg use it. It adds no arithmetic of its own: each
job calls ``vsa_oracle`` on one (batch, head), whose results do not depend
on any other pair (selection and attention are per (batch, head): R13). The
parallelism is one process per host core, each with one BLAS thread, so the
core count is what the run actually used.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import time
from concurrent.futures import ProcessPoolExecutor
from typing import Callable, Iterable, List, Optional, Sequence

import numpy as np

from oracle import vsa_oracle as O

_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS")


def host_cores() -> int:
    """Cores this process may run on."""
    return len(os.sched_getaffinity(0))


def _one_blas_thread() -> None:
    for v in _THREAD_VARS:
        os.environ[v] = "1"
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:  # pragma: no cover - the variables above still apply
        pass


def map_jobs(fn: Callable, jobs: Sequence, workers: Optional[int] = None) -> List:
    """fn over jobs in spawned worker processes (one BLAS thread each), in
    order. fn must be a module-level function."""
    workers = max(1, min(len(jobs), workers or host_cores()))
    saved = {v: os.environ.get(v) for v in _THREAD_VARS}
    for v in _THREAD_VARS:          # inherited by the spawned children
        os.environ[v] = "1"
    try:
        with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"),
                                 initializer=_one_blas_thread) as ex:
            return list(ex.map(fn, jobs))
    finally:
        for v, x in saved.items():
            if x is None:
                os.environ.pop(v, None)
            else:
                os.environ[v] = x


def check_head(job: dict) -> dict:
    """One (batch, head): the oracle's dense-masked output under the given
    selection for the given query blocks, compared with an output to check
    (all 16-bit bit patterns of one head: q [Nq, D], k, v [Nk, D], out
    [Nq, D]). Returns whether the checked rows are finite, the norms over
    all of them and per query block."""
    dt = job["dtype"]
    g = O.geometry(job["latent"], job["cube"], job["prefix_len"])
    gk = g if job.get("latent_k") is None else O.geometry(job["latent_k"], job["cube_k"], job["prefix_len"])
    blocks = list(range(g.num_q_blocks)) if job.get("blocks") is None else list(job["blocks"])
    qf, kf, vf = (O.decode(job[n], dt) for n in ("q", "k", "v"))
    ref = O.attend_dense_masked(qf, kf, vf, job["sel"], g, query_blocks=blocks, gk=gk)
    out = O.decode(job["out"], dt)
    rows = np.concatenate([g.members[i] for i in blocks])
    per = O.error_norms_by_block(out, ref, g, blocks)
    worst = max(per, key=lambda i: per[i]["rel_l2"])
    return {"finite": bool(np.all(np.isfinite(out[rows]))), "whole": O.error_norms(out[rows], ref[rows]),
            "per_block": per, "worst_block": worst, "blocks": len(blocks)}


def time_head(job: dict) -> dict:
    """One (batch, head) of the whole method, timed: pool, score and top-k,
    then dense-masked attention of every query block."""
    dt = job["dtype"]
    g = O.geometry(job["latent"], job["cube"], job["prefix_len"])
    t0 = time.perf_counter()
    qf, kf, vf = (O.decode(job[n], dt) for n in ("q", "k", "v"))
    s = O.block_scores(O.pool(qf, g), O.pool(kf, g, video_only=True), qf.shape[-1])
    sel = O.select_topk(s, job["topk"])
    t1 = time.perf_counter()
    O.attend_dense_masked(qf, kf, vf, sel, g)
    t2 = time.perf_counter()
    return {"select_s": t1 - t0, "attend_s": t2 - t1, "peak_rss_mib": _peak_rss_mib()}


def _peak_rss_mib() -> float:
    """This process's peak resident set (VmHWM), in MiB."""
    try:
        with open("/proc/self/status") as f:
            for line in f:
                if line.startswith("VmHWM:"):
                    return int(line.split()[1]) / 1024.0
    except OSError:
        pass
    return float("nan")


def head_jobs(bits: Iterable, pairs: Iterable, **common) -> List[dict]:
    """Jobs of the given (batch, head) pairs from [B, Hh, N, D] bit arrays
    (q, k, v[, out]) and, when given, a [B, Hh, nq, topk] selection."""
    arrays = list(bits)
    names = ("q", "k", "v", "out")[:len(arrays)]
    sel = common.pop("sel", None)
    jobs = []
    for b, h in pairs:
        j = {n: np.ascontiguousarray(a[b, h]) for n, a in zip(names, arrays)}
        if sel is not None:
            j["sel"] = np.ascontiguousarray(sel[b, h])
        j.update(common)
        jobs.append(j)
    return jobs
