"""fp64 CPU oracle for top-k block-sparse attention over a raster-ordered
(T, H, W) latent grid (Video Sparse Attention / fastbsa method).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, the package's smoke check and the
benchmark's CPU-baseline leg may import this module. It imports nothing from
the GPU library and the GPU library never imports it.

What it computes, per (batch, head), following the pages:

* "FastVideo VSA" user guide (vllm-omni docs), opening definition: the
  post-patch latent grid is cut into spatiotemporal blocks; every query block
  scores the key/value blocks and attends only to the kept top-k blocks.
* same guide, section "Wan top-k behavior": top-k counts key/value blocks
  kept per query block; the routing log line fixes the geometry
  (seq_len 27280, grid (31, 22, 40), blocks (4, 8, 8), 120 blocks); top-k
  above the block count is invalid; top-k equal to it keeps every block.
* same guide, section "Choose top-k": the H3 route uses 64-token blocks and
  keeps all prefix blocks.
* same guide, section "Verify routing and fallback": non-causal
  self-attention, equal query and key lengths, scale head_size ** -0.5.
* "fastbsa" package page, section "How it works": selection is checked
  exactly, the output against dense-masked attention. The oracle is that
  dense-masked formulation, in float64.

Readings taken where the pages are silent (each is listed in the design
notes with its reason):
  R1  a block's pooled vector is the mean over its valid tokens only;
  R2  tokens are raster ordered: t slowest, then h, then w;
  R3  video cubes are numbered in raster order of the cube grid;
  R4  equal scores: the lower cube id wins;
  R5  the query's own cube is not forced into the kept set;
  R6  block score = (mean q) . (mean k) * head_dim ** -0.5, no softmax;
  R8  prefix query blocks select top-k video cubes like any other block;
  R9  prefix tokens come first, form ceil(P / V) blocks of V = ct*ch*cw
      tokens (last one partial) and are kept by every query block in
      addition to its top-k video cubes;
  R13 selection is per (batch, head);
  R20 q and k/v may lie on different grids with different cube shapes
      (fastbsa "Use": latent_shape_q / latent_shape_k, chunk_3d_shape_q /
      chunk_3d_shape_k). Query blocks come from q's grid and cubes, key
      blocks from k's; the prefix length is the same for both sequences and
      each side cuts its prefix by its own cube volume;
  R21 sparsity s (fastbsa "Use") keeps floor(nb * (1 - s)) key cubes, at
      least one (the kept fraction never exceeds 1 - s); a product within
      1e-9 of an integer counts as that integer, since decimal sparsities
      such as 0.9 are not exact in binary.

Parity pins: every function here, the comparison helpers included, is
pinned by tests in ``tests/test_oracle_pins.py`` against closed forms, the
pages' numbers, exact rational arithmetic, library routines (torch
scaled_dot_product_attention in float64) and an independent per-token brute
force; ``test_planted_mistakes`` shows that a plausible slip in each is
caught.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np


# ----------------------------------------------------------------------------
# 16-bit float decoding (exact)
# ----------------------------------------------------------------------------

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode_f16(bits: np.ndarray) -> np.ndarray:
    """IEEE 754 binary16 bit patterns (uint16) -> float64, exactly, from the
    format's definition: sign bit 15, biased exponent bits 14..10 (bias 15),
    fraction bits 9..0; exponent 0 is subnormal (fraction * 2^-24), exponent
    31 is infinity or NaN. (User guide, section "Verify routing and
    fallback": the Wan route accepts FP16 as well as BF16.)"""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    normal = np.ldexp(1.0 + f / 1024.0, (e - 15).astype(np.int64))
    sub = np.ldexp(f, -24)
    special = np.where(f == 0, np.inf, np.nan)
    mag = np.where(e == 0, sub, np.where(e == 31, special, normal))
    return sign * mag


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Bit patterns of the named 16-bit type ("bf16" or "f16") -> float64."""
    if dtype == "bf16":
        return decode_bf16(bits)
    if dtype == "f16":
        return decode_f16(bits)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------
# Geometry (user guide, "Wan top-k behavior"; fastbsa "Use")
# ----------------------------------------------------------------------------

def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


@dataclass
class Geometry:
    latent: Tuple[int, int, int]
    cube: Tuple[int, int, int]
    prefix_len: int
    nblk: Tuple[int, int, int]
    num_blocks: int            # video cubes
    num_prefix_blocks: int
    num_q_blocks: int          # prefix blocks + video cubes
    cube_volume: int
    seq_len: int
    block_of_token: np.ndarray  # int64 [N]: query-block id of each token
    members: List[np.ndarray]   # token indices (ascending) of each query block

    @property
    def counts(self) -> np.ndarray:
        return np.array([m.size for m in self.members], dtype=np.int64)


def geometry(latent: Sequence[int], cube: Sequence[int], prefix_len: int = 0) -> Geometry:
    """Partition the raster token sequence into blocks.

    Token n < P is prefix token n, in prefix block n // V. Token n >= P is the
    grid point (t, h, w) with n - P = (t * H + h) * W + w (R2) and belongs to
    video cube (t // ct, h // ch, w // cw), numbered in raster order of the
    cube grid (R3) and offset by the prefix block count.
    """
    T, H, W = (int(x) for x in latent)
    ct, ch, cw = (int(x) for x in cube)
    P = int(prefix_len)
    if min(T, H, W, ct, ch, cw) <= 0 or P < 0:
        raise ValueError("grid, cube and prefix sizes must be positive")
    nT, nH, nW = _ceil_div(T, ct), _ceil_div(H, ch), _ceil_div(W, cw)
    V = ct * ch * cw
    Pb = _ceil_div(P, V)
    nb = nT * nH * nW
    N = P + T * H * W
    n = np.arange(N, dtype=np.int64)
    blk = np.empty(N, dtype=np.int64)
    blk[:P] = n[:P] // V
    r = n[P:] - P
    t = r // (H * W)
    h = (r // W) % H
    w = r % W
    blk[P:] = Pb + ((t // ct) * nH + (h // ch)) * nW + (w // cw)
    order = np.argsort(blk, kind="stable")
    bounds = np.searchsorted(blk[order], np.arange(Pb + nb + 1))
    members = [order[bounds[i]:bounds[i + 1]] for i in range(Pb + nb)]
    return Geometry((T, H, W), (ct, ch, cw), P, (nT, nH, nW), nb, Pb, Pb + nb,
                    V, N, blk, members)


def routing_summary(g: Geometry, topk: int) -> dict:
    """The fields of the Wan routing log line for this geometry."""
    return {
        "seq_len": g.seq_len,
        "dit_seq_shape": tuple(g.latent),
        "block_size": tuple(g.cube),
        "num_blocks": g.num_blocks,
        "topk": int(topk),
        "keep_ratio": f"{100.0 * topk / g.num_blocks:.1f}%",
    }


def topk_for_sparsity(num_blocks: int, sparsity: float) -> int:
    """Key cubes kept for a sparsity s in [0, 1) (fastbsa "Use": 0.9375
    keeps 1/16; R21): floor(nb * (1 - s)), at least 1. A product within
    1e-9 (relative) of an integer is that integer."""
    s = float(sparsity)
    if not (0.0 <= s < 1.0):
        raise ValueError("sparsity must be in [0, 1)")
    x = num_blocks * (1.0 - s)
    n = round(x)
    keep = n if abs(x - n) <= 1e-9 * max(1.0, x) else math.floor(x)
    return int(min(max(keep, 1), num_blocks))


def validate_topk(topk: int, num_blocks: int) -> None:
    """Top-k must be positive (user guide, "Alternative configuration
    formats") and at most the block count ("Wan top-k behavior")."""
    if topk < 1:
        raise ValueError("topk must be positive")
    if topk > num_blocks:
        raise ValueError("topk exceeds the number of key/value blocks")


# ----------------------------------------------------------------------------
# Pool (R1) and score (R6)
# ----------------------------------------------------------------------------

def pool(x: np.ndarray, g: Geometry, video_only: bool = False) -> np.ndarray:
    """Mean of x over each block's tokens. x: [..., N, D] float64.

    Returns [..., nq, D] (all query blocks), or [..., nb, D] for the video
    cubes only when ``video_only``.
    """
    first = g.num_prefix_blocks if video_only else 0
    out = np.empty(x.shape[:-2] + (g.num_q_blocks - first, x.shape[-1]), dtype=np.float64)
    for i in range(first, g.num_q_blocks):
        out[..., i - first, :] = x[..., g.members[i], :].mean(axis=-2)
    return out


def block_scores(qbar: np.ndarray, kbar: np.ndarray, head_dim: int) -> np.ndarray:
    """s[i, j] = (qbar_i . kbar_j) * head_dim ** -0.5 for every query block i
    and video cube j. qbar: [..., nq, D], kbar: [..., nb, D]."""
    return np.matmul(qbar, np.swapaxes(kbar, -1, -2)) * (float(head_dim) ** -0.5)


# ----------------------------------------------------------------------------
# Select (user guide, opening definition and "Wan top-k behavior"; R4)
# ----------------------------------------------------------------------------

def select_topk(scores: np.ndarray, topk: int) -> np.ndarray:
    """The topk largest scores of every row; equal scores go to the lower
    index (R4). Returned ids are ascending. scores: [..., nq, nb]."""
    validate_topk(topk, scores.shape[-1])
    order = np.argsort(-scores, axis=-1, kind="stable")[..., :topk]
    return np.sort(order, axis=-1).astype(np.int64)


def kth_largest(scores: np.ndarray, topk: int) -> np.ndarray:
    """Value of the topk-th largest score of each row."""
    return -np.sort(-scores, axis=-1)[..., topk - 1]


def kept_blocks(sel_row: Iterable[int], g: Geometry) -> np.ndarray:
    """Query-block ids a query block attends to: every prefix block (R9)
    plus the selected video cubes."""
    ids = [p for p in range(g.num_prefix_blocks)]
    ids += [g.num_prefix_blocks + int(j) for j in sel_row]
    return np.array(ids, dtype=np.int64)


# ----------------------------------------------------------------------------
# Attend, dense-masked (user guide, opening definition; fastbsa "How it works")
# ----------------------------------------------------------------------------

def attend_dense_masked(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                        sel: np.ndarray, g: Geometry,
                        query_blocks: Optional[Iterable[int]] = None,
                        return_rowsums: bool = False, gk: Optional[Geometry] = None):
    """Exact softmax attention of each query token over the tokens of its
    query block's kept blocks, for one (batch, head).

    q: [Nq, D], k, v: [Nk, D] float64; sel: [nq, topk] video-cube ids of the
    key grid. ``g`` partitions q; ``gk`` partitions k and v (default ``g``,
    R20). L[n, m] = q_n . k_m * D ** -0.5 where key block(m) is kept by
    query block(n), else -inf; P = softmax over m; O_n = sum_m P[n, m] v_m.
    Rows of blocks not in ``query_blocks`` are left as NaN.
    """
    gk = g if gk is None else gk
    N, D = q.shape
    scale = float(D) ** -0.5
    out = np.full((N, v.shape[1]), np.nan, dtype=np.float64)
    rowsums = np.full(N, np.nan, dtype=np.float64)
    blocks = range(g.num_q_blocks) if query_blocks is None else query_blocks
    for i in blocks:
        rows = g.members[i]
        keep = np.isin(gk.block_of_token, kept_blocks(sel[i], gk))
        L = (q[rows] @ k.T) * scale
        L[:, ~keep] = -np.inf
        L -= L.max(axis=1, keepdims=True)
        Pm = np.exp(L)
        Pm /= Pm.sum(axis=1, keepdims=True)
        out[rows] = Pm @ v
        rowsums[rows] = Pm.sum(axis=1)
    return (out, rowsums) if return_rowsums else out


def forward_head(q, k, v, g: Geometry, topk: int,
                 query_blocks: Optional[Iterable[int]] = None, gk: Optional[Geometry] = None):
    """Whole method for one (batch, head): returns (scores, sel, out). ``gk``
    is the key/value grid when it differs from the query grid ``g``."""
    gk = g if gk is None else gk
    D = q.shape[-1]
    qbar = pool(q, g)
    kbar = pool(k, gk, video_only=True)
    s = block_scores(qbar, kbar, D)
    sel = select_topk(s, topk)
    out = attend_dense_masked(q, k, v, sel, g, query_blocks, gk=gk)
    return s, sel, out


# ----------------------------------------------------------------------------
# Independent per-token brute force (tiny grids only; pure Python loops)
# ----------------------------------------------------------------------------

def brute_force_token(q, k, v, latent, cube, prefix_len: int, topk: int, n: int,
                      latent_k=None, cube_k=None):
    """Output row of query token n, recomputed from scratch with Python loops.

    q: nested list (or array) [Nq][D], k, v: [Nk][D] for one head; k and v
    lie on ``latent_k`` cut into ``cube_k`` (default: q's grid and cube).
    The blocks are found by walking the grid coordinates; the cube list is
    ordered by its (bt, bh, bw) coordinates. Shares no code with the
    vectorised path.
    """
    P = prefix_len
    D = len(q[0])

    def blocks_of(lat, cb):
        T, H, W = lat
        ct, ch, cw = cb
        V = ct * ch * cw
        prefix_groups = {}
        for tok in range(P):
            prefix_groups.setdefault(tok // V, []).append(tok)
        cubes = {}
        for t in range(T):
            for hh in range(H):
                for w in range(W):
                    tok = P + (t * H + hh) * W + w
                    cubes.setdefault((t // ct, hh // ch, w // cw), []).append(tok)
        return prefix_groups, cubes

    q_prefix, q_cubes = blocks_of(latent, cube)
    k_prefix, k_cubes = blocks_of(latent if latent_k is None else latent_k,
                                  cube if cube_k is None else cube_k)
    cube_keys = sorted(k_cubes)

    def mean(x, toks):
        return [sum(x[t][d] for t in toks) / len(toks) for d in range(D)]

    T, H, W = latent
    ct, ch, cw = cube
    if n < P:
        my_tokens = q_prefix[n // (ct * ch * cw)]
    else:
        r = n - P
        t, hh, w = r // (H * W), (r // W) % H, r % W
        my_tokens = q_cubes[(t // ct, hh // ch, w // cw)]
    qm = mean(q, my_tokens)
    sc = []
    for key in cube_keys:
        km = mean(k, k_cubes[key])
        sc.append(sum(qm[d] * km[d] for d in range(D)) / math.sqrt(D))
    ranked = sorted(range(len(cube_keys)), key=lambda j: (-sc[j], j))[:topk]
    keys = [tok for grp in k_prefix.values() for tok in grp]
    for j in ranked:
        keys += k_cubes[cube_keys[j]]
    logits = [sum(q[n][d] * k[m][d] for d in range(D)) / math.sqrt(D) for m in keys]
    mx = max(logits)
    ex = [math.exp(x - mx) for x in logits]
    tot = sum(ex)
    return [sum(ex[i] * v[m][d] for i, m in enumerate(keys)) / tot for d in range(D)]


# ----------------------------------------------------------------------------
# Comparison helpers (selection with a tie band; output error norms)
# ----------------------------------------------------------------------------

def check_selection(sel: np.ndarray, scores: np.ndarray, topk: int,
                    band: float = 1e-6) -> dict:
    """Tie-aware check of a selection against float64 scores.

    For each row with k-th largest score s_k: every id whose score exceeds
    s_k + band must be selected, no id whose score is below s_k - band may
    be selected, and the row must hold topk distinct ascending ids in range.
    Ids whose scores lie inside the band are free.
    """
    sel = np.asarray(sel).reshape(-1, topk)
    sc = np.asarray(scores, dtype=np.float64).reshape(-1, scores.shape[-1])
    nb = sc.shape[1]
    kth = kth_largest(sc, topk)
    bad_rows = []
    band_rows = 0
    for r in range(sc.shape[0]):
        row = sel[r]
        ok = bool(np.all(row >= 0) and np.all(row < nb) and np.all(np.diff(row) > 0))
        if ok:
            chosen = np.zeros(nb, dtype=bool)
            chosen[row] = True
            must = sc[r] > kth[r] + band
            never = sc[r] < kth[r] - band
            ok = bool(np.all(chosen[must]) and not np.any(chosen[never]))
            # a row is a "band row" when more than one id sits in the band,
            # i.e. when the choice at the boundary is not unique
            if np.count_nonzero(~must & ~never) > 1:
                band_rows += 1
        if not ok:
            bad_rows.append(r)
    return {"rows": sc.shape[0], "mismatch_rows": bad_rows, "band_rows": band_rows}


def error_norms(out: np.ndarray, ref: np.ndarray) -> dict:
    """Error of ``out`` against the reference ``ref`` (same shape), in
    float64: max_abs = max |out - ref| over all elements, rel_l2 =
    ||out - ref||_2 / ||ref||_2 (Frobenius norms over all elements). A zero
    reference gives rel_l2 0 when out is zero too, else infinity. Empty
    inputs give zeros."""
    o = np.asarray(out, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if o.shape != r.shape:
        raise ValueError(f"shape mismatch {o.shape} vs {r.shape}")
    if o.size == 0:
        return {"max_abs": 0.0, "rel_l2": 0.0}
    diff = o - r
    nd, nr = float(np.linalg.norm(diff)), float(np.linalg.norm(r))
    rel = nd / nr if nr > 0.0 else (0.0 if nd == 0.0 else math.inf)
    return {"max_abs": float(np.max(np.abs(diff))), "rel_l2": rel}


def error_norms_by_block(out: np.ndarray, ref: np.ndarray, g: Geometry,
                         blocks: Optional[Iterable[int]] = None) -> dict:
    """error_norms of the rows of each query block of ``g`` on its own
    (out, ref: [N, D] of one (batch, head)), so that an error confined to
    a few blocks is not averaged away. Returns {block id: norms} for the
    given blocks (default all)."""
    ids = range(g.num_q_blocks) if blocks is None else blocks
    return {int(i): error_norms(np.asarray(out)[g.members[i]], np.asarray(ref)[g.members[i]]) for i in ids}
