"""Seeded synthetic inputs for top-k block-sparse attention on a 3D latent grid.

This module only draws numbers and lays them out. It holds none of the
method's arithmetic (no block ids, pooling, scoring, selection or softmax),
so both the GPU path and the CPU oracle can be fed from it without sharing
any computation. It depends on numpy alone.

Workloads. The pages give one concrete shape: the Wan routing log in the
"FastVideo VSA" user guide (section "Wan top-k behavior"): a (31, 22, 40)
post-patch grid, (4, 8, 8) blocks, top-k 64. The fastbsa package page
(section "Use") gives (4, 4, 4) chunks and a sparsity of 0.9375 (keep 1/16),
and the same user guide (section "Choose top-k") names 64-token blocks that
always keep the prefix. The five workloads below are built around those.

Recipe, for every workload:
  1. rng = numpy.random.Generator(numpy.random.PCG64(seed))
  2. draw q, k, v in that order, each rng.standard_normal((B, Hh, N, D),
     dtype=float32), layout [B, Hh, N, D] with tokens in raster order;
  3. apply the workload's modification in float32 (see ``_modify``);
  4. round to bfloat16 (default) or float16 with round-to-nearest-even; the
     result is returned as the raw uint16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    heads: int
    head_dim: int
    latent: Tuple[int, int, int]
    cube: Tuple[int, int, int]
    topks: Tuple[int, ...]
    prefix_len: int = 0
    modification: str = "none"   # "none" | "cube_bias" | "prefix_k_x2"
    note: str = ""

    @property
    def seq_len(self) -> int:
        t, h, w = self.latent
        return self.prefix_len + t * h * w

    @property
    def topk(self) -> int:
        return self.topks[0]


WORKLOADS = {
    "tiny": Workload(
        "tiny", 1, 1, 2, 64, (8, 8, 8), (4, 4, 4), (4,),
        note="512 tokens, 8 cubes of 64 tokens, keep 4"),
    "wan": Workload(
        "wan", 2, 1, 24, 128, (31, 22, 40), (4, 8, 8), (64,),
        note="Wan routing-log shape: 27280 tokens, 120 cubes of up to 256 "
             "tokens, partial cubes on T and H, keep 64"),
    "wan_sweep": Workload(
        "wan_sweep", 3, 1, 24, 128, (31, 22, 40), (4, 8, 8), (16, 32, 120),
        modification="cube_bias",
        note="Wan shape with a per-head, per-key-cube bias on K that makes "
             "cube scores peaked; top-k 16, 32 and 120 (all blocks)"),
    "wan_whole": Workload(
        "wan_whole", 2, 1, 24, 128, (32, 24, 40), (4, 8, 8), (64,),
        note="Wan's heads, head dim, cube and keep on a (32, 24, 40) grid: "
             "120 whole cubes of 256 tokens; times the attention without "
             "partial query cubes"),
    "long720p": Workload(
        "long720p", 4, 1, 32, 128, (16, 46, 80), (4, 4, 4), (60,),
        note="58880 tokens, 960 cubes of up to 64 tokens, partial cubes "
             "on H, keep 1/16 (60)"),
    "prefix": Workload(
        "prefix", 5, 2, 24, 128, (21, 30, 52), (4, 4, 4), (96,),
        prefix_len=512, modification="prefix_k_x2",
        note="512 prefix tokens always kept (8 blocks of 64) plus a "
             "(21, 30, 52) grid in 624 cubes, partial on T and H, keep 96"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even) and return
    the 16-bit patterns. Inputs must be finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_u.size, step):
        c = flat_u[s:s + step]
        bias = ((c >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
        flat_o[s:s + step] = ((c + bias) >> np.uint32(16)).astype(np.uint16)
    return out


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE binary16 (numpy's conversion: round to nearest,
    ties to even) and return the 16-bit patterns. Inputs must be finite and
    below 65520 in magnitude."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.abs(x) < 65520.0):
        raise ValueError("value out of float16 range")
    return x.astype(np.float16).view(np.uint16)


def _cube_bias(rng, heads, head_dim, latent, cube):
    """Per-head, per-key-cube bias a[h, cube] * g[h, :] laid out per token.

    g ~ N(0, I_D) per head, a ~ N(0, 2^2) per (head, cube), drawn after v.
    The per-token array is built by repeating the per-cube amplitudes along
    each grid axis and cropping to the grid, so no block numbering is used.
    """
    T, H, W = latent
    ct, ch, cw = cube
    nT, nH, nW = -(-T // ct), -(-H // ch), -(-W // cw)
    g = rng.standard_normal((heads, head_dim), dtype=np.float32)
    a = (2.0 * rng.standard_normal((heads, nT, nH, nW), dtype=np.float32)
         ).astype(np.float32)
    grid = np.repeat(np.repeat(np.repeat(a, ct, axis=1), ch, axis=2), cw, axis=3)
    grid = grid[:, :T, :H, :W].reshape(heads, T * H * W)      # [Hh, THW]
    return grid, g


def make_inputs(w: Workload, seed: Optional[int] = None, dtype: str = "bf16"):
    """Return (q, k, v) as uint16 bit arrays of shape [B, Hh, N, D] holding
    bfloat16 (dtype "bf16") or float16 ("f16") values. Both types are drawn
    from the same float32 numbers."""
    if dtype not in ("bf16", "f16"):
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    shape = (w.batch, w.heads, w.seq_len, w.head_dim)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    _modify(w, rng, k)
    conv = f32_to_bf16_bits if dtype == "bf16" else f32_to_f16_bits
    return conv(q), conv(k), conv(v)


def make_inputs_two_grids(seed: int, batch: int, heads: int, head_dim: int, seq_len_q: int,
                          seq_len_k: int, dtype: str = "bf16"):
    """(q, k, v) for q and k/v on different grids: q [B, Hh, Nq, D] then k
    and v [B, Hh, Nk, D], drawn in that order with the recipe above (no
    modification)."""
    if dtype not in ("bf16", "f16"):
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((batch, heads, seq_len_q, head_dim), dtype=np.float32)
    k = rng.standard_normal((batch, heads, seq_len_k, head_dim), dtype=np.float32)
    v = rng.standard_normal((batch, heads, seq_len_k, head_dim), dtype=np.float32)
    conv = f32_to_bf16_bits if dtype == "bf16" else f32_to_f16_bits
    return conv(q), conv(k), conv(v)


def _modify(w: Workload, rng, k: np.ndarray) -> None:
    if w.modification == "none":
        return
    if w.modification == "cube_bias":
        amp, g = _cube_bias(rng, w.heads, w.head_dim, w.latent, w.cube)
        P = w.prefix_len
        for h in range(w.heads):
            k[:, h, P:, :] += amp[h][:, None] * g[h][None, :]
        return
    if w.modification == "prefix_k_x2":
        k[:, :, :w.prefix_len, :] *= np.float32(2.0)
        return
    raise ValueError(f"unknown modification {w.modification!r}")


def custom_workload(name="custom", seed=0, batch=1, heads=2, head_dim=128,
                    latent=(8, 8, 8), cube=(4, 4, 4), topk=4, prefix_len=0,
                    modification="none") -> Workload:
    return Workload(name, seed, batch, heads, head_dim, tuple(latent),
                    tuple(cube), (topk,), prefix_len, modification)


def bits_to_torch(bits: np.ndarray, device=None, dtype: str = "bf16"):
    """View uint16 bit patterns as a torch.bfloat16 ("bf16") or
    torch.float16 ("f16") tensor."""
    import torch
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt)
    return t if device is None else t.to(device)
