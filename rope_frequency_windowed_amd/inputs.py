"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

Holds none of the attention arithmetic: it only draws iid N(0,1) tensors from
fixed seeds (torch Philox on a GPU, torch's CPU generator on the host), casts
them to the compute dtype, and picks seeded row samples.  Both the oracle side
and the HIP side receive the very same cast values.
"""
from __future__ import annotations

import numpy as np
import torch

SEED_Q, SEED_K, SEED_V = 1000, 1001, 1002


def _randn(shape, seed: int, device, dtype) -> torch.Tensor:
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x.to(dtype)


def make_qkv(B: int, Hq: int, Hkv: int, Sq: int, Sk: int, d: int, *,
             dtype=torch.bfloat16, device="cpu", seeds=(SEED_Q, SEED_K, SEED_V),
             high_freq_scale: float | None = None, layout: str = "neox"):
    """q [B,Hq,Sq,d], k/v [B,Hkv,Sk,d], iid N(0,1) drawn in fp32 then cast.

    ``high_freq_scale``: if set, the first half of the rotary pairs (the fast
    ones, p < d/4) of q and k is multiplied by this factor before the cast,
    so that the distance windows change the output a lot (a structured input
    for discrimination checks).  Where those pairs sit depends on ``layout``:
    dims [0, d/4) and [d/2, 3d/4) in the half-split ("neox") layout, dims
    [0, d/2) in the interleaved ("gptj") layout.
    """
    if layout not in ("neox", "gptj"):
        raise ValueError("layout must be 'neox' or 'gptj'")
    q = _randn((B, Hq, Sq, d), seeds[0], device, torch.float32)
    k = _randn((B, Hkv, Sk, d), seeds[1], device, torch.float32)
    v = _randn((B, Hkv, Sk, d), seeds[2], device, torch.float32)
    if high_freq_scale is not None:
        half, quarter = d // 2, d // 4
        for t in (q, k):
            if layout == "gptj":
                t[..., :half] *= high_freq_scale
            else:
                t[..., :quarter] *= high_freq_scale
                t[..., half:half + quarter] *= high_freq_scale
    return q.to(dtype), k.to(dtype), v.to(dtype)


def tile_edge_rows(S: int, n_tiles: int, seed: int, tile: int = 256) -> np.ndarray:
    """Query rows at the edges of 256-query tiles (offsets 0, 31, 32 and 255
    within a tile: a workgroup's first row, the boundary between its first two
    32-row waves, its last row) in n_tiles seeded tiles, always including the
    last whole tile."""
    n_full = S // tile
    if n_full == 0:
        return np.array([], dtype=np.int64)
    rng = np.random.default_rng(seed)
    tiles = {n_full - 1} | {int(t) for t in rng.integers(0, n_full, size=max(n_tiles - 1, 0))}
    rows = sorted({t * tile + e for t in tiles for e in (0, 31, 32, tile - 1)})
    return np.array(rows, dtype=np.int64)


def sample_rows(S: int, n: int, seed: int = 7) -> np.ndarray:
    """n distinct query indices in [0, S): always 0 and S-1, the rest seeded uniform."""
    n = min(n, S)
    rng = np.random.default_rng(seed)
    picked = {0, S - 1}
    while len(picked) < n:
        picked.add(int(rng.integers(0, S)))
    return np.array(sorted(picked), dtype=np.int64)[:max(n, 1)]
