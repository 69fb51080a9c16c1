"""Seeded synthetic inputs for the hybrid global-attention path.

This module holds none of the method's arithmetic: it draws random numbers
and does the index bookkeeping that places each query near a chosen key
tile. Both the HIP path (through the tests and the benchmark) and the CPU
oracle consume what it returns, so it is the only code the two share.

Shapes follow a VGGT-shaped global-attention stage: every view contributes
``VIEW_TOKENS`` tokens, all views attend to each other, 16 heads of width 64.
The pages measure on real scenes (ScanNet-50, RealEstate10K, CO3Dv2); these
seeded draws stand in for them. Sensitive stages are concentrated (each
query tile looks at a few hot key tiles) and tolerant stages are diffuse, as
the Zebra3D paper page (thelatestinai.com) describes in Figure 3 and
Figure 9.

Recipe of a clustered (sparse-stage) draw, in draw order:
  1. K, V ~ N(0, 1), float32, shape [H][N][d].
  2. For every (head, query tile): ``n_hot`` distinct hot key tiles, drawn
     uniformly without replacement (or one tile from each of ``n_hot``
     distinct views when ``distinct_views`` is set).
  3. For every query token: one of its tile's hot tiles, uniformly.
  4. For every query token: an anchor token, uniform over the valid tokens
     of that hot tile.
  5. eps ~ N(0, 1) of shape [H][N][d]; q = 2 * k[anchor] + 0.5 * eps.
A diffuse (linear-stage) draw is Q, K, V ~ N(0, 1) in that order.
Values are float32; the GPU receives them rounded to bfloat16 (round to
nearest even) and parity runs hand the oracle those same rounded values.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

VIEW_TOKENS = 1374
HEADS = 16
HEAD_DIM = 64


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def keep_count(keep_percent: int, n_key_tiles: int) -> int:
    """Key tiles kept per query tile: ceil(keep_percent * T_k / 100) in integers."""
    return (keep_percent * n_key_tiles + 99) // 100


@dataclasses.dataclass(frozen=True)
class Workload:
    """One named synthetic workload (a stage or a stack of stages)."""

    name: str
    kind: str  # "sparse", "linear" or "stack"
    n_views: int
    view_tokens: int
    heads: int
    head_dim: int
    seed: int
    q_tile: int = 64
    k_tile: int = 64
    keep_percent: Optional[int] = None  # sparse stages
    top_k: Optional[int] = None  # overrides keep_percent when set
    n_hot: int = 3
    distinct_views: bool = False
    fit_samples: int = 4096
    linear_stages: Sequence[int] = ()
    n_stages: int = 1

    @property
    def n_tokens(self) -> int:
        return self.n_views * self.view_tokens

    @property
    def t_q(self) -> int:
        return ceil_div(self.n_tokens, self.q_tile)

    @property
    def t_k(self) -> int:
        return ceil_div(self.n_tokens, self.k_tile)

    @property
    def k(self) -> int:
        if self.top_k is not None:
            return self.top_k
        return keep_count(self.keep_percent, self.t_k)

    def stage_seed(self, stage: int) -> int:
        return self.seed + stage if self.kind == "stack" else self.seed

    def stage_kind(self, stage: int) -> str:
        if self.kind != "stack":
            return self.kind
        return "linear" if stage in set(self.linear_stages) else "sparse"


# The five workloads: a tiny CPU-checkable case, one 16-view sparse stage, one
# 128-view linear stage, a 24-stage stack at 512 views and a 1,024-view sparse
# stage at 94% sparsity.
TINY = Workload("tiny-2v", "sparse", n_views=2, view_tokens=64, heads=2, head_dim=64,
                seed=0, q_tile=32, k_tile=32, top_k=1, n_hot=1, fit_samples=128)
SPARSE_16V = Workload("sparse-16v", "sparse", n_views=16, view_tokens=VIEW_TOKENS,
                      heads=HEADS, head_dim=HEAD_DIM, seed=2, keep_percent=20, n_hot=3)
LINEAR_128V = Workload("linear-128v", "linear", n_views=128, view_tokens=VIEW_TOKENS,
                       heads=HEADS, head_dim=HEAD_DIM, seed=3)
STACK_512V = Workload("stack24-512v", "stack", n_views=512, view_tokens=VIEW_TOKENS,
                      heads=HEADS, head_dim=HEAD_DIM, seed=4000, keep_percent=20,
                      n_hot=3, n_stages=24,
                      linear_stages=tuple(range(0, 9)) + tuple(range(21, 24)))
SPARSE_1024V = Workload("sparse-1024v", "sparse", n_views=1024, view_tokens=VIEW_TOKENS,
                        heads=HEADS, head_dim=HEAD_DIM, seed=5, q_tile=128, k_tile=64,
                        keep_percent=6, n_hot=4, distinct_views=True)
WORKLOADS = {w.name: w for w in (TINY, SPARSE_16V, LINEAR_128V, STACK_512V, SPARSE_1024V)}


# ----------------------------------------------------------------------------
# distinct draws without replacement, the same recipe for numpy and torch:
# draw r uniform in [0, n - i), then step r past every value already taken
# (visited in ascending order). Each draw is uniform over the values not yet
# taken.
# ----------------------------------------------------------------------------

def _distinct_np(rng: np.random.Generator, n: int, count: int, shape) -> np.ndarray:
    if count > n:
        raise ValueError(f"cannot draw {count} distinct values from {n}")
    taken = np.zeros(tuple(shape) + (0,), dtype=np.int64)
    order = []
    for i in range(count):
        r = rng.integers(0, n - i, size=shape, dtype=np.int64)
        for j in range(i):  # taken is sorted along the last axis
            r = r + (r >= taken[..., j])
        order.append(r)
        taken = np.sort(np.concatenate([taken, r[..., None]], axis=-1), axis=-1)
    return np.stack(order, axis=-1)


def _view_tile_range(view: np.ndarray, view_tokens: int, k_tile: int):
    """First tile and tile count of each view (a tile belongs to the view of its first token)."""
    lo = -(-(view * view_tokens) // k_tile)
    hi = -(-((view + 1) * view_tokens) // k_tile)
    return lo, hi - lo


def hot_tiles_np(rng, heads, t_q, t_k, n_hot, distinct_views=False, view_tokens=None,
                 k_tile=None, n_tokens=None) -> np.ndarray:
    """[H][T_q][n_hot] hot key tiles per query tile (draw step 2)."""
    if not distinct_views:
        return _distinct_np(rng, t_k, n_hot, (heads, t_q))
    n_views = ceil_div(n_tokens, view_tokens)
    views = _distinct_np(rng, n_views, n_hot, (heads, t_q))
    lo, cnt = _view_tile_range(views, view_tokens, k_tile)
    cnt = np.minimum(cnt, t_k - lo)
    off = np.floor(rng.random(views.shape) * cnt).astype(np.int64)
    return lo + np.minimum(off, cnt - 1)


def clustered_qkv_np(seed: int, heads: int, n: int, d: int, q_tile: int, k_tile: int,
                     n_hot: int, distinct_views: bool = False,
                     view_tokens: int = VIEW_TOKENS, n_kv: Optional[int] = None):
    """Concentrated-attention draw (see the module docstring); float32 numpy [H][N][d]."""
    n_kv = n if n_kv is None else n_kv
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((heads, n_kv, d), dtype=np.float32)
    v = rng.standard_normal((heads, n_kv, d), dtype=np.float32)
    t_q, t_k = ceil_div(n, q_tile), ceil_div(n_kv, k_tile)
    hot = hot_tiles_np(rng, heads, t_q, t_k, n_hot, distinct_views, view_tokens, k_tile, n_kv)
    pick = rng.integers(0, n_hot, size=(heads, n), dtype=np.int64)
    tok = np.arange(n)
    tile = np.take_along_axis(hot[:, tok // q_tile, :], pick[..., None], axis=-1)[..., 0]
    start = tile * k_tile
    count = np.minimum(k_tile, n_kv - start)
    anchor = start + np.minimum(np.floor(rng.random((heads, n)) * count).astype(np.int64),
                                count - 1)
    eps = rng.standard_normal((heads, n, d), dtype=np.float32)
    q = 2.0 * np.take_along_axis(k, anchor[..., None], axis=1) + 0.5 * eps
    return q.astype(np.float32), k, v, hot


def diffuse_qkv_np(seed: int, heads: int, n: int, d: int):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((heads, n, d), dtype=np.float32)
    k = rng.standard_normal((heads, n, d), dtype=np.float32)
    v = rng.standard_normal((heads, n, d), dtype=np.float32)
    return q, k, v


def fit_sample_indices(n: int, m: int, seed: int) -> np.ndarray:
    """M query indices for the affine fit: uniform without replacement, sorted."""
    m = min(m, n)
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(n, size=m, replace=False)).astype(np.int64)


def sample_rows(heads: int, t_q: int, count: int, seed: int) -> np.ndarray:
    """Seeded (head, query tile) pairs checked one by one at full sizes."""
    rng = np.random.default_rng(seed)
    flat = rng.choice(heads * t_q, size=min(count, heads * t_q), replace=False)
    flat.sort()
    return np.stack([flat // t_q, flat % t_q], axis=1).astype(np.int64)


# ----------------------------------------------------------------------------
# torch versions for the large workloads (drawn on the device with a seeded
# torch.Generator; the same recipe, another random stream)
# ----------------------------------------------------------------------------

def _distinct_torch(gen, n: int, count: int, shape, device):
    import torch
    taken = None
    order = []
    for i in range(count):
        r = torch.randint(0, n - i, tuple(shape), generator=gen, device=device,
                          dtype=torch.int64)
        if taken is not None:
            for j in range(taken.shape[-1]):
                r = r + (r >= taken[..., j]).to(torch.int64)
        order.append(r)
        taken = r[..., None] if taken is None else torch.sort(
            torch.cat([taken, r[..., None]], dim=-1), dim=-1).values
    return torch.stack(order, dim=-1)


def clustered_qkv_torch(seed: int, heads: int, n: int, d: int, q_tile: int, k_tile: int,
                        n_hot: int, device, distinct_views: bool = False,
                        view_tokens: int = VIEW_TOKENS, dtype=None):
    """Concentrated-attention draw on ``device``; returns bf16 (or ``dtype``) [H][N][d]."""
    import torch
    dtype = torch.bfloat16 if dtype is None else dtype
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    k32 = torch.randn((heads, n, d), generator=gen, device=device, dtype=torch.float32)
    v = torch.randn((heads, n, d), generator=gen, device=device,
                    dtype=torch.float32).to(dtype)
    t_q, t_k = ceil_div(n, q_tile), ceil_div(n, k_tile)
    if distinct_views:
        n_views = ceil_div(n, view_tokens)
        views = _distinct_torch(gen, n_views, n_hot, (heads, t_q), device)
        lo = torch.div(views * view_tokens + k_tile - 1, k_tile, rounding_mode="floor")
        hi = torch.div((views + 1) * view_tokens + k_tile - 1, k_tile, rounding_mode="floor")
        cnt = torch.minimum(hi - lo, t_k - lo)
        u = torch.rand((heads, t_q, n_hot), generator=gen, device=device, dtype=torch.float64)
        hot = lo + torch.minimum(torch.floor(u * cnt).to(torch.int64), cnt - 1)
    else:
        hot = _distinct_torch(gen, t_k, n_hot, (heads, t_q), device)
    pick = torch.randint(0, n_hot, (heads, n), generator=gen, device=device, dtype=torch.int64)
    tok = torch.arange(n, device=device)
    tile = torch.gather(hot[:, tok // q_tile, :], 2, pick[..., None])[..., 0]
    start = tile * k_tile
    count = torch.clamp(n - start, max=k_tile)
    u = torch.rand((heads, n), generator=gen, device=device, dtype=torch.float64)
    anchor = start + torch.minimum(torch.floor(u * count).to(torch.int64), count - 1)
    q = torch.empty((heads, n, d), device=device, dtype=dtype)
    chunk = 1 << 20
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        eps = torch.randn((heads, e - s, d), generator=gen, device=device, dtype=torch.float32)
        ka = torch.gather(k32, 1, anchor[:, s:e, None].expand(-1, -1, d))
        q[:, s:e] = (2.0 * ka + 0.5 * eps).to(dtype)
    return q, k32.to(dtype), v, hot


def diffuse_qkv_torch(seed: int, heads: int, n: int, d: int, device, dtype=None):
    import torch
    dtype = torch.bfloat16 if dtype is None else dtype
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = []
    for _ in range(3):
        out.append(torch.randn((heads, n, d), generator=gen, device=device,
                               dtype=torch.float32).to(dtype))
    return tuple(out)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to bfloat16 (nearest even), returned as float32."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.bfloat16).to(torch.float32).numpy()


def stage_inputs(w: Workload, stage: int, device):
    """Q, K, V (bf16 on ``device``) for one stage of a workload, drawn with torch."""
    seed = w.stage_seed(stage)
    if w.stage_kind(stage) == "linear":
        return diffuse_qkv_torch(seed, w.heads, w.n_tokens, w.head_dim, device)
    q, k, v, _ = clustered_qkv_torch(seed, w.heads, w.n_tokens, w.head_dim, w.q_tile,
                                     w.k_tile, w.n_hot, device, w.distinct_views,
                                     w.view_tokens)
    return q, k, v
