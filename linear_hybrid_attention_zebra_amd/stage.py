"""Stage runners: one global-attention stage as a sequence of libzebra calls.

A tile-sparse stage is pool(Q) + pool(K) + pool(V) -> select -> attend; a
linear stage is one zebra_linear_attn call with the stage's fitted affine
map. The affine map is fitted once per linear stage (calibration) against
dense softmax attention of the same stage at sampled queries. Every step runs
in libzebra's kernels; this module only allocates buffers and sequences calls
on the current stream.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch

from . import (ceil_div, zebra_fit_affine, zebra_linear_attn, zebra_permute_tokens,
               zebra_pool_landmarks, zebra_select_tiles, zebra_tile_sparse_attn,
               zebra_tile_sparse_attn_ex)


@dataclasses.dataclass
class SparseBuffers:
    """Reusable outputs and workspaces of one tile-sparse stage shape."""

    qbar: torch.Tensor
    kbar: torch.Tensor
    vbar: torch.Tensor
    sel: torch.Tensor
    out: torch.Tensor
    select_ws: Optional[torch.Tensor] = None
    attn_ws: Optional[torch.Tensor] = None

    @classmethod
    def allocate(cls, heads: int, n_q: int, n_kv: int, q_tile: int, k_tile: int, top_k: int,
                 device, out_dtype=torch.bfloat16):
        from . import library
        t_q, t_k = ceil_div(n_q, q_tile), ceil_div(n_kv, k_tile)
        lib = library()
        f32 = dict(dtype=torch.float32, device=device)
        sws = lib.zebra_select_tiles_workspace(heads, t_q, t_k)
        aws = lib.zebra_tile_sparse_attn_workspace(n_q, n_kv, heads, 64, q_tile, k_tile, top_k)
        return cls(
            qbar=torch.empty((heads, t_q, 64), **f32),
            kbar=torch.empty((heads, t_k, 64), **f32),
            vbar=torch.empty((heads, t_k, 64), **f32),
            sel=torch.empty((heads, t_q, top_k), dtype=torch.int32, device=device),
            out=torch.empty((heads, n_q, 64), dtype=out_dtype, device=device),
            select_ws=torch.empty(max(sws, 1), dtype=torch.uint8, device=device),
            attn_ws=torch.empty(max(aws, 1), dtype=torch.uint8, device=device),
        )


def sparse_select(q, k, v, q_tile: int, k_tile: int, top_k: int,
                  bufs: SparseBuffers) -> SparseBuffers:
    """The first half of a tile-sparse stage: pool Q, K and V into tile means,
    score pooled query tiles against pooled key tiles and keep top_k per row."""
    zebra_pool_landmarks(q, q_tile, out=bufs.qbar)
    zebra_pool_landmarks(k, k_tile, out=bufs.kbar)
    zebra_pool_landmarks(v, k_tile, out=bufs.vbar)
    zebra_select_tiles(bufs.qbar, bufs.kbar, top_k, out=bufs.sel, workspace=bufs.select_ws)
    return bufs


def sparse_attend(q, k, v, q_tile: int, k_tile: int, top_k: int, scale: float,
                  bufs: SparseBuffers, flags: int = 0) -> SparseBuffers:
    """The second half: tile-sparse attention over the kept tiles plus landmarks."""
    zebra_tile_sparse_attn_ex(q, k, v, bufs.kbar, bufs.vbar, bufs.sel, q_tile, k_tile, top_k,
                              scale, flags, out=bufs.out, workspace=bufs.attn_ws)
    return bufs


def sparse_stage(q, k, v, q_tile: int, k_tile: int, top_k: int, scale: float,
                 bufs: Optional[SparseBuffers] = None, flags: int = 0) -> SparseBuffers:
    """One tile-sparse stage; returns the buffers (out, sel, means) it filled.

    flags selects an operator variant (ZEBRA_SPARSE_NO_LANDMARKS or
    ZEBRA_SPARSE_LANDMARK_LOG_COUNT); 0 is the method's operator.
    """
    if bufs is None:
        bufs = SparseBuffers.allocate(q.shape[0], q.shape[1], k.shape[1], q_tile, k_tile, top_k,
                                      q.device)
    sparse_select(q, k, v, q_tile, k_tile, top_k, bufs)
    return sparse_attend(q, k, v, q_tile, k_tile, top_k, scale, bufs, flags)


def spatial_sparse_stage(q, k, v, order: torch.Tensor, q_tile: int, k_tile: int, top_k: int,
                         scale: float, bufs: Optional[SparseBuffers] = None, flags: int = 0,
                         out: Optional[torch.Tensor] = None):
    """A tile-sparse stage with spatial tiles: gather q, k, v into the spatial
    order (int32 device vector), run the stage there, scatter the output back.
    Returns (out in the original order, the buffers of the permuted stage)."""
    qp, kp, vp = (zebra_permute_tokens(t.contiguous() if t.stride(2) != 1 else t, order)
                  for t in (q, k, v))
    bufs = sparse_stage(qp, kp, vp, q_tile, k_tile, top_k, scale, bufs, flags)
    if out is None:
        out = torch.empty(q.shape, dtype=bufs.out.dtype, device=q.device)
    zebra_permute_tokens(bufs.out, order, inverse=True, out=out)
    return out, bufs


def linear_stage(q, k, v, aff_scale=None, aff_bias=None, out=None, workspace=None):
    """One linear stage with its affine map."""
    return zebra_linear_attn(q, k, v, aff_scale, aff_bias, out=out, workspace=workspace)


@dataclasses.dataclass
class Calibration:
    aff_scale: torch.Tensor  # [H][64]
    aff_bias: torch.Tensor   # [H][64]
    n_degenerate: int
    sample_index: torch.Tensor
    x: Optional[torch.Tensor] = None  # unfitted linear output at the samples, float32 [H][M][64]
    y: Optional[torch.Tensor] = None  # dense softmax output at the samples, float32 [H][M][64]


def calibrate_linear(q, k, v, sample_index: torch.Tensor, scale: float, k_tile: int = 64,
                     q_tile: int = 128) -> Calibration:
    """Fit a, b of one linear stage against dense softmax attention at the sampled queries.

    The dense target runs in 128-query tiles (tiling does not change dense
    attention; four waves then share each staged key/value block)."""
    qs = q.index_select(1, sample_index).contiguous()
    t_k = ceil_div(k.shape[1], k_tile)
    y = zebra_tile_sparse_attn(qs, k, v, None, None, None, q_tile, k_tile, t_k, scale,
                               out_dtype=torch.float32)
    x = zebra_linear_attn(qs, k, v, out_dtype=torch.float32)
    a, b, n_deg = zebra_fit_affine(x, y)
    return Calibration(a, b, int(n_deg.item()), sample_index, x, y)


def save_calibrations(path, cals: Dict[int, Calibration]) -> None:
    """Write the fitted affine map of every linear stage to one ``.npz``.

    Per stage ``s`` the file holds ``s{s}_aff_scale`` and ``s{s}_aff_bias``
    (float32 [H][64]), ``s{s}_sample_index`` (int64 [M]) and
    ``s{s}_n_degenerate`` (int64 scalar). A converted stack is then usable
    again without re-fitting. The samples x, y are not stored."""
    arrays = {}
    for s, c in sorted(cals.items()):
        arrays[f"s{s}_aff_scale"] = c.aff_scale.detach().float().cpu().numpy()
        arrays[f"s{s}_aff_bias"] = c.aff_bias.detach().float().cpu().numpy()
        arrays[f"s{s}_sample_index"] = c.sample_index.detach().to(torch.int64).cpu().numpy()
        arrays[f"s{s}_n_degenerate"] = np.int64(c.n_degenerate)
    np.savez(path, **arrays)


def load_calibrations(path, device) -> Dict[int, Calibration]:
    """Read a file written by :func:`save_calibrations` (no pickled objects are
    loaded) and place the maps on ``device``."""
    cals: Dict[int, Calibration] = {}
    with np.load(path, allow_pickle=False) as z:
        stages = sorted({int(k[1:].split("_", 1)[0]) for k in z.files})
        for s in stages:
            a = torch.from_numpy(z[f"s{s}_aff_scale"]).to(device=device, dtype=torch.float32)
            b = torch.from_numpy(z[f"s{s}_aff_bias"]).to(device=device, dtype=torch.float32)
            if a.dim() != 2 or a.shape[1] != 64 or b.shape != a.shape:
                raise ValueError(f"stage {s}: affine map of shape {tuple(a.shape)}, "
                                 f"{tuple(b.shape)}; expected [H][64] twice")
            idx = torch.from_numpy(z[f"s{s}_sample_index"]).to(device)
            cals[s] = Calibration(a.contiguous(), b.contiguous(),
                                  int(z[f"s{s}_n_degenerate"]), idx)
    return cals
