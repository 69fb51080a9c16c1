"""Shared checks of the GPU path against the oracle.

Tolerances (bf16 inputs, float32 accumulation):
  * outputs: max |gpu - oracle| <= 2e-2 AND ||gpu - oracle||_F / ||oracle||_F <= 5e-3;
  * tile selections: identical, except in near-tie rows where the k-th and
    (k+1)-th oracle scores differ by less than 1e-4 relative; there the GPU
    may only exchange tiles whose scores lie inside that band. Such rows are
    counted and reported.
"""

from __future__ import annotations

import numpy as np
import torch

MAX_ABS = 2e-2
REL_FRO = 5e-3
TIE_REL = 1e-4


def to_f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def bf16_gpu(x: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device).to(torch.bfloat16)


def errors(gpu, ref):
    g, r = to_f64(gpu), to_f64(ref)
    assert g.shape == r.shape, f"shape {g.shape} != {r.shape}"
    d = g - r
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    nref = float(np.linalg.norm(r))
    rel = float(np.linalg.norm(d) / nref) if nref > 0 else float(np.linalg.norm(d))
    return max_abs, rel


def assert_close(gpu, ref, what: str, max_abs: float = MAX_ABS, rel_fro: float = REL_FRO):
    ma, rf = errors(gpu, ref)
    print(f"[parity] {what}: max_abs={ma:.3e} rel_fro={rf:.3e}", flush=True)
    assert ma <= max_abs, f"{what}: max abs error {ma:.3e} > {max_abs}"
    assert rf <= rel_fro, f"{what}: relative Frobenius error {rf:.3e} > {rel_fro}"
    return ma, rf


def check_selection_row(gpu_row, scores_row, top_k: int) -> bool:
    """Validate one GPU selection row against oracle scores; returns True if it
    differs from the oracle's set (allowed only inside the near-tie band)."""
    g = np.asarray(gpu_row, dtype=np.int64)
    s = np.asarray(scores_row, dtype=np.float64)
    assert g.shape == (top_k,)
    assert np.all(np.diff(g) > 0), f"selection not strictly ascending: {g}"
    assert g.min() >= 0 and g.max() < s.shape[0], "selection index out of range"
    order = np.lexsort((np.arange(s.shape[0]), -s))
    ref = np.sort(order[:top_k])
    if np.array_equal(g, ref):
        return False
    tau = s[order[top_k - 1]]
    band = TIE_REL * max(abs(tau), abs(s[order[top_k]]) if top_k < s.shape[0] else 0.0)
    nxt = s[order[top_k]] if top_k < s.shape[0] else -np.inf
    assert abs(tau - nxt) < band, (
        f"selection differs outside a near tie: k-th {tau!r}, (k+1)-th {nxt!r}")
    lo, hi = tau - band, tau + band
    inside = (s >= lo) & (s <= hi)
    must_in = np.nonzero(s > hi)[0]
    must_out = np.nonzero(s < lo)[0]
    gs = set(g.tolist())
    assert all(j in gs for j in must_in), "a tile above the tie band was dropped"
    assert not any(j in gs for j in must_out), "a tile below the tie band was kept"
    assert all(inside[j] or s[j] > hi for j in g), "kept tile outside the band"
    return True


def check_selection(gpu_sel, scores, top_k: int) -> int:
    """All rows of [Tq][k] (or [H][Tq][k]) vs oracle scores; returns the near-tie swap count."""
    g = np.asarray(gpu_sel)
    s = np.asarray(scores, dtype=np.float64)
    g2 = g.reshape(-1, top_k)
    s2 = s.reshape(-1, s.shape[-1])
    return sum(check_selection_row(g2[i], s2[i], top_k) for i in range(g2.shape[0]))


def oracle_kept_mask(scores, top_k: int) -> np.ndarray:
    """[R][T] boolean mask of the oracle's kept tiles for every row of scores:
    all tiles above the k-th largest score, then the lowest-indexed tiles
    equal to it (the tie rule of the selection)."""
    s = np.asarray(scores, dtype=np.float64)
    t = s.shape[1]
    tau = np.partition(s, t - top_k, axis=1)[:, t - top_k]
    above = s > tau[:, None]
    ties = s == tau[:, None]
    room = top_k - above.sum(axis=1)
    return above | (ties & (np.cumsum(ties, axis=1) <= room[:, None]))


def selection_report(gpu_sel, scores, top_k: int, chunk: int = 1024) -> dict:
    """Every row of a GPU selection ([..][k]) against the oracle's float64 scores
    ([..][T]), vectorised over rows. Returns the row count, the rows identical to
    the oracle's, the near-tie swaps (rows that differ only inside the tie band)
    and the mismatches (rows that differ anywhere else: a parity failure)."""
    g = np.asarray(gpu_sel).reshape(-1, top_k).astype(np.int64)
    s = np.asarray(scores, dtype=np.float64)
    s = s.reshape(-1, s.shape[-1])
    rows, t = s.shape
    assert g.shape[0] == rows, f"{g.shape[0]} selection rows for {rows} score rows"
    if top_k > 1:
        assert np.all(np.diff(g, axis=1) > 0), "a selection row is not strictly ascending"
    assert g.min() >= 0 and g.max() < t, "selection index out of range"
    exact = near = bad = 0
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        ref = oracle_kept_mask(s[r0:r1], top_k)
        got = np.zeros_like(ref)
        np.put_along_axis(got, g[r0:r1], True, axis=1)
        same = (got == ref).all(axis=1)
        exact += int(same.sum())
        for r in np.nonzero(~same)[0]:
            try:
                check_selection_row(g[r0 + r], s[r0 + r], top_k)
                near += 1
            except AssertionError:
                bad += 1
    return {"rows": rows, "exact": exact, "near_tie_swaps": near, "mismatches": bad}


def assert_grad_close(gpu, ref, what: str):
    """Gradients: relative Frobenius error <= 5e-3 and max |gpu - ref| <= 2e-2 of
    max(1, max |ref|) (their scale grows with the sequence length)."""
    g, r = to_f64(gpu), to_f64(ref)
    scale = max(1.0, float(np.max(np.abs(r))) if r.size else 1.0)
    return assert_close(g / scale, r / scale, what)
