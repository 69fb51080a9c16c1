"""The selection report used by the GPU tests and the benchmark, on the CPU.

It must count rows equal to the oracle's selection, rows that differ only by a
swap inside the near-tie band, and rows that differ anywhere else, and agree
with the row-by-row check on every row.
"""

import numpy as np

import oracle.zebra_oracle as zo
from parity_util import check_selection_row, oracle_kept_mask, selection_report


def _rows(seed, r, t):
    rng = np.random.default_rng(seed)
    s = rng.integers(-20, 20, size=(r, t)).astype(np.float64)  # many exact ties
    return s


def test_kept_mask_matches_oracle_selection():
    s = _rows(1, 40, 30)
    for k in (1, 5, 29, 30):
        mask = oracle_kept_mask(s, k)
        for r in range(s.shape[0]):
            ref = zo.select_top_tiles(s[r], k)
            assert np.array_equal(np.nonzero(mask[r])[0], ref), (k, r)


def test_report_counts_exact_near_tie_and_mismatch():
    rng = np.random.default_rng(2)
    r, t, k = 12, 50, 7
    s = rng.standard_normal((r, t))
    # row 3: the k-th and (k+1)-th scores 1e-6 apart (a near tie)
    o = np.argsort(-s[3], kind="stable")
    s[3, o[k]] = s[3, o[k - 1]] - 1e-6 * abs(s[3, o[k - 1]])
    sel = np.stack([zo.select_top_tiles(s[i], k) for i in range(r)])
    rep = selection_report(sel, s, k)
    assert rep == {"rows": r, "exact": r, "near_tie_swaps": 0, "mismatches": 0}
    swapped = sel.copy()
    o = np.argsort(-s[3], kind="stable")
    row = set(swapped[3].tolist()) - {int(o[k - 1])} | {int(o[k])}
    swapped[3] = np.sort(list(row))
    assert check_selection_row(swapped[3], s[3], k)
    # row 8: the k-th kept tile replaced by one far below it (a mismatch)
    o8 = np.argsort(-s[8], kind="stable")
    row = set(swapped[8].tolist()) - {int(o8[k - 1])} | {int(o8[-1])}
    swapped[8] = np.sort(list(row))
    rep = selection_report(swapped, s, k, chunk=5)
    assert rep == {"rows": r, "exact": r - 2, "near_tie_swaps": 1, "mismatches": 1}
