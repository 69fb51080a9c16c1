"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

Every mutation below replaces one oracle function with a copy that carries a
single mistake: a dropped term, a wrong sign or index, a transposed operand,
a wrong tie rule. The pins must fail for every one of them; a mutation that
no pin notices would mean that part of the oracle is not really pinned.
"""

import numpy as np
import pytest

import oracle.zebra_oracle as zo
from oracle_pins import ALL_PINS

_orig = {name: getattr(zo, name) for name in dir(zo) if not name.startswith("__")}


def _pool_full_tile_divisor(x, tile):
    x = np.asarray(x, dtype=np.float64)
    b = zo.tile_bounds(x.shape[0], tile)
    return np.stack([x[s:e].sum(axis=0) / tile for s, e in b]) if b else np.zeros((0, x.shape[1]))


def _select_ties_high(scores_row, top_k):
    s = np.asarray(scores_row, dtype=np.float64)
    idx = np.arange(s.shape[0])
    return np.sort(np.lexsort((-idx, -s))[:top_k])


def _select_lowest(scores_row, top_k):
    s = np.asarray(scores_row, dtype=np.float64)
    return np.sort(np.lexsort((np.arange(s.shape[0]), s))[:top_k])


def _scores_transposed(qbar, kbar):
    return np.asarray(kbar, np.float64) @ np.asarray(qbar, np.float64).T


def _columns_with(kept_bias=False, landmarks_for_all=False, drop_landmarks=False,
                  ignore_switch=False, count_base2=False, count_full_tiles=False):
    def cols(k, v, k_tile, kept, landmarks=True, landmark_log_count=False):
        k = np.asarray(k, np.float64)
        v = np.asarray(v, np.float64)
        bounds = zo.tile_bounds(k.shape[0], k_tile)
        kbar, vbar = zo.pool_tiles(k, k_tile), zo.pool_tiles(v, k_tile)
        keys, vals, bias = [], [], []
        for j in sorted(int(t) for t in kept):
            s, e = bounds[j]
            keys.append(k[s:e])
            vals.append(v[s:e])
            bias.append(np.zeros(e - s))
        for j in range(len(bounds)):
            if drop_landmarks or not (landmarks or ignore_switch):
                continue
            if landmarks_for_all or j not in set(int(t) for t in kept):
                n = bounds[j][1] - bounds[j][0]
                rep = n if kept_bias else 1  # a landmark counted n_j times
                keys.append(np.repeat(kbar[j:j + 1], rep, axis=0))
                vals.append(np.repeat(vbar[j:j + 1], rep, axis=0))
                cnt = k_tile if count_full_tiles else n
                lg = (np.log2(cnt) if count_base2 else np.log(cnt)) if landmark_log_count else 0.0
                bias.append(np.full(rep, lg))
        return np.concatenate(keys), np.concatenate(vals), np.concatenate(bias)
    return cols


def _sparse_tile_no_scale(q_rows, k, v, k_tile, kept, scale, *variant):
    return _orig["tile_sparse_attention_tile"](q_rows, k, v, k_tile, kept, 1.0, *variant)


def _dense_wrong_axis(q, k, v, scale, row_block=1024):
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    lg = scale * (q @ k.T)
    w = np.exp(lg - lg.max(axis=0, keepdims=True))
    return (w / w.sum(axis=0, keepdims=True)) @ v


def _phi_no_exp(x):
    return np.asarray(x, np.float64) + 1.0


def _linear_transposed_state(q, k, v, aff_scale=None, aff_bias=None):
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    fq, fk = zo.elu_plus_one(q), zo.elu_plus_one(k)
    state = (fk.T @ v).T
    z = fk.sum(axis=0)
    o = (fq @ state) / (fq @ z)[:, None]
    if aff_scale is not None or aff_bias is not None:
        o = zo.affine_apply(o, aff_scale, aff_bias)
    return o, state, z


def _linear_no_normaliser(q, k, v, aff_scale=None, aff_bias=None):
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    fq, fk = zo.elu_plus_one(q), zo.elu_plus_one(k)
    state = fk.T @ v
    z = fk.sum(axis=0)
    o = fq @ state
    if aff_scale is not None or aff_bias is not None:
        o = zo.affine_apply(o, aff_scale, aff_bias)
    return o, state, z


def _fit_uncentred(x, y, degenerate_rel=1e-30):
    x, y = np.asarray(x, np.float64), np.asarray(y, np.float64)
    a = (x * y).sum(axis=0) / (x * x).sum(axis=0)
    return a, np.zeros_like(a), 0


def _fit_bias_sign(x, y, degenerate_rel=1e-30):
    a, b, n = _orig["fit_affine"](x, y, degenerate_rel)
    xbar = np.asarray(x, np.float64).mean(axis=0)
    return a, b + 2 * a * xbar, n


def _mass_with(divide_by_k_tile=False, no_mean=False, skip_last_tile=False):
    def mass(q, k, q_tile, k_tile, scale, row_block=1024):
        q, k = np.asarray(q, np.float64), np.asarray(k, np.float64)
        qb, kb = zo.tile_bounds(q.shape[0], q_tile), zo.tile_bounds(k.shape[0], k_tile)
        lg = scale * (q @ k.T)
        p = np.exp(lg - lg.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        out = np.zeros((len(qb), len(kb)))
        for i, (a, b) in enumerate(qb):
            for j, (c, d) in enumerate(kb):
                if skip_last_tile and j == len(kb) - 1:
                    continue
                tot = p[a:b, c:d].sum()
                out[i, j] = tot if no_mean else tot / ((d - c) if divide_by_k_tile else (b - a))
        return out
    return mass


def _scale_fit_centred(x, y, degenerate_rel=1e-30):
    x, y = np.asarray(x, np.float64), np.asarray(y, np.float64)
    dx, dy = x - x.mean(axis=0), y - y.mean(axis=0)
    return (dx * dy).sum(axis=0) / (dx * dx).sum(axis=0), np.zeros(x.shape[1]), 0


def _scale_fit_keeps_intercept(x, y, degenerate_rel=1e-30):
    a, b, n = _orig["fit_affine"](x, y, degenerate_rel)
    return a, b, n


def _spatial_order_with(col_major_blocks=False, special_last=False):
    def order(n_views, n_special, grid_h, grid_w, block):
        per_view = n_special + grid_h * grid_w
        out = []
        for view in range(n_views):
            base = view * per_view
            sp = [base + t for t in range(n_special)]
            if not special_last:
                out.extend(sp)
            starts = [(r0, c0) for r0 in range(0, grid_h, block) for c0 in range(0, grid_w, block)]
            if col_major_blocks:
                starts.sort(key=lambda rc: (rc[1], rc[0]))
            for r0, c0 in starts:
                for r in range(r0, min(grid_h, r0 + block)):
                    for c in range(c0, min(grid_w, c0 + block)):
                        out.append(base + n_special + r * grid_w + c)
            if special_last:
                out.extend(sp)
        return np.asarray(out, dtype=np.int64)
    return order


def _spatial_attention_not_unpermuted(q, k, v, order, q_tile, k_tile, top_k, scale, sel=None,
                                      **variant):
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    order = np.asarray(order)
    return zo.tile_sparse_attention(q[:, order], k[:, order], v[:, order], q_tile, k_tile,
                                    top_k, scale, sel=sel, **variant)


def _sparse_bwd_with(no_d=False, no_spread=False, dv_from_dl=False, dq_no_scale=False):
    def bwd(q, k, v, q_tile, k_tile, sel, scale, dout, landmarks=True, landmark_log_count=False):
        q, k, v, dout = (np.asarray(x, np.float64) for x in (q, k, v, dout))
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        kb = zo.tile_bounds(k.shape[1], k_tile)
        for h in range(q.shape[0]):
            for i, (s0, e0) in enumerate(zo.tile_bounds(q.shape[1], q_tile)):
                kept = sorted(int(j) for j in sel[h][i])
                ck, cv, bias = zo.attention_columns(k[h], v[h], k_tile, kept, landmarks,
                                                    landmark_log_count)
                owner = [("tok", t) for j in kept for t in range(*kb[j])]
                if landmarks:
                    owner += [("lm", j) for j in range(len(kb)) if j not in set(kept)]
                lg = scale * (q[h, s0:e0] @ ck.T) + bias[None, :]
                p = np.exp(lg - lg.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                dp = dout[h, s0:e0] @ cv.T
                dl = p * dp if no_d else p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[h, s0:e0] = (1.0 if dq_no_scale else scale) * (dl @ ck)
                dck = scale * (dl.T @ q[h, s0:e0])
                dcv = (dl if dv_from_dl else p).T @ dout[h, s0:e0]
                for c, (kind, idx) in enumerate(owner):
                    if kind == "tok":
                        dk[h, idx] += dck[c]
                        dv[h, idx] += dcv[c]
                    else:
                        a, b = kb[idx]
                        n = 1 if no_spread else b - a
                        dk[h, a:b] += dck[c] / n
                        dv[h, a:b] += dcv[c] / n
        return dq, dk, dv
    return bwd


def _linear_bwd_with(no_dphi=False, dden_sign=False, no_db=False):
    def bwd(q, k, v, dout, aff_scale=None, aff_bias=None):
        dq, dk, dv, da, db = _orig["linear_attention_backward"](q, k, v, dout, aff_scale,
                                                                aff_bias)
        q, k, v, dout = (np.asarray(x, np.float64) for x in (q, k, v, dout))
        if no_dphi or dden_sign:
            a = np.ones(v.shape[1]) if aff_scale is None else np.asarray(aff_scale, np.float64)
            fq, fk = zo.elu_plus_one(q), zo.elu_plus_one(k)
            dfq = np.ones_like(q) if no_dphi else np.where(q > 0, 1.0, np.exp(np.minimum(q, 0)))
            state, z = fk.T @ v, fk.sum(axis=0)
            den = fq @ z
            o = (fq @ state) / den[:, None]
            do = dout * a
            dnum = do / den[:, None]
            dden = (1.0 if dden_sign else -1.0) * (do * o).sum(axis=1) / den
            dq = (dnum @ state.T + dden[:, None] * z[None, :]) * dfq
        if no_db:
            db = np.zeros_like(db)
        return dq, dk, dv, da, db
    return bwd


def _sparsity_without_landmarks(linear_frac, keep_frac, k_tile):
    return linear_frac + (1.0 - linear_frac) * (1.0 - keep_frac)


def _sparsity_linear_as_dense(linear_frac, keep_frac, k_tile):
    return (1.0 - linear_frac) * (1.0 - keep_frac - (1.0 - keep_frac) / k_tile)


def _sparsity_landmark_per_key(linear_frac, keep_frac, k_tile):
    dense = keep_frac + (1.0 - keep_frac)
    return linear_frac + (1.0 - linear_frac) * (1.0 - dense)


def _top_mass_lowest(mass, top_k):
    m = np.asarray(mass, np.float64)
    return np.sort(m, axis=1)[:, :top_k].sum(axis=1)


MUTATIONS = {
    "pool divides by the full tile size": ("pool_tiles", _pool_full_tile_divisor),
    "ties go to the highest index": ("select_top_tiles", _select_ties_high),
    "selection keeps the lowest scores": ("select_top_tiles", _select_lowest),
    "tile scores transposed": ("block_scores", _scores_transposed),
    "landmark counted n_j times": ("attention_columns", _columns_with(kept_bias=True)),
    "landmarks also for kept tiles": ("attention_columns", _columns_with(landmarks_for_all=True)),
    "omitted tiles dropped": ("attention_columns", _columns_with(drop_landmarks=True)),
    "softmax scale dropped": ("tile_sparse_attention_tile", _sparse_tile_no_scale),
    "dense softmax over the key axis": ("dense_attention", _dense_wrong_axis),
    "phi without the exponential branch": ("elu_plus_one", _phi_no_exp),
    "linear state transposed": ("linear_attention", _linear_transposed_state),
    "linear normaliser dropped": ("linear_attention", _linear_no_normaliser),
    "fit through the origin": ("fit_affine", _fit_uncentred),
    "fit bias sign": ("fit_affine", _fit_bias_sign),
    "block mass averaged over key tokens": ("block_attention_mass",
                                            _mass_with(divide_by_k_tile=True)),
    "block mass not averaged over queries": ("block_attention_mass", _mass_with(no_mean=True)),
    "block mass drops the last key tile": ("block_attention_mass",
                                           _mass_with(skip_last_tile=True)),
    "top mass takes the lowest blocks": ("top_mass", _top_mass_lowest),
    "mean sparsity drops the landmark columns": ("mean_attention_sparsity",
                                                  _sparsity_without_landmarks),
    "mean sparsity counts linear stages as dense": ("mean_attention_sparsity",
                                                     _sparsity_linear_as_dense),
    "mean sparsity counts a landmark per key": ("mean_attention_sparsity",
                                                _sparsity_landmark_per_key),
    "landmark switch ignored": ("attention_columns", _columns_with(ignore_switch=True)),
    "landmark count in base 2": ("attention_columns", _columns_with(count_base2=True)),
    "landmark count ignores the short last tile": ("attention_columns",
                                                   _columns_with(count_full_tiles=True)),
    "uncentered fit centred": ("fit_scale_only", _scale_fit_centred),
    "uncentered fit keeps an intercept": ("fit_scale_only", _scale_fit_keeps_intercept),
    "spatial blocks in column order": ("spatial_token_order",
                                       _spatial_order_with(col_major_blocks=True)),
    "special tokens after the patches": ("spatial_token_order",
                                         _spatial_order_with(special_last=True)),
    "spatial output left in the spatial order": ("spatial_tile_sparse_attention",
                                                 _spatial_attention_not_unpermuted),
    "sparse backward drops the row term D": ("tile_sparse_attention_backward",
                                             _sparse_bwd_with(no_d=True)),
    "landmark gradient not spread over its tile": ("tile_sparse_attention_backward",
                                                   _sparse_bwd_with(no_spread=True)),
    "dv from the logit gradient": ("tile_sparse_attention_backward",
                                   _sparse_bwd_with(dv_from_dl=True)),
    "dq without the softmax scale": ("tile_sparse_attention_backward",
                                     _sparse_bwd_with(dq_no_scale=True)),
    "linear backward without phi'": ("linear_attention_backward", _linear_bwd_with(no_dphi=True)),
    "linear backward normaliser sign": ("linear_attention_backward",
                                        _linear_bwd_with(dden_sign=True)),
    "linear backward drops the bias gradient": ("linear_attention_backward",
                                                _linear_bwd_with(no_db=True)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(zo, attr, bad)
    caught = []
    for pin in ALL_PINS:
        try:
            pin()
        except Exception as e:  # AssertionError or a crash both count as caught
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"no pin notices the planted mistake '{name}'"
