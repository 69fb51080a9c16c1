"""CPU oracle for Zebra3D's layerwise hybrid global attention.

TEST INFRASTRUCTURE ONLY. This module is the plain, slow, obviously correct
reference that the HIP path is checked against. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the library and its Python binding never do, and they share no
code with it (the seeded input generators are the only common module).

Everything is NumPy float64, one step per definition, in the order the pages
state it, with no blocking, fusion or reordering of any sum. Query rows are
independent, so functions that loop over rows or tiles do so only to keep
memory bounded; that changes no arithmetic.

Sources. Citations name the page by its title and host, then the part of it:
  [paper page] "Zebra3D: Efficient Hybrid Foundation Models For Scalable 3D
               Reconstruction", thelatestinai.com paper page
  [news page]  "Zebra3D speeds up 3D reconstruction by up to 7.1x on 1024
               frames without training from scratch", news.hamidun.com
  [synopsis]   "3D reconstruction drops dense attention layer by layer: up to
               5.6x end-to-end speedup at 1,024 views", ai4snews.wisdomeyes.cn

Readings taken where the pages are silent (each is listed again where used):
  R1 tiles are contiguous runs of the token order; the last tile may be short
     and its mean is over its valid tokens only.
  R2 tile selection: score s_ij = mean(Q_tile_i) . mean(K_tile_j) (unscaled),
     keep the top_k key tiles per query tile under the order (score
     descending, tile index ascending); the kept list is returned ascending.
  R3 a landmark is one ordinary softmax column with key mean(K_tile_j) and
     value mean(V_tile_j), logit scale * q . kbar_j, with no multiplicity term;
     only omitted tiles (j not kept) contribute a landmark.
  R4 the linear feature map is phi(x) = elu(x) + 1, with no scale and no
     epsilon in the normaliser; "linear-centered" is read as the centred least
     squares fit (with intercept) of a per-head, per-channel affine map.
  R5 the fit target is dense softmax attention of the same stage at sampled
     queries; a channel whose inputs do not vary gets scale 0 and bias mean(y).

Operator variants of the pages' ablations ([paper page] Table 3(a) and (b);
appendix Tables 15-17: block or tile sparse, each with and without landmark),
off by default:
  V1 without landmarks: omitted tiles are dropped; softmax runs over the
     tokens of the kept tiles only.
  V2 landmark log count: a landmark stands for the n_j valid tokens of its
     tile, so its logit gains ln(n_j) (the short last tile counts its valid
     tokens).
  V3 uncentered fit: the map through the origin, a = sum x y / sum x^2, b = 0.
  V4 spatial tiles ("selected spatial tiles", [paper page] abstract; "Tile
     sparse" vs "Block sparse", appendix Tables 15-17): the tokens are first
     put in a spatial order and tiles are contiguous runs of that order. Per
     view (n_special leading tokens, then a grid_h x grid_w row-major patch
     grid): the special tokens, then the patches in s x s blocks taken in
     raster order of blocks, each block row-major (edge blocks are smaller).

Gradients (for the optional refinement, [paper page] Tables 18-19: the
converted model can be refined with a frozen teacher): the backward passes of
the two operators for a given output gradient, with the tile selection held
fixed (top-k is not differentiable). A landmark's key and value are tile
means, so each token of tile j receives 1/n_j of its landmark's gradient.

Parity status: every function on the attention path is pinned by
``tests/oracle_pins.py`` against closed forms, library routines or brute
force. ``mean_attention_sparsity`` (bookkeeping outside the path) is pinned
by a column-by-column count over small stacks through ``attention_columns``,
by the paper page's Table 6 layer roles, and by the pages' "about 79%" and
"about 94%" figures.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "tile_bounds", "pool_tiles", "block_scores", "select_top_tiles",
    "select_tiles", "attention_columns", "tile_sparse_attention_tile",
    "tile_sparse_attention", "dense_attention", "elu_plus_one",
    "linear_attention", "fit_affine", "fit_scale_only", "affine_apply",
    "mean_attention_sparsity", "block_attention_mass",
    "retained_mass", "top_mass", "spatial_token_order", "spatial_tile_sparse_attention",
    "tile_sparse_attention_backward", "linear_attention_backward",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------
# tiles and landmarks
# ----------------------------------------------------------------------------

def tile_bounds(n_tokens: int, tile: int):
    """Token ranges [start, end) of the contiguous tiles of a sequence (reading R1).

    The paper page (Figure 8 caption) measures attention on 64x64 token
    blocks; tiles here are runs of ``tile`` consecutive tokens, the last one
    possibly short.
    """
    if tile <= 0:
        raise ValueError("tile must be positive")
    return [(s, min(s + tile, n_tokens)) for s in range(0, n_tokens, tile)]


def pool_tiles(x, tile: int) -> np.ndarray:
    """Mean over the valid tokens of every tile: [N][d] -> [T][d].

    Omitted tiles are summarised by the mean key and mean value of their
    tokens ([paper page] Figure 1 caption; [news page] "How Zebra3D works",
    landmark summaries of unselected regions). The same means of the query
    tiles feed the tile scores (reading R2).
    """
    x = _f64(x)
    bounds = tile_bounds(x.shape[0], tile)
    out = np.zeros((len(bounds), x.shape[1]), dtype=np.float64)
    for t, (s, e) in enumerate(bounds):
        out[t] = x[s:e].sum(axis=0) / (e - s)
    return out


def block_scores(qbar, kbar) -> np.ndarray:
    """s_ij = qbar_i . kbar_j, unscaled (reading R2): [Tq][d] x [Tk][d] -> [Tq][Tk]."""
    return _f64(qbar) @ _f64(kbar).T


def select_top_tiles(scores_row, top_k: int) -> np.ndarray:
    """Kept key tiles of one query tile, ascending (reading R2).

    The tile-sparse stage computes only selected blocks ([news page] "How
    Zebra3D works"). Ranking is by score, highest first; equal scores go to
    the lower tile index. The kept set is returned in ascending index order.
    """
    s = _f64(scores_row)
    if not 0 <= top_k <= s.shape[0]:
        raise ValueError("top_k out of range")
    idx = np.arange(s.shape[0])
    order = np.lexsort((idx, -s))  # primary: -score ascending; secondary: index
    return np.sort(order[:top_k]).astype(np.int64)


def select_tiles(qbar, kbar, top_k: int) -> np.ndarray:
    """Kept tiles of every query tile: [Tq][top_k] int64, each row ascending."""
    s = block_scores(qbar, kbar)
    if s.shape[0] == 0:
        return np.zeros((0, top_k), dtype=np.int64)
    return np.stack([select_top_tiles(s[i], top_k) for i in range(s.shape[0])])


# ----------------------------------------------------------------------------
# tile-sparse softmax attention with mean-key/value landmarks
# ----------------------------------------------------------------------------

def attention_columns(k, v, k_tile: int, kept, landmarks: bool = True,
                      landmark_log_count: bool = False):
    """Keys, values and additive logits of the columns one query tile attends to
    (readings R1, R3).

    Every token of every kept tile, then one landmark (kbar_j, vbar_j) for
    every omitted tile j. Kept tiles keep full softmax interactions and
    omitted tiles become mean-key/value landmarks ([paper page] Figure 1
    caption); the [synopsis] ("Interpretation") calls the kept part exact
    softmax over selected tiles. The additive logit is zero for every column,
    except that under variant V2 a landmark gets ln(n_j), n_j the valid tokens
    of its tile. With landmarks=False (variant V1) the omitted tiles
    contribute nothing. Returns ([C][d] keys, [C][d] values, [C] logits).
    """
    k = _f64(k)
    v = _f64(v)
    bounds = tile_bounds(k.shape[0], k_tile)
    kept = [int(j) for j in kept]
    kept_set = set(kept)
    if len(kept_set) != len(kept):
        raise ValueError("kept tiles must be distinct")
    kbar = pool_tiles(k, k_tile)
    vbar = pool_tiles(v, k_tile)
    keys, vals, bias = [], [], []
    for j in sorted(kept):
        s, e = bounds[j]
        keys.append(k[s:e])
        vals.append(v[s:e])
        bias.append(np.zeros(e - s))
    for j in range(len(bounds)):
        if landmarks and j not in kept_set:
            s, e = bounds[j]
            keys.append(kbar[j:j + 1])
            vals.append(vbar[j:j + 1])
            bias.append(np.full(1, np.log(e - s) if landmark_log_count else 0.0))
    if not keys:
        return np.zeros((0, k.shape[1])), np.zeros((0, v.shape[1])), np.zeros(0)
    return (np.concatenate(keys, axis=0), np.concatenate(vals, axis=0),
            np.concatenate(bias))


def _softmax_rows(logits: np.ndarray) -> np.ndarray:
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    return w / w.sum(axis=1, keepdims=True)


def tile_sparse_attention_tile(q_rows, k, v, k_tile: int, kept, scale: float,
                               landmarks: bool = True,
                               landmark_log_count: bool = False) -> np.ndarray:
    """Output of the queries of one query tile: softmax(scale q C_k^T + bias) C_v.

    bias is zero except under variant V2 (attention_columns).
    """
    q_rows = _f64(q_rows)
    ck, cv, bias = attention_columns(k, v, k_tile, kept, landmarks, landmark_log_count)
    return _softmax_rows(scale * (q_rows @ ck.T) + bias[None, :]) @ cv


def tile_sparse_attention(q, k, v, q_tile: int, k_tile: int, top_k: int, scale: float,
                          sel=None, landmarks: bool = True, landmark_log_count: bool = False):
    """Tile-sparse stage over all heads: [H][Nq][d], [H][Nk][d] x2 -> ([H][Nq][d], sel).

    ``sel`` ([H][Tq][top_k]) replaces the oracle's own selection when given,
    which lets the attention step be checked on another implementation's
    choice of tiles. ``landmarks`` and ``landmark_log_count`` select the
    variants V1 and V2.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    heads, n_q, _ = q.shape
    out = np.zeros((heads, n_q, v.shape[2]), dtype=np.float64)
    sels = []
    for h in range(heads):
        if sel is None:
            sel_h = select_tiles(pool_tiles(q[h], q_tile), pool_tiles(k[h], k_tile), top_k)
        else:
            sel_h = np.asarray(sel[h])
        sels.append(sel_h)
        for i, (s, e) in enumerate(tile_bounds(n_q, q_tile)):
            out[h, s:e] = tile_sparse_attention_tile(q[h, s:e], k[h], v[h], k_tile,
                                                     sel_h[i], scale, landmarks,
                                                     landmark_log_count)
    return out, np.stack(sels) if sels else np.zeros((0, 0, top_k), dtype=np.int64)


def tile_sparse_attention_backward(q, k, v, q_tile: int, k_tile: int, sel, scale: float, dout,
                                   landmarks: bool = True, landmark_log_count: bool = False):
    """Gradients (dq, dk, dv) of sum(dout * out) for tile_sparse_attention on the
    selection ``sel`` ([H][Tq][top_k], held fixed). [H][N][d] arrays.

    Per query row with columns c (attention_columns), logits l_c and P = softmax(l):
        dP_c = dout . v_c,  D = sum_c P_c dP_c,  dl_c = P_c (dP_c - D),
        dq = scale sum_c dl_c k_c,  dk_c = scale dl_c q,  dv_c = P_c dout.
    Kept columns are tokens; a landmark column's dk_c and dv_c go to every
    token of its tile, divided by the tile's token count.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    heads, n_q, d = q.shape
    n_k = k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    kb = tile_bounds(n_k, k_tile)
    for h in range(heads):
        for i, (s0, e0) in enumerate(tile_bounds(n_q, q_tile)):
            kept = sorted(int(j) for j in sel[h][i])
            ck, cv, bias = attention_columns(k[h], v[h], k_tile, kept, landmarks,
                                             landmark_log_count)
            # the token (or tile) each column belongs to
            owner = [("tok", t) for j in kept for t in range(*kb[j])]
            if landmarks:
                owner += [("lm", j) for j in range(len(kb)) if j not in set(kept)]
            p = _softmax_rows(scale * (q[h, s0:e0] @ ck.T) + bias[None, :])
            dp = dout[h, s0:e0] @ cv.T
            dl = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[h, s0:e0] = scale * (dl @ ck)
            dck = scale * (dl.T @ q[h, s0:e0])
            dcv = p.T @ dout[h, s0:e0]
            for c, (kind, idx) in enumerate(owner):
                if kind == "tok":
                    dk[h, idx] += dck[c]
                    dv[h, idx] += dcv[c]
                else:
                    a, b = kb[idx]
                    dk[h, a:b] += dck[c] / (b - a)
                    dv[h, a:b] += dcv[c] / (b - a)
    return dq, dk, dv


def dense_attention(q, k, v, scale: float, row_block: int = 1024) -> np.ndarray:
    """Exact softmax attention of every query over every key, one head: [Nq][d] -> [Nq][d].

    This is the dense global attention that the hybrid replaces ([news page]
    "Where scaling breaks down": the tokens of all frames attend to each other)
    and the target of the affine fit (reading R5). Rows are independent; they
    are taken ``row_block`` at a time to bound memory.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    out = np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    for s in range(0, q.shape[0], row_block):
        e = min(q.shape[0], s + row_block)
        out[s:e] = _softmax_rows(scale * (q[s:e] @ k.T)) @ v
    return out


# ----------------------------------------------------------------------------
# linear attention and the closed-form affine fit
# ----------------------------------------------------------------------------

def elu_plus_one(x) -> np.ndarray:
    """phi(x) = x + 1 for x > 0, exp(x) otherwise (reading R4)."""
    x = _f64(x)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def linear_attention(q, k, v, aff_scale=None, aff_bias=None):
    """Linear attention of one head, then the per-channel affine map (reading R4).

    Tolerant stages run linear(-centered) attention ([paper page] Abstract;
    [news page] "How Zebra3D works"). With phi = elu + 1:
        S = sum_n phi(k_n) v_n^T,  z = sum_n phi(k_n),
        o_n = (phi(q_n)^T S) / (phi(q_n)^T z),
    then out = a * o + b per channel ([paper page] Table 3(a), "Linear-centered
    + fit"). Returns (out, S, z).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    fq = elu_plus_one(q)
    fk = elu_plus_one(k)
    state = fk.T @ v
    z = fk.sum(axis=0)
    o = (fq @ state) / (fq @ z)[:, None]
    if aff_scale is not None or aff_bias is not None:
        o = affine_apply(o, aff_scale, aff_bias)
    return o, state, z


def linear_attention_backward(q, k, v, dout, aff_scale=None, aff_bias=None):
    """Gradients of sum(dout * out) for linear_attention of one head:
    (dq, dk, dv, da, db), [N][d] and [d].

    With num = phi(q) S, den = phi(q) . z, o = num / den, out = a * o + b:
        da = sum_n dout * o,  db = sum_n dout,  do = a * dout,
        dnum = do / den,  dden = -(do . o) / den,
        dq = (S dnum + z dden) * phi'(q),
        dS = sum_n phi(q_n) dnum_n^T,  dz = sum_n phi(q_n) dden_n,
        dv_m = dS^T phi(k_m),  dk_m = (dS v_m + dz) * phi'(k_m),
    phi'(x) = 1 for x > 0, exp(x) otherwise.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    d = v.shape[1]
    a = np.ones(d) if aff_scale is None else _f64(aff_scale)
    fq, fk = elu_plus_one(q), elu_plus_one(k)
    dfq = np.where(q > 0, 1.0, np.exp(np.minimum(q, 0.0)))
    dfk = np.where(k > 0, 1.0, np.exp(np.minimum(k, 0.0)))
    state = fk.T @ v
    z = fk.sum(axis=0)
    den = fq @ z
    o = (fq @ state) / den[:, None]
    da = (dout * o).sum(axis=0)
    db = dout.sum(axis=0)
    do = dout * a[None, :]
    dnum = do / den[:, None]
    dden = -(do * o).sum(axis=1) / den
    dq = (dnum @ state.T + dden[:, None] * z[None, :]) * dfq
    d_state = fq.T @ dnum
    dz = fq.T @ dden
    dv = fk @ d_state
    dk = (v @ d_state.T + dz[None, :]) * dfk
    return dq, dk, dv, da, db


def affine_apply(o, aff_scale=None, aff_bias=None) -> np.ndarray:
    """out = a * o + b, per channel; a defaults to 1 and b to 0."""
    o = _f64(o)
    a = np.ones(o.shape[-1]) if aff_scale is None else _f64(aff_scale)
    b = np.zeros(o.shape[-1]) if aff_bias is None else _f64(aff_bias)
    return o * a + b


def fit_affine(x, y, degenerate_rel: float = 1e-30):
    """Closed-form least squares a, b per channel: min sum_i (a x_ic + b - y_ic)^2.

    The linear components are fitted by a closed-form affine map with no
    gradient descent ([news page] "How Zebra3D works"; [paper page] Table 3(a)
    contrasts an uncentered fit with the centred fit used here, reading R4).
    x is the linear output before the map and y the dense output at the same
    M queries, both [M][d]. Centred form of the 2x2 normal equations:
        a = sum (x - xbar)(y - ybar) / sum (x - xbar)^2,  b = ybar - a xbar.
    A channel with sum (x - xbar)^2 <= degenerate_rel * M gets a = 0, b = ybar
    (reading R5). Returns (a, b, n_degenerate).
    """
    x, y = _f64(x), _f64(y)
    m = x.shape[0]
    if m == 0:
        raise ValueError("fit needs at least one sample")
    xbar = x.sum(axis=0) / m
    ybar = y.sum(axis=0) / m
    dx = x - xbar
    sxx = (dx * dx).sum(axis=0)
    sxy = (dx * (y - ybar)).sum(axis=0)
    ok = sxx > degenerate_rel * m
    a = np.where(ok, sxy / np.where(ok, sxx, 1.0), 0.0)
    b = ybar - a * xbar
    return a, b, int((~ok).sum())


def fit_scale_only(x, y, degenerate_rel: float = 1e-30):
    """Variant V3, the uncentered fit: per channel min over a of sum_i (a x_ic - y_ic)^2.

    [paper page] Table 3(a) lists "Linear, uncentered fit" between no fit and
    the centred fit; read here as the least-squares map through the origin:
        a = sum x y / sum x^2,  b = 0.
    A channel with sum x^2 <= degenerate_rel * M gets a = 0. Returns
    (a, b, n_degenerate) like fit_affine.
    """
    x, y = _f64(x), _f64(y)
    m = x.shape[0]
    if m == 0:
        raise ValueError("fit needs at least one sample")
    sxx = (x * x).sum(axis=0)
    sxy = (x * y).sum(axis=0)
    ok = sxx > degenerate_rel * m
    a = np.where(ok, sxy / np.where(ok, sxx, 1.0), 0.0)
    return a, np.zeros_like(a), int((~ok).sum())


def spatial_token_order(n_views: int, n_special: int, grid_h: int, grid_w: int,
                        block: int) -> np.ndarray:
    """Variant V4: position i of the spatial order holds original token order[i]."""
    per_view = n_special + grid_h * grid_w
    order = []
    for view in range(n_views):
        base = view * per_view
        order.extend(base + t for t in range(n_special))
        for r0 in range(0, grid_h, block):
            for c0 in range(0, grid_w, block):
                for r in range(r0, min(grid_h, r0 + block)):
                    for c in range(c0, min(grid_w, c0 + block)):
                        order.append(base + n_special + r * grid_w + c)
    return np.asarray(order, dtype=np.int64)


def spatial_tile_sparse_attention(q, k, v, order, q_tile: int, k_tile: int, top_k: int,
                                  scale: float, sel=None, **variant):
    """Tile-sparse attention with spatial tiles (V4): tokens in ``order`` (the same
    for queries and keys), tiles as contiguous runs of it, the output returned in
    the original token order. ``sel`` refers to tiles of the spatial order."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    order = np.asarray(order, dtype=np.int64)
    out_perm, sel = tile_sparse_attention(q[:, order], k[:, order], v[:, order], q_tile, k_tile,
                                          top_k, scale, sel=sel, **variant)
    out = np.empty_like(out_perm)
    out[:, order] = out_perm
    return out, sel


# ----------------------------------------------------------------------------
# bookkeeping of the xL/yS budget
# ----------------------------------------------------------------------------

def mean_attention_sparsity(linear_frac: float, keep_frac: float, k_tile: int) -> float:
    """Fraction of attention entries not computed exactly, averaged over stages.

    In the xL/yS shorthand x is the fraction of layers that use linear
    attention and y the sparsity of attention rows in the other layers
    ([paper page] Table 20 and Table 21 captions). A linear stage computes no
    softmax entries; a tile-sparse stage computes the kept fraction of keys
    plus one landmark column per omitted tile of ``k_tile`` keys.
    """
    dense_frac = keep_frac + (1.0 - keep_frac) / k_tile
    return linear_frac + (1.0 - linear_frac) * (1.0 - dense_frac)


# ----------------------------------------------------------------------------
# selection-quality diagnostic
# ----------------------------------------------------------------------------

def block_attention_mass(q, k, q_tile: int, k_tile: int, scale: float,
                         row_block: int = 1024) -> np.ndarray:
    """Attention mass of every (query tile, key tile) block under dense softmax, one head.

    The pages measure how much attention mass the highest-mass 20% of 64x64
    token blocks retain ([paper page] Figure 2 caption, panel (b); Figure 8
    caption). For query tile i and key tile j (reading R1 tiles):
        M[i][j] = (1 / |Q_i|) sum_{q in Q_i} sum_{k in K_j} softmax_q(scale q . k),
    so every row of M sums to one. [Nq][d], [Nk][d] -> [Tq][Tk].
    """
    q, k = _f64(q), _f64(k)
    qb = tile_bounds(q.shape[0], q_tile)
    kb = tile_bounds(k.shape[0], k_tile)
    mass = np.zeros((len(qb), len(kb)), dtype=np.float64)
    # per-query block sums, then the mean over each query tile
    col = np.zeros((q.shape[0], len(kb)), dtype=np.float64)
    for s0 in range(0, q.shape[0], row_block):
        e0 = min(q.shape[0], s0 + row_block)
        p = _softmax_rows(scale * (q[s0:e0] @ k.T))
        for j, (a, b) in enumerate(kb):
            col[s0:e0, j] = p[:, a:b].sum(axis=1)
    for i, (a, b) in enumerate(qb):
        mass[i] = col[a:b].sum(axis=0) / (b - a)
    return mass


def retained_mass(mass, sel) -> np.ndarray:
    """Mass each query tile keeps on its selected key tiles: sum_{j in sel_i} M[i][j]."""
    mass = _f64(mass)
    sel = np.asarray(sel, dtype=np.int64)
    return np.take_along_axis(mass, sel, axis=1).sum(axis=1)


def top_mass(mass, top_k: int) -> np.ndarray:
    """Mass of the top_k highest-mass key tiles of each query tile (the pages' oracle selection)."""
    mass = _f64(mass)
    return -np.sort(-mass, axis=1)[:, :top_k].sum(axis=1)
