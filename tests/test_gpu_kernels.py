"""GPU parity of every libzebra entry point against the CPU oracle, small and ragged shapes.

All calls go through the C ABI (the ctypes binding). Inputs are seeded
synthetic draws; the oracle receives the same bf16-rounded values in float64.
"""

import numpy as np
import pytest
import torch

import oracle.zebra_oracle as zo
import linear_hybrid_attention_zebra_amd as zb
from linear_hybrid_attention_zebra_amd import stage, synth
from parity_util import assert_close, assert_grad_close, bf16_gpu, check_selection, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _clustered(seed, heads, n_q, n_kv, q_tile, k_tile, n_hot):
    q, k, v, _ = synth.clustered_qkv_np(seed, heads, n_q, 64, q_tile, k_tile, n_hot, n_kv=n_kv)
    return synth.bf16_round(q), synth.bf16_round(k), synth.bf16_round(v)


# ----------------------------------------------------------------------------
# pool
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("heads,n,tile,layout", [
    (2, 128, 32, "hnd"), (3, 70, 32, "hnd"), (2, 300, 64, "nhd"), (1, 1, 64, "hnd"),
    (2, 1000, 128, "nhd"), (2, 65, 1, "hnd"), (2, 3000, 1024, "hnd"), (16, 21984, 64, "hnd"),
])
def test_pool_parity(heads, n, tile, layout):
    print(f"[case] pool H={heads} N={n} tile={tile} {layout}", flush=True)
    rng = np.random.default_rng(n + tile)
    x = synth.bf16_round(rng.standard_normal((heads, n, 64)).astype(np.float32) * 3)
    xg = bf16_gpu(x)
    if layout == "nhd":
        xg = xg.permute(1, 0, 2).contiguous().permute(1, 0, 2)  # token-major storage
    got = zb.zebra_pool_landmarks(xg, tile)
    torch.cuda.synchronize()
    ref = np.stack([zo.pool_tiles(x[h], tile) for h in range(heads)])
    err = np.max(np.abs(to_f64(got) - ref) / np.maximum(1.0, np.abs(ref)))
    assert err <= 2e-6, f"pool relative error {err:.2e}"


def test_pool_empty_is_noop():
    x = torch.empty((2, 0, 64), dtype=torch.bfloat16, device=DEV)
    out = zb.zebra_pool_landmarks(x, 64)
    assert out.shape == (2, 0, 64)


# ----------------------------------------------------------------------------
# select
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("tq,tk,top_k", [(7, 300, 1), (7, 300, 69), (7, 300, 300), (5, 4, 1),
                                         (3, 9000, 1320), (4, 21984, 1320)])
def test_select_parity(tq, tk, top_k):
    print(f"[case] select Tq={tq} Tk={tk} k={top_k}", flush=True)
    rng = np.random.default_rng(tk + top_k)
    qbar = rng.standard_normal((2, tq, 64)).astype(np.float32)
    kbar = rng.standard_normal((2, tk, 64)).astype(np.float32)
    sel = zb.zebra_select_tiles(torch.from_numpy(qbar).to(DEV), torch.from_numpy(kbar).to(DEV),
                                top_k)
    torch.cuda.synchronize()
    scores = np.stack([zo.block_scores(qbar[h], kbar[h]) for h in range(2)])
    swaps = check_selection(sel.cpu().numpy(), scores, top_k)
    print(f"[parity] select near-tie rows with swaps: {swaps}", flush=True)


def test_select_exact_ties_go_to_lowest_index():
    """Duplicated key means tie bitwise; the lower tile index must win every tie."""
    rng = np.random.default_rng(7)
    base = rng.integers(-3, 4, size=(6, 64)).astype(np.float32)
    kbar = base[rng.integers(0, 6, size=500)][None]  # 500 tiles, 6 distinct rows
    qbar = rng.integers(-2, 3, size=(1, 9, 64)).astype(np.float32)
    for top_k in (1, 37, 250, 499):
        sel = zb.zebra_select_tiles(torch.from_numpy(qbar).to(DEV), torch.from_numpy(kbar).to(DEV),
                                    top_k).cpu().numpy()
        ref = zo.select_tiles(qbar[0], kbar[0], top_k)
        assert np.array_equal(sel[0], ref), f"top_k={top_k}"


def test_select_all_equal_scores():
    qbar = torch.zeros((1, 3, 64), device=DEV)
    kbar = torch.ones((1, 2000, 64), device=DEV)
    sel = zb.zebra_select_tiles(qbar, kbar, 700).cpu().numpy()
    assert np.array_equal(sel[0, 0], np.arange(700))


# ----------------------------------------------------------------------------
# tile-sparse attention
# ----------------------------------------------------------------------------

SPARSE_CASES = [
    # (q_tile, k_tile, n_q, n_kv, top_k, n_hot, heads)
    (32, 32, 128, 128, 1, 1, 2),      # the tiny two-view workload
    (64, 64, 300, 300, 2, 2, 2),      # ragged last tiles on both sides
    (128, 64, 300, 450, 3, 2, 2),     # 128-token query tiles, Nq != Nk
    (32, 32, 200, 97, 2, 1, 3),
    (64, 32, 130, 200, 3, 2, 2),
    (128, 32, 257, 300, 4, 2, 1),
    (64, 64, 64, 64, 1, 1, 1),        # a single key tile
    (64, 64, 1000, 1000, 16, 3, 2),   # every tile kept: sel given, no landmarks
    (64, 64, 2000, 2000, 7, 3, 2),
]


@pytest.mark.parametrize("case", SPARSE_CASES, ids=[str(c) for c in SPARSE_CASES])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_sparse_stage_parity(case, out_dtype):
    q_tile, k_tile, n_q, n_kv, top_k, n_hot, heads = case
    print(f"[case] sparse {case} {out_dtype}", flush=True)
    q, k, v = _clustered(sum(case), heads, n_q, n_kv, q_tile, k_tile, n_hot)
    qg, kg, vg = bf16_gpu(q), bf16_gpu(k), bf16_gpu(v)
    bufs = stage.SparseBuffers.allocate(heads, n_q, n_kv, q_tile, k_tile, top_k, DEV, out_dtype)
    stage.sparse_stage(qg, kg, vg, q_tile, k_tile, top_k, 0.125, bufs)
    torch.cuda.synchronize()
    sel = bufs.sel.cpu().numpy()
    scores = np.stack([zo.block_scores(zo.pool_tiles(q[h], q_tile), zo.pool_tiles(k[h], k_tile))
                       for h in range(heads)])
    swaps = check_selection(sel, scores, top_k)
    ref, _ = zo.tile_sparse_attention(q, k, v, q_tile, k_tile, top_k, 0.125, sel=sel)
    assert_close(bufs.out, ref, f"sparse {case}")
    print(f"[parity] near-tie swaps {swaps}", flush=True)


# With query tiles of at most 64, key ranges of at least 1,024 tiles of 64
# (2,048 of 32) run as split keys: items per (head, key chunk of 512 tiles of
# 64 / 1,024 of 32, query tile). With 64-query and 64-key tiles the landmark
# pass merges the chunks' partials; other tiles merge them in a combine kernel.
SPLIT_CASES = [
    # (q_tile, k_tile, n_q, n_kv, top_k, n_hot, heads)
    (64, 64, 300, 65536 + 333, 1, 1, 2),     # 3 chunks, ragged tail; most chunks keep nothing
    (64, 64, 300, 65536 + 333, 206, 3, 2),   # 20% kept
    (64, 64, 130, 65536, 1023, 2, 1),        # 2 whole chunks; all but one tile kept
    (64, 32, 257, 70000, 440, 2, 1),         # 32-key tiles: 3 chunks of 1,024 tiles
    (128, 64, 257, 70000, 220, 2, 1),        # 128-query tiles: one pass, no split
    (32, 64, 100, 98304, 300, 2, 2),         # 32-query tiles
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[str(c) for c in SPLIT_CASES])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_split_keys_parity(case, out_dtype):
    test_sparse_stage_parity(case, out_dtype)


def test_split_keys_both_softmax_references():
    """Split keys with some query tiles on the running-maximum path."""
    n_q, n_kv = 300, 65536 + 100
    print(f"[case] split keys reference paths Nq={n_q} Nk={n_kv}", flush=True)
    q, k, v = _clustered(23, 2, n_q, n_kv, 64, 64, 3)
    q = q.copy()
    q[:, 64:192] *= 8.0  # query tiles 1 and 2: bound far above the fast-path limit
    q = synth.bf16_round(q)
    bufs = stage.SparseBuffers.allocate(2, n_q, n_kv, 64, 64, 100, DEV, torch.float32)
    stage.sparse_stage(bf16_gpu(q), bf16_gpu(k), bf16_gpu(v), 64, 64, 100, 0.125, bufs)
    torch.cuda.synchronize()
    ref, _ = zo.tile_sparse_attention(q, k, v, 64, 64, 100, 0.125, sel=bufs.sel.cpu().numpy())
    assert_close(bufs.out, ref, "split keys reference paths")


def test_split_keys_is_deterministic():
    q, k, v = _clustered(12, 1, 200, 70000, 64, 64, 3)
    outs = []
    for _ in range(2):
        bufs = stage.sparse_stage(bf16_gpu(q), bf16_gpu(k), bf16_gpu(v), 64, 64, 220, 0.125)
        outs.append(bufs.out.clone())
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("top_k,q_mul", [(100, 1.0), (2, 1.0), (100, 8.0)],
                         ids=["k100", "k2", "k100-running-max"])
def test_split_keys_phased_walks(top_k, q_mul):
    """Split keys with enough items (4 heads x 3 chunks x 500 query tiles, several
    times what the device runs at once) that every item walks its kept tiles from
    a phase-dependent start, wrapping around (top_k 2: most chunks keep at most
    one tile and do not rotate). The last chunk holds 501 tiles and the short
    36-token last key tile, which must stay the last step of the walks that keep
    it. Every selection row against the oracle's pooled scores; every output
    element of head 0 and up to 48 rows of the other heads that keep the short
    tile against the oracle on the GPU's selection; two runs bitwise equal. With the
    queries times 8 (exact in bf16) every item's logit bound exceeds the fixed-
    reference limit and the walks run on the running-maximum path."""
    heads, n_q, n_kv = 4, 32000, 2 * 32768 + 500 * 64 + 36
    print(f"[case] phased split keys H={heads} Nq={n_q} Nk={n_kv} top_k={top_k} "
          f"q x{q_mul:g}", flush=True)
    q, k, v = _clustered(31, heads, n_q, n_kv, 64, 64, 3)
    q = synth.bf16_round(q * np.float32(q_mul))
    outs = []
    for _ in range(2):
        bufs = stage.SparseBuffers.allocate(heads, n_q, n_kv, 64, 64, top_k, DEV)
        stage.sparse_stage(bf16_gpu(q), bf16_gpu(k), bf16_gpu(v), 64, 64, top_k, 0.125, bufs)
        outs.append(bufs.out.clone())
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]), "phased walks are not repeatable"
    sel = bufs.sel.cpu().numpy()
    scores = np.stack([zo.block_scores(zo.pool_tiles(q[h], 64), zo.pool_tiles(k[h], 64))
                       for h in range(heads)])
    swaps = check_selection(sel, scores, top_k)
    ref, _ = zo.tile_sparse_attention(q[:1], k[:1], v[:1], 64, 64, top_k, 0.125, sel=sel[:1])
    assert_close(outs[0][:1], ref, "phased split keys, head 0")
    t_k = -(-n_kv // 64)
    tail_rows = np.argwhere(np.any(sel[1:] == t_k - 1, axis=2))
    print(f"[case] rows of heads 1-3 keeping the short last tile: {len(tail_rows)}", flush=True)
    assert len(tail_rows) >= (48 if top_k > 50 else 1)
    n_pick = min(48, len(tail_rows))
    for hh, i in tail_rows[np.random.default_rng(5).choice(len(tail_rows), n_pick, replace=False)]:
        h = int(hh) + 1
        s0, e0 = 64 * int(i), min(n_q, 64 * int(i) + 64)
        r = zo.tile_sparse_attention_tile(q[h, s0:e0], k[h], v[h], 64, sel[h, i], 0.125)
        assert_close(outs[0][h, s0:e0], r, f"phased split keys head {h} tile {i}")
    print(f"[parity] near-tie swaps {swaps}", flush=True)


def test_split_keys_long_chunks_phased_walks():
    """Key ranges of at least 4 x 65,536 keys split into 65,536-key chunks (here 4 of
    1,024 tiles and one of 301 ending in a 36-token tile), with phased walks (2
    heads x 5 chunks x 410 query tiles). Every selection row against the oracle's
    pooled scores; 24 rows that keep the short last tile and 24 other rows against
    the oracle on the GPU's selection; two runs bitwise equal."""
    heads, n_q, n_kv, top_k = 2, 410 * 64, 4 * 65536 + 300 * 64 + 36, 220
    print(f"[case] long-chunk split keys H={heads} Nq={n_q} Nk={n_kv} top_k={top_k}", flush=True)
    q, k, v = _clustered(37, heads, n_q, n_kv, 64, 64, 3)
    outs = []
    for _ in range(2):
        bufs = stage.SparseBuffers.allocate(heads, n_q, n_kv, 64, 64, top_k, DEV)
        stage.sparse_stage(bf16_gpu(q), bf16_gpu(k), bf16_gpu(v), 64, 64, top_k, 0.125, bufs)
        outs.append(bufs.out.clone())
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]), "long-chunk phased walks are not repeatable"
    sel = bufs.sel.cpu().numpy()
    scores = np.stack([zo.block_scores(zo.pool_tiles(q[h], 64), zo.pool_tiles(k[h], 64))
                       for h in range(heads)])
    swaps = check_selection(sel, scores, top_k)
    t_k = -(-n_kv // 64)
    keeps = np.any(sel == t_k - 1, axis=2)
    rng = np.random.default_rng(38)
    tail_rows, other_rows = np.argwhere(keeps), np.argwhere(~keeps)
    print(f"[case] rows keeping the short last tile: {len(tail_rows)}", flush=True)
    assert len(tail_rows) >= 24
    rows = np.concatenate([tail_rows[rng.choice(len(tail_rows), 24, replace=False)],
                           other_rows[rng.choice(len(other_rows), 24, replace=False)]])
    for h, i in rows:
        s0 = 64 * int(i)
        r = zo.tile_sparse_attention_tile(q[h, s0:s0 + 64], k[h], v[h], 64, sel[h, i], 0.125)
        assert_close(outs[0][h, s0:s0 + 64], r, f"long-chunk split keys head {h} tile {i}")
    print(f"[parity] near-tie swaps {swaps}", flush=True)


@pytest.mark.parametrize("q_tile,k_tile,n_q,n_kv", [(64, 64, 300, 300), (128, 64, 130, 700),
                                                    (32, 32, 100, 65)])
def test_dense_mode_parity(q_tile, k_tile, n_q, n_kv):
    """sel = NULL with top_k = T_k is exact dense softmax attention."""
    print(f"[case] dense q_tile={q_tile} k_tile={k_tile} Nq={n_q} Nk={n_kv}", flush=True)
    q, k, v = _clustered(5, 2, n_q, n_kv, q_tile, k_tile, 2)
    t_k = -(-n_kv // k_tile)
    out = zb.zebra_tile_sparse_attn(bf16_gpu(q), bf16_gpu(k), bf16_gpu(v), None, None, None,
                                    q_tile, k_tile, t_k, 0.125, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = np.stack([zo.dense_attention(q[h], k[h], v[h], 0.125) for h in range(2)])
    assert_close(out, ref, "dense mode")


@pytest.mark.parametrize("kind", ["mixed_q", "large_v", "dense_large_q"])
def test_sparse_both_softmax_references(kind):
    """Items whose logit bound is loose (large |q|) or whose values are huge take
    the running-maximum path; the others the fixed-bound path, in one launch."""
    print(f"[case] sparse reference paths {kind}", flush=True)
    q, k, v = _clustered(21, 2, 700, 700, 64, 64, 3)
    v_scale = 1.0
    if kind == "mixed_q":
        q = q.copy()
        q[:, 128:320] *= 8.0  # query tiles 2..4: bound far above the fast-path limit
        q = synth.bf16_round(q)
    elif kind == "large_v":
        v_scale = 2.0 ** 41
        v = synth.bf16_round(v * v_scale)
    else:
        q = synth.bf16_round(q * 8.0)
    qg, kg, vg = bf16_gpu(q), bf16_gpu(k), bf16_gpu(v)
    if kind == "dense_large_q":
        out = zb.zebra_tile_sparse_attn(qg, kg, vg, None, None, None, 64, 64, 11, 0.125,
                                        out_dtype=torch.float32)
        torch.cuda.synchronize()
        ref = np.stack([zo.dense_attention(q[h], k[h], v[h], 0.125) for h in range(2)])
    else:
        bufs = stage.SparseBuffers.allocate(2, 700, 700, 64, 64, 3, DEV, torch.float32)
        stage.sparse_stage(qg, kg, vg, 64, 64, 3, 0.125, bufs)
        torch.cuda.synchronize()
        out = bufs.out
        ref, _ = zo.tile_sparse_attention(q, k, v, 64, 64, 3, 0.125, sel=bufs.sel.cpu().numpy())
    assert_close(to_f64(out) / v_scale, ref / v_scale, f"reference paths {kind}")


# (q_tile, n, top_k): key rows 192 bytes apart take the 32-query layout for
# every tile shape, including split keys (n >= 2 x 32,768)
STRIDED_CASES = [(64, 250, 2), (128, 300, 2), (64, 65536 + 100, 40)]


@pytest.mark.parametrize("q_tile,n,top_k", STRIDED_CASES, ids=[str(c) for c in STRIDED_CASES])
def test_sparse_strided_layout(q_tile, n, top_k):
    """Token-major [N][H][64] storage for q, k, v and the output."""
    print(f"[case] strided sparse q_tile={q_tile} N={n} top_k={top_k}", flush=True)
    nq = 250 if n > 1000 else n
    q, k, v = _clustered(9, 3, nq, n, q_tile, 64, 2)
    tm = lambda x: bf16_gpu(x).permute(1, 0, 2).contiguous().permute(1, 0, 2)
    qg, kg, vg = tm(q), tm(k), tm(v)
    out = torch.empty((nq, 3, 64), dtype=torch.bfloat16, device=DEV).permute(1, 0, 2)
    bufs = stage.SparseBuffers.allocate(3, nq, n, q_tile, 64, top_k, DEV)
    bufs.out = out
    stage.sparse_stage(qg, kg, vg, q_tile, 64, top_k, 0.125, bufs)
    torch.cuda.synchronize()
    sel = bufs.sel.cpu().numpy()
    ref, _ = zo.tile_sparse_attention(q, k, v, q_tile, 64, top_k, 0.125, sel=sel)
    assert_close(out, ref, "strided sparse")


def test_sparse_is_deterministic():
    q, k, v = _clustered(11, 2, 700, 700, 64, 64, 3)
    outs = []
    for _ in range(2):
        bufs = stage.sparse_stage(bf16_gpu(q), bf16_gpu(k), bf16_gpu(v), 64, 64, 3, 0.125)
        outs.append((bufs.out.clone(), bufs.sel.clone()))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_constant_tiles_closed_form_on_gpu():
    """Key tiles of one repeated key/value: the landmark counts once, a kept
    tile n_j times (pins the single-column landmark reading on the GPU)."""
    rng = np.random.default_rng(3)
    n_kv, bk = 64 * 5 + 20, 64
    t_k = -(-n_kv // bk)
    kap = synth.bf16_round(rng.standard_normal((t_k, 64)).astype(np.float32))
    nu = synth.bf16_round(rng.standard_normal((t_k, 64)).astype(np.float32))
    k = np.repeat(kap, bk, axis=0)[:n_kv][None]
    v = np.repeat(nu, bk, axis=0)[:n_kv][None]
    q = synth.bf16_round(rng.standard_normal((1, 64, 64)).astype(np.float32))
    bufs = stage.sparse_stage(bf16_gpu(q), bf16_gpu(k), bf16_gpu(v), 64, 64, 2, 0.125)
    torch.cuda.synchronize()
    kept = bufs.sel.cpu().numpy()[0, 0]
    n_j = np.array([min(bk, n_kv - j * bk) for j in range(t_k)], dtype=np.float64)
    mult = np.where(np.isin(np.arange(t_k), kept), n_j, 1.0)
    ell = 0.125 * (q[0].astype(np.float64) @ kap.T.astype(np.float64))
    w = mult * np.exp(ell - ell.max(axis=1, keepdims=True))
    expect = (w @ nu) / w.sum(axis=1, keepdims=True)
    assert_close(bufs.out[0], expect, "constant tiles")


# ----------------------------------------------------------------------------
# operator variants: no landmarks, landmark log count
# ----------------------------------------------------------------------------

VARIANT_CASES = [
    # (q_tile, k_tile, n_q, n_kv, top_k, n_hot, heads); every case has a short last key tile
    (64, 64, 300, 300, 2, 2, 2),
    (128, 32, 257, 300, 4, 2, 1),
    (32, 64, 100, 450, 1, 1, 2),
    (64, 64, 300, 65536 + 333, 1, 1, 2),    # split keys: most chunks keep nothing
    (64, 64, 300, 65536 + 333, 206, 3, 1),  # split keys, 20% kept
]
VARIANTS = {"no_landmarks": (1, dict(landmarks=False)),
            "log_count": (2, dict(landmark_log_count=True))}


@pytest.mark.parametrize("variant", sorted(VARIANTS))
@pytest.mark.parametrize("case", VARIANT_CASES, ids=[str(c) for c in VARIANT_CASES])
def test_sparse_variant_parity(case, variant):
    q_tile, k_tile, n_q, n_kv, top_k, n_hot, heads = case
    flags, kw = VARIANTS[variant]
    print(f"[case] sparse variant {variant} {case}", flush=True)
    q, k, v = _clustered(sum(case) + flags, heads, n_q, n_kv, q_tile, k_tile, n_hot)
    bufs = stage.SparseBuffers.allocate(heads, n_q, n_kv, q_tile, k_tile, top_k, DEV,
                                        torch.float32)
    stage.sparse_stage(bf16_gpu(q), bf16_gpu(k), bf16_gpu(v), q_tile, k_tile, top_k, 0.125, bufs,
                       flags=flags)
    torch.cuda.synchronize()
    ref, _ = zo.tile_sparse_attention(q, k, v, q_tile, k_tile, top_k, 0.125,
                                      sel=bufs.sel.cpu().numpy(), **kw)
    assert_close(bufs.out, ref, f"sparse {variant} {case}")


@pytest.mark.parametrize("variant", sorted(VARIANTS))
def test_sparse_variant_running_max_path(variant):
    """Query tiles with a loose logit bound take the running-maximum path."""
    flags, kw = VARIANTS[variant]
    q, k, v = _clustered(31, 2, 700, 700, 64, 64, 3)
    q = q.copy()
    q[:, 128:320] *= 8.0
    q = synth.bf16_round(q)
    bufs = stage.SparseBuffers.allocate(2, 700, 700, 64, 64, 3, DEV, torch.float32)
    stage.sparse_stage(bf16_gpu(q), bf16_gpu(k), bf16_gpu(v), 64, 64, 3, 0.125, bufs, flags=flags)
    torch.cuda.synchronize()
    ref, _ = zo.tile_sparse_attention(q, k, v, 64, 64, 3, 0.125, sel=bufs.sel.cpu().numpy(), **kw)
    assert_close(bufs.out, ref, f"{variant} running-maximum path")


@pytest.mark.parametrize("n_kv", [64 * 5 + 20, 65536 + 100])
def test_log_count_constant_tiles_is_dense_on_gpu(n_kv):
    """Key tiles of one repeated key/value (short last tile): a landmark that counts
    its tile's tokens stands in exactly for the tile, so the output is dense
    attention whatever is kept."""
    rng = np.random.default_rng(5)
    bk = 64
    t_k = -(-n_kv // bk)
    kap = synth.bf16_round(rng.standard_normal((t_k, 64)).astype(np.float32))
    nu = synth.bf16_round(rng.standard_normal((t_k, 64)).astype(np.float32))
    k = np.repeat(kap, bk, axis=0)[:n_kv][None]
    v = np.repeat(nu, bk, axis=0)[:n_kv][None]
    q = synth.bf16_round(rng.standard_normal((1, 128, 64)).astype(np.float32))
    top_k = max(1, t_k // 5)
    bufs = stage.SparseBuffers.allocate(1, 128, n_kv, 64, 64, top_k, DEV, torch.float32)
    stage.sparse_stage(bf16_gpu(q), bf16_gpu(k), bf16_gpu(v), 64, 64, top_k, 0.125, bufs,
                       flags=zb.ZEBRA_SPARSE_LANDMARK_LOG_COUNT)
    torch.cuda.synchronize()
    expect = zo.dense_attention(q[0], k[0], v[0], 0.125)
    assert_close(bufs.out[0], expect, "log-count landmarks, constant tiles")


def test_fit_scale_only_parity():
    rng = np.random.default_rng(6)
    heads, m = 4, 4096
    x = rng.standard_normal((heads, m, 64)).astype(np.float32) * 0.01
    y = (0.8 * x + 0.003 * rng.standard_normal((heads, m, 64)) + 0.001).astype(np.float32)
    x[2, :, 7] = 0.0  # a degenerate channel
    a, b, nd = zb.zebra_fit_scale_only(torch.from_numpy(x).to(DEV), torch.from_numpy(y).to(DEV))
    torch.cuda.synchronize()
    for h in range(heads):
        ra, rb, _ = zo.fit_scale_only(x[h], y[h])
        np.testing.assert_allclose(to_f64(a[h]), ra, rtol=1e-5, atol=1e-7)
        assert np.all(to_f64(b[h]) == 0.0)
    assert int(nd.item()) == 1


# ----------------------------------------------------------------------------
# spatial tiles: token permutation
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_permute_tokens_exact(dtype):
    rng = np.random.default_rng(8)
    heads, n = 3, 1000
    x = rng.standard_normal((heads, n, 64)).astype(np.float32)
    order = rng.permutation(n).astype(np.int32)
    xg = torch.from_numpy(x).to(DEV).to(dtype)
    xg = xg.permute(1, 0, 2).contiguous().permute(1, 0, 2)  # token-major source
    og = torch.from_numpy(order).to(DEV)
    g = zb.zebra_permute_tokens(xg, og)
    back = zb.zebra_permute_tokens(g, og, inverse=True)
    torch.cuda.synchronize()
    xr = xg.cpu()
    assert torch.equal(g.cpu(), xr[:, torch.from_numpy(order).long()])
    assert torch.equal(back.cpu(), xr)


@pytest.mark.parametrize("views,n_special,grid,block,q_tile,k_tile,top_k", [
    (2, 5, 12, 8, 64, 64, 2), (3, 1, 10, 4, 32, 32, 3), (2, 5, 37, 8, 64, 64, 9),
])
def test_spatial_stage_parity(views, n_special, grid, block, q_tile, k_tile, top_k):
    print(f"[case] spatial tiles views={views} grid={grid} block={block}", flush=True)
    order = zb.zebra_spatial_order(views, n_special, grid, grid, block).numpy()
    n = order.size
    q, k, v = _clustered(n + block, 2, n, n, q_tile, k_tile, 2)
    og = torch.from_numpy(order).to(DEV)
    out, bufs = stage.spatial_sparse_stage(bf16_gpu(q), bf16_gpu(k), bf16_gpu(v), og, q_tile,
                                           k_tile, top_k, 0.125)
    torch.cuda.synchronize()
    ref, _ = zo.spatial_tile_sparse_attention(q, k, v, zo.spatial_token_order(
        views, n_special, grid, grid, block), q_tile, k_tile, top_k, 0.125,
        sel=bufs.sel.cpu().numpy())
    assert_close(out, ref, f"spatial tiles {views}x{grid}/{block}")


# ----------------------------------------------------------------------------
# linear attention and the fit
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("n_q,n_kv,affine,out_dtype", [
    (128, 128, False, torch.bfloat16), (300, 300, True, torch.bfloat16),
    (70, 1000, True, torch.float32), (1, 5, False, torch.float32), (5000, 5000, True, torch.bfloat16),
])
def test_linear_parity(n_q, n_kv, affine, out_dtype):
    print(f"[case] linear Nq={n_q} Nk={n_kv} affine={affine} {out_dtype}", flush=True)
    rng = np.random.default_rng(n_q + n_kv)
    heads = 3
    q = synth.bf16_round(rng.standard_normal((heads, n_q, 64)).astype(np.float32))
    k = synth.bf16_round(rng.standard_normal((heads, n_kv, 64)).astype(np.float32))
    v = synth.bf16_round(rng.standard_normal((heads, n_kv, 64)).astype(np.float32))
    a = rng.uniform(0.5, 2.0, (heads, 64)).astype(np.float32) if affine else None
    b = rng.uniform(-0.1, 0.1, (heads, 64)).astype(np.float32) if affine else None
    tg = lambda x: None if x is None else torch.from_numpy(x).to(DEV)
    out = zb.zebra_linear_attn(bf16_gpu(q), bf16_gpu(k), bf16_gpu(v), tg(a), tg(b),
                               out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref = np.stack([zo.linear_attention(q[h], k[h], v[h], None if a is None else a[h],
                                        None if b is None else b[h])[0] for h in range(heads)])
    tol = 5e-3 if out_dtype == torch.bfloat16 else 1e-4
    assert_close(out, ref, f"linear Nq={n_q} Nk={n_kv}", rel_fro=tol)


def test_linear_is_deterministic():
    rng = np.random.default_rng(1)
    q, k, v = (bf16_gpu(rng.standard_normal((2, 4000, 64)).astype(np.float32)) for _ in range(3))
    o1 = zb.zebra_linear_attn(q, k, v, out_dtype=torch.float32)
    o2 = zb.zebra_linear_attn(q, k, v, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_fit_parity():
    rng = np.random.default_rng(4)
    heads, m = 4, 4096
    x = rng.standard_normal((heads, m, 64)).astype(np.float32) * 0.01
    y = (0.8 * x + 0.003 * rng.standard_normal((heads, m, 64)) + 0.001).astype(np.float32)
    x[1, :, 5] = 0.25  # a degenerate channel
    a, b, nd = zb.zebra_fit_affine(torch.from_numpy(x).to(DEV), torch.from_numpy(y).to(DEV))
    torch.cuda.synchronize()
    for h in range(heads):
        ra, rb, _ = zo.fit_affine(x[h], y[h])
        np.testing.assert_allclose(to_f64(a[h]), ra, rtol=1e-5, atol=1e-7)
        np.testing.assert_allclose(to_f64(b[h]), rb, rtol=1e-5, atol=1e-7)
    assert int(nd.item()) == 1


def test_calibration_pipeline_small():
    """Fit against dense attention at sampled queries: the GPU's fit equals the
    oracle's on the same (x, y), and x, y each match the oracle."""
    rng = np.random.default_rng(8)
    heads, n = 2, 3000
    q, k, v = (synth.bf16_round(rng.standard_normal((heads, n, 64)).astype(np.float32))
               for _ in range(3))
    idx = synth.fit_sample_indices(n, 512, 8)
    cal = stage.calibrate_linear(bf16_gpu(q), bf16_gpu(k), bf16_gpu(v),
                                 torch.from_numpy(idx).to(DEV), 0.125)
    torch.cuda.synchronize()
    for h in range(heads):
        y_ref = zo.dense_attention(q[h, idx], k[h], v[h], 0.125)
        x_ref = zo.linear_attention(q[h, idx], k[h], v[h])[0]
        assert_close(cal.y[h], y_ref, "fit target y")
        assert_close(cal.x[h], x_ref, "fit input x", rel_fro=1e-4)
        ra, rb, _ = zo.fit_affine(to_f64(cal.x[h]), to_f64(cal.y[h]))
        np.testing.assert_allclose(to_f64(cal.aff_scale[h]), ra, rtol=1e-4, atol=1e-6)
        np.testing.assert_allclose(to_f64(cal.aff_bias[h]), rb, rtol=1e-4, atol=1e-7)


# ----------------------------------------------------------------------------
# block attention mass (selection-quality diagnostic)
# ----------------------------------------------------------------------------

# float32 scores and exponentials against float64: per-element relative error
# of a few 1e-6 per term; the sums over up to 10^4 terms stay well inside these.
MASS_RTOL = 1e-3
MASS_ATOL = 1e-6


@pytest.mark.parametrize("heads,n_q,n_kv,q_tile,k_tile,n_hot", [
    (2, 300, 300, 64, 64, 2), (1, 130, 700, 128, 64, 3), (3, 97, 65, 32, 32, 1),
    (2, 1, 40, 64, 64, 1), (1, 2000, 1500, 64, 32, 4),
])
def test_block_mass_parity(heads, n_q, n_kv, q_tile, k_tile, n_hot):
    print(f"[case] block mass H={heads} Nq={n_q} Nk={n_kv} tiles {q_tile}x{k_tile}", flush=True)
    q, k, _ = _clustered(n_q + n_kv, heads, n_q, n_kv, q_tile, k_tile, n_hot)
    got = zb.zebra_block_mass(bf16_gpu(q), bf16_gpu(k), q_tile, k_tile, 0.125)
    torch.cuda.synchronize()
    g = to_f64(got)
    for h in range(heads):
        ref = zo.block_attention_mass(q[h], k[h], q_tile, k_tile, 0.125)
        np.testing.assert_allclose(g[h], ref, rtol=MASS_RTOL, atol=MASS_ATOL)
    np.testing.assert_allclose(g.sum(axis=2), 1.0, atol=1e-4)


def test_block_mass_large_scores_and_strided_layout():
    # scores far beyond float32's exp range: the running maximum must absorb them
    rng = np.random.default_rng(7)
    heads, n = 2, 700
    q = synth.bf16_round(rng.standard_normal((heads, n, 64)).astype(np.float32) * 12)
    k = synth.bf16_round(rng.standard_normal((heads, n, 64)).astype(np.float32) * 12)
    qg = bf16_gpu(q).permute(1, 0, 2).contiguous().permute(1, 0, 2)  # token-major
    got = zb.zebra_block_mass(qg, bf16_gpu(k), 64, 64, 0.125)
    torch.cuda.synchronize()
    for h in range(heads):
        ref = zo.block_attention_mass(q[h], k[h], 64, 64, 0.125)
        np.testing.assert_allclose(to_f64(got[h]), ref, rtol=MASS_RTOL, atol=MASS_ATOL)


def test_block_mass_is_deterministic():
    q, k, _ = _clustered(11, 2, 600, 900, 64, 64, 2)
    qg, kg = bf16_gpu(q), bf16_gpu(k)
    a = zb.zebra_block_mass(qg, kg, 64, 64, 0.125)
    b = zb.zebra_block_mass(qg, kg, 64, 64, 0.125)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_block_mass_retained_by_gpu_selection():
    # the mass the GPU's own selection keeps, from the GPU's masses, matches the
    # oracle's, and never exceeds the oracle's top-k mass
    heads, n, tile, top_k = 2, 1024, 64, 4
    q, k, _ = _clustered(5, heads, n, n, tile, tile, 2)
    qg, kg = bf16_gpu(q), bf16_gpu(k)
    sel = zb.zebra_select_tiles(zb.zebra_pool_landmarks(qg, tile),
                                zb.zebra_pool_landmarks(kg, tile), top_k)
    mass = zb.zebra_block_mass(qg, kg, tile, tile, 0.125)
    torch.cuda.synchronize()
    for h in range(heads):
        ref = zo.block_attention_mass(q[h], k[h], tile, tile, 0.125)
        kept = zo.retained_mass(to_f64(mass[h]), sel[h].cpu().numpy())
        kept_ref = zo.retained_mass(ref, sel[h].cpu().numpy())
        np.testing.assert_allclose(kept, kept_ref, rtol=MASS_RTOL, atol=1e-5)
        best = zo.top_mass(ref, top_k)
        assert np.all(kept_ref <= best + 1e-12)
        print(f"[parity] head {h}: retained {kept_ref.mean():.4f} of top {best.mean():.4f}",
              flush=True)


# ----------------------------------------------------------------------------
# gradients
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("n_q,n_kv,affine,g_dtype", [
    (300, 500, True, torch.float32), (1, 5, False, torch.float32), (70, 64, True, torch.bfloat16),
    (5000, 3000, True, torch.float32), (0, 100, True, torch.float32),
])
def test_linear_backward_parity(n_q, n_kv, affine, g_dtype):
    print(f"[case] linear backward Nq={n_q} Nk={n_kv} affine={affine} {g_dtype}", flush=True)
    rng = np.random.default_rng(n_q + n_kv)
    heads = 2
    q = synth.bf16_round(rng.standard_normal((heads, n_q, 64)).astype(np.float32))
    k = synth.bf16_round(rng.standard_normal((heads, n_kv, 64)).astype(np.float32))
    v = synth.bf16_round(rng.standard_normal((heads, n_kv, 64)).astype(np.float32))
    dout = rng.standard_normal((heads, n_q, 64)).astype(np.float32)
    if g_dtype == torch.bfloat16:
        dout = synth.bf16_round(dout)
    a = rng.uniform(0.5, 1.5, (heads, 64)).astype(np.float32) if affine else None
    dq, dk, dv, da, db = zb.zebra_linear_attn_backward(
        bf16_gpu(q), bf16_gpu(k), bf16_gpu(v), torch.from_numpy(dout).to(DEV).to(g_dtype),
        None if a is None else torch.from_numpy(a).to(DEV))
    torch.cuda.synchronize()
    for h in range(heads):
        rq, rk, rv, ra, rb = zo.linear_attention_backward(q[h], k[h], v[h], dout[h],
                                                          None if a is None else a[h])
        assert_grad_close(dq[h], rq, f"linear dq head {h}")
        assert_grad_close(dk[h], rk, f"linear dk head {h}")
        assert_grad_close(dv[h], rv, f"linear dv head {h}")
        assert_grad_close(da[h], ra, f"linear da head {h}")
        assert_grad_close(db[h], rb, f"linear db head {h}")


SPARSE_BWD_CASES = [
    # (q_tile, k_tile, n_q, n_kv, top_k, n_hot, heads, variant)
    (64, 64, 300, 300, 2, 2, 2, "default"),
    (128, 32, 257, 300, 4, 2, 1, "default"),
    (32, 64, 100, 450, 1, 1, 2, "default"),
    (64, 32, 130, 200, 3, 2, 2, "log_count"),
    (64, 64, 300, 300, 2, 2, 2, "no_landmarks"),
    (32, 32, 2000, 2000, 7, 3, 1, "default"),        # many query tiles per key tile
    (64, 64, 1000, 1000, 16, 3, 1, "default"),       # every tile kept
    (64, 64, 300, 65536 + 333, 206, 3, 1, "default"),  # forward in split keys
    (64, 64, 333, 700, 3, 2, 2, "log_count"),  # short last landmark block under the log count
]
BWD_FLAGS = {"default": (0, {}), "no_landmarks": (1, dict(landmarks=False)),
             "log_count": (2, dict(landmark_log_count=True))}


@pytest.mark.parametrize("g_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("case", SPARSE_BWD_CASES, ids=[str(c) for c in SPARSE_BWD_CASES])
def test_sparse_backward_parity(case, g_dtype):
    q_tile, k_tile, n_q, n_kv, top_k, n_hot, heads, variant = case
    flags, kw = BWD_FLAGS[variant]
    print(f"[case] sparse backward {case} {g_dtype}", flush=True)
    q, k, v = _clustered(n_q + 3 * n_kv + top_k, heads, n_q, n_kv, q_tile, k_tile, n_hot)
    rng = np.random.default_rng(n_q * 7 + top_k)
    dout = synth.bf16_round(rng.standard_normal((heads, n_q, 64)).astype(np.float32))
    qg, kg, vg = bf16_gpu(q), bf16_gpu(k), bf16_gpu(v)
    bufs = stage.SparseBuffers.allocate(heads, n_q, n_kv, q_tile, k_tile, top_k, DEV)
    stage.sparse_stage(qg, kg, vg, q_tile, k_tile, top_k, 0.125, bufs, flags=flags)
    dq, dk, dv = zb.zebra_tile_sparse_attn_backward(
        qg, kg, vg, bufs.kbar, bufs.vbar, bufs.sel, q_tile, k_tile, top_k, 0.125,
        torch.from_numpy(dout).to(DEV).to(g_dtype), flags)
    torch.cuda.synchronize()
    sel = bufs.sel.cpu().numpy()
    rq, rk, rv = zo.tile_sparse_attention_backward(q, k, v, q_tile, k_tile, sel, 0.125, dout, **kw)
    assert_grad_close(dq, rq, f"sparse dq {case}")
    assert_grad_close(dk, rk, f"sparse dk {case}")
    assert_grad_close(dv, rv, f"sparse dv {case}")


LSE_CASES = [
    # (q_tile, k_tile, n_q, n_kv, top_k, n_hot, heads, variant)
    (64, 64, 300, 300, 2, 2, 2, "default"),
    (128, 32, 257, 300, 4, 2, 1, "log_count"),
    (32, 64, 100, 450, 1, 1, 2, "no_landmarks"),
    (64, 64, 300, 65536 + 333, 206, 3, 1, "default"),  # split keys: the landmark pass merges and writes lse
]


@pytest.mark.parametrize("case", LSE_CASES, ids=[str(c) for c in LSE_CASES])
def test_forward_lse_and_backward_from_it(case):
    """The forward's normaliser equals the oracle's log2-sum-exp of the column weights
    (bf16-rounded probabilities are summed: 1e-2 in log2 units) and the output is bitwise
    the plain forward's. The backward from the saved normaliser and float32 output is
    bitwise the backward that runs its own forward; the backward from the normaliser
    alone (its first sweep forms D and renormalises) matches the oracle."""
    q_tile, k_tile, n_q, n_kv, top_k, n_hot, heads, variant = case
    flags, kw = BWD_FLAGS[variant]
    print(f"[case] forward lse + backward from it {case}", flush=True)
    q, k, v = _clustered(n_q + 5 * n_kv + top_k, heads, n_q, n_kv, q_tile, k_tile, n_hot)
    qg, kg, vg = bf16_gpu(q), bf16_gpu(k), bf16_gpu(v)
    bufs = stage.SparseBuffers.allocate(heads, n_q, n_kv, q_tile, k_tile, top_k, DEV)
    stage.sparse_select(qg, kg, vg, q_tile, k_tile, top_k, bufs)
    lse = torch.empty((heads, n_q), dtype=torch.float32, device=DEV)
    out_l = zb.zebra_tile_sparse_attn_ex(qg, kg, vg, bufs.kbar, bufs.vbar, bufs.sel, q_tile,
                                         k_tile, top_k, 0.125, flags, lse_out=lse)
    out_p = zb.zebra_tile_sparse_attn_ex(qg, kg, vg, bufs.kbar, bufs.vbar, bufs.sel, q_tile,
                                         k_tile, top_k, 0.125, flags)
    lse32 = torch.empty((heads, n_q), dtype=torch.float32, device=DEV)
    out32 = zb.zebra_tile_sparse_attn_ex(qg, kg, vg, bufs.kbar, bufs.vbar, bufs.sel, q_tile,
                                         k_tile, top_k, 0.125, flags, out_dtype=torch.float32,
                                         lse_out=lse32)
    rng = np.random.default_rng(n_q + top_k)
    dout_np = synth.bf16_round(rng.standard_normal((heads, n_q, 64)).astype(np.float32))
    dout = torch.from_numpy(dout_np).to(DEV)
    g_self = zb.zebra_tile_sparse_attn_backward(qg, kg, vg, bufs.kbar, bufs.vbar, bufs.sel,
                                                q_tile, k_tile, top_k, 0.125, dout, flags)
    g_saved = zb.zebra_tile_sparse_attn_backward(qg, kg, vg, bufs.kbar, bufs.vbar, bufs.sel,
                                                 q_tile, k_tile, top_k, 0.125, dout, flags,
                                                 lse=lse32, out=out32)
    g_lse = zb.zebra_tile_sparse_attn_backward(qg, kg, vg, bufs.kbar, bufs.vbar, bufs.sel,
                                               q_tile, k_tile, top_k, 0.125, dout, flags, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out_l, out_p)
    assert torch.equal(lse, lse32)
    for a, b, name in zip(g_self, g_saved, ("dq", "dk", "dv")):
        assert torch.equal(a, b), f"{name} from the saved normaliser and output differs"
    sel = bufs.sel.cpu().numpy()
    rq, rk, rv = zo.tile_sparse_attention_backward(q, k, v, q_tile, k_tile, sel, 0.125, dout_np,
                                                    **kw)
    assert_grad_close(g_lse[0], rq, f"dq from the normaliser alone {case}")
    assert_grad_close(g_lse[1], rk, f"dk from the normaliser alone {case}")
    assert_grad_close(g_lse[2], rv, f"dv from the normaliser alone {case}")
    got = lse.cpu().numpy()
    worst = 0.0
    for h in range(heads):
        for i, (s0, e0) in enumerate(zo.tile_bounds(n_q, q_tile)):
            ck, _, bias = zo.attention_columns(k[h], v[h], k_tile, sel[h, i], **kw)
            lg = 0.125 * (q[h, s0:e0].astype(np.float64) @ ck.T) + bias[None, :]
            m = lg.max(axis=1)
            ref = (m + np.log(np.exp(lg - m[:, None]).sum(axis=1))) / np.log(2.0)
            worst = max(worst, float(np.abs(got[h, s0:e0] - ref).max()))
    print(f"[parity] lse max abs error (log2 units) {worst:.3e}", flush=True)
    assert worst <= 1e-2


def test_backward_from_saved_output_strided():
    """The saved float32 output may be token-major (head stride 64, token stride H x 64)
    and the gradients float32: the saved-output backward is still bitwise the backward
    that runs its own forward. Split keys (three chunks and the landmark pass): the
    landmark pass merges the chunks' partials and writes the normaliser and the output."""
    heads, n, top_k = 2, 65536 + 333, 206
    print(f"[case] saved-output backward, token-major output: H={heads} N={n}", flush=True)
    q, k, v = _clustered(77, heads, 300, n, 64, 64, 3)
    qg, kg, vg = bf16_gpu(q), bf16_gpu(k), bf16_gpu(v)
    bufs = stage.SparseBuffers.allocate(heads, 300, n, 64, 64, top_k, DEV)
    stage.sparse_select(qg, kg, vg, 64, 64, top_k, bufs)
    out = torch.empty((300, heads, 64), dtype=torch.float32, device=DEV).permute(1, 0, 2)
    lse = torch.empty((heads, 300), dtype=torch.float32, device=DEV)
    zb.zebra_tile_sparse_attn_ex(qg, kg, vg, bufs.kbar, bufs.vbar, bufs.sel, 64, 64, top_k,
                                 0.125, 0, out=out, lse_out=lse)
    rng = np.random.default_rng(78)
    dout = torch.from_numpy(rng.standard_normal((heads, 300, 64)).astype(np.float32)).to(DEV)
    g_self = zb.zebra_tile_sparse_attn_backward(qg, kg, vg, bufs.kbar, bufs.vbar, bufs.sel, 64,
                                                64, top_k, 0.125, dout)
    g_saved = zb.zebra_tile_sparse_attn_backward(qg, kg, vg, bufs.kbar, bufs.vbar, bufs.sel, 64,
                                                 64, top_k, 0.125, dout, lse=lse, out=out)
    torch.cuda.synchronize()
    for a, b, name in zip(g_self, g_saved, ("dq", "dk", "dv")):
        assert a.dtype == torch.float32
        assert torch.equal(a, b), f"{name} from the token-major saved output differs"
    rq, rk, rv = zo.tile_sparse_attention_backward(q, k, v, 64, 64, bufs.sel.cpu().numpy(), 0.125,
                                                    dout.cpu().numpy())
    assert_grad_close(g_saved[0], rq, "saved-output dq")
    assert_grad_close(g_saved[1], rk, "saved-output dk")
    assert_grad_close(g_saved[2], rv, "saved-output dv")


def test_sparse_backward_token_major_inputs():
    """Token-major [N][H][64] q, k and v (rows H x 64 elements apart) with 64-query and
    64-key tiles: the key-half dq kernel and the dK/dV kernels stage strided rows."""
    heads, nq, n, top_k = 3, 250, 900, 3
    print(f"[case] sparse backward, token-major inputs: H={heads} Nq={nq} N={n}", flush=True)
    q, k, v = _clustered(19, heads, nq, n, 64, 64, 2)
    tm = lambda x: bf16_gpu(x).permute(1, 0, 2).contiguous().permute(1, 0, 2)
    qg, kg, vg = tm(q), tm(k), tm(v)
    bufs = stage.SparseBuffers.allocate(heads, nq, n, 64, 64, top_k, DEV)
    stage.sparse_select(qg, kg, vg, 64, 64, top_k, bufs)
    rng = np.random.default_rng(20)
    dout = synth.bf16_round(rng.standard_normal((heads, nq, 64)).astype(np.float32))
    dq, dk, dv = zb.zebra_tile_sparse_attn_backward(
        qg, kg, vg, bufs.kbar, bufs.vbar, bufs.sel, 64, 64, top_k, 0.125,
        torch.from_numpy(dout).to(DEV))
    torch.cuda.synchronize()
    rq, rk, rv = zo.tile_sparse_attention_backward(q, k, v, 64, 64, bufs.sel.cpu().numpy(),
                                                    0.125, dout)
    assert_grad_close(dq, rq, "token-major dq")
    assert_grad_close(dk, rk, "token-major dk")
    assert_grad_close(dv, rv, "token-major dv")


def test_sparse_backward_multirow_bits_partial_group():
    """dk and dv through the kept-tile bit matrix built several query tiles per
    workgroup: 16 heads x 283 query tiles of 32 (4,528 rows) give 2 rows per
    workgroup with a last group of one row, and an LDS histogram of per-key-tile
    counts per workgroup. One whole head against the oracle, all three gradients."""
    heads, q_tile, k_tile, n, top_k = 16, 32, 64, 9050, 29
    print(f"[case] sparse backward multirow bits: H={heads} N={n} tiles {q_tile}x{k_tile} "
          f"top_k={top_k}", flush=True)
    q, k, v = _clustered(9050, heads, n, n, q_tile, k_tile, 3)
    rng = np.random.default_rng(9051)
    dout = synth.bf16_round(rng.standard_normal((heads, n, 64)).astype(np.float32))
    qg, kg, vg = bf16_gpu(q), bf16_gpu(k), bf16_gpu(v)
    bufs = stage.sparse_stage(qg, kg, vg, q_tile, k_tile, top_k, 0.125)
    dq, dk, dv = zb.zebra_tile_sparse_attn_backward(
        qg, kg, vg, bufs.kbar, bufs.vbar, bufs.sel, q_tile, k_tile, top_k, 0.125,
        torch.from_numpy(dout).to(DEV))
    torch.cuda.synchronize()
    sel = bufs.sel.cpu().numpy()
    for h in (0, 11):
        rq, rk, rv = zo.tile_sparse_attention_backward(q[h:h + 1], k[h:h + 1], v[h:h + 1],
                                                       q_tile, k_tile, sel[h:h + 1], 0.125,
                                                       dout[h:h + 1])
        assert_grad_close(dq[h], rq[0], f"multirow bits dq head {h}")
        assert_grad_close(dk[h], rk[0], f"multirow bits dk head {h}")
        assert_grad_close(dv[h], rv[0], f"multirow bits dv head {h}")


def test_sparse_backward_phased_walks():
    """dq and the key tiles' dk, dv with phased walks: 64 heads x 142 query and key
    tiles (9,088 workgroups per launch, several times what the device runs at
    once), so every item walks its kept tiles (dq) or the query tiles keeping
    its key tile (dk, dv) from a phase-dependent start and wraps around; a
    26-token last key tile is kept by some rows. Two whole heads against the
    oracle, all three gradients, and two runs bitwise equal."""
    heads, q_tile, k_tile, n, top_k = 64, 64, 64, 9050, 29
    print(f"[case] sparse backward phased walks: H={heads} N={n} top_k={top_k}", flush=True)
    q, k, v = _clustered(9052, heads, n, n, q_tile, k_tile, 3)
    rng = np.random.default_rng(9053)
    dout = synth.bf16_round(rng.standard_normal((heads, n, 64)).astype(np.float32))
    qg, kg, vg = bf16_gpu(q), bf16_gpu(k), bf16_gpu(v)
    bufs = stage.sparse_stage(qg, kg, vg, q_tile, k_tile, top_k, 0.125)
    dg = torch.from_numpy(dout).to(DEV)
    runs = [zb.zebra_tile_sparse_attn_backward(qg, kg, vg, bufs.kbar, bufs.vbar, bufs.sel, q_tile,
                                               k_tile, top_k, 0.125, dg) for _ in range(2)]
    torch.cuda.synchronize()
    for a, b, name in zip(runs[0], runs[1], ("dq", "dk", "dv")):
        assert torch.equal(a, b), f"phased backward {name} is not repeatable"
    dq, dk, dv = runs[0]
    sel = bufs.sel.cpu().numpy()
    assert np.any(sel == -(-n // k_tile) - 1)
    for h in (0, 63):
        rq, rk, rv = zo.tile_sparse_attention_backward(q[h:h + 1], k[h:h + 1], v[h:h + 1],
                                                       q_tile, k_tile, sel[h:h + 1], 0.125,
                                                       dout[h:h + 1])
        assert_grad_close(dq[h], rq[0], f"phased walks dq head {h}")
        assert_grad_close(dk[h], rk[0], f"phased walks dk head {h}")
        assert_grad_close(dv[h], rv[0], f"phased walks dv head {h}")


def test_sparse_backward_running_max_path_and_determinism():
    """Query tiles with a loose logit bound (the forward's running-maximum path)
    and bitwise-equal gradients on a second call."""
    q, k, v = _clustered(41, 2, 700, 700, 64, 64, 3)
    q = q.copy()
    q[:, 128:320] *= 8.0
    q = synth.bf16_round(q)
    dout = synth.bf16_round(np.random.default_rng(3).standard_normal((2, 700, 64)).astype(np.float32))
    qg, kg, vg = bf16_gpu(q), bf16_gpu(k), bf16_gpu(v)
    bufs = stage.sparse_stage(qg, kg, vg, 64, 64, 3, 0.125)
    dg = torch.from_numpy(dout).to(DEV)
    g1 = zb.zebra_tile_sparse_attn_backward(qg, kg, vg, bufs.kbar, bufs.vbar, bufs.sel, 64, 64, 3,
                                            0.125, dg)
    g2 = zb.zebra_tile_sparse_attn_backward(qg, kg, vg, bufs.kbar, bufs.vbar, bufs.sel, 64, 64, 3,
                                            0.125, dg)
    torch.cuda.synchronize()
    ref = zo.tile_sparse_attention_backward(q, k, v, 64, 64, bufs.sel.cpu().numpy(), 0.125, dout)
    for a, b, r, name in zip(g1, g2, ref, ("dq", "dk", "dv")):
        assert torch.equal(a, b), f"{name} not reproducible"
        assert_grad_close(a, r, f"running-max path {name}")
