"""GPU parity at the benchmark workloads' full sizes, on sampled outputs.

Each test runs one whole stage exactly as bench.py launches it (same buffers,
tiles, top_k and scale) on the seeded full-size inputs, then checks a seeded
sample of (head, query tile) rows against the CPU oracle one by one:
  * the selection of each sampled row against the oracle's float64 pooled
    scores of the whole head (bit-exact outside near ties);
  * the attention output of each sampled query tile against the oracle run on
    that row's GPU selection (max-abs 2e-2, rel-Frobenius 5e-3);
  * linear stages: sampled query outputs against the oracle's state over all
    keys with the GPU's fitted (a, b); the fit against the oracle on the GPU's
    own (x, y); the dense calibration target on a sample of its queries.
"""

import numpy as np
import pytest
import torch

import oracle.zebra_oracle as zo
import linear_hybrid_attention_zebra_amd as zb
from linear_hybrid_attention_zebra_amd import stage as stage_mod
from linear_hybrid_attention_zebra_amd import synth
from parity_util import assert_close, check_selection_row, selection_report, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCALE = 0.125
ROWS = 6  # sampled (head, query tile) rows per sparse stage


def _head(t, h):
    return t[h].to("cpu", torch.float64).numpy()


SPARSE_STAGES = [("sparse-16v", 0), ("stack24-512v", 9), ("sparse-1024v", 0)]


@pytest.mark.parametrize("name,stage", SPARSE_STAGES, ids=[f"{n}:{s}" for n, s in SPARSE_STAGES])
def test_full_size_sparse_stage_sampled(name, stage):
    w = synth.WORKLOADS[name]
    print(f"[case] full-size sparse {name} stage {stage}: N={w.n_tokens} H={w.heads} "
          f"tiles {w.q_tile}x{w.k_tile} top_k={w.k}", flush=True)
    q, k, v = synth.stage_inputs(w, stage, DEV)
    bufs = stage_mod.SparseBuffers.allocate(w.heads, w.n_tokens, w.n_tokens, w.q_tile, w.k_tile,
                                            w.k, DEV)
    stage_mod.sparse_stage(q, k, v, w.q_tile, w.k_tile, w.k, SCALE, bufs)
    torch.cuda.synchronize()
    rows = synth.sample_rows(w.heads, w.t_q, ROWS, 100 + stage)
    swaps = 0
    for h in sorted(set(rows[:, 0].tolist())):
        qh, kh, vh = _head(q, h), _head(k, h), _head(v, h)
        kbar = zo.pool_tiles(kh, w.k_tile)
        for i in rows[rows[:, 0] == h][:, 1]:
            s0, e0 = i * w.q_tile, min(w.n_tokens, (i + 1) * w.q_tile)
            qbar_i = qh[s0:e0].mean(axis=0)
            scores = zo.block_scores(qbar_i[None], kbar)[0]
            gsel = bufs.sel[h, i].cpu().numpy()
            swaps += check_selection_row(gsel, scores, w.k)
            ref = zo.tile_sparse_attention_tile(qh[s0:e0], kh, vh, w.k_tile, gsel, SCALE)
            assert_close(bufs.out[h, s0:e0], ref, f"{name} stage {stage} head {h} tile {i}")
    print(f"[parity] near-tie swaps {swaps} of {len(rows)} sampled rows", flush=True)


def test_whole_16_view_stage_every_row_and_element():
    """The whole 16-view sparse stage (21,984 tokens, 16 heads, 344 query tiles
    with a 32-token last tile): every selection row of every head against the
    oracle's float64 pooled scores, and every output element against the oracle
    run on the GPU's selection."""
    w = synth.WORKLOADS["sparse-16v"]
    print(f"[case] whole sparse-16v stage: N={w.n_tokens} H={w.heads} top_k={w.k}", flush=True)
    q, k, v = synth.stage_inputs(w, 0, DEV)
    bufs = stage_mod.sparse_stage(q, k, v, w.q_tile, w.k_tile, w.k, SCALE)
    torch.cuda.synchronize()
    sel = bufs.sel.cpu().numpy()
    qn, kn, vn = (t.to("cpu", torch.float64).numpy() for t in (q, k, v))
    scores = np.stack([zo.block_scores(zo.pool_tiles(qn[h], w.q_tile),
                                       zo.pool_tiles(kn[h], w.k_tile)) for h in range(w.heads)])
    rep = selection_report(sel, scores, w.k)
    print(f"[parity] sparse-16v selection: {rep}", flush=True)
    assert rep["rows"] == w.heads * w.t_q and rep["mismatches"] == 0
    ref, _ = zo.tile_sparse_attention(qn, kn, vn, w.q_tile, w.k_tile, w.k, SCALE, sel=sel)
    assert_close(bufs.out, ref, "sparse-16v, every element of every head")


WHOLE_HEAD = [("stack24-512v", 9, 3), ("sparse-1024v", 0, 12)]


@pytest.mark.parametrize("name,stage,head", WHOLE_HEAD, ids=[f"{n}:{s}" for n, s, _ in WHOLE_HEAD])
def test_full_size_selection_whole_head(name, stage, head):
    """Every selection row of one whole head at full size against the oracle's
    float64 pooled scores of that head (10,992 rows of 10,992 or 21,984 scores)."""
    w = synth.WORKLOADS[name]
    print(f"[case] whole-head selection {name} stage {stage} head {head}: T_q={w.t_q} "
          f"T_k={w.t_k} top_k={w.k}", flush=True)
    q, k, v = synth.stage_inputs(w, stage, DEV)
    bufs = stage_mod.SparseBuffers.allocate(w.heads, w.n_tokens, w.n_tokens, w.q_tile, w.k_tile,
                                            w.k, DEV)
    stage_mod.sparse_select(q, k, v, w.q_tile, w.k_tile, w.k, bufs)
    torch.cuda.synchronize()
    qbar = zo.pool_tiles(_head(q, head), w.q_tile)
    kbar = zo.pool_tiles(_head(k, head), w.k_tile)
    rep = selection_report(bufs.sel[head].cpu().numpy(), zo.block_scores(qbar, kbar), w.k)
    print(f"[parity] {name} stage {stage} head {head} selection: {rep}", flush=True)
    assert rep["rows"] == w.t_q and rep["mismatches"] == 0


def test_full_size_sparse_stage_is_deterministic():
    """Stage 9 of the 512-view stack, twice: selection and output bitwise equal.
    Every sum runs in a fixed order (no float atomics), so any difference is a
    race in staging; some show only at full size, where the waves of a
    workgroup drift furthest apart."""
    w = synth.WORKLOADS["stack24-512v"]
    print(f"[case] full-size sparse determinism stack24-512v stage 9: N={w.n_tokens}", flush=True)
    q, k, v = synth.stage_inputs(w, 9, DEV)
    bufs = stage_mod.SparseBuffers.allocate(w.heads, w.n_tokens, w.n_tokens, w.q_tile, w.k_tile,
                                            w.k, DEV)
    stage_mod.sparse_stage(q, k, v, w.q_tile, w.k_tile, w.k, SCALE, bufs)
    first_out, first_sel = bufs.out.clone(), bufs.sel.clone()
    stage_mod.sparse_stage(q, k, v, w.q_tile, w.k_tile, w.k, SCALE, bufs)
    torch.cuda.synchronize()
    assert torch.equal(first_sel, bufs.sel)
    assert torch.equal(first_out, bufs.out)


LINEAR_STAGES = [("linear-128v", 0), ("stack24-512v", 0)]


@pytest.mark.parametrize("name,stage", LINEAR_STAGES, ids=[f"{n}:{s}" for n, s in LINEAR_STAGES])
def test_full_size_linear_stage_sampled(name, stage):
    w = synth.WORKLOADS[name]
    n = w.n_tokens
    print(f"[case] full-size linear {name} stage {stage}: N={n} H={w.heads}", flush=True)
    q, k, v = synth.stage_inputs(w, stage, DEV)
    idx = torch.from_numpy(synth.fit_sample_indices(n, w.fit_samples, w.stage_seed(stage))).to(DEV)
    cal = stage_mod.calibrate_linear(q, k, v, idx, SCALE, w.k_tile)
    out = zb.zebra_linear_attn(q, k, v, cal.aff_scale, cal.aff_bias)
    torch.cuda.synchronize()
    a, b = to_f64(cal.aff_scale), to_f64(cal.aff_bias)
    x, y = to_f64(cal.x), to_f64(cal.y)
    rng = np.random.default_rng(200 + stage)
    for h in rng.choice(w.heads, size=2, replace=False):
        qh, kh, vh = _head(q, h), _head(k, h), _head(v, h)
        # the fit on the GPU's own (x, y)
        a_ref, b_ref, _ = zo.fit_affine(x[h], y[h])
        np.testing.assert_allclose(a[h], a_ref, rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(b[h], b_ref, rtol=1e-5, atol=1e-7)
        # the linear output at sampled queries, with the GPU's (a, b)
        tok = np.sort(rng.choice(n, size=512, replace=False))
        ref, _, _ = zo.linear_attention(qh[tok], kh, vh, a[h], b[h])
        assert_close(out[h, torch.from_numpy(tok).to(DEV)], ref, f"{name} linear head {h}")
        # the unfitted linear output and the dense target at a few fit samples
        pick = np.sort(rng.choice(idx.numel(), size=64, replace=False))
        qs = qh[idx.cpu().numpy()[pick]]
        assert_close(x[h, pick], zo.linear_attention(qs, kh, vh)[0], f"{name} x head {h}")
        assert_close(y[h, pick], zo.dense_attention(qs, kh, vh, SCALE), f"{name} y head {h}")


def test_full_size_block_mass_sampled():
    w = synth.WORKLOADS["sparse-16v"]
    print(f"[case] full-size block mass {w.name}: N={w.n_tokens} H={w.heads}", flush=True)
    q, k, _ = synth.stage_inputs(w, 0, DEV)
    mass = zb.zebra_block_mass(q, k, w.q_tile, w.k_tile, SCALE)
    torch.cuda.synchronize()
    g = to_f64(mass)
    np.testing.assert_allclose(g.sum(axis=2), 1.0, atol=1e-4)
    rows = synth.sample_rows(w.heads, w.t_q, 4, 300)
    for h, i in rows:
        qh, kh = _head(q, h), _head(k, h)
        s0, e0 = i * w.q_tile, min(w.n_tokens, (i + 1) * w.q_tile)
        ref = zo.block_attention_mass(qh[s0:e0], kh, w.q_tile, w.k_tile, SCALE)[0]
        np.testing.assert_allclose(g[h, i], ref, rtol=1e-3, atol=1e-6)


def test_full_size_sparse_backward_sampled():
    """Gradients of the 16-view stage: one whole head for dq, dk, dv (every query
    tile reaches every key tile, directly or through its landmark), dq on
    sampled query tiles of the other heads (dq of a tile depends on its own
    columns only)."""
    from parity_util import assert_grad_close
    w = synth.WORKLOADS["sparse-16v"]
    n = w.n_tokens
    print(f"[case] full-size sparse backward {w.name}: N={n} H={w.heads}", flush=True)
    q, k, v = synth.stage_inputs(w, 0, DEV)
    bufs = stage_mod.SparseBuffers.allocate(w.heads, n, n, w.q_tile, w.k_tile, w.k, DEV)
    stage_mod.sparse_stage(q, k, v, w.q_tile, w.k_tile, w.k, SCALE, bufs)
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    dout = torch.randn((w.heads, n, 64), generator=g, device=DEV).bfloat16()
    dq, dk, dv = zb.zebra_tile_sparse_attn_backward(q, k, v, bufs.kbar, bufs.vbar, bufs.sel,
                                                    w.q_tile, w.k_tile, w.k, SCALE, dout)
    torch.cuda.synchronize()
    sel = bufs.sel.cpu().numpy()
    h0 = 5
    rq, rk, rv = zo.tile_sparse_attention_backward(
        _head(q, h0)[None], _head(k, h0)[None], _head(v, h0)[None], w.q_tile, w.k_tile,
        sel[h0:h0 + 1], SCALE, _head(dout, h0)[None])
    assert_grad_close(dq[h0], rq[0], "full-size dq, whole head")
    assert_grad_close(dk[h0], rk[0], "full-size dk, whole head")
    assert_grad_close(dv[h0], rv[0], "full-size dv, whole head")
    for h, i in synth.sample_rows(w.heads, w.t_q, 4, 400):
        s0, e0 = i * w.q_tile, min(n, (i + 1) * w.q_tile)
        ref, _, _ = zo.tile_sparse_attention_backward(
            _head(q, h)[None, s0:e0], _head(k, h)[None], _head(v, h)[None], w.q_tile, w.k_tile,
            sel[h:h + 1, i:i + 1], SCALE, _head(dout, h)[None, s0:e0])
        assert_grad_close(dq[h, s0:e0], ref[0], f"full-size dq head {h} tile {i}")


def test_full_size_stack_backward_dq_sampled():
    """dq of two sampled query tiles of the 512-view sparse stage 9 (forward and
    gradients in split-key chunks, 2,199 of 10,992 key tiles kept)."""
    from parity_util import assert_grad_close
    w = synth.WORKLOADS["stack24-512v"]
    n = w.n_tokens
    print(f"[case] full-size backward dq {w.name} stage 9: N={n}", flush=True)
    q, k, v = synth.stage_inputs(w, 9, DEV)
    bufs = stage_mod.SparseBuffers.allocate(w.heads, n, n, w.q_tile, w.k_tile, w.k, DEV)
    stage_mod.sparse_stage(q, k, v, w.q_tile, w.k_tile, w.k, SCALE, bufs)
    g = torch.Generator(device=DEV)
    g.manual_seed(12)
    dout = torch.randn((w.heads, n, 64), generator=g, device=DEV).bfloat16()
    dq, _, _ = zb.zebra_tile_sparse_attn_backward(q, k, v, bufs.kbar, bufs.vbar, bufs.sel,
                                                  w.q_tile, w.k_tile, w.k, SCALE, dout)
    torch.cuda.synchronize()
    for h, i in synth.sample_rows(w.heads, w.t_q, 2, 401):
        s0, e0 = i * w.q_tile, min(n, (i + 1) * w.q_tile)
        ref, _, _ = zo.tile_sparse_attention_backward(
            _head(q, h)[None, s0:e0], _head(k, h)[None], _head(v, h)[None], w.q_tile, w.k_tile,
            bufs.sel[h:h + 1, i:i + 1].cpu().numpy(), SCALE, _head(dout, h)[None, s0:e0])
        assert_grad_close(dq[h, s0:e0], ref[0], f"512-view dq head {h} tile {i}")
