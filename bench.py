#!/usr/bin/env python3
"""Benchmark of the hybrid global-attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload: the 24-stage global-attention stack of a VGGT-shaped
backbone at 512 views (703,488 tokens, 16 heads x 64), stages 0-8 and 21-23
linear, 9-20 tile-sparse with 64x64 tiles keeping 20% of key tiles (80%
omitted as landmarks). One step is one pass over all 24 stages:
  * tile-sparse stage: pool Q/K/V -> select -> tile-sparse attention;
  * linear stage: the linear forward with its fitted affine map.
The affine map of each linear stage is a per-model constant, fitted once by
calibration (dense softmax target at 4,096 sampled queries, unfitted linear
output there, closed-form fit) before timing starts; its time is reported as
stage_ms.calibration_ms, outside the step. Inputs (all 24 stages' Q/K/V,
seeded synthetic draws) are resident in HBM before timing starts. Prints ONE
JSON line.

Other workloads (--workload): sparse-16v, linear-128v, sparse-1024v (one
stage each) report the same fields for that stage.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

METRIC = "hybrid global-attn ms/stage + % bf16 MFMA / % HBM peak, 16→1,024 views"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
SCALE = 0.125


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3)
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--workload", default="stack24-512v")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the per-workload stages timed after the stack")
    p.add_argument("--extra-launches", type=int, default=20,
                   help="timed launches per workload in the per-workload section")
    p.add_argument("--single-stage", type=int, default=None, metavar="S",
                   help="only time stage S of the workload on its own (pool+select and "
                        "attention apart, --steps launches after --warmup) and exit; the "
                        "command the committed kernel profiles are taken with")
    p.add_argument("--fallback", action="store_true",
                   help="with --single-stage: queries x8, so every item takes the "
                        "running-maximum softmax path")
    p.add_argument("--cpu-rows", type=int, default=64,
                   help="sampled (head, query tile) rows for the oracle's attention step")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB three times (the "
                        "reference kernel that scales the HBM byte counters) and exit")
    p.add_argument("--peak-probe", action="store_true",
                   help="only measure the achievable peaks the rooflines are read against: a "
                        "large bf16 GEMM (torch.matmul) and a 4 GiB device copy, and exit")
    p.add_argument("--selection-quality", action="store_true",
                   help="only measure how much dense attention mass the pooled-score selection "
                        "keeps, against the top-k blocks by mass, on the workload's first sparse "
                        "stage (at most 65,536 tokens) and exit")
    p.add_argument("--backward", action="store_true",
                   help="only time the gradients of the workload's first sparse stage (and, for "
                        "the stack and linear workloads, of its first linear stage) and exit")
    p.add_argument("--save-affine", default=None, metavar="NPZ",
                   help="write the fitted affine map of every linear stage to NPZ")
    p.add_argument("--load-affine", default=None, metavar="NPZ",
                   help="take the linear stages' affine maps from NPZ instead of fitting them")
    return p.parse_args()


def copy_probe(mib: int):
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters, divided by
    the bytes it must move, give the scale applied to the attention kernel's counters."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)


def peak_probe():
    """Achievable bf16 MFMA rate (an 8192^3 GEMM through the vendor library) and
    achievable HBM rates with the runtime's own kernels on 4 GiB buffers: a
    copy (reads and writes 8 GiB), a read-only sum and a write-only fill,
    median of 10."""
    import torch
    n = 8192
    a = torch.randn((n, n), device="cuda").bfloat16()
    b = torch.randn((n, n), device="cuda").bfloat16()
    src = torch.empty(4 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    src_f = src.view(torch.float32)

    def med_ms(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(10):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[len(ts) // 2]

    gemm_ms = med_ms(lambda: torch.matmul(a, b))
    copy_ms = med_ms(lambda: dst.copy_(src))
    read_ms = med_ms(lambda: torch.sum(src_f))
    write_ms = med_ms(lambda: dst.fill_(3))
    nb = src.numel()
    print(json.dumps({"gemm_bf16_tflops": 2.0 * n ** 3 / (gemm_ms * 1e-3) / 1e12,
                      "copy_gbs": 2.0 * nb / (copy_ms * 1e-3) / 1e9,
                      "read_gbs": nb / (read_ms * 1e-3) / 1e9,
                      "write_gbs": nb / (write_ms * 1e-3) / 1e9,
                      "gemm_ms": gemm_ms, "copy_ms": copy_ms, "read_ms": read_ms,
                      "write_ms": write_ms}), flush=True)


# ----------------------------------------------------------------------------
# algorithmic work (what the method must compute)
# ----------------------------------------------------------------------------

def sparse_flops(n_q, n_kv, q_tile, k_tile, top_k, sel):
    """Algorithmic flops of one tile-sparse launch, from its selection sel [H][Tq][k].

    Kept pairs: 4*d*|q tile i|*|k tile j| summed over every kept (h, i, j)
    (QK^T and PV, 2*d each). Landmarks: 4*d*|q tile i| per omitted tile.
    """
    d = 64
    heads, t_q = sel.shape[0], sel.shape[1]
    t_k = -(-n_kv // k_tile)
    q_sizes = np.full(t_q, q_tile, dtype=np.float64)
    q_sizes[-1] = n_q - (t_q - 1) * q_tile
    k_last = n_kv - (t_k - 1) * k_tile
    has_last = (sel == t_k - 1).any(axis=-1)  # [H][Tq]
    kept_tokens = top_k * k_tile - has_last * (k_tile - k_last)
    selected = 4.0 * d * float(np.sum(q_sizes[None, :] * kept_tokens))
    landmark = 4.0 * d * float(heads * np.sum(q_sizes) * (t_k - top_k))
    return selected, landmark


def recorded_traffic(workload: str):
    """HBM bytes per sparse launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, copy-scaled), or None when the summary does not
    cover this workload or the attention kernel source has changed since."""
    names = {"stack24-512v": "tile_sparse_kh_kernel_stack24-512v_hbm_bytes.md",
             "sparse-1024v": "tile_sparse_kh_kernel_sparse-1024v_hbm_bytes.md"}
    if workload not in names:
        return None
    root = os.path.dirname(os.path.abspath(__file__))
    summary = os.path.join(root, "profiles", names[workload])
    source = os.path.join(root, "linear_hybrid_attention_zebra_amd", "csrc", "sparse_attn.hip")
    try:
        text = open(summary).read()
        digest = hashlib.sha256(open(source, "rb").read()).hexdigest()
    except OSError:
        return None
    vals = dict(re.findall(r"^(\w+): (\S+)$", text, re.M))
    if vals.get("source_sha256") != digest:
        return None
    return float(vals["fetch_bytes_per_launch"]) + float(vals["write_bytes_per_launch"])


# ----------------------------------------------------------------------------
# GPU side
# ----------------------------------------------------------------------------

class Timer:
    """HIP events on the current stream, accumulated per label."""

    def __init__(self, torch):
        self.torch = torch
        self.open = {}
        self.pairs = {}

    def start(self, label):
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record()
        self.open[label] = ev

    def stop(self, label):
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record()
        self.pairs.setdefault(label, []).append((self.open.pop(label), ev))

    def ms(self, label):
        return [a.elapsed_time(b) for a, b in self.pairs.get(label, [])]

    def reset(self):
        self.pairs = {}


def run_gpu(args, w, torch, zb, stage_mod, synth):
    dev = torch.device("cuda", 0)
    heads, n = w.heads, w.n_tokens
    stages = list(range(w.n_stages)) if w.kind == "stack" else [0]
    kinds = {s: w.stage_kind(s) for s in stages}
    t_gen = time.time()
    inputs = {s: synth.stage_inputs(w, s, dev) for s in stages}
    torch.cuda.synchronize()
    gen_s = time.time() - t_gen

    t_k = -(-n // w.k_tile)
    top_k = w.k if any(k == "sparse" for k in kinds.values()) else None
    sparse_bufs = None
    if top_k is not None:
        sparse_bufs = stage_mod.SparseBuffers.allocate(heads, n, n, w.q_tile, w.k_tile, top_k, dev)
    lin_out = torch.empty((heads, n, 64), dtype=torch.bfloat16, device=dev)
    lin_ws = torch.empty(zb.library().zebra_linear_attn_workspace(n, heads, 64),
                         dtype=torch.uint8, device=dev)
    fit_idx = {s: torch.from_numpy(synth.fit_sample_indices(n, w.fit_samples, w.stage_seed(s)))
               .to(dev) for s in stages if kinds[s] == "linear"}
    timer = Timer(torch)
    # calibration, once per linear stage before timing (warm call, then a timed one)
    cal_timer = Timer(torch)
    cals = {}
    if args.load_affine:
        cals = stage_mod.load_calibrations(args.load_affine, dev)
        missing = [s for s in stages if kinds[s] == "linear" and s not in cals]
        if missing or any(c.aff_scale.shape[0] != heads for c in cals.values()):
            raise SystemExit(f"{args.load_affine}: no {heads}-head affine map for stages "
                             f"{missing or sorted(cals)}")
    for s in stages:
        if kinds[s] == "linear" and s not in cals:
            q, k, v = inputs[s]
            stage_mod.calibrate_linear(q, k, v, fit_idx[s], SCALE, w.k_tile)
            cal_timer.start("calibration")
            cals[s] = stage_mod.calibrate_linear(q, k, v, fit_idx[s], SCALE, w.k_tile)
            cal_timer.stop("calibration")
    torch.cuda.synchronize()
    if args.save_affine:
        stage_mod.save_calibrations(args.save_affine, cals)
    # one roctx range per stage (torch's nvtx calls are roctx on ROCm), for
    # rocprofv3 --marker-trace
    mark_push, mark_pop = torch.cuda.nvtx.range_push, torch.cuda.nvtx.range_pop
    labels = {s: f"stage {s} {kinds[s]}" for s in stages}

    def step():
        for s in stages:
            q, k, v = inputs[s]
            mark_push(labels[s])
            if kinds[s] == "sparse":
                timer.start("sparse_stage")
                stage_mod.sparse_select(q, k, v, w.q_tile, w.k_tile, top_k, sparse_bufs)
                timer.start("sparse_attn")
                stage_mod.sparse_attend(q, k, v, w.q_tile, w.k_tile, top_k, SCALE, sparse_bufs)
                timer.stop("sparse_attn")
                timer.stop("sparse_stage")
            else:
                cal = cals[s]
                timer.start("linear_stage")
                stage_mod.linear_stage(q, k, v, cal.aff_scale, cal.aff_bias, out=lin_out,
                                       workspace=lin_ws)
                timer.stop("linear_stage")
            mark_pop()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timer.reset()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    res = {"wall_s": wall, "gen_s": gen_s, "stages": len(stages),
           "n_sparse": sum(k == "sparse" for k in kinds.values()),
           "n_linear": sum(k == "linear" for k in kinds.values())}
    for label in ("sparse_stage", "sparse_attn", "calibration", "linear_stage"):
        vals = (cal_timer if label == "calibration" else timer).ms(label)
        if vals:
            res[label + "_ms"] = float(np.mean(vals))
            res[label + "_ms_median"] = float(np.median(vals))
    if top_k is not None:
        sel = sparse_bufs.sel.cpu().numpy()
        res["selected_flops"], res["landmark_flops"] = sparse_flops(
            n, n, w.q_tile, w.k_tile, top_k, sel)
        res["top_k"] = top_k
        res["t_k"] = t_k
        # the first sparse stage's selection, for the parity report (outside timing)
        s0 = min(s for s in stages if kinds[s] == "sparse")
        stage_mod.sparse_select(*inputs[s0], w.q_tile, w.k_tile, top_k, sparse_bufs)
        res["report_sel"] = (s0, sparse_bufs.sel.cpu().numpy())
    res["linear_bytes"] = heads * 64 * 4 * n * 2  # Q, K, V in and O out, bf16
    return res, inputs


def _timed_launches(torch, fn, warmup, launches, flush=None):
    """Mean and median HIP-event time (ms) of fn over `launches` calls after
    `warmup` untimed ones; flush() (if given) runs before each call, outside
    the events (it evicts the inputs from the 256 MB Infinity Cache)."""
    for _ in range(warmup):
        fn()
    pairs = []
    for _ in range(launches):
        if flush is not None:
            flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        pairs.append((a, b))
    torch.cuda.synchronize()
    ms = [x.elapsed_time(y) for x, y in pairs]
    return float(np.mean(ms)), float(np.median(ms))


def time_stage(args, torch, zb, stage_mod, synth, name, stage, q_mul, launches, flush):
    """One stage of a workload timed on its own (pool+select and attention apart
    for a sparse stage), with its roofline. q_mul scales the queries (a power
    of two: exact in bf16, the selection unchanged) to push every item past the
    fixed-reference bound onto the running-maximum softmax path."""
    dev = torch.device("cuda", 0)
    w = synth.WORKLOADS[name]
    n, heads = w.n_tokens, w.heads
    q, k, v = synth.stage_inputs(w, stage, dev)
    if w.stage_kind(stage) == "linear":
        idx = torch.from_numpy(synth.fit_sample_indices(n, w.fit_samples,
                                                        w.stage_seed(stage))).to(dev)
        cal = stage_mod.calibrate_linear(q, k, v, idx, SCALE, w.k_tile)
        o = torch.empty((heads, n, 64), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(zb.library().zebra_linear_attn_workspace(n, heads, 64),
                         dtype=torch.uint8, device=dev)
        mean, med = _timed_launches(
            torch, lambda: stage_mod.linear_stage(q, k, v, cal.aff_scale, cal.aff_bias, out=o,
                                                  workspace=ws),
            2, launches, flush)
        by = heads * 64 * 4 * n * 2
        return {"views": w.n_views, "tokens": n, "stage_ms": mean, "stage_ms_median": med,
                "launches": launches, "bound": "hbm", "bytes_per_launch": by,
                "achieved": by / (mean * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": by / (mean * 1e-3) / 1e9 / PEAK_HBM_GBS}
    if q_mul != 1.0:
        q = q * q_mul
    bufs = stage_mod.SparseBuffers.allocate(heads, n, n, w.q_tile, w.k_tile, w.k, dev)
    sel_ms, _ = _timed_launches(
        torch, lambda: stage_mod.sparse_select(q, k, v, w.q_tile, w.k_tile, w.k, bufs),
        min(2, args.warmup + 1), launches, flush)
    att_ms, att_med = _timed_launches(
        torch, lambda: stage_mod.sparse_attend(q, k, v, w.q_tile, w.k_tile, w.k, SCALE, bufs),
        min(1, args.warmup), launches, flush)
    sel_fl, lm_fl = sparse_flops(n, n, w.q_tile, w.k_tile, w.k, bufs.sel.cpu().numpy())
    ach = sel_fl / (att_ms * 1e-3) / 1e12
    out = {"views": w.n_views, "tokens": n, "q_tile": w.q_tile, "k_tile": w.k_tile,
           "top_k": w.k, "t_k": w.t_k, "launches": launches,
           "stage_ms": sel_ms + att_ms, "pool_select_ms": sel_ms,
           "attn_ms": att_ms, "attn_ms_median": att_med, "bound": "mfma",
           "selected_flops": sel_fl, "landmark_flops": lm_fl, "achieved": ach,
           "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS,
           "achieved_with_landmarks": (sel_fl + lm_fl) / (att_ms * 1e-3) / 1e12,
           "pool_bytes": 3 * heads * n * 64 * 2}
    if q_mul != 1.0:
        out["softmax"] = (f"running maximum (queries x{q_mul:g}: every item's logit bound "
                          "exceeds the fixed-reference limit)")
    elif w.kind != "stack":
        out["traffic"] = recorded_traffic(w.name)
    return out


def per_workload(args, torch, zb, stage_mod, synth):
    """One stage of each single-stage workload (16 and 1,024 views sparse, 128
    views linear) and stage 9 of the 512-view stack on the running-maximum
    softmax path: pool+select and attention timed apart, with their rooflines.
    Outside the step and its value."""
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    flush = lambda: scratch.zero_()  # evicts the inputs from the 256 MB Infinity Cache
    out = {}
    for name, stage, q_mul in (("sparse-16v", 0, 1.0), ("linear-128v", 0, 1.0),
                               ("sparse-1024v", 0, 1.0), ("stack24-512v", 9, 8.0)):
        key = f"{name}:{stage}" + (":fallback" if q_mul != 1.0 else "")
        # the running-maximum leg is a comparison point: a few launches suffice
        launches = args.extra_launches if q_mul == 1.0 else max(3, args.extra_launches // 4)
        out[key] = time_stage(args, torch, zb, stage_mod, synth, name, stage, q_mul, launches,
                              flush)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        print(f"[bench] {key}: {json.dumps(out[key])}", file=sys.stderr, flush=True)
    del scratch
    return out


def selection_quality(args, w, torch, zb, synth):
    """Block attention mass of the first sparse stage (dense softmax), the mass
    the pooled-score selection retains, and the mass of the top-k blocks by mass."""
    if w.kind == "linear" or w.n_tokens > 65536:
        print(f"--selection-quality needs a sparse workload of at most 65,536 tokens "
              f"({w.name} has {w.n_tokens})", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda", 0)
    s = next(i for i in range(w.n_stages) if w.stage_kind(i) == "sparse")
    q, k, _ = synth.stage_inputs(w, s, dev)
    qbar = zb.zebra_pool_landmarks(q, w.q_tile)
    kbar = zb.zebra_pool_landmarks(k, w.k_tile)
    sel = zb.zebra_select_tiles(qbar, kbar, w.k)
    mass = zb.zebra_block_mass(q, k, w.q_tile, w.k_tile, SCALE)  # warm-up, then timed
    ms = []
    for _ in range(max(1, args.steps)):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        zb.zebra_block_mass(q, k, w.q_tile, w.k_tile, SCALE, out=mass)
        b.record()
        ms.append((a, b))
    torch.cuda.synchronize()
    m = mass.cpu().numpy().astype(np.float64)  # [H][Tq][Tk]
    sel_np = sel.cpu().numpy().astype(np.int64)
    kept = np.take_along_axis(m, sel_np, axis=2).sum(axis=2)
    best = -np.partition(-m, w.k - 1, axis=2)[:, :, :w.k].sum(axis=2)
    out = {"workload": w.name, "stage": s, "tokens": w.n_tokens, "heads": w.heads,
           "q_tile": w.q_tile, "k_tile": w.k_tile, "top_k": w.k,
           "keep_fraction": w.k / m.shape[2],
           "retained_mass_mean": float(kept.mean()), "retained_mass_min": float(kept.min()),
           "top_mass_mean": float(best.mean()), "top_mass_min": float(best.min()),
           "retained_over_top_mean": float((kept / best).mean()),
           "row_sum_max_dev": float(np.abs(m.sum(axis=2) - 1.0).max()),
           "block_mass_ms": float(np.median([x.elapsed_time(y) for x, y in ms]))}
    print(json.dumps({"selection_quality": out}), flush=True)


def backward(args, w, torch, zb, stage_mod, synth):
    """Time zebra_tile_sparse_attn_backward / zebra_linear_attn_backward on one
    stage of the workload (inputs and output gradient resident in HBM)."""
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    n, heads = w.n_tokens, w.heads
    stages = list(range(w.n_stages)) if w.kind == "stack" else [0]
    out = {"workload": w.name, "tokens": n, "heads": heads}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(max(1, args.steps)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            ms.append((a, b))
        torch.cuda.synchronize()
        return float(np.median([x.elapsed_time(y) for x, y in ms]))

    sparse_s = [s for s in stages if w.stage_kind(s) == "sparse"]
    if sparse_s:
        s = sparse_s[0]
        q, k, v = synth.stage_inputs(w, s, dev)
        bufs = stage_mod.SparseBuffers.allocate(heads, n, n, w.q_tile, w.k_tile, w.k, dev)
        stage_mod.sparse_stage(q, k, v, w.q_tile, w.k_tile, w.k, SCALE, bufs)
        dout = torch.randn((heads, n, 64), generator=g, device=dev).bfloat16()
        ws = torch.empty(zb.library().zebra_tile_sparse_attn_backward_workspace(
            n, n, heads, 64, w.q_tile, w.k_tile, w.k), dtype=torch.uint8, device=dev)
        ms = timed(lambda: zb.zebra_tile_sparse_attn_backward(
            q, k, v, bufs.kbar, bufs.vbar, bufs.sel, w.q_tile, w.k_tile, w.k, SCALE, dout,
            workspace=ws))
        # a training step keeps the forward's normaliser, and its output in float32: the
        # backward then skips its forward and forms D from that output (one dq sweep)
        lse = torch.empty((heads, n), dtype=torch.float32, device=dev)
        out32 = zb.zebra_tile_sparse_attn_ex(q, k, v, bufs.kbar, bufs.vbar, bufs.sel, w.q_tile,
                                             w.k_tile, w.k, SCALE, 0, out_dtype=torch.float32,
                                             workspace=bufs.attn_ws, lse_out=lse)
        ms_saved = timed(lambda: zb.zebra_tile_sparse_attn_backward(
            q, k, v, bufs.kbar, bufs.vbar, bufs.sel, w.q_tile, w.k_tile, w.k, SCALE, dout,
            workspace=ws, lse=lse, out=out32))
        # ... or only the normaliser (bf16 output): a first dq sweep forms D
        ms_lse = timed(lambda: zb.zebra_tile_sparse_attn_backward(
            q, k, v, bufs.kbar, bufs.vbar, bufs.sel, w.q_tile, w.k_tile, w.k, SCALE, dout,
            workspace=ws, lse=lse))
        sel_fl, lm_fl = sparse_flops(n, n, w.q_tile, w.k_tile, w.k, bufs.sel.cpu().numpy())
        # gradient work: S, dP, dq, dk, dv = 10 d flop per column (forward: 4 d)
        bw = 2.5 * sel_fl / (ms * 1e-3) / 1e12
        bw_saved = 2.5 * sel_fl / (ms_saved * 1e-3) / 1e12
        bw_lse = 2.5 * sel_fl / (ms_lse * 1e-3) / 1e12
        out["sparse"] = {"stage": s, "ms": ms, "bound": "mfma", "achieved": bw,
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": bw / PEAK_BF16_TFLOPS,
                         "achieved_with_landmarks": 2.5 * (sel_fl + lm_fl) / (ms * 1e-3) / 1e12,
                         "flops_per_launch": 2.5 * sel_fl, "workspace_bytes": ws.numel(),
                         "from_saved_output": {
                             "ms": ms_saved, "achieved": bw_saved,
                             "frac": bw_saved / PEAK_BF16_TFLOPS,
                             "note": "zebra_tile_sparse_attn_backward_saved with the normaliser "
                                     "and float32 output the forward wrote (no forward, one dq "
                                     "sweep)"},
                         "from_saved_normaliser": {
                             "ms": ms_lse, "achieved": bw_lse, "frac": bw_lse / PEAK_BF16_TFLOPS,
                             "note": "zebra_tile_sparse_attn_backward_lse with the normaliser "
                                     "alone (no forward; a first dq sweep forms D)"}}
        del q, k, v, bufs, dout, ws, out32
    linear_s = [s for s in stages if w.stage_kind(s) == "linear"]
    if linear_s:
        s = linear_s[0]
        q, k, v = synth.stage_inputs(w, s, dev)
        dout = torch.randn((heads, n, 64), generator=g, device=dev).bfloat16()
        a = torch.rand((heads, 64), generator=g, device=dev) + 0.5
        ws = torch.empty(zb.library().zebra_linear_attn_backward_workspace(n, n, heads, 64),
                         dtype=torch.uint8, device=dev)
        ms = timed(lambda: zb.zebra_linear_attn_backward(q, k, v, dout, a, workspace=ws))
        # float32 products: 3 (query pass) + 2 (key pass) 64 x 64 products per row
        fl = 5 * 2 * 64 * 64 * n * heads
        out["linear"] = {"stage": s, "ms": ms, "bound": "alu", "achieved": fl / (ms * 1e-3) / 1e12,
                         "peak": 157.3, "unit": "TFLOP/s",
                         "frac": fl / (ms * 1e-3) / 1e12 / 157.3,
                         "hbm_bytes": 7 * n * heads * 64 * 2,
                         "hbm_frac": 7 * n * heads * 64 * 2 / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    print(json.dumps({"backward": out}), flush=True)


# ----------------------------------------------------------------------------
# CPU oracle baseline on a bounded sample of the same workload
# ----------------------------------------------------------------------------

def cpu_baseline(args, w, torch, inputs, synth, report_sel=None):
    import oracle.zebra_oracle as zo
    sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "tests"))
    from parity_util import selection_report
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    n, heads = w.n_tokens, w.heads
    stages = list(range(w.n_stages)) if w.kind == "stack" else [0]
    sparse_s = [s for s in stages if w.stage_kind(s) == "sparse"]
    linear_s = [s for s in stages if w.stage_kind(s) == "linear"]
    f64 = lambda t: t.to("cpu", torch.float32).numpy().astype(np.float64)
    est = {}
    sample = []
    if sparse_s:
        s = sparse_s[0]
        q, k, v = (f64(t[0]) for t in inputs[s])  # head 0
        t0 = time.perf_counter()
        qbar, kbar = zo.pool_tiles(q, w.q_tile), zo.pool_tiles(k, w.k_tile)
        zo.pool_tiles(v, w.k_tile)
        sel = zo.select_tiles(qbar, kbar, w.k)
        per_head = time.perf_counter() - t0
        if report_sel is not None and report_sel[0] == s:
            rep = selection_report(report_sel[1][0], zo.block_scores(qbar, kbar), w.k)
            rep.update({"stage": s, "head": 0, "top_k": w.k, "t_k": kbar.shape[0],
                        "rule": "bit-exact except near ties (k-th and (k+1)-th oracle float64 "
                                "scores within 1e-4 relative), where only tiles inside the "
                                "band may swap"})
            est["selection"] = rep
        rows = synth.sample_rows(1, qbar.shape[0], args.cpu_rows, 17)[:, 1]
        t0 = time.perf_counter()
        for i in rows:
            s0, e0 = i * w.q_tile, min(n, (i + 1) * w.q_tile)
            zo.tile_sparse_attention_tile(q[s0:e0], k, v, w.k_tile, sel[i], SCALE)
        per_row = (time.perf_counter() - t0) / len(rows)
        est["sparse_stage_s"] = heads * per_head + heads * qbar.shape[0] * per_row
        sample.append(f"sparse stage {s}: pool+select of head 0 in full, attention of "
                      f"{len(rows)} query tiles of head 0")
    if linear_s:
        s = linear_s[0]
        q, k, v = (f64(t[0]) for t in inputs[s])
        t0 = time.perf_counter()
        zo.linear_attention(q, k, v)
        lin_head = time.perf_counter() - t0
        m_sub = 64
        idx = synth.fit_sample_indices(n, m_sub, 23)
        t0 = time.perf_counter()
        y = zo.dense_attention(q[idx], k, v, SCALE)
        x = zo.linear_attention(q[idx], k, v)[0]
        zo.fit_affine(x, y)
        cal_part = time.perf_counter() - t0
        est["linear_stage_s"] = heads * lin_head
        est["calibration_s"] = heads * cal_part * (w.fit_samples / m_sub)
        sample.append(f"linear stage {s}: head 0 in full (calibration of head 0 on "
                      f"{m_sub} of {w.fit_samples} sampled queries timed too, reported in "
                      f"per_stage_s, outside the step)")
    # the step's work: the affine fit is a one-off calibration, as on the GPU side
    total = (len(sparse_s) * est.get("sparse_stage_s", 0.0)
             + len(linear_s) * est.get("linear_stage_s", 0.0))
    selection = est.pop("selection", None)
    return {"value": 1000.0 * total / len(stages), "unit": "ms/stage", "cores": int(threads),
            "kind": "oracle",
            "sample": "; ".join(sample) + "; scaled to all heads, query tiles and samples "
                      "(extrapolated)",
            "per_stage_s": est}, selection


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.peak_probe:
        peak_probe()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path "
              "would shard by head across GPUs; this implementation runs on one GPU.", file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import torch
    import linear_hybrid_attention_zebra_amd as zb
    from linear_hybrid_attention_zebra_amd import stage as stage_mod, synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    zb.library()  # fails loudly if libzebra.so is missing
    w = synth.WORKLOADS[args.workload]
    if args.selection_quality:
        selection_quality(args, w, torch, zb, synth)
        return
    if args.backward:
        backward(args, w, torch, zb, stage_mod, synth)
        return
    if args.single_stage is not None:
        res = time_stage(args, torch, zb, stage_mod, synth, w.name, args.single_stage,
                         8.0 if args.fallback else 1.0, max(1, args.steps), None)
        print(json.dumps({"single_stage": {"workload": w.name, "stage": args.single_stage,
                                           **res}}), flush=True)
        return
    res, inputs = run_gpu(args, w, torch, zb, stage_mod, synth)
    report_sel = res.pop("report_sel", None)
    print(f"[bench] gpu done: {json.dumps(res)}", file=sys.stderr, flush=True)

    ms_per_step = 1000.0 * res["wall_s"] / args.steps
    n_stages = res["stages"]
    out = {
        "metric": METRIC, "value": ms_per_step / n_stages, "unit": "ms/stage", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "views": w.n_views, "tokens": w.n_tokens,
                   "heads": w.heads, "head_dim": w.head_dim, "stages": n_stages,
                   "linear_stages": list(w.linear_stages) if w.kind == "stack" else None,
                   "q_tile": w.q_tile, "k_tile": w.k_tile, "keep_percent": w.keep_percent,
                   "top_k": res.get("top_k"), "fit_samples": w.fit_samples,
                   "parallelism": "single GPU"},
    }
    stage_ms = {}
    for key in ("sparse_stage_ms", "sparse_attn_ms", "linear_stage_ms", "calibration_ms"):
        if key in res:
            stage_ms[key] = res[key]
    fwd = res.get("n_sparse", 0) * res.get("sparse_stage_ms", 0.0) + res.get("n_linear", 0) * \
        res.get("linear_stage_ms", 0.0)
    stage_ms["forward_ms_per_stage"] = fwd / n_stages  # sum of the per-kind stage times
    if "linear_stage_ms" in res:
        stage_ms["linear_hbm_frac"] = (res["linear_bytes"] / (res["linear_stage_ms"] * 1e-3)
                                       / 1e9) / PEAK_HBM_GBS
    out["stage_ms"] = stage_ms
    if "sparse_attn_ms" in res:
        sec = res["sparse_attn_ms"] * 1e-3
        achieved = res["selected_flops"] / sec / 1e12
        out["roofline"] = {"kernel": "tile_sparse_kh_kernel (timed as its whole zebra_tile_sparse_attn "
                                     "call: landmark packing, key ranges, chunk offsets, the key-chunk "
                                     "kernel and its landmark pass, which merges the chunks' "
                                     "partials)", "bound": "mfma",
                           "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": achieved / PEAK_BF16_TFLOPS,
                           "traffic": recorded_traffic(w.name),
                           "achieved_with_landmarks": (res["selected_flops"]
                                                       + res["landmark_flops"]) / sec / 1e12,
                           "flops_per_launch": res["selected_flops"]}
    elif "linear_stage_ms" in res:
        sec = res["linear_stage_ms"] * 1e-3
        achieved = res["linear_bytes"] / sec / 1e9
        out["roofline"] = {"kernel": "linear attention (state+reduce+apply)", "bound": "hbm",
                           "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": achieved / PEAK_HBM_GBS, "traffic": None,
                           "bytes_per_launch": res["linear_bytes"]}
    if w.kind == "stack" and not args.no_extra:
        # free the stages the CPU leg does not read, then the single-stage workloads
        keep = {min(s for s in inputs if w.stage_kind(s) == k)
                for k in ("sparse", "linear") if any(w.stage_kind(s) == k for s in inputs)}
        for s in list(inputs):
            if s not in keep:
                del inputs[s]
        torch.cuda.empty_cache()
        out["per_workload"] = per_workload(args, torch, zb, stage_mod, synth)
    if not args.no_cpu_baseline:
        out["cpu_baseline"], selection = cpu_baseline(args, w, torch, inputs, synth, report_sel)
        if selection is not None:
            out["selection"] = selection
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
