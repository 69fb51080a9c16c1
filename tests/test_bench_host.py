"""Host logic of bench.py (no GPU): the algorithmic flop count the roofline is
read against, the recorded-traffic lookup, and the one-GPU guard."""

import hashlib
import os
import re
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _brute_flops(n_q, n_kv, q_tile, k_tile, sel):
    """4 d |q tile| |k tile| per kept (head, query tile, key tile); 4 d |q tile|
    per omitted key tile (its landmark column), by plain loops."""
    d = 64
    t_q = -(-n_q // q_tile)
    t_k = -(-n_kv // k_tile)
    selected = landmark = 0
    for h in range(sel.shape[0]):
        for i in range(t_q):
            qs = min(n_q, (i + 1) * q_tile) - i * q_tile
            kept = set(int(j) for j in sel[h, i])
            for j in range(t_k):
                if j in kept:
                    selected += 4 * d * qs * (min(n_kv, (j + 1) * k_tile) - j * k_tile)
                else:
                    landmark += 4 * d * qs
    return selected, landmark


@pytest.mark.parametrize("n_q,n_kv,q_tile,k_tile,top_k", [
    (300, 450, 64, 64, 3),     # ragged last tiles on both sides
    (256, 256, 64, 64, 2),     # whole tiles
    (130, 97, 32, 32, 2),      # 32-token tiles, short key tail
    (257, 700, 128, 64, 4),
])
def test_sparse_flops_matches_loops(n_q, n_kv, q_tile, k_tile, top_k):
    rng = np.random.default_rng(n_q + n_kv)
    heads, t_q, t_k = 3, -(-n_q // q_tile), -(-n_kv // k_tile)
    sel = np.stack([np.stack([np.sort(rng.choice(t_k, top_k, replace=False))
                              for _ in range(t_q)]) for _ in range(heads)]).astype(np.int32)
    sel[0, 0] = np.arange(t_k - top_k, t_k)  # one row keeps the short last tile
    got = bench.sparse_flops(n_q, n_kv, q_tile, k_tile, top_k, sel)
    want = _brute_flops(n_q, n_kv, q_tile, k_tile, sel)
    assert got == pytest.approx(want, rel=0, abs=0)


def test_sparse_flops_full_selection_is_dense_attention():
    n, tile = 1000, 64
    t = -(-n // tile)
    sel = np.tile(np.arange(t, dtype=np.int32), (2, t, 1))
    selected, landmark = bench.sparse_flops(n, n, tile, tile, t, sel)
    assert selected == 2 * 4 * 64 * n * n and landmark == 0


def test_recorded_traffic_follows_the_source_hash():
    """A workload with a committed byte summary gets its traffic only while the
    summary names the current kernel source; others get none."""
    src = os.path.join(ROOT, "linear_hybrid_attention_zebra_amd", "csrc", "sparse_attn.hip")
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    summary = open(os.path.join(ROOT, "profiles",
                                "tile_sparse_kh_kernel_stack24-512v_hbm_bytes.md")).read()
    vals = dict(re.findall(r"^(\w+): (\S+)$", summary, re.M))
    t = bench.recorded_traffic("stack24-512v")
    if vals.get("source_sha256") == digest:
        assert t == float(vals["fetch_bytes_per_launch"]) + float(vals["write_bytes_per_launch"])
    else:
        assert t is None
    assert bench.recorded_traffic("linear-128v") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
