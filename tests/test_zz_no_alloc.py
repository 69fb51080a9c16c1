"""The allocation-free linear-attention entry point against the workspace one.

zebra_linear_attn_noalloc keeps its partial and folded states in the
library's fixed device array; zebra_linear_attn takes a caller workspace.
Both run the same kernels, so outputs must be bitwise equal. Two calls in a
row, the second smaller, check that nothing of the first call's contents of
the shared array leaks into the second; the oracle checks one head of each.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle.zebra_oracle as zo
import linear_hybrid_attention_zebra_amd as zb
from linear_hybrid_attention_zebra_amd import synth
from parity_util import assert_close, bf16_gpu

DEV = "cuda"


def test_noalloc_rejects_sizes_beyond_its_array():
    """Host-side: a state too large for the fixed array is refused before any HIP call."""
    lib = zb.library()
    cap = lib.zebra_linear_attn_noalloc_max_bytes()
    assert cap == 40 << 20
    assert lib.zebra_linear_attn_workspace(10 ** 7, 64, 64) <= cap
    heads = 4096
    assert lib.zebra_linear_attn_workspace(300, heads, 64) > cap
    s = zb.ZebraSeq(300, heads, 64, 64, 300 * 64)
    P = ctypes.c_void_p
    st = lib.zebra_linear_attn_noalloc(P(1 << 16), s, P(1 << 34), P(1 << 35), s, None, None,
                                       P(1 << 36), s, 0, None)
    assert st == zb.ZEBRA_ERR_WORKSPACE, zb.status_string(st)
    bad = zb.ZebraSeq(300, 2, 64, 0, 300 * 64)  # zero token stride on the output
    ok = zb.ZebraSeq(300, 2, 64, 64, 300 * 64)
    st = lib.zebra_linear_attn_noalloc(P(1 << 16), ok, P(1 << 20), P(1 << 22), ok, None, None,
                                       P(1 << 26), bad, 0, None)
    assert st == zb.ZEBRA_ERR_INVALID_ARG


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_twice():
    cases = [(16, 70001, 65537, True, torch.bfloat16),   # large first (many state chunks)
             (3, 300, 257, False, torch.float32)]        # then a smaller call
    for i, (heads, n_q, n_kv, affine, dtype) in enumerate(cases):
        print(f"[case] noalloc call {i}: H={heads} Nq={n_q} Nk={n_kv} affine={affine} "
              f"{dtype}", flush=True)
        rng = np.random.default_rng(900 + i)
        q = synth.bf16_round(rng.standard_normal((heads, n_q, 64)).astype(np.float32))
        k = synth.bf16_round(rng.standard_normal((heads, n_kv, 64)).astype(np.float32))
        v = synth.bf16_round(rng.standard_normal((heads, n_kv, 64)).astype(np.float32))
        qg, kg, vg = bf16_gpu(q), bf16_gpu(k), bf16_gpu(v)
        a = b = None
        if affine:
            a = torch.from_numpy(rng.uniform(0.5, 1.5, (heads, 64)).astype(np.float32)).to(DEV)
            b = torch.from_numpy(rng.uniform(-0.1, 0.1, (heads, 64)).astype(np.float32)).to(DEV)
        ref = zb.zebra_linear_attn(qg, kg, vg, a, b, out_dtype=dtype)
        out = torch.empty((heads, n_q, 64), dtype=dtype, device=DEV)
        zb.zebra_linear_attn_noalloc(qg, kg, vg, a, b, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"call {i}: differs from zebra_linear_attn"
        h = heads - 1
        o_ref, _, _ = zo.linear_attention(q[h], k[h], v[h],
                                          None if a is None else a[h].cpu().numpy(),
                                          None if b is None else b[h].cpu().numpy())
        assert_close(out[h], o_ref, f"noalloc call {i} head {h}")
