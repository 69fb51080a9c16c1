"""Host-side checks of the C ABI: exported symbols and argument validation.

Nothing here launches a kernel: every call below is rejected by validation,
which the library performs before any HIP call, so these run without a GPU.
Device pointers are stand-in integers that are never dereferenced.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import linear_hybrid_attention_zebra_amd as zb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zebra.h")
P = lambda a: ctypes.c_void_p(a)  # fake, 16-byte aligned device addresses


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zebra_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return zb.library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 25, names
    for name in names:
        assert hasattr(lib, name), f"{name} declared in zebra.h but not exported"
    assert set(names) == set(zb.ENTRY_POINTS)


def test_no_unresolved_library_symbols(lib):
    """Every symbol of the library's own namespace is defined in it (a kernel
    whose host launch stub was not emitted would only fail at load time on a
    machine that binds eagerly)."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", zb.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    missing = [line.split()[-1] for line in out.splitlines() if "5zebra" in line]
    assert not missing, missing


def test_version_and_status_strings(lib):
    assert "gfx950" in zb.version()
    for s in range(5):
        assert zb.status_string(s).startswith("ZEBRA_")


def seq(n, h=2, d=64, st=64, sh=None):
    return zb.ZebraSeq(n, h, d, st, n * st if sh is None else sh)


def test_pool_validation(lib):
    f = lib.zebra_pool_landmarks
    assert f(None, seq(128), 32, P(1 << 20), None) == zb.ZEBRA_ERR_INVALID_ARG
    assert f(P(1 << 16), seq(128, d=32), 32, P(1 << 20), None) == zb.ZEBRA_ERR_UNSUPPORTED
    assert f(P(1 << 16), seq(128), 0, P(1 << 20), None) == zb.ZEBRA_ERR_INVALID_ARG
    assert f(P(1 << 16), seq(128), 2048, P(1 << 20), None) == zb.ZEBRA_ERR_UNSUPPORTED
    assert f(P(1 << 16), seq(128), 32, None, None) == zb.ZEBRA_ERR_INVALID_ARG
    assert f(P((1 << 16) + 2), seq(128), 32, P(1 << 20), None) == zb.ZEBRA_ERR_UNSUPPORTED
    assert f(P(1 << 16), seq(128, st=60), 32, P(1 << 20), None) == zb.ZEBRA_ERR_UNSUPPORTED
    assert f(P(1 << 16), seq(-1), 32, P(1 << 20), None) == zb.ZEBRA_ERR_INVALID_ARG
    # output overlapping the input
    assert f(P(1 << 16), seq(128), 32, P((1 << 16) + 64), None) == zb.ZEBRA_ERR_INVALID_ARG
    # empty input: nothing to do, no launch
    assert f(P(1 << 16), seq(0), 32, None, None) == zb.ZEBRA_OK


def test_select_validation(lib):
    f = lib.zebra_select_tiles
    ws = lib.zebra_select_tiles_workspace(2, 10, 20)
    assert ws == 2 * 10 * 32 * 4  # rows padded to 32 scores
    args = lambda top_k=5, hd=64, ws_ptr=P(1 << 30), ws_b=ws, tk=20: (
        P(1 << 16), P(1 << 20), 2, 10, tk, hd, top_k, P(1 << 24), ws_ptr, ws_b, None)
    assert f(*args(top_k=0)) == zb.ZEBRA_ERR_INVALID_ARG
    assert f(*args(top_k=21)) == zb.ZEBRA_ERR_INVALID_ARG
    assert f(*args(hd=128)) == zb.ZEBRA_ERR_UNSUPPORTED
    assert f(*args(ws_ptr=None)) == zb.ZEBRA_ERR_WORKSPACE
    assert f(*args(ws_b=ws - 1)) == zb.ZEBRA_ERR_WORKSPACE
    assert f(*args(tk=40000)) == zb.ZEBRA_ERR_UNSUPPORTED
    assert f(P(1 << 16), P(1 << 20), 2, 10, 20, 64, 5, P(1 << 16), P(1 << 30), ws, None) == \
        zb.ZEBRA_ERR_INVALID_ARG  # selection written over qbar


def test_sparse_validation(lib):
    f = lib.zebra_tile_sparse_attn
    s = seq(256)
    ws = lib.zebra_tile_sparse_attn_workspace(256, 256, 2, 64, 64, 64, 2)
    assert ws > 0

    def call(q_tile=64, k_tile=64, top_k=2, scale=0.125, o=P(1 << 28), sel=P(1 << 24),
             kbar=P(1 << 22), ws_p=P(1 << 30), ws_b=ws, os_=s, dtype=0):
        return f(P(1 << 16), s, P(1 << 18), P(1 << 20), s, kbar, P(1 << 23), sel, q_tile, k_tile,
                 top_k, scale, o, os_, dtype, ws_p, ws_b, None)

    assert call(q_tile=48) == zb.ZEBRA_ERR_UNSUPPORTED
    assert call(k_tile=128) == zb.ZEBRA_ERR_UNSUPPORTED
    assert call(top_k=0) == zb.ZEBRA_ERR_INVALID_ARG
    assert call(top_k=5) == zb.ZEBRA_ERR_INVALID_ARG  # t_k = 4
    assert call(scale=0.0) == zb.ZEBRA_ERR_INVALID_ARG
    assert call(sel=None) == zb.ZEBRA_ERR_INVALID_ARG  # sparse needs sel
    assert call(kbar=None) == zb.ZEBRA_ERR_INVALID_ARG
    assert call(ws_p=None) == zb.ZEBRA_ERR_WORKSPACE
    assert call(ws_b=ws - 1) == zb.ZEBRA_ERR_WORKSPACE
    assert call(o=P(1 << 16)) == zb.ZEBRA_ERR_INVALID_ARG  # output over q
    assert call(os_=seq(255)) == zb.ZEBRA_ERR_INVALID_ARG  # output length != query length
    assert call(os_=seq(256, st=32)) == zb.ZEBRA_ERR_UNSUPPORTED or \
        call(os_=seq(256, st=32)) == zb.ZEBRA_ERR_INVALID_ARG  # rows overlap themselves
    assert call(dtype=7) == zb.ZEBRA_ERR_INVALID_ARG
    # a zero stride over more than one token or head writes rows onto each other
    assert call(os_=seq(256, st=0)) == zb.ZEBRA_ERR_INVALID_ARG
    assert call(os_=seq(256, sh=0)) == zb.ZEBRA_ERR_INVALID_ARG
    assert call(os_=seq(256, st=0, sh=0)) == zb.ZEBRA_ERR_INVALID_ARG


def test_zero_stride_outputs_rejected_everywhere(lib):
    """Every entry point that writes a token sequence rejects an output whose
    token or head stride is zero over an extent above one (rows would collide)."""
    s = seq(300)
    lin_ws = lib.zebra_linear_attn_workspace(300, 2, 64)
    for bad in (seq(300, st=0), seq(300, sh=0)):
        assert lib.zebra_linear_attn(P(1 << 16), s, P(1 << 18), P(1 << 20), s, None, None,
                                     P(1 << 28), bad, 0, P(1 << 30), lin_ws, None) == \
            zb.ZEBRA_ERR_INVALID_ARG
        assert lib.zebra_permute_tokens(P(1 << 16), s, P(1 << 24), 0, 0, P(1 << 28), bad,
                                        None) == zb.ZEBRA_ERR_INVALID_ARG


def test_lse_entry_points_validation(lib):
    """The normaliser-carrying forward and backward need their lse pointer, refuse an
    lse that overlaps an output, and otherwise validate as their plain forms."""
    f = lib.zebra_tile_sparse_attn_lse
    s = seq(256)
    ws = lib.zebra_tile_sparse_attn_workspace(256, 256, 2, 64, 64, 64, 2)

    def fwd(lse, ws_b=ws):
        return f(P(1 << 16), s, P(1 << 18), P(1 << 20), s, P(1 << 22), P(1 << 23), P(1 << 24), 64,
                 64, 2, 0.125, P(1 << 28), s, 0, 0, lse, P(1 << 30), ws_b, None)

    assert fwd(None) == zb.ZEBRA_ERR_INVALID_ARG
    assert fwd(P((1 << 28) + 64)) == zb.ZEBRA_ERR_INVALID_ARG  # inside the output
    assert fwd(P((1 << 16) + 64)) == zb.ZEBRA_ERR_INVALID_ARG  # inside q
    assert fwd(P((1 << 29) + 2)) == zb.ZEBRA_ERR_INVALID_ARG   # misaligned
    assert fwd(P(1 << 29), ws_b=ws - 1) == zb.ZEBRA_ERR_WORKSPACE
    b = lib.zebra_tile_sparse_attn_backward_lse
    bws = lib.zebra_tile_sparse_attn_backward_workspace(256, 256, 2, 64, 64, 64, 2)

    def bwd(lse, ws_b=bws):
        return b(P(1 << 16), s, P(1 << 18), P(1 << 20), s, P(1 << 22), P(1 << 23), P(1 << 24), 64,
                 64, 2, 0.125, 0, lse, P(1 << 25), s, 0, P(1 << 26), s, P(1 << 27), P(1 << 28), s,
                 P(1 << 31), ws_b, None)

    assert bwd(None) == zb.ZEBRA_ERR_INVALID_ARG
    assert bwd(P((1 << 26) + 64)) == zb.ZEBRA_ERR_INVALID_ARG  # read from inside dq
    assert bwd(P(1 << 30), ws_b=bws - 1) == zb.ZEBRA_ERR_WORKSPACE
    # ... and from the saved float32 output too
    sv = lib.zebra_tile_sparse_attn_backward_saved

    def saved(lse, out, os=s, ws_b=bws):
        return sv(P(1 << 16), s, P(1 << 18), P(1 << 20), s, P(1 << 22), P(1 << 23), P(1 << 24),
                  64, 64, 2, 0.125, 0, lse, out, os, P(1 << 25), s, 0, P(1 << 26), s, P(1 << 27),
                  P(1 << 28), s, P(1 << 31), ws_b, None)

    assert saved(P(1 << 30), None) == zb.ZEBRA_ERR_INVALID_ARG
    assert saved(None, P(1 << 29)) == zb.ZEBRA_ERR_INVALID_ARG
    assert saved(P(1 << 30), P((1 << 27) + 256)) == zb.ZEBRA_ERR_INVALID_ARG  # inside dk
    assert saved(P(1 << 30), P((1 << 29) + 4)) == zb.ZEBRA_ERR_UNSUPPORTED    # misaligned rows
    assert saved(P(1 << 30), P(1 << 29), os=seq(255)) == zb.ZEBRA_ERR_INVALID_ARG  # wrong Nq
    assert saved(P(1 << 30), P(1 << 29), ws_b=bws - 1) == zb.ZEBRA_ERR_WORKSPACE


def test_sparse_variant_flags_validation(lib):
    f = lib.zebra_tile_sparse_attn_ex
    s = seq(256)
    ws = lib.zebra_tile_sparse_attn_workspace(256, 256, 2, 64, 64, 64, 2)

    def call(flags, kbar=P(1 << 22), vbar=P(1 << 23), sel=P(1 << 24), ws_b=ws):
        return f(P(1 << 16), s, P(1 << 18), P(1 << 20), s, kbar, vbar, sel, 64, 64, 2, 0.125,
                 P(1 << 28), s, 0, flags, P(1 << 30), ws_b, None)

    assert call(4) == zb.ZEBRA_ERR_INVALID_ARG  # unknown flag bit
    assert call(zb.ZEBRA_SPARSE_NO_LANDMARKS | zb.ZEBRA_SPARSE_LANDMARK_LOG_COUNT) == \
        zb.ZEBRA_ERR_INVALID_ARG  # a count needs landmarks
    assert call(zb.ZEBRA_SPARSE_LANDMARK_LOG_COUNT, kbar=None) == zb.ZEBRA_ERR_INVALID_ARG
    assert call(zb.ZEBRA_SPARSE_NO_LANDMARKS, sel=None) == zb.ZEBRA_ERR_INVALID_ARG
    # without landmarks kbar/vbar are not read: the next check reached is the workspace
    assert call(zb.ZEBRA_SPARSE_NO_LANDMARKS, kbar=None, vbar=None, ws_b=ws - 1) == \
        zb.ZEBRA_ERR_WORKSPACE
    assert call(0, ws_b=ws - 1) == zb.ZEBRA_ERR_WORKSPACE


def test_split_key_workspace_sizes(lib):
    """Long key ranges with q_tile <= 64 add float32 partials (264 B per query and
    chunk of 32,768 keys) to the workspace; 128-query tiles and dense calls do not."""
    n = 65536 * 2 + 100  # 3 chunks of 512 tiles of 64
    base = lib.zebra_tile_sparse_attn_workspace(300, n, 2, 64, 128, 64, 100)
    split = lib.zebra_tile_sparse_attn_workspace(300, n, 2, 64, 64, 64, 100)
    assert split - base >= 2 * 300 * 3 * 264
    assert lib.zebra_tile_sparse_attn_workspace(300, 60000, 2, 64, 64, 64, 100) == \
        lib.zebra_tile_sparse_attn_workspace(300, 60000, 2, 64, 128, 64, 100)
    t_k = -(-n // 64)
    dense = lib.zebra_tile_sparse_attn_workspace(300, n, 2, 64, 64, 64, t_k)
    assert 0 < dense < base


def test_linear_validation(lib):
    f = lib.zebra_linear_attn
    s = seq(300)
    ws = lib.zebra_linear_attn_workspace(300, 2, 64)
    assert ws > 0

    def call(o=P(1 << 28), ws_p=P(1 << 30), ws_b=ws, kvs=s, a=None):
        return f(P(1 << 16), s, P(1 << 18), P(1 << 20), kvs, a, None, o, s, 0, ws_p, ws_b, None)

    assert call(ws_p=None) == zb.ZEBRA_ERR_WORKSPACE
    assert call(ws_b=ws - 4) == zb.ZEBRA_ERR_WORKSPACE
    assert call(o=P(1 << 18)) == zb.ZEBRA_ERR_INVALID_ARG  # output over k
    assert call(kvs=seq(0)) == zb.ZEBRA_ERR_INVALID_ARG
    assert call(a=P(1 << 28)) == zb.ZEBRA_ERR_INVALID_ARG  # affine scale inside the output
    assert call(kvs=seq(300, h=3)) == zb.ZEBRA_ERR_INVALID_ARG  # head count mismatch


def test_block_mass_validation(lib):
    f = lib.zebra_block_mass
    s = seq(256)
    ws = lib.zebra_block_mass_workspace(256, 2)
    assert ws == 256 * 2 * 8

    def call(q_tile=64, k_tile=64, scale=0.125, out=P(1 << 28), ws_p=P(1 << 30), ws_b=ws, ks=s):
        return f(P(1 << 16), s, P(1 << 20), ks, q_tile, k_tile, scale, out, ws_p, ws_b, None)

    assert call(q_tile=16) == zb.ZEBRA_ERR_UNSUPPORTED
    assert call(k_tile=128) == zb.ZEBRA_ERR_UNSUPPORTED
    assert call(scale=-1.0) == zb.ZEBRA_ERR_INVALID_ARG
    assert call(out=None) == zb.ZEBRA_ERR_INVALID_ARG
    assert call(out=P(1 << 20)) == zb.ZEBRA_ERR_INVALID_ARG  # mass written over k
    assert call(ws_p=None) == zb.ZEBRA_ERR_WORKSPACE
    assert call(ws_b=ws - 8) == zb.ZEBRA_ERR_WORKSPACE
    assert call(ks=seq(0)) == zb.ZEBRA_ERR_INVALID_ARG
    assert call(ks=seq(256, h=3)) == zb.ZEBRA_ERR_INVALID_ARG  # head count mismatch


def test_fit_validation(lib):
    f = lib.zebra_fit_affine
    assert f(P(1 << 16), P(1 << 20), 0, 2, 64, P(1 << 24), P(1 << 25), None, None) == \
        zb.ZEBRA_ERR_INVALID_ARG
    assert f(P(1 << 16), P(1 << 20), 10, 2, 32, P(1 << 24), P(1 << 25), None, None) == \
        zb.ZEBRA_ERR_UNSUPPORTED
    assert f(None, P(1 << 20), 10, 2, 64, P(1 << 24), P(1 << 25), None, None) == \
        zb.ZEBRA_ERR_INVALID_ARG
    assert f(P(1 << 16), P(1 << 20), 10, 2, 64, P(1 << 16), P(1 << 25), None, None) == \
        zb.ZEBRA_ERR_INVALID_ARG  # scale written over x


def test_scale_only_fit_validation(lib):
    f = lib.zebra_fit_scale_only
    assert f(P(1 << 16), P(1 << 20), 0, 2, 64, P(1 << 24), P(1 << 25), None, None) == \
        zb.ZEBRA_ERR_INVALID_ARG
    assert f(P(1 << 16), P(1 << 20), 10, 2, 48, P(1 << 24), P(1 << 25), None, None) == \
        zb.ZEBRA_ERR_UNSUPPORTED
    assert f(P(1 << 16), P(1 << 20), 10, 2, 64, P(1 << 24), P(1 << 24), None, None) == \
        zb.ZEBRA_ERR_INVALID_ARG  # scale and bias outputs overlap


def test_spatial_order_matches_oracle(lib):
    """The host-side spatial order of the library equals the oracle's (host logic)."""
    import oracle.zebra_oracle as zo
    for args in [(2, 5, 37, 37, 8), (3, 1, 2, 4, 2), (1, 0, 9, 5, 4), (2, 5, 37, 37, 1)]:
        got = zb.zebra_spatial_order(*args).numpy()
        assert np.array_equal(got, zo.spatial_token_order(*args)), args
    assert lib.zebra_spatial_order(1, 0, 2, 2, 0, P(1 << 16), 4) == zb.ZEBRA_ERR_INVALID_ARG
    assert lib.zebra_spatial_order(1, 0, 2, 2, 1, P(1 << 16), 5) == zb.ZEBRA_ERR_INVALID_ARG


def test_permute_validation(lib):
    f = lib.zebra_permute_tokens
    s = seq(256)

    def call(order=P(1 << 24), inverse=0, dtype=0, dst=P(1 << 28), ds=s):
        return f(P(1 << 16), s, order, inverse, dtype, dst, ds, None)

    assert call(order=None) == zb.ZEBRA_ERR_INVALID_ARG
    assert call(inverse=2) == zb.ZEBRA_ERR_INVALID_ARG
    assert call(dtype=5) == zb.ZEBRA_ERR_INVALID_ARG
    assert call(ds=seq(255)) == zb.ZEBRA_ERR_INVALID_ARG  # lengths differ
    assert call(dst=P(1 << 16)) == zb.ZEBRA_ERR_INVALID_ARG  # in place
    assert call(dst=P(1 << 24)) == zb.ZEBRA_ERR_INVALID_ARG  # over the order vector


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((1, 64, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        zb.zebra_pool_landmarks(x, 64)
