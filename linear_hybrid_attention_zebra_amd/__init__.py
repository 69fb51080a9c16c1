"""Python binding of libzebra, the gfx950 HIP library for Zebra3D's hybrid global attention.

Every function here marshals torch tensors into the C ABI declared in
``include/zebra.h`` and calls it on the current HIP stream; all arithmetic
runs in the library's kernels. PyTorch provides device memory and streams.
There is no fallback: if ``libzebra.so`` is missing or was built for another
ABI, the first call raises ``ZebraLibraryError``.

Tensors are [H][N][64] (heads, tokens, channels) with the channel dimension
contiguous; other strides are passed through. Call ``torch`` first (this
module imports it) so the library binds to the HIP runtime torch loaded.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

# the in-tree build; ZEBRA_LIBRARY selects another build of the same library
# (the host-AddressSanitizer copy that the host ABI tests run against)
LIB_PATH = os.environ.get("ZEBRA_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libzebra.so")
HEAD_DIM = 64

ZEBRA_OK, ZEBRA_ERR_INVALID_ARG, ZEBRA_ERR_UNSUPPORTED, ZEBRA_ERR_WORKSPACE, ZEBRA_ERR_HIP = range(5)
ZEBRA_BF16, ZEBRA_F32 = 0, 1
ZEBRA_SPARSE_NO_LANDMARKS, ZEBRA_SPARSE_LANDMARK_LOG_COUNT = 1, 2

ENTRY_POINTS = (
    "zebra_pool_landmarks", "zebra_select_tiles_workspace", "zebra_select_tiles",
    "zebra_tile_sparse_attn_workspace", "zebra_tile_sparse_attn", "zebra_tile_sparse_attn_ex",
    "zebra_tile_sparse_attn_lse", "zebra_tile_sparse_attn_backward_lse",
    "zebra_tile_sparse_attn_backward_saved",
    "zebra_linear_attn_workspace", "zebra_linear_attn", "zebra_linear_attn_noalloc_max_bytes",
    "zebra_linear_attn_noalloc", "zebra_fit_affine", "zebra_fit_scale_only",
    "zebra_block_mass_workspace", "zebra_block_mass", "zebra_spatial_order",
    "zebra_permute_tokens", "zebra_linear_attn_backward_workspace", "zebra_linear_attn_backward",
    "zebra_tile_sparse_attn_backward_workspace", "zebra_tile_sparse_attn_backward",
    "zebra_status_string", "zebra_version",
)


class ZebraLibraryError(RuntimeError):
    """libzebra.so is missing or unusable."""


class ZebraError(RuntimeError):
    """A libzebra call returned a non-OK status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)}")


class ZebraSeq(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("stride_token", ctypes.c_int64),
                ("stride_head", ctypes.c_int64)]


_lib = None


def _declare(lib):
    c_i32, c_i64, c_sz, c_p, c_f = (ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                    ctypes.c_void_p, ctypes.c_float)
    sigs = {
        "zebra_pool_landmarks": (c_i32, [c_p, ZebraSeq, c_i32, c_p, c_p]),
        "zebra_select_tiles_workspace": (c_sz, [c_i32, c_i32, c_i32]),
        "zebra_select_tiles": (c_i32, [c_p, c_p, c_i32, c_i32, c_i32, c_i32, c_i32, c_p, c_p,
                                       c_sz, c_p]),
        "zebra_tile_sparse_attn_workspace": (c_sz, [c_i64, c_i64, c_i32, c_i32, c_i32, c_i32,
                                                     c_i32]),
        "zebra_tile_sparse_attn": (c_i32, [c_p, ZebraSeq, c_p, c_p, ZebraSeq, c_p, c_p, c_p,
                                           c_i32, c_i32, c_i32, c_f, c_p, ZebraSeq, c_i32, c_p,
                                           c_sz, c_p]),
        "zebra_tile_sparse_attn_ex": (c_i32, [c_p, ZebraSeq, c_p, c_p, ZebraSeq, c_p, c_p, c_p,
                                              c_i32, c_i32, c_i32, c_f, c_p, ZebraSeq, c_i32,
                                              ctypes.c_uint32, c_p, c_sz, c_p]),
        "zebra_tile_sparse_attn_lse": (c_i32, [c_p, ZebraSeq, c_p, c_p, ZebraSeq, c_p, c_p, c_p,
                                               c_i32, c_i32, c_i32, c_f, c_p, ZebraSeq, c_i32,
                                               ctypes.c_uint32, c_p, c_p, c_sz, c_p]),
        "zebra_tile_sparse_attn_backward_lse": (c_i32, [c_p, ZebraSeq, c_p, c_p, ZebraSeq, c_p,
                                                        c_p, c_p, c_i32, c_i32, c_i32, c_f,
                                                        ctypes.c_uint32, c_p, c_p, ZebraSeq, c_i32,
                                                        c_p, ZebraSeq, c_p, c_p, ZebraSeq, c_p,
                                                        c_sz, c_p]),
        "zebra_tile_sparse_attn_backward_saved": (c_i32, [c_p, ZebraSeq, c_p, c_p, ZebraSeq,
                                                          c_p, c_p, c_p, c_i32, c_i32, c_i32, c_f,
                                                          ctypes.c_uint32, c_p, c_p, ZebraSeq,
                                                          c_p, ZebraSeq, c_i32, c_p, ZebraSeq,
                                                          c_p, c_p, ZebraSeq, c_p, c_sz, c_p]),
        "zebra_linear_attn_workspace": (c_sz, [c_i64, c_i32, c_i32]),
        "zebra_linear_attn": (c_i32, [c_p, ZebraSeq, c_p, c_p, ZebraSeq, c_p, c_p, c_p, ZebraSeq,
                                      c_i32, c_p, c_sz, c_p]),
        "zebra_linear_attn_noalloc_max_bytes": (c_sz, []),
        "zebra_linear_attn_noalloc": (c_i32, [c_p, ZebraSeq, c_p, c_p, ZebraSeq, c_p, c_p, c_p,
                                              ZebraSeq, c_i32, c_p]),
        "zebra_fit_affine": (c_i32, [c_p, c_p, c_i32, c_i32, c_i32, c_p, c_p, c_p, c_p]),
        "zebra_fit_scale_only": (c_i32, [c_p, c_p, c_i32, c_i32, c_i32, c_p, c_p, c_p, c_p]),
        "zebra_block_mass_workspace": (c_sz, [c_i64, c_i32]),
        "zebra_block_mass": (c_i32, [c_p, ZebraSeq, c_p, ZebraSeq, c_i32, c_i32, c_f, c_p, c_p,
                                     c_sz, c_p]),
        "zebra_spatial_order": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32, c_p, c_i64]),
        "zebra_permute_tokens": (c_i32, [c_p, ZebraSeq, c_p, c_i32, c_i32, c_p, ZebraSeq, c_p]),
        "zebra_tile_sparse_attn_backward_workspace": (c_sz, [c_i64, c_i64, c_i32, c_i32, c_i32,
                                                             c_i32, c_i32]),
        "zebra_tile_sparse_attn_backward": (c_i32, [c_p, ZebraSeq, c_p, c_p, ZebraSeq, c_p, c_p,
                                                    c_p, c_i32, c_i32, c_i32, c_f,
                                                    ctypes.c_uint32, c_p, ZebraSeq, c_i32, c_p,
                                                    ZebraSeq, c_p, c_p, ZebraSeq, c_p, c_sz,
                                                    c_p]),
        "zebra_linear_attn_backward_workspace": (c_sz, [c_i64, c_i64, c_i32, c_i32]),
        "zebra_linear_attn_backward": (c_i32, [c_p, ZebraSeq, c_p, c_p, ZebraSeq, c_p, c_p,
                                               ZebraSeq, c_i32, c_p, ZebraSeq, c_p, c_p, ZebraSeq,
                                               c_p, c_p, c_p, c_sz, c_p]),
        "zebra_status_string": (ctypes.c_char_p, [c_i32]),
        "zebra_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


def library():
    """The loaded libzebra (raises ZebraLibraryError when it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ZebraLibraryError(
                f"{LIB_PATH} is not built; run `python -m linear_hybrid_attention_zebra_amd.build`")
        try:
            lib = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_GLOBAL)
            _declare(lib)
        except (OSError, AttributeError) as e:
            raise ZebraLibraryError(f"cannot load {LIB_PATH}: {e}") from e
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return library().zebra_status_string(status).decode()


def version() -> str:
    return library().zebra_version().decode()


def _check(fn: str, status: int):
    if status != ZEBRA_OK:
        raise ZebraError(fn, status)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def seq_of(t: torch.Tensor) -> ZebraSeq:
    """zebra_seq of a [H][N][64] tensor (channel dimension contiguous)."""
    if t.dim() != 3 or t.shape[2] != HEAD_DIM or (t.numel() and t.stride(2) != 1):
        raise ValueError(f"expected a [H][N][{HEAD_DIM}] tensor with contiguous channels, "
                         f"got shape {tuple(t.shape)} strides {tuple(t.stride())}")
    return ZebraSeq(t.shape[1], t.shape[0], t.shape[2], t.stride(1), t.stride(0))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, dtype, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]):
    if nbytes == 0:
        return ws
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


# ----------------------------------------------------------------------------
# the five entry points
# ----------------------------------------------------------------------------

def zebra_pool_landmarks(x: torch.Tensor, tile: int,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Mean over the valid tokens of each tile: bf16 [H][N][64] -> float32 [H][ceil(N/tile)][64]."""
    _need(x, torch.bfloat16, "x")
    h, n = x.shape[0], x.shape[1]
    if out is None:
        out = torch.empty((h, ceil_div(n, tile), HEAD_DIM), dtype=torch.float32, device=x.device)
    _need(out, torch.float32, "out")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    _check("zebra_pool_landmarks", library().zebra_pool_landmarks(
        _ptr(x), seq_of(x), tile, _ptr(out), _stream(x.device)))
    return out


def zebra_select_tiles(qbar: torch.Tensor, kbar: torch.Tensor, top_k: int,
                       out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Top-k key tiles per query tile by qbar . kbar (ties to the lower index), ascending int32."""
    _need(qbar, torch.float32, "qbar")
    _need(kbar, torch.float32, "kbar")
    if not (qbar.is_contiguous() and kbar.is_contiguous()):
        raise ValueError("qbar and kbar must be contiguous")
    h, tq, tk = qbar.shape[0], qbar.shape[1], kbar.shape[1]
    if out is None:
        out = torch.empty((h, tq, top_k), dtype=torch.int32, device=qbar.device)
    _need(out, torch.int32, "out")
    lib = library()
    nbytes = lib.zebra_select_tiles_workspace(h, tq, tk)
    workspace = _workspace(nbytes, qbar.device, workspace)
    _check("zebra_select_tiles", lib.zebra_select_tiles(
        _ptr(qbar), _ptr(kbar), h, tq, tk, qbar.shape[2], top_k, _ptr(out), _ptr(workspace),
        nbytes, _stream(qbar.device)))
    return out


def zebra_tile_sparse_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                           kbar: Optional[torch.Tensor], vbar: Optional[torch.Tensor],
                           sel: Optional[torch.Tensor], q_tile: int, k_tile: int, top_k: int,
                           scale: float, out: Optional[torch.Tensor] = None,
                           out_dtype=torch.bfloat16,
                           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Tile-sparse softmax attention with mean-key/value landmarks (sel=None: dense)."""
    return zebra_tile_sparse_attn_ex(q, k, v, kbar, vbar, sel, q_tile, k_tile, top_k, scale, 0,
                                     out, out_dtype, workspace)


def zebra_tile_sparse_attn_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                              kbar: Optional[torch.Tensor], vbar: Optional[torch.Tensor],
                              sel: Optional[torch.Tensor], q_tile: int, k_tile: int, top_k: int,
                              scale: float, flags: int, out: Optional[torch.Tensor] = None,
                              out_dtype=torch.bfloat16,
                              workspace: Optional[torch.Tensor] = None,
                              lse_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Sparse-operator variants: flags ZEBRA_SPARSE_NO_LANDMARKS (kbar, vbar may be
    None) or ZEBRA_SPARSE_LANDMARK_LOG_COUNT; 0 is zebra_tile_sparse_attn. With
    lse_out (float32 [H][Nq]) it calls zebra_tile_sparse_attn_lse, which also
    writes each query's softmax normaliser for zebra_tile_sparse_attn_backward."""
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, name)
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v must share shape and strides")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out must be bfloat16 or float32")
    if sel is not None:
        _need(sel, torch.int32, "sel")
        if not sel.is_contiguous():
            raise ValueError("sel must be contiguous")
        for t, name in ((kbar, "kbar"), (vbar, "vbar")):
            if t is not None or not flags & ZEBRA_SPARSE_NO_LANDMARKS:
                _need(t, torch.float32, name)
                if not t.is_contiguous():
                    raise ValueError(f"{name} must be contiguous")
    lib = library()
    nbytes = lib.zebra_tile_sparse_attn_workspace(q.shape[1], k.shape[1], k.shape[0], HEAD_DIM,
                                                  q_tile, k_tile, top_k)
    workspace = _workspace(nbytes, q.device, workspace)
    if lse_out is not None:
        _need(lse_out, torch.float32, "lse_out")
        if not lse_out.is_contiguous() or lse_out.numel() != q.shape[0] * q.shape[1]:
            raise ValueError("lse_out must be a contiguous [H][Nq] float32 tensor")
        _check("zebra_tile_sparse_attn_lse", lib.zebra_tile_sparse_attn_lse(
            _ptr(q), seq_of(q), _ptr(k), _ptr(v), seq_of(k), _ptr(kbar), _ptr(vbar), _ptr(sel),
            q_tile, k_tile, top_k, scale, _ptr(out), seq_of(out),
            ZEBRA_F32 if out.dtype == torch.float32 else ZEBRA_BF16, flags, _ptr(lse_out),
            _ptr(workspace), nbytes, _stream(q.device)))
        return out
    _check("zebra_tile_sparse_attn_ex", lib.zebra_tile_sparse_attn_ex(
        _ptr(q), seq_of(q), _ptr(k), _ptr(v), seq_of(k), _ptr(kbar), _ptr(vbar), _ptr(sel),
        q_tile, k_tile, top_k, scale, _ptr(out), seq_of(out),
        ZEBRA_F32 if out.dtype == torch.float32 else ZEBRA_BF16, flags, _ptr(workspace), nbytes,
        _stream(q.device)))
    return out


def zebra_linear_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      aff_scale: Optional[torch.Tensor] = None,
                      aff_bias: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """elu+1 linear attention, then a (*) o + b per head and channel."""
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, name)
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v must share shape and strides")
    for t, name in ((aff_scale, "aff_scale"), (aff_bias, "aff_bias")):
        if t is not None:
            _need(t, torch.float32, name)
            if not t.is_contiguous() or t.numel() != q.shape[0] * HEAD_DIM:
                raise ValueError(f"{name} must be a contiguous [H][64] float32 tensor")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    lib = library()
    nbytes = lib.zebra_linear_attn_workspace(k.shape[1], k.shape[0], HEAD_DIM)
    workspace = _workspace(nbytes, q.device, workspace)
    _check("zebra_linear_attn", lib.zebra_linear_attn(
        _ptr(q), seq_of(q), _ptr(k), _ptr(v), seq_of(k), _ptr(aff_scale), _ptr(aff_bias),
        _ptr(out), seq_of(out), ZEBRA_F32 if out.dtype == torch.float32 else ZEBRA_BF16,
        _ptr(workspace), nbytes, _stream(q.device)))
    return out


def zebra_linear_attn_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                              aff_scale: Optional[torch.Tensor] = None,
                              aff_bias: Optional[torch.Tensor] = None,
                              out: Optional[torch.Tensor] = None,
                              out_dtype=torch.bfloat16) -> torch.Tensor:
    """zebra_linear_attn with the library's fixed device scratch instead of a
    workspace (the C call allocates nothing; pass `out` to allocate nothing here)."""
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, name)
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v must share shape and strides")
    for t, name in ((aff_scale, "aff_scale"), (aff_bias, "aff_bias")):
        if t is not None:
            _need(t, torch.float32, name)
            if not t.is_contiguous() or t.numel() != q.shape[0] * HEAD_DIM:
                raise ValueError(f"{name} must be a contiguous [H][64] float32 tensor")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _check("zebra_linear_attn_noalloc", library().zebra_linear_attn_noalloc(
        _ptr(q), seq_of(q), _ptr(k), _ptr(v), seq_of(k), _ptr(aff_scale), _ptr(aff_bias),
        _ptr(out), seq_of(out), ZEBRA_F32 if out.dtype == torch.float32 else ZEBRA_BF16,
        _stream(q.device)))
    return out


def zebra_fit_affine(x: torch.Tensor, y: torch.Tensor, scale_out: Optional[torch.Tensor] = None,
                     bias_out: Optional[torch.Tensor] = None,
                     n_degenerate: Optional[torch.Tensor] = None):
    """Closed-form least-squares a, b per (head, channel) from x, y float32 [H][M][64]."""
    return _fit("zebra_fit_affine", x, y, scale_out, bias_out, n_degenerate)


def zebra_fit_scale_only(x: torch.Tensor, y: torch.Tensor,
                         scale_out: Optional[torch.Tensor] = None,
                         bias_out: Optional[torch.Tensor] = None,
                         n_degenerate: Optional[torch.Tensor] = None):
    """Uncentered fit: a = sum x y / sum x^2, b = 0 per (head, channel)."""
    return _fit("zebra_fit_scale_only", x, y, scale_out, bias_out, n_degenerate)


def _fit(entry, x, y, scale_out, bias_out, n_degenerate):
    _need(x, torch.float32, "x")
    _need(y, torch.float32, "y")
    if x.shape != y.shape or not (x.is_contiguous() and y.is_contiguous()):
        raise ValueError("x and y must be contiguous and of the same shape")
    h, m = x.shape[0], x.shape[1]
    if scale_out is None:
        scale_out = torch.empty((h, HEAD_DIM), dtype=torch.float32, device=x.device)
    if bias_out is None:
        bias_out = torch.empty((h, HEAD_DIM), dtype=torch.float32, device=x.device)
    if n_degenerate is None:
        n_degenerate = torch.empty(1, dtype=torch.int32, device=x.device)
    _check(entry, getattr(library(), entry)(
        _ptr(x), _ptr(y), m, h, x.shape[2], _ptr(scale_out), _ptr(bias_out), _ptr(n_degenerate),
        _stream(x.device)))
    return scale_out, bias_out, n_degenerate


def zebra_block_mass(q: torch.Tensor, k: torch.Tensor, q_tile: int, k_tile: int, scale: float,
                     out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Dense-softmax attention mass of every (query tile, key tile) block: float32 [H][Tq][Tk]."""
    _need(q, torch.bfloat16, "q")
    _need(k, torch.bfloat16, "k")
    h = q.shape[0]
    if out is None:
        out = torch.empty((h, ceil_div(q.shape[1], q_tile), ceil_div(k.shape[1], k_tile)),
                          dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    lib = library()
    nbytes = lib.zebra_block_mass_workspace(q.shape[1], h)
    workspace = _workspace(nbytes, q.device, workspace)
    _check("zebra_block_mass", lib.zebra_block_mass(
        _ptr(q), seq_of(q), _ptr(k), seq_of(k), q_tile, k_tile, scale, _ptr(out),
        _ptr(workspace), nbytes, _stream(q.device)))
    return out


def zebra_spatial_order(n_views: int, n_special: int, grid_h: int, grid_w: int,
                        block: int) -> torch.Tensor:
    """Spatial token order (host int32 tensor): position i holds original token order[i]."""
    n = n_views * (n_special + grid_h * grid_w)
    out = torch.empty(n, dtype=torch.int32)
    _check("zebra_spatial_order", library().zebra_spatial_order(
        n_views, n_special, grid_h, grid_w, block, out.data_ptr() if n else None, n))
    return out


def zebra_permute_tokens(src: torch.Tensor, order: torch.Tensor, inverse: bool = False,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gather (out[h][i] = src[h][order[i]]) or, with inverse, scatter of [H][N][64] rows."""
    if src.dtype not in (torch.bfloat16, torch.float32) or not src.is_cuda:
        raise ValueError("src must be a bfloat16 or float32 CUDA tensor")
    _need(order, torch.int32, "order")
    if not order.is_contiguous() or order.numel() != src.shape[1]:
        raise ValueError("order must be a contiguous int32 vector of N entries")
    if out is None:
        out = torch.empty_like(src)
    if out.dtype != src.dtype:
        raise ValueError("out must have the dtype of src")
    _check("zebra_permute_tokens", library().zebra_permute_tokens(
        _ptr(src), seq_of(src), _ptr(order), 1 if inverse else 0,
        ZEBRA_F32 if src.dtype == torch.float32 else ZEBRA_BF16, _ptr(out), seq_of(out),
        _stream(src.device)))
    return out


def zebra_linear_attn_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                               dout: torch.Tensor, aff_scale: Optional[torch.Tensor] = None,
                               workspace: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv, d_scale, d_bias) of sum(dout * out) for one linear stage;
    the gradients take dout's dtype (bfloat16 or float32)."""
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, name)
    if dout.dtype not in (torch.bfloat16, torch.float32) or not dout.is_cuda:
        raise ValueError("dout must be a bfloat16 or float32 CUDA tensor")
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v must share shape and strides")
    if aff_scale is not None:
        _need(aff_scale, torch.float32, "aff_scale")
    h = q.shape[0]
    dq = torch.empty(q.shape, dtype=dout.dtype, device=q.device)
    dk = torch.empty(k.shape, dtype=dout.dtype, device=q.device)
    dv = torch.empty(k.shape, dtype=dout.dtype, device=q.device)
    d_scale = torch.empty((h, HEAD_DIM), dtype=torch.float32, device=q.device)
    d_bias = torch.empty((h, HEAD_DIM), dtype=torch.float32, device=q.device)
    lib = library()
    nbytes = lib.zebra_linear_attn_backward_workspace(q.shape[1], k.shape[1], h, HEAD_DIM)
    workspace = _workspace(nbytes, q.device, workspace)
    _check("zebra_linear_attn_backward", lib.zebra_linear_attn_backward(
        _ptr(q), seq_of(q), _ptr(k), _ptr(v), seq_of(k), _ptr(aff_scale), _ptr(dout),
        seq_of(dout), ZEBRA_F32 if dout.dtype == torch.float32 else ZEBRA_BF16, _ptr(dq),
        seq_of(dq), _ptr(dk), _ptr(dv), seq_of(dk), _ptr(d_scale), _ptr(d_bias),
        _ptr(workspace), nbytes, _stream(q.device)))
    return dq, dk, dv, d_scale, d_bias


def zebra_tile_sparse_attn_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                    kbar: Optional[torch.Tensor], vbar: Optional[torch.Tensor],
                                    sel: torch.Tensor, q_tile: int, k_tile: int, top_k: int,
                                    scale: float, dout: torch.Tensor, flags: int = 0,
                                    workspace: Optional[torch.Tensor] = None,
                                    lse: Optional[torch.Tensor] = None,
                                    out: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv) of sum(dout * out) for one tile-sparse stage, sel fixed;
    the gradients take dout's dtype (bfloat16 or float32). With lse, the normaliser a
    forward call wrote (zebra_tile_sparse_attn_ex with lse_out), the call does not
    run the forward again: with that call's float32 output as out too, through
    zebra_tile_sparse_attn_backward_saved (bitwise the plain backward), else through
    zebra_tile_sparse_attn_backward_lse."""
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, name)
    _need(sel, torch.int32, "sel")
    if dout.dtype not in (torch.bfloat16, torch.float32) or not dout.is_cuda:
        raise ValueError("dout must be a bfloat16 or float32 CUDA tensor")
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v must share shape and strides")
    for t, name in ((kbar, "kbar"), (vbar, "vbar")):
        if t is not None:
            _need(t, torch.float32, name)
    dq = torch.empty(q.shape, dtype=dout.dtype, device=q.device)
    dk = torch.empty(k.shape, dtype=dout.dtype, device=q.device)
    dv = torch.empty(k.shape, dtype=dout.dtype, device=q.device)
    lib = library()
    nbytes = lib.zebra_tile_sparse_attn_backward_workspace(q.shape[1], k.shape[1], q.shape[0],
                                                           HEAD_DIM, q_tile, k_tile, top_k)
    workspace = _workspace(nbytes, q.device, workspace)
    g_dtype = ZEBRA_F32 if dout.dtype == torch.float32 else ZEBRA_BF16
    if out is not None and lse is None:
        raise ValueError("out is read only together with lse")
    if lse is not None:
        _need(lse, torch.float32, "lse")
        if not lse.is_contiguous() or lse.numel() != q.shape[0] * q.shape[1]:
            raise ValueError("lse must be a contiguous [H][Nq] float32 tensor")
    if out is not None:
        _need(out, torch.float32, "out")
        _check("zebra_tile_sparse_attn_backward_saved", lib.zebra_tile_sparse_attn_backward_saved(
            _ptr(q), seq_of(q), _ptr(k), _ptr(v), seq_of(k), _ptr(kbar), _ptr(vbar), _ptr(sel),
            q_tile, k_tile, top_k, scale, flags, _ptr(lse), _ptr(out), seq_of(out), _ptr(dout),
            seq_of(dout), g_dtype, _ptr(dq), seq_of(dq), _ptr(dk), _ptr(dv), seq_of(dk),
            _ptr(workspace), nbytes, _stream(q.device)))
        return dq, dk, dv
    if lse is not None:
        _check("zebra_tile_sparse_attn_backward_lse", lib.zebra_tile_sparse_attn_backward_lse(
            _ptr(q), seq_of(q), _ptr(k), _ptr(v), seq_of(k), _ptr(kbar), _ptr(vbar), _ptr(sel),
            q_tile, k_tile, top_k, scale, flags, _ptr(lse), _ptr(dout), seq_of(dout), g_dtype,
            _ptr(dq), seq_of(dq), _ptr(dk), _ptr(dv), seq_of(dk), _ptr(workspace), nbytes,
            _stream(q.device)))
        return dq, dk, dv
    _check("zebra_tile_sparse_attn_backward", lib.zebra_tile_sparse_attn_backward(
        _ptr(q), seq_of(q), _ptr(k), _ptr(v), seq_of(k), _ptr(kbar), _ptr(vbar), _ptr(sel),
        q_tile, k_tile, top_k, scale, flags, _ptr(dout), seq_of(dout), g_dtype, _ptr(dq),
        seq_of(dq), _ptr(dk), _ptr(dv), seq_of(dk), _ptr(workspace), nbytes, _stream(q.device)))
    return dq, dk, dv
