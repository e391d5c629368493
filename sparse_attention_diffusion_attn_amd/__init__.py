"""MC-Sparse attention hot path on AMD Instinct MI355X (gfx950).

Thin Python binding over the C-ABI library libmcs.so (include/mcs.h).  The
functions here only check and marshal arguments; every step of the path runs
in the library's HIP kernels.  PyTorch supplies device memory and the current
stream.  There is no fallback: if libmcs.so is missing or fails to load, every
call raises.

Anchor step:  perm = group(q, ...);  o_full, lse, kv_idx = anchor_select(...);
              r = residual(...)
Reuse step:   o = sparse_attn(q_t, k_t, v_t, perm, kv_idx, r, ...)
Selection variants of the oracle analysis (block oracle, vanilla BSA):
              kv_idx, kv_count = block_select(...);  r = residual_counts(...);
              o = sparse_attn_counts(...)
Grouping comparator (size-balanced k-means): perm = group_kmeans(...)

group, anchor_select, residual, sparse_attn and dense_attn also take Q, K, V
and the output as strided [B, H, n_pad, d] views with contiguous rows (e.g. a
[B, N, H, d] tensor transposed, or slices of a fused QKV projection); they are
then passed to the library's `_strided` calls.
"""
from __future__ import annotations

import ctypes
import math
import os
import re
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MCS_LIBRARY may name another build of the same library (e.g. the
# sanitizer-instrumented one the build step makes with --sanitized)
LIB_PATH = os.environ.get("MCS_LIBRARY") or os.path.join(_PKG, "libmcs.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "mcs.h")

MCS_OK, MCS_ERR_INVALID_ARG, MCS_ERR_UNSUPPORTED, MCS_ERR_WORKSPACE, MCS_ERR_HIP = range(5)
BLOCK_EXACT, BLOCK_MEANPOOL = 0, 1


class MCSError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {message} (status {status})")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("n_valid", ctypes.c_int32),
                ("n_pad", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("group_size", ctypes.c_int32)]


class Strides(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64), ("token", ctypes.c_int64)]


class Layout(ctypes.Structure):
    _fields_ = [("q", Strides), ("k", Strides), ("v", Strides), ("o", Strides)]


_LIB: Optional[ctypes.CDLL] = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_SZ = ctypes.c_size_t
_F = ctypes.c_float
_DP = ctypes.POINTER(Dims)
_LP = ctypes.POINTER(Layout)

_SIGNATURES = {
    "mcs_abi_version": (_I, []),
    "mcs_status_string": (ctypes.c_char_p, [_I]),
    "mcs_last_error": (ctypes.c_char_p, []),
    "mcs_group_workspace_bytes": (_SZ, [_DP]),
    "mcs_group": (_I, [_DP, _P, _I, _I, _P, _P, _SZ, _P]),
    "mcs_anchor_select_workspace_bytes": (_SZ, [_DP, _I]),
    "mcs_anchor_select_min_workspace_bytes": (_SZ, [_DP, _I]),
    "mcs_anchor_select": (_I, [_DP, _P, _P, _P, _P, _I, _F, _P, _P, _P, _P, _SZ, _P]),
    "mcs_anchor_select_noalloc": (_I, [_DP, _P, _P, _P, _P, _I, _F, _P, _P, _P, _P]),
    "mcs_residual": (_I, [_DP, _P, _P, _P, _P, _P, _I, _F, _P, _P, _P]),
    "mcs_sparse_attn": (_I, [_DP, _P, _P, _P, _P, _P, _I, _F, _P, _P, _P]),
    "mcs_dense_attn": (_I, [_DP, _P, _P, _P, _F, _P, _P, _P]),
    "mcs_block_select_workspace_bytes": (_SZ, [_DP, _I, _I, _I]),
    "mcs_block_select_min_workspace_bytes": (_SZ, [_DP, _I, _I, _I]),
    "mcs_block_select": (_I, [_DP, _P, _P, _P, _P, _I, _I, _I, _F, _P, _P, _P, _SZ, _P]),
    "mcs_sparse_attn_counts": (_I, [_DP, _P, _P, _P, _P, _P, _I, _P, _F, _P, _P, _P]),
    "mcs_residual_counts": (_I, [_DP, _P, _P, _P, _P, _P, _I, _P, _F, _P, _P, _P]),
    "mcs_group_kmeans_workspace_bytes": (_SZ, [_DP]),
    "mcs_group_kmeans": (_I, [_DP, _P, _I, _P, _P, _P, _SZ, _P]),
    "mcs_layout_bhnd": (None, [_DP, _LP]),
    "mcs_layout_bnhd": (None, [_DP, _LP]),
    "mcs_group_strided": (_I, [_DP, _LP, _P, _I, _I, _P, _P, _SZ, _P]),
    "mcs_anchor_select_strided": (_I, [_DP, _LP, _P, _P, _P, _P, _I, _F, _P, _P, _P, _P, _SZ, _P]),
    "mcs_residual_strided": (_I, [_DP, _LP, _P, _P, _P, _P, _P, _I, _F, _P, _P, _P]),
    "mcs_sparse_attn_strided": (_I, [_DP, _LP, _P, _P, _P, _P, _P, _I, _F, _P, _P, _P]),
    "mcs_dense_attn_strided": (_I, [_DP, _LP, _P, _P, _P, _F, _P, _P, _P]),
}


def lib() -> ctypes.CDLL:
    """Load libmcs.so (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_attention_diffusion_attn_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def header_functions() -> list:
    """Names of the functions include/mcs.h declares."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"\b(mcs_[a-z_]+)\s*\(", text)))


def _check(status: int, where: str) -> None:
    if status != MCS_OK:
        msg = lib().mcs_last_error().decode()
        raise MCSError(status, where, msg)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def make_dims(batch, heads, n_valid, n_pad, head_dim, group_size) -> Dims:
    return Dims(batch, heads, n_valid, n_pad, head_dim, group_size)


def _dims_of(q: torch.Tensor, n_valid: int, group_size: int) -> Dims:
    if q.dim() != 4:
        raise ValueError("q must be [batch, heads, n_pad, head_dim]")
    b, h, n_pad, d = q.shape
    return Dims(b, h, n_valid, n_pad, d, group_size)


def _need(t: torch.Tensor, name: str, dtype, shape) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _view(t: torch.Tensor, name: str, shape) -> int:
    """A bf16 device tensor of `shape` [B, H, n_pad, d] whose rows are
    contiguous (stride 1 along d); other strides are passed in a Layout."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be torch.bfloat16, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.stride(-1) != 1:
        raise ValueError(f"{name} must have contiguous rows (stride 1 along head_dim)")
    return t.data_ptr()


def _strides(t: torch.Tensor) -> Strides:
    return Strides(t.stride(0), t.stride(1), t.stride(2))


def layout_of(q, k, v, o) -> Optional[Layout]:
    """None if q, k, v and o are all contiguous, else their Layout."""
    if all(t.is_contiguous() for t in (q, k, v, o)):
        return None
    return Layout(_strides(q), _strides(k), _strides(v), _strides(o))


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def group_workspace_bytes(dims: Dims) -> int:
    return int(lib().mcs_group_workspace_bytes(ctypes.byref(dims)))


def anchor_select_workspace_bytes(dims: Dims, topk: int, minimum: bool = False) -> int:
    fn = lib().mcs_anchor_select_min_workspace_bytes if minimum else lib().mcs_anchor_select_workspace_bytes
    return int(fn(ctypes.byref(dims), topk))


def anchor_scores(workspace: torch.Tensor, dims: Dims) -> torch.Tensor:
    """The fp32 group scores [B*H, n_pad/C, n_valid] that mcs_anchor_select
    left in an all-heads workspace (the layout include/mcs.h documents), as a
    view of `workspace`."""
    bh = dims.batch * dims.heads
    G = dims.n_pad // dims.group_size
    if workspace.numel() * workspace.element_size() < anchor_select_workspace_bytes(dims, 1):
        raise ValueError("workspace does not hold the scores of all heads")
    n = bh * G * dims.n_valid
    return workspace.view(torch.uint8)[: 4 * n].view(torch.float32).view(bh, G, dims.n_valid)


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is None:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    return ws


def group(q: torch.Tensor, n_valid: int, group_size: int, power_iters: int = 20,
          max_levels: int = -1, perm: Optional[torch.Tensor] = None,
          workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Fast PDDP grouping -> perm int32 [B, H, n_pad] (mcs_group).  `q` may be
    a strided [B, H, n_pad, d] view with contiguous rows (mcs_group_strided)."""
    dims = _dims_of(q, n_valid, group_size)
    b, h, n_pad, d = q.shape
    if perm is None:
        perm = torch.empty((b, h, n_pad), dtype=torch.int32, device=q.device)
    ws = _workspace(group_workspace_bytes(dims), q.device, workspace)
    qp = _view(q, "q", q.shape)
    pp = _need(perm, "perm", torch.int32, (b, h, n_pad))
    wsp, wsn = ws.data_ptr(), ws.numel() * ws.element_size()
    if q.is_contiguous():
        st = lib().mcs_group(ctypes.byref(dims), qp, power_iters, max_levels, pp, wsp, wsn,
                             _stream(stream))
    else:
        lay = Layout(_strides(q), _strides(q), _strides(q), _strides(q))
        st = lib().mcs_group_strided(ctypes.byref(dims), ctypes.byref(lay), qp, power_iters,
                                     max_levels, pp, wsp, wsn, _stream(stream))
    _check(st, "mcs_group")
    return perm


def group_kmeans(q: torch.Tensor, n_valid: int, group_size: int, iters: int = 10,
                 perm: Optional[torch.Tensor] = None, labels: Optional[torch.Tensor] = None,
                 want_labels: bool = False, workspace: Optional[torch.Tensor] = None,
                 stream=None):
    """Size-balanced k-means grouping, the comparator of Fast PDDP
    (mcs_group_kmeans) -> perm int32 [B, H, n_pad], or (perm, labels) with
    want_labels (the last iteration's nearest centroid of every token)."""
    dims = _dims_of(q, n_valid, group_size)
    b, h, n_pad, d = q.shape
    if perm is None:
        perm = torch.empty((b, h, n_pad), dtype=torch.int32, device=q.device)
    if labels is None and want_labels:
        labels = torch.empty((b, h, n_pad), dtype=torch.int32, device=q.device)
    lp = None if labels is None else _need(labels, "labels", torch.int32, (b, h, n_pad))
    nbytes = int(lib().mcs_group_kmeans_workspace_bytes(ctypes.byref(dims)))
    ws = _workspace(nbytes, q.device, workspace)
    st = lib().mcs_group_kmeans(ctypes.byref(dims), _need(q, "q", torch.bfloat16, q.shape), iters,
                                _need(perm, "perm", torch.int32, (b, h, n_pad)), lp,
                                ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "mcs_group_kmeans")
    return (perm, labels) if want_labels else perm


def _contig_out(q: torch.Tensor) -> torch.Tensor:
    return torch.empty(q.shape, dtype=q.dtype, device=q.device)


def anchor_select(q, k, v, perm, n_valid: int, group_size: int, topk: int,
                  scale: Optional[float] = None, o_full=None, lse=None, kv_idx=None,
                  workspace: Optional[torch.Tensor] = None, stream=None):
    """Two-pass exact selection -> (o_full, lse, kv_idx) (mcs_anchor_select).
    q, k, v and o_full may be strided views (mcs_anchor_select_strided); the
    default o_full has q's layout where torch can reproduce it."""
    dims = _dims_of(q, n_valid, group_size)
    b, h, n_pad, d = q.shape
    G = n_pad // group_size
    scale = default_scale(d) if scale is None else scale
    if o_full is None:
        o_full = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((b, h, n_pad), dtype=torch.float32, device=q.device)
    if kv_idx is None:
        kv_idx = torch.empty((b, h, G, topk), dtype=torch.int32, device=q.device)
    ws = _workspace(anchor_select_workspace_bytes(dims, topk), q.device, workspace)
    args = (_view(q, "q", q.shape), _view(k, "k", q.shape), _view(v, "v", q.shape),
            _need(perm, "perm", torch.int32, (b, h, n_pad)), topk, scale,
            _view(o_full, "o_full", q.shape), _need(lse, "lse", torch.float32, (b, h, n_pad)),
            _need(kv_idx, "kv_idx", torch.int32, (b, h, G, topk)),
            ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream))
    lay = layout_of(q, k, v, o_full)
    if lay is None:
        st = lib().mcs_anchor_select(ctypes.byref(dims), *args)
    else:
        st = lib().mcs_anchor_select_strided(ctypes.byref(dims), ctypes.byref(lay), *args)
    _check(st, "mcs_anchor_select")
    return o_full, lse, kv_idx


def anchor_select_noalloc(q, k, v, perm, n_valid: int, group_size: int, topk: int,
                          scale: Optional[float] = None, o_full=None, lse=None, kv_idx=None,
                          stream=None):
    """mcs_anchor_select with the library's fixed device scratch as workspace
    (mcs_anchor_select_noalloc): nothing is allocated beyond the outputs
    (pass them in to allocate nothing at all).  Contiguous tensors only."""
    dims = _dims_of(q, n_valid, group_size)
    b, h, n_pad, d = q.shape
    G = n_pad // group_size
    scale = default_scale(d) if scale is None else scale
    if o_full is None:
        o_full = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((b, h, n_pad), dtype=torch.float32, device=q.device)
    if kv_idx is None:
        kv_idx = torch.empty((b, h, G, topk), dtype=torch.int32, device=q.device)
    st = lib().mcs_anchor_select_noalloc(
        ctypes.byref(dims), _need(q, "q", torch.bfloat16, q.shape), _need(k, "k", torch.bfloat16, q.shape),
        _need(v, "v", torch.bfloat16, q.shape), _need(perm, "perm", torch.int32, (b, h, n_pad)), topk, scale,
        _need(o_full, "o_full", torch.bfloat16, q.shape), _need(lse, "lse", torch.float32, (b, h, n_pad)),
        _need(kv_idx, "kv_idx", torch.int32, (b, h, G, topk)), _stream(stream))
    _check(st, "mcs_anchor_select_noalloc")
    return o_full, lse, kv_idx


NOALLOC_SCRATCH_BYTES = 192 << 20


def residual(q, k, v, perm, kv_idx, o_full, n_valid: int, group_size: int,
             scale: Optional[float] = None, r=None, stream=None) -> torch.Tensor:
    """R = O_full - SparseAttn(Q, K, V; perm, kv_idx) (mcs_residual).  q, k, v
    and o_full may be strided views (mcs_residual_strided); R is contiguous."""
    dims = _dims_of(q, n_valid, group_size)
    b, h, n_pad, d = q.shape
    G = n_pad // group_size
    topk = kv_idx.shape[-1]
    scale = default_scale(d) if scale is None else scale
    if r is None:
        r = _contig_out(q)
    args = (_view(q, "q", q.shape), _view(k, "k", q.shape), _view(v, "v", q.shape),
            _need(perm, "perm", torch.int32, (b, h, n_pad)),
            _need(kv_idx, "kv_idx", torch.int32, (b, h, G, topk)), topk, scale,
            _view(o_full, "o_full", q.shape), _need(r, "r", torch.bfloat16, q.shape),
            _stream(stream))
    lay = layout_of(q, k, v, o_full)
    if lay is None:
        st = lib().mcs_residual(ctypes.byref(dims), *args)
    else:
        st = lib().mcs_residual_strided(ctypes.byref(dims), ctypes.byref(lay), *args)
    _check(st, "mcs_residual")
    return r


def sparse_attn(q, k, v, perm, kv_idx, r, n_valid: int, group_size: int,
                scale: Optional[float] = None, o=None, stream=None) -> torch.Tensor:
    """Reuse step O = SparseAttn(Q, K, V; perm, kv_idx) + R (mcs_sparse_attn).
    `r` may be None (no residual).  q, k, v and o may be strided views
    (mcs_sparse_attn_strided); the default o has q's layout where torch can
    reproduce it."""
    dims = _dims_of(q, n_valid, group_size)
    b, h, n_pad, d = q.shape
    G = n_pad // group_size
    topk = kv_idx.shape[-1]
    scale = default_scale(d) if scale is None else scale
    if o is None:
        o = torch.empty_like(q)
    rp = None if r is None else _need(r, "r", torch.bfloat16, q.shape)
    args = (_view(q, "q", q.shape), _view(k, "k", q.shape), _view(v, "v", q.shape),
            _need(perm, "perm", torch.int32, (b, h, n_pad)),
            _need(kv_idx, "kv_idx", torch.int32, (b, h, G, topk)), topk, scale, rp,
            _view(o, "o", q.shape), _stream(stream))
    lay = layout_of(q, k, v, o)
    if lay is None:
        st = lib().mcs_sparse_attn(ctypes.byref(dims), *args)
    else:
        st = lib().mcs_sparse_attn_strided(ctypes.byref(dims), ctypes.byref(lay), *args)
    _check(st, "mcs_sparse_attn")
    return o


def dense_attn(q, k, v, n_valid: int, group_size: int = 128, scale: Optional[float] = None,
               o=None, lse=None, want_lse: bool = True, stream=None):
    """Dense attention -> (o, lse) (mcs_dense_attn).  q, k, v and o may be
    strided views (mcs_dense_attn_strided)."""
    dims = _dims_of(q, n_valid, group_size)
    b, h, n_pad, d = q.shape
    scale = default_scale(d) if scale is None else scale
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((b, h, n_pad), dtype=torch.float32, device=q.device)
    lp = None if lse is None else _need(lse, "lse", torch.float32, (b, h, n_pad))
    args = (_view(q, "q", q.shape), _view(k, "k", q.shape), _view(v, "v", q.shape), scale,
            _view(o, "o", q.shape), lp, _stream(stream))
    lay = layout_of(q, k, v, o)
    if lay is None:
        st = lib().mcs_dense_attn(ctypes.byref(dims), *args)
    else:
        st = lib().mcs_dense_attn_strided(ctypes.byref(dims), ctypes.byref(lay), *args)
    _check(st, "mcs_dense_attn")
    return o, lse


def block_select_workspace_bytes(dims: Dims, mode: int, block: int, nblocks: int,
                                 minimum: bool = False) -> int:
    fn = lib().mcs_block_select_min_workspace_bytes if minimum else lib().mcs_block_select_workspace_bytes
    return int(fn(ctypes.byref(dims), mode, block, nblocks))


def block_select(q, k, perm, lse, mode: int, block: int, nblocks: int, n_valid: int,
                 group_size: int, scale: Optional[float] = None, kv_idx=None, kv_count=None,
                 workspace: Optional[torch.Tensor] = None, stream=None):
    """Block selection of the oracle analysis -> (kv_idx [B,H,G,nblocks*block],
    kv_count [B,H,G]) (mcs_block_select).  `lse` is needed for BLOCK_EXACT and
    may be None for BLOCK_MEANPOOL."""
    dims = _dims_of(q, n_valid, group_size)
    b, h, n_pad, d = q.shape
    G = n_pad // group_size
    scale = default_scale(d) if scale is None else scale
    stride = nblocks * block
    if kv_idx is None:
        kv_idx = torch.empty((b, h, G, stride), dtype=torch.int32, device=q.device)
    if kv_count is None:
        kv_count = torch.empty((b, h, G), dtype=torch.int32, device=q.device)
    lp = None if lse is None else _need(lse, "lse", torch.float32, (b, h, n_pad))
    ws = _workspace(block_select_workspace_bytes(dims, mode, block, nblocks), q.device, workspace)
    st = lib().mcs_block_select(
        ctypes.byref(dims), _need(q, "q", torch.bfloat16, q.shape), _need(k, "k", torch.bfloat16, q.shape),
        _need(perm, "perm", torch.int32, (b, h, n_pad)), lp, mode, block, nblocks, scale,
        _need(kv_idx, "kv_idx", torch.int32, (b, h, G, stride)),
        _need(kv_count, "kv_count", torch.int32, (b, h, G)),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "mcs_block_select")
    return kv_idx, kv_count


def sparse_attn_counts(q, k, v, perm, kv_idx, kv_count, r, n_valid: int, group_size: int,
                       scale: Optional[float] = None, o=None, stream=None) -> torch.Tensor:
    """Reuse step over index rows with per-group counts (mcs_sparse_attn_counts)."""
    dims = _dims_of(q, n_valid, group_size)
    b, h, n_pad, d = q.shape
    G = n_pad // group_size
    stride = kv_idx.shape[-1]
    scale = default_scale(d) if scale is None else scale
    if o is None:
        o = torch.empty_like(q)
    rp = None if r is None else _need(r, "r", torch.bfloat16, q.shape)
    st = lib().mcs_sparse_attn_counts(
        ctypes.byref(dims), _need(q, "q", torch.bfloat16, q.shape), _need(k, "k", torch.bfloat16, q.shape),
        _need(v, "v", torch.bfloat16, q.shape), _need(perm, "perm", torch.int32, (b, h, n_pad)),
        _need(kv_idx, "kv_idx", torch.int32, (b, h, G, stride)), stride,
        _need(kv_count, "kv_count", torch.int32, (b, h, G)), scale, rp,
        _need(o, "o", torch.bfloat16, q.shape), _stream(stream))
    _check(st, "mcs_sparse_attn_counts")
    return o


def residual_counts(q, k, v, perm, kv_idx, kv_count, o_full, n_valid: int, group_size: int,
                    scale: Optional[float] = None, r=None, stream=None) -> torch.Tensor:
    """R = O_full - SparseAttn over index rows with per-group counts
    (mcs_residual_counts)."""
    dims = _dims_of(q, n_valid, group_size)
    b, h, n_pad, d = q.shape
    G = n_pad // group_size
    stride = kv_idx.shape[-1]
    scale = default_scale(d) if scale is None else scale
    if r is None:
        r = torch.empty_like(q)
    st = lib().mcs_residual_counts(
        ctypes.byref(dims), _need(q, "q", torch.bfloat16, q.shape), _need(k, "k", torch.bfloat16, q.shape),
        _need(v, "v", torch.bfloat16, q.shape), _need(perm, "perm", torch.int32, (b, h, n_pad)),
        _need(kv_idx, "kv_idx", torch.int32, (b, h, G, stride)), stride,
        _need(kv_count, "kv_count", torch.int32, (b, h, G)), scale,
        _need(o_full, "o_full", torch.bfloat16, q.shape), _need(r, "r", torch.bfloat16, q.shape),
        _stream(stream))
    _check(st, "mcs_residual_counts")
    return r


def identity_perm(batch: int, heads: int, n_pad: int, device) -> torch.Tensor:
    """The partition whose groups are contiguous token blocks (the query blocks
    of block-sparse attention)."""
    return torch.arange(n_pad, dtype=torch.int32, device=device).expand(batch, heads, n_pad).contiguous()
