"""sparse_kv_amd -- block-sparse long-context decode attention for AMD MI355X.

Thin Python binding (ctypes) over the C ABI of ``libsparse_kv.so``
(declared in include/sparse_kv.h).  Functions carry the C names and only
marshal arguments: they check tensors, allocate outputs with torch when the
caller passes none, and queue the HIP kernels on the current torch stream.
Every step of the computation runs in the library's kernels; there is no
fallback: the first call raises ImportError if the library has not been
built (``python -m sparse_kv_amd.build``).
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparse_kv.so")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP, ATTN_ERR_WORKSPACE = 0, -1, -2, -3, -4
ATTN_F32, ATTN_BF16 = 0, 1
BLOCK = 64

EXPORTS = (
    "attn_decode_dense",
    "attn_merge_states",
    "attn_build_centroids",
    "attn_update_centroids",
    "attn_score_centroids",
    "attn_select_topk",
    "attn_build_super_centroids",
    "attn_select_two_level",
    "attn_decode_sparse",
    "attn_decode_art",
    "attn_decode_art_ws",
    "attn_decode_art_list_ws",
    "attn_decode_art_paged_ws",
    "attn_art_workspace_bytes",
    "attn_decode_art_list",
    "attn_order_blocks",
    "attn_decode_dense_paged",
    "attn_decode_sparse_paged",
    "attn_build_centroids_paged",
    "attn_update_centroids_paged",
    "attn_decode_art_paged",
    "attn_decode_routed",
    "attn_routed_workspace_bytes",
    "attn_decode_routed_static",
    "attn_status_string",
)


class AttnDims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


class AttnPagedKV(ctypes.Structure):
    _fields_ = [
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("pool_blocks", ctypes.c_int64),
        ("block_table", ctypes.c_void_p),
        ("table_stride", ctypes.c_int32),
    ]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_D = ctypes.POINTER(AttnDims)
_K = ctypes.POINTER(AttnPagedKV)
_SIG = {
    "attn_decode_dense": [_D, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P],
    "attn_merge_states": [_I, _I, _I, _P, _P, _P, _P, _P, _P, _P],
    "attn_build_centroids": [_D, _P, _P, _P, _P],
    "attn_update_centroids": [_D, _P, _P, _P, _I, _P, _P],
    "attn_score_centroids": [_D, _P, _P, _P, _P, _P],
    "attn_select_topk": [_D, _P, _P, _I, _I, _I, _I, _P, _P, _P],
    "attn_build_super_centroids": [_D, _P, _P, _I, _P, _P],
    "attn_select_two_level": [_D, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P],
    "attn_decode_sparse": [_D, _P, _P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _P],
    "attn_decode_art": [_D, _P, _P, _P, _P, _P, _F, _F, _I, _I, _P, _P, _P, _P],
    "attn_decode_art_ws": [_D, _P, _P, _P, _P, _P, _F, _F, _I, _I, _P, ctypes.c_size_t, _P, _P, _P, _P],
    "attn_art_workspace_bytes": [_D],
    "attn_decode_art_list_ws": [_D, _P, _P, _P, _P, _P, _P, _I, _F, _F, _I, _I, _P, ctypes.c_size_t, _P, _P, _P, _P],
    "attn_decode_art_paged_ws": [_D, _P, _K, _P, _P, _F, _F, _I, _I, _P, ctypes.c_size_t, _P, _P, _P, _P],
    "attn_decode_art_list": [_D, _P, _P, _P, _P, _P, _P, _I, _F, _F, _I, _I, _P, _P, _P, _P],
    "attn_order_blocks": [_D, _P, _P, _P, _P],
    "attn_decode_dense_paged": [_D, _P, _K, _P, _I, _I, _I, _P, _P, _P, _P],
    "attn_decode_sparse_paged": [_D, _P, _K, _P, _P, _P, _I, _I, _P, _P, _P, _P],
    "attn_build_centroids_paged": [_D, _K, _P, _P, _P],
    "attn_update_centroids_paged": [_D, _K, _P, _P, _I, _P, _P],
    "attn_decode_art_paged": [_D, _P, _K, _P, _P, _F, _F, _I, _I, _P, _P, _P, _P],
    "attn_decode_routed": [_D, _I, _P, _P, _P, _P, _P, _I, _I, _P, _P, _I, _I, _P, ctypes.c_size_t, _P, _P],
    "attn_routed_workspace_bytes": [_D, _I, _I, _I],
    "attn_decode_routed_static": [_D, _I, _P, _P, _P, _P, _P, _I, _I, _P, _P, _I, _I, _P, _P],
}
ROUTED_STATIC_BYTES = 8 << 20  # ATTN_ROUTED_STATIC_BYTES
_lib = None


def lib():
    """The loaded ctypes library; raises ImportError if it was never built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m sparse_kv_amd.build` (needs hipcc)")
        h = ctypes.CDLL(LIB_PATH)
        for name, args in _SIG.items():
            fn = getattr(h, name)
            fn.argtypes = args
            fn.restype = ctypes.c_size_t if name.endswith("_workspace_bytes") else ctypes.c_int
        h.attn_status_string.argtypes = [ctypes.c_int]
        h.attn_status_string.restype = ctypes.c_char_p
        _lib = h
    return _lib


def attn_status_string(status: int) -> str:
    return lib().attn_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status == ATTN_OK:
        return
    msg = f"{what}: {attn_status_string(status)} (status {status})"
    if status in (ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE):
        raise ValueError(msg)
    raise RuntimeError(msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class _on_device:
    """Make `dev` current for the duration of a call (cheap when it already is)."""

    __slots__ = ("dev", "prev")

    def __init__(self, dev):
        self.dev = dev
        self.prev = None

    def __enter__(self):
        cur = torch.cuda.current_device()
        if cur != self.dev.index:
            self.prev = cur
            torch.cuda.set_device(self.dev)

    def __exit__(self, *exc):
        if self.prev is not None:
            torch.cuda.set_device(self.prev)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise ValueError(f"unsupported dtype {t.dtype}: q, k, v must be bfloat16 or float32")


def _norm_dev(device):
    d = torch.device(device)
    if d.type == "cuda" and d.index is None:
        d = torch.device("cuda", torch.cuda.current_device())
    return d


def _need(t, name, device, dtype=None, shape=None):
    device = _norm_dev(device)
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _dims_from(q, k, scale=None):
    if q.dim() != 3 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, d] and k, v [B, Hkv, Lmax, d]")
    B, Hq, d = q.shape
    Bk, Hkv, Lmax, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} disagree")
    if Lmax % BLOCK != 0:
        raise ValueError(f"KV length {Lmax} must be a multiple of the block size {BLOCK}")
    if q.dtype != k.dtype:
        raise ValueError("q, k, v must share one dtype")
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    return AttnDims(B, Hq, Hkv, d, BLOCK, Lmax // BLOCK, _dtype_code(k), s)


def _out(t, shape, dtype, device, name):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    return _need(t, name, device, dtype, shape)


def _seq(seq_lens, B, device):
    if seq_lens is None:
        return None
    return _need(seq_lens, "seq_lens", device, torch.int32, (B,))


def attn_decode_dense(q, k, v, seq_lens=None, num_splits=16, block_begin=0, block_end=-1,
                      scale=None, m=None, l=None, o=None):
    """Per-split softmax states (m, l, o) of decode attention over a block range."""
    dev = q.device
    dims = _dims_from(q, k, scale)
    _need(q, "q", dev)
    _need(k, "k", dev)
    _need(v, "v", dev, k.dtype, k.shape)
    seq = _seq(seq_lens, dims.batch, dev)
    rows = (dims.batch, dims.num_q_heads, int(num_splits))
    m = _out(m, rows, torch.float32, dev, "m")
    l = _out(l, rows, torch.float32, dev, "l")
    o = _out(o, rows + (dims.head_dim,), torch.float32, dev, "o")
    with _on_device(dev):
        st = lib().attn_decode_dense(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(seq),
                                    int(block_begin), int(block_end), int(num_splits),
                                    _ptr(m), _ptr(l), _ptr(o), _stream(dev))
    _check(st, "attn_decode_dense")
    return m, l, o


def attn_merge_states(m, l, o, out=None, m_out=None, l_out=None):
    """Merge the last split axis: m, l [..., S], o [..., S, d] -> out [..., d].

    Returns out, or (out, m_out, l_out) when m_out / l_out are requested by
    passing tensors or True.
    """
    dev = o.device
    S, d = o.shape[-2], o.shape[-1]
    lead = tuple(o.shape[:-2])
    _need(o, "o", dev, torch.float32)
    _need(m, "m", dev, torch.float32, lead + (S,))
    _need(l, "l", dev, torch.float32, lead + (S,))
    rows = int(math.prod(lead))
    want_state = m_out is not None or l_out is not None
    out = _out(out, lead + (d,), torch.float32, dev, "out")
    if m_out is True or (want_state and m_out is None):
        m_out = torch.empty(lead, dtype=torch.float32, device=dev)
    if l_out is True or (want_state and l_out is None):
        l_out = torch.empty(lead, dtype=torch.float32, device=dev)
    if want_state:
        _need(m_out, "m_out", dev, torch.float32, lead)
        _need(l_out, "l_out", dev, torch.float32, lead)
    with _on_device(dev):
        st = lib().attn_merge_states(rows, S, d, _ptr(m), _ptr(l), _ptr(o), _ptr(out),
                                    _ptr(m_out) if want_state else None,
                                    _ptr(l_out) if want_state else None, _stream(dev))
    _check(st, "attn_merge_states")
    return (out, m_out, l_out) if want_state else out


def attn_build_centroids(k, seq_lens=None, out=None, num_q_heads=None):
    """Block-mean centroids [B, Hkv, NBmax, d] float32."""
    dev = k.device
    _need(k, "k", dev)
    B, Hkv, Lmax, d = k.shape
    if Lmax % BLOCK:
        raise ValueError(f"KV length {Lmax} must be a multiple of {BLOCK}")
    dims = AttnDims(B, num_q_heads or Hkv, Hkv, d, BLOCK, Lmax // BLOCK, _dtype_code(k), 1.0)
    seq = _seq(seq_lens, B, dev)
    out = _out(out, (B, Hkv, Lmax // BLOCK, d), torch.float32, dev, "out")
    with _on_device(dev):
        st = lib().attn_build_centroids(ctypes.byref(dims), _ptr(k), _ptr(seq), _ptr(out), _stream(dev))
    _check(st, "attn_build_centroids")
    return out


def attn_update_centroids(k, centroids, seq_lens=None, prev_lens=None, span_hint=1):
    """Refresh centroids [B, Hkv, NBmax, d] in place after tokens were appended (see the C header)."""
    dev = k.device
    _need(k, "k", dev)
    B, Hkv, Lmax, d = k.shape
    if Lmax % BLOCK:
        raise ValueError(f"KV length {Lmax} must be a multiple of {BLOCK}")
    _need(centroids, "centroids", dev, torch.float32, (B, Hkv, Lmax // BLOCK, d))
    dims = AttnDims(B, Hkv, Hkv, d, BLOCK, Lmax // BLOCK, _dtype_code(k), 1.0)
    seq = _seq(seq_lens, B, dev)
    prev = None if prev_lens is None else _need(prev_lens, "prev_lens", dev, torch.int32, (B,))
    with _on_device(dev):
        st = lib().attn_update_centroids(ctypes.byref(dims), _ptr(k), _ptr(seq), _ptr(prev), int(span_hint),
                                        _ptr(centroids), _stream(dev))
    _check(st, "attn_update_centroids")
    return centroids


def attn_score_centroids(q, centroids, seq_lens=None, scale=None, out=None):
    """Group scores [B, Hkv, NBmax] float32 (-inf past each sequence's end)."""
    dev = q.device
    _need(q, "q", dev)
    _need(centroids, "centroids", dev, torch.float32)
    B, Hq, d = q.shape
    Bc, Hkv, NBmax, dc = centroids.shape
    if Bc != B or dc != d:
        raise ValueError("q and centroids disagree")
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dims = AttnDims(B, Hq, Hkv, d, BLOCK, NBmax, _dtype_code(q), s)
    seq = _seq(seq_lens, B, dev)
    out = _out(out, (B, Hkv, NBmax), torch.float32, dev, "out")
    with _on_device(dev):
        st = lib().attn_score_centroids(ctypes.byref(dims), _ptr(q), _ptr(centroids), _ptr(seq),
                                       _ptr(out), _stream(dev))
    _check(st, "attn_score_centroids")
    return out


def attn_select_topk(scores, seq_lens=None, k=0, n_sink_blocks=1, n_recent_blocks=0, max_sel=None,
                     block_idx=None, n_sel=None, shape=None, device=None):
    """Chosen blocks (ascending, -1 padded) [B, Hkv, max_sel] and counts [B, Hkv].

    scores [B, Hkv, NBmax] float32, or None with k == 0 and shape=(B, Hkv, NBmax).
    """
    if scores is not None:
        dev = scores.device
        _need(scores, "scores", dev, torch.float32)
        B, Hkv, NBmax = scores.shape
    else:
        if k != 0 or shape is None:
            raise ValueError("scores may only be omitted with k == 0 and an explicit shape")
        B, Hkv, NBmax = shape
        dev = _norm_dev(device) if device is not None else seq_lens.device
    if max_sel is None:
        max_sel = max(1, min(NBmax, int(n_sink_blocks) + int(n_recent_blocks) + int(k)))
    dims = AttnDims(B, Hkv, Hkv, 64, BLOCK, NBmax, ATTN_F32, 1.0)
    seq = _seq(seq_lens, B, dev)
    block_idx = _out(block_idx, (B, Hkv, max_sel), torch.int32, dev, "block_idx")
    n_sel = _out(n_sel, (B, Hkv), torch.int32, dev, "n_sel")
    with _on_device(dev):
        st = lib().attn_select_topk(ctypes.byref(dims), _ptr(scores), _ptr(seq), int(k), int(n_sink_blocks),
                                   int(n_recent_blocks), int(max_sel), _ptr(block_idx), _ptr(n_sel),
                                   _stream(dev))
    _check(st, "attn_select_topk")
    return block_idx, n_sel


def attn_build_super_centroids(centroids, group, seq_lens=None, out=None):
    """Super-block centroids [B, Hkv, ceil(NBmax / group), d] from block centroids."""
    dev = centroids.device
    _need(centroids, "centroids", dev, torch.float32)
    if centroids.dim() != 4:
        raise ValueError("centroids must be [B, Hkv, NBmax, d]")
    B, Hkv, NBmax, d = centroids.shape
    group = int(group)
    if group < 1:
        raise ValueError("group must be >= 1")
    dims = AttnDims(B, Hkv, Hkv, d, BLOCK, NBmax, ATTN_F32, 1.0)
    seq = _seq(seq_lens, B, dev)
    out = _out(out, (B, Hkv, -(-NBmax // group), d), torch.float32, dev, "out")
    with _on_device(dev):
        st = lib().attn_build_super_centroids(ctypes.byref(dims), _ptr(centroids), _ptr(seq), group, _ptr(out),
                                             _stream(dev))
    _check(st, "attn_build_super_centroids")
    return out


def attn_select_two_level(q, centroids, super_centroids, group, seq_lens=None, k_coarse=16, k=0,
                          n_sink_blocks=1, n_recent_blocks=0, max_sel=None, scale=None, block_idx=None,
                          n_sel=None):
    """Two-level selection: (block_idx [B, Hkv, max_sel] ascending, -1 padded; n_sel [B, Hkv])."""
    dev = q.device
    _need(q, "q", dev)
    _need(centroids, "centroids", dev, torch.float32)
    B, Hq, d = q.shape
    Bc, Hkv, NBmax, dc = centroids.shape
    if Bc != B or dc != d:
        raise ValueError("q and centroids disagree")
    _need(super_centroids, "super_centroids", dev, torch.float32, (B, Hkv, -(-NBmax // int(group)), d))
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if max_sel is None:
        max_sel = max(1, min(NBmax, int(n_sink_blocks) + int(n_recent_blocks) + int(k)))
    dims = AttnDims(B, Hq, Hkv, d, BLOCK, NBmax, _dtype_code(q), s)
    seq = _seq(seq_lens, B, dev)
    block_idx = _out(block_idx, (B, Hkv, max_sel), torch.int32, dev, "block_idx")
    n_sel = _out(n_sel, (B, Hkv), torch.int32, dev, "n_sel")
    with _on_device(dev):
        st = lib().attn_select_two_level(ctypes.byref(dims), _ptr(q), _ptr(centroids), _ptr(super_centroids),
                                        _ptr(seq), int(group), int(k_coarse), int(k), int(n_sink_blocks),
                                        int(n_recent_blocks), int(max_sel), _ptr(block_idx), _ptr(n_sel),
                                        _stream(dev))
    _check(st, "attn_select_two_level")
    return block_idx, n_sel


def attn_decode_sparse(q, k, v, block_idx, n_sel, seq_lens=None, num_splits=4, scale=None,
                       m=None, l=None, o=None):
    """Per-split states of attention over the listed blocks only."""
    dev = q.device
    dims = _dims_from(q, k, scale)
    _need(q, "q", dev)
    _need(k, "k", dev)
    _need(v, "v", dev, k.dtype, k.shape)
    _need(block_idx, "block_idx", dev, torch.int32)
    if block_idx.dim() != 3 or tuple(block_idx.shape[:2]) != (dims.batch, dims.num_kv_heads):
        raise ValueError("block_idx must be [B, Hkv, max_sel]")
    _need(n_sel, "n_sel", dev, torch.int32, (dims.batch, dims.num_kv_heads))
    seq = _seq(seq_lens, dims.batch, dev)
    rows = (dims.batch, dims.num_q_heads, int(num_splits))
    m = _out(m, rows, torch.float32, dev, "m")
    l = _out(l, rows, torch.float32, dev, "l")
    o = _out(o, rows + (dims.head_dim,), torch.float32, dev, "o")
    with _on_device(dev):
        st = lib().attn_decode_sparse(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(seq),
                                     _ptr(block_idx), _ptr(n_sel), int(block_idx.shape[2]),
                                     int(num_splits), _ptr(m), _ptr(l), _ptr(o), _stream(dev))
    _check(st, "attn_decode_sparse")
    return m, l, o


def attn_decode_art(q, k, v, seq_lens=None, order=None, tau=1e-3, phi=1e-4, patience=2, probe_dim=8,
                    scale=None, out=None, stop_pos=None, blocks_fetched=None):
    """ART decode: (out [B, Hq, d] float32, stop_pos [B, Hq], blocks_fetched [B, Hkv])."""
    dev = q.device
    dims = _dims_from(q, k, scale)
    _need(q, "q", dev)
    _need(k, "k", dev)
    _need(v, "v", dev, k.dtype, k.shape)
    seq = _seq(seq_lens, dims.batch, dev)
    if order is not None:
        _need(order, "order", dev, torch.int32, (dims.batch, dims.num_kv_heads, dims.max_blocks))
    out = _out(out, (dims.batch, dims.num_q_heads, dims.head_dim), torch.float32, dev, "out")
    stop_pos = _out(stop_pos, (dims.batch, dims.num_q_heads), torch.int32, dev, "stop_pos")
    blocks_fetched = _out(blocks_fetched, (dims.batch, dims.num_kv_heads), torch.int32, dev, "blocks_fetched")
    with _on_device(dev):
        st = lib().attn_decode_art(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(seq), _ptr(order),
                                  float(tau), float(phi), int(patience), int(probe_dim), _ptr(out),
                                  _ptr(stop_pos), _ptr(blocks_fetched), _stream(dev))
    _check(st, "attn_decode_art")
    return out, stop_pos, blocks_fetched


def _art_workspace(dims, workspace, dev):
    """(workspace, bytes) for the ART calls across workgroups; allocated when None and needed."""
    need = int(lib().attn_art_workspace_bytes(ctypes.byref(dims)))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _need(workspace, "workspace", dev)
    return workspace, (workspace.numel() * workspace.element_size() if workspace is not None else 0)


def attn_art_workspace_bytes(q, k, scale=None):
    """Bytes of workspace attn_decode_art_ws uses for these shapes (0: none)."""
    dims = _dims_from(q, k, scale)
    return int(lib().attn_art_workspace_bytes(ctypes.byref(dims)))


def attn_decode_art_ws(q, k, v, seq_lens=None, order=None, tau=1e-3, phi=1e-4, patience=2, probe_dim=8,
                       scale=None, workspace=None, out=None, stop_pos=None, blocks_fetched=None):
    """attn_decode_art that may spread each (b, kv head) over several CUs through
    `workspace` (uint8 device tensor of attn_art_workspace_bytes; allocated if None)."""
    dev = q.device
    dims = _dims_from(q, k, scale)
    _need(q, "q", dev)
    _need(k, "k", dev)
    _need(v, "v", dev, k.dtype, k.shape)
    seq = _seq(seq_lens, dims.batch, dev)
    if order is not None:
        _need(order, "order", dev, torch.int32, (dims.batch, dims.num_kv_heads, dims.max_blocks))
    workspace, ws_bytes = _art_workspace(dims, workspace, dev)
    out = _out(out, (dims.batch, dims.num_q_heads, dims.head_dim), torch.float32, dev, "out")
    stop_pos = _out(stop_pos, (dims.batch, dims.num_q_heads), torch.int32, dev, "stop_pos")
    blocks_fetched = _out(blocks_fetched, (dims.batch, dims.num_kv_heads), torch.int32, dev, "blocks_fetched")
    with _on_device(dev):
        st = lib().attn_decode_art_ws(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(seq), _ptr(order),
                                     float(tau), float(phi), int(patience), int(probe_dim), _ptr(workspace),
                                     ws_bytes, _ptr(out), _ptr(stop_pos), _ptr(blocks_fetched), _stream(dev))
    _check(st, "attn_decode_art_ws")
    return out, stop_pos, blocks_fetched


def attn_decode_art_list(q, k, v, block_list, n_list, seq_lens=None, tau=1e-3, phi=1e-4, patience=2,
                         probe_dim=8, scale=None, out=None, stop_pos=None, blocks_fetched=None):
    """ART over listed blocks, visited in list order: same outputs as attn_decode_art."""
    dev = q.device
    dims = _dims_from(q, k, scale)
    _need(q, "q", dev)
    _need(k, "k", dev)
    _need(v, "v", dev, k.dtype, k.shape)
    _need(block_list, "block_list", dev, torch.int32)
    if block_list.dim() != 3 or tuple(block_list.shape[:2]) != (dims.batch, dims.num_kv_heads):
        raise ValueError("block_list must be [B, Hkv, max_list]")
    _need(n_list, "n_list", dev, torch.int32, (dims.batch, dims.num_kv_heads))
    seq = _seq(seq_lens, dims.batch, dev)
    out = _out(out, (dims.batch, dims.num_q_heads, dims.head_dim), torch.float32, dev, "out")
    stop_pos = _out(stop_pos, (dims.batch, dims.num_q_heads), torch.int32, dev, "stop_pos")
    blocks_fetched = _out(blocks_fetched, (dims.batch, dims.num_kv_heads), torch.int32, dev, "blocks_fetched")
    with _on_device(dev):
        st = lib().attn_decode_art_list(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(seq),
                                       _ptr(block_list), _ptr(n_list), int(block_list.shape[2]),
                                       float(tau), float(phi), int(patience), int(probe_dim), _ptr(out),
                                       _ptr(stop_pos), _ptr(blocks_fetched), _stream(dev))
    _check(st, "attn_decode_art_list")
    return out, stop_pos, blocks_fetched


def attn_decode_art_list_ws(q, k, v, block_list, n_list, seq_lens=None, tau=1e-3, phi=1e-4, patience=2,
                            probe_dim=8, scale=None, workspace=None, out=None, stop_pos=None, blocks_fetched=None):
    """attn_decode_art_list that may spread each (b, kv head) over several CUs through `workspace`."""
    dev = q.device
    dims = _dims_from(q, k, scale)
    _need(q, "q", dev)
    _need(k, "k", dev)
    _need(v, "v", dev, k.dtype, k.shape)
    _need(block_list, "block_list", dev, torch.int32)
    if block_list.dim() != 3 or tuple(block_list.shape[:2]) != (dims.batch, dims.num_kv_heads):
        raise ValueError("block_list must be [B, Hkv, max_list]")
    _need(n_list, "n_list", dev, torch.int32, (dims.batch, dims.num_kv_heads))
    seq = _seq(seq_lens, dims.batch, dev)
    workspace, ws_bytes = _art_workspace(dims, workspace, dev)
    out = _out(out, (dims.batch, dims.num_q_heads, dims.head_dim), torch.float32, dev, "out")
    stop_pos = _out(stop_pos, (dims.batch, dims.num_q_heads), torch.int32, dev, "stop_pos")
    blocks_fetched = _out(blocks_fetched, (dims.batch, dims.num_kv_heads), torch.int32, dev, "blocks_fetched")
    with _on_device(dev):
        st = lib().attn_decode_art_list_ws(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(seq),
                                          _ptr(block_list), _ptr(n_list), int(block_list.shape[2]),
                                          float(tau), float(phi), int(patience), int(probe_dim), _ptr(workspace),
                                          ws_bytes, _ptr(out), _ptr(stop_pos), _ptr(blocks_fetched), _stream(dev))
    _check(st, "attn_decode_art_list_ws")
    return out, stop_pos, blocks_fetched


def attn_order_blocks(scores, seq_lens=None, out=None):
    """Importance-first visit order [B, Hkv, NBmax] int32 from block scores [B, Hkv, NBmax]."""
    dev = scores.device
    _need(scores, "scores", dev, torch.float32)
    if scores.dim() != 3:
        raise ValueError("scores must be [B, Hkv, NBmax]")
    B, Hkv, NBmax = scores.shape
    dims = AttnDims(B, Hkv, Hkv, 64, BLOCK, NBmax, ATTN_F32, 1.0)
    seq = _seq(seq_lens, B, dev)
    out = _out(out, (B, Hkv, NBmax), torch.int32, dev, "out")
    with _on_device(dev):
        st = lib().attn_order_blocks(ctypes.byref(dims), _ptr(scores), _ptr(seq), _ptr(out), _stream(dev))
    _check(st, "attn_order_blocks")
    return out


def attn_routed_workspace_bytes(q, k, n_shards=8, splits_per_shard=4, sa_splits=4, scale=None):
    dims = _dims_from(q, k, scale)
    return int(lib().attn_routed_workspace_bytes(ctypes.byref(dims), int(n_shards), int(splits_per_shard),
                                                int(sa_splits)))


def _routed_args(qs, ks, vs, route_mask, seq_lens, outs, scale):
    """Checked (dims, device, seq, outs, C arrays) shared by the routed entry points."""
    n = len(qs)
    if not (len(ks) == len(vs) == len(route_mask) == n):
        raise ValueError("qs, ks, vs and route_mask must have one entry per layer")
    dev = qs[0].device
    dims = _dims_from(qs[0], ks[0], scale)
    for i in range(n):
        _need(qs[i], f"qs[{i}]", dev, qs[0].dtype, qs[0].shape)
        _need(ks[i], f"ks[{i}]", dev, ks[0].dtype, ks[0].shape)
        _need(vs[i], f"vs[{i}]", dev, ks[0].dtype, ks[0].shape)
    seq = _seq(seq_lens, dims.batch, dev)
    if outs is None:
        outs = [torch.empty((dims.batch, dims.num_q_heads, dims.head_dim), dtype=torch.float32, device=dev)
                for _ in range(n)]
    if len(outs) != n:
        raise ValueError("outs must have one entry per layer")
    for i, t in enumerate(outs):
        _need(t, f"outs[{i}]", dev, torch.float32, (dims.batch, dims.num_q_heads, dims.head_dim))
    mask = (ctypes.c_uint8 * n)(*[1 if int(x) else 0 for x in route_mask])
    arr = ctypes.c_void_p * n
    ptrs = [ctypes.cast(a, _P) for a in (arr(*[t.data_ptr() for t in qs]), arr(*[t.data_ptr() for t in ks]),
                                           arr(*[t.data_ptr() for t in vs]), arr(*[t.data_ptr() for t in outs]))]
    return dims, dev, seq, outs, ctypes.cast(mask, _P), ptrs, (mask,)


def attn_decode_routed(qs, ks, vs, route_mask, seq_lens=None, n_shards=8, splits_per_shard=4,
                       sa_block_idx=None, sa_n_sel=None, sa_splits=4, workspace=None, outs=None,
                       scale=None):
    """One decode step of a layer stack under a per-layer hard route mask.

    qs, ks, vs: per-layer tensors of one shape; route_mask: sequence of 0/1
    (1 = full attention).  Returns the list of per-layer outputs [B, Hq, d].
    """
    if len(qs) == 0:
        return []
    dims, dev, seq, outs, mask, (qa, ka, va, oa), keep = _routed_args(qs, ks, vs, route_mask, seq_lens, outs, scale)
    need = int(lib().attn_routed_workspace_bytes(ctypes.byref(dims), int(n_shards), int(splits_per_shard),
                                                int(sa_splits)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", dev)
    max_sel = int(sa_block_idx.shape[-1]) if sa_block_idx is not None else 0
    with _on_device(dev):
        st = lib().attn_decode_routed(ctypes.byref(dims), len(qs), mask, qa, ka, va, _ptr(seq), int(n_shards),
                                     int(splits_per_shard), _ptr(sa_block_idx), _ptr(sa_n_sel), max_sel,
                                     int(sa_splits), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), oa, _stream(dev))
    _check(st, "attn_decode_routed")
    return outs


def attn_decode_routed_static(qs, ks, vs, route_mask, seq_lens=None, n_shards=8, splits_per_shard=4,
                              sa_block_idx=None, sa_n_sel=None, sa_splits=4, outs=None, scale=None):
    """attn_decode_routed without a workspace: the library's own static device scratch
    (ROUTED_STATIC_BYTES per device) holds the states; the C call allocates nothing
    (pass `outs` to allocate nothing here either).  Overlapping calls on one device race."""
    if len(qs) == 0:
        return []
    dims, dev, seq, outs, mask, (qa, ka, va, oa), keep = _routed_args(qs, ks, vs, route_mask, seq_lens, outs, scale)
    max_sel = int(sa_block_idx.shape[-1]) if sa_block_idx is not None else 0
    with _on_device(dev):
        st = lib().attn_decode_routed_static(ctypes.byref(dims), len(qs), mask, qa, ka, va, _ptr(seq),
                                            int(n_shards), int(splits_per_shard), _ptr(sa_block_idx),
                                            _ptr(sa_n_sel), max_sel, int(sa_splits), oa, _stream(dev))
    _check(st, "attn_decode_routed_static")
    return outs


# ---- paged cache ----------------------------------------------------------

def _paged(k_pool, v_pool, block_table, device):
    """(AttnPagedKV, Hkv, NBmax, d, dtype code) from pools [P, Hkv, 64, d] and a table [B, NBmax]."""
    _need(k_pool, "k_pool", device)
    if k_pool.dim() != 4 or k_pool.shape[2] != BLOCK:
        raise ValueError(f"k_pool must be [pool_blocks, Hkv, {BLOCK}, d]")
    if v_pool is not None:
        _need(v_pool, "v_pool", device, k_pool.dtype, k_pool.shape)
    _need(block_table, "block_table", device, torch.int32)
    if block_table.dim() != 2:
        raise ValueError("block_table must be [B, max_blocks]")
    P, Hkv, _, d = k_pool.shape
    kv = AttnPagedKV(k_pool.data_ptr(), None if v_pool is None else v_pool.data_ptr(), P, block_table.data_ptr(),
                     block_table.shape[1])
    return kv, Hkv, block_table.shape[1], d, _dtype_code(k_pool)


def _paged_dims(q, k_pool, v_pool, block_table, scale):
    dev = q.device
    _need(q, "q", dev)
    kv, Hkv, NBmax, d, code = _paged(k_pool, v_pool, block_table, dev)
    if q.dim() != 3 or q.shape[2] != d or q.shape[0] != block_table.shape[0]:
        raise ValueError("q must be [B, Hq, d] with B = block_table rows")
    if q.dtype != k_pool.dtype:
        raise ValueError("q and the pools must share one dtype")
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    return AttnDims(q.shape[0], q.shape[1], Hkv, d, BLOCK, NBmax, code, s), kv


def attn_decode_dense_paged(q, k_pool, v_pool, block_table, seq_lens=None, num_splits=16, block_begin=0,
                            block_end=-1, scale=None, m=None, l=None, o=None):
    """attn_decode_dense over a paged cache: per-split states (m, l, o)."""
    dev = q.device
    dims, kv = _paged_dims(q, k_pool, v_pool, block_table, scale)
    seq = _seq(seq_lens, dims.batch, dev)
    rows = (dims.batch, dims.num_q_heads, int(num_splits))
    m = _out(m, rows, torch.float32, dev, "m")
    l = _out(l, rows, torch.float32, dev, "l")
    o = _out(o, rows + (dims.head_dim,), torch.float32, dev, "o")
    with _on_device(dev):
        st = lib().attn_decode_dense_paged(ctypes.byref(dims), _ptr(q), ctypes.byref(kv), _ptr(seq),
                                          int(block_begin), int(block_end), int(num_splits), _ptr(m), _ptr(l),
                                          _ptr(o), _stream(dev))
    _check(st, "attn_decode_dense_paged")
    return m, l, o


def attn_decode_sparse_paged(q, k_pool, v_pool, block_table, block_idx, n_sel, seq_lens=None, num_splits=4,
                             scale=None, m=None, l=None, o=None):
    """attn_decode_sparse over a paged cache: per-split states over the listed blocks."""
    dev = q.device
    dims, kv = _paged_dims(q, k_pool, v_pool, block_table, scale)
    _need(block_idx, "block_idx", dev, torch.int32)
    if block_idx.dim() != 3 or tuple(block_idx.shape[:2]) != (dims.batch, dims.num_kv_heads):
        raise ValueError("block_idx must be [B, Hkv, max_sel]")
    _need(n_sel, "n_sel", dev, torch.int32, (dims.batch, dims.num_kv_heads))
    seq = _seq(seq_lens, dims.batch, dev)
    rows = (dims.batch, dims.num_q_heads, int(num_splits))
    m = _out(m, rows, torch.float32, dev, "m")
    l = _out(l, rows, torch.float32, dev, "l")
    o = _out(o, rows + (dims.head_dim,), torch.float32, dev, "o")
    with _on_device(dev):
        st = lib().attn_decode_sparse_paged(ctypes.byref(dims), _ptr(q), ctypes.byref(kv), _ptr(seq),
                                           _ptr(block_idx), _ptr(n_sel), int(block_idx.shape[2]), int(num_splits),
                                           _ptr(m), _ptr(l), _ptr(o), _stream(dev))
    _check(st, "attn_decode_sparse_paged")
    return m, l, o


def attn_build_centroids_paged(k_pool, block_table, seq_lens=None, out=None):
    """Block centroids [B, Hkv, NBmax, d] of a paged cache."""
    dev = k_pool.device
    kv, Hkv, NBmax, d, code = _paged(k_pool, None, block_table, dev)
    B = block_table.shape[0]
    dims = AttnDims(B, Hkv, Hkv, d, BLOCK, NBmax, code, 1.0)
    seq = _seq(seq_lens, B, dev)
    out = _out(out, (B, Hkv, NBmax, d), torch.float32, dev, "out")
    with _on_device(dev):
        st = lib().attn_build_centroids_paged(ctypes.byref(dims), ctypes.byref(kv), _ptr(seq), _ptr(out),
                                             _stream(dev))
    _check(st, "attn_build_centroids_paged")
    return out


def attn_update_centroids_paged(k_pool, block_table, centroids, seq_lens=None, prev_lens=None, span_hint=1):
    """attn_update_centroids over a paged cache (centroids updated in place)."""
    dev = k_pool.device
    kv, Hkv, NBmax, d, code = _paged(k_pool, None, block_table, dev)
    B = block_table.shape[0]
    _need(centroids, "centroids", dev, torch.float32, (B, Hkv, NBmax, d))
    dims = AttnDims(B, Hkv, Hkv, d, BLOCK, NBmax, code, 1.0)
    seq = _seq(seq_lens, B, dev)
    prev = None if prev_lens is None else _need(prev_lens, "prev_lens", dev, torch.int32, (B,))
    with _on_device(dev):
        st = lib().attn_update_centroids_paged(ctypes.byref(dims), ctypes.byref(kv), _ptr(seq), _ptr(prev),
                                              int(span_hint), _ptr(centroids), _stream(dev))
    _check(st, "attn_update_centroids_paged")
    return centroids


def attn_decode_art_paged(q, k_pool, v_pool, block_table, seq_lens=None, order=None, tau=1e-3, phi=1e-4,
                          patience=2, probe_dim=8, scale=None, out=None, stop_pos=None, blocks_fetched=None):
    """attn_decode_art over a paged cache: (out, stop_pos, blocks_fetched)."""
    dev = q.device
    dims, kv = _paged_dims(q, k_pool, v_pool, block_table, scale)
    seq = _seq(seq_lens, dims.batch, dev)
    if order is not None:
        _need(order, "order", dev, torch.int32, (dims.batch, dims.num_kv_heads, dims.max_blocks))
    out = _out(out, (dims.batch, dims.num_q_heads, dims.head_dim), torch.float32, dev, "out")
    stop_pos = _out(stop_pos, (dims.batch, dims.num_q_heads), torch.int32, dev, "stop_pos")
    blocks_fetched = _out(blocks_fetched, (dims.batch, dims.num_kv_heads), torch.int32, dev, "blocks_fetched")
    with _on_device(dev):
        st = lib().attn_decode_art_paged(ctypes.byref(dims), _ptr(q), ctypes.byref(kv), _ptr(seq), _ptr(order),
                                        float(tau), float(phi), int(patience), int(probe_dim), _ptr(out),
                                        _ptr(stop_pos), _ptr(blocks_fetched), _stream(dev))
    _check(st, "attn_decode_art_paged")
    return out, stop_pos, blocks_fetched


def attn_decode_art_paged_ws(q, k_pool, v_pool, block_table, seq_lens=None, order=None, tau=1e-3, phi=1e-4,
                             patience=2, probe_dim=8, scale=None, workspace=None, out=None, stop_pos=None,
                             blocks_fetched=None):
    """attn_decode_art_paged that may spread each (b, kv head) over several CUs through `workspace`."""
    dev = q.device
    dims, kv = _paged_dims(q, k_pool, v_pool, block_table, scale)
    seq = _seq(seq_lens, dims.batch, dev)
    if order is not None:
        _need(order, "order", dev, torch.int32, (dims.batch, dims.num_kv_heads, dims.max_blocks))
    workspace, ws_bytes = _art_workspace(dims, workspace, dev)
    out = _out(out, (dims.batch, dims.num_q_heads, dims.head_dim), torch.float32, dev, "out")
    stop_pos = _out(stop_pos, (dims.batch, dims.num_q_heads), torch.int32, dev, "stop_pos")
    blocks_fetched = _out(blocks_fetched, (dims.batch, dims.num_kv_heads), torch.int32, dev, "blocks_fetched")
    with _on_device(dev):
        st = lib().attn_decode_art_paged_ws(ctypes.byref(dims), _ptr(q), ctypes.byref(kv), _ptr(seq),
                                           _ptr(order), float(tau), float(phi), int(patience), int(probe_dim),
                                           _ptr(workspace), ws_bytes, _ptr(out), _ptr(stop_pos),
                                           _ptr(blocks_fetched), _stream(dev))
    _check(st, "attn_decode_art_paged_ws")
    return out, stop_pos, blocks_fetched
