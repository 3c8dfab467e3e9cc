"""ctypes binding of libkascade.so (argument marshalling only).

The functions named ``kascade_*`` mirror the C entry points of
``include/kascade.h`` one to one: tensors are passed as device pointers
(``tensor.data_ptr()``), the stream as torch's current HIP stream.  The
small helpers below them (``anchor_decode`` etc.) only allocate outputs and
workspace with torch and call those entry points; every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkascade.so")

KASCADE_F32, KASCADE_BF16, KASCADE_F16 = 0, 1, 2
KASCADE_OK, KASCADE_ERR_NULL, KASCADE_ERR_SHAPE, KASCADE_ERR_DTYPE = 0, -1, -2, -3
KASCADE_ERR_TOPK, KASCADE_ERR_HEADMAP, KASCADE_ERR_WORKSPACE, KASCADE_ERR_HIP = -4, -5, -6, -7
KASCADE_ERR_ARG = -8
OP_ANCHOR_DECODE, OP_REUSE_DECODE, OP_ANCHOR_PREFILL, OP_REUSE_PREFILL = 0, 1, 2, 3
OP_DENSE_DECODE, OP_DENSE_PREFILL, OP_ANCHOR_DECODE_FUSED = 4, 5, 6
K_DECODE_SPLITK, K_DECODE_COMBINE, K_DECODE_POOL, K_TOPK_SELECT = 0, 1, 2, 3
K_REUSE_DECODE, K_PREFILL_FLASH, K_PREFILL_POOL, K_PREFILL_SPARSE = 4, 5, 6, 7
K_ANCHOR_FUSED = 8

EXPORTS = [
    "kascade_anchor_decode", "kascade_reuse_decode", "kascade_anchor_prefill",
    "kascade_reuse_prefill", "kascade_workspace_bytes", "kascade_topk_for_len",
    "kascade_topk_select_f32", "kascade_dense_decode", "kascade_dense_prefill",
    "kascade_kernel_timer_enable", "kascade_kernel_timer_read", "kascade_status_str",
    "kascade_last_hip_error", "kascade_version",
    "kascade_anchor_decode_paged", "kascade_reuse_decode_paged", "kascade_reuse_prefill_paged",
    "kascade_calib_head_similarity", "kascade_layer_weight", "kascade_layer_weight_workspace_bytes",
    "kascade_weighted_similarity", "kascade_select_anchors", "kascade_head_maps",
    "kascade_reuse_decode_noalloc", "kascade_stream_read", "kascade_anchor_decode_fused",
]


class Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("ctx_len", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float), ("reserved", ctypes.c_int32),
        ("q_stride_b", ctypes.c_int64), ("q_stride_h", ctypes.c_int64), ("q_stride_n", ctypes.c_int64),
        ("kv_stride_b", ctypes.c_int64), ("kv_stride_h", ctypes.c_int64), ("kv_stride_n", ctypes.c_int64),
    ]


class PagedKV(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("table_stride", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("block_stride", ctypes.c_int64)]


class TopkRule(ctypes.Structure):
    _fields_ = [("tile", ctypes.c_int32), ("pct", ctypes.c_int32),
                ("round_to", ctypes.c_int32), ("k_min", ctypes.c_int32)]


PREFILL_RULE = TopkRule(128, 10, 64, 256)
# decode k for a context of n keys: 10% of n to the nearest multiple of 64, at least 128
DECODE_RULE = TopkRule(128, 10, 64, 128)


class KascadeError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = _LIB
        msg = lib.kascade_status_str(status).decode() if lib else str(status)
        hip = lib.kascade_last_hip_error() if lib else 0
        super().__init__("%s failed: %s (status %d, hip error %d)" % (where, msg, status, hip))
        self.status = status


_LIB: Optional[ctypes.CDLL] = None
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_SIGS = {
    "kascade_anchor_decode": (_i32, [ctypes.POINTER(Shape), _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kascade_anchor_decode_fused": (_i32, [ctypes.POINTER(Shape), _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp,
                                             ctypes.c_uint32, _vp, _sz, _vp]),
    "kascade_reuse_decode": (_i32, [ctypes.POINTER(Shape), _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kascade_reuse_decode_noalloc": (_i32, [ctypes.POINTER(Shape), _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp]),
    "kascade_anchor_prefill": (_i32, [ctypes.POINTER(Shape), _vp, _vp, _vp, ctypes.POINTER(TopkRule), _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kascade_reuse_prefill": (_i32, [ctypes.POINTER(Shape), _vp, _vp, _vp, ctypes.POINTER(TopkRule), _vp, _vp, _vp, _vp, _sz, _vp]),
    "kascade_workspace_bytes": (_sz, [_i32, ctypes.POINTER(Shape), _i32, ctypes.POINTER(TopkRule)]),
    "kascade_topk_for_len": (_i32, [_i32, ctypes.POINTER(TopkRule)]),
    "kascade_topk_select_f32": (_i32, [_vp, _i64, _i32, _i32, _i32, _vp, _i64, _vp]),
    "kascade_dense_decode": (_i32, [ctypes.POINTER(Shape), _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kascade_dense_prefill": (_i32, [ctypes.POINTER(Shape), _vp, _vp, _vp, _vp, _vp, _vp]),
    "kascade_kernel_timer_enable": (_i32, [_i32, _i32]),
    "kascade_kernel_timer_read": (_i32, [_i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]),
    "kascade_status_str": (ctypes.c_char_p, [_i32]),
    "kascade_last_hip_error": (_i32, []),
    "kascade_version": (ctypes.c_char_p, []),
    "kascade_anchor_decode_paged": (_i32, [ctypes.POINTER(Shape), ctypes.POINTER(PagedKV), _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kascade_reuse_decode_paged": (_i32, [ctypes.POINTER(Shape), ctypes.POINTER(PagedKV), _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kascade_reuse_prefill_paged": (_i32, [ctypes.POINTER(Shape), ctypes.POINTER(PagedKV), _vp, _vp, _vp, ctypes.POINTER(TopkRule), _vp, _vp, _vp, _vp, _sz, _vp]),
    "kascade_calib_head_similarity": (_i32, [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "kascade_layer_weight": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _sz, _vp]),
    "kascade_layer_weight_workspace_bytes": (_sz, [_i32]),
    "kascade_weighted_similarity": (_i32, [_i32, _i32, _vp, _vp, _vp]),
    "kascade_select_anchors": (_i32, [_i32, _i32, _vp, _vp, _vp]),
    "kascade_head_maps": (_i32, [_i32, _i32, _vp, _vp, _i32, _vp]),
    "kascade_stream_read": (_i32, [_vp, _sz, _vp, _vp]),
}


def lib() -> ctypes.CDLL:
    """Load libkascade.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkascade.so is not built (run __graft_entry__.build() or "
                               "python -m long_context_anchor_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


# ---------------------------------------------------------------------------
# raw entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def _p(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream


def kascade_anchor_decode(shape, q, k, v, topk, out, lse_out, topk_idx, pooled_out, workspace,
                          workspace_bytes, stream=None) -> int:
    return lib().kascade_anchor_decode(ctypes.byref(shape), _p(q), _p(k), _p(v), topk, _p(out),
                                       _p(lse_out), _p(topk_idx), _p(pooled_out), _p(workspace),
                                       workspace_bytes, _stream(stream))


def kascade_anchor_decode_fused(shape, q, k, v, topk, out, lse_out, topk_idx, pooled_out, max_polls,
                                workspace, workspace_bytes, stream=None) -> int:
    return lib().kascade_anchor_decode_fused(ctypes.byref(shape), _p(q), _p(k), _p(v), topk, _p(out),
                                             _p(lse_out), _p(topk_idx), _p(pooled_out), max_polls,
                                             _p(workspace), workspace_bytes, _stream(stream))


def kascade_reuse_decode(shape, q, k, v, topk, anchor_topk_idx, head_map, out, workspace,
                         workspace_bytes, stream=None) -> int:
    hm = (ctypes.c_int32 * len(head_map))(*[int(x) for x in head_map]) if head_map is not None else None
    return lib().kascade_reuse_decode(ctypes.byref(shape), _p(q), _p(k), _p(v), topk,
                                      _p(anchor_topk_idx), ctypes.cast(hm, _vp) if hm is not None else None,
                                      _p(out), _p(workspace), workspace_bytes, _stream(stream))


def kascade_reuse_decode_noalloc(shape, q, k, v, topk, anchor_topk_idx, head_map, out, stream=None) -> int:
    hm = (ctypes.c_int32 * len(head_map))(*[int(x) for x in head_map]) if head_map is not None else None
    return lib().kascade_reuse_decode_noalloc(ctypes.byref(shape), _p(q), _p(k), _p(v), topk,
                                              _p(anchor_topk_idx),
                                              ctypes.cast(hm, _vp) if hm is not None else None,
                                              _p(out), _stream(stream))


def kascade_anchor_prefill(shape, q, k, v, rule, out, lse_out, tile_topk_idx, pooled_out,
                           workspace, workspace_bytes, stream=None) -> int:
    return lib().kascade_anchor_prefill(ctypes.byref(shape), _p(q), _p(k), _p(v), ctypes.byref(rule),
                                        _p(out), _p(lse_out), _p(tile_topk_idx), _p(pooled_out),
                                        _p(workspace), workspace_bytes, _stream(stream))


def kascade_reuse_prefill(shape, q, k, v, rule, anchor_tile_topk_idx, head_map, out, workspace,
                          workspace_bytes, stream=None) -> int:
    hm = (ctypes.c_int32 * len(head_map))(*[int(x) for x in head_map]) if head_map is not None else None
    return lib().kascade_reuse_prefill(ctypes.byref(shape), _p(q), _p(k), _p(v), ctypes.byref(rule),
                                       _p(anchor_tile_topk_idx),
                                       ctypes.cast(hm, _vp) if hm is not None else None,
                                       _p(out), _p(workspace), workspace_bytes, _stream(stream))


def kascade_workspace_bytes(op, shape, topk=0, rule=None) -> int:
    return lib().kascade_workspace_bytes(op, ctypes.byref(shape), topk,
                                         ctypes.byref(rule) if rule is not None else None)


def kascade_topk_for_len(n, rule) -> int:
    return lib().kascade_topk_for_len(n, ctypes.byref(rule))


def kascade_stream_read(src, nbytes, sink, stream=None) -> int:
    return lib().kascade_stream_read(_p(src), nbytes, _p(sink), _stream(stream))


def kascade_topk_select_f32(scores, row_stride, rows, n, k, idx, idx_stride, stream=None) -> int:
    return lib().kascade_topk_select_f32(_p(scores), row_stride, rows, n, k, _p(idx), idx_stride,
                                         _stream(stream))


def kascade_dense_decode(shape, q, k, v, out, lse_out, workspace, workspace_bytes, stream=None) -> int:
    return lib().kascade_dense_decode(ctypes.byref(shape), _p(q), _p(k), _p(v), _p(out), _p(lse_out),
                                      _p(workspace), workspace_bytes, _stream(stream))


def kascade_dense_prefill(shape, q, k, v, out, lse_out, stream=None) -> int:
    return lib().kascade_dense_prefill(ctypes.byref(shape), _p(q), _p(k), _p(v), _p(out), _p(lse_out),
                                       _stream(stream))


def kascade_kernel_timer_enable(kernel_id: int, enable: bool) -> int:
    return lib().kascade_kernel_timer_enable(kernel_id, 1 if enable else 0)


def kascade_kernel_timer_read(kernel_id: int):
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    st = lib().kascade_kernel_timer_read(kernel_id, ctypes.byref(ms), ctypes.byref(n))
    if st:
        raise KascadeError(st, "kascade_kernel_timer_read")
    return ms.value, n.value


def kascade_anchor_decode_paged(shape, paged, q, k_cache, v_cache, topk, out, lse_out, topk_idx, pooled_out,
                                workspace, workspace_bytes, stream=None) -> int:
    return lib().kascade_anchor_decode_paged(ctypes.byref(shape), ctypes.byref(paged), _p(q), _p(k_cache),
                                             _p(v_cache), topk, _p(out), _p(lse_out), _p(topk_idx),
                                             _p(pooled_out), _p(workspace), workspace_bytes,
                                             _stream(stream))


def kascade_reuse_decode_paged(shape, paged, q, k_cache, v_cache, topk, anchor_topk_idx, head_map, out,
                               workspace, workspace_bytes, stream=None) -> int:
    hm = (ctypes.c_int32 * len(head_map))(*[int(x) for x in head_map]) if head_map is not None else None
    return lib().kascade_reuse_decode_paged(ctypes.byref(shape), ctypes.byref(paged), _p(q), _p(k_cache),
                                            _p(v_cache), topk, _p(anchor_topk_idx),
                                            ctypes.cast(hm, _vp) if hm is not None else None, _p(out),
                                            _p(workspace), workspace_bytes, _stream(stream))


def kascade_reuse_prefill_paged(shape, paged, q, k_cache, v_cache, rule, anchor_tile_topk_idx, head_map, out,
                                workspace=None, workspace_bytes=0, stream=None) -> int:
    hm = (ctypes.c_int32 * len(head_map))(*[int(x) for x in head_map]) if head_map is not None else None
    return lib().kascade_reuse_prefill_paged(ctypes.byref(shape), ctypes.byref(paged), _p(q), _p(k_cache),
                                             _p(v_cache), ctypes.byref(rule), _p(anchor_tile_topk_idx),
                                             ctypes.cast(hm, _vp) if hm is not None else None, _p(out),
                                             _p(workspace), workspace_bytes, _stream(stream))


def kascade_calib_head_similarity(L, S, n_kv_heads, n, k, pooled, topk_idx, sim, stream=None) -> int:
    return lib().kascade_calib_head_similarity(L, S, n_kv_heads, n, k, _p(pooled), _p(topk_idx), _p(sim),
                                               _stream(stream))


def kascade_layer_weight(x, y, tokens, dim, dtype, w_out, workspace, workspace_bytes, stream=None) -> int:
    return lib().kascade_layer_weight(_p(x), _p(y), tokens, dim, dtype, _p(w_out), _p(workspace),
                                      workspace_bytes, _stream(stream))


def kascade_layer_weight_workspace_bytes(tokens) -> int:
    return lib().kascade_layer_weight_workspace_bytes(tokens)


def _host(a, dtype):
    """A C-contiguous NumPy array of `dtype` and its address (host arguments)."""
    import numpy as np
    arr = np.ascontiguousarray(a, dtype=dtype)
    return arr, arr.ctypes.data


def kascade_weighted_similarity(L, n_kv_heads, sim_host, w_host=None):
    """Host call; returns S [L, L] float64."""
    import numpy as np
    sim, ps = _host(sim_host, np.float32)
    w, pw = _host(w_host, np.float32) if w_host is not None else (None, None)
    S = np.zeros((L, L), dtype=np.float64)
    check(lib().kascade_weighted_similarity(L, n_kv_heads, ps, pw, S.ctypes.data),
          "kascade_weighted_similarity")
    return S


def kascade_select_anchors(L, M, S_host):
    """Host call; returns (anchors list, score)."""
    import numpy as np
    S, ps = _host(S_host, np.float64)
    out = np.zeros(M, dtype=np.int32)
    score = ctypes.c_double(0.0)
    check(lib().kascade_select_anchors(L, M, ps, out.ctypes.data, ctypes.addressof(score)),
          "kascade_select_anchors")
    return [int(x) for x in out], score.value


def kascade_head_maps(L, n_kv_heads, sim_host, anchors):
    """Host call; returns head_maps int32 [L, n_kv_heads]."""
    import numpy as np
    sim, ps = _host(sim_host, np.float32)
    an, pa = _host(anchors, np.int32)
    out = np.zeros((L, n_kv_heads), dtype=np.int32)
    check(lib().kascade_head_maps(L, n_kv_heads, ps, pa, len(an), out.ctypes.data), "kascade_head_maps")
    return out


def kascade_status_str(status: int) -> str:
    return lib().kascade_status_str(status).decode()


def kascade_last_hip_error() -> int:
    return lib().kascade_last_hip_error()


def kascade_version() -> str:
    return lib().kascade_version().decode()


# ---------------------------------------------------------------------------
# shape marshalling and allocating helpers
# ---------------------------------------------------------------------------

def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return KASCADE_F32
    if t.dtype == torch.bfloat16:
        return KASCADE_BF16
    if t.dtype == torch.float16:
        return KASCADE_F16
    raise TypeError("unsupported dtype %s" % t.dtype)


def make_shape(q: torch.Tensor, k: torch.Tensor, ctx_len: int, scale: float = 0.0) -> Shape:
    """Shape from q ([B,Hq,d] decode or [B,Hq,N,d] prefill) and the cache k
    ([B,Hkv,N_cap,d]); strides in elements."""
    if q.dim() == 3:
        qsb, qsh, qsn = q.stride(0), q.stride(1), 0
    else:
        qsb, qsh, qsn = q.stride(0), q.stride(1), q.stride(2)
    if q.stride(-1) != 1 or k.stride(-1) != 1:
        raise ValueError("the head_dim axis must be contiguous")
    return Shape(q.shape[0], q.shape[1], k.shape[1], q.shape[-1], ctx_len, _dtype_code(q), scale, 0,
                 qsb, qsh, qsn, k.stride(0), k.stride(1), k.stride(2))


def check(status: int, where: str) -> None:
    if status != 0:
        raise KascadeError(status, where)


def workspace(op: int, shape: Shape, topk: int = 0, rule: Optional[TopkRule] = None,
              device="cuda") -> torch.Tensor:
    n = kascade_workspace_bytes(op, shape, topk, rule)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def anchor_decode(q, k, v, topk: int, ctx_len: Optional[int] = None, want_pooled=False, ws=None):
    """Returns (out [B,Hq,d], lse [B,Hq], idx int32 [B,Hkv,topk], pooled or None)."""
    N = ctx_len or k.shape[2]
    sh = make_shape(q, k, N)
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    out = torch.empty((B, Hq, d), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    idx = torch.empty((B, Hkv, topk), dtype=torch.int32, device=q.device)
    pooled = torch.empty((B, Hkv, N), dtype=torch.float32, device=q.device) if want_pooled else None
    ws = ws if ws is not None else workspace(OP_ANCHOR_DECODE, sh, topk)
    check(kascade_anchor_decode(sh, q, k, v, topk, out, lse, idx, pooled, ws, ws.numel()),
          "kascade_anchor_decode")
    return out, lse, idx, pooled


def anchor_decode_fused(q, k, v, topk: int, ctx_len: Optional[int] = None, want_pooled=False, ws=None,
                        max_polls: int = 0):
    """anchor_decode in one launch.  `ws` must come from workspace(OP_ANCHOR_DECODE_FUSED, ...)
    (allocated zeroed: its status word and barrier counters start at zero and
    every call leaves the counters zero); ws[0:4] holds the status word."""
    N = ctx_len or k.shape[2]
    sh = make_shape(q, k, N)
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    out = torch.empty((B, Hq, d), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    idx = torch.empty((B, Hkv, topk), dtype=torch.int32, device=q.device)
    pooled = torch.empty((B, Hkv, N), dtype=torch.float32, device=q.device) if want_pooled else None
    ws = ws if ws is not None else workspace(OP_ANCHOR_DECODE_FUSED, sh, topk)
    check(kascade_anchor_decode_fused(sh, q, k, v, topk, out, lse, idx, pooled, max_polls, ws, ws.numel()),
          "kascade_anchor_decode_fused")
    return out, lse, idx, pooled


def fused_status(ws) -> int:
    """The status word of a fused anchor-decode workspace (waits for the stream)."""
    return int(ws[0:4].view(torch.int32).item())


def reuse_decode(q, k, v, anchor_idx, head_map: Sequence[int], ctx_len: Optional[int] = None, ws=None):
    N = ctx_len or k.shape[2]
    sh = make_shape(q, k, N)
    topk = anchor_idx.shape[-1]
    out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    ws = ws if ws is not None else workspace(OP_REUSE_DECODE, sh, topk)
    check(kascade_reuse_decode(sh, q, k, v, topk, anchor_idx, head_map, out, ws, ws.numel()),
          "kascade_reuse_decode")
    return out


def dense_decode(q, k, v, ctx_len: Optional[int] = None, ws=None):
    N = ctx_len or k.shape[2]
    sh = make_shape(q, k, N)
    out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    ws = ws if ws is not None else workspace(OP_DENSE_DECODE, sh)
    check(kascade_dense_decode(sh, q, k, v, out, lse, ws, ws.numel()), "kascade_dense_decode")
    return out, lse


def topk_select(scores: torch.Tensor, k: int) -> torch.Tensor:
    rows, n = scores.shape
    idx = torch.empty((rows, k), dtype=torch.int32, device=scores.device)
    check(kascade_topk_select_f32(scores, scores.stride(0), rows, n, k, idx, k),
          "kascade_topk_select_f32")
    return idx


def prefill_k_max(n: int, rule: TopkRule = PREFILL_RULE) -> int:
    return kascade_topk_for_len(n, rule)


def anchor_prefill(q, k, v, rule: TopkRule = PREFILL_RULE, want_pooled=False, ws=None):
    """Returns (out [B,Hq,N,d], lse [B,Hq,N], tile idx [B,T,Hkv,k_max], pooled or None)."""
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    sh = make_shape(q, k, N)
    T = -(-N // rule.tile)
    kmax = prefill_k_max(N, rule)
    out = torch.empty((B, Hq, N, d), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    idx = torch.empty((B, T, Hkv, kmax), dtype=torch.int32, device=q.device)
    pooled = None
    if want_pooled:
        per_batch = packed_size(N, Hkv, rule.tile)
        pooled = torch.empty((B, per_batch), dtype=torch.float32, device=q.device)
    ws = ws if ws is not None else workspace(OP_ANCHOR_PREFILL, sh, 0, rule)
    check(kascade_anchor_prefill(sh, q, k, v, rule, out, lse, idx, pooled, ws, ws.numel()),
          "kascade_anchor_prefill")
    return out, lse, idx, pooled


def reuse_prefill(q, k, v, anchor_tile_idx, head_map: Sequence[int], rule: TopkRule = PREFILL_RULE):
    N = q.shape[2]
    sh = make_shape(q, k, N)
    out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    check(kascade_reuse_prefill(sh, q, k, v, rule, anchor_tile_idx, head_map, out, None, 0),
          "kascade_reuse_prefill")
    return out


def dense_prefill(q, k, v):
    N = q.shape[2]
    sh = make_shape(q, k, N)
    out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    check(kascade_dense_prefill(sh, q, k, v, out, lse), "kascade_dense_prefill")
    return out, lse


def packed_size(n: int, n_kv: int, tile: int = 128) -> int:
    """Elements of one batch's packed pooled rows: n_kv * sum_t P_t."""
    T = -(-n // tile)
    return n_kv * sum(min(n, tile * (t + 1)) for t in range(T))


def packed_row(pooled_b: torch.Tensor, t: int, g: int, n: int, n_kv: int, tile: int = 128):
    """View of packed row (t, g) of one batch's pooled buffer."""
    off = n_kv * sum(min(n, tile * (u + 1)) for u in range(t))
    P = min(n, tile * (t + 1))
    off += g * P
    return pooled_b[off:off + P]


def calib_head_similarity(pooled, topk_idx):
    """pooled [L,S,Hkv,n] fp32, topk_idx [L,S,Hkv,k] int32 (device) -> sim [L,L,Hkv,Hkv] fp32."""
    L, S, Hkv, n = pooled.shape
    k = topk_idx.shape[-1]
    sim = torch.zeros((L, L, Hkv, Hkv), dtype=torch.float32, device=pooled.device)
    check(kascade_calib_head_similarity(L, S, Hkv, n, k, pooled, topk_idx, sim),
          "kascade_calib_head_similarity")
    return sim


def layer_weight(x, y):
    """x, y [tokens, dim] (f32 or bf16, device) -> w (0-d fp32 device tensor)."""
    tokens, dim = x.shape
    w = torch.empty((), dtype=torch.float32, device=x.device)
    nb = max(kascade_layer_weight_workspace_bytes(tokens), 8)
    ws = torch.empty(nb, dtype=torch.uint8, device=x.device)
    check(kascade_layer_weight(x, y, tokens, dim, _dtype_code(x), w, ws, nb), "kascade_layer_weight")
    return w


def paged_shape(q, k_cache, n_ctx: int, scale: float = 0.0) -> Shape:
    """Shape for a paged cache [num_blocks, Hkv, block_size, d] (vLLM-style layout); q is
    [B,Hq,d] (decode) or [B,Hq,N,d] (prefill)."""
    qsn = q.stride(2) if q.dim() == 4 else 0
    return Shape(q.shape[0], q.shape[1], k_cache.shape[1], q.shape[-1], n_ctx, _dtype_code(q), scale, 0,
                 q.stride(0), q.stride(1), qsn, 0, k_cache.stride(1), k_cache.stride(2))


def paged_kv(block_table, k_cache) -> PagedKV:
    """Descriptor for caches laid out [num_blocks, Hkv, block_size, d]."""
    return PagedKV(block_table.data_ptr(), block_table.stride(0), k_cache.shape[2], k_cache.shape[0], 0,
                   k_cache.stride(0))


def anchor_decode_paged(q, k_cache, v_cache, block_table, n_ctx: int, topk: int, want_pooled=False):
    """Paged anchor decode; returns (out, lse, idx, pooled or None)."""
    sh = paged_shape(q, k_cache, n_ctx)
    pg = paged_kv(block_table, k_cache)
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    out = torch.empty((B, Hq, d), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    idx = torch.empty((B, Hkv, topk), dtype=torch.int32, device=q.device)
    pooled = torch.empty((B, Hkv, n_ctx), dtype=torch.float32, device=q.device) if want_pooled else None
    ws = workspace(OP_ANCHOR_DECODE, sh, topk)
    check(kascade_anchor_decode_paged(sh, pg, q, k_cache, v_cache, topk, out, lse, idx, pooled, ws, ws.numel()),
          "kascade_anchor_decode_paged")
    return out, lse, idx, pooled


def reuse_decode_paged(q, k_cache, v_cache, block_table, n_ctx: int, anchor_idx, head_map):
    sh = paged_shape(q, k_cache, n_ctx)
    pg = paged_kv(block_table, k_cache)
    topk = anchor_idx.shape[-1]
    out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    ws = workspace(OP_REUSE_DECODE, sh, topk)
    check(kascade_reuse_decode_paged(sh, pg, q, k_cache, v_cache, topk, anchor_idx, head_map, out, ws,
                                     ws.numel()), "kascade_reuse_decode_paged")
    return out


def reuse_prefill_paged(q, k_cache, v_cache, block_table, anchor_tile_idx, head_map: Sequence[int],
                        rule: TopkRule = PREFILL_RULE):
    """Paged reuse prefill: q [B,Hq,N,d], caches [num_blocks,Hkv,block_size,d]; returns out [B,Hq,N,d]."""
    N = q.shape[2]
    sh = paged_shape(q, k_cache, N)
    pg = paged_kv(block_table, k_cache)
    out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    check(kascade_reuse_prefill_paged(sh, pg, q, k_cache, v_cache, rule, anchor_tile_idx, head_map, out),
          "kascade_reuse_prefill_paged")
    return out
