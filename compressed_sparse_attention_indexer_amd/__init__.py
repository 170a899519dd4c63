"""Compressed sparse attention (CSA) decode path for AMD MI355X (gfx950).

Python binding of libcsa.so with the same entry points as include/csa.h.
This module only marshals arguments: torch tensors supply device memory and
the current HIP stream; every step of the path runs in the HIP kernels of
libcsa.so.  There is no CPU fallback: without the built library every call
raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
from typing import List, Optional, Sequence, Union

from ._lib import (CSA_ACT_NONE, CSA_ACT_RELU, CSA_BF16, CSA_F32, CSA_OP_ATTENTION, CSA_OP_ATTENTION_FP8, CSA_OP_HCA_MQA,
                   CSA_OP_INDEX_SCORES, CSA_OP_SPARSE_MQA, CSA_OP_TOPK, EXPORTS, CsaCompressDims, CsaDims,
                   CsaError, check, load_library)

__all__ = ["CsaDims", "CsaError", "make_dims", "workspace_size", "ptr_array", "csa_index_scores",
           "csa_index_scores_fp8", "CsaCompressDims", "make_compress_dims", "compress_workspace_size",
           "csa_compress", "csa_topk_select", "csa_sparse_mqa_decode", "hca_mqa_decode", "csa_attention",
           "csa_attention_fp8", "csa_attention_noalloc",
           "attention", "index_scores", "index_scores_fp8", "topk", "sparse_mqa", "hca_mqa", "load_library",
           "CSA_F32", "CSA_BF16", "CSA_ACT_RELU", "CSA_ACT_NONE"]


def make_dims(*, batch: int, q_len: int = 1, n_heads: int = 64, head_dim: int = 512, index_heads: int = 64,
              index_dim: int = 128, topk: int = 512, window: int = 128, ratio: int = 4, max_entries: int,
              dtype: int = CSA_BF16, index_act: int = CSA_ACT_RELU, softmax_scale: float = 0.0) -> CsaDims:
    return CsaDims(batch, q_len, n_heads, head_dim, index_heads, index_dim, topk, window, ratio, max_entries,
                   dtype, index_act, softmax_scale)


def workspace_size(dims: CsaDims, op: int) -> int:
    n = ctypes.c_size_t(0)
    check(load_library().csa_workspace_size(ctypes.byref(dims), op, ctypes.byref(n)), "csa_workspace_size")
    return int(n.value)


def _torch():
    import torch
    return torch


def ptr_array(tensors: Optional[Sequence], device) -> Optional["torch.Tensor"]:
    """Device int64 array holding the data pointers of per-sequence tensors."""
    if tensors is None:
        return None
    torch = _torch()
    return torch.tensor([t.data_ptr() for t in tensors], dtype=torch.int64, device=device)


PtrArg = Union[None, "torch.Tensor", List["torch.Tensor"]]


def _pa(x: PtrArg, device):
    """A per-sequence argument: a prebuilt device pointer array or a list of tensors."""
    if x is None:
        return None, None
    torch = _torch()
    if isinstance(x, torch.Tensor):
        return x.data_ptr(), x
    arr = ptr_array(x, device)
    return arr.data_ptr(), arr


def _p(t):
    return None if t is None else t.data_ptr()


@contextlib.contextmanager
def _on_stream(stream):
    """Run one call on `stream` (None: the current stream).  A stream other than
    the current one first waits for the current stream, and the call's
    temporaries, outputs and pointer-array uploads are made on it, so the
    caching allocator cannot hand their memory to other work before the
    kernels are done with it.  Outputs are ready on `stream`.  Yields the raw
    stream handle."""
    torch = _torch()
    cur = torch.cuda.current_stream()
    if stream is None:
        yield cur.cuda_stream
        return
    handle = stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream)
    if handle == cur.cuda_stream:
        yield handle
        return
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(handle)
    s.wait_stream(cur)
    with torch.cuda.stream(s):
        yield s.cuda_stream


def _ws(dims, op, workspace, device):
    need = workspace_size(dims, op)
    if workspace is not None:
        return workspace, workspace.numel() * workspace.element_size()
    if need == 0:
        return None, 0
    torch = _torch()
    # zero-filled: the top-k counters start clean (any contents are still correct, only slower once)
    return torch.zeros(need, dtype=torch.uint8, device=device), need


def csa_index_scores(dims: CsaDims, q_idx, w, k_idx: PtrArg, seq_len, q_pos, scores=None, workspace=None,
                     stream=None):
    """Indexer scores [B,T,max_entries] float32 (see csa.h)."""
    torch = _torch()
    dev = q_idx.device
    with _on_stream(stream) as st:
        if scores is None:
            scores = torch.empty((dims.batch, dims.q_len, dims.max_entries), dtype=torch.float32, device=dev)
        kp, _keep = _pa(k_idx, dev)
        ws, nws = _ws(dims, CSA_OP_INDEX_SCORES, workspace, dev)
        check(load_library().csa_index_scores(ctypes.byref(dims), _p(q_idx), _p(w), kp, _p(seq_len), _p(q_pos),
                                              _p(scores), _p(ws), nws, st), "csa_index_scores")
    return scores


def csa_index_scores_fp8(dims: CsaDims, q8, q_scale, w, k8: PtrArg, k_scale: PtrArg, seq_len, q_pos, scores=None,
                         stream=None):
    """Indexer scores from fp8 (E4M3) index tensors with per-row scales (see csa.h)."""
    torch = _torch()
    dev = q8.device
    with _on_stream(stream) as st:
        if scores is None:
            scores = torch.empty((dims.batch, dims.q_len, dims.max_entries), dtype=torch.float32, device=dev)
        kp, _keep = _pa(k8, dev)
        sp, _keep2 = _pa(k_scale, dev)
        check(load_library().csa_index_scores_fp8(ctypes.byref(dims), _p(q8), _p(q_scale), _p(w), kp, sp,
                                                  _p(seq_len), _p(q_pos), _p(scores), st), "csa_index_scores_fp8")
    return scores


def csa_topk_select(dims: CsaDims, scores, seq_len, q_pos, topk_idx=None, workspace=None, stream=None):
    """Top-k indices [B,T,K] int32, ascending, -1 padded (see csa.h)."""
    torch = _torch()
    dev = scores.device
    with _on_stream(stream) as st:
        if topk_idx is None:
            topk_idx = torch.empty((dims.batch, dims.q_len, dims.topk), dtype=torch.int32, device=dev)
        ws, nws = _ws(dims, CSA_OP_TOPK, workspace, dev)
        check(load_library().csa_topk_select(ctypes.byref(dims), _p(scores), _p(seq_len), _p(q_pos), _p(topk_idx),
                                             _p(ws), nws, st), "csa_topk_select")
    return topk_idx


def _attn_outputs(dims, device, out, lse, want_lse):
    torch = _torch()
    if out is None:
        out = torch.empty((dims.batch, dims.q_len, dims.n_heads, dims.head_dim), dtype=torch.float32,
                          device=device)
    if lse is None and want_lse:
        lse = torch.empty((dims.batch, dims.q_len, dims.n_heads), dtype=torch.float32, device=device)
    return out, lse


def csa_sparse_mqa_decode(dims: CsaDims, q, kv: PtrArg, v: PtrArg, topk_idx, win: PtrArg, win_v: PtrArg,
                          win_pos0, win_rows, seq_len, q_pos, sink, out=None, lse=None, want_lse=True,
                          workspace=None, stream=None):
    """Sparse MQA with sink over top-k rows + window rows; returns (out, lse)."""
    dev = q.device
    with _on_stream(stream) as st:
        out, lse = _attn_outputs(dims, dev, out, lse, want_lse)
        (kp, k1), (vp, k2), (wp, k3), (wvp, k4) = (_pa(x, dev) for x in (kv, v, win, win_v))
        ws, nws = _ws(dims, CSA_OP_SPARSE_MQA, workspace, dev)
        check(load_library().csa_sparse_mqa_decode(
            ctypes.byref(dims), _p(q), kp, vp, _p(topk_idx), wp, wvp, _p(win_pos0), _p(win_rows), _p(seq_len),
            _p(q_pos), _p(sink), _p(out), _p(lse), _p(ws), nws, st), "csa_sparse_mqa_decode")
    return out, lse


def hca_mqa_decode(dims: CsaDims, q, kv: PtrArg, v: PtrArg, win: PtrArg, win_v: PtrArg, win_pos0, win_rows,
                   seq_len, q_pos, sink, out=None, lse=None, want_lse=True, workspace=None, stream=None):
    """Dense MQA with sink over every visible HCA entry + window rows; returns (out, lse)."""
    dev = q.device
    with _on_stream(stream) as st:
        out, lse = _attn_outputs(dims, dev, out, lse, want_lse)
        (kp, k1), (vp, k2), (wp, k3), (wvp, k4) = (_pa(x, dev) for x in (kv, v, win, win_v))
        ws, nws = _ws(dims, CSA_OP_HCA_MQA, workspace, dev)
        check(load_library().hca_mqa_decode(
            ctypes.byref(dims), _p(q), kp, vp, wp, wvp, _p(win_pos0), _p(win_rows), _p(seq_len), _p(q_pos),
            _p(sink), _p(out), _p(lse), _p(ws), nws, st), "hca_mqa_decode")
    return out, lse


def csa_attention(dims: CsaDims, q, q_idx, w, k_idx: PtrArg, kv: PtrArg, v: PtrArg, win: PtrArg,
                  win_v: PtrArg, win_pos0, win_rows, seq_len, q_pos, sink, out=None, lse=None, want_lse=True,
                  topk_idx_out=None, scores_out=None, workspace=None, stream=None):
    """Whole CSA step (scores -> top-k -> sparse MQA with sink); returns (out, lse)."""
    dev = q.device
    with _on_stream(stream) as st:
        out, lse = _attn_outputs(dims, dev, out, lse, want_lse)
        (kip, k0), (kp, k1), (vp, k2), (wp, k3), (wvp, k4) = (_pa(x, dev) for x in (k_idx, kv, v, win, win_v))
        ws, nws = _ws(dims, CSA_OP_ATTENTION, workspace, dev)
        check(load_library().csa_attention(
            ctypes.byref(dims), _p(q), _p(q_idx), _p(w), kip, kp, vp, wp, wvp, _p(win_pos0), _p(win_rows),
            _p(seq_len), _p(q_pos), _p(sink), _p(out), _p(lse), _p(topk_idx_out), _p(scores_out), _p(ws), nws,
            st), "csa_attention")
    return out, lse


def csa_attention_fp8(dims: CsaDims, q, q8, q_scale, w, k8: PtrArg, k_scale: PtrArg, kv: PtrArg, v: PtrArg,
                      win: PtrArg, win_v: PtrArg, win_pos0, win_rows, seq_len, q_pos, sink, out=None, lse=None,
                      want_lse=True, topk_idx_out=None, scores_out=None, workspace=None, stream=None):
    """Whole CSA step with fp8 (E4M3) index tensors and per-row scales; bf16
    attention side; returns (out, lse)."""
    dev = q.device
    with _on_stream(stream) as st:
        out, lse = _attn_outputs(dims, dev, out, lse, want_lse)
        (k8p, k0), (ksp, k5), (kp, k1), (vp, k2), (wp, k3), (wvp, k4) = (
            _pa(x, dev) for x in (k8, k_scale, kv, v, win, win_v))
        ws, nws = _ws(dims, CSA_OP_ATTENTION_FP8, workspace, dev)
        check(load_library().csa_attention_fp8(
            ctypes.byref(dims), _p(q), _p(q8), _p(q_scale), _p(w), k8p, ksp, kp, vp, wp, wvp, _p(win_pos0),
            _p(win_rows), _p(seq_len), _p(q_pos), _p(sink), _p(out), _p(lse), _p(topk_idx_out), _p(scores_out),
            _p(ws), nws, st), "csa_attention_fp8")
    return out, lse


def csa_attention_noalloc(dims: CsaDims, q, q_idx, w, k_idx: PtrArg, kv: PtrArg, v: PtrArg, win: PtrArg,
                          win_v: PtrArg, win_pos0, win_rows, seq_len, q_pos, sink, out=None, lse=None,
                          want_lse=True, topk_idx_out=None, scores_out=None, stream=None):
    """csa_attention on the library's own static work area (no workspace
    argument); returns (out, lse).  Pass prebuilt device pointer arrays and
    outputs to keep the call free of allocations."""
    dev = q.device
    with _on_stream(stream) as st:
        out, lse = _attn_outputs(dims, dev, out, lse, want_lse)
        (kip, k0), (kp, k1), (vp, k2), (wp, k3), (wvp, k4) = (_pa(x, dev) for x in (k_idx, kv, v, win, win_v))
        check(load_library().csa_attention_noalloc(
            ctypes.byref(dims), _p(q), _p(q_idx), _p(w), kip, kp, vp, wp, wvp, _p(win_pos0), _p(win_rows),
            _p(seq_len), _p(q_pos), _p(sink), _p(out), _p(lse), _p(topk_idx_out), _p(scores_out), st),
            "csa_attention_noalloc")
    return out, lse


def make_compress_dims(*, tokens: int, hidden: int, out_dim: int, ratio: int, window: int, first_entry: int,
                       n_entries: int, pos0: int, rope_dims: int = 0, hadamard: bool = False,
                       rope_theta: float = 160000.0, rms_eps: float = 1e-6) -> CsaCompressDims:
    return CsaCompressDims(tokens, hidden, out_dim, ratio, window, rope_dims, int(hadamard), first_entry, n_entries,
                           pos0, rope_theta, rms_eps)


def compress_workspace_size(dims: CsaCompressDims) -> int:
    n = ctypes.c_size_t(0)
    check(load_library().csa_compress_workspace_size(ctypes.byref(dims), ctypes.byref(n)),
          "csa_compress_workspace_size")
    return int(n.value)


def csa_compress(dims: CsaCompressDims, x, wkv, wgate, ape, gamma, out=None, workspace=None, stream=None):
    """Compressed entries [n_entries, out_dim] bf16 (see csa.h)."""
    torch = _torch()
    dev = x.device
    with _on_stream(stream) as st:
        if out is None:
            out = torch.empty((dims.n_entries, dims.out_dim), dtype=torch.bfloat16, device=dev)
        n = compress_workspace_size(dims)
        if workspace is None:
            workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
        check(load_library().csa_compress(ctypes.byref(dims), _p(x), _p(wkv), _p(wgate), _p(ape), _p(gamma),
                                          _p(out), _p(workspace), workspace.numel(), st), "csa_compress")
    return out


# ----------------------------------------------------------------------------- tensor-level calls
# The same operations with their sizes taken from the tensors' shapes: the
# caller passes per-sequence lists of cache tensors and keyword options; the
# csa_dims struct and the device pointer arrays are built here.  Marshalling
# only, like the calls above.

def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    if t.dtype == torch.float32:
        return CSA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _act_code(act) -> int:
    if act in ("relu", CSA_ACT_RELU):
        return CSA_ACT_RELU
    if act in (None, "none", CSA_ACT_NONE):
        return CSA_ACT_NONE
    raise ValueError(f"unknown index activation {act!r} ('relu' or 'none')")


def _i32(x, device, name):
    """A [B] or [B*T] int32 argument: device tensor as given, else uploaded."""
    torch = _torch()
    if isinstance(x, torch.Tensor):
        if x.dtype != torch.int32:
            raise TypeError(f"{name} must be int32 (got {x.dtype})")
        return x.reshape(-1).to(device)
    return torch.tensor(list(x), dtype=torch.int32, device=device)


def _host_ints(x):
    """Host values of an int argument, or None if it lives on the device."""
    torch = _torch()
    if isinstance(x, torch.Tensor):
        return None if x.is_cuda else [int(v) for v in x.reshape(-1).tolist()]
    return [int(v) for v in x]


def _windows(win, seq_len, win_pos0, device):
    """(win_pos0, win_rows) device tensors.  win_rows come from the window
    tensors' lengths; win_pos0 defaults to L_b - win_rows[b] (each window
    buffer holds the newest raw rows of its sequence), which needs seq_len on
    the host."""
    torch = _torch()
    rows = [int(t.shape[0]) for t in win]
    if win_pos0 is None:
        lens = _host_ints(seq_len)
        if lens is None:
            raise ValueError("win_pos0 is needed when seq_len is a device tensor")
        win_pos0 = [L - r for L, r in zip(lens, rows)]
    return _i32(win_pos0, device, "win_pos0"), torch.tensor(rows, dtype=torch.int32, device=device)


def _n_max(caches, max_entries):
    if max_entries is not None:
        return int(max_entries)
    return max(1, max(int(t.shape[0]) for t in caches))


def attention(q, q_idx, w, k_idx: Sequence, kv: Sequence, win: Sequence, seq_len, q_pos, sink, *, topk: int = 512,
              window: int = 128, ratio: int = 4, v: Optional[Sequence] = None, win_v: Optional[Sequence] = None,
              scale: Optional[float] = None, win_pos0=None, act="relu", max_entries: Optional[int] = None,
              workspace=None, stream=None):
    """The whole CSA step from tensors: indexer scores, top-k, sparse MQA with
    the window and the sink.  q [B,T,H,D], q_idx [B,T,HI,DI], w [B,T,HI]
    float32, per-sequence lists k_idx[b] [N_b,DI], kv[b] [N_b,D], win[b]
    [R_b,D] (and optional v, win_v), seq_len [B] and q_pos [B*T] int32 (device
    tensors or host values), sink [H] float32.  Returns (out [B,T,H,D]
    float32, lse [B,T,H] float32, idx [B,T,topk] int32)."""
    torch = _torch()
    dev = q.device
    B, T, H, D = q.shape
    with _on_stream(stream) as st:
        wp0, wrows = _windows(win, seq_len, win_pos0, dev)
        sl, qp = _i32(seq_len, dev, "seq_len"), _i32(q_pos, dev, "q_pos")
        dims = make_dims(batch=B, q_len=T, n_heads=H, head_dim=D, index_heads=q_idx.shape[2],
                         index_dim=q_idx.shape[3], topk=topk, window=window, ratio=ratio,
                         max_entries=_n_max(k_idx, max_entries), dtype=_dtype_code(q), index_act=_act_code(act),
                         softmax_scale=0.0 if scale is None else float(scale))
        idx = torch.empty((B, T, topk), dtype=torch.int32, device=dev)
        out, lse = csa_attention(dims, q, q_idx, w, list(k_idx), list(kv), None if v is None else list(v), list(win),
                                 None if win_v is None else list(win_v), wp0, wrows, sl, qp, sink,
                                 topk_idx_out=idx, workspace=workspace, stream=st)
    return out, lse, idx


def index_scores(q_idx, w, k_idx: Sequence, seq_len, q_pos, *, ratio: int = 4, act="relu",
                 max_entries: Optional[int] = None, stream=None):
    """Indexer scores [B,T,max_entries] float32 from tensors (-inf where not visible)."""
    dev = q_idx.device
    B, T, HI, DI = q_idx.shape
    with _on_stream(stream) as st:
        dims = make_dims(batch=B, q_len=T, index_heads=HI, index_dim=DI, ratio=ratio,
                         max_entries=_n_max(k_idx, max_entries), dtype=_dtype_code(q_idx), index_act=_act_code(act))
        return csa_index_scores(dims, q_idx, w, list(k_idx), _i32(seq_len, dev, "seq_len"),
                                _i32(q_pos, dev, "q_pos"), stream=st)


def index_scores_fp8(q8, q_scale, w, k8: Sequence, k_scale: Sequence, seq_len, q_pos, *, ratio: int = 4,
                     act="relu", max_entries: Optional[int] = None, stream=None):
    """Indexer scores from fp8 (E4M3) codes (uint8) with per-row float32 scales."""
    dev = q8.device
    B, T, HI, DI = q8.shape
    with _on_stream(stream) as st:
        dims = make_dims(batch=B, q_len=T, index_heads=HI, index_dim=DI, ratio=ratio,
                         max_entries=_n_max(k8, max_entries), index_act=_act_code(act))
        return csa_index_scores_fp8(dims, q8, q_scale, w, list(k8), list(k_scale), _i32(seq_len, dev, "seq_len"),
                                    _i32(q_pos, dev, "q_pos"), stream=st)


def topk(scores, seq_len, q_pos, *, topk: int = 512, ratio: int = 4, workspace=None, stream=None):
    """Top-k indices [B,T,topk] int32 of a [B,T,max_entries] score tensor."""
    dev = scores.device
    B, T, n_max = scores.shape
    with _on_stream(stream) as st:
        dims = make_dims(batch=B, q_len=T, topk=topk, ratio=ratio, max_entries=n_max)
        return csa_topk_select(dims, scores, _i32(seq_len, dev, "seq_len"), _i32(q_pos, dev, "q_pos"),
                               workspace=workspace, stream=st)


def sparse_mqa(q, kv: Sequence, topk_idx, win: Sequence, seq_len, q_pos, sink, *, window: int = 128, ratio: int = 4,
               v: Optional[Sequence] = None, win_v: Optional[Sequence] = None, scale: Optional[float] = None,
               win_pos0=None, max_entries: Optional[int] = None, workspace=None, stream=None):
    """Sparse MQA with sink over the rows topk_idx [B,T,K] selects, then the window; returns (out, lse)."""
    dev = q.device
    B, T, H, D = q.shape
    with _on_stream(stream) as st:
        wp0, wrows = _windows(win, seq_len, win_pos0, dev)
        dims = make_dims(batch=B, q_len=T, n_heads=H, head_dim=D, topk=topk_idx.shape[-1], window=window,
                         ratio=ratio, max_entries=_n_max(kv, max_entries), dtype=_dtype_code(q),
                         softmax_scale=0.0 if scale is None else float(scale))
        return csa_sparse_mqa_decode(dims, q, list(kv), None if v is None else list(v), topk_idx, list(win),
                                     None if win_v is None else list(win_v), wp0, wrows,
                                     _i32(seq_len, dev, "seq_len"), _i32(q_pos, dev, "q_pos"), sink,
                                     workspace=workspace, stream=st)


def hca_mqa(q, kv: Sequence, win: Sequence, seq_len, q_pos, sink, *, window: int = 128, ratio: int = 128,
            v: Optional[Sequence] = None, win_v: Optional[Sequence] = None, scale: Optional[float] = None,
            win_pos0=None, max_entries: Optional[int] = None, workspace=None, stream=None):
    """Dense MQA with sink over every visible entry of a ratio-r cache, then the window; returns (out, lse)."""
    dev = q.device
    B, T, H, D = q.shape
    with _on_stream(stream) as st:
        wp0, wrows = _windows(win, seq_len, win_pos0, dev)
        dims = make_dims(batch=B, q_len=T, n_heads=H, head_dim=D, window=window, ratio=ratio,
                         max_entries=_n_max(kv, max_entries), dtype=_dtype_code(q),
                         softmax_scale=0.0 if scale is None else float(scale))
        return hca_mqa_decode(dims, q, list(kv), None if v is None else list(v), list(win),
                              None if win_v is None else list(win_v), wp0, wrows, _i32(seq_len, dev, "seq_len"),
                              _i32(q_pos, dev, "q_pos"), sink, workspace=workspace, stream=st)
