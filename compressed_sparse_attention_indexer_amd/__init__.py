"""Compressed sparse attention (CSA) decode path for AMD MI355X (gfx950).

Python binding of libcsa.so with the same entry points as include/csa.h.
This module only marshals arguments: torch tensors supply device memory and
the current HIP stream; every step of the path runs in the HIP kernels of
libcsa.so.  There is no CPU fallback: without the built library every call
raises.
"""
from __future__ import annotations

import ctypes
import math
from typing import List, Optional, Sequence, Union

from ._lib import (CSA_ACT_NONE, CSA_ACT_RELU, CSA_BF16, CSA_F32, CSA_OP_ATTENTION, CSA_OP_HCA_MQA,
                   CSA_OP_INDEX_SCORES, CSA_OP_SPARSE_MQA, CSA_OP_TOPK, EXPORTS, CsaCompressDims, CsaDims,
                   CsaError, check, load_library)

__all__ = ["CsaDims", "CsaError", "make_dims", "workspace_size", "ptr_array", "csa_index_scores",
           "csa_index_scores_fp8", "CsaCompressDims", "make_compress_dims", "compress_workspace_size",
           "csa_compress",
           "csa_topk_select", "csa_sparse_mqa_decode", "hca_mqa_decode", "csa_attention", "load_library",
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


def _stream(stream):
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


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
    if scores is None:
        scores = torch.empty((dims.batch, dims.q_len, dims.max_entries), dtype=torch.float32, device=dev)
    kp, _keep = _pa(k_idx, dev)
    ws, nws = _ws(dims, CSA_OP_INDEX_SCORES, workspace, dev)
    check(load_library().csa_index_scores(ctypes.byref(dims), _p(q_idx), _p(w), kp, _p(seq_len), _p(q_pos),
                                          _p(scores), _p(ws), nws, _stream(stream)), "csa_index_scores")
    return scores


def csa_index_scores_fp8(dims: CsaDims, q8, q_scale, w, k8: PtrArg, k_scale: PtrArg, seq_len, q_pos, scores=None,
                         stream=None):
    """Indexer scores from fp8 (E4M3) index tensors with per-row scales (see csa.h)."""
    torch = _torch()
    dev = q8.device
    if scores is None:
        scores = torch.empty((dims.batch, dims.q_len, dims.max_entries), dtype=torch.float32, device=dev)
    kp, _keep = _pa(k8, dev)
    sp, _keep2 = _pa(k_scale, dev)
    check(load_library().csa_index_scores_fp8(ctypes.byref(dims), _p(q8), _p(q_scale), _p(w), kp, sp, _p(seq_len),
                                              _p(q_pos), _p(scores), _stream(stream)), "csa_index_scores_fp8")
    return scores


def csa_topk_select(dims: CsaDims, scores, seq_len, q_pos, topk_idx=None, workspace=None, stream=None):
    """Top-k indices [B,T,K] int32, ascending, -1 padded (see csa.h)."""
    torch = _torch()
    dev = scores.device
    if topk_idx is None:
        topk_idx = torch.empty((dims.batch, dims.q_len, dims.topk), dtype=torch.int32, device=dev)
    ws, nws = _ws(dims, CSA_OP_TOPK, workspace, dev)
    check(load_library().csa_topk_select(ctypes.byref(dims), _p(scores), _p(seq_len), _p(q_pos), _p(topk_idx),
                                         _p(ws), nws, _stream(stream)), "csa_topk_select")
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
    out, lse = _attn_outputs(dims, dev, out, lse, want_lse)
    (kp, k1), (vp, k2), (wp, k3), (wvp, k4) = (_pa(x, dev) for x in (kv, v, win, win_v))
    ws, nws = _ws(dims, CSA_OP_SPARSE_MQA, workspace, dev)
    check(load_library().csa_sparse_mqa_decode(
        ctypes.byref(dims), _p(q), kp, vp, _p(topk_idx), wp, wvp, _p(win_pos0), _p(win_rows), _p(seq_len),
        _p(q_pos), _p(sink), _p(out), _p(lse), _p(ws), nws, _stream(stream)), "csa_sparse_mqa_decode")
    return out, lse


def hca_mqa_decode(dims: CsaDims, q, kv: PtrArg, v: PtrArg, win: PtrArg, win_v: PtrArg, win_pos0, win_rows,
                   seq_len, q_pos, sink, out=None, lse=None, want_lse=True, workspace=None, stream=None):
    """Dense MQA with sink over every visible HCA entry + window rows; returns (out, lse)."""
    dev = q.device
    out, lse = _attn_outputs(dims, dev, out, lse, want_lse)
    (kp, k1), (vp, k2), (wp, k3), (wvp, k4) = (_pa(x, dev) for x in (kv, v, win, win_v))
    ws, nws = _ws(dims, CSA_OP_HCA_MQA, workspace, dev)
    check(load_library().hca_mqa_decode(
        ctypes.byref(dims), _p(q), kp, vp, wp, wvp, _p(win_pos0), _p(win_rows), _p(seq_len), _p(q_pos),
        _p(sink), _p(out), _p(lse), _p(ws), nws, _stream(stream)), "hca_mqa_decode")
    return out, lse


def csa_attention(dims: CsaDims, q, q_idx, w, k_idx: PtrArg, kv: PtrArg, v: PtrArg, win: PtrArg,
                  win_v: PtrArg, win_pos0, win_rows, seq_len, q_pos, sink, out=None, lse=None, want_lse=True,
                  topk_idx_out=None, scores_out=None, workspace=None, stream=None):
    """Whole CSA step (scores -> top-k -> sparse MQA with sink); returns (out, lse)."""
    dev = q.device
    out, lse = _attn_outputs(dims, dev, out, lse, want_lse)
    (kip, k0), (kp, k1), (vp, k2), (wp, k3), (wvp, k4) = (_pa(x, dev) for x in (k_idx, kv, v, win, win_v))
    ws, nws = _ws(dims, CSA_OP_ATTENTION, workspace, dev)
    check(load_library().csa_attention(
        ctypes.byref(dims), _p(q), _p(q_idx), _p(w), kip, kp, vp, wp, wvp, _p(win_pos0), _p(win_rows),
        _p(seq_len), _p(q_pos), _p(sink), _p(out), _p(lse), _p(topk_idx_out), _p(scores_out), _p(ws), nws,
        _stream(stream)), "csa_attention")
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
    if out is None:
        out = torch.empty((dims.n_entries, dims.out_dim), dtype=torch.bfloat16, device=dev)
    n = compress_workspace_size(dims)
    if workspace is None:
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    check(load_library().csa_compress(ctypes.byref(dims), _p(x), _p(wkv), _p(wgate), _p(ape), _p(gamma), _p(out),
                                      _p(workspace), workspace.numel(), _stream(stream)), "csa_compress")
    return out
