"""CPU oracle for the CSA decode path -- TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper around ``liboracle.so`` (plain C, float64, built with gcc
from ``oracle.c``).  Only the tests, the smoke check and the benchmark's
CPU-baseline leg import this package; the product library never does, and the
oracle shares no code with the HIP path.  Definitions and sources are in
``oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1
ACT_RELU, ACT_NONE = 0, 1
OK, EINVAL, EWINDOW, ENOMEM = 0, -1, -2, -3


def build() -> str:
    """Compile liboracle.so with gcc (OpenMP)."""
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fopenmp", "-fPIC",
                           "-shared", os.path.join(_HERE, "oracle.c"), os.path.join(_HERE, "compressor.c"), "-o", tmp,
                           "-lm"])
    os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        P, I, D, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_int64
        L.oracle_num_threads.restype = I
        L.oracle_visible_count.argtypes = [I64, I64, I]
        L.oracle_visible_count.restype = I64
        L.oracle_index_scores.argtypes = [I] * 7 + [P, P, P, P, P, I, P]
        L.oracle_topk.argtypes = [I, I, I, I, P, I, P, P, P]
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_value.restype = D
        L.oracle_index_scores_fp8.argtypes = [I] * 6 + [P] * 7 + [I, P]
        L.oracle_compress.argtypes = [I] * 6 + [D, D, I, P, I, P, P, P, P, I, I, P]
        L.oracle_attend_rows.argtypes = [I, I, I, D, P, P, P, I, P, P, P]
        L.oracle_partial_rows.argtypes = [I, I, I, D, P, P, P, I, P, P, P]
        L.oracle_merge_partials.argtypes = [I, I, I, P, P, P, P, P, P]
        L.oracle_sparse_mqa.argtypes = [I] * 8 + [D] + [P] * 13
        L.oracle_hca_mqa.argtypes = [I] * 7 + [D] + [P] * 12
        L.oracle_csa_attention.argtypes = [I] * 11 + [D] + [P] * 13 + [I] + [P] * 4
        for f in ("oracle_index_scores", "oracle_index_scores_fp8", "oracle_compress", "oracle_topk", "oracle_attend_rows", "oracle_partial_rows",
                  "oracle_merge_partials", "oracle_sparse_mqa", "oracle_hca_mqa",
                  "oracle_csa_attention"):
            getattr(L, f).restype = I
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != OK:
        raise OracleError(f"{what} failed with code {rc}")


def _dt(dtype: str) -> int:
    return BF16 if dtype == "bf16" else F32


def _arr(x: np.ndarray, dtype: str) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.uint16 if dtype == "bf16" else np.float32)


def _p(x: Optional[np.ndarray]):
    return None if x is None else x.ctypes.data


class _PtrArray:
    """Host array of host pointers to per-sequence buffers (keeps them alive)."""

    def __init__(self, arrs: Optional[Sequence[np.ndarray]], dtype: str):
        self.keep = None if arrs is None else [_arr(a, dtype) for a in arrs]
        self.c = None if arrs is None else (ctypes.c_void_p * len(self.keep))(
            *[a.ctypes.data for a in self.keep])

    @property
    def ptr(self):
        return None if self.c is None else ctypes.cast(self.c, ctypes.c_void_p)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def visible_count(seq_len: int, pos: int, ratio: int) -> int:
    return int(lib().oracle_visible_count(seq_len, pos, ratio))


def index_scores(q_idx, w, k_idx: List[np.ndarray], seq_len, q_pos, *, ratio: int, n_max: int,
                 dtype: str, act: int = ACT_RELU) -> np.ndarray:
    B, T, HI, DI = q_idx.shape
    qa, wa = _arr(q_idx, dtype), np.ascontiguousarray(w, dtype=np.float32)
    ks = _PtrArray(k_idx, dtype)
    sl, qp = np.ascontiguousarray(seq_len, np.int32), np.ascontiguousarray(q_pos, np.int32)
    out = np.empty((B, T, n_max), dtype=np.float32)
    _check(lib().oracle_index_scores(B, T, HI, DI, ratio, act, _dt(dtype), _p(qa), _p(wa), ks.ptr,
                                     _p(sl), _p(qp), n_max, _p(out)), "oracle_index_scores")
    return out


def e4m3_value(code: int) -> float:
    return float(lib().oracle_e4m3_value(code))


def index_scores_fp8(q8, q_scale, w, k8: List[np.ndarray], k_scale: List[np.ndarray], seq_len, q_pos, *,
                     ratio: int, n_max: int, act: int = ACT_RELU) -> np.ndarray:
    """q8 [B,T,HI,DI] uint8 codes, q_scale [B,T,HI], k8[b] [N_b,DI] codes, k_scale[b] [N_b]."""
    B, T, HI, DI = q8.shape
    qa = np.ascontiguousarray(q8, np.uint8)
    qs = np.ascontiguousarray(q_scale, np.float32)
    wa = np.ascontiguousarray(w, np.float32)
    kc = [np.ascontiguousarray(k, np.uint8) for k in k8]
    kss = [np.ascontiguousarray(x, np.float32) for x in k_scale]
    kp = (ctypes.c_void_p * len(kc))(*[k.ctypes.data for k in kc])
    sp = (ctypes.c_void_p * len(kss))(*[x.ctypes.data for x in kss])
    sl, qp = np.ascontiguousarray(seq_len, np.int32), np.ascontiguousarray(q_pos, np.int32)
    out = np.empty((B, T, n_max), dtype=np.float32)
    _check(lib().oracle_index_scores_fp8(B, T, HI, DI, ratio, act, _p(qa), _p(qs), _p(wa), kp, sp, _p(sl), _p(qp),
                                         n_max, _p(out)), "oracle_index_scores_fp8")
    return out


def compress(x, wkv, wgate, ape, gamma, *, pos0: int, ratio: int, window: int, first_entry: int, n_entries: int,
             rope_dims: int = 0, rope_theta: float = 160000.0, eps: float = 1e-6, hadamard: bool = False) -> np.ndarray:
    """x [tokens, hidden] bf16 bits; wkv/wgate [out_dim, hidden] bf16 bits; ape [window, out_dim];
    gamma [out_dim].  Returns [n_entries, out_dim] float64."""
    tokens, hidden = x.shape
    out_dim = wkv.shape[0]
    xa, wk, wg = (np.ascontiguousarray(a, np.uint16) for a in (x, wkv, wgate))
    ap, gm = np.ascontiguousarray(ape, np.float32), np.ascontiguousarray(gamma, np.float32)
    out = np.empty((n_entries, out_dim), np.float64)
    _check(lib().oracle_compress(tokens, hidden, out_dim, ratio, window, rope_dims, rope_theta, eps, int(hadamard),
                                 _p(xa), pos0, _p(wk), _p(wg), _p(ap), _p(gm), first_entry, n_entries, _p(out)),
           "oracle_compress")
    return out


def topk(scores, seq_len, q_pos, *, ratio: int, k: int) -> np.ndarray:
    B, T, n_max = scores.shape
    sc = np.ascontiguousarray(scores, dtype=np.float32)
    sl, qp = np.ascontiguousarray(seq_len, np.int32), np.ascontiguousarray(q_pos, np.int32)
    out = np.empty((B, T, k), dtype=np.int32)
    _check(lib().oracle_topk(B, T, ratio, k, _p(sc), n_max, _p(sl), _p(qp), _p(out)), "oracle_topk")
    return out


def _row_ptrs(rows: np.ndarray):
    return (ctypes.c_void_p * max(1, len(rows)))(*[rows[i].ctypes.data for i in range(len(rows))])


def attend_rows(q, rows, vrows=None, sink=None, *, scale: float, dtype: str):
    """q [H,D]; rows/vrows [n,D]; returns (out [H,D], lse [H]) in float64."""
    H, D = q.shape
    qa, ra = _arr(q, dtype), _arr(rows, dtype)
    va = None if vrows is None else _arr(vrows, dtype)
    rp = _row_ptrs(ra)
    vp = None if va is None else _row_ptrs(va)
    sk = None if sink is None else np.ascontiguousarray(sink, np.float32)
    out = np.empty((H, D), np.float64)
    lse = np.empty(H, np.float64)
    _check(lib().oracle_attend_rows(H, D, _dt(dtype), scale, _p(qa), ctypes.cast(rp, ctypes.c_void_p),
                                    None if vp is None else ctypes.cast(vp, ctypes.c_void_p),
                                    len(ra), _p(sk), _p(out), _p(lse)), "oracle_attend_rows")
    return out, lse


def partial_rows(q, rows, vrows=None, *, scale: float, dtype: str):
    H, D = q.shape
    qa, ra = _arr(q, dtype), _arr(rows, dtype)
    va = None if vrows is None else _arr(vrows, dtype)
    rp = _row_ptrs(ra)
    vp = None if va is None else _row_ptrs(va)
    m, l, o = np.empty(H), np.empty(H), np.empty((H, D))
    _check(lib().oracle_partial_rows(H, D, _dt(dtype), scale, _p(qa), ctypes.cast(rp, ctypes.c_void_p),
                                     None if vp is None else ctypes.cast(vp, ctypes.c_void_p),
                                     len(ra), _p(m), _p(l), _p(o)), "oracle_partial_rows")
    return m, l, o


def merge_partials(m, l, o, sink=None):
    S, H, D = o.shape
    m, l, o = (np.ascontiguousarray(x, np.float64) for x in (m, l, o))
    sk = None if sink is None else np.ascontiguousarray(sink, np.float32)
    out, lse = np.empty((H, D)), np.empty(H)
    _check(lib().oracle_merge_partials(S, H, D, _p(m), _p(l), _p(o), _p(sk), _p(out), _p(lse)),
           "oracle_merge_partials")
    return out, lse


def sparse_mqa(q, kv, v, win, win_v, win_pos0, win_rows, idx, seq_len, q_pos, sink, *, window: int,
               ratio: int, scale: float, dtype: str):
    B, T, H, D = q.shape
    K = idx.shape[-1]
    qa = _arr(q, dtype)
    kvp, vp, wp, wvp = (_PtrArray(kv, dtype), _PtrArray(v, dtype), _PtrArray(win, dtype),
                        _PtrArray(win_v, dtype))
    ints = [np.ascontiguousarray(x, np.int32) for x in (win_pos0, win_rows, idx, seq_len, q_pos)]
    sk = np.ascontiguousarray(sink, np.float32)
    out, lse = np.empty((B, T, H, D)), np.empty((B, T, H))
    _check(lib().oracle_sparse_mqa(B, T, H, D, K, window, ratio, _dt(dtype), scale, _p(qa), kvp.ptr,
                                   vp.ptr, wp.ptr, wvp.ptr, *[_p(x) for x in ints], _p(sk), _p(out),
                                   _p(lse)), "oracle_sparse_mqa")
    return out, lse


def hca_mqa(q, kv, v, win, win_v, win_pos0, win_rows, seq_len, q_pos, sink, *, window: int,
            ratio: int, scale: float, dtype: str):
    B, T, H, D = q.shape
    qa = _arr(q, dtype)
    kvp, vp, wp, wvp = (_PtrArray(kv, dtype), _PtrArray(v, dtype), _PtrArray(win, dtype),
                        _PtrArray(win_v, dtype))
    ints = [np.ascontiguousarray(x, np.int32) for x in (win_pos0, win_rows, seq_len, q_pos)]
    sk = np.ascontiguousarray(sink, np.float32)
    out, lse = np.empty((B, T, H, D)), np.empty((B, T, H))
    _check(lib().oracle_hca_mqa(B, T, H, D, window, ratio, _dt(dtype), scale, _p(qa), kvp.ptr, vp.ptr,
                                wp.ptr, wvp.ptr, *[_p(x) for x in ints], _p(sk), _p(out), _p(lse)),
           "oracle_hca_mqa")
    return out, lse


def csa_attention(case, *, act: int = ACT_RELU, scale: Optional[float] = None):
    """Whole CSA step on a ``Case`` from the shared input generator.
    Returns (scores, idx, out, lse)."""
    wl = case.wl
    B, T, H, D = case.q.shape
    HI, DI = wl.index_heads, wl.index_dim
    dtype = wl.dtype
    scale = (1.0 / np.sqrt(D)) if scale is None else scale
    n_max = case.max_entries
    qa, qia = _arr(case.q, dtype), _arr(case.q_idx, dtype)
    wa = np.ascontiguousarray(case.w, np.float32)
    kp, kvp, vp = _PtrArray(case.k_idx, dtype), _PtrArray(case.kv, dtype), _PtrArray(case.v, dtype)
    wp, wvp = _PtrArray(case.win, dtype), _PtrArray(case.win_v, dtype)
    ints = [np.ascontiguousarray(x, np.int32) for x in
            (case.win_pos0, case.win_rows, case.seq_len, case.q_pos)]
    sk = np.ascontiguousarray(case.sink, np.float32)
    scores = np.empty((B, T, n_max), np.float32)
    idx = np.empty((B, T, wl.topk), np.int32)
    out, lse = np.empty((B, T, H, D)), np.empty((B, T, H))
    _check(lib().oracle_csa_attention(B, T, H, D, HI, DI, wl.topk, wl.window, wl.ratio, act, _dt(dtype),
                                      scale, _p(qa), _p(qia), _p(wa), kp.ptr, kvp.ptr, vp.ptr, wp.ptr,
                                      wvp.ptr, *[_p(x) for x in ints], _p(sk), n_max, _p(scores),
                                      _p(idx), _p(out), _p(lse)), "oracle_csa_attention")
    return scores, idx, out, lse
