"""ctypes loader for libcsa.so (the C ABI declared in include/csa.h).

Loading needs no GPU; calls that pass argument checks enqueue HIP kernels.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcsa.so")

CSA_OK, CSA_ERR_NULL, CSA_ERR_DIM, CSA_ERR_ALIGN, CSA_ERR_UNSUPPORTED, CSA_ERR_WORKSPACE, CSA_ERR_HIP = range(7)
CSA_F32, CSA_BF16 = 0, 1
CSA_ACT_RELU, CSA_ACT_NONE = 0, 1
CSA_OP_INDEX_SCORES, CSA_OP_TOPK, CSA_OP_SPARSE_MQA, CSA_OP_HCA_MQA, CSA_OP_ATTENTION, CSA_OP_ATTENTION_FP8 = range(6)

# every symbol include/csa.h declares
EXPORTS = ("csa_workspace_size", "csa_index_scores", "csa_index_scores_fp8", "csa_topk_select",
           "csa_sparse_mqa_decode", "hca_mqa_decode", "csa_attention", "csa_attention_fp8", "csa_attention_noalloc",
           "csa_compress_workspace_size", "csa_compress", "csa_status_string", "csa_last_error", "csa_abi_version")


class CsaDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_len", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("index_heads", ctypes.c_int32), ("index_dim", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("window", ctypes.c_int32), ("ratio", ctypes.c_int32),
                ("max_entries", ctypes.c_int32), ("dtype", ctypes.c_int32), ("index_act", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]


class CsaCompressDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("tokens", "hidden", "out_dim", "ratio", "window", "rope_dims",
                                               "hadamard", "first_entry", "n_entries", "pos0")] + \
               [("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float)]


class CsaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libcsa.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m compressed_sparse_attention_indexer_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    DP = ctypes.POINTER(CsaDims)
    L.csa_abi_version.restype = I32
    L.csa_last_error.restype = ctypes.c_char_p
    L.csa_status_string.restype = ctypes.c_char_p
    L.csa_status_string.argtypes = [I32]
    L.csa_workspace_size.argtypes = [DP, I32, ctypes.POINTER(SZ)]
    L.csa_index_scores.argtypes = [DP, P, P, P, P, P, P, P, SZ, P]
    L.csa_index_scores_fp8.argtypes = [DP] + [P] * 9
    L.csa_topk_select.argtypes = [DP, P, P, P, P, P, SZ, P]
    L.csa_sparse_mqa_decode.argtypes = [DP] + [P] * 13 + [P, SZ, P]
    L.hca_mqa_decode.argtypes = [DP] + [P] * 12 + [P, SZ, P]
    L.csa_attention.argtypes = [DP] + [P] * 17 + [P, SZ, P]
    L.csa_attention_fp8.argtypes = [DP] + [P] * 19 + [P, SZ, P]
    L.csa_attention_noalloc.argtypes = [DP] + [P] * 17 + [P]
    CP = ctypes.POINTER(CsaCompressDims)
    L.csa_compress_workspace_size.argtypes = [CP, ctypes.POINTER(SZ)]
    L.csa_compress.argtypes = [CP] + [P] * 7 + [SZ, P]
    for f in ("csa_workspace_size", "csa_index_scores", "csa_index_scores_fp8", "csa_topk_select",
              "csa_sparse_mqa_decode", "hca_mqa_decode", "csa_attention", "csa_attention_fp8",
              "csa_attention_noalloc", "csa_compress_workspace_size", "csa_compress"):
        getattr(L, f).restype = I32
    _lib = L
    return L


def check(status: int, where: str):
    if status != CSA_OK:
        L = load_library()
        raise CsaError(status, where, f"{L.csa_status_string(status).decode()} ({L.csa_last_error().decode()})")
