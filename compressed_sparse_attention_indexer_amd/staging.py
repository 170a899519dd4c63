"""Copy a host ``inputs.Case`` into device memory (torch tensors) and build the
device pointer arrays and size structs the C ABI takes.  Plumbing only."""
from __future__ import annotations

import math
from typing import List, Optional

import numpy as np

from . import CSA_BF16, CSA_F32, make_dims, ptr_array
from .inputs import Case


def _dev(x: np.ndarray, dtype: str, device):
    import torch
    if dtype == "bf16" and x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def _devs(xs: Optional[List[np.ndarray]], dtype: str, device):
    return None if xs is None else [_dev(x, dtype, device) for x in xs]


class DeviceCase:
    """Device-resident copy of a Case with pointer arrays ready for the ABI."""

    def __init__(self, case: Case, device="cuda"):
        import torch
        wl = case.wl
        dt = wl.dtype
        self.case, self.wl, self.device = case, wl, device
        self.seq_len = torch.from_numpy(case.seq_len).to(device)
        self.q_pos = torch.from_numpy(case.q_pos).to(device)
        self.win_pos0 = torch.from_numpy(case.win_pos0).to(device)
        self.win_rows = torch.from_numpy(case.win_rows).to(device)
        self.q = _dev(case.q, dt, device)
        self.q_idx = _dev(case.q_idx, dt, device)
        self.w = _dev(case.w, "f32", device)
        self.sink = _dev(case.sink, "f32", device)
        self.k_idx = _devs(case.k_idx, dt, device)
        self.kv = _devs(case.kv, dt, device)
        self.v = _devs(case.v, dt, device)
        self.win = _devs(case.win, dt, device)
        self.win_v = _devs(case.win_v, dt, device)
        self.k_idx_p, self.kv_p, self.v_p, self.win_p, self.win_v_p = (
            ptr_array(x, device) for x in (self.k_idx, self.kv, self.v, self.win, self.win_v))
        self.has_hca = case.hca_q is not None
        if self.has_hca:
            self.hca_q = _dev(case.hca_q, dt, device)
            self.hca_kv = _devs(case.hca_kv, dt, device)
            self.hca_win = _devs(case.hca_win, dt, device)
            self.hca_sink = _dev(case.hca_sink, "f32", device)
            self.hca_kv_p, self.hca_win_p = ptr_array(self.hca_kv, device), ptr_array(self.hca_win, device)

    def csa_dims(self, **over):
        wl = self.wl
        kw = dict(batch=wl.batch, q_len=wl.q_len, n_heads=wl.n_heads, head_dim=wl.head_dim,
                  index_heads=wl.index_heads, index_dim=wl.index_dim, topk=wl.topk, window=wl.window,
                  ratio=wl.ratio, max_entries=max(1, self.case.max_entries),
                  dtype=CSA_BF16 if wl.dtype == "bf16" else CSA_F32)
        kw.update(over)
        return make_dims(**kw)

    def hca_dims(self, **over):
        ratio = self.wl.hca_ratio
        n_max = max(1, int((self.case.seq_len // ratio).max()))
        return self.csa_dims(ratio=ratio, max_entries=n_max, **over)
