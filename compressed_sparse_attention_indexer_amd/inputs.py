"""Seeded synthetic inputs for the CSA/HCA decode path.

This module only draws and lays out numbers; it holds none of the method's
arithmetic (no scores, no selection, no softmax).  The HIP path and the CPU
oracle both consume exactly the bytes produced here.

Workload shapes follow the DeepSeek-V4-Flash attention description
(llm-atlas DeepSeek-V4-Flash page, raw config.json table: head_dim 512,
num_attention_heads 64, num_key_value_heads 1, index_n_heads 64,
index_head_dim 128, index_topk 512, sliding_window 128; the open-deepseek-v4
architecture_analysis.py page, ARCHITECTURE_SPEC "csa_ratio" 4 and
"hca_ratio" 128).  The fixture workload mirrors the shrunken-model idea of the
DeepSeek-V4-Flash-0731 coverage report (4 query heads, head_dim 16).

Recipe (every tensor is independent of generation order):
  * numpy ``Generator(PCG64(SeedSequence([seed, tensor_id, seq, chunk])))``,
    ``seed = 12345 + workload index``.
  * q, kv, v, window rows ~ N(0,1)/sqrt(D); q_idx, k_idx ~ N(0,1)/sqrt(DI);
    importance weights ~ U(0,1); sink ~ N(0,1).
  * float32 draws are rounded to bfloat16 with round-to-nearest-even; the
    bf16 tensors are kept as their uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

# tensor ids (fixed, so no draw depends on the order of generation)
_TID = {
    "q": 1, "q_idx": 2, "w": 3, "k_idx": 4, "kv": 5, "v": 6, "win": 7,
    "sink": 8, "seq_len": 9, "win_v": 10,
    "hca_q": 11, "hca_kv": 12, "hca_win": 13, "hca_sink": 14,
    "q8": 15, "k8": 16,
    "cx": 17, "wkv": 18, "wgate": 19, "ape": 20, "gamma": 21,
}
_ROW_CHUNK = 65536  # rows per independently seeded chunk of a per-sequence cache


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one synthetic workload."""
    name: str
    index: int               # seed = 12345 + index
    batch: int
    q_len: int               # query tokens per sequence (1 = decode)
    n_heads: int
    head_dim: int
    index_heads: int
    index_dim: int
    topk: int
    window: int
    ratio: int
    dtype: str               # "f32" or "bf16"
    seq_len: Optional[int]   # fixed raw length, or None for ragged draws
    seq_len_range: Optional[tuple] = None   # inclusive [lo, hi] for ragged draws
    separate_v: bool = False
    q_pos0: Optional[int] = None            # first query position (prefill chunk)
    hca_ratio: Optional[int] = None         # paired HCA layer (dense, no indexer)

    @property
    def seed(self) -> int:
        return 12345 + self.index


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("fixture_b2_l512_fp32", 0, batch=2, q_len=1, n_heads=4, head_dim=16,
                 index_heads=4, index_dim=16, topk=32, window=16, ratio=4, dtype="f32",
                 seq_len=512, separate_v=True),
        Workload("decode_b1_64k", 1, batch=1, q_len=1, n_heads=64, head_dim=512,
                 index_heads=64, index_dim=128, topk=512, window=128, ratio=4, dtype="bf16",
                 seq_len=65536),
        Workload("decode_b32_ragged_64k_128k", 2, batch=32, q_len=1, n_heads=64, head_dim=512,
                 index_heads=64, index_dim=128, topk=512, window=128, ratio=4, dtype="bf16",
                 seq_len=None, seq_len_range=(65536, 131072)),
        Workload("decode_b4_1m", 3, batch=4, q_len=1, n_heads=64, head_dim=512,
                 index_heads=64, index_dim=128, topk=512, window=128, ratio=4, dtype="bf16",
                 seq_len=1048576, hca_ratio=128),
        Workload("prefill_t2048_1m", 4, batch=1, q_len=2048, n_heads=64, head_dim=512,
                 index_heads=64, index_dim=128, topk=512, window=128, ratio=4, dtype="bf16",
                 seq_len=1048576, q_pos0=1046528),
        # V4-Pro attention shape (128 query heads, top-1024) on the million-token batch
        Workload("pro_decode_b4_1m", 5, batch=4, q_len=1, n_heads=128, head_dim=512,
                 index_heads=64, index_dim=128, topk=1024, window=128, ratio=4, dtype="bf16",
                 seq_len=1048576),
    ]
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def scaled(base: Workload, name: str, **changes) -> Workload:
    """A variant of a workload with some fields replaced (test sizes)."""
    return dataclasses.replace(base, name=name, **changes)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *key])))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit pattern (uint16) -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(shape, scale: float, dtype: str, seed: int, *key: int) -> np.ndarray:
    x = _rng(seed, *key).standard_normal(size=shape, dtype=np.float32)
    x *= np.float32(scale)
    return bf16_bits(x) if dtype == "bf16" else x


def _rows(n_rows: int, dim: int, scale: float, dtype: str, seed: int, tid: int, seq: int) -> np.ndarray:
    """A per-sequence [n_rows, dim] cache, drawn in independently seeded row chunks."""
    out = np.empty((n_rows, dim), dtype=np.uint16 if dtype == "bf16" else np.float32)
    for c0 in range(0, n_rows, _ROW_CHUNK):
        c1 = min(n_rows, c0 + _ROW_CHUNK)
        out[c0:c1] = _normal((c1 - c0, dim), scale, dtype, seed, tid, seq, c0 // _ROW_CHUNK)
    return out


@dataclasses.dataclass
class Case:
    """All inputs of one workload, host-resident (numpy)."""
    wl: Workload
    seq_len: np.ndarray            # [B] int32 raw lengths
    q_pos: np.ndarray              # [B*T] int32 query positions
    q: np.ndarray                  # [B,T,H,D]
    q_idx: np.ndarray              # [B,T,HI,DI]
    w: np.ndarray                  # [B,T,HI] float32
    k_idx: List[np.ndarray]        # B x [N_b, DI]
    kv: List[np.ndarray]           # B x [N_b, D]
    v: Optional[List[np.ndarray]]  # B x [N_b, D] or None (V = K)
    win: List[np.ndarray]          # B x [win_rows_b, D]
    win_v: Optional[List[np.ndarray]]  # B x [win_rows_b, D] or None (V = K)
    win_pos0: np.ndarray           # [B] int32
    win_rows: np.ndarray           # [B] int32
    sink: np.ndarray               # [H] float32
    # paired HCA layer (dense over all ratio-128 entries), when the workload has one
    hca_q: Optional[np.ndarray] = None
    hca_kv: Optional[List[np.ndarray]] = None
    hca_win: Optional[List[np.ndarray]] = None
    hca_sink: Optional[np.ndarray] = None

    @property
    def n_entries(self) -> np.ndarray:
        return self.seq_len // self.wl.ratio

    @property
    def max_entries(self) -> int:
        return int(self.n_entries.max())


def draw_seq_lens(wl: Workload) -> np.ndarray:
    if wl.seq_len is not None:
        return np.full(wl.batch, wl.seq_len, dtype=np.int32)
    lo, hi = wl.seq_len_range
    return _rng(wl.seed, _TID["seq_len"]).integers(lo, hi, size=wl.batch, endpoint=True).astype(np.int32)


def query_positions(wl: Workload, seq_len: np.ndarray) -> np.ndarray:
    B, T = wl.batch, wl.q_len
    if wl.q_pos0 is None:  # decode: the query is the newest token of each sequence
        assert T == 1
        return (seq_len - 1).astype(np.int32)
    pos = np.empty(B * T, dtype=np.int32)
    for b in range(B):
        pos[b * T:(b + 1) * T] = wl.q_pos0 + np.arange(T, dtype=np.int32)
        assert pos[(b + 1) * T - 1] < seq_len[b]
    return pos


def window_span(wl: Workload, seq_len: np.ndarray, q_pos: np.ndarray):
    """Raw rows each sequence keeps for the sliding window: from the earliest
    window start of its queries to its last query position."""
    B, T, W = wl.batch, wl.q_len, wl.window
    pos0 = np.empty(B, dtype=np.int32)
    rows = np.empty(B, dtype=np.int32)
    for b in range(B):
        p = q_pos[b * T:(b + 1) * T]
        lo = max(0, int(p.min()) - W + 1)
        pos0[b] = lo
        rows[b] = int(p.max()) - lo + 1
    return pos0, rows


def make_case(wl: Workload, with_hca: bool = True, seq_lens=None) -> Case:
    """Draw every tensor of a workload; `seq_lens` overrides the raw lengths."""
    s = wl.seed
    B, T, H, D, HI, DI = wl.batch, wl.q_len, wl.n_heads, wl.head_dim, wl.index_heads, wl.index_dim
    seq_len = draw_seq_lens(wl) if seq_lens is None else np.asarray(seq_lens, dtype=np.int32).copy()
    assert seq_len.shape == (B,)
    q_pos = query_positions(wl, seq_len)
    n_ent = seq_len // wl.ratio
    pos0, rows = window_span(wl, seq_len, q_pos)
    sd, si = 1.0 / math.sqrt(D), 1.0 / math.sqrt(DI)
    case = Case(
        wl=wl, seq_len=seq_len, q_pos=q_pos,
        q=_normal((B, T, H, D), sd, wl.dtype, s, _TID["q"]),
        q_idx=_normal((B, T, HI, DI), si, wl.dtype, s, _TID["q_idx"]),
        w=_rng(s, _TID["w"]).random(size=(B, T, HI), dtype=np.float32),
        k_idx=[_rows(int(n_ent[b]), DI, si, wl.dtype, s, _TID["k_idx"], b) for b in range(B)],
        kv=[_rows(int(n_ent[b]), D, sd, wl.dtype, s, _TID["kv"], b) for b in range(B)],
        v=([_rows(int(n_ent[b]), D, sd, wl.dtype, s, _TID["v"], b) for b in range(B)]
           if wl.separate_v else None),
        win=[_rows(int(rows[b]), D, sd, wl.dtype, s, _TID["win"], b) for b in range(B)],
        win_v=([_rows(int(rows[b]), D, sd, wl.dtype, s, _TID["win_v"], b) for b in range(B)]
               if wl.separate_v else None),
        win_pos0=pos0, win_rows=rows,
        sink=_rng(s, _TID["sink"]).standard_normal(size=H, dtype=np.float32),
    )
    if with_hca and wl.hca_ratio is not None:
        n_h = seq_len // wl.hca_ratio
        case.hca_q = _normal((B, T, H, D), sd, wl.dtype, s, _TID["hca_q"])
        case.hca_kv = [_rows(int(n_h[b]), D, sd, wl.dtype, s, _TID["hca_kv"], b) for b in range(B)]
        case.hca_win = [_rows(int(rows[b]), D, sd, wl.dtype, s, _TID["hca_win"], b) for b in range(B)]
        case.hca_sink = _rng(s, _TID["hca_sink"]).standard_normal(size=H, dtype=np.float32)
    return case


def as_float64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of a drawn tensor (bf16 bits or float32)."""
    return (bf16_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)).astype(np.float64)


# ---------------------------------------------------------------- fp8 (OCP E4M3) index tensors
# Input preparation for the fp8 indexer: float draws are stored as E4M3 codes
# with one float32 scale per row (amax / 448), codes rounded to nearest even
# and saturated at the largest finite value.  The path only ever reads codes
# and scales.

def _e4m3_table() -> np.ndarray:
    """Values of the non-negative finite codes 0..126, ascending."""
    c = np.arange(127)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e.astype(np.float64) - 7))


def e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float -> E4M3 code (uint8): round to nearest, ties to even code, saturating."""
    t = _e4m3_table()
    a = np.minimum(np.abs(np.asarray(x, np.float64)), t[-1])
    hi = np.clip(np.searchsorted(t, a), 1, 126)
    lo = hi - 1
    dl, dh = a - t[lo], t[hi] - a
    pick = np.where(dl < dh, lo, np.where(dh < dl, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a == 0, 0, pick)
    sign = (np.signbit(np.asarray(x)) & (pick != 0)).astype(np.uint8) << 7
    return (pick.astype(np.uint8) | sign).astype(np.uint8)


def quantize_rows_e4m3(x: np.ndarray):
    """x [..., D] float -> (codes [..., D] uint8, scale [...] float32), scale = amax / 448."""
    x = np.asarray(x, np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    return e4m3_codes(x / scale[..., None]), scale


def make_fp8_index(case: "Case"):
    """fp8 index tensors for a case's shapes, drawn like q_idx / k_idx: returns
    (q8 [B,T,HI,DI], q_scale [B,T,HI], k8: B x [N_b,DI], k_scale: B x [N_b])."""
    wl = case.wl
    B, T, HI, DI = wl.batch, wl.q_len, wl.index_heads, wl.index_dim
    si = 1.0 / math.sqrt(DI)
    qf = _normal((B, T, HI, DI), si, "f32", wl.seed, _TID["q8"])
    q8, qs = quantize_rows_e4m3(qf)
    k8, ks = [], []
    for b in range(B):
        c, sc = quantize_rows_e4m3(_rows(int(case.n_entries[b]), DI, si, "f32", wl.seed, _TID["k8"], b))
        k8.append(c)
        ks.append(sc)
    return q8, qs, k8, ks


# ---------------------------------------------------------------- compressor inputs

def make_compressor_inputs(seed: int, tokens: int, hidden: int, out_dim: int, window: int):
    """Hidden states x [tokens, hidden] ~ N(0,1) and synthetic weights: wkv, wgate
    ~ N(0,1)/sqrt(hidden) (bf16 bits), ape ~ N(0, 0.5^2), gamma ~ U(0.5, 1.5)."""
    sh = 1.0 / math.sqrt(hidden)
    x = _normal((tokens, hidden), 1.0, "bf16", seed, _TID["cx"])
    wkv = _normal((out_dim, hidden), sh, "bf16", seed, _TID["wkv"])
    wgate = _normal((out_dim, hidden), sh, "bf16", seed, _TID["wgate"])
    ape = _normal((window, out_dim), 0.5, "f32", seed, _TID["ape"])
    gamma = _rng(seed, _TID["gamma"]).uniform(0.5, 1.5, size=out_dim).astype(np.float32)
    return x, wkv, wgate, ape, gamma
