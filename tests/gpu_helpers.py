"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same host inputs, and compare under the stated rules."""
import math
import sys

import numpy as np

import oracle
from compressed_sparse_attention_indexer_amd import inputs

# Attention outputs: max |gpu - oracle| <= 1e-2 * RMS(oracle) over the tensor
# (bf16 inputs, fp32 accumulation).  fp32 inputs are held to 1e-4.
ATT_TOL_BF16 = 1e-2
ATT_TOL_F32 = 1e-4
# Top-k: sets equal except for entries whose fp32 oracle score lies within
# 1e-3 (relative) of the oracle's K-th score.
TOPK_BAND = 1e-3
# Scores: fp32 accumulation of exact bf16 products vs float64 rounded to fp32.
SCORE_TOL = 1e-4


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def nvis_of(case, bt, ratio=None):
    wl = case.wl
    r = wl.ratio if ratio is None else ratio
    b = bt // wl.q_len
    return min(int(case.seq_len[b]) // r, (int(case.q_pos[bt]) + 1) // r)


def assert_scores_close(gpu, ora, case, tol=SCORE_TOL):
    """gpu/ora [B,T,n_max]; visible entries within tol * RMS of the row's
    visible scores; invisible entries exactly -inf in both."""
    B, T, n_max = ora.shape
    for bt in range(B * T):
        b, t = divmod(bt, T)
        nv = nvis_of(case, bt)
        g, o = gpu[b, t], ora[b, t]
        assert np.isneginf(o[nv:]).all() and np.isneginf(g[nv:]).all(), f"query {bt}: masked tail"
        if nv == 0:
            continue
        rms = float(np.sqrt(np.mean(o[:nv].astype(np.float64) ** 2))) or 1.0
        err = float(np.max(np.abs(g[:nv].astype(np.float64) - o[:nv])))
        assert err <= tol * rms, f"query {bt}: score err {err:.3e} > {tol:.0e} * rms {rms:.3e}"


def check_topk_valid(idx, nvis, K):
    """Ascending, unique, in range, -1 padding only at the end, size min(K, nvis)."""
    sel = idx[idx >= 0]
    assert len(sel) == min(K, nvis), (len(sel), K, nvis)
    assert (idx[len(sel):] == -1).all()
    assert (np.diff(sel) > 0).all()
    if len(sel):
        assert sel[0] >= 0 and sel[-1] < nvis


def assert_topk_band(gpu_idx, ora_idx, ora_scores, case, band=TOPK_BAND):
    """Per query: GPU set equals the oracle set except for entries within the
    band around the oracle's K-th score."""
    B, T, K = ora_idx.shape
    n_diff = 0
    for bt in range(B * T):
        b, t = divmod(bt, T)
        nv = nvis_of(case, bt)
        gi, oi = gpu_idx[b, t], ora_idx[b, t]
        check_topk_valid(gi, nv, K)
        A, Bs = set(gi[gi >= 0].tolist()), set(oi[oi >= 0].tolist())
        if nv <= K:
            assert A == Bs == set(range(nv))
            continue
        s = ora_scores[b, t]
        s_star = float(min(s[j] for j in Bs))
        for j in A ^ Bs:
            assert abs(float(s[j]) - s_star) <= band * abs(s_star), \
                f"query {bt}: entry {j} score {s[j]} vs k-th {s_star}"
        n_diff += len(A ^ Bs)
    return n_diff


def assert_attention_close(gpu, ora, tol, what=""):
    gpu = np.asarray(gpu, np.float64)
    rms = float(np.sqrt(np.mean(np.square(ora))))
    err = float(np.max(np.abs(gpu - ora)))
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    assert err <= tol * rms, f"{what}: max err {err:.3e} > {tol:.0e} * rms {rms:.3e}"
    return err / rms


def oracle_sparse(case, idx, scale=None):
    wl = case.wl
    D = wl.head_dim
    return oracle.sparse_mqa(case.q, case.kv, case.v, case.win, case.win_v, case.win_pos0, case.win_rows, idx,
                             case.seq_len, case.q_pos, case.sink, window=wl.window, ratio=wl.ratio,
                             scale=1.0 / math.sqrt(D) if scale is None else scale, dtype=wl.dtype)


def oracle_hca(case):
    wl = case.wl
    return oracle.hca_mqa(case.hca_q, case.hca_kv, None, case.hca_win, None, case.win_pos0, case.win_rows,
                          case.seq_len, case.q_pos, case.hca_sink, window=wl.window, ratio=wl.hca_ratio,
                          scale=1.0 / math.sqrt(wl.head_dim), dtype=wl.dtype)


def oracle_scores(case, act=oracle.ACT_RELU):
    wl = case.wl
    return oracle.index_scores(case.q_idx, case.w, case.k_idx, case.seq_len, case.q_pos, ratio=wl.ratio,
                               n_max=max(1, case.max_entries), dtype=wl.dtype, act=act)


def flash_case(name, seq_lens, *, batch=None, q_len=1, q_pos0=None, topk=512, window=128, hca=None, index=101):
    """A Flash-shaped bf16 workload with given raw lengths (seeded like the others)."""
    base = inputs.WORKLOADS["decode_b1_64k"]
    seq_lens = list(seq_lens)
    wl = inputs.scaled(base, name, index=index, batch=len(seq_lens) if batch is None else batch, q_len=q_len,
                       seq_len=None, seq_len_range=None, topk=topk, window=window, q_pos0=q_pos0, hca_ratio=hca)
    return wl, np.array(seq_lens, np.int32)


def make_case_with_lens(wl, seq_lens):
    return inputs.make_case(wl, seq_lens=seq_lens)


def query_subset(case, ts):
    """The same inputs restricted to queries ts of a single-sequence case (the
    oracle then evaluates only those queries)."""
    import dataclasses
    assert case.wl.batch == 1
    ts = np.asarray(ts)
    wl = dataclasses.replace(case.wl, q_len=len(ts))
    return dataclasses.replace(case, wl=wl, q_pos=case.q_pos[ts].copy(), q=case.q[:, ts].copy(),
                               q_idx=case.q_idx[:, ts].copy(), w=case.w[:, ts].copy())
