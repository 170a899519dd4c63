"""Pins for the CPU oracle: closed forms, brute force, invariants.

Each test fixes the oracle against something other than itself, so that a
dropped term, a wrong sign, an off-by-one or a transposed operand in
``oracle/oracle.c`` fails at least one of them.  The method's definitions are
those of the "DeepSeek-V4 Architecture Analysis" page (INNOVATIONS section 1,
compressed sparse attention: window, 4:1 / 128:1 compression, indexer with
per-head importance weights, top-k, per-head sink; section 2: K = V) and the
DeepSeek-V4-Flash config table (index_n_heads, index_head_dim, index_topk,
sliding_window).
"""
import itertools
import math

import numpy as np
import pytest

import oracle
from compressed_sparse_attention_indexer_amd import inputs

F32 = "f32"


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------- visibility (a0)

def test_visible_count_matches_span_definition():
    """Entry j spans raw tokens [r*j, r*j+r-1]; it is visible when every token
    of the span is at or before the query (checked token by token here)."""
    for r in (1, 2, 4, 128):
        for L in (0, 1, 3, 4, 5, 17, 128, 300):
            for p in range(0, max(L, 1)):
                if p >= L:
                    continue
                brute = sum(1 for j in range(L // r)
                            if all(t <= p and t < L for t in range(r * j, r * j + r)))
                assert oracle.visible_count(L, p, r) == brute, (r, L, p)


def test_prefill_visible_counts_closed_form():
    """2048 queries at positions 1,046,528..1,048,575 over 262,144 entries:
    counts run from 261,632 to 262,144 and sum to 536,346,112."""
    pos = range(1046528, 1048576)
    counts = [oracle.visible_count(1048576, p, 4) for p in (pos[0], pos[-1])]
    assert counts == [261632, 262144]
    # sum over t of floor((1046529 + t) / 4) = 2048 * 261632 + sum_{u=1}^{2048} floor(u/4)
    closed = 2048 * 261632 + (4 * (511 * 512 // 2) + 512)
    assert closed == 536346112
    sampled = sum(oracle.visible_count(1048576, p, 4) for p in pos[::97])
    assert sampled == sum((p + 1) // 4 for p in pos[::97])


# ----------------------------------------------------------------------------- scores (a1)

def _scores(q_idx, w, k, L=None, p=None, ratio=1, act=oracle.ACT_RELU, n_max=None):
    """Single query helper: q_idx [HI,DI], w [HI], k [N,DI]."""
    N = k.shape[0]
    L = N * ratio if L is None else L
    p = L - 1 if p is None else p
    n_max = N if n_max is None else n_max
    s = oracle.index_scores(q_idx[None, None].astype(np.float32), w[None, None].astype(np.float32),
                            [k.astype(np.float32)], np.array([L]), np.array([p]), ratio=ratio,
                            n_max=n_max, dtype=F32, act=act)
    return s[0, 0]


def test_scores_hand_example():
    """Two heads, two dims, worked by hand:
    head 0 reads dim 0, head 1 reads dim 1; weights 1 and 1/2.
    k0=( 2,-1): relu 2, relu -1 -> 1*2 + 0.5*0 = 2
    k1=(-3, 4): 0 + 0.5*4 = 2;  k2=(1,1): 1 + 0.5 = 1.5;  k3=(-1,-1): 0.
    Without the activation: 1.5, -1, 1.5, -1.5."""
    q = np.array([[1, 0], [0, 1]], np.float32)
    w = np.array([1.0, 0.5], np.float32)
    k = np.array([[2, -1], [-3, 4], [1, 1], [-1, -1]], np.float32)
    assert _scores(q, w, k).tolist() == [2.0, 2.0, 1.5, 0.0]
    assert _scores(q, w, k, act=oracle.ACT_NONE).tolist() == [1.5, -1.0, 1.5, -1.5]


def test_scores_one_head_is_relu_dot():
    rng = _rng(1)
    q = rng.standard_normal((1, 16)).astype(np.float32)
    k = rng.standard_normal((50, 16)).astype(np.float32)
    got = _scores(q, np.ones(1, np.float32), k)
    want = np.maximum(0.0, k.astype(np.float64) @ q[0].astype(np.float64)).astype(np.float32)
    np.testing.assert_array_equal(got, want)


def test_scores_without_activation_fold_the_weights():
    """With no nonlinearity the weighted head sum is one dot product with the
    weight-folded query: s_j = (sum_h w_h q_h) . k_j."""
    rng = _rng(2)
    q = rng.standard_normal((8, 16)).astype(np.float32)
    w = rng.random(8).astype(np.float32)
    k = rng.standard_normal((40, 16)).astype(np.float32)
    got = _scores(q, w, k, act=oracle.ACT_NONE)
    folded = (w.astype(np.float64)[:, None] * q.astype(np.float64)).sum(0)
    np.testing.assert_allclose(got, k.astype(np.float64) @ folded, rtol=1e-6, atol=1e-6)


def test_scores_head_and_dim_orientation():
    """One-hot queries and keys: head h reads only dim h, key j is nonzero
    only on dim j % DI, so each score picks exactly one weight.  A transposed
    query or key indexing breaks the pattern."""
    HI, DI, N = 4, 6, 12
    q = np.zeros((HI, DI), np.float32)
    for h in range(HI):
        q[h, h + 1] = 1.0          # head h looks at dim h+1
    w = np.array([1.0, 2.0, 4.0, 8.0], np.float32)
    k = np.zeros((N, DI), np.float32)
    for j in range(N):
        k[j, j % DI] = 3.0
    got = _scores(q, w, k)
    want = [3.0 * w[(j % DI) - 1] if 1 <= j % DI <= HI else 0.0 for j in range(N)]
    assert got.tolist() == want


def test_scores_invariances():
    rng = _rng(3)
    q = rng.standard_normal((6, 16)).astype(np.float32)
    w = rng.random(6).astype(np.float32)
    k = rng.standard_normal((64, 16)).astype(np.float32)
    base = _scores(q, w, k)
    perm = rng.permutation(6)
    np.testing.assert_allclose(_scores(q[perm], w[perm], k), base, rtol=1e-6)  # head order
    np.testing.assert_array_equal(_scores(q, 2 * w, k), 2 * base)             # exact scaling
    assert (base >= 0).all()


def test_scores_visibility_mask():
    """ratio 4, L = 40 (10 entries), query at position 21: entries whose span
    ends at or before 21 are j <= 4 (span of j=4 is 16..19; j=5 is 20..23)."""
    rng = _rng(4)
    q = rng.standard_normal((2, 8)).astype(np.float32)
    k = rng.standard_normal((10, 8)).astype(np.float32)
    s = _scores(q, np.ones(2, np.float32), k, L=40, p=21, ratio=4, n_max=12)
    assert np.isfinite(s[:5]).all() and np.isneginf(s[5:]).all()
    s = _scores(q, np.ones(2, np.float32), k, L=40, p=23, ratio=4, n_max=12)
    assert np.isfinite(s[:6]).all() and np.isneginf(s[6:]).all()


# ----------------------------------------------------------------------------- top-k (a2)

def _topk1(s, k, L=None, p=None, ratio=1):
    n = s.shape[0]
    L = n * ratio if L is None else L
    p = L - 1 if p is None else p
    return oracle.topk(s[None, None].astype(np.float32), np.array([L]), np.array([p]),
                       ratio=ratio, k=k)[0, 0]


def _brute_topk(s, k):
    """O(N^2) rank counting: j is kept iff fewer than k entries beat it, where
    i beats j when s_i > s_j or (s_i == s_j and i < j)."""
    n = len(s)
    keep = [j for j in range(n)
            if sum(1 for i in range(n) if s[i] > s[j] or (s[i] == s[j] and i < j)) < k]
    return keep + [-1] * (k - len(keep))


@pytest.mark.parametrize("seed,n,k", [(0, 7, 3), (1, 64, 16), (2, 300, 32), (3, 513, 512),
                                      (4, 40, 64), (5, 1, 1), (6, 200, 1)])
def test_topk_brute_force(seed, n, k):
    rng = _rng(seed)
    s = rng.standard_normal(n).astype(np.float32)
    s[rng.integers(0, n, n // 3)] = s[rng.integers(0, n, n // 3)]  # plenty of exact ties
    if n > 4:
        s[: n // 4] = 0.5
    assert _topk1(s, k).tolist() == _brute_topk(s.tolist(), k)


def test_topk_textbook_sort():
    """numpy lexsort by (-score, index), first k, sorted ascending."""
    rng = _rng(7)
    s = np.round(rng.standard_normal(5000), 1).astype(np.float32)  # many ties
    order = np.lexsort((np.arange(len(s)), -s.astype(np.float64)))
    want = np.sort(order[:512])
    np.testing.assert_array_equal(_topk1(s, 512), want)


def test_topk_ties_go_to_lower_index():
    s = np.array([1, 3, 3, 2, 3, 3], np.float32)
    assert _topk1(s, 3).tolist() == [1, 2, 4]
    assert _topk1(s, 1).tolist() == [1]
    assert _topk1(np.zeros(5, np.float32), 2).tolist() == [0, 1]


def test_topk_invariants_and_padding():
    rng = _rng(8)
    s = rng.standard_normal(1000).astype(np.float32)
    sel = _topk1(s, 100)
    assert (np.diff(sel) > 0).all()
    rest = np.setdiff1d(np.arange(1000), sel)
    assert s[sel].min() >= s[rest].max()
    np.testing.assert_array_equal(_topk1(2.5 * s, 100), sel)          # positive scaling
    perm = rng.permutation(1000)                                      # equivariance (no ties)
    np.testing.assert_array_equal(np.sort(perm[_topk1(s[perm], 100)]), sel)
    short = _topk1(s[:10], 16)
    assert short[:10].tolist() == list(range(10)) and short[10:].tolist() == [-1] * 6


def test_topk_only_visible_entries():
    """Scores of entries that are not visible are never selected, whatever
    their value (ratio 4, L=40, p=21: only j<=4 visible)."""
    s = np.arange(12, dtype=np.float32)[::-1].copy()
    s[6:] = 100.0
    sel = _topk1(s, 3, L=40, p=21, ratio=4)
    assert sel.tolist() == [0, 1, 2]


# ----------------------------------------------------------------------------- attention (a3, a4)

def _att(q, rows, vrows=None, sink=None, scale=1.0):
    return oracle.attend_rows(np.asarray(q, np.float32), np.asarray(rows, np.float32),
                              None if vrows is None else np.asarray(vrows, np.float32),
                              None if sink is None else np.asarray(sink, np.float32),
                              scale=scale, dtype=F32)


def test_attention_single_row_is_sigmoid_gate():
    """One row with logit z and a sink s: weight sigma(z - s) on its value."""
    q = np.array([[0.5, 0.25, 0.0, 1.0]])
    k = np.array([[1.0, 2.0, 3.0, 0.25]])         # q.k = 0.5 + 0.5 + 0 + 0.25 = 1.25
    v = np.array([[2.0, -1.0, 4.0, 8.0]])
    sink = np.array([-0.5], np.float32)
    out, lse = _att(q, k, v, sink, scale=0.5)     # z = 0.625
    z, s = 0.625, float(sink[0])
    np.testing.assert_allclose(out[0], v[0] / (1.0 + math.exp(s - z)), rtol=1e-12)
    np.testing.assert_allclose(lse[0], math.log(math.exp(z) + math.exp(s)), rtol=1e-12)


def test_attention_zero_query_uniform_with_sink():
    """q = 0: every logit is 0, so each of the n rows gets 1/(n + e^sink)."""
    rng = _rng(9)
    n, D = 7, 5
    rows = rng.standard_normal((n, D)).astype(np.float32)
    vrows = rng.standard_normal((n, D)).astype(np.float32).astype(np.float64)
    sink = np.array([0.3, -2.0], np.float32)
    out, lse = _att(np.zeros((2, D)), rows, vrows, sink)
    for h in range(2):
        den = n + math.exp(float(sink[h]))
        np.testing.assert_allclose(out[h], vrows.sum(0) / den, rtol=1e-12)
        np.testing.assert_allclose(lse[h], math.log(den), rtol=1e-12)


def test_attention_constant_values_and_sink_mass():
    """Every value row equal to c gives (1 - p_sink) c with p_sink = e^(sink - lse)."""
    rng = _rng(10)
    H, n, D = 3, 11, 6
    q, rows = rng.standard_normal((H, D)), rng.standard_normal((n, D))
    c = rng.standard_normal(D).astype(np.float32).astype(np.float64)
    sink = rng.standard_normal(H).astype(np.float32)
    out, lse = _att(q, rows, np.tile(c, (n, 1)), sink, scale=0.7)
    for h in range(H):
        p_sink = math.exp(float(sink[h]) - lse[h])
        assert 0 < p_sink < 1
        np.testing.assert_allclose(out[h], (1 - p_sink) * c, rtol=1e-12, atol=1e-14)


def test_attention_probabilities_from_one_hot_values():
    """With value row i = e_i the output row is the probability vector; it must
    equal exp(z_i - lse) with z_i = scale * q.k_i and, with the sink's share,
    sum to one."""
    rng = _rng(11)
    H, n, D, scale = 4, 9, 12, 0.37
    q, rows = rng.standard_normal((H, D)), rng.standard_normal((n, D))
    vrows = np.eye(n, D)
    sink = rng.standard_normal(H).astype(np.float32)
    out, lse = _att(q, rows, vrows, sink, scale=scale)
    z = scale * (q.astype(np.float32).astype(np.float64) @ rows.astype(np.float32).astype(np.float64).T)
    np.testing.assert_allclose(out[:, :n], np.exp(z - lse[:, None]), rtol=1e-12)
    np.testing.assert_allclose(out[:, :n].sum(1) + np.exp(sink.astype(np.float64) - lse), 1.0, rtol=1e-12)
    assert (out[:, n:] == 0).all()


def test_attention_two_rows_no_sink():
    q = np.array([[1.0, 0.0]])
    rows = np.array([[2.0, 0.0], [0.0, 5.0]])      # z = 2, 0
    vrows = np.array([[1.0, 0.0], [0.0, 1.0]])
    out, lse = _att(q, rows, vrows, None)
    e = math.exp(2.0)
    np.testing.assert_allclose(out[0], [e / (e + 1), 1 / (e + 1)], rtol=1e-12)
    np.testing.assert_allclose(lse[0], math.log(e + 1), rtol=1e-12)


def test_attention_values_default_to_keys():
    rng = _rng(12)
    q, rows = rng.standard_normal((2, 8)), rng.standard_normal((5, 8))
    a = _att(q, rows, None, np.zeros(2))
    b = _att(q, rows, rows, np.zeros(2))
    np.testing.assert_array_equal(a[0], b[0])


def test_merge_of_partials_equals_whole():
    """Split the rows into random parts, attend to each part without the sink,
    merge with the sink: same as attending to all rows at once."""
    rng = _rng(13)
    H, n, D = 5, 60, 16
    q, rows, vrows = (rng.standard_normal(s) * 2 for s in ((H, D), (n, D), (n, D)))
    sink = rng.standard_normal(H).astype(np.float32)
    whole, lse = _att(q, rows, vrows, sink, scale=0.5)
    for parts in (1, 2, 7):
        cuts = np.sort(rng.choice(np.arange(1, n), parts - 1, replace=False)) if parts > 1 else []
        bounds = [0, *cuts, n]
        ms, ls, os_ = [], [], []
        for a, b in zip(bounds[:-1], bounds[1:]):
            m, l, o = oracle.partial_rows(q.astype(np.float32), rows[a:b].astype(np.float32),
                                          vrows[a:b].astype(np.float32), scale=0.5, dtype=F32)
            ms.append(m), ls.append(l), os_.append(o)
        # an empty part must be harmless
        ms.append(np.full(H, -np.inf)), ls.append(np.zeros(H)), os_.append(np.zeros((H, D)))
        out, lse2 = oracle.merge_partials(np.array(ms), np.array(ls), np.array(os_), sink)
        np.testing.assert_allclose(out, whole, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse2, lse, rtol=1e-12)


# ----------------------------------------------------------------------------- row sets of the sparse / HCA paths

def _tagged_case(L=64, ratio=4, W=8, K=5, D=64, p=None, H=2):
    """Compressed rows and window rows whose values are one-hot tags, a zero
    query (uniform weights) and no sink: the output row shows exactly which
    rows were attended."""
    p = L - 1 if p is None else p
    N = L // ratio
    kv = np.zeros((N, D), np.float32)
    for j in range(N):
        kv[j, j] = 1.0
    pos0, nrow = max(0, p - W + 1), p - max(0, p - W + 1) + 1
    win = np.zeros((nrow, D), np.float32)
    for t in range(nrow):
        win[t, N + t] = 1.0
    q = np.zeros((1, 1, H, D), np.float32)
    sink = np.full(H, -np.inf, np.float32)
    return dict(q=q, kv=[kv], win=[win], pos0=np.array([pos0]), nrow=np.array([nrow]),
                L=np.array([L]), p=np.array([p]), sink=sink, N=N)


def test_sparse_rows_are_selected_then_window():
    c = _tagged_case()
    idx = np.array([[[1, 4, 9, 15, -1]]], np.int32)
    out, _ = oracle.sparse_mqa(c["q"], c["kv"], None, c["win"], None, c["pos0"], c["nrow"], idx, c["L"],
                               c["p"], c["sink"], window=8, ratio=4, scale=1.0, dtype=F32)
    n = 4 + 8
    want = np.zeros(64)
    want[[1, 4, 9, 15]] = 1.0 / n
    want[c["N"]:c["N"] + 8] = 1.0 / n     # raw positions 56..63
    np.testing.assert_allclose(out[0, 0, 0], want, rtol=1e-12)


def test_window_is_last_w_positions_including_query():
    """Query at position 13 of a 64-token buffer with W=8: raw positions 6..13."""
    c = _tagged_case(p=13, L=64)
    W = 8
    # window buffer covering positions 0..20, tagged by position
    win = np.zeros((21, 64), np.float32)
    for t in range(21):
        win[t, 30 + t] = 1.0
    idx = np.full((1, 1, 3), -1, np.int32)
    idx[0, 0, 0] = 2                       # entry 2 spans 8..11 (visible at 13)
    out, _ = oracle.sparse_mqa(c["q"], c["kv"], None, [win], None, np.array([0]), np.array([21]), idx,
                               c["L"], c["p"], c["sink"], window=W, ratio=4, scale=1.0, dtype=F32)
    got = np.nonzero(out[0, 0, 0])[0].tolist()
    assert got == [2] + [30 + t for t in range(6, 14)]


def test_sparse_rejects_invisible_index_and_short_window():
    c = _tagged_case(p=21, L=64)
    idx = np.array([[[5, -1, -1, -1, -1]]], np.int32)   # entry 5 spans 20..23, not visible at 21
    with pytest.raises(oracle.OracleError):
        oracle.sparse_mqa(c["q"], c["kv"], None, c["win"], None, c["pos0"], c["nrow"], idx, c["L"],
                          c["p"], c["sink"], window=8, ratio=4, scale=1.0, dtype=F32)
    idx[0, 0, 0] = 2
    with pytest.raises(oracle.OracleError):   # window buffer starting one position too late
        oracle.sparse_mqa(c["q"], c["kv"], None, c["win"], None, c["pos0"] + 1, c["nrow"], idx, c["L"],
                          c["p"], c["sink"], window=8, ratio=4, scale=1.0, dtype=F32)


def test_hca_rows_are_all_visible_entries_then_window():
    c = _tagged_case(L=64, p=45, ratio=4)   # 11 visible entries (spans up to 40..43)
    out, _ = oracle.hca_mqa(c["q"], c["kv"], None, c["win"], None, c["pos0"], c["nrow"], c["L"], c["p"],
                            c["sink"], window=8, ratio=4, scale=1.0, dtype=F32)
    got = np.nonzero(out[0, 0, 0])[0].tolist()
    assert got == list(range(11)) + [c["N"] + t for t in range(8)]


def test_sparse_with_all_entries_equals_hca():
    rng = _rng(14)
    B, H, D, L, W, r = 2, 3, 16, 96, 8, 4
    N = L // r
    q = rng.standard_normal((B, 1, H, D)).astype(np.float32)
    kv = [rng.standard_normal((N, D)).astype(np.float32) for _ in range(B)]
    v = [rng.standard_normal((N, D)).astype(np.float32) for _ in range(B)]
    win = [rng.standard_normal((W, D)).astype(np.float32) for _ in range(B)]
    args = (np.full(B, L - W), np.full(B, W))
    sink = rng.standard_normal(H).astype(np.float32)
    Ls, ps = np.full(B, L), np.full(B, L - 1)
    idx = np.tile(np.arange(N, dtype=np.int32), (B, 1, 1))
    a = oracle.sparse_mqa(q, kv, v, win, None, *args, idx, Ls, ps, sink, window=W, ratio=r, scale=0.25,
                          dtype=F32)
    b = oracle.hca_mqa(q, kv, v, win, None, *args, Ls, ps, sink, window=W, ratio=r, scale=0.25, dtype=F32)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-12)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-12)


# ----------------------------------------------------------------------------- whole step, tiny sizes

def _dense_brute(case):
    """A second route for the whole step on tiny inputs: dense masked softmax.
    Scores by einsum, top-k by rank counting, attention as one softmax over
    [all compressed rows | window rows | sink column] with -inf on compressed
    rows that were not selected."""
    wl = case.wl
    f = lambda x: inputs.as_float64(x, wl.dtype)
    B, T, H, D = case.q.shape
    scale = 1.0 / math.sqrt(D)
    outs, lses = np.zeros((B, T, H, D)), np.zeros((B, T, H))
    for b, t in itertools.product(range(B), range(T)):
        p = int(case.q_pos[b * T + t])
        N = int(case.seq_len[b]) // wl.ratio
        nv = min(N, (p + 1) // wl.ratio)
        dots = np.einsum("hd,jd->hj", f(case.q_idx[b, t]), f(case.k_idx[b]))
        s = (case.w[b, t].astype(np.float64)[:, None] * np.maximum(dots, 0)).sum(0).astype(np.float32)
        keep = _brute_topk(s[:nv].tolist(), wl.topk)
        keep = [j for j in keep if j >= 0]
        lo = max(0, p - wl.window + 1)
        wrows = f(case.win[b])[lo - case.win_pos0[b]: p - case.win_pos0[b] + 1]
        wvals = wrows if case.win_v is None else f(case.win_v[b])[lo - case.win_pos0[b]: p - case.win_pos0[b] + 1]
        K = f(case.kv[b])
        V = K if case.v is None else f(case.v[b])
        allk, allv = np.concatenate([K, wrows]), np.concatenate([V, wvals])
        z = scale * f(case.q[b, t]) @ allk.T                     # [H, N + nwin]
        mask = np.full(z.shape[1], -np.inf)
        mask[keep] = 0.0
        mask[N:] = 0.0
        z = z + mask
        zs = np.concatenate([z, case.sink.astype(np.float64)[:, None]], axis=1)
        pr = np.exp(zs - zs.max(1, keepdims=True))
        pr /= pr.sum(1, keepdims=True)
        outs[b, t] = pr[:, :-1] @ allv
        lses[b, t] = zs.max(1) + np.log(np.exp(zs - zs.max(1, keepdims=True)).sum(1))
    return outs, lses


@pytest.mark.parametrize("L,K", [(512, 32), (160, 64), (64, 8)])
def test_whole_step_against_dense_brute_force(L, K):
    wl = inputs.scaled(inputs.WORKLOADS["fixture_b2_l512_fp32"], f"tiny_{L}_{K}", seq_len=L, topk=K)
    case = inputs.make_case(wl)
    _, _, out, lse = oracle.csa_attention(case)
    want, want_lse = _dense_brute(case)
    np.testing.assert_allclose(out, want, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(lse, want_lse, rtol=1e-12, atol=1e-12)


def _causal_multi_query_case(seed=31):
    """Two sequences of ragged raw lengths (70 and 53), six queries each at
    distinct positions (causal visibility, as in a prefill chunk): one query
    sees no compressed entry (p = 2), several see fewer than K, and the two
    sequences' positions differ, so every query indexes its own sequence's
    caches, position, window and visible count.  The window buffers hold every
    raw row of their sequence."""
    base = inputs.WORKLOADS["fixture_b2_l512_fp32"]
    B, T, H, D, HI, DI, K, W, r = 2, 6, 4, 16, 4, 16, 5, 8, 4
    wl = inputs.scaled(base, "tiny_causal_b2_t6", q_len=T, topk=K, window=W, seq_len=None,
                       seq_len_range=(53, 70), q_pos0=0)
    g = _rng(seed)
    L = np.array([70, 53], np.int32)
    q_pos = np.array([20, 33, 34, 47, 60, 69, 2, 11, 12, 30, 44, 52], np.int32)
    nrm = lambda *shape: (g.standard_normal(shape) / math.sqrt(shape[-1])).astype(np.float32)
    return inputs.Case(
        wl=wl, seq_len=L, q_pos=q_pos,
        q=nrm(B, T, H, D), q_idx=nrm(B, T, HI, DI), w=g.random((B, T, HI)).astype(np.float32),
        k_idx=[nrm(int(n) // r, DI) for n in L], kv=[nrm(int(n) // r, D) for n in L],
        v=[nrm(int(n) // r, D) for n in L], win=[nrm(int(n), D) for n in L], win_v=[nrm(int(n), D) for n in L],
        win_pos0=np.zeros(B, np.int32), win_rows=L.copy(), sink=g.standard_normal(H).astype(np.float32))


def test_multi_query_causal_scores_topk_and_attention_against_dense_brute():
    """Several queries per sequence (T > 1) at their own positions: scores by
    einsum with the causal mask, top-k by rank counting, attention by the dense
    masked softmax, each query against its own sequence (b = query // T) and
    its own position."""
    case = _causal_multi_query_case()
    wl = case.wl
    B, T = wl.batch, wl.q_len
    n_max = case.max_entries
    scores = oracle.index_scores(case.q_idx, case.w, case.k_idx, case.seq_len, case.q_pos, ratio=wl.ratio,
                                 n_max=n_max, dtype=F32)
    idx = oracle.topk(scores, case.seq_len, case.q_pos, ratio=wl.ratio, k=wl.topk)
    nvis = []
    for b, t in itertools.product(range(B), range(T)):
        p = int(case.q_pos[b * T + t])
        nv = min(int(case.seq_len[b]) // wl.ratio, (p + 1) // wl.ratio)
        nvis.append(nv)
        dots = np.einsum("hd,jd->hj", case.q_idx[b, t].astype(np.float64), case.k_idx[b][:nv].astype(np.float64))
        want = (case.w[b, t].astype(np.float64)[:, None] * np.maximum(dots, 0)).sum(0)
        np.testing.assert_allclose(scores[b, t, :nv], want, rtol=1e-6)
        assert np.isneginf(scores[b, t, nv:]).all()
        assert idx[b, t].tolist() == _brute_topk(scores[b, t, :nv].tolist(), wl.topk)
    assert 0 in nvis and any(0 < n < wl.topk for n in nvis) and max(nvis) > wl.topk
    s2, idx2, out, lse = oracle.csa_attention(case)
    np.testing.assert_array_equal(s2, scores)
    np.testing.assert_array_equal(idx2, idx)
    want, want_lse = _dense_brute(case)
    np.testing.assert_allclose(out, want, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(lse, want_lse, rtol=1e-12, atol=1e-12)


def test_multi_query_hca_against_dense_brute():
    """The dense (HCA) path with T > 1: every visible entry of the query's own
    sequence at its own position, then its window, in one softmax with the sink."""
    case = _causal_multi_query_case(32)
    wl = case.wl
    B, T, H, D = case.q.shape
    out, lse = oracle.hca_mqa(case.q, case.kv, case.v, case.win, case.win_v, case.win_pos0, case.win_rows,
                              case.seq_len, case.q_pos, case.sink, window=wl.window, ratio=wl.ratio,
                              scale=0.25, dtype=F32)
    for b, t in itertools.product(range(B), range(T)):
        p = int(case.q_pos[b * T + t])
        nv = min(int(case.seq_len[b]) // wl.ratio, (p + 1) // wl.ratio)
        lo = max(0, p - wl.window + 1)
        keys = np.concatenate([case.kv[b][:nv], case.win[b][lo:p + 1]]).astype(np.float64)
        vals = np.concatenate([case.v[b][:nv], case.win_v[b][lo:p + 1]]).astype(np.float64)
        z = 0.25 * case.q[b, t].astype(np.float64) @ keys.T
        zs = np.concatenate([z, case.sink.astype(np.float64)[:, None]], axis=1)
        pr = np.exp(zs - zs.max(1, keepdims=True))
        np.testing.assert_allclose(out[b, t], (pr[:, :-1] @ vals) / pr.sum(1, keepdims=True), rtol=1e-9,
                                   atol=1e-12)
        np.testing.assert_allclose(lse[b, t], zs.max(1) + np.log(pr.sum(1)), rtol=1e-12)


def test_fixture_golden_file_matches():
    """The stored fixture outputs were written by tests/golden/make_golden.py
    (which calls only the oracle); a change of the oracle's arithmetic shows
    here."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "fixture_b2_l512_fp32.json")
    g = json.load(open(path))
    case = inputs.make_case(inputs.WORKLOADS["fixture_b2_l512_fp32"])
    scores, idx, out, lse = oracle.csa_attention(case)
    assert idx.tolist() == g["topk_idx"]
    np.testing.assert_array_equal(scores, np.array(g["scores"], np.float32))
    np.testing.assert_allclose(out, np.array(g["out"]), rtol=1e-12)
    np.testing.assert_allclose(lse, np.array(g["lse"]), rtol=1e-12)


# --------------------------------------------------------------------------- fp8 index tensors (E4M3)

@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0), (0x3F, 1.875),
    (0x40, 2.0), (0x77, 240.0), (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0), (0x81, -(2.0 ** -9)),
])
def test_e4m3_decode_matches_format_table(code, value):
    """OCP E4M3: bias 7, 3 mantissa bits, subnormals m * 2^-9, largest finite 448."""
    assert oracle.e4m3_value(code) == value


def test_e4m3_special_codes():
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))
    z = oracle.e4m3_value(0x80)
    assert z == 0.0 and math.copysign(1.0, z) == -1.0


def test_e4m3_round_trip_of_the_input_encoder():
    """Every finite code decodes to a value the encoder maps back to that code."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], np.uint8)
    vals = np.array([oracle.e4m3_value(int(c)) for c in codes])
    np.testing.assert_array_equal(inputs.e4m3_codes(vals), codes)


def _fp8_case(seed, B=2, T=1, HI=3, DI=8, N=11):
    r = np.random.default_rng(seed)
    q8 = r.integers(0, 256, size=(B, T, HI, DI)).astype(np.uint8)
    q8[(q8 & 0x7F) == 0x7F] = 0x38  # no NaN codes
    k8 = [r.integers(0, 256, size=(N, DI)).astype(np.uint8) for _ in range(B)]
    for k in k8:
        k[(k & 0x7F) == 0x7F] = 0x30
    w = r.random((B, T, HI)).astype(np.float32)
    seq = np.array([4 * N] * B, np.int32)
    return q8, w, k8, seq


def test_fp8_scores_with_unit_scales_equal_the_bf16_definition():
    """E4M3 values are exact in bf16: with all scales 1 the fp8 scores are the
    bf16 scores of the decoded values, bit for bit."""
    q8, w, k8, seq = _fp8_case(3)
    B, T, HI, DI = q8.shape
    dec = np.vectorize(oracle.e4m3_value)
    qv = dec(q8).astype(np.float32)
    kv = [dec(k).astype(np.float32) for k in k8]
    ones_q = np.ones((B, T, HI), np.float32)
    ones_k = [np.ones(len(k), np.float32) for k in k8]
    got = oracle.index_scores_fp8(q8, ones_q, w, k8, ones_k, seq, seq - 1, ratio=4, n_max=11)
    want = oracle.index_scores(inputs.bf16_bits(qv), w, [inputs.bf16_bits(k) for k in kv], seq, seq - 1,
                               ratio=4, n_max=11, dtype="bf16")
    np.testing.assert_array_equal(got, want)


def test_fp8_row_scales_act_per_entry_and_per_head():
    """A power-of-two key scale multiplies exactly that entry's score; a query
    scale on head h acts like the same factor on w_h (ReLU commutes with
    positive scaling)."""
    q8, w, k8, seq = _fp8_case(4)
    B, T, HI, DI = q8.shape
    r = np.random.default_rng(5)
    qs = r.uniform(0.5, 2.0, (B, T, HI)).astype(np.float32)
    ks = [r.uniform(0.5, 2.0, len(k)).astype(np.float32) for k in k8]
    base = oracle.index_scores_fp8(q8, qs, w, k8, ks, seq, seq - 1, ratio=4, n_max=11)
    ks2 = [k.copy() for k in ks]
    ks2[1][7] *= 4.0
    s2 = oracle.index_scores_fp8(q8, qs, w, k8, ks2, seq, seq - 1, ratio=4, n_max=11)
    want = base.copy()
    want[1, 0, 7] *= 4.0
    np.testing.assert_array_equal(s2, want)
    qs3, w3 = qs.copy(), w.copy()
    qs3[0, 0, 1] *= 2.0
    w3[0, 0, 1] *= 2.0
    a = oracle.index_scores_fp8(q8, qs3, w, k8, ks, seq, seq - 1, ratio=4, n_max=11)
    b = oracle.index_scores_fp8(q8, qs, w3, k8, ks, seq, seq - 1, ratio=4, n_max=11)
    np.testing.assert_allclose(a, b, rtol=1e-6)


# --------------------------------------------------------------------------- compressor (R8-R12)

def _comp_inputs(seed, tokens=24, hidden=32, out_dim=16, window=8):
    r = np.random.default_rng(seed)
    x = inputs.bf16_bits(r.standard_normal((tokens, hidden)).astype(np.float32) * 0.5)
    wkv = inputs.bf16_bits(r.standard_normal((out_dim, hidden)).astype(np.float32) * 0.2)
    wg = inputs.bf16_bits(r.standard_normal((out_dim, hidden)).astype(np.float32) * 0.2)
    ape = r.standard_normal((window, out_dim)).astype(np.float32)
    gamma = r.uniform(0.5, 1.5, out_dim).astype(np.float32)
    return x, wkv, wg, ape, gamma


def _f64(b):
    return inputs.bf16_to_f32(b).astype(np.float64)


def _rms_norm(c, gamma, eps=1e-6):
    return c / np.sqrt(np.mean(c ** 2) + eps) * gamma


def test_compress_uniform_gates_is_mean_pooling():
    """Zero gate weights and embeddings make the softmax uniform: an entry is
    RMSNorm(wkv . mean of its window's tokens), a matrix-vector product."""
    x, wkv, _, _, gamma = _comp_inputs(1)
    out = oracle.compress(x, wkv, np.zeros_like(wkv), np.zeros((8, 16), np.float32), gamma, pos0=0, ratio=4,
                          window=8, first_entry=1, n_entries=4)
    for i, e in enumerate(range(1, 5)):
        want = _rms_norm(_f64(wkv) @ _f64(x)[4 * e - 4:4 * e + 4].mean(0), gamma)
        np.testing.assert_allclose(out[i], want, rtol=1e-12, atol=1e-12)


def test_compress_first_entry_has_no_tokens_before_zero():
    """Entry 0 of an overlapping 2r window only has tokens 0..r-1."""
    x, wkv, _, _, gamma = _comp_inputs(2)
    out = oracle.compress(x, wkv, np.zeros_like(wkv), np.zeros((8, 16), np.float32), gamma, pos0=0, ratio=4,
                          window=8, first_entry=0, n_entries=1)
    np.testing.assert_allclose(out[0], _rms_norm(_f64(wkv) @ _f64(x)[0:4].mean(0), gamma), rtol=1e-12)


def test_compress_dominant_slot_selects_one_token():
    """A huge position embedding at slot 5 of the window puts all the weight on that token."""
    x, wkv, wg, _, gamma = _comp_inputs(3)
    ape = np.zeros((8, 16), np.float32)
    ape[5] = 1e4
    out = oracle.compress(x, wkv, wg, ape, gamma, pos0=0, ratio=4, window=8, first_entry=2, n_entries=2)
    for i, e in enumerate((2, 3)):
        t = 4 * e + 4 - 8 + 5
        np.testing.assert_allclose(out[i], _rms_norm(_f64(wkv) @ _f64(x)[t], gamma), rtol=1e-9)


def test_compress_hca_window_is_the_span_itself():
    """Without overlap (window = ratio) an entry pools exactly its own r tokens."""
    x, wkv, _, _, gamma = _comp_inputs(4, tokens=32)
    out = oracle.compress(x, wkv, np.zeros_like(wkv), np.zeros((8, 16), np.float32), gamma, pos0=0, ratio=8,
                          window=8, first_entry=2, n_entries=1)
    np.testing.assert_allclose(out[0], _rms_norm(_f64(wkv) @ _f64(x)[16:24].mean(0), gamma), rtol=1e-12)


def test_compress_rope_rotates_pairs_by_position():
    """Identical tokens give every entry the same pre-RoPE vector; the rope
    slice of entry e is that vector's pairs rotated by (r e) theta^(-2k/R),
    the other dims untouched."""
    x, wkv, wg, ape, gamma = _comp_inputs(5)
    x[:] = x[0]
    base = oracle.compress(x, wkv, wg, ape, gamma, pos0=0, ratio=4, window=8, first_entry=2, n_entries=3)
    rot = oracle.compress(x, wkv, wg, ape, gamma, pos0=0, ratio=4, window=8, first_entry=2, n_entries=3,
                          rope_dims=8, rope_theta=160000.0)
    np.testing.assert_array_equal(rot[:, :8], base[:, :8])
    for i, e in enumerate((2, 3, 4)):
        for k in range(4):
            ang = 4 * e * 160000.0 ** (-2.0 * k / 8)
            a, b = base[i, 8 + 2 * k], base[i, 9 + 2 * k]
            np.testing.assert_allclose(rot[i, 8 + 2 * k], a * math.cos(ang) - b * math.sin(ang), rtol=1e-12, atol=1e-15)
            np.testing.assert_allclose(rot[i, 9 + 2 * k], a * math.sin(ang) + b * math.cos(ang), rtol=1e-12, atol=1e-15)


def test_compress_output_has_unit_rms_with_unit_gamma():
    x, wkv, wg, ape, _ = _comp_inputs(6)
    out = oracle.compress(x, wkv, wg, ape, np.ones(16, np.float32), pos0=0, ratio=4, window=8, first_entry=1,
                          n_entries=4, rope_dims=8)
    np.testing.assert_allclose(np.sqrt(np.mean(out ** 2, axis=1)), 1.0, atol=1e-4)


def test_compress_hadamard_is_the_normalized_sylvester_matrix():
    from scipy.linalg import hadamard
    x, wkv, wg, ape, gamma = _comp_inputs(7)
    plain = oracle.compress(x, wkv, wg, ape, gamma, pos0=0, ratio=4, window=8, first_entry=1, n_entries=3)
    rot = oracle.compress(x, wkv, wg, ape, gamma, pos0=0, ratio=4, window=8, first_entry=1, n_entries=3,
                          hadamard=True)
    np.testing.assert_allclose(rot, plain @ (hadamard(16) / 4.0).T, rtol=1e-12, atol=1e-14)


def _one_hot_tokens(n_tokens, hidden):
    x = np.zeros((n_tokens, hidden), np.float32)
    x[np.arange(n_tokens), np.arange(n_tokens)] = 1.0
    return inputs.bf16_bits(x)


def test_compress_gate_term_weights_the_tokens():
    """Two one-hot tokens and no position embeddings: token t's projection is
    column t of wkv and its gate logit column t of wgate, so per dim d the pooled
    value is sigma(g0 - g1) kv0 + sigma(g1 - g0) kv1 with g = wgate[d, t], here
    different per dim (a per-dim softmax, not one shared by all dims)."""
    hidden, out_dim = 32, 16
    g = _rng(40)
    x = _one_hot_tokens(2, hidden)
    wkv = inputs.bf16_bits(g.standard_normal((out_dim, hidden)).astype(np.float32))
    wg = np.zeros((out_dim, hidden), np.float32)
    wg[:, 0] = np.arange(out_dim) % 5 - 2.0       # gate logit of token 0, per dim: -2 .. 2
    wg[:, 1] = -0.5 * (np.arange(out_dim) % 3)    # token 1: 0, -0.5, -1
    wg = inputs.bf16_bits(wg)
    gamma = g.uniform(0.5, 1.5, out_dim).astype(np.float32)
    out = oracle.compress(x, wkv, wg, np.zeros((2, out_dim), np.float32), gamma, pos0=0, ratio=2, window=2,
                          first_entry=0, n_entries=1)
    g0, g1 = _f64(wg)[:, 0], _f64(wg)[:, 1]
    p0 = 1.0 / (1.0 + np.exp(g1 - g0))
    c = p0 * _f64(wkv)[:, 0] + (1.0 - p0) * _f64(wkv)[:, 1]
    np.testing.assert_allclose(out[0], _rms_norm(c, gamma), rtol=1e-12, atol=1e-14)


def test_compress_gate_adds_the_position_embedding():
    """With both terms present the logit of token t in window slot i is
    wgate x_t + ape[i] (a sum): tokens 4..7 of an overlapping 8-token window
    (slots 4..7), one-hot, so entry 1's weights are a softmax of
    wgate[d, t] + ape[t, d] over t = 0..7 (entry 1 pools tokens 0..7)."""
    hidden, out_dim = 32, 8
    g = _rng(41)
    x = _one_hot_tokens(8, hidden)
    wkv = inputs.bf16_bits(g.standard_normal((out_dim, hidden)).astype(np.float32))
    wg = inputs.bf16_bits(g.standard_normal((out_dim, hidden)).astype(np.float32))
    ape = g.standard_normal((8, out_dim)).astype(np.float32)
    out = oracle.compress(x, wkv, wg, ape, np.ones(out_dim, np.float32), pos0=0, ratio=4, window=8,
                          first_entry=1, n_entries=1)
    logit = _f64(wg)[:, :8] + ape.astype(np.float64).T          # [d, t]
    p = np.exp(logit - logit.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    c = (p * _f64(wkv)[:, :8]).sum(1)
    np.testing.assert_allclose(out[0], _rms_norm(c, np.ones(out_dim)), rtol=1e-12, atol=1e-14)


def test_compress_rejects_windows_not_supplied():
    x, wkv, wg, ape, gamma = _comp_inputs(8)
    with pytest.raises(RuntimeError):
        oracle.compress(x, wkv, wg, ape, gamma, pos0=4, ratio=4, window=8, first_entry=0, n_entries=1)
