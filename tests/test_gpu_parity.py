"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Rules: top-k computed from the same fp32 scores is bit-exact; top-k from the
GPU's own scores matches the oracle's set except inside the 1e-3 band around
the K-th score; attention outputs are within 1e-2 x RMS of the oracle (bf16
inputs), evaluated on the GPU's own selected set so that legal near-tie swaps
do not count; scores are within 1e-4 x RMS of the row.
"""
import math

import numpy as np
import pytest

import oracle
from compressed_sparse_attention_indexer_amd import inputs
from tests.gpu_helpers import (ATT_TOL_BF16, ATT_TOL_F32, SCORE_TOL, assert_attention_close, assert_scores_close,
                               assert_topk_band, check_topk_valid, flash_case, make_case_with_lens, nvis_of,
                               oracle_hca, oracle_scores, oracle_sparse, query_subset, say)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import compressed_sparse_attention_indexer_amd as csa  # noqa: E402
from compressed_sparse_attention_indexer_amd.staging import DeviceCase  # noqa: E402


# a ragged batch of 12: long and short sequences, one with fewer visible
# entries than K, one with none
RAGGED_12 = [4 * 30000 + 1, 4 * 2000, 4 * 90 + 3, 50, 4 * 12000 + 2, 4 * 64000, 4 * 700 + 1, 4 * 5000 + 3,
             4 * 40000, 4 * 1500 + 2, 4 * 300, 4 * 20000 + 1]


def _np(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def run_fused_t(dc, act=csa.CSA_ACT_RELU):
    """csa_attention with the intermediate scores and indices exposed (device tensors)."""
    dims = dc.csa_dims(index_act=act)
    scores = torch.empty((dims.batch, dims.q_len, dims.max_entries), dtype=torch.float32, device="cuda")
    idx = torch.empty((dims.batch, dims.q_len, dims.topk), dtype=torch.int32, device="cuda")
    out, lse = csa.csa_attention(dims, dc.q, dc.q_idx, dc.w, dc.k_idx_p, dc.kv_p, dc.v_p, dc.win_p, dc.win_v_p,
                                 dc.win_pos0, dc.win_rows, dc.seq_len, dc.q_pos, dc.sink, topk_idx_out=idx,
                                 scores_out=scores)
    torch.cuda.synchronize()
    return scores, idx, out, lse


def run_fused(dc, act=csa.CSA_ACT_RELU):
    """csa_attention with the intermediate scores and indices exposed."""
    dims = dc.csa_dims(index_act=act)
    Q = dims.batch * dims.q_len
    scores = torch.empty((dims.batch, dims.q_len, dims.max_entries), dtype=torch.float32, device="cuda")
    idx = torch.empty((dims.batch, dims.q_len, dims.topk), dtype=torch.int32, device="cuda")
    out, lse = csa.csa_attention(dims, dc.q, dc.q_idx, dc.w, dc.k_idx_p, dc.kv_p, dc.v_p, dc.win_p, dc.win_v_p,
                                 dc.win_pos0, dc.win_rows, dc.seq_len, dc.q_pos, dc.sink, topk_idx_out=idx,
                                 scores_out=scores)
    assert Q == dc.case.q_pos.shape[0]
    return _np(scores), _np(idx), _np(out), _np(lse)


def check_whole_step(case, tol, act=csa.CSA_ACT_RELU):
    say(f"[case] {case.wl.name} B={case.wl.batch} T={case.wl.q_len} max_entries={case.max_entries}")
    dc = DeviceCase(case)
    g_scores, g_idx, g_out, g_lse = run_fused(dc, act)
    o_scores = oracle_scores(case, act=oracle.ACT_NONE if act == csa.CSA_ACT_NONE else oracle.ACT_RELU)
    assert_scores_close(g_scores, o_scores, case)
    o_idx = oracle.topk(o_scores, case.seq_len, case.q_pos, ratio=case.wl.ratio, k=case.wl.topk)
    n_diff = assert_topk_band(g_idx, o_idx, o_scores, case)
    # the top-k kernel alone, fed the oracle's scores: bit-exact
    dims = dc.csa_dims()
    t_idx = _np(csa.csa_topk_select(dims, torch.from_numpy(o_scores).cuda(), dc.seq_len, dc.q_pos))
    np.testing.assert_array_equal(t_idx, o_idx)
    # attention on the GPU's own selection
    o_out, o_lse = oracle_sparse(case, g_idx)
    rel = assert_attention_close(g_out, o_out, tol, "out")
    np.testing.assert_allclose(g_lse, o_lse, atol=1e-3, rtol=0)
    say(f"  ok: topk band swaps={n_diff} out err/rms={rel:.2e}")
    return dc


# --------------------------------------------------------------------------- fixture (fp32)

def test_fixture_fp32_whole_step():
    case = inputs.make_case(inputs.WORKLOADS["fixture_b2_l512_fp32"])
    check_whole_step(case, ATT_TOL_F32)


def test_fixture_fp32_no_activation():
    case = inputs.make_case(inputs.WORKLOADS["fixture_b2_l512_fp32"])
    check_whole_step(case, ATT_TOL_F32, act=csa.CSA_ACT_NONE)


# --------------------------------------------------------------------------- Flash shapes, small

@pytest.mark.parametrize("lens", [
    [4 * 1000 + 3, 4 * 257, 130],        # several scorer steps, ragged tails
    [4 * 3000, 4 * 700 + 1],             # n_vis > K: real selection
    [50, 2, 4 * 128 + 2],                # L < W, p < 3 (nothing compressed), n_vis < K
])
def test_flash_whole_step_small(lens):
    wl, sl = flash_case(f"flash_small_{len(lens)}_{lens[0]}", lens)
    check_whole_step(make_case_with_lens(wl, sl), ATT_TOL_BF16)


@pytest.mark.parametrize("lens,T,q_pos0", [
    ([4 * 9000 + 1, 4 * 3000 + 2], 1, None),     # decode: several splits and the combine
    ([4 * 2500 + 3], 24, 4 * 2500 + 3 - 30),     # a few queries of a prefill chunk
])
def test_separate_value_rows(lens, T, q_pos0):
    """Value rows apart from the key rows (compressed cache and window): the
    attention kernel's separate-value instance against the oracle."""
    import dataclasses
    wl, sl = flash_case(f"flash_sepv_{T}", lens, q_len=T, q_pos0=q_pos0)
    check_whole_step(make_case_with_lens(dataclasses.replace(wl, separate_v=True), sl), ATT_TOL_BF16)


@pytest.mark.parametrize("vmax,sharp", [(6e4, False), (6e4, True), (1e6, False), (1e-6, False), (1e-6, True)])
def test_value_rows_across_the_range(vmax, sharp):
    """Split partials O/l are kept in fp16, each head's values of a dim half
    scaled by a power of two into [2^14, 2^15).  Value rows scaled so that
    max |v| is about 6e4 (near fp16's largest), 1e6 (past it) and 1e-6 (where
    unscaled fp16 would be subnormal), with sharp logits too (single rows
    dominating, so that O/l reaches those values): still within the bf16
    attention tolerance of the oracle."""
    import dataclasses
    wl, sl = flash_case(f"flash_vrange_{vmax:g}_{int(sharp)}", [4 * 9000 + 1, 4 * 3000 + 2])
    case = make_case_with_lens(dataclasses.replace(wl, separate_v=True), sl)
    cur = max(float(np.max(np.abs(inputs.bf16_to_f32(x)))) for x in case.v + case.win_v)
    s = np.float32(vmax / cur)
    case.v = [inputs.bf16_bits(inputs.bf16_to_f32(x) * s) for x in case.v]
    case.win_v = [inputs.bf16_bits(inputs.bf16_to_f32(x) * s) for x in case.win_v]
    got = max(float(np.max(np.abs(inputs.bf16_to_f32(x)))) for x in case.v + case.win_v)
    assert 0.9 * vmax < got < 1.1 * vmax
    if sharp:
        case.q = inputs.bf16_bits(inputs.bf16_to_f32(case.q) * np.float32(60.0))
    check_whole_step(case, ATT_TOL_BF16)


@pytest.mark.parametrize("sharp", [False, True])
def test_value_rows_with_two_large_dims(sharp):
    """One dim in each half of the value rows eight times larger than the
    others (up to about 6e4, near fp16's largest value): the power of two of a
    head's dim half must come from the largest magnitude over all of its 256
    dims (one taken from part of them overflows the large dim, or leaves lanes
    of one head with different scales).  The ratio is kept at 8: the fp16
    partials round each value to 2^-11 of its head's largest, which against a
    bound of 1e-2 times the output's RMS allows a largest-to-RMS ratio of
    about 20, not a few dims carrying all of the output."""
    import dataclasses
    wl, sl = flash_case(f"flash_vdims_{int(sharp)}", [4 * 9000 + 1, 4 * 3000 + 2])
    case = make_case_with_lens(dataclasses.replace(wl, separate_v=True), sl)
    cur = max(float(np.max(np.abs(inputs.bf16_to_f32(x)))) for x in case.v + case.win_v)
    col = np.full(wl.head_dim, np.float32(6e4 / 8 / cur), dtype=np.float32)
    col[37] = col[300] = np.float32(6e4 / cur)
    case.v = [inputs.bf16_bits(inputs.bf16_to_f32(x) * col) for x in case.v]
    case.win_v = [inputs.bf16_bits(inputs.bf16_to_f32(x) * col) for x in case.win_v]
    if sharp:
        case.q = inputs.bf16_bits(inputs.bf16_to_f32(case.q) * np.float32(60.0))
    check_whole_step(case, ATT_TOL_BF16)


def test_flash_no_activation():
    wl, sl = flash_case("flash_noact", [4 * 2000, 4 * 900])
    check_whole_step(make_case_with_lens(wl, sl), ATT_TOL_BF16, act=csa.CSA_ACT_NONE)


def test_flash_exact_ties_in_scores():
    """Duplicated index keys give exact score ties across the K-th boundary."""
    wl, sl = flash_case("flash_ties", [4 * 4096])
    case = make_case_with_lens(wl, sl)
    k = case.k_idx[0]
    k[1::3] = k[0:-1:3][: len(k[1::3])]
    k[2::3] = k[0:-2:3][: len(k[2::3])]
    check_whole_step(case, ATT_TOL_BF16)


def test_flash_sharp_logits_and_sink():
    """q scaled so logits spread over several units and a large sink: exercises
    the running max, the rescaling and the sink merge."""
    wl, sl = flash_case("flash_sharp", [4 * 3000, 4 * 1500])
    case = make_case_with_lens(wl, sl)
    q = inputs.bf16_to_f32(case.q) * np.float32(60.0)
    case.q = inputs.bf16_bits(q)
    case.sink = (case.sink * 2 + np.float32(math.log(640))).astype(np.float32)
    check_whole_step(case, ATT_TOL_BF16)


# --------------------------------------------------------------------------- tensor-level calls

def test_tensor_level_attention_on_a_side_stream():
    """csa.attention with sizes taken from the tensors and keyword options, on
    a stream other than the current one (its temporaries and outputs are made
    on that stream), against the oracle: the selected sets under the band rule,
    attention on the GPU's own set."""
    wl, sl = flash_case("flash_tensor_api", [4 * 9000 + 1, 4 * 3000 + 2, 4 * 100 + 3])
    case = make_case_with_lens(wl, sl)
    say(f"[case] {wl.name} tensor-level attention on a side stream")
    dc = DeviceCase(case)
    side = torch.cuda.Stream()
    out, lse, idx = csa.attention(dc.q, dc.q_idx, dc.w, dc.k_idx, dc.kv, dc.win, case.seq_len.tolist(), dc.q_pos,
                                  dc.sink, topk=wl.topk, window=wl.window, ratio=wl.ratio, stream=side)
    side.synchronize()
    g_idx, g_out, g_lse = idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
    o_scores = oracle_scores(case)
    o_idx = oracle.topk(o_scores, case.seq_len, case.q_pos, ratio=wl.ratio, k=wl.topk)
    assert_topk_band(g_idx, o_idx, o_scores, case)
    o_out, o_lse = oracle_sparse(case, g_idx)
    assert_attention_close(g_out, o_out, ATT_TOL_BF16, "out")
    np.testing.assert_allclose(g_lse, o_lse, atol=1e-3, rtol=0)


def test_tensor_level_ops_match_the_abi_calls():
    """csa.index_scores, csa.topk, csa.sparse_mqa and csa.hca_mqa give the same
    results as the struct-based calls they marshal to."""
    wl, sl = flash_case("flash_tensor_ops", [4 * 5000 + 2, 128 * 37 + 5], hca=128)
    case = make_case_with_lens(wl, sl)
    say(f"[case] {wl.name} tensor-level ops")
    dc = DeviceCase(case)
    dims = dc.csa_dims()
    s_ref = csa.csa_index_scores(dims, dc.q_idx, dc.w, dc.k_idx_p, dc.seq_len, dc.q_pos)
    s = csa.index_scores(dc.q_idx, dc.w, dc.k_idx, dc.seq_len, dc.q_pos, ratio=wl.ratio)
    np.testing.assert_array_equal(_np(s), _np(s_ref))
    i_ref = csa.csa_topk_select(dims, s_ref, dc.seq_len, dc.q_pos)
    i = csa.topk(s, dc.seq_len, dc.q_pos, topk=wl.topk, ratio=wl.ratio)
    np.testing.assert_array_equal(_np(i), _np(i_ref))
    o_ref, l_ref = csa.csa_sparse_mqa_decode(dims, dc.q, dc.kv_p, None, i_ref, dc.win_p, None, dc.win_pos0,
                                             dc.win_rows, dc.seq_len, dc.q_pos, dc.sink)
    o, l = csa.sparse_mqa(dc.q, dc.kv, i, dc.win, dc.seq_len, dc.q_pos, dc.sink, window=wl.window, ratio=wl.ratio,
                          win_pos0=dc.win_pos0)
    np.testing.assert_array_equal(_np(o), _np(o_ref))
    np.testing.assert_array_equal(_np(l), _np(l_ref))
    h_ref, hl_ref = csa.hca_mqa_decode(dc.hca_dims(), dc.hca_q, dc.hca_kv_p, None, dc.hca_win_p, None, dc.win_pos0,
                                       dc.win_rows, dc.seq_len, dc.q_pos, dc.hca_sink)
    h, hl = csa.hca_mqa(dc.hca_q, dc.hca_kv, dc.hca_win, case.seq_len.tolist(), dc.q_pos, dc.hca_sink,
                        window=wl.window, ratio=128)
    np.testing.assert_array_equal(_np(h), _np(h_ref))
    np.testing.assert_array_equal(_np(hl), _np(hl_ref))


# --------------------------------------------------------------------------- top-k alone (integer work: exact)

def _topk_case(n_vis_list, n_max, K, seed, ties=False):
    rng = np.random.default_rng(seed)
    B = len(n_vis_list)
    scores = np.full((B, 1, n_max), -np.inf, np.float32)
    for b, nv in enumerate(n_vis_list):
        s = rng.standard_normal(nv).astype(np.float32)
        if ties:
            s = np.round(s * 8) / 8
        scores[b, 0, :nv] = s
    seq = np.array([4 * nv for nv in n_vis_list], np.int32)
    return scores, seq, seq - 1


@pytest.mark.parametrize("n_vis,n_max,K,ties", [
    ([100, 513, 600], 600, 512, False),
    ([16384], 16384, 512, False),          # one query at 65,536 tokens
    ([4097, 16384, 9000], 16384, 512, True),
    ([32769, 100], 32769, 512, True),
    ([5000, 32768, 20000], 32768, 512, True),
    ([32768], 32768, 2048, False),
    ([40000, 33000], 40000, 512, False),
    ([262144, 200000, 300, 262144], 262144, 512, True),
    ([262144], 262144, 1, False),
    ([70001, 65537], 70001, 512, True),  # many-workgroup path with a row length that is not a multiple of 4
    ([65540], 65540, 512, False),        # many-workgroup path, row length 4 mod 8 (last chunk ends mid-thread)
])
def test_topk_exact(n_vis, n_max, K, ties):
    say(f"[case] topk n_vis={n_vis} n_max={n_max} K={K} ties={ties}")
    scores, seq, pos = _topk_case(n_vis, n_max, K, seed=len(n_vis) * 7 + K, ties=ties)
    want = oracle.topk(scores, seq, pos, ratio=4, k=K)
    dims = csa.make_dims(batch=len(n_vis), topk=K, max_entries=n_max)
    got = _np(csa.csa_topk_select(dims, torch.from_numpy(scores).cuda(), torch.from_numpy(seq).cuda(),
                                  torch.from_numpy(pos).cuda()))
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("n_q,ties", [(300, False), (256, True)])
def test_topk_many_long_rows(n_q, ties):
    """Enough queries to fill the GPU with one selecting workgroup each: the
    histogram windows then cover long chunks (rows over 65,536 entries)."""
    n_vis = [70000 - 37 * i for i in range(n_q)]
    say(f"[case] topk many rows n_q={n_q} ties={ties}")
    scores, seq, pos = _topk_case(n_vis, 70000, 512, seed=n_q, ties=ties)
    want = oracle.topk(scores, seq, pos, ratio=4, k=512)
    dims = csa.make_dims(batch=n_q, topk=512, max_entries=70000)
    got = _np(csa.csa_topk_select(dims, torch.from_numpy(scores).cuda(), torch.from_numpy(seq).cuda(),
                                  torch.from_numpy(pos).cuda()))
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("n", [4096, 20000, 32768])
def test_topk_all_equal_scores_medium_row(n):
    """Every score equal in a row of up to 32,768 entries (the row kept in LDS,
    or the one-kernel threshold scan): the lowest K indices are taken."""
    say(f"[case] topk all equal n={n}")
    scores = np.full((1, 1, n), -1.5, np.float32)
    seq = np.array([4 * n], np.int32)
    dims = csa.make_dims(batch=1, topk=512, max_entries=n)
    got = _np(csa.csa_topk_select(dims, torch.from_numpy(scores).cuda(), torch.from_numpy(seq).cuda(),
                                  torch.from_numpy(seq - 1).cuda()))
    np.testing.assert_array_equal(got.reshape(-1), np.arange(512, dtype=np.int32))


def test_topk_all_equal_scores_long_row():
    """Every score equal: the candidate bin overflows and the exact whole-row
    fallback must return indices 0..K-1."""
    n = 100000
    scores = np.full((1, 1, n), 0.25, np.float32)
    seq = np.array([4 * n], np.int32)
    dims = csa.make_dims(batch=1, topk=512, max_entries=n)
    got = _np(csa.csa_topk_select(dims, torch.from_numpy(scores).cuda(), torch.from_numpy(seq).cuda(),
                                  torch.from_numpy(seq - 1).cuda()))
    np.testing.assert_array_equal(got[0, 0], np.arange(512))


@pytest.mark.parametrize("fill", [0xFF, 0x01, None])
def test_topk_any_workspace_contents_stay_exact(fill):
    """The multi-workgroup top-k keeps its histogram and counters in the
    workspace; whatever the workspace holds, results are exact, and the call
    leaves it clean for the next one."""
    scores, seq, pos = _topk_case([262144, 50000, 300], 262144, 512, seed=5, ties=True)
    want = oracle.topk(scores, seq, pos, ratio=4, k=512)
    dims = csa.make_dims(batch=3, topk=512, max_entries=262144)
    n = csa.workspace_size(dims, csa._lib.CSA_OP_TOPK)
    if fill is None:
        ws = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    else:
        ws = torch.full((n,), fill, dtype=torch.uint8, device="cuda")
    sc, sq, ps = (torch.from_numpy(x).cuda() for x in (scores, seq, pos))
    for call in range(3):
        say(f"[case] dirty workspace fill={fill} call={call}")
        got = _np(csa.csa_topk_select(dims, sc, sq, ps, workspace=ws))
        np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("act", [csa.CSA_ACT_RELU, csa.CSA_ACT_NONE])
def test_fused_selection_equals_standalone_topk(act):
    wl, sl = flash_case("flash_fused_vs_standalone", [4 * 40000, 4 * 9000, 4 * 20000 + 1])
    case = make_case_with_lens(wl, sl)
    say(f"[case] {wl.name} act={act}")
    dc = DeviceCase(case)
    g_scores, g_idx, _, _ = run_fused(dc, act)
    dims = dc.csa_dims()
    t_idx = _np(csa.csa_topk_select(dims, torch.from_numpy(g_scores).cuda(), dc.seq_len, dc.q_pos))
    np.testing.assert_array_equal(t_idx, g_idx)
    want = oracle.topk(g_scores, case.seq_len, case.q_pos, ratio=4, k=512)
    np.testing.assert_array_equal(g_idx, want)


def test_fused_selection_when_emitted_lists_fall_short():
    """The decode scorer hands the selection only its workgroups' highest
    entries.  Sequence 0: a contiguous block of 700 strong index keys puts the
    whole top-512 into one or two scorer workgroups, more than they can emit,
    so the selection scans the row instead.  Sequence 1: every index key equal,
    so every score ties and only the exact radix selection can decide.  Both
    must equal the oracle's top-k on the same scores, and the attention must
    match on that selection."""
    wl, sl = flash_case("flash_lists_fall_short", [4 * 100000, 4 * 60000])
    case = make_case_with_lens(wl, sl)
    k0 = inputs.bf16_to_f32(case.k_idx[0])
    k0[50000:50700] *= np.float32(4.0)
    case.k_idx[0] = inputs.bf16_bits(k0)
    case.k_idx[1][:] = case.k_idx[1][0]
    say(f"[case] {wl.name}: clustered tops and all-equal scores through the fused call")
    dc = DeviceCase(case)
    g_scores, g_idx, g_out, g_lse = run_fused(dc)
    want = oracle.topk(g_scores, case.seq_len, case.q_pos, ratio=4, k=512)
    np.testing.assert_array_equal(g_idx, want)
    assert set(g_idx[0, 0].tolist()) <= set(range(50000, 50700))
    np.testing.assert_array_equal(g_idx[1, 0], np.arange(512))
    o_out, o_lse = oracle_sparse(case, g_idx)
    assert_attention_close(g_out, o_out, ATT_TOL_BF16, "out")
    np.testing.assert_allclose(g_lse, o_lse, atol=1e-3, rtol=0)


@pytest.mark.parametrize("n", [40000, 262144])
def test_topk_extreme_range_and_clustered_tops(n):
    """Shortcut guards: (a) one huge score puts the K-th key far below the
    16-octave histogram window of the largest key; (b) every top score sits in
    one contiguous block, overflowing per-workgroup lists.  Both must stay
    exact."""
    rng = np.random.default_rng(n)
    s1 = rng.standard_normal(n).astype(np.float32) + 3.0
    s1[n // 3] = 1e30
    s2 = rng.random(n).astype(np.float32)
    s2[n // 2:n // 2 + 3000] += 10.0
    scores = np.stack([s1, s2])[:, None, :]
    seq = np.array([4 * n, 4 * n], np.int32)
    want = oracle.topk(scores, seq, seq - 1, ratio=4, k=512)
    dims = csa.make_dims(batch=2, topk=512, max_entries=n)
    say(f"[case] topk guards n={n}")
    got = _np(csa.csa_topk_select(dims, torch.from_numpy(scores).cuda(), torch.from_numpy(seq).cuda(),
                                  torch.from_numpy(seq - 1).cuda()))
    np.testing.assert_array_equal(got, want)


def test_topk_negative_zero_equals_zero():
    scores = np.zeros((1, 1, 2000), np.float32)
    scores[0, 0, ::2] = -0.0
    scores[0, 0, 1500:] = -1.0
    seq = np.array([8000], np.int32)
    dims = csa.make_dims(batch=1, topk=512, max_entries=2000)
    got = _np(csa.csa_topk_select(dims, torch.from_numpy(scores).cuda(), torch.from_numpy(seq).cuda(),
                                  torch.from_numpy(seq - 1).cuda()))
    np.testing.assert_array_equal(got[0, 0], np.arange(512))


# --------------------------------------------------------------------------- attention alone

def test_sparse_mqa_many_splits_and_padding():
    wl, sl = flash_case("flash_attn", [4 * 2000, 4 * 300, 4 * 100 + 3])
    case = make_case_with_lens(wl, sl)
    say(f"[case] {wl.name}")
    dc = DeviceCase(case)
    o_scores = oracle_scores(case)
    idx = oracle.topk(o_scores, case.seq_len, case.q_pos, ratio=4, k=512)
    dims = dc.csa_dims()
    out, lse = csa.csa_sparse_mqa_decode(dims, dc.q, dc.kv_p, None, torch.from_numpy(idx).cuda(), dc.win_p, None,
                                         dc.win_pos0, dc.win_rows, dc.seq_len, dc.q_pos, dc.sink)
    o_out, o_lse = oracle_sparse(case, idx)
    assert_attention_close(_np(out), o_out, ATT_TOL_BF16, "out")
    np.testing.assert_allclose(_np(lse), o_lse, atol=1e-3, rtol=0)


def test_hca_small():
    wl, sl = flash_case("hca_small", [128 * 4, 128 * 37 + 5, 100, 128 * 200], hca=128)
    case = make_case_with_lens(wl, sl)
    say(f"[case] {wl.name}")
    dc = DeviceCase(case)
    out, lse = csa.hca_mqa_decode(dc.hca_dims(), dc.hca_q, dc.hca_kv_p, None, dc.hca_win_p, None, dc.win_pos0,
                                  dc.win_rows, dc.seq_len, dc.q_pos, dc.hca_sink)
    o_out, o_lse = oracle_hca(case)
    assert_attention_close(_np(out), o_out, ATT_TOL_BF16, "hca out")
    np.testing.assert_allclose(_np(lse), o_lse, atol=1e-3, rtol=0)


def test_deterministic_and_no_out_of_bounds_writes():
    wl, sl = flash_case("flash_det", [4 * 5000, 4 * 1234 + 2])
    case = make_case_with_lens(wl, sl)
    dc = DeviceCase(case)
    dims = dc.csa_dims()
    guard = 4096
    res = []
    for _ in range(2):
        buf = torch.full((dims.batch * 64 * 512 + 2 * guard,), 7.0, dtype=torch.float32, device="cuda")
        out = buf[guard:guard + dims.batch * 64 * 512].view(dims.batch, 1, 64, 512)
        ibuf = torch.full((dims.batch * 512 + 2 * guard,), 12345, dtype=torch.int32, device="cuda")
        idx = ibuf[guard:guard + dims.batch * 512].view(dims.batch, 1, 512)
        csa.csa_attention(dims, dc.q, dc.q_idx, dc.w, dc.k_idx_p, dc.kv_p, None, dc.win_p, None, dc.win_pos0,
                          dc.win_rows, dc.seq_len, dc.q_pos, dc.sink, out=out, topk_idx_out=idx)
        b, ib = _np(buf), _np(ibuf)
        assert (b[:guard] == 7.0).all() and (b[-guard:] == 7.0).all()
        assert (ib[:guard] == 12345).all() and (ib[-guard:] == 12345).all()
        res.append((b.copy(), ib.copy()))
    np.testing.assert_array_equal(res[0][0], res[1][0])
    np.testing.assert_array_equal(res[0][1], res[1][1])


# --------------------------------------------------------------------------- prefill chunk (many queries)

@pytest.mark.parametrize("lens,T,q_pos0", [
    ([4 * 3000 + 2], 48, 4 * 3000 + 2 - 48),          # 3 query blocks; the causal edge inside the last tile
    ([4 * 2500 + 1, 4 * 1700 + 3], 20, 4 * 1700 - 20),  # two ragged sequences, a partial query block
    ([4 * 64 * 40], 16, 4 * 64 * 40 - 16),             # one query block; entries a whole number of tiles
])
def test_prefill_chunk_small(lens, T, q_pos0):
    wl, sl = flash_case(f"prefill_small_{len(lens)}_{T}", lens, q_len=T, q_pos0=q_pos0)
    check_whole_step(make_case_with_lens(wl, sl), ATT_TOL_BF16)


def test_prefill_chunk_no_activation():
    wl, sl = flash_case("prefill_noact", [4 * 1500 + 3], q_len=33, q_pos0=4 * 1500 + 3 - 40)
    check_whole_step(make_case_with_lens(wl, sl), ATT_TOL_BF16, act=csa.CSA_ACT_NONE)


def test_large_attention_launch_one_split():
    """300 queries x 2 head groups: more attention workgroups than are resident
    at once, so they take the one-dimensional order (one split per query: the
    output is written directly)."""
    wl, sl = flash_case("prefill_300", [4 * 1200 + 1], q_len=300, q_pos0=4 * 1200 + 1 - 300)
    check_whole_step(make_case_with_lens(wl, sl), ATT_TOL_BF16)


def test_pro_shapes_large_attention_launch_two_splits():
    """128 heads (four head groups) and 100 causal queries: two splits per
    query and 800 attention workgroups, so the split partials are written in
    the one-dimensional order and merged by the combine."""
    base = inputs.WORKLOADS["pro_decode_b4_1m"]
    wl = inputs.scaled(base, "pro_q100", index=112, batch=2, q_len=50, seq_len=None, seq_len_range=None,
                       q_pos0=4 * 2000 + 3 - 50)
    check_whole_step(inputs.make_case(wl, seq_lens=np.array([4 * 3000 + 1, 4 * 2000 + 3], np.int32)), ATT_TOL_BF16)


@pytest.mark.parametrize("lens,T,q_pos0,act", [
    ([4 * 20000 + 3], 300, 4 * 20000 + 3 - 300, csa.CSA_ACT_RELU),  # many queries: one selecting workgroup each
    ([4 * 6000 + 1, 4 * 9000 + 2], 40, 2030, csa.CSA_ACT_RELU),     # visible counts cross K inside the chunk
    ([4 * 70000], 16, 4 * 70000 - 16, csa.CSA_ACT_RELU),            # long rows, few queries: filter and final
    ([4 * 30000 + 1], 24, 4 * 30000 - 30, csa.CSA_ACT_NONE),        # signed scores: keys in both halves
])
def test_prefill_fused_selection_equals_standalone_topk(lens, T, q_pos0, act):
    """The tiled scorer builds the key histograms for the selection while it
    writes the scores; the selection must equal the top-k kernel run alone
    (its own histogram pass) and the oracle's top-k on the same scores."""
    wl, sl = flash_case(f"prefill_fused_{len(lens)}_{T}", lens, q_len=T, q_pos0=q_pos0)
    case = make_case_with_lens(wl, sl)
    say(f"[case] {wl.name} B={wl.batch} T={T} max_entries={case.max_entries} act={act}")
    dc = DeviceCase(case)
    g_scores, g_idx, g_out, g_lse = run_fused(dc, act)
    if act == csa.CSA_ACT_NONE:
        assert (g_scores[np.isfinite(g_scores)] < 0).any(), "the case should hold negative scores"
    assert np.isfinite(g_out).all() and np.isfinite(g_lse).all()
    t_idx = _np(csa.csa_topk_select(dc.csa_dims(), torch.from_numpy(g_scores).cuda(), dc.seq_len, dc.q_pos))
    np.testing.assert_array_equal(t_idx, g_idx)
    want = oracle.topk(g_scores, case.seq_len, case.q_pos, ratio=4, k=512)
    np.testing.assert_array_equal(g_idx, want)


def run_fused_stream(dc, act=csa.CSA_ACT_RELU, sentinel=0x5A):
    """csa_attention without a score output (the tiled scorer's streaming
    selection); the workspace starts filled with `sentinel`, and the bytes
    where the scores would go are returned as well."""
    dims = dc.csa_dims(index_act=act)
    Q = dims.batch * dims.q_len
    ws = torch.full((max(256, csa.workspace_size(dims, csa._lib.CSA_OP_ATTENTION)),), sentinel, dtype=torch.uint8,
                    device="cuda")
    idx = torch.full((dims.batch, dims.q_len, dims.topk), 7777, dtype=torch.int32, device="cuda")
    out, lse = csa.csa_attention(dims, dc.q, dc.q_idx, dc.w, dc.k_idx_p, dc.kv_p, dc.v_p, dc.win_p, dc.win_v_p,
                                 dc.win_pos0, dc.win_rows, dc.seq_len, dc.q_pos, dc.sink, topk_idx_out=idx,
                                 workspace=ws)
    torch.cuda.synchronize()
    untouched = bool((ws[:Q * dims.max_entries * 4] == sentinel).all())
    return idx, out, lse, untouched


# (the streaming selection runs when the chunks' K best fit the selection's
# slots: chunks x K <= 8192, e.g. 16 chunks at K = 512 from 1,024 queries on)
@pytest.mark.parametrize("lens,T,q_pos0,act,topk", [
    ([4 * 12000 + 3], 1024, 4 * 12000 + 3 - 1024, csa.CSA_ACT_RELU, 512),  # 16 chunks of 768 entries
    ([4 * 6000 + 1, 4 * 9000 + 2], 512, 800, csa.CSA_ACT_RELU, 256),     # visible counts cross K inside the chunk
    ([4 * 30000 + 1], 1024, 4 * 30000 - 1030, csa.CSA_ACT_NONE, 512),   # signed scores: keys in both halves
    ([4 * 70000], 2048, 4 * 70000 - 2048, csa.CSA_ACT_RELU, 64),        # 8 chunks of 8,832 entries: compactions
    ([4 * 12000 + 2], 9, 4 * 12000 - 9, csa.CSA_ACT_RELU, 1),            # K = 1, a partial query block
])
def test_prefill_streaming_selection(lens, T, q_pos0, act, topk):
    """Without a score output the tiled scorer keeps each (query, entry
    chunk)'s K best entries itself and writes no scores, and the selection
    works from those alone.  Its selection and attention must be those of the
    call that writes the scores (bit for bit), and the selection the oracle's
    exact top-k of those scores; no score may be written to the workspace."""
    wl, sl = flash_case(f"prefill_stream_{len(lens)}_{T}_{topk}", lens, q_len=T, q_pos0=q_pos0, topk=topk)
    case = make_case_with_lens(wl, sl)
    say(f"[case] {wl.name} B={wl.batch} T={T} max_entries={case.max_entries} act={act} K={topk}")
    dc = DeviceCase(case)
    g_scores, g_idx, g_out, g_lse = run_fused(dc, act)
    s_idx, s_out, s_lse, untouched = run_fused_stream(dc, act)
    assert untouched, "the streaming selection wrote scores"
    np.testing.assert_array_equal(_np(s_idx), g_idx)
    np.testing.assert_array_equal(_np(s_out), g_out)
    np.testing.assert_array_equal(_np(s_lse), g_lse)
    want = oracle.topk(g_scores, case.seq_len, case.q_pos, ratio=4, k=topk)
    np.testing.assert_array_equal(_np(s_idx), want)


@pytest.mark.parametrize("rep", [8, 0])
def test_prefill_streaming_selection_ties(rep):
    """Equal scores through the streaming selection: index-key rows repeated
    `rep` times (rep 0: every row the same, so every visible entry of a query
    has the same score), so the K-th score is shared by many entries and the
    lower indices must win; the result must be the materialized call's and
    the oracle's exact top-k of the same scores."""
    wl, sl = flash_case(f"prefill_stream_ties_{rep}", [4 * 12000 + 3], q_len=1024, q_pos0=4 * 12000 + 3 - 1024)
    case = make_case_with_lens(wl, sl)
    k = case.k_idx[0]
    src = np.arange(k.shape[0]) // rep if rep else np.zeros(k.shape[0], np.int64)
    case.k_idx[0] = np.ascontiguousarray(k[src])
    say(f"[case] {wl.name} T={wl.q_len} max_entries={case.max_entries} rows repeated {rep or 'all'}")
    dc = DeviceCase(case)
    g_scores, g_idx, g_out, g_lse = run_fused(dc)
    s_idx, s_out, s_lse, untouched = run_fused_stream(dc)
    assert untouched, "the streaming selection wrote scores"
    want = oracle.topk(g_scores, case.seq_len, case.q_pos, ratio=4, k=wl.topk)
    np.testing.assert_array_equal(g_idx, want)
    np.testing.assert_array_equal(_np(s_idx), want)
    np.testing.assert_array_equal(_np(s_out), g_out)
    np.testing.assert_array_equal(_np(s_lse), g_lse)
    if rep == 0:  # every visible entry ties: the K lowest indices
        np.testing.assert_array_equal(want[0, :, :], np.broadcast_to(np.arange(wl.topk), want.shape[1:]))


# --------------------------------------------------------------------------- full-size workloads

def test_decode_b1_64k_full():
    check_whole_step(inputs.make_case(inputs.WORKLOADS["decode_b1_64k"]), ATT_TOL_BF16)


def test_decode_b32_ragged_full():
    check_whole_step(inputs.make_case(inputs.WORKLOADS["decode_b32_ragged_64k_128k"]), ATT_TOL_BF16)


def test_decode_b4_1m_full_csa_and_hca():
    case = inputs.make_case(inputs.WORKLOADS["decode_b4_1m"])
    dc = check_whole_step(case, ATT_TOL_BF16)
    say("[case] decode_b4_1m HCA layer")
    out, lse = csa.hca_mqa_decode(dc.hca_dims(), dc.hca_q, dc.hca_kv_p, None, dc.hca_win_p, None, dc.win_pos0,
                                  dc.win_rows, dc.seq_len, dc.q_pos, dc.hca_sink)
    o_out, o_lse = oracle_hca(case)
    assert_attention_close(_np(out), o_out, ATT_TOL_BF16, "hca out")
    np.testing.assert_allclose(_np(lse), o_lse, atol=1e-3, rtol=0)


def test_prefill_t2048_1m_sampled():
    """The 2,048-query chunk over a 1M-token cache at full size: every query's
    selection is checked for validity and every score row for its causal
    mask; every query's scores at 128 sampled entries (seen by all queries)
    are compared with the oracle's; sampled queries (both ends, query-block
    edges) are compared with the oracle in full: scores, the selected set,
    and attention on that set."""
    case = inputs.make_case(inputs.WORKLOADS["prefill_t2048_1m"], with_hca=False)
    wl = case.wl
    say(f"[case] {wl.name} T={wl.q_len} max_entries={case.max_entries}")
    dc = DeviceCase(case)
    scores, idx, out, lse = run_fused_t(dc)
    nvis = np.array([nvis_of(case, t) for t in range(wl.q_len)])
    # properties of every query
    nv_t = torch.from_numpy(nvis).cuda()
    col = torch.arange(case.max_entries, device="cuda")
    row = scores[0]
    masked = col[None, :] >= nv_t[:, None]
    assert bool(torch.isneginf(row[masked]).all()), "causal mask"
    assert bool(torch.isfinite(row[~masked]).all()), "visible scores finite"
    del masked
    g_idx = idx.cpu().numpy()
    for t in range(wl.q_len):
        check_topk_valid(g_idx[0, t], int(nvis[t]), wl.topk)
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())
    # every query at sampled entries: the oracle scores a cache made of just
    # those rows, every one visible (entry j's score does not depend on where
    # the row sits once it is visible)
    n_common = int(nvis.min())
    rng = np.random.default_rng(2048)
    js = np.unique(np.concatenate([[0, n_common - 1], rng.choice(n_common, 126, replace=False)]))
    k_sub = [np.ascontiguousarray(case.k_idx[0][js])]
    n_s = len(js)
    o_s = oracle.index_scores(case.q_idx, case.w, k_sub, np.array([n_s * wl.ratio], np.int32),
                              np.full(wl.q_len, n_s * wl.ratio - 1, np.int32), ratio=wl.ratio, n_max=n_s,
                              dtype=wl.dtype)[0].astype(np.float64)
    g_s = row[:, torch.from_numpy(js).cuda()].cpu().numpy().astype(np.float64)
    rms = np.sqrt(np.mean(o_s ** 2, axis=1))
    worst = float(np.max(np.max(np.abs(g_s - o_s), axis=1) / rms))
    assert worst <= SCORE_TOL, f"sampled entries: worst score err / rms {worst:.2e}"
    say(f"  ok: all {wl.q_len} queries at {n_s} sampled entries, worst score err/rms={worst:.2e}")
    # sampled queries against the oracle
    ts = [0, 1, 15, 16, 1000, 2046, 2047]
    sub = query_subset(case, ts)
    o_scores = oracle_scores(sub)
    g_sub = row[ts].cpu().numpy()[None]
    assert_scores_close(g_sub, o_scores, sub)
    o_idx = oracle.topk(o_scores, sub.seq_len, sub.q_pos, ratio=wl.ratio, k=wl.topk)
    n_diff = assert_topk_band(g_idx[:, ts], o_idx, o_scores, sub)
    o_out, o_lse = oracle_sparse(sub, g_idx[:, ts])
    rel = assert_attention_close(out[:, ts].cpu().numpy(), o_out, ATT_TOL_BF16, "out")
    np.testing.assert_allclose(lse[:, ts].cpu().numpy(), o_lse, atol=1e-3, rtol=0)
    say(f"  ok: sampled {len(ts)} queries, topk band swaps={n_diff} out err/rms={rel:.2e}")
    # the same chunk without a score output (the streaming selection, as the
    # fused call runs it when no scores are asked for): every query's
    # selection and attention bit for bit
    del scores, row, col
    torch.cuda.empty_cache()
    s_idx, s_out, s_lse, untouched = run_fused_stream(dc)
    assert untouched, "the streaming selection wrote scores"
    assert torch.equal(s_idx, idx), "streaming selection differs"
    assert torch.equal(s_out, out) and torch.equal(s_lse, lse)
    say(f"  ok: streaming selection equals the materialized one for all {wl.q_len} queries")


# --------------------------------------------------------------------------- fp8 (E4M3) index tensors

def check_fp8_scores(case, act=csa.CSA_ACT_RELU, topk=True):
    """csa_index_scores_fp8 against the oracle's fp8 definition (every score),
    then the top-k of the GPU scores against the oracle's set (band rule)."""
    wl = case.wl
    say(f"[case] fp8 scores {wl.name} B={wl.batch} T={wl.q_len} max_entries={case.max_entries} act={act}")
    q8, qs, k8, ks = inputs.make_fp8_index(case)
    dev = "cuda"
    k8_t = [torch.from_numpy(k).to(dev) for k in k8]
    ks_t = [torch.from_numpy(x).to(dev) for x in ks]
    seq_t = torch.from_numpy(case.seq_len).to(dev)
    pos_t = torch.from_numpy(case.q_pos).to(dev)
    dims = csa.make_dims(batch=wl.batch, q_len=wl.q_len, topk=wl.topk, window=wl.window, ratio=wl.ratio,
                         max_entries=case.max_entries, index_act=act)
    g = _np(csa.csa_index_scores_fp8(dims, torch.from_numpy(q8).to(dev), torch.from_numpy(qs).to(dev),
                                     torch.from_numpy(case.w).to(dev), k8_t, ks_t, seq_t, pos_t))
    o = oracle.index_scores_fp8(q8, qs, case.w, k8, ks, case.seq_len, case.q_pos, ratio=wl.ratio,
                                n_max=case.max_entries, act=oracle.ACT_NONE if act == csa.CSA_ACT_NONE else oracle.ACT_RELU)
    assert_scores_close(g, o, case)
    if topk:
        o_idx = oracle.topk(o, case.seq_len, case.q_pos, ratio=wl.ratio, k=wl.topk)
        g_idx = _np(csa.csa_topk_select(dims, torch.from_numpy(g).to(dev), seq_t, pos_t))
        n_diff = assert_topk_band(g_idx, o_idx, o, case)
        say(f"  ok: fp8 scores, topk band swaps={n_diff}")


@pytest.mark.parametrize("lens", [
    [4 * 3000 + 2, 4 * 500 + 1, 4 * 64 * 7],   # ragged tails, several wave-steps
    [50, 4 * 700 + 3],                         # nothing compressed visible in one sequence
])
def test_fp8_scores_small(lens):
    wl, sl = flash_case(f"fp8_small_{len(lens)}_{lens[0]}", lens)
    check_fp8_scores(make_case_with_lens(wl, sl))


def test_fp8_scores_no_activation_and_many_queries():
    wl, sl = flash_case("fp8_noact_prefill", [4 * 1500 + 3], q_len=20, q_pos0=4 * 1500 + 3 - 25)
    check_fp8_scores(make_case_with_lens(wl, sl), act=csa.CSA_ACT_NONE, topk=False)


def test_fp8_scores_decode_b4_1m_full():
    check_fp8_scores(inputs.make_case(inputs.WORKLOADS["decode_b4_1m"], with_hca=False))


def check_fp8_step(case, act=csa.CSA_ACT_RELU, fp8=None):
    """csa_attention_fp8 (fp8 index, bf16 attention): its scores against the
    oracle's fp8 definition, its selection against the standalone top-k on the
    same scores (bit-exact) and the oracle's set (band rule), its attention
    against the oracle on its own selection."""
    wl = case.wl
    say(f"[case] fp8 step {wl.name} B={wl.batch} T={wl.q_len} max_entries={case.max_entries} act={act}")
    q8, qs, k8, ks = inputs.make_fp8_index(case) if fp8 is None else fp8
    dev = "cuda"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    dc = DeviceCase(case)
    dims = dc.csa_dims(index_act=act)
    scores = torch.empty((dims.batch, dims.q_len, dims.max_entries), dtype=torch.float32, device=dev)
    idx = torch.empty((dims.batch, dims.q_len, dims.topk), dtype=torch.int32, device=dev)
    out, lse = csa.csa_attention_fp8(dims, dc.q, t(q8), t(qs), dc.w, [t(k) for k in k8], [t(x) for x in ks],
                                     dc.kv_p, dc.v_p, dc.win_p, dc.win_v_p, dc.win_pos0, dc.win_rows, dc.seq_len,
                                     dc.q_pos, dc.sink, topk_idx_out=idx, scores_out=scores)
    g_scores, g_idx, g_out, g_lse = _np(scores), _np(idx), _np(out), _np(lse)
    o_scores = oracle.index_scores_fp8(q8, qs, case.w, k8, ks, case.seq_len, case.q_pos, ratio=wl.ratio,
                                       n_max=max(1, case.max_entries),
                                       act=oracle.ACT_NONE if act == csa.CSA_ACT_NONE else oracle.ACT_RELU)
    assert_scores_close(g_scores, o_scores, case)
    t_idx = _np(csa.csa_topk_select(dims, scores, dc.seq_len, dc.q_pos))
    np.testing.assert_array_equal(g_idx, t_idx)
    o_idx = oracle.topk(o_scores, case.seq_len, case.q_pos, ratio=wl.ratio, k=wl.topk)
    n_diff = assert_topk_band(g_idx, o_idx, o_scores, case)
    o_out, o_lse = oracle_sparse(case, g_idx)
    rel = assert_attention_close(g_out, o_out, ATT_TOL_BF16, "out")
    np.testing.assert_allclose(g_lse, o_lse, atol=1e-3, rtol=0)
    say(f"  ok: topk band swaps={n_diff} out err/rms={rel:.2e}")


@pytest.mark.parametrize("lens,T,q_pos0", [
    ([4 * 9000 + 2, 4 * 3000 + 1, 4 * 64 * 7], 1, None),   # ragged, emitted lists, several splits
    ([50, 4 * 700 + 3], 1, None),                          # nothing compressed visible in one sequence
    ([4 * 20000 + 3], 12, 4 * 20000 + 3 - 40),              # several queries of one sequence
])
def test_fp8_step_small(lens, T, q_pos0):
    wl, sl = flash_case(f"fp8_step_{T}_{lens[0]}", lens, q_len=T, q_pos0=q_pos0)
    check_fp8_step(make_case_with_lens(wl, sl))


def test_fp8_step_ragged_batch():
    wl, sl = flash_case("fp8_step_ragged12", RAGGED_12)
    check_fp8_step(make_case_with_lens(wl, sl))


def test_fp8_step_no_activation():
    wl, sl = flash_case("fp8_step_noact", [4 * 6000 + 1, 4 * 2500])
    check_fp8_step(make_case_with_lens(wl, sl), act=csa.CSA_ACT_NONE)


def test_fp8_step_when_emitted_lists_fall_short():
    """Every key row of sequence 0 equal (all scores tie) and sequence 1's key
    codes clustered: the scorer's emitted lists overflow or cut too high and the
    selection falls back to scanning the scores, still exact."""
    wl, sl = flash_case("fp8_step_ties", [4 * 30000 + 1, 4 * 16000 + 2])
    case = make_case_with_lens(wl, sl)
    q8, qs, k8, ks = inputs.make_fp8_index(case)
    k8[0][:] = k8[0][0]
    ks[0][:] = ks[0][0]
    k8[1][: len(k8[1]) // 2] = k8[1][0]
    check_fp8_step(case, fp8=(q8, qs, k8, ks))


def test_fp8_step_decode_b4_1m_full():
    check_fp8_step(inputs.make_case(inputs.WORKLOADS["decode_b4_1m"], with_hca=False))


# --------------------------------------------------------------------------- V4-Pro shapes (128 heads, top-1024)

def _pro_case(name, lens, index=111):
    base = inputs.WORKLOADS["pro_decode_b4_1m"]
    wl = inputs.scaled(base, name, index=index, batch=len(lens), seq_len=None, seq_len_range=None)
    return inputs.make_case(wl, seq_lens=np.array(lens, np.int32))


@pytest.mark.parametrize("lens", [
    [4 * 6000 + 3, 4 * 900 + 1, 4 * 200],   # n_vis above and below K = 1024, ragged
])
def test_pro_shapes_whole_step_small(lens):
    check_whole_step(_pro_case(f"pro_small_{lens[0]}", lens), ATT_TOL_BF16)


def test_pro_decode_b4_1m_full():
    check_whole_step(inputs.make_case(inputs.WORKLOADS["pro_decode_b4_1m"]), ATT_TOL_BF16)


# --------------------------------------------------------------------------- compressor (the step before the path)

def check_compress(name, *, tokens, hidden, out_dim, ratio, window, first_entry, n_entries, pos0, rope_dims,
                   hadamard=False, seed=501):
    say(f"[case] compress {name}: tokens={tokens} hidden={hidden} out={out_dim} r={ratio} window={window} "
        f"entries={first_entry}+{n_entries} rope={rope_dims} hadamard={hadamard}")
    x, wkv, wg, ape, gamma = inputs.make_compressor_inputs(seed, tokens, hidden, out_dim, window)
    dims = csa.make_compress_dims(tokens=tokens, hidden=hidden, out_dim=out_dim, ratio=ratio, window=window,
                                  first_entry=first_entry, n_entries=n_entries, pos0=pos0, rope_dims=rope_dims,
                                  hadamard=hadamard)
    dev = "cuda"
    bf = lambda a: torch.from_numpy(a.view(np.int16)).to(dev)
    g = csa.csa_compress(dims, bf(x), bf(wkv), bf(wg), torch.from_numpy(ape).to(dev), torch.from_numpy(gamma).to(dev))
    torch.cuda.synchronize()
    got = g.float().cpu().numpy().astype(np.float64)
    want = oracle.compress(x, wkv, wg, ape, gamma, pos0=pos0, ratio=ratio, window=window, first_entry=first_entry,
                           n_entries=n_entries, rope_dims=rope_dims, hadamard=hadamard)
    # the GPU rounds its fp32 result to bf16: within one bf16 ulp of the exact value
    err = np.abs(got - want)
    bound = 2.0 ** -7 * np.abs(want) + 1e-5
    worst = float(np.max(err / bound))
    assert np.isfinite(got).all() and worst <= 1.0, f"{name}: worst err/bound {worst:.3f}"
    say(f"  ok: worst err / (1 bf16 ulp) = {worst:.3f}")


def test_compress_csa_decode_entry():
    """One new 4:1 entry at a decode step: its 8-token overlapping window, full hidden size, RoPE on 64 dims."""
    e = 1000
    check_compress("csa_decode", tokens=8, hidden=4096, out_dim=512, ratio=4, window=8, first_entry=e, n_entries=1,
                   pos0=4 * e + 4 - 8, rope_dims=64)


def test_compress_csa_chunk_from_position_zero():
    """A chunk of entries from the sequence start (entry 0's window is cut at position 0)."""
    check_compress("csa_chunk", tokens=256, hidden=1024, out_dim=512, ratio=4, window=8, first_entry=0,
                   n_entries=64, pos0=0, rope_dims=64)


def test_compress_hca_entries():
    check_compress("hca", tokens=384, hidden=1024, out_dim=512, ratio=128, window=128, first_entry=2, n_entries=3,
                   pos0=256, rope_dims=64)


def test_compress_index_keys_with_hadamard():
    """The indexer's key compressor: 128-d output, Hadamard rotation last."""
    check_compress("index_keys", tokens=40, hidden=2048, out_dim=128, ratio=4, window=8, first_entry=3,
                   n_entries=8, pos0=8, rope_dims=64, hadamard=True)


def test_compress_full_chunk_of_entries():
    """512 entries from 2,052 tokens: the pooling runs fewer token groups per entry when many entries fill the GPU."""
    check_compress("kv_chunk_512", tokens=2052, hidden=1024, out_dim=512, ratio=4, window=8, first_entry=1000,
                   n_entries=512, pos0=3996, rope_dims=64)


def test_compress_index_keys_eight_way_split():
    """Few token tiles: hidden split over 8 workgroups, 8 partial sums per row."""
    check_compress("index_keys_split8", tokens=1000, hidden=2048, out_dim=128, ratio=4, window=8, first_entry=0,
                   n_entries=250, pos0=0, rope_dims=64, hadamard=True)


def test_compress_odd_stage_count():
    """hidden = 17 x 64: an odd number of 64-wide stages (one stage of loads in flight), no split."""
    check_compress("odd_stages", tokens=300, hidden=1088, out_dim=256, ratio=4, window=8, first_entry=20,
                   n_entries=70, pos0=76, rope_dims=32)


def test_compress_hca_decode_window():
    """One 128:1 entry from its 128-token window: the weight-streaming projection over 8 token tiles."""
    check_compress("hca_decode", tokens=128, hidden=2048, out_dim=512, ratio=128, window=128, first_entry=4000,
                   n_entries=1, pos0=512000, rope_dims=64)


def test_compress_small_hidden_ragged_tokens():
    """hidden 256 (4 blocks for 8 waves: half the waves idle) and 20 tokens (a ragged second token tile)."""
    check_compress("small_hidden", tokens=20, hidden=256, out_dim=128, ratio=4, window=8, first_entry=7,
                   n_entries=4, pos0=24, rope_dims=0, hadamard=True)
