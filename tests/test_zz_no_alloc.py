"""The allocation-free fused call (csa_attention_noalloc, through the C ABI)
against csa_attention with a caller workspace: two calls in a row, the second
with a smaller input, on the library's static work area.  The same kernels run
on the same inputs, so the selected indices must be identical and the outputs
identical too; both are also held to the oracle's bar (top-k band rule,
attention within 1e-2 x RMS on the GPU's own selection)."""
import numpy as np
import pytest

import oracle
from compressed_sparse_attention_indexer_amd import inputs
from tests.gpu_helpers import (ATT_TOL_BF16, assert_attention_close, assert_topk_band, flash_case,
                               make_case_with_lens, oracle_scores, oracle_sparse, say)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import compressed_sparse_attention_indexer_amd as csa  # noqa: E402
from compressed_sparse_attention_indexer_amd.staging import DeviceCase  # noqa: E402


def _run_both(case):
    dc = DeviceCase(case)
    dims = dc.csa_dims()
    shape_i = (dims.batch, dims.q_len, dims.topk)
    res = []
    for fn in ("csa_attention_noalloc", "csa_attention"):
        idx = torch.full(shape_i, -7, dtype=torch.int32, device="cuda")
        out = torch.full((dims.batch, dims.q_len, dims.n_heads, dims.head_dim), 7.0, device="cuda")
        lse = torch.full((dims.batch, dims.q_len, dims.n_heads), 7.0, device="cuda")
        getattr(csa, fn)(dims, dc.q, dc.q_idx, dc.w, dc.k_idx_p, dc.kv_p, dc.v_p, dc.win_p, dc.win_v_p, dc.win_pos0,
                         dc.win_rows, dc.seq_len, dc.q_pos, dc.sink, out=out, lse=lse, topk_idx_out=idx)
        torch.cuda.synchronize()
        res.append((idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()))
    return res


def test_noalloc_matches_caller_workspace_on_two_calls():
    big_wl, big_lens = flash_case("noalloc_big", [4 * 200000 + 3, 4 * 90000 + 1, 4 * 150000])
    small_wl, small_lens = flash_case("noalloc_small", [4 * 6000 + 2, 4 * 300 + 1], index=102)
    for case in (make_case_with_lens(big_wl, big_lens), make_case_with_lens(small_wl, small_lens)):
        say(f"[case] noalloc {case.wl.name} B={case.wl.batch} max_entries={case.max_entries}")
        (i0, o0, l0), (i1, o1, l1) = _run_both(case)
        np.testing.assert_array_equal(i0, i1)
        np.testing.assert_array_equal(o0, o1)
        np.testing.assert_array_equal(l0, l1)
        o_scores = oracle_scores(case)
        o_idx = oracle.topk(o_scores, case.seq_len, case.q_pos, ratio=case.wl.ratio, k=case.wl.topk)
        assert_topk_band(i0, o_idx, o_scores, case)
        o_out, o_lse = oracle_sparse(case, i0)
        assert_attention_close(o0, o_out, ATT_TOL_BF16, "noalloc out")
        np.testing.assert_allclose(l0, o_lse, atol=1e-3, rtol=0)
