"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and every validation path returns its status before any
launch (only fake, never-dereferenced pointers are passed)."""
import ctypes
import os
import re
import subprocess

import pytest

import compressed_sparse_attention_indexer_amd as csa
from compressed_sparse_attention_indexer_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libcsa.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)) - {"defined"})


def test_header_declares_expected_entry_points():
    assert _declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = csa.load_library()
    for name in _declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], stdout=subprocess.PIPE, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(_declared_functions()) <= exported


def test_abi_version_and_enums_match_header():
    text = open(HEADER).read()
    assert csa.load_library().csa_abi_version() == int(re.search(r"#define CSA_ABI_VERSION (\d+)", text).group(1))
    for name, val in [("CSA_OK", _lib.CSA_OK), ("CSA_ERR_NULL", _lib.CSA_ERR_NULL), ("CSA_ERR_DIM", _lib.CSA_ERR_DIM),
                      ("CSA_ERR_ALIGN", _lib.CSA_ERR_ALIGN), ("CSA_ERR_UNSUPPORTED", _lib.CSA_ERR_UNSUPPORTED),
                      ("CSA_ERR_WORKSPACE", _lib.CSA_ERR_WORKSPACE), ("CSA_ERR_HIP", _lib.CSA_ERR_HIP),
                      ("CSA_OP_ATTENTION", _lib.CSA_OP_ATTENTION)]:
        assert int(re.search(rf"{name} = (\d+)", text).group(1)) == val, name
    assert ctypes.sizeof(_lib.CsaDims) == 13 * 4


def _flash(**over):
    kw = dict(batch=4, max_entries=262144)
    kw.update(over)
    return csa.make_dims(**kw)


def _fixture(**over):
    kw = dict(batch=2, n_heads=4, head_dim=16, index_heads=4, index_dim=16, topk=32, window=16, ratio=4,
              max_entries=128, dtype=csa.CSA_F32)
    kw.update(over)
    return csa.make_dims(**kw)


FAKE = 0x7F0000000000          # 256-byte aligned, never dereferenced
MIS = FAKE + 4                 # misaligned


def _scores(dims, q_idx=FAKE, w=FAKE, k=FAKE, sl=FAKE, qp=FAKE, out=FAKE):
    return csa.load_library().csa_index_scores(ctypes.byref(dims), q_idx, w, k, sl, qp, out, None, 0, None)


def _topk(dims, ws=None, nws=0, scores=FAKE, idx=FAKE):
    return csa.load_library().csa_topk_select(ctypes.byref(dims), scores, FAKE, FAKE, idx, ws, nws, None)


def _sparse(dims, ws=None, nws=0, q=FAKE, kv=FAKE, idx=FAKE, sink=FAKE, out=FAKE):
    return csa.load_library().csa_sparse_mqa_decode(ctypes.byref(dims), q, kv, None, idx, FAKE, None, FAKE, FAKE,
                                                    FAKE, FAKE, sink, out, None, ws, nws, None)


def _hca(dims, ws=None, nws=0):
    return csa.load_library().hca_mqa_decode(ctypes.byref(dims), FAKE, FAKE, None, FAKE, None, FAKE, FAKE, FAKE,
                                             FAKE, FAKE, FAKE, None, ws, nws, None)


def _fused(dims, ws=None, nws=0, q_idx=FAKE):
    return csa.load_library().csa_attention(ctypes.byref(dims), FAKE, q_idx, FAKE, FAKE, FAKE, None, FAKE, None,
                                            FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, ws, nws, None)


def test_null_arguments():
    L = csa.load_library()
    assert L.csa_index_scores(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == _lib.CSA_ERR_NULL
    assert _scores(_flash(), q_idx=None) == _lib.CSA_ERR_NULL
    assert "q_idx" in L.csa_last_error().decode()
    assert _scores(_flash(), k=None) == _lib.CSA_ERR_NULL
    assert _topk(_flash(max_entries=1000), scores=None) == _lib.CSA_ERR_NULL
    assert _sparse(_flash(), sink=None) == _lib.CSA_ERR_NULL
    assert _fused(_flash(), q_idx=None) == _lib.CSA_ERR_NULL
    n = ctypes.c_size_t(1)
    assert L.csa_workspace_size(ctypes.byref(_flash()), 0, None) == _lib.CSA_ERR_NULL
    assert L.csa_workspace_size(None, 0, ctypes.byref(n)) == _lib.CSA_ERR_NULL


@pytest.mark.parametrize("over", [dict(batch=0), dict(q_len=0), dict(batch=1 << 11, q_len=1 << 10),
                                  dict(ratio=0), dict(max_entries=0), dict(max_entries=(1 << 26) + 1)])
def test_bad_common_sizes(over):
    assert _scores(_flash(**over)) == _lib.CSA_ERR_DIM


def test_bad_op_sizes():
    assert _topk(_flash(topk=0)) == _lib.CSA_ERR_DIM
    assert _topk(_flash(topk=4096)) == _lib.CSA_ERR_DIM
    assert _sparse(_flash(window=0)) == _lib.CSA_ERR_DIM
    assert _sparse(_flash(softmax_scale=float("nan"))) == _lib.CSA_ERR_DIM
    assert _sparse(_flash(softmax_scale=-1.0)) == _lib.CSA_ERR_DIM
    assert _scores(_fixture(index_heads=0)) == _lib.CSA_ERR_DIM


def test_unsupported_shapes():
    assert _scores(_flash(index_heads=32)) == _lib.CSA_ERR_UNSUPPORTED
    assert _scores(_flash(index_dim=64)) == _lib.CSA_ERR_UNSUPPORTED
    assert _scores(_flash(dtype=7)) == _lib.CSA_ERR_UNSUPPORTED
    assert _scores(_flash(index_act=5)) == _lib.CSA_ERR_UNSUPPORTED
    assert _sparse(_flash(n_heads=96)) == _lib.CSA_ERR_UNSUPPORTED  # bf16 attention: 64 or 128 heads
    assert _sparse(_flash(head_dim=256)) == _lib.CSA_ERR_UNSUPPORTED
    assert _sparse(_fixture(head_dim=1024)) == _lib.CSA_ERR_UNSUPPORTED
    assert _scores(_fixture(index_dim=256)) == _lib.CSA_ERR_UNSUPPORTED


def test_misaligned_pointers():
    assert _scores(_flash(), q_idx=MIS) == _lib.CSA_ERR_ALIGN
    assert _scores(_flash(), out=MIS) == _lib.CSA_ERR_ALIGN
    assert _scores(_flash(), k=FAKE + 4) == _lib.CSA_ERR_ALIGN
    assert _sparse(_flash(), q=MIS) == _lib.CSA_ERR_ALIGN
    assert _sparse(_flash(), out=MIS) == _lib.CSA_ERR_ALIGN


def test_workspace_checks():
    d = _flash(max_entries=262144)
    need = csa.workspace_size(d, _lib.CSA_OP_TOPK)
    assert need > 0
    assert _topk(d) == _lib.CSA_ERR_WORKSPACE
    assert _topk(d, ws=FAKE, nws=need - 1) == _lib.CSA_ERR_WORKSPACE
    h = _flash(ratio=128, max_entries=8192)
    assert csa.workspace_size(h, _lib.CSA_OP_HCA_MQA) > 0
    assert _hca(h) == _lib.CSA_ERR_WORKSPACE
    f = _flash()
    assert _fused(f, ws=FAKE, nws=csa.workspace_size(f, _lib.CSA_OP_ATTENTION) - 1) == _lib.CSA_ERR_WORKSPACE


def test_noalloc_rejects_before_any_launch():
    """The allocation-free fused call checks its sizes first: dims errors as
    csa_attention, and a work area beyond its 64 MiB static one (the 2,048-query
    prefill chunk needs its 2 GiB of scores) is refused before any HIP call."""
    L = csa.load_library()

    def call(dims, q_idx=FAKE):
        return L.csa_attention_noalloc(ctypes.byref(dims), FAKE, q_idx, FAKE, FAKE, FAKE, None, FAKE, None, FAKE,
                                       FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, None)

    assert L.csa_attention_noalloc(None, *([FAKE] * 17), None) == _lib.CSA_ERR_NULL
    assert call(_flash(batch=0)) == _lib.CSA_ERR_DIM
    assert call(_flash(n_heads=96)) == _lib.CSA_ERR_UNSUPPORTED
    prefill = _flash(batch=1, q_len=2048, max_entries=262144)
    assert csa.workspace_size(prefill, _lib.CSA_OP_ATTENTION) > 64 << 20
    assert call(prefill) == _lib.CSA_ERR_WORKSPACE
    assert "static" in L.csa_last_error().decode()
    # the decode shapes fit its work area
    for d in (_flash(), _flash(batch=32, max_entries=32768), _flash(n_heads=128, topk=1024)):
        assert csa.workspace_size(d, _lib.CSA_OP_ATTENTION) <= 64 << 20


def test_workspace_sizes():
    # short rows are selected by one workgroup in LDS: no workspace
    assert csa.workspace_size(_flash(max_entries=4096), _lib.CSA_OP_TOPK) == 0
    assert csa.workspace_size(_flash(max_entries=4097), _lib.CSA_OP_TOPK) > 0
    assert csa.workspace_size(_fixture(), _lib.CSA_OP_ATTENTION) >= 2 * 128 * 4 + 2 * 32 * 4
    big = csa.workspace_size(_flash(max_entries=262144), _lib.CSA_OP_ATTENTION)
    assert big >= 4 * 262144 * 4 + 4 * 512 * 4
    with pytest.raises(csa.CsaError):
        csa.workspace_size(_flash(), 99)


def test_status_strings():
    L = csa.load_library()
    for s in range(7):
        assert L.csa_status_string(s).decode().startswith("CSA_")
    assert b"unknown" in L.csa_status_string(42)


def test_product_path_has_no_fallback(monkeypatch):
    """Without the built library every entry point raises: nothing falls back to the CPU."""
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load_library("/nonexistent/libcsa.so")


def _scores_fp8(dims, q8=FAKE, qs=FAKE, w=FAKE, k8=FAKE, ks=FAKE, out=FAKE):
    return csa.load_library().csa_index_scores_fp8(ctypes.byref(dims), q8, qs, w, k8, ks, FAKE, FAKE, out, None)


def test_fp8_scorer_validation_before_any_launch():
    """Shape, pointer and alignment errors come back before anything is enqueued."""
    flash = csa.make_dims(batch=1, max_entries=16384)
    assert _scores_fp8(_fixture()) == _lib.CSA_ERR_UNSUPPORTED          # index dims 4 x 16
    assert _scores_fp8(flash, qs=None) == _lib.CSA_ERR_NULL
    assert _scores_fp8(flash, ks=None) == _lib.CSA_ERR_NULL
    assert _scores_fp8(flash, q8=MIS) == _lib.CSA_ERR_ALIGN
    assert _scores_fp8(flash, k8=FAKE + 4) == _lib.CSA_ERR_ALIGN
    bad_act = csa.make_dims(batch=1, max_entries=16384, index_act=7)
    assert _scores_fp8(bad_act) == _lib.CSA_ERR_UNSUPPORTED


def _compress(dims, ws_bytes=1 << 30, x=FAKE, out=FAKE, ws=FAKE):
    return csa.load_library().csa_compress(ctypes.byref(dims), x, FAKE, FAKE, FAKE, FAKE, out, ws, ws_bytes, None)


def test_compressor_validation_before_any_launch():
    """Window coverage, sizes, pointers, alignment and workspace are checked before anything is enqueued."""
    ok = dict(tokens=8, hidden=4096, out_dim=512, ratio=4, window=8, first_entry=1000, n_entries=1, pos0=3996,
              rope_dims=64)
    d = csa.make_compress_dims(**ok)
    assert csa.compress_workspace_size(d) > 0
    assert _compress(csa.make_compress_dims(**{**ok, "pos0": 3997})) == _lib.CSA_ERR_DIM       # first window row missing
    assert _compress(csa.make_compress_dims(**{**ok, "tokens": 7})) == _lib.CSA_ERR_DIM         # last window row missing
    assert _compress(csa.make_compress_dims(**{**ok, "out_dim": 192})) == _lib.CSA_ERR_UNSUPPORTED
    assert _compress(csa.make_compress_dims(**{**ok, "hidden": 4000})) == _lib.CSA_ERR_DIM
    assert _compress(csa.make_compress_dims(**{**ok, "window": 3})) == _lib.CSA_ERR_DIM          # window < ratio
    assert _compress(csa.make_compress_dims(**{**ok, "rope_dims": 63})) == _lib.CSA_ERR_DIM
    assert _compress(csa.make_compress_dims(**{**ok, "n_entries": 0})) == _lib.CSA_ERR_DIM
    # entry 0's window is cut at position 0, so x may start there
    assert csa.compress_workspace_size(csa.make_compress_dims(**{**ok, "first_entry": 0, "pos0": 0})) > 0
    assert _compress(d, x=None) == _lib.CSA_ERR_NULL
    assert _compress(d, x=MIS) == _lib.CSA_ERR_ALIGN
    assert _compress(d, ws_bytes=16) == _lib.CSA_ERR_WORKSPACE
    assert csa.load_library().csa_compress(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == _lib.CSA_ERR_NULL
