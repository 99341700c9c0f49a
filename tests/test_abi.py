"""The C ABI of libdsa.so, checked without a GPU: it loads, exports every function that
include/dsa.h declares, and rejects bad arguments on the host before any HIP call.

Only argument combinations that fail validation (or are empty) are passed here, so no
kernel is ever launched; the fake device pointers are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import sparse_attention_08_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")
FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every call below fails validation first

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    return dsa.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert "dsa_indexer_logits" in names and "dsa_sparse_mla_decode_paged" in names
    assert "dsa_indexer_topk" in names and "dsa_indexer_topk_workspace_size" in names
    for n in names:
        assert hasattr(lib, n), f"libdsa.so does not export {n}"


def test_version_and_status_strings(lib):
    assert dsa.abi_version() == 2
    assert dsa.status_string(0) == "DSA_OK"
    for s in (1, 2, 3, 4):
        assert dsa.status_string(s).startswith(dsa.STATUS[s])
    assert "unknown" in dsa.status_string(99)


def _rows(num_rows=2, num_seqs=2, max_row_len=100, paged=False, page_size=64, max_pages=None,
          seq_start=True, page_table=None, row_ptrs=True):
    if max_pages is None:
        max_pages = (max_row_len + 63) // 64 if paged else 0
    return dsa.DsaRows(num_rows, num_seqs, FAKE if row_ptrs else None, FAKE if row_ptrs else None,
                       max_row_len, FAKE if (seq_start and not paged) else None,
                       FAKE if (paged or page_table) else None, max_pages, page_size if paged else 0)


def _idx(lib, rows, dtype=1, H=64, D=128, ld=100, qs=None, ks=None, paged=False, ptrs=True):
    fn = lib.dsa_indexer_logits_paged if paged else lib.dsa_indexer_logits
    p = FAKE if ptrs else None
    return fn(ctypes.byref(rows) if rows is not None else None, dtype, H, D, p, qs, p, ks, p, p, ld,
              None)


def test_indexer_validation(lib):
    assert _idx(lib, None) == INVALID
    assert _idx(lib, _rows(num_rows=0)) == OK                       # empty batch: nothing launched
    assert _idx(lib, _rows(row_ptrs=False)) == INVALID
    assert _idx(lib, _rows(num_seqs=0)) == INVALID
    assert _idx(lib, _rows(max_row_len=0)) == INVALID
    assert _idx(lib, _rows(), ld=99) == INVALID                     # ld < max_row_len
    assert _idx(lib, _rows(), dtype=7) == INVALID
    assert _idx(lib, _rows(), H=0) == INVALID
    assert _idx(lib, _rows(), ptrs=False) == INVALID
    assert _idx(lib, _rows(), dtype=2) == INVALID                   # fp8 without scales
    assert _idx(lib, _rows(), dtype=2, qs=FAKE) == INVALID          # fp8 missing k scale
    assert _idx(lib, _rows(), dtype=1, qs=FAKE, ks=FAKE) == INVALID  # scales only for fp8
    assert _idx(lib, _rows(), dtype=1, H=32, D=128) == UNSUPPORTED
    assert _idx(lib, _rows(), dtype=2, H=64, D=64, qs=FAKE, ks=FAKE) == UNSUPPORTED
    assert _idx(lib, _rows(), dtype=0, H=65, D=32) == UNSUPPORTED
    # layout must match the entry point
    assert _idx(lib, _rows(page_table=True)) == INVALID             # both layouts given
    assert _idx(lib, _rows(seq_start=False)) == INVALID             # neither
    assert _idx(lib, _rows(paged=True), paged=True, dtype=9) == INVALID
    assert _idx(lib, _rows(), paged=True) == INVALID                # contiguous rows, paged call
    assert _idx(lib, _rows(paged=True, page_size=32), paged=True) == INVALID
    assert _idx(lib, _rows(paged=True, max_row_len=200, max_pages=3), paged=True) == INVALID
    assert _idx(lib, _rows(paged=True, num_rows=0), paged=True) == OK


def test_topk_validation(lib):
    f = lib.dsa_topk
    assert f(FAKE, 100, FAKE, 4, 100, 0, FAKE, None, 0, None) == INVALID       # k = 0
    assert f(FAKE, 100, FAKE, 4, 100, 2049, FAKE, None, 0, None) == INVALID    # k > 2048
    assert f(FAKE, 99, FAKE, 4, 100, 16, FAKE, None, 0, None) == INVALID       # ld < max_row_len
    assert f(None, 100, FAKE, 4, 100, 16, FAKE, None, 0, None) == INVALID
    assert f(FAKE, 100, FAKE, -1, 100, 16, FAKE, None, 0, None) == INVALID
    assert f(FAKE, 100, FAKE, 0, 100, 16, FAKE, None, 0, None) == OK           # empty batch
    assert f(FAKE, 100, FAKE, 4, 0, 16, FAKE, None, 0, None) == INVALID
    assert dsa.topk_workspace_size(4, 100, 0) == 0


def test_indexer_topk_validation(lib):
    def call(rows, dtype=1, ld=100, topk=16, idx=True, ws=None, ws_bytes=0, qs=None, ks=None,
             name="dsa_indexer_topk"):
        return getattr(lib, name)(ctypes.byref(rows), dtype, 64, 128, FAKE, qs, FAKE, ks, FAKE, FAKE,
                                  ld, topk, FAKE if idx else None, ws, ws_bytes, None)
    r = _rows()
    assert call(r, topk=0) == INVALID
    assert call(r, topk=2049) == INVALID
    assert call(r, idx=False) == INVALID
    assert call(r, ld=99) == INVALID
    assert call(r, dtype=2) == INVALID                                 # fp8 without scales
    assert call(_rows(num_rows=0)) == OK
    assert call(r, name="dsa_indexer_topk_paged") == INVALID           # layout mismatch
    # few long rows: the leading-digit histograms live in the workspace
    big = _rows(num_rows=8, num_seqs=8, max_row_len=131072)
    need = lib.dsa_indexer_topk_workspace_size(8, 131072, 2, 2048)
    assert need >= dsa.topk_workspace_size(8, 131072, 2048) > 0
    assert call(big, dtype=2, ld=131072, topk=2048, qs=FAKE, ks=FAKE) == WORKSPACE
    assert call(big, dtype=2, ld=131072, topk=2048, qs=FAKE, ks=FAKE, ws=FAKE,
                ws_bytes=need - 1) == WORKSPACE
    assert lib.dsa_indexer_topk_workspace_size(8, 131072, 7, 2048) == 0   # bad dtype


def _mla(lib, rows, name="dsa_sparse_mla_decode", dtype=1, H=128, Dqk=576, Dv=512, scale=0.07,
         k=2048, ws=None, ws_bytes=0, ptrs=True):
    p = FAKE if ptrs else None
    return getattr(lib, name)(ctypes.byref(rows), dtype, H, Dqk, Dv, scale, p, p, p, k, p, None, ws,
                              ws_bytes, None)


def test_mla_validation(lib):
    r8 = _rows(num_rows=8, num_seqs=8)
    assert _mla(lib, r8, k=0) == INVALID
    assert _mla(lib, r8, k=2049) == INVALID
    assert _mla(lib, r8, Dv=600) == INVALID                         # d_v > d_qk
    assert _mla(lib, r8, scale=float("nan")) == INVALID
    assert _mla(lib, r8, scale=float("inf")) == INVALID
    assert _mla(lib, r8, scale=0.0) == INVALID
    assert _mla(lib, r8, scale=-0.07) == INVALID
    assert _mla(lib, r8, ptrs=False) == INVALID
    assert _mla(lib, r8, H=96) == UNSUPPORTED
    assert _mla(lib, r8, H=64) == UNSUPPORTED
    assert _mla(lib, r8, Dqk=512) == UNSUPPORTED
    assert _mla(lib, r8, dtype=2) == UNSUPPORTED                    # no fp8 attention
    assert _mla(lib, r8, dtype=0, H=129, Dqk=80, Dv=64) == UNSUPPORTED
    # eight rows split the 2048 slots over several workgroups: a workspace is required
    need = dsa.sparse_mla_workspace_size(8, 128, 512, 2048)
    assert need > 0
    assert _mla(lib, r8) == WORKSPACE
    assert _mla(lib, r8, ws=FAKE, ws_bytes=need - 1) == WORKSPACE
    assert _mla(lib, _rows(num_rows=0)) == OK
    assert _mla(lib, _rows(), name="dsa_sparse_mla_decode_paged") == INVALID   # layout mismatch
    assert _mla(lib, _rows(paged=True), name="dsa_sparse_mla_prefill") == INVALID
    assert _mla(lib, _rows(), name="dsa_sparse_mla_prefill_paged") == INVALID   # layout mismatch
    assert _mla(lib, _rows(paged=True), name="dsa_sparse_mla_prefill_paged", k=0) == INVALID
    assert _mla(lib, _rows(num_rows=0, paged=True), name="dsa_sparse_mla_prefill_paged") == OK


def test_workspace_queries_are_consistent():
    # few rows: split partials (bf16 [R, splits, H, d_v] + fp32 [R, splits, H]); many rows: none
    few = dsa.sparse_mla_workspace_size(8, 128, 512, 2048)
    assert few % (8 * 128 * (2 * 512 + 4)) == 0
    assert dsa.sparse_mla_workspace_size(4096, 128, 512, 2048) == 0
    assert dsa.sparse_mla_workspace_size(0, 128, 512, 2048) == 0


def test_attention_decode_validation(lib):
    def call(rows, idx_dtype=1, topk=2048, dtype=1, H=128, Dqk=576, Dv=512, scale=0.07, ld=None,
             ws=None, ws_bytes=0, qs=None, ks=None, ptrs=True, name="dsa_sparse_attention_decode"):
        p = FAKE if ptrs else None
        ld = rows.max_row_len if ld is None else ld
        return getattr(lib, name)(ctypes.byref(rows), idx_dtype, 64, 128, FAKE, qs, FAKE, ks, FAKE,
                                  FAKE, ld, topk, p, dtype, H, Dqk, Dv, scale, p, p, p, None, ws,
                                  ws_bytes, None)
    r = _rows()
    assert call(r, topk=0) == INVALID
    assert call(r, topk=2049) == INVALID
    assert call(r, scale=0.0) == INVALID
    assert call(r, scale=float("nan")) == INVALID
    assert call(r, Dv=600) == INVALID
    assert call(r, ptrs=False) == INVALID
    assert call(r, ld=99) == INVALID
    assert call(r, idx_dtype=2) == INVALID                      # fp8 indexer without scales
    assert call(r, name="dsa_sparse_attention_decode_paged") == INVALID   # layout mismatch
    assert call(r, dtype=2) == UNSUPPORTED                      # no fp8 attention
    assert call(r, H=64) == UNSUPPORTED
    assert call(_rows(num_rows=0)) == OK
    # few long rows: the selection's and the attention's scratch live in one workspace
    big = _rows(num_rows=8, num_seqs=8, max_row_len=131072)
    need = dsa.sparse_attention_decode_workspace_size(8, 131072, 2, 2048, 128, 512)
    assert need >= dsa.indexer_topk_workspace_size(8, 131072, 2, 2048) + \
        dsa.sparse_mla_workspace_size(8, 128, 512, 2048)
    assert call(big, idx_dtype=2, qs=FAKE, ks=FAKE) == WORKSPACE
    assert call(big, idx_dtype=2, qs=FAKE, ks=FAKE, ws=FAKE, ws_bytes=need - 1) == WORKSPACE
    assert dsa.sparse_attention_decode_workspace_size(8, 131072, 7, 2048, 128, 512) == 0


def test_prep_validation(lib):
    def keys(T=4, pos=True, rows=True, n_rows=64, cs=True, max_pos=128, dt=1, scale=None,
             ptrs=True):
        p = FAKE if ptrs else None
        return lib.dsa_prep_cache_write(T, FAKE if pos else None, FAKE if rows else None, n_rows,
                                        FAKE if cs else None, max_pos, dt, p, p, scale, p, p, None)

    def queries(R=2, max_pos=128, dt=1, scale=None, H=128, ptrs=True):
        p = FAKE if ptrs else None
        return lib.dsa_prep_queries(R, FAKE, FAKE if ptrs else None, max_pos, dt, p, p, scale, H,
                                    p, None)
    assert keys(T=0) == OK and queries(R=0) == OK                 # empty: nothing launched
    assert keys(T=-1) == INVALID and queries(R=-1) == INVALID
    assert keys(pos=False) == INVALID and keys(rows=False) == INVALID and keys(cs=False) == INVALID
    assert keys(ptrs=False) == INVALID and queries(ptrs=False) == INVALID
    assert keys(n_rows=0) == INVALID
    assert keys(max_pos=0) == INVALID and queries(max_pos=0) == INVALID
    assert keys(dt=2) == INVALID and queries(dt=2) == INVALID     # fp8 without scales
    assert keys(dt=1, scale=FAKE) == INVALID and queries(scale=FAKE) == INVALID
    assert keys(dt=0) == UNSUPPORTED and queries(dt=0) == UNSUPPORTED
    assert keys(dt=5) == INVALID and queries(dt=5) == INVALID
    assert queries(H=0) == INVALID

    def both(T=4, dt=1, ks=None, qs=None, H=128, ptrs=True):
        p = FAKE if ptrs else None
        return lib.dsa_prep(T, FAKE, FAKE, 64, FAKE, 128, dt, p, p, ks, p, p, p, p, qs, H, p, None)
    assert both(T=0) == OK
    assert both(T=-2) == INVALID and both(ptrs=False) == INVALID and both(H=0) == INVALID
    assert both(dt=2, ks=FAKE) == INVALID and both(dt=2, qs=FAKE) == INVALID   # one scale missing
    assert both(dt=1, qs=FAKE) == INVALID
    assert both(dt=0) == UNSUPPORTED


def test_mha_validation(lib):
    def call(rows, H=128, scale=0.07, idx=None, k=0, ws=None, ws_bytes=0, ptrs=True,
             name="dsa_mha_prefill"):
        p = FAKE if ptrs else None
        return getattr(lib, name)(ctypes.byref(rows), H, scale, p, p, p, p, idx, k, p, None, ws,
                                  ws_bytes, None)
    r = _rows()
    assert call(r, H=0) == INVALID
    assert call(r, scale=0.0) == INVALID and call(r, scale=float("nan")) == INVALID
    assert call(r, idx=FAKE, k=0) == INVALID and call(r, idx=FAKE, k=2049) == INVALID
    assert call(r, ptrs=False) == INVALID
    assert call(r, name="dsa_mha_prefill_paged") == INVALID            # layout mismatch
    assert call(_rows(num_rows=0)) == OK
    assert call(_rows(max_row_len=16385)) == UNSUPPORTED
    # the decompressed keys and values cover max_row_len positions of each sequence, whatever
    # the cache's size
    need = lib.dsa_mha_prefill_workspace_size(2, 128, 2, 100, 0)
    assert need >= 2 * 2 * 100 * 128 * 256
    assert lib.dsa_mha_prefill_workspace_size(2, 128, 2, 100, 1) > need   # + the masks
    assert lib.dsa_mha_prefill_workspace_size(0, 128, 2, 100, 0) == 0
    assert call(r) == WORKSPACE and call(r, ws=FAKE, ws_bytes=need - 1) == WORKSPACE
    assert lib.dsa_prefill_dense_mode(2048, 2048) == 1 and lib.dsa_prefill_dense_mode(2049, 2048) == 0
    assert lib.dsa_prefill_dense_mode(0, 2048) == 0


def test_prefill_dispatch_validation_and_sizes(lib):
    def call(rows, threshold, H=128, topk=2048, ws=None, ws_bytes=0, idx=FAKE, ptrs=True,
             name="dsa_sparse_attention_prefill"):
        p = FAKE if ptrs else None
        return getattr(lib, name)(ctypes.byref(rows), 1, 64, 128, p, None, p, None, p, p, 100,
                                  topk, idx, H, 0.07, p, p, p, p, p, None, threshold, ws,
                                  ws_bytes, None)
    r = _rows()
    size = lambda R, L, t, H=128, topk=2048: lib.dsa_sparse_attention_prefill_workspace_size(
        R, 2, L, 1, topk, H, t)
    # short batch under the threshold: the dense MHA mode (no selection, no absorption buffers)
    assert size(2, 100, 100) == lib.dsa_mha_prefill_workspace_size(2, 128, 2, 100, 0)
    # rows longer than topk under the threshold: selection + masked MHA
    assert size(2, 100, 100, topk=64) >= lib.dsa_mha_prefill_workspace_size(2, 128, 2, 100, 1)
    # over the threshold (0: always): the MQA path with its absorbed query and latent output
    assert size(2, 100, 0) >= 2 * 128 * (576 + 512) * 2 + 128 * 512 * 128 * 2
    assert size(2, 100, 99) == size(2, 100, 0)
    assert size(2, 100, 0, topk=0) == 0
    assert call(r, 0, ptrs=False) == INVALID
    assert call(r, 0, topk=0) == INVALID
    assert call(r, 0, H=64) == UNSUPPORTED or call(r, 0, H=64) == WORKSPACE
    assert call(r, 0) == WORKSPACE
    assert call(r, 0, idx=None) == INVALID                           # the selection needs idx
    assert call(r, 0, name="dsa_sparse_attention_prefill_paged") == INVALID
    assert call(_rows(num_rows=0), 0) == OK


def test_noalloc_decode_rejects_batches_beyond_its_scratch(lib):
    # 64 rows of 1M scores need far more than the static scratch: refused before any HIP call
    rows = _rows(num_rows=64, num_seqs=64, max_row_len=1 << 20)
    need = lib.dsa_sparse_attention_decode_workspace_size(64, 1 << 20, 2, 2048, 128, 512)
    assert need > (64 << 20)
    s = lib.dsa_sparse_attention_decode_noalloc(
        ctypes.byref(rows), 2, 64, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, 2048, FAKE,
        1, 128, 576, 512, 0.1, FAKE, FAKE, FAKE, None, None)
    assert s == WORKSPACE
    assert lib.dsa_sparse_attention_decode_noalloc(None, 2, 64, 128, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                   FAKE, 100, 64, FAKE, 1, 128, 576, 512, 0.1,
                                                   FAKE, FAKE, FAKE, None, None) == INVALID


def test_mfma_probe_validation(lib):
    """The matrix-core rate probe rejects a loop count outside 1 .. 1,000,000 and a null
    output before launching anything."""
    for iters in (0, -5, 1000001):
        assert lib.dsa_mfma_rate_probe(iters, FAKE, None) == INVALID
    assert lib.dsa_mfma_rate_probe(10, None, None) == INVALID
