"""The Python binding refuses mis-sized tensors with ValueError before any call into the
library: the C ABI receives raw pointers and could not tell.  The shape helpers are checked
on the CPU; every public wrapper is checked on the GPU with one mis-sized argument at a time
(nothing is launched: the checks come first)."""
import types

import pytest
import torch

import sparse_attention_08_amd as dsa


def _rows(R=3, L=100, paged=False):
    return types.SimpleNamespace(num_rows=R, max_row_len=L, paged=paged, page_size=64, num_seqs=2)


def test_shape_helpers_on_cpu():
    t = torch.empty(3, 4)
    dsa._shape(t, "t", (3, 4))
    dsa._shape(t, "t", (None, 4))
    dsa._shape(None, "t", (1, 2))
    for bad in ((3, 5), (4, 4), (3,), (3, 4, 1)):
        with pytest.raises(ValueError):
            dsa._shape(t, "t", bad)
    dsa._rows_of(_rows(R=3), t, "t")
    with pytest.raises(ValueError):
        dsa._rows_of(_rows(R=2), t, "t")
    dsa._logits_shape(_rows(R=3, L=4), t)
    with pytest.raises(ValueError):
        dsa._logits_shape(_rows(R=3, L=5), t)          # rows shorter than max_row_len
    with pytest.raises(ValueError):
        dsa._logits_shape(_rows(R=3, L=4), torch.empty(12))
    dsa._key_cache_shape(_rows(), torch.empty(10, 128), 128, torch.empty(10))
    with pytest.raises(ValueError):
        dsa._key_cache_shape(_rows(), torch.empty(10, 128), 128, torch.empty(9))
    dsa._key_cache_shape(_rows(paged=True), torch.empty(2, 64, 128), 128, torch.empty(2, 64))
    with pytest.raises(ValueError):
        dsa._key_cache_shape(_rows(paged=True), torch.empty(128, 128), 128, None)
    with pytest.raises(ValueError):
        dsa._latent_cache_shape(_rows(), torch.empty(10, 512), 576)
    q = torch.empty(3, 64, 128)
    dsa._indexer_shapes(_rows(), q, torch.empty(3, 64), torch.empty(9, 128), torch.empty(3, 100),
                        None, None)
    for kw in ({"w": torch.empty(3, 32)}, {"logits": torch.empty(2, 100)},
               {"q_scale": torch.empty(3, 63)}, {"k": torch.empty(9, 64)}):
        args = {"w": torch.empty(3, 64), "k": torch.empty(9, 128), "logits": torch.empty(3, 100),
                "q_scale": None}
        args.update(kw)
        with pytest.raises(ValueError):
            dsa._indexer_shapes(_rows(), q, args["w"], args["k"], args["logits"], args["q_scale"],
                                None)


@pytest.mark.gpu
def test_public_wrappers_refuse_mis_sized_tensors():
    dev = "cuda"
    R, L, k, H = 3, 100, 16, 128
    rows = dsa.Rows(torch.zeros(R, dtype=torch.int32, device=dev),
                    torch.full((R,), L, dtype=torch.int32, device=dev), L, 1,
                    seq_start=torch.zeros(1, dtype=torch.int64, device=dev))
    bf = dict(dtype=torch.bfloat16, device=dev)
    q_idx = torch.zeros(R, 64, 128, **bf)
    w = torch.zeros(R, 64, dtype=torch.float32, device=dev)
    k_idx = torch.zeros(L, 128, **bf)
    logits = torch.zeros(R, L, dtype=torch.float32, device=dev)
    q = torch.zeros(R, H, 576, **bf)
    kv = torch.zeros(L, 576, **bf)
    idx = torch.zeros(R, k, dtype=torch.int32, device=dev)
    cases = [
        lambda: dsa.indexer_logits(rows, q_idx[:2], w, k_idx, logits),
        lambda: dsa.indexer_logits(rows, q_idx, torch.zeros(R, 32, dtype=torch.float32, device=dev), k_idx, logits),
        lambda: dsa.indexer_logits(rows, q_idx, w, k_idx, torch.zeros(R, 50, dtype=torch.float32, device=dev)),
        lambda: dsa.topk(logits, rows.row_len[:2], k, L),
        lambda: dsa.topk(logits, rows.row_len, k, L, idx=torch.zeros(R, 8, dtype=torch.int32, device=dev)),
        lambda: dsa.indexer_topk(rows, q_idx, w, k_idx, logits, k, idx=idx[:2]),
        lambda: dsa.sparse_mla_decode(rows, q[:2], kv, idx, 0.1, 512),
        lambda: dsa.sparse_mla_decode(rows, q, torch.zeros(L, 512, **bf), idx, 0.1, 512),
        lambda: dsa.sparse_mla_decode(rows, q, kv, idx[:2], 0.1, 512),
        lambda: dsa.sparse_mla_decode(rows, q, kv, idx, 0.1, 512,
                                      out=torch.zeros(R, H, 256, **bf)),
        lambda: dsa.sparse_mla_decode(rows, q, kv, idx, 0.1, 512,
                                      lse=torch.zeros(R, 64, dtype=torch.float32, device=dev)),
        lambda: dsa.sparse_attention_decode(rows, q_idx, w, k_idx, logits, k, q, kv, 0.1, 512,
                                            idx=torch.zeros(R, 8, dtype=torch.int32, device=dev)),
        lambda: dsa.sparse_attention_decode(rows, q_idx, w, k_idx, logits, k, q, kv, 0.1, 512,
                                            out=torch.zeros(R, 64, 512, **bf)),
        lambda: dsa.mha_prefill(rows, torch.zeros(R, H, 128, **bf), kv,
                                torch.zeros(H, 128, 512, **bf), torch.zeros(H, 128, 512, **bf), 0.1),
        lambda: dsa.mha_prefill(rows, torch.zeros(R, H, 192, **bf), kv,
                                torch.zeros(H, 64, 512, **bf), torch.zeros(H, 128, 512, **bf), 0.1),
        lambda: dsa.sparse_attention_prefill(rows, q_idx, w, k_idx, logits, k,
                                             torch.zeros(R, H, 192, **bf), kv,
                                             torch.zeros(H, 128, 512, **bf),
                                             torch.zeros(H, 128, 512, **bf), 0.1, 0,
                                             idx=torch.zeros(R, 4, dtype=torch.int32,
                                                             device=dev)),
    ]
    for i, fn in enumerate(cases):
        with pytest.raises(ValueError, match="shape|rows|must be|scores"):
            fn()
        torch.cuda.synchronize()
