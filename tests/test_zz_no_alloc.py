"""dsa_sparse_attention_decode_noalloc (scratch in the library's static per-GPU array)
against dsa_sparse_attention_decode with a workspace of its own, bit for bit, on two calls in
a row whose second batch is smaller (it finds the array as the first call left it)."""
import pytest
import torch

import sparse_attention_08_amd as dsa
import workloads
from helpers import dev_rows, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _call(wl, noalloc):
    R = wl.num_rows
    logits = torch.full((R, wl.max_row_len), float("nan"), dtype=torch.float32, device=DEV)
    idx = torch.full((R, wl.topk), -7, dtype=torch.int32, device=DEV)
    out = torch.full((R, wl.H, wl.D_v), float("nan"), dtype=wl.q.dtype, device=DEV)
    lse = torch.full((R, wl.H), float("nan"), dtype=torch.float32, device=DEV)
    dsa.sparse_attention_decode(dev_rows(wl), wl.q_idx, wl.w, wl.k_idx, logits, wl.topk, wl.q,
                                wl.kv, wl.scale, wl.D_v, idx=idx, out=out, lse=lse,
                                q_scale=wl.q_scale, k_scale=wl.k_scale, noalloc=noalloc)
    return torch.nan_to_num(logits, nan=-1.0), idx, out, lse


def test_noalloc_decode_matches_workspace_call_twice():
    big = workloads.decode([131072] * 4, idx_dtype="fp8", seed=501, device=DEV,
                           name="noalloc_fp8_4x128k")
    small = workloads.decode([9000, 3000, 40961], idx_dtype="bf16", seed=502, device=DEV,
                             name="noalloc_bf16_ragged")
    for wl in (big, small):
        need = dsa.sparse_attention_decode_workspace_size(wl.num_rows, wl.max_row_len,
                                                          wl.q_idx.dtype, wl.topk, wl.H, wl.D_v)
        assert 0 < need <= 64 << 20
        say(f"noalloc decode {wl.name} (scratch {need} B)")
        got = _call(wl, True)
        ref = _call(wl, False)
        torch.cuda.synchronize()
        for g, r, name in zip(got, ref, ("logits", "idx", "out", "lse")):
            assert torch.equal(g, r), f"{wl.name}: {name} differs"
