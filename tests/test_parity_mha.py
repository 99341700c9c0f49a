"""GPU parity of the masked MHA mode (short prefill) against the oracle.

Tolerance: max-abs-relative 2e-2 on out and lse, as for the bf16 attention (the decompressed
keys and values are rounded to bf16, then the bf16 products of the attention).  The oracle
decompresses in fp64.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_08_amd as dsa
import workloads
from helpers import TOL, dev_rows, oracle_rows, say

pytestmark = pytest.mark.gpu

DEV = "cuda"
raw = workloads.raw_numpy


def _check(mb, which, idx=None, tol=TOL["bf16"]):
    wl = mb.wl
    R, H = mb.q.shape[0], mb.q.shape[1]
    say(f"mha {wl.name} H={H} R={R} {'masked' if idx is not None else 'dense'}")
    out = torch.full((R, H, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((R, H), float("nan"), dtype=torch.float32, device=DEV)
    dsa.mha_prefill(dev_rows(wl), mb.q, wl.kv, mb.w_uk, mb.w_uv, mb.scale, idx=idx, out=out,
                    lse=lse)
    K, V = oracle.mha_decompress(raw(wl.kv), raw(mb.w_uk), raw(mb.w_uv))
    ref_o, ref_l = oracle.mha(raw(mb.q), K, V, oracle_rows(wl), mb.scale,
                              idx=None if idx is None else raw(idx), which=which)
    o = out.float().cpu().numpy()[which]
    l = lse.cpu().numpy()[which]
    err = oracle.max_abs_rel(o, ref_o)
    assert err <= tol, f"mha out err {err}"
    lerr = oracle.max_abs_rel(l, ref_l)
    assert lerr <= tol, f"mha lse err {lerr}"
    return out


@pytest.mark.parametrize("paged", [False, True])
def test_dense_mode_ragged_prefill(paged):
    """Two sequences prefilled together (300 and 77 tokens: 64-row tiles that straddle the two
    sequences, a ragged last key tile), all 128 heads, every row: dense causal mode."""
    mb = workloads.mha_batch([300, 77], paged=paged, seed=61, device=DEV)
    assert dsa.prefill_dense_mode(mb.wl.max_row_len, 2048)
    _check(mb, list(range(mb.wl.num_rows)))


def test_masked_mode_topk_sets():
    """A 700-token prefill with top-64 sets (a random subset of each longer row's positions,
    -1 padded for short rows): the masked mode attends over exactly the set; 16 heads."""
    mb = workloads.mha_batch([700], H=16, seed=62, device=DEV)
    R, k = mb.wl.num_rows, 64
    g = np.random.default_rng(7)
    idx = np.full((R, k), -1, np.int32)
    for r in range(R):
        n = r + 1
        pick = g.choice(n, size=min(n, k), replace=False)
        idx[r, :len(pick)] = np.sort(pick)[::-1] if r % 2 else pick   # order does not matter
    _check(mb, list(range(0, R, 7)) + [R - 1], idx=torch.from_numpy(idx).to(DEV))


def test_masked_mode_topk_sets_paged():
    """The masked mode on a paged cache (pages permuted): a 700-token prefill with top-64 sets
    (a random subset of each longer row's positions, -1 padded); 16 heads."""
    mb = workloads.mha_batch([700], H=16, paged=True, seed=66, device=DEV)
    R, k = mb.wl.num_rows, 64
    g = np.random.default_rng(8)
    idx = np.full((R, k), -1, np.int32)
    for r in range(R):
        pick = g.choice(r + 1, size=min(r + 1, k), replace=False)
        idx[r, :len(pick)] = pick
    _check(mb, list(range(0, R, 5)) + [R - 1], idx=torch.from_numpy(idx).to(DEV))


def test_chunk_over_cached_prefix_paged():
    """A chunk of 96 new rows over a 1500-token prefix in a paged cache (rows start mid-tile),
    dense causal over the whole sequence."""
    mb = workloads.mha_batch([1596], new=[96], H=32, paged=True, seed=63, device=DEV)
    _check(mb, list(range(mb.wl.num_rows)))


def test_dense_equals_masked_with_every_position():
    """The dense mode and the masked mode with every position listed agree bit for bit."""
    mb = workloads.mha_batch([130], H=8, seed=64, device=DEV)
    R = mb.wl.num_rows
    idx = torch.full((R, 130), -1, dtype=torch.int32, device=DEV)
    for r in range(R):
        idx[r, :r + 1] = torch.arange(r + 1, dtype=torch.int32)
    say("mha dense vs full mask")
    a = dsa.mha_prefill(dev_rows(mb.wl), mb.q, mb.wl.kv, mb.w_uk, mb.w_uv, mb.scale)
    b = dsa.mha_prefill(dev_rows(mb.wl), mb.q, mb.wl.kv, mb.w_uk, mb.w_uv, mb.scale, idx=idx)
    assert torch.equal(a, b)
