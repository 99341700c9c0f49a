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


def _outputs(mb, idx=None, kv=None, rows=None):
    wl = mb.wl
    R, H = mb.q.shape[0], mb.q.shape[1]
    out = torch.full((R, H, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((R, H), float("nan"), dtype=torch.float32, device=DEV)
    dsa.mha_prefill(rows or dev_rows(wl), mb.q, wl.kv if kv is None else kv, mb.w_uk, mb.w_uv,
                    mb.scale, idx=idx, out=out, lse=lse)
    return out, lse


@pytest.mark.parametrize("paged", [False, True])
def test_foreign_cache_rows_are_never_read(paged):
    """The cache also holds rows no sequence of the batch reaches, filled with NaN: the pages
    the page table lists past each sequence's end (paged), or rows in front of and between
    the sequences (contiguous).  The results equal those on the plain cache bit for bit, and
    the workspace does not grow with the cache."""
    mb = workloads.mha_batch([300, 77], H=16, paged=paged, seed=67, device=DEV)
    wl = mb.wl
    say(f"mha foreign rows {'paged' if paged else 'contiguous'}")
    ref_o, ref_l = _outputs(mb)
    if paged:
        P = wl.kv.shape[0]
        F = 5
        kv2 = torch.cat([wl.kv, torch.full((F, 64, 576), float("nan"), dtype=wl.kv.dtype,
                                           device=DEV)])
        pt = wl.page_table.clone()
        tail = pt < 0
        pt[tail] = P + torch.arange(int(tail.sum()), device=DEV, dtype=torch.int32) % F
        rows = dsa.Rows(wl.row_seq, wl.row_len, wl.max_row_len, wl.num_seqs, page_table=pt)
    else:
        pad = 1000
        kv2 = torch.cat([torch.full((pad, 576), float("nan"), dtype=wl.kv.dtype, device=DEV),
                         wl.kv[:300], torch.full((pad, 576), float("nan"), dtype=wl.kv.dtype,
                                                 device=DEV), wl.kv[300:]])
        ss = torch.tensor([pad, 2 * pad + 300], dtype=torch.int64, device=DEV)
        rows = dsa.Rows(wl.row_seq, wl.row_len, wl.max_row_len, wl.num_seqs, seq_start=ss)
    o, l = _outputs(mb, kv=kv2, rows=rows)
    assert torch.isfinite(o.float()).all()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
    assert dsa.mha_prefill_workspace_size(2, 16, wl.num_rows, wl.max_row_len, False) < \
        kv2.numel() // 576 * 16 * 512


def test_hip_graph_replays_match_eager_mha_and_dispatch():
    """The MHA mode (dense and masked) and the prefill dispatch in both forms, captured once in
    a HIP graph and replayed three times with eager work in between: every replay equals the
    eager call bit for bit."""
    mb = workloads.mha_batch([600], H=128, H_I=64, seed=68, device=DEV)
    wl = mb.wl
    R, H, k = wl.num_rows, 128, 256
    logits = torch.empty((R, wl.max_row_len), dtype=torch.float32, device=DEV)
    idx = torch.empty((R, k), dtype=torch.int32, device=DEV)
    dsa.indexer_topk(dev_rows(wl), wl.q_idx, wl.w, wl.k_idx, logits, k, idx=idx)
    cases = {}
    for name in ("dense", "masked", "dispatch_mha", "dispatch_mqa"):
        out = torch.empty((R, H, 128), dtype=torch.bfloat16, device=DEV)
        lg = torch.empty_like(logits)
        ix = torch.empty_like(idx)
        if name == "dense":
            ws = torch.empty(dsa.mha_prefill_workspace_size(1, H, R, R, False), dtype=torch.uint8,
                             device=DEV)
            fn = lambda out=out, ws=ws: dsa.mha_prefill(dev_rows(wl), mb.q, wl.kv, mb.w_uk,
                                                        mb.w_uv, mb.scale, out=out, ws=ws)
        elif name == "masked":
            ws = torch.empty(dsa.mha_prefill_workspace_size(1, H, R, R, True), dtype=torch.uint8,
                             device=DEV)
            fn = lambda out=out, ws=ws: dsa.mha_prefill(dev_rows(wl), mb.q, wl.kv, mb.w_uk,
                                                        mb.w_uv, mb.scale, idx=idx, out=out, ws=ws)
        else:
            t = R if name == "dispatch_mha" else 0
            ws = torch.empty(dsa.sparse_attention_prefill_workspace_size(
                R, 1, R, wl.q_idx.dtype, k, H, t), dtype=torch.uint8, device=DEV)
            fn = lambda out=out, ws=ws, t=t, lg=lg, ix=ix: dsa.sparse_attention_prefill(
                dev_rows(wl), wl.q_idx, wl.w, wl.k_idx, lg, k, mb.q, wl.kv, mb.w_uk, mb.w_uv,
                mb.scale, t, idx=ix, out=out, ws=ws)
        cases[name] = (fn, out)
    for name, (fn, out) in cases.items():
        say(f"graph replay {name}")
        fn()
        torch.cuda.synchronize()
        eager = out.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        for rep in range(3):
            out.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), f"{name}: replay {rep} differs"
            junk = torch.randn(1 << 20, device=DEV)   # eager work between the replays
            junk.sum().item()
        del graph


@pytest.mark.parametrize("paged", [False, True])
def test_prefill_dispatch_both_forms_against_the_oracle(paged):
    """dsa_sparse_attention_prefill on one 300-token sequence with top-96 selection, in both
    forms: the masked MHA mode (threshold 300) and the MQA path (threshold 0: absorbed query,
    sparse MLA over the latent, output through W_UV).  Both select the same idx (the indexer
    and top-k calls), and both match the oracle's MHA over that set (decompression in fp64)
    on sampled rows; the short rows (at most 96 positions) are dense."""
    mb = workloads.mha_batch([300], H=128, H_I=64, paged=paged, seed=69, device=DEV)
    wl = mb.wl
    R, H, k = wl.num_rows, 128, 96
    which = list(range(0, R, 13)) + [R - 1]
    K, V = oracle.mha_decompress(raw(wl.kv), raw(mb.w_uk), raw(mb.w_uv))
    outs = {}
    for t in (R, 0):
        say(f"prefill dispatch threshold {t} {'paged' if paged else 'contiguous'}")
        logits = torch.empty((R, wl.max_row_len), dtype=torch.float32, device=DEV)
        idx = torch.full((R, k), -7, dtype=torch.int32, device=DEV)
        out = torch.full((R, H, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full((R, H), float("nan"), dtype=torch.float32, device=DEV)
        dsa.sparse_attention_prefill(dev_rows(wl), wl.q_idx, wl.w, wl.k_idx, logits, k, mb.q,
                                     wl.kv, mb.w_uk, mb.w_uv, mb.scale, t, idx=idx, out=out,
                                     lse=lse)
        ref_o, ref_l = oracle.mha(raw(mb.q), K, V, oracle_rows(wl), mb.scale, idx=raw(idx),
                                  which=which)
        err = oracle.max_abs_rel(out.float().cpu().numpy()[which], ref_o)
        lerr = oracle.max_abs_rel(lse.cpu().numpy()[which], ref_l)
        assert err <= TOL["bf16"] and lerr <= TOL["bf16"], f"threshold {t}: {err} {lerr}"
        outs[t] = (idx, out)
    assert torch.equal(outs[R][0], outs[0][0])   # one selection
