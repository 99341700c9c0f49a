"""GPU parity: every stage of the HIP path against the fp64 oracle on the same seeded bytes.

Tolerances: indexer and attention outputs max-abs-relative <= 1e-5 (fp32) / 2e-2
(bf16, fp8 indexer); top-k index sets bit-exact, both when fed the oracle's scores
rounded to fp32 and on the GPU's own scores.  Attention is compared on the same index
set on both sides.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_08_amd as dsa
import workloads
from helpers import (TOL, dev_rows, gpu_indexer, gpu_mla, oracle_indexer, oracle_mla, raw, say,
                     valid_logits)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _check_indexer(wl, which, tol):
    say(f"indexer {wl.name} rows={list(which)[:6]}")
    g = gpu_indexer(wl).cpu().numpy()
    ref = oracle_indexer(wl, which=which)
    lens = wl.row_len.cpu().numpy()
    gv = valid_logits(g[list(which)], lens, which)
    rv = valid_logits(ref, lens, which)
    err = oracle.max_abs_rel(gv, rv)
    assert err <= tol, f"indexer err {err}"
    # nothing written beyond a row's length
    for i, r in enumerate(which):
        assert np.all(np.isnan(g[r, lens[r]:])), "wrote past row_len"
    return g, ref, err


def _check_topk_on_oracle_scores(wl, ref_scores, which):
    """GPU top-k fed the oracle's scores rounded to fp32 == oracle top-k on that array."""
    lens = wl.row_len.cpu().numpy()[list(which)]
    x32 = np.nan_to_num(ref_scores, nan=0.0).astype(np.float32)
    say(f"topk on oracle scores {wl.name}")
    logits = torch.from_numpy(x32).to(DEV)
    rl = torch.from_numpy(lens.astype(np.int32)).to(DEV)
    got = dsa.topk(logits, rl, wl.topk, int(lens.max())).cpu().numpy()
    exp = oracle.topk(x32, lens, wl.topk)
    assert np.array_equal(got, exp)


def _check_topk_on_gpu_scores(wl, g_logits):
    say(f"topk on gpu scores {wl.name}")
    lens = wl.row_len.cpu().numpy()
    got = dsa.topk(torch.from_numpy(g_logits).to(DEV), wl.row_len, wl.topk, wl.max_row_len)
    exp = oracle.topk(np.nan_to_num(g_logits, nan=0.0).astype(np.float32), lens, wl.topk)
    assert np.array_equal(got.cpu().numpy(), exp)
    return got


def _check_mla(wl, idx_dev, which, tol):
    say(f"mla {wl.name} rows={list(which)[:6]}")
    out, lse = gpu_mla(wl, idx_dev)
    o = out.float().cpu().numpy()[list(which)]
    l = lse.cpu().numpy()[list(which)]
    ref_o, ref_l = oracle_mla(wl, idx_dev.cpu().numpy(), which=which)
    err = oracle.max_abs_rel(o, ref_o)
    assert err <= tol, f"attention err {err}"
    lerr = oracle.max_abs_rel(l, ref_l)
    assert lerr <= tol, f"lse err {lerr}"
    return out, lse, err


# ------------------------------------------------------------------------ tiny fp32 prefill

def test_c1_tiny_fp32_prefill_full():
    wl = workloads.config(1).to(DEV)
    which = list(range(wl.num_rows))
    g, ref, _ = _check_indexer(wl, which, TOL["f32"])
    _check_topk_on_oracle_scores(wl, ref, which)
    idx = _check_topk_on_gpu_scores(wl, g)
    _check_mla(wl, idx, which, TOL["f32"])
    # rows with at most k predecessors select everything: sparse == dense causal MQA
    short = list(range(64))
    out, _ = gpu_mla(wl, idx)
    dense, _ = oracle.dense_mqa("f32", raw(wl.q), raw(wl.kv), oracle.Rows(
        np.zeros(256), np.arange(1, 257), seq_start=np.zeros(1)), wl.scale, wl.D_v, which=short)
    assert oracle.max_abs_rel(out.cpu().numpy()[short], dense) <= TOL["f32"]


def test_f32_paged_prefill_batch():
    """The f32 path (the tiny config's shapes: 4 x 32 indexer, 8 heads of 80 / 64) on a paged
    cache: two sequences of 200 and 77 tokens prefilled together, pages permuted; indexer,
    top-64 and attention against the oracle on every row."""
    wl = workloads.prefill_batch([200, 77], idx_dtype="f32", mla_dtype="f32", paged=True, H_I=4,
                                 D_I=32, H=8, D_qk=80, D_v=64, topk=64, seed=96, device=DEV,
                                 name="f32_paged_prefill")
    which = list(range(wl.num_rows))
    g, ref, _ = _check_indexer(wl, which, TOL["f32"])
    _check_topk_on_oracle_scores(wl, ref, which)
    idx = _check_topk_on_gpu_scores(wl, g)
    _check_mla(wl, idx, which, TOL["f32"])


@pytest.mark.parametrize("paged", [False, True])
def test_f32_at_the_advertised_bounds(paged):
    """The f32 path at the largest shapes the header allows: indexer 64 heads x 256 dims
    (65,792 bytes of query block and weights in LDS, above the default 64 KB), attention 128
    heads with d_qk = d_v = 256, over two sequences (240 and 97 tokens, k = 64 so the longer
    rows select); indexer, top-k and attention against the oracle on every row."""
    wl = workloads.prefill_batch([240, 97], idx_dtype="f32", mla_dtype="f32", paged=paged, H_I=64,
                                 D_I=256, H=128, D_qk=256, D_v=256, topk=64,
                                 scale=1.0 / math.sqrt(256.0), w_div=64.0, seed=98, device=DEV,
                                 name=f"f32_bounds_{'paged' if paged else 'contig'}")
    which = list(range(wl.num_rows))
    g, ref, _ = _check_indexer(wl, which, TOL["f32"])
    _check_topk_on_oracle_scores(wl, ref, which)
    idx = _check_topk_on_gpu_scores(wl, g)
    _check_mla(wl, idx, which, TOL["f32"])


# ------------------------------------------------------------------------ small ragged decode

RAGGED = [1, 17, 100, 2047, 2048, 2049, 3000, 5001]


@pytest.mark.parametrize("idx_dtype,paged", [("bf16", False), ("fp8", False), ("bf16", True),
                                             ("fp8", True)])
def test_ragged_decode(idx_dtype, paged):
    wl = workloads.decode(RAGGED, idx_dtype=idx_dtype, paged=paged, seed=77, device=DEV,
                          name=f"ragged_{idx_dtype}_{'paged' if paged else 'contig'}")
    which = list(range(wl.num_rows))
    g, ref, _ = _check_indexer(wl, which, TOL[idx_dtype])
    _check_topk_on_oracle_scores(wl, ref, which)
    idx = _check_topk_on_gpu_scores(wl, g)
    _check_mla(wl, idx, which, TOL["bf16"])


def test_paged_physical_permutation_is_bit_identical():
    wl = workloads.decode([700, 130, 64, 2100], paged=True, seed=31, device=DEV, name="perm")
    g1 = gpu_indexer(wl)
    idx = dsa.topk(g1, wl.row_len, wl.topk, wl.max_row_len)
    o1, l1 = gpu_mla(wl, idx)
    P = wl.kv.shape[0]
    perm = torch.randperm(P, generator=torch.Generator().manual_seed(5)).to(DEV)
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(P, device=DEV)
    wl2 = workloads.Workload(**{f: getattr(wl, f) for f in wl.__dataclass_fields__})
    # physical page p moves to slot inv[p]
    wl2.kv = wl.kv[perm].contiguous()
    wl2.k_idx = wl.k_idx[perm].contiguous()
    pt = wl.page_table.clone()
    pt[pt >= 0] = inv[pt[pt >= 0].long()].to(torch.int32)
    wl2.page_table = pt
    say("paged permutation")
    g2 = gpu_indexer(wl2)
    idx2 = dsa.topk(g2, wl2.row_len, wl2.topk, wl2.max_row_len)
    o2, l2 = gpu_mla(wl2, idx2)
    assert torch.equal(torch.nan_to_num(g1, nan=-1.0), torch.nan_to_num(g2, nan=-1.0))
    assert torch.equal(idx, idx2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ------------------------------------------------------------------------ prefill-shaped indexer

@pytest.mark.parametrize("idx_dtype,paged", [("bf16", False), ("bf16", True), ("fp8", False),
                                             ("fp8", True)])
def test_prefill_indexer_shares_key_tiles(idx_dtype, paged):
    """Batches with many rows per sequence: bf16 takes the indexer whose workgroups share key
    tiles between 8 consecutive rows (blocks that straddle sequences, rows crossing key-chunk
    boundaries), fp8 the one-row-at-a-time indexer with cached key loads; the first and last
    row of every sequence are checked."""
    lens = [13, 29, 2100]
    wl = workloads.prefill_batch(lens, idx_dtype=idx_dtype, paged=paged, seed=95, device=DEV,
                                 name=f"prefill_batch_{idx_dtype}_{'paged' if paged else 'contig'}")
    assert wl.num_rows >= 8 * wl.num_seqs
    starts = np.concatenate([[0], np.cumsum(lens)])
    which = sorted(set(range(0, 42)) | {42, 43, 49, 50, 1000, 2047 + 42, 2048 + 42, 2049 + 42,
                                        int(starts[-1]) - 2, int(starts[-1]) - 1})
    _check_indexer(wl, which, TOL[idx_dtype])


def test_chunked_prefill_over_paged_prefix():
    """New tokens over cached prefixes in a paged cache: the paged indexer (key-sharing kernel),
    the top-k and the paged attention, each against the oracle on sampled rows."""
    wl = workloads.prefill_batch([3000, 700], new=[300, 40], paged=True, seed=96, device=DEV,
                                 name="chunked_prefill_paged")
    assert wl.num_rows >= 8 * wl.num_seqs and int(wl.row_len.min()) > 600
    which = [0, 1, 7, 8, 150, 298, 299, 300, 301, 320, 339]
    g, ref, _ = _check_indexer(wl, which, TOL["bf16"])
    _check_topk_on_oracle_scores(wl, ref, which)
    idx = _check_topk_on_gpu_scores(wl, g.copy())
    _check_mla(wl, idx, which, TOL["bf16"])


# ------------------------------------------------------------------------ multi-token decode

# a few new tokens per sequence (speculative or multi-token decode) over cached contexts
MTP_LENS, MTP_NEW = [5000, 1300, 70, 9000, 2049], [4, 2, 3, 4, 2]


@pytest.mark.parametrize("idx_dtype,paged", [("bf16", False), ("fp8", False), ("bf16", True),
                                             ("fp8", True)])
def test_multi_token_decode(idx_dtype, paged):
    """Several query rows per sequence share the key stream: the key-sharing indexer in bf16 and
    fp8 (workgroups of 8 rows straddling three sequences, rows on both sides of the 2048-key
    chunk boundary), the top-k and the split attention on every row, and the one-call decode
    against the separate calls."""
    wl = workloads.prefill_batch(MTP_LENS, new=MTP_NEW, idx_dtype=idx_dtype, paged=paged, seed=97,
                                 device=DEV,
                                 name=f"mtp_{idx_dtype}_{'paged' if paged else 'contig'}")
    wl = dataclasses.replace(wl, mode="decode")
    assert wl.num_rows >= 2 * wl.num_seqs
    which = list(range(wl.num_rows))
    g, ref, _ = _check_indexer(wl, which, TOL[idx_dtype])
    _check_topk_on_oracle_scores(wl, ref, which)
    idx = _check_topk_on_gpu_scores(wl, g.copy())
    _check_mla(wl, idx, which, TOL["bf16"])
    say(f"one-call decode {wl.name}")
    _, idx1 = _attention_decode_vs_separate(wl)
    assert torch.equal(idx1, idx)


def test_multi_token_decode_full_size():
    """Two new tokens on each of 8 sequences of 131072 (fp8 indexer): the one-call decode
    against the separate calls on every row, and the oracle on sampled rows."""
    wl = workloads.prefill_batch([131072] * 8, new=[2] * 8, idx_dtype="fp8", seed=99, device=DEV,
                                 name="mtp_full_128k_fp8")
    wl = dataclasses.replace(wl, mode="decode")
    say("one-call decode 8 x 128K x 2")
    g, idx = _attention_decode_vs_separate(wl)
    which = [0, 1, 9, 15]
    g = g.cpu().numpy()
    ref = oracle_indexer(wl, which=which)
    lens = wl.row_len.cpu().numpy()
    err = oracle.max_abs_rel(valid_logits(g[which], lens, which), valid_logits(ref, lens, which))
    assert err <= TOL["fp8"], f"indexer err {err}"
    exp = oracle.topk(np.nan_to_num(g[which], nan=0.0).astype(np.float32), lens[which], wl.topk)
    assert np.array_equal(idx.cpu().numpy()[which], exp)
    _check_mla(wl, idx, which, TOL["bf16"])
    del wl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("paged", [False, True])
def test_multi_token_decode_shared_keys(paged):
    """16 rows per sequence over two sequences (bf16): the key-sharing indexer with fewer than 8
    row blocks (consecutive workgroups take consecutive key chunks of a block, chunks shrunk
    to 256 keys to fill the grid), a block straddling the two sequences; every row against the
    oracle, then the top-k, the split attention and the one-call decode."""
    wl = workloads.prefill_batch([5000, 9000], new=[12, 20], paged=paged, seed=98, device=DEV,
                                 name=f"mtp_shared_{'paged' if paged else 'contig'}")
    wl = dataclasses.replace(wl, mode="decode")
    assert wl.num_rows >= 8 * wl.num_seqs
    which = list(range(wl.num_rows))
    g, ref, _ = _check_indexer(wl, which, TOL["bf16"])
    _check_topk_on_oracle_scores(wl, ref, which)
    idx = _check_topk_on_gpu_scores(wl, g.copy())
    _check_mla(wl, idx, which, TOL["bf16"])
    say(f"one-call decode {wl.name}")
    _attention_decode_vs_separate(wl)


# ------------------------------------------------------------------------ fused indexer + top-k

# few rows with a long maximum length: the indexer workgroups feed the selection directly
FUSED_LENS = [1, 17, 2047, 2048, 2049, 9000, 20000, 40961]


def _fused_vs_separate(wl):
    rows = dev_rows(wl)
    g = gpu_indexer(wl)
    idx_sep = dsa.topk(g, wl.row_len, wl.topk, wl.max_row_len)
    logits = torch.full_like(g, float("nan"))
    idx_f = dsa.indexer_topk(rows, wl.q_idx, wl.w, wl.k_idx, logits, wl.topk, q_scale=wl.q_scale,
                             k_scale=wl.k_scale)
    assert torch.equal(torch.nan_to_num(g, nan=-1.0), torch.nan_to_num(logits, nan=-1.0))
    assert torch.equal(idx_sep, idx_f)
    return g, idx_f


@pytest.mark.parametrize("idx_dtype,paged", [("bf16", False), ("fp8", False), ("bf16", True),
                                             ("fp8", True)])
def test_fused_indexer_topk_matches_separate_calls(idx_dtype, paged):
    wl = workloads.decode(FUSED_LENS, idx_dtype=idx_dtype, paged=paged, seed=91, device=DEV,
                          name=f"fused_{idx_dtype}_{'paged' if paged else 'contig'}")
    say(f"fused indexer+topk {wl.name}")
    g, idx = _fused_vs_separate(wl)
    lens = wl.row_len.cpu().numpy()
    exp = oracle.topk(np.nan_to_num(g.cpu().numpy(), nan=0.0).astype(np.float32), lens, wl.topk)
    assert np.array_equal(idx.cpu().numpy(), exp)
    # a second call on the same workspace (left as the first call left it) agrees
    ws = torch.empty(dsa.indexer_topk_workspace_size(wl.num_rows, wl.max_row_len, wl.q_idx.dtype,
                                                     wl.topk), dtype=torch.uint8, device=DEV)
    logits = torch.empty_like(g)
    rows = dev_rows(wl)
    a = dsa.indexer_topk(rows, wl.q_idx, wl.w, wl.k_idx, logits, wl.topk, q_scale=wl.q_scale,
                         k_scale=wl.k_scale, ws=ws).clone()
    b = dsa.indexer_topk(rows, wl.q_idx, wl.w, wl.k_idx, logits, wl.topk, q_scale=wl.q_scale,
                         k_scale=wl.k_scale, ws=ws)
    assert torch.equal(a, idx) and torch.equal(b, idx)


def _boost(wl, row, lo, hi):
    """Scales the indexer keys of positions [lo, hi) of sequence `row` so their scores are the
    row's largest (bf16 keys x 4, fp8 key scales x 16: both exact)."""
    if wl.paged:
        raise ValueError("contiguous workloads only")
    base = int(wl.seq_start[row])
    if wl.idx_dtype == "fp8":
        wl.k_scale[base + lo:base + hi] *= 16.0
    else:
        wl.k_idx[base + lo:base + hi] *= 4.0


@pytest.mark.parametrize("idx_dtype", ["bf16", "fp8"])
def test_fused_selection_crowded_rows(idx_dtype):
    """Rows whose largest scores crowd into one or two stretches of positions (a few
    workgroups of the indexer grid hold the whole top-k), on rows of mixed lengths.  Fused
    against separate calls, the selection against the oracle's top-k on the same scores, and
    the scores against the oracle on sampled rows."""
    wl = workloads.decode([131072, 40961, 9000, 65536, 3000], idx_dtype=idx_dtype, seed=97,
                          device=DEV, name=f"crowded_{idx_dtype}")
    _boost(wl, 0, 4096, 8192)
    _boost(wl, 1, 0, 1500)
    _boost(wl, 1, 40000, 40961)
    _boost(wl, 3, 65536 - 2500, 65536)
    say(f"crowded rows {wl.name}")
    g, idx = _fused_vs_separate(wl)
    lens = wl.row_len.cpu().numpy()
    exp = oracle.topk(np.nan_to_num(g.cpu().numpy(), nan=0.0).astype(np.float32), lens, wl.topk)
    assert np.array_equal(idx.cpu().numpy(), exp)
    sel = idx.cpu().numpy()
    assert np.mean((sel[0] >= 4096) & (sel[0] < 8192)) > 0.95   # the boosted stretch dominates
    ref = oracle_indexer(wl, which=[1, 2])
    assert oracle.max_abs_rel(valid_logits(g.cpu().numpy()[[1, 2]], lens, [1, 2]),
                              valid_logits(ref, lens, [1, 2])) <= TOL[idx_dtype]
    _attention_decode_vs_separate(wl)


def test_fused_indexer_topk_other_schedules_and_full_size():
    # short rows take the one-workgroup-per-row selection: the call runs the stages in turn
    wl = workloads.decode(RAGGED, idx_dtype="bf16", seed=92, device=DEV, name="fused_short")
    say("fused indexer+topk short rows")
    _fused_vs_separate(wl)
    # the 128K-context decode batch at full size
    wl = workloads.config(4, device=DEV)
    say("fused indexer+topk config 4")
    _fused_vs_separate(wl)


# ------------------------------------------------------------------------ fused decode (stages 1-3)

def _attention_decode_vs_separate(wl):
    """The one-call decode against the indexer+top-k call followed by the attention call."""
    rows = dev_rows(wl)
    R = wl.num_rows
    logits_s = torch.full((R, wl.max_row_len), float("nan"), dtype=torch.float32, device=DEV)
    idx_s = dsa.indexer_topk(rows, wl.q_idx, wl.w, wl.k_idx, logits_s, wl.topk, q_scale=wl.q_scale,
                             k_scale=wl.k_scale)
    lse_s = torch.empty((R, wl.H), dtype=torch.float32, device=DEV)
    mla = dsa.sparse_mla_decode_paged if wl.paged else dsa.sparse_mla_decode
    out_s = mla(rows, wl.q, wl.kv, idx_s, wl.scale, wl.D_v, lse=lse_s)
    ws = torch.empty(max(dsa.sparse_attention_decode_workspace_size(
        R, wl.max_row_len, wl.q_idx.dtype, wl.topk, wl.H, wl.D_v), 1), dtype=torch.uint8, device=DEV)
    for call in range(2):   # the second call finds the workspace as the first left it
        logits = torch.full_like(logits_s, float("nan"))
        idx = torch.full_like(idx_s, -7)
        lse = torch.full_like(lse_s, float("nan"))
        out = dsa.sparse_attention_decode(rows, wl.q_idx, wl.w, wl.k_idx, logits, wl.topk, wl.q,
                                          wl.kv, wl.scale, wl.D_v, idx=idx, lse=lse,
                                          q_scale=wl.q_scale, k_scale=wl.k_scale, ws=ws)
        assert torch.equal(torch.nan_to_num(logits, nan=-1.0), torch.nan_to_num(logits_s, nan=-1.0))
        assert torch.equal(idx, idx_s)
        assert torch.equal(out, out_s)
        assert torch.equal(lse, lse_s)
    return logits_s, idx_s


@pytest.mark.parametrize("idx_dtype,paged", [("bf16", False), ("fp8", False), ("bf16", True),
                                             ("fp8", True)])
def test_attention_decode_matches_separate_calls(idx_dtype, paged):
    wl = workloads.decode(FUSED_LENS, idx_dtype=idx_dtype, paged=paged, seed=93, device=DEV,
                          name=f"decode3_{idx_dtype}_{'paged' if paged else 'contig'}")
    say(f"fused decode {wl.name}")
    g, idx = _attention_decode_vs_separate(wl)
    exp = oracle.topk(np.nan_to_num(g.cpu().numpy(), nan=0.0).astype(np.float32),
                      wl.row_len.cpu().numpy(), wl.topk)
    assert np.array_equal(idx.cpu().numpy(), exp)


@pytest.mark.parametrize("paged", [False, True])
def test_head_groups_are_bit_identical(paged):
    """The decode attention gives a (row, split) two 64-head workgroups when the batch is small
    enough (16 rows: their 16 splits halved to 8, with two head groups) and one 128-head
    workgroup otherwise (33 rows: 8 splits, one group).  Each head's wave runs the same
    operations either way, so with the same 8 splits per row the outputs of the same rows must
    be bit-identical, through the attention call and through the one-call decode (whose
    attention also finishes the selection in the 16-row batch).  The rows' results are
    checked against the oracle by the tests above."""
    wl = workloads.decode(FUSED_LENS, idx_dtype="fp8", paged=paged, seed=94, device=DEV,
                          name=f"head_groups_{'paged' if paged else 'contig'}")
    say(f"head groups {wl.name}")
    idx = dsa.topk(gpu_indexer(wl), wl.row_len, wl.topk, wl.max_row_len)

    def repeat(n, extra):   # the 8 rows n times over, then `extra` copies of row 0
        w2 = workloads.Workload(**{f: getattr(wl, f) for f in wl.__dataclass_fields__})
        for f in ("row_seq", "row_len", "q_idx", "q_scale", "w", "q"):
            t = getattr(wl, f)
            setattr(w2, f, torch.cat([t] * n + [t[:1]] * extra).contiguous())
        return w2, torch.cat([idx] * n + [idx[:1]] * extra).contiguous()

    def one_call(w):
        R = w.num_rows
        ws = torch.empty(max(dsa.sparse_attention_decode_workspace_size(
            R, w.max_row_len, w.q_idx.dtype, w.topk, w.H, w.D_v), 1), dtype=torch.uint8,
            device=DEV)
        logits = torch.empty((R, w.max_row_len), dtype=torch.float32, device=DEV)
        ix = torch.empty((R, w.topk), dtype=torch.int32, device=DEV)
        lse = torch.empty((R, w.H), dtype=torch.float32, device=DEV)
        out = dsa.sparse_attention_decode(dev_rows(w), w.q_idx, w.w, w.k_idx, logits, w.topk, w.q,
                                          w.kv, w.scale, w.D_v, idx=ix, lse=lse,
                                          q_scale=w.q_scale, k_scale=w.k_scale, ws=ws)
        return out, lse, ix

    w16, i16 = repeat(2, 0)    # 16 rows: two head groups
    w33, i33 = repeat(4, 1)    # 33 rows: one head group
    assert w16.num_rows == 16 and w33.num_rows == 33
    o16, l16 = gpu_mla(w16, i16)
    o33, l33 = gpu_mla(w33, i33)
    assert torch.equal(o16, o33[:16]) and torch.equal(l16, l33[:16])
    assert torch.equal(o16[:8], o16[8:]) and torch.equal(o33[:8], o33[16:24])
    a16, b16, x16 = one_call(w16)
    a33, b33, x33 = one_call(w33)
    assert torch.equal(x16, i16) and torch.equal(x33, i33)
    assert torch.equal(a16, o16) and torch.equal(b16, l16)
    assert torch.equal(a33, o33) and torch.equal(b33, l33)


@pytest.mark.parametrize("idx_dtype", ["bf16", "fp8"])
def test_attention_decode_all_scores_tied(idx_dtype):
    """Zero head weights make every score +0: every position of a row ties, the rows' survivor
    lists overflow the LDS selection (rows above 10240 positions), and both the fused top-k and
    the attention that finishes its own selection take the select over the whole score row.
    The selection is then the row's lowest min(len, k) positions, ascending."""
    wl = workloads.decode(FUSED_LENS, idx_dtype=idx_dtype, seed=95, device=DEV,
                          name=f"decode3_tied_{idx_dtype}")
    wl.w.zero_()
    say(f"fused decode all tied {idx_dtype}")
    g, idx = _attention_decode_vs_separate(wl)
    lens = wl.row_len.cpu().numpy()
    exp = np.full((wl.num_rows, wl.topk), -1, dtype=np.int32)
    for r, n in enumerate(lens):
        exp[r, :min(n, wl.topk)] = np.arange(min(n, wl.topk))
    assert np.array_equal(idx.cpu().numpy(), exp)
    g_np = g.cpu().numpy()
    for r, n in enumerate(lens):
        assert np.all(g_np[r, :n] == 0.0)
    _check_mla(wl, idx, [0, 5, 7], TOL["bf16"])


def test_attention_decode_other_schedules_and_full_size():
    # short rows: the call runs the indexer+top-k call and the attention call in turn
    wl = workloads.decode(RAGGED, idx_dtype="bf16", seed=94, device=DEV, name="decode3_short")
    say("fused decode short rows")
    _attention_decode_vs_separate(wl)
    for cfg in (4, 5):
        wl = workloads.config(cfg, device=DEV)
        say(f"fused decode config {cfg}")
        _attention_decode_vs_separate(wl)
        del wl
        torch.cuda.empty_cache()


@pytest.mark.parametrize("k,idx_dtype", [(1, "bf16"), (100, "fp8"), (700, "bf16")])
def test_attention_decode_other_topk_sizes(k, idx_dtype):
    """k below 2048 through the one-call decode: one split of one slot (k = 1), one split of a
    partial tile (k = 100), six splits with a short last one (k = 700); rows shorter than k,
    longer than k, and long enough for the chunked schedule."""
    wl = workloads.decode([1, 150, 9000, 40961, 70000], idx_dtype=idx_dtype, topk=k, seed=98 + k,
                          device=DEV, name=f"decode_k{k}_{idx_dtype}")
    say(f"fused decode k={k} {idx_dtype}")
    g, idx = _attention_decode_vs_separate(wl)
    lens = wl.row_len.cpu().numpy()
    exp = oracle.topk(np.nan_to_num(g.cpu().numpy(), nan=0.0).astype(np.float32), lens, k)
    assert np.array_equal(idx.cpu().numpy(), exp)
    _check_mla(wl, idx, [0, 1, 2, 4], TOL["bf16"])


def test_decode_at_the_longest_chunked_row():
    """A row of 2^20 positions, the longest the chunked top-k schedule takes (256 chunks of
    4096 scores), beside a mid-length row, through the one-call decode (fused indexer with
    histograms, chunk filter, selecting attention, combine): every stage against the oracle."""
    wl = workloads.decode([1 << 20, 70001], idx_dtype="fp8", seed=97, device=DEV, name="decode_1m")
    say("fused decode, a 2^20-position row")
    g, idx = _attention_decode_vs_separate(wl)
    lens = wl.row_len.cpu().numpy()
    exp = oracle.topk(np.nan_to_num(g.cpu().numpy(), nan=0.0).astype(np.float32), lens, wl.topk)
    assert np.array_equal(idx.cpu().numpy(), exp)
    _check_indexer(wl, [0, 1], TOL["fp8"])
    _check_mla(wl, idx, [0, 1], TOL["bf16"])
    del wl
    torch.cuda.empty_cache()


# ------------------------------------------------------------------------ full-size configs

def selection_recall(idx_gpu, ref_scores, lens, k):
    """Per row: the share of the exact top-k (the oracle's selection on its own fp64 scores)
    that the GPU selection also holds, |GPU set & exact set| / min(k, len)."""
    exact = oracle.topk(np.nan_to_num(ref_scores, nan=0.0), lens, k)
    out = []
    for g, e, n in zip(idx_gpu, exact, lens):
        kk = min(k, int(n))
        out.append(len(set(g[:kk].tolist()) & set(e[:kk].tolist())) / kk)
    return np.array(out)


# The smallest share of the exact top-k a sampled row of the full-size workloads may hold: the
# selection runs on the kernel's scores, whose bf16 head sum moves boundary scores by about
# 1e-3 relative (measured 0.9956 .. 1.0 over the sampled rows; printed with each case).
MIN_RECALL = 0.99


@pytest.mark.parametrize("cfg,which", [(2, [0, 17, 63]), (4, [0, 5]), (5, [0, 1, 9, 31])])
def test_full_decode_configs_sampled(cfg, which):
    wl = workloads.config(cfg, device=DEV)
    say(f"full config {cfg} ({wl.name}), sampled rows {which}")
    g, ref, _ = _check_indexer(wl, which, TOL[wl.idx_dtype])
    _check_topk_on_oracle_scores(wl, ref, which)
    idx = _check_topk_on_gpu_scores(wl, g.copy())
    rec = selection_recall(idx.cpu().numpy()[which], ref, wl.row_len.cpu().numpy()[which], wl.topk)
    say(f"selection recall {wl.name} rows {which}: {np.round(rec, 5).tolist()}")
    assert rec.min() >= MIN_RECALL
    _check_mla(wl, idx, which, TOL["bf16"])
    del wl
    torch.cuda.empty_cache()


def test_c3_prefill_16k_sampled():
    wl = workloads.config(3, device=DEV)
    which = [0, 1, 63, 64, 2046, 2047, 2048, 2049, 9000, 16383]
    g, ref, _ = _check_indexer(wl, which, TOL["bf16"])
    _check_topk_on_oracle_scores(wl, ref, which)
    say("c3 topk all rows")
    idx = dsa.topk(torch.from_numpy(g).to(DEV), wl.row_len, wl.topk, wl.max_row_len)
    lens = wl.row_len.cpu().numpy()
    exp = oracle.topk(np.nan_to_num(g[which], nan=0.0).astype(np.float32), lens[which], wl.topk)
    assert np.array_equal(idx.cpu().numpy()[which], exp)
    _check_mla(wl, idx, which, TOL["bf16"])
    del wl, g
    torch.cuda.empty_cache()


@pytest.mark.parametrize("idx_dtype", ["bf16", "fp8"])
def test_prefill_other_topk_size(idx_dtype):
    """A 3000-token prefill with k = 300: rows below, at and above k; the fused indexer + top-k
    call against separate calls bit for bit, every row's selection against the oracle on the
    kernel's scores, sampled rows of the indexer and the attention against the oracle."""
    wl = workloads.prefill(3000, idx_dtype=idx_dtype, topk=300, seed=110, device=DEV,
                           name=f"prefill_k300_{idx_dtype}")
    say(f"prefill k=300 {idx_dtype}")
    which = [0, 1, 298, 299, 300, 301, 1500, 2999]
    g, ref, _ = _check_indexer(wl, which, TOL[idx_dtype])
    _check_topk_on_oracle_scores(wl, ref, which)
    idx = _check_topk_on_gpu_scores(wl, g.copy())
    rows = dev_rows(wl)
    logits = torch.full((wl.num_rows, wl.max_row_len), float("nan"), dtype=torch.float32, device=DEV)
    idx_f = dsa.indexer_topk(rows, wl.q_idx, wl.w, wl.k_idx, logits, wl.topk, q_scale=wl.q_scale,
                             k_scale=wl.k_scale)
    assert torch.equal(idx_f, idx)
    _check_mla(wl, idx, which, TOL["bf16"])


# ------------------------------------------------------------------------ determinism, edges

def test_two_runs_bitwise_equal():
    wl = workloads.decode([3000, 9000, 40000], idx_dtype="fp8", seed=3, device=DEV, name="det")
    say("determinism")
    outs = []
    for _ in range(2):
        g = gpu_indexer(wl)
        idx = dsa.topk(g, wl.row_len, wl.topk, wl.max_row_len)
        o, l = gpu_mla(wl, idx)
        outs.append((torch.nan_to_num(g, nan=-1.0), idx, o, l))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def _topk_case(x: np.ndarray, lens, k):
    xs = torch.from_numpy(x.astype(np.float32)).to(DEV)
    rl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    got = dsa.topk(xs, rl, k, int(max(lens))).cpu().numpy()
    exp = oracle.topk(x.astype(np.float32), np.array(lens), k)
    assert np.array_equal(got, exp)


def test_topk_edge_cases():
    say("topk edges")
    n = 40000   # beyond the LDS-staged size: streamed passes
    rng = np.random.default_rng(0)
    for k in (1, 7, 2048):
        rows = np.zeros((6, n), dtype=np.float32)
        rows[0] = 3.5                                          # all equal
        rows[1] = np.arange(n, dtype=np.float32)               # strictly increasing
        rows[2] = rng.integers(-3, 4, size=n)                  # heavy ties
        rows[2][rows[2] == 0] = np.where(rng.random(int((rows[2] == 0).sum())) < 0.5, -0.0, 0.0)
        rows[3] = -np.abs(rng.standard_normal(n))              # all negative
        rows[4] = np.where(rng.random(n) < 0.01, 1.0, 0.0)     # sparse ones among zeros
        rows[5] = rng.standard_normal(n)
        _topk_case(rows, [n, n, n, 5000, 30000, 1], k)
        _topk_case(rows[:, :3000], [3000, 2048, 2049, 1, 17, 3000], k)
    # the longest rows staged in LDS, whose histogram counts bins in 16 bits: one bin holding
    # every key, and two neighbouring bins that share one histogram word
    n = 28672
    rows = np.zeros((4, n), dtype=np.float32)
    rows[0] = 3.5
    rows[1] = np.where(np.arange(n) % 2 == 0, 1.0, 1.125)
    rows[2] = rng.standard_normal(n)
    rows[3] = rng.integers(-3, 4, size=n)
    for k in (7, 2048):
        _topk_case(rows, [n, n, 16384, 20000], k)
    # rows up to 2^18 scores are selected by one workgroup each; longer ones take the chunked
    # filter and a final workgroup
    n = 300000
    rows = np.zeros((3, n), dtype=np.float32)
    rows[0] = rng.standard_normal(n)
    rows[1] = rng.integers(-40, 41, size=n) / 8.0          # ties at the threshold
    rows[2] = np.where(rng.random(n) < 0.5, 0.0, rng.standard_normal(n))
    _topk_case(rows[:, :262144], [262144, 200001, 5], 2048)
    _topk_case(rows, [300000, 262145, 40000], 2048)


def test_mla_skips_invalid_and_empty_selections():
    wl = workloads.decode([50, 3000], seed=9, device=DEV, name="mla_edges")
    idx = torch.full((2, 2048), -1, dtype=torch.int32, device=DEV)
    idx[0, :10] = torch.tensor([3, -1, 49, 50, 1000, 0, 7, -5, 7, 2], dtype=torch.int32)  # dup 7
    idx[1, 100:140] = torch.arange(2960, 3000, dtype=torch.int32)
    rows = dev_rows(wl)
    say("mla invalid/dup entries")
    out, lse = gpu_mla(wl, idx)
    ref_o, ref_l = oracle_mla(wl, idx.cpu().numpy())
    assert oracle.max_abs_rel(out.float().cpu().numpy(), ref_o) <= TOL["bf16"]
    assert oracle.max_abs_rel(lse.cpu().numpy(), ref_l) <= TOL["bf16"]
    empty = torch.full((2, 64), -1, dtype=torch.int32, device=DEV)
    o2 = torch.empty((2, wl.H, wl.D_v), dtype=torch.bfloat16, device=DEV)
    l2 = torch.empty((2, wl.H), dtype=torch.float32, device=DEV)
    dsa.sparse_mla_decode(rows, wl.q, wl.kv, empty, wl.scale, wl.D_v, out=o2, lse=l2)
    assert torch.all(o2 == 0) and torch.all(torch.isneginf(l2))


def test_mfma_rate_probe_writes_every_wave():
    """The matrix-core rate probe (a measurement aid): every one of its waves writes a finite
    sum, and the sum grows with the loop count (the products are not folded away)."""
    say("mfma probe")
    out = torch.full((dsa.MFMA_PROBE_WAVES,), float("nan"), device=DEV)
    dsa.mfma_rate_probe(4, out)
    a = out.cpu().numpy()
    assert np.all(np.isfinite(a))
    dsa.mfma_rate_probe(8, out)
    b = out.cpu().numpy()
    assert np.allclose(b, 2 * a, rtol=1e-5, atol=1e-6) and np.abs(a).max() > 0


def test_rows_beyond_the_grid_y_limit():
    """More query rows (70,000) than one grid dimension holds (65,535 blocks): the indexer
    that gives every row its own blocks (fp8 and f32) and the f32 attention continue the rows
    in the grid's third dimension.  Rows share one 256-token sequence, row r sees
    1 + (r % 256) positions; rows on both sides of the limit are checked."""
    R, L = 70000, 256
    gen = torch.Generator(device=DEV)
    gen.manual_seed(77)
    row_seq = torch.zeros(R, dtype=torch.int32, device=DEV)
    row_len = (torch.arange(R, device=DEV, dtype=torch.int32) % L) + 1
    seq_start = torch.zeros(1, dtype=torch.int64, device=DEV)
    rows = dsa.Rows(row_seq, row_len, L, 1, seq_start=seq_start)
    lens = row_len.cpu().numpy()
    orows = oracle.Rows(np.zeros(R, np.int32), lens, seq_start=np.zeros(1, np.int64))
    which = [0, 1, 65534, 65535, 65536, 69999]

    say("fp8 indexer, 70000 rows")
    q8, qs = workloads.quantize_e4m3(torch.randn((R, 64, 128), generator=gen, device=DEV), 1)
    qs = qs[:, None].expand(R, 64).contiguous()
    k8, ks = workloads.quantize_e4m3(torch.randn((L, 128), generator=gen, device=DEV), 1)
    w = torch.rand((R, 64), generator=gen, device=DEV) / 8
    logits = torch.full((R, L), float("nan"), device=DEV)
    dsa.indexer_logits(rows, q8, w, k8, logits, q_scale=qs, k_scale=ks)
    ref = oracle.indexer("fp8", raw(q8), raw(w), raw(k8), orows, q_scale=raw(qs),
                         k_scale=raw(ks), which=which, ld=L)
    got = logits.cpu().numpy()[which]
    assert oracle.max_abs_rel(valid_logits(got, lens, which),
                              valid_logits(ref, lens, which)) <= TOL["fp8"]
    del q8, qs, logits

    say("f32 indexer, 70000 rows")
    qf = torch.randn((R, 4, 32), generator=gen, device=DEV)
    kf = torch.randn((L, 32), generator=gen, device=DEV)
    wf = torch.rand((R, 4), generator=gen, device=DEV)
    logits = torch.full((R, L), float("nan"), device=DEV)
    dsa.indexer_logits(rows, qf, wf, kf, logits)
    ref = oracle.indexer("f32", raw(qf), raw(wf), raw(kf), orows, which=which, ld=L)
    got = logits.cpu().numpy()[which]
    assert oracle.max_abs_rel(valid_logits(got, lens, which),
                              valid_logits(ref, lens, which)) <= TOL["f32"]

    say("f32 attention, 70000 rows")
    k = 16
    q = torch.randn((R, 8, 80), generator=gen, device=DEV)
    kv = torch.randn((L, 80), generator=gen, device=DEV)
    j = torch.arange(k, device=DEV, dtype=torch.int32)
    idx = torch.where(j[None, :] < row_len[:, None], (row_len[:, None] - 1 - j[None, :]) % L,
                      torch.full_like(j[None, :], -1)).to(torch.int32).contiguous()
    out = torch.empty((R, 8, 64), device=DEV)
    lse = torch.empty((R, 8), device=DEV)
    dsa.sparse_mla_decode(rows, q, kv, idx, 80 ** -0.5, 64, out=out, lse=lse)
    ref_o, ref_l = oracle.sparse_mla("f32", raw(q), raw(kv), idx.cpu().numpy(), orows,
                                     80 ** -0.5, 64, which=which)
    assert oracle.max_abs_rel(out.cpu().numpy()[which], ref_o) <= TOL["f32"]
    assert oracle.max_abs_rel(lse.cpu().numpy()[which], ref_l) <= TOL["f32"]


@pytest.mark.parametrize("paged", [False, True])
def test_many_row_attention_edges(paged):
    """The no-split attention (one workgroup per row): a short row whose valid slots are
    compacted, duplicate and out-of-range slots, k = 1000 (a ragged last tile), a row with
    no valid slot, and cache values that grow across the cache so that the running maximum
    of the softmax moves by more than its lazy threshold between tiles (rescales)."""
    lens = [40, 700, 3000, 5000]
    wl = workloads.decode(lens, paged=paged, seed=21, device=DEV, name="many_row_edges")
    kv = wl.kv.reshape(-1, wl.kv.shape[-1])
    grow = 1.0 + 7.0 * torch.arange(kv.shape[0], device=DEV, dtype=torch.float32) / kv.shape[0]
    kv.copy_((kv.float() * grow[:, None]).to(kv.dtype))
    k = 1000
    rng = np.random.default_rng(5)
    idx = np.full((4, k), -1, dtype=np.int32)
    idx[0, :40] = np.arange(40)
    idx[1] = rng.integers(-20, 760, size=k)                       # dups, < 0 and >= len
    idx[2] = np.sort(rng.choice(3000, size=k, replace=False))
    idx_dev = torch.from_numpy(idx).to(DEV)
    rows = dev_rows(wl)
    out = torch.empty((4, wl.H, wl.D_v), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((4, wl.H), dtype=torch.float32, device=DEV)
    say(f"many-row attention edges paged={paged}")
    fn = dsa.sparse_mla_prefill_paged if paged else dsa.sparse_mla_prefill
    fn(rows, wl.q, wl.kv, idx_dev, wl.scale, wl.D_v, out=out, lse=lse)
    ref_o, ref_l = oracle_mla(wl, idx, which=[0, 1, 2])
    o = out.float().cpu().numpy()
    assert oracle.max_abs_rel(o[:3], ref_o) <= TOL["bf16"]
    assert oracle.max_abs_rel(lse.cpu().numpy()[:3], ref_l) <= TOL["bf16"]
    assert np.all(o[3] == 0) and np.all(np.isneginf(lse.cpu().numpy()[3]))


def test_prefill_and_decode_entry_points_agree():
    """Many-row (no split) and few-row (split + combine) attention give the same answer."""
    wl = workloads.decode([2500, 4000, 9000], seed=12, device=DEV, name="agree")
    g = gpu_indexer(wl)
    idx = dsa.topk(g, wl.row_len, wl.topk, wl.max_row_len)
    rows = dev_rows(wl)
    say("decode vs prefill entry")
    a = dsa.sparse_mla_decode(rows, wl.q, wl.kv, idx, wl.scale, wl.D_v)
    b = dsa.sparse_mla_prefill(rows, wl.q, wl.kv, idx, wl.scale, wl.D_v)
    ref, _ = oracle_mla(wl, idx.cpu().numpy())
    assert oracle.max_abs_rel(a.float().cpu().numpy(), ref) <= TOL["bf16"]
    assert oracle.max_abs_rel(b.float().cpu().numpy(), ref) <= TOL["bf16"]


def test_hip_graph_replays_match_eager():
    """The whole decode step captured in a HIP graph: every replay (with eager work and
    synchronisations in between) equals the eager result bit for bit."""
    wl = workloads.decode([3000, 20000, 9000, 2047], idx_dtype="fp8", seed=21, device=DEV,
                          name="graph")
    rows = dev_rows(wl)
    R = wl.num_rows
    logits = torch.zeros((R, wl.max_row_len), dtype=torch.float32, device=DEV)
    idx = torch.empty((R, wl.topk), dtype=torch.int32, device=DEV)
    out = torch.empty((R, wl.H, wl.D_v), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((R, wl.H), dtype=torch.float32, device=DEV)
    tk_ws = torch.zeros(max(dsa.topk_workspace_size(R, wl.max_row_len, wl.topk), 1),
                        dtype=torch.uint8, device=DEV)
    ml_ws = torch.zeros(max(dsa.sparse_mla_workspace_size(R, wl.H, wl.D_v, wl.topk), 1),
                        dtype=torch.uint8, device=DEV)

    def step():
        dsa.indexer_logits(rows, wl.q_idx, wl.w, wl.k_idx, logits, q_scale=wl.q_scale,
                           k_scale=wl.k_scale)
        dsa.topk(logits, wl.row_len, wl.topk, wl.max_row_len, idx=idx, ws=tk_ws)
        dsa.sparse_mla_decode(rows, wl.q, wl.kv, idx, wl.scale, wl.D_v, out=out, lse=lse, ws=ml_ws)

    say("graph capture")
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (logits, idx, out, lse)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (logits, idx, out, lse):
            t.fill_(7)                         # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        valid = torch.arange(wl.max_row_len, device=DEV)[None, :] < wl.row_len[:, None]
        assert torch.equal(logits[valid], ref[0][valid]), rep   # only s < row_len is written
        for a, b in zip((idx, out, lse), ref[1:]):
            assert torch.equal(a, b), rep
