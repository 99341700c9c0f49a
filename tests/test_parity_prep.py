"""GPU parity of the indexer-input and cache-write prep against the oracle, bit for bit.

Every output is a code chosen by rounding (bf16, or e4m3 with its fp32 scale), and both sides
compute it in fp32 one IEEE operation at a time, so the caches, scales and rotated queries must
match exactly; rows no token names must keep their previous contents.  Then the prepared fp8
caches and queries go through the paged indexer and are compared with the oracle's indexer on
the oracle-prepared data.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_08_amd as dsa
import workloads
from helpers import TOL, say

pytestmark = pytest.mark.gpu

DEV = "cuda"
raw = workloads.raw_numpy


def _gpu_keys(b):
    kc, kvc = b.k_cache.clone(), b.kv_cache.clone()
    ks = None if b.k_scale is None else b.k_scale.clone()
    dsa.prep_cache_write(b.positions, b.cache_rows, b.cos_sin, b.k_idx_in, kc, b.kv_in, kvc,
                         k_idx_scale=ks)
    return kc, kvc, ks


def _oracle_keys(b):
    return oracle.prep_keys(b.idx_dtype, raw(b.positions), raw(b.cache_rows), raw(b.cos_sin),
                            raw(b.k_idx_in), raw(b.kv_in), raw(b.k_cache), raw(b.kv_cache),
                            raw(b.k_scale))


def _gpu_queries(b):
    T = b.positions.numel()
    if b.idx_dtype == "fp8":
        qi = torch.zeros((T, 64, 128), dtype=torch.uint8, device=DEV)
        qs = torch.zeros((T, 64), dtype=torch.float32, device=DEV)
    else:
        qi, qs = torch.zeros((T, 64, 128), dtype=torch.bfloat16, device=DEV), None
    q = b.q.clone()
    dsa.prep_queries(b.positions, b.cos_sin, b.q_idx_in, qi, q, q_idx_scale=qs)
    return qi, qs, q


@pytest.mark.parametrize("idx_dtype,paged", [("bf16", False), ("fp8", False), ("bf16", True),
                                             ("fp8", True)])
def test_prep_bit_exact(idx_dtype, paged):
    """Ragged new-token counts (a single token, a page-straddling run, a whole page, a run of
    300), positions up to 4999, padding tokens (row -1); keys, latent entries, scales and
    queries bit for bit."""
    b = workloads.prep_batch([1, 130, 4999, 700, 64], [1, 70, 300, 64, 64], idx_dtype=idx_dtype,
                             paged=paged, pad=5, seed=41, device=DEV)
    say(f"prep keys {idx_dtype} {'paged' if paged else 'contig'} T={b.positions.numel()}")
    kc, kvc, ks = _gpu_keys(b)
    ekc, ekvc, eks = _oracle_keys(b)
    assert np.array_equal(raw(kc), ekc)
    assert np.array_equal(raw(kvc), ekvc)
    if idx_dtype == "fp8":
        assert np.array_equal(raw(ks), eks)
    say(f"prep queries {idx_dtype}")
    qi, qs, q = _gpu_queries(b)
    eqi, eqs, eq = oracle.prep_queries(idx_dtype, raw(b.positions), raw(b.cos_sin),
                                       raw(b.q_idx_in), raw(b.q))
    assert np.array_equal(raw(qi), eqi)
    assert np.array_equal(raw(q), eq)
    if idx_dtype == "fp8":
        assert np.array_equal(raw(qs), eqs)


@pytest.mark.parametrize("idx_dtype", ["bf16", "fp8"])
def test_one_call_prep_equals_the_two_calls(idx_dtype):
    """dsa_prep (both sides in one launch) writes the same bytes as dsa_prep_cache_write followed
    by dsa_prep_queries."""
    b = workloads.prep_batch([900, 65, 3000], [33, 1, 64], idx_dtype=idx_dtype, paged=True,
                             seed=46, device=DEV)
    kc, kvc, ks = _gpu_keys(b)
    qi, qs, q = _gpu_queries(b)
    kc2, kvc2, q2 = b.k_cache.clone(), b.kv_cache.clone(), b.q.clone()
    ks2 = None if b.k_scale is None else b.k_scale.clone()
    qi2, qs2 = torch.zeros_like(qi), None if qs is None else torch.zeros_like(qs)
    say(f"one-call prep {idx_dtype}")
    dsa.prep(b.positions, b.cache_rows, b.cos_sin, b.k_idx_in, kc2, b.kv_in, kvc2, b.q_idx_in, qi2,
             q2, k_idx_scale=ks2, q_idx_scale=qs2)
    assert torch.equal(kc2, kc) and torch.equal(kvc2, kvc) and torch.equal(q2, q)
    assert torch.equal(qi2, qi)
    if idx_dtype == "fp8":
        assert torch.equal(ks2, ks) and torch.equal(qs2, qs)


def test_prep_in_place_bf16_queries_and_positions_out_of_range():
    """bf16 indexer queries rotated in place equal the out-of-place result; a position outside
    the table leaves its row untouched (keys and queries)."""
    b = workloads.prep_batch([200, 90], [7, 3], idx_dtype="bf16", seed=42, device=DEV)
    b.positions[2] = b.cos_sin.shape[0]        # one past the table
    qi, _, q = _gpu_queries(b)
    qi2, q2 = b.q_idx_in.clone(), b.q.clone()
    say("prep queries in place")
    dsa.prep_queries(b.positions, b.cos_sin, qi2, qi2, q2)
    other = torch.arange(10, device=DEV) != 2
    assert torch.equal(qi2[other], qi[other])
    assert torch.equal(qi2[2], b.q_idx_in[2]) and torch.equal(q2[2], b.q[2])
    assert torch.equal(q2, q)
    kc, kvc, _ = _gpu_keys(b)
    row = int(b.cache_rows[2])
    assert torch.equal(kc[row], b.k_cache[row]) and torch.equal(kvc[row], b.kv_cache[row])


def test_prepared_fp8_cache_feeds_the_paged_indexer():
    """Prep of a decode step (one new token per sequence, paged fp8 cache), then the paged
    indexer on the prepared cache and queries, against the oracle's indexer on the
    oracle-prepared data: the cache layout the prep writes is the one the indexer reads."""
    lens = [3000, 129, 64, 2049]
    b = workloads.prep_batch(lens, [1] * 4, idx_dtype="fp8", paged=True, seed=43, device=DEV)
    say("prep + indexer decode step")
    kc, kvc, ks = _gpu_keys(b)
    qi, qs, _ = _gpu_queries(b)
    ekc, _, eks = _oracle_keys(b)
    eqi, eqs, _ = oracle.prep_queries("fp8", raw(b.positions), raw(b.cos_sin), raw(b.q_idx_in),
                                      raw(b.q))
    P = kc.shape[0] // 64
    pt = raw(b.page_table)
    w = torch.rand((4, 64), generator=torch.Generator(device=DEV).manual_seed(44), device=DEV) / 8
    row_seq = torch.arange(4, dtype=torch.int32, device=DEV)
    row_len = torch.tensor(lens, dtype=torch.int32, device=DEV)
    rows = dsa.Rows(row_seq, row_len, max(lens), 4, page_table=b.page_table)
    logits = torch.full((4, max(lens)), float("nan"), device=DEV)
    dsa.indexer_logits_paged(rows, qi.view(torch.float8_e4m3fn), w, kc.view(P, 64, 128)
                             .view(torch.float8_e4m3fn), logits, q_scale=qs,
                             k_scale=ks.view(P, 64))
    orows = oracle.Rows(np.arange(4), np.array(lens), page_table=pt)
    ref = oracle.indexer("fp8", eqi, raw(w), ekc.reshape(P, 64, 128), orows, q_scale=eqs,
                         k_scale=eks.reshape(P, 64))
    g_np = logits.cpu().numpy()
    for r, L in enumerate(lens):
        assert oracle.max_abs_rel(g_np[r, :L], ref[r, :L]) <= TOL["fp8"]


def test_prep_decode_step_full_size():
    """A 128K-context decode step's prep: 8 sequences of 131072 tokens, one new token each, fp8
    paged cache (8 x 2048 pages), bit for bit on the 8 rows written, every other row kept."""
    b = workloads.prep_batch([131072] * 8, [1] * 8, idx_dtype="fp8", paged=True, seed=45,
                             device=DEV)
    say("prep decode step 8 x 128K")
    kc, kvc, ks = _gpu_keys(b)
    sel = b.cache_rows
    # the oracle works on the 8 written rows only (renumbered 0..7)
    ekc, ekvc, eks = oracle.prep_keys("fp8", raw(b.positions), np.arange(8), raw(b.cos_sin),
                                      raw(b.k_idx_in), raw(b.kv_in), raw(b.k_cache[sel]),
                                      raw(b.kv_cache[sel]), raw(b.k_scale[sel]))
    assert np.array_equal(raw(kc[sel]), ekc) and np.array_equal(raw(kvc[sel]), ekvc)
    assert np.array_equal(raw(ks[sel]), eks)
    keep = torch.ones(kc.shape[0], dtype=torch.bool, device=DEV)
    keep[sel] = False
    assert torch.equal(kc[keep], b.k_cache[keep]) and torch.equal(kvc[keep], b.kv_cache[keep])
    assert torch.equal(ks[keep], b.k_scale[keep])
