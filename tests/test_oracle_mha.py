"""Pins for the oracle's masked MHA mode (short prefill), against facts that do not come from
the oracle itself.

Sources: "DeepSeek-V3.2 技术报告摘要", section 1 ("短序列优化": short prefill runs DSA as masked
MHA; DSA runs MLA in MQA mode); the "DeepSeek-V3.2 -- Model techniques map" code table
(multi-head latent attention: 128 nope + 64 rope query/key dims, 128 value dims, latent 512).
"""
import math

import numpy as np
import torch

import oracle


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _val(bits):
    return oracle.bf16_to_f64(bits)


def _inputs(rng, n, H=4, R=None):
    kv = _bf16_bits(rng.standard_normal((n, 576)) * 0.5)
    w_uk = _bf16_bits(rng.standard_normal((H, 128, 512)) * 0.05)
    w_uv = _bf16_bits(rng.standard_normal((H, 128, 512)) * 0.05)
    q = _bf16_bits(rng.standard_normal((R or n, H, 192)))
    return kv, w_uk, w_uv, q


def _contig(lens):
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    row_seq = np.concatenate([np.full(l, b) for b, l in enumerate(lens)])
    row_len = np.concatenate([np.arange(1, l + 1) for l in lens])
    return oracle.Rows(row_seq, row_len, seq_start=starts)


def test_mha_equals_absorbed_mqa():
    """Per-head MHA over decompressed keys/values equals MQA over the 576-d latent entries with
    the query absorbed through W_UK and the output projected through W_UV (the identity that
    lets DSA run in either mode), on top-k sets and on dense causal rows."""
    rng = np.random.default_rng(31)
    H, n = 4, 40
    kv, w_uk, w_uv, q = _inputs(rng, n, H)
    rows = _contig([n])
    K, V = oracle.mha_decompress(kv, w_uk, w_uv)
    scale = 1.0 / math.sqrt(192.0)
    idx = np.full((n, 8), -1, np.int32)
    for r in range(n):
        pick = rng.choice(r + 1, size=min(r + 1, 8), replace=False)
        idx[r, :len(pick)] = pick
    qv, wk, wv = _val(q), _val(w_uk), _val(w_uv)
    q_abs = np.concatenate([np.einsum("rhd,hdc->rhc", qv[..., :128], wk), qv[..., 128:]],
                           axis=-1).astype(np.float32)
    entries = _val(kv).astype(np.float32)
    for use_idx in (True, False):
        out, lse = oracle.mha(q, K, V, rows, scale, idx=idx if use_idx else None)
        mqa_idx = idx if use_idx else np.where(np.arange(n)[None] <= np.arange(n)[:, None],
                                               np.arange(n)[None], -1).astype(np.int32)
        o_lat, lse_mqa = oracle.sparse_mla("f32", q_abs, entries, mqa_idx, rows, scale, 512)
        o_mqa = np.einsum("hdc,rhc->rhd", wv, o_lat)
        assert oracle.max_abs_rel(out, o_mqa) < 1e-5
        assert np.max(np.abs(lse - lse_mqa)) < 1e-5


def test_dense_mode_is_causal_sdpa():
    """Without idx every row attends causally to its sequence: torch's causal scaled dot-product
    attention in fp64 on the decompressed keys and values, two sequences back to back."""
    rng = np.random.default_rng(32)
    H, lens = 3, [17, 26]
    kv, w_uk, w_uv, q = _inputs(rng, sum(lens), H)
    K, V = oracle.mha_decompress(kv, w_uk, w_uv)
    scale = 0.11
    out, lse = oracle.mha(q, K, V, _contig(lens), scale)
    qv = _val(q)
    o = 0
    for L in lens:
        qt = torch.from_numpy(qv[o:o + L]).transpose(0, 1)
        kt = torch.from_numpy(K[o:o + L]).transpose(0, 1)
        vt = torch.from_numpy(V[o:o + L]).transpose(0, 1)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                               scale=scale).transpose(0, 1)
        assert oracle.max_abs_rel(out[o:o + L], ref.numpy()) < 1e-12
        o += L


def test_mask_is_a_set_and_decompression_places_rope_last():
    """idx naming every position (shuffled, with duplicates and -1 padding) equals dense mode;
    a row whose set is one position returns that position's value exactly; the decompressed
    key is W_UK c followed by the entry's 64 RoPE dims."""
    rng = np.random.default_rng(33)
    H, n = 2, 12
    kv, w_uk, w_uv, q = _inputs(rng, n, H)
    rows = _contig([n])
    K, V = oracle.mha_decompress(kv, w_uk, w_uv)
    lat = _val(kv)
    assert np.array_equal(K[:, :, 128:], np.broadcast_to(lat[:, None, 512:], (n, H, 64)))
    assert np.allclose(K[:, :, :128], np.einsum("hdc,nc->nhd", _val(w_uk), lat[:, :512]),
                       rtol=1e-12, atol=1e-12)
    idx = np.full((n, 2 * n), -1, np.int32)
    for r in range(n):
        pos = list(range(r + 1)) * 2
        rng.shuffle(pos)
        idx[r, :len(pos)] = pos
    dense, _ = oracle.mha(q, K, V, rows, 0.1)
    masked, _ = oracle.mha(q, K, V, rows, 0.1, idx=idx)
    assert np.array_equal(dense, masked)
    one = np.full((n, 1), 3, np.int32)
    out, _ = oracle.mha(q, K, V, rows, 0.1, idx=one, which=np.arange(4, n))
    assert np.allclose(out, np.broadcast_to(V[3], out.shape), rtol=0, atol=1e-15)


def test_paged_equals_contiguous():
    """The same sequence in a paged cache (pages permuted) gives bit-identical results."""
    rng = np.random.default_rng(34)
    H, n = 2, 150
    kv, w_uk, w_uv, q = _inputs(rng, n, H)
    K, V = oracle.mha_decompress(kv, w_uk, w_uv)
    out_c, lse_c = oracle.mha(q, K, V, _contig([n]), 0.07)
    P = 3
    perm = np.array([2, 0, 1])
    Kp = np.zeros((P * 64, H, 192))
    Vp = np.zeros((P * 64, H, 128))
    for j in range(P):
        seg = slice(64 * j, min(64 * (j + 1), n))
        m = seg.stop - seg.start
        Kp[64 * perm[j]:64 * perm[j] + m] = K[seg]
        Vp[64 * perm[j]:64 * perm[j] + m] = V[seg]
    rows_p = oracle.Rows(np.zeros(n), np.arange(1, n + 1), page_table=perm[None].astype(np.int32))
    out_p, lse_p = oracle.mha(q, Kp, Vp, rows_p, 0.07)
    assert np.array_equal(out_c, out_p) and np.array_equal(lse_c, lse_p)
