"""Pins for the fp64 oracle, against facts that do not come from the oracle itself.

Each test names what it pins.  Sources: the lightning-indexer formula and token
selection of "DeepSeek-V3.2 技术报告摘要" (section 1, DSA ① and ②, MLA-based MQA
mode), and the "DeepSeek-V3.2 -- Model techniques map" code table (k capped at the
row length, int32 indices, latent 512 + RoPE 64, 192-d per-head q/k, no sink).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(":", 1)
            vals[key.strip()] = rest.strip()
    return vals


def _nums(s):
    return [float(x) for x in s.split()]


def _bf16_bits(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _rows_contig(lens, per_seq_rows=None):
    """One query row per sequence (decode) with len = lens[b], contiguous cache."""
    lens = list(lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    return oracle.Rows(np.arange(len(lens)), lens, seq_start=starts)


def _rows_prefill(L):
    return oracle.Rows(np.zeros(L), np.arange(1, L + 1), seq_start=np.zeros(1))


# --------------------------------------------------------------------------- decoders

def test_bf16_decoder_exhaustive(oracle_lib):
    """All 2^16 bf16 codes decode like torch's bf16 -> float64 cast (a library routine)."""
    codes = np.arange(1 << 16, dtype=np.uint16)
    ours = oracle.bf16_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_e4m3_decoder_exhaustive(oracle_lib):
    """All 256 OCP e4m3fn codes decode like torch.float8_e4m3fn -> float64; max 448; NaN only at 0x7f/0xff."""
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert set(np.nonzero(np.isnan(ours))[0].tolist()) == {0x7F, 0xFF}
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.nanmax(ours) == 448.0
    assert ours[1] == 2.0 ** -9          # smallest subnormal


# --------------------------------------------------------------------------- indexer

def test_indexer_hand_fixture(oracle_lib):
    g = _read_golden("indexer_hand.txt")
    q = np.array([_nums(g["q_head0"]), _nums(g["q_head1"])], dtype=np.float32)[None]
    w = np.array([_nums(g["w"])], dtype=np.float32)
    k = np.array([_nums(g[f"k_s{s}"]) for s in range(4)], dtype=np.float32)
    rows = _rows_contig([4])
    out = oracle.indexer("f32", q, w, k, rows)
    assert out[0].tolist() == _nums(g["expected"])
    for kk in (2, 3, 4):
        sel = oracle.topk(out, rows.row_len, kk)[0]
        assert sel.tolist() == [int(x) for x in _nums(g[f"top{kk}"])]


def test_indexer_orthonormal_closed_form(oracle_lib):
    """Keys = unit vectors e_s, q_j = sum_s c[j,s] e_s  =>  I[s] = sum_j w_j * max(c[j,s], 0)."""
    rng = np.random.default_rng(1)
    H, D = 5, 16
    c = rng.integers(-4, 5, size=(H, D)).astype(np.float32)
    w = rng.integers(0, 4, size=(1, H)).astype(np.float32)
    k = np.eye(D, dtype=np.float32)
    out = oracle.indexer("f32", c[None], w, k, _rows_contig([D]))[0]
    expect = (w[0][:, None] * np.maximum(c, 0)).sum(0)
    assert np.array_equal(out, expect)


def test_indexer_causal_extent_and_per_sequence_keys(oracle_lib):
    """Prefill row t scores exactly positions 0..t (self included); decode rows read their own sequence."""
    rng = np.random.default_rng(2)
    L, H, D = 9, 2, 4
    q = rng.standard_normal((L, H, D)).astype(np.float32)
    w = rng.random((L, H)).astype(np.float32)
    k = rng.standard_normal((L, D)).astype(np.float32)
    out = oracle.indexer("f32", q, w, k, _rows_prefill(L), ld=L)
    for t in range(L):
        assert np.all(np.isfinite(out[t, :t + 1]))
        assert np.all(np.isnan(out[t, t + 1:]))
    # two sequences back to back: row 1 must only see the second block of keys
    rows = _rows_contig([3, 5])
    out2 = oracle.indexer("f32", q[:2], w[:2], k[:8], rows, ld=5)
    solo = oracle.indexer("f32", q[1:2], w[1:2], k[3:8], _rows_contig([5]), ld=5)
    assert np.array_equal(out2[1], solo[0])


def test_indexer_nonnegative_and_linear_in_w(oracle_lib):
    """ReLU terms are >= 0, so I >= 0 for w >= 0; I is linear in w."""
    wl = workloads.config(1)
    q, k = workloads.raw_numpy(wl.q_idx), workloads.raw_numpy(wl.k_idx)
    w = (np.round(workloads.raw_numpy(wl.w) * 256) / 256).astype(np.float32)   # sums stay exact
    rows = _rows_prefill(256)
    which = [0, 1, 7, 100, 255]
    a = oracle.indexer("f32", q, w, k, rows, which=which, ld=256)
    b = oracle.indexer("f32", q, 2 * w, k, rows, which=which, ld=256)
    w2 = np.flip(w, axis=1).copy()
    c = oracle.indexer("f32", q, w2, k, rows, which=which, ld=256)
    d = oracle.indexer("f32", q, w + w2, k, rows, which=which, ld=256)
    fin = np.isfinite(a)
    assert np.all(a[fin] >= 0)
    assert np.array_equal(b[fin], 2 * a[fin])
    np.testing.assert_allclose(d[fin], a[fin] + c[fin], rtol=1e-13, atol=0)


def test_indexer_matches_numpy_einsum_c1(oracle_lib):
    """Library cross-check on the tiny fp32 prefill workload: numpy fp64 einsum + where."""
    wl = workloads.config(1)
    q = workloads.raw_numpy(wl.q_idx).astype(np.float64)
    k = workloads.raw_numpy(wl.k_idx).astype(np.float64)
    w = workloads.raw_numpy(wl.w).astype(np.float64)
    L = q.shape[0]
    out = oracle.indexer("f32", workloads.raw_numpy(wl.q_idx), workloads.raw_numpy(wl.w),
                         workloads.raw_numpy(wl.k_idx), _rows_prefill(L), ld=L)
    dots = np.einsum("thd,sd->ths", q, k)
    ref = np.einsum("th,ths->ts", w, np.where(dots > 0, dots, 0.0))
    mask = np.tril(np.ones((L, L), dtype=bool))
    err = np.max(np.abs(out[mask] - ref[mask])) / np.max(np.abs(ref[mask]))
    assert err < 1e-12
    assert np.all(np.isnan(out[~mask]))


def test_indexer_fp8_factored_scales(oracle_lib):
    """fp8: the literal dequantise-then-dot form equals s_k * sum_j (w_j s_q) relu(q8 . k8)."""
    wl = workloads.decode([40, 70], idx_dtype="fp8", H_I=8, D_I=32, H=4, D_qk=16, D_v=8, topk=16,
                          seed=3)
    q8, k8 = workloads.raw_numpy(wl.q_idx), workloads.raw_numpy(wl.k_idx)
    qs, ks, w = workloads.raw_numpy(wl.q_scale), workloads.raw_numpy(wl.k_scale), workloads.raw_numpy(wl.w)
    rows = oracle.Rows(**{k_: v for k_, v in wl.host_rows().items()})
    out = oracle.indexer("fp8", q8, w, k8, rows, q_scale=qs, k_scale=ks)
    qd = torch.from_numpy(q8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    kd = torch.from_numpy(k8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    starts = wl.seq_start.numpy()
    for r, n in enumerate(wl.lens):
        kr = kd[starts[r]:starts[r] + n]
        dots = qd[r] @ kr.T                               # [H, n] on raw codes
        ref = ks[starts[r]:starts[r] + n].astype(np.float64) * (
            (w[r].astype(np.float64) * qs[r].astype(np.float64)) @ np.maximum(dots, 0))
        np.testing.assert_allclose(out[r, :n], ref, rtol=1e-12, atol=1e-12)


def test_indexer_paged_equals_contiguous_and_permutation_invariant(oracle_lib):
    """Paged cache (64-token pages) gives bit-identical scores to the contiguous cache,
    for any physical placement of the pages."""
    rng = np.random.default_rng(5)
    lens = [130, 64, 3]
    H, D, P = 3, 8, 64
    N = sum(lens)
    q = _bf16_bits(rng.standard_normal((3, H, D)))
    w = rng.random((3, H)).astype(np.float32)
    k = _bf16_bits(rng.standard_normal((N, D)))
    contig = oracle.indexer("bf16", q, w, k, _rows_contig(lens), ld=max(lens))
    npages = [math.ceil(n / P) for n in lens]
    for trial in range(3):
        perm = rng.permutation(sum(npages))
        pt = np.full((3, max(npages)), -1, dtype=np.int32)
        kp = np.zeros((sum(npages), P, D), dtype=np.uint16)
        off = 0
        starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
        for b, n in enumerate(lens):
            for j in range(npages[b]):
                phys = perm[off + j]
                pt[b, j] = phys
                lo = j * P
                hi = min(n, lo + P)
                kp[phys, :hi - lo] = k[starts[b] + lo:starts[b] + hi]
            off += npages[b]
        rows = oracle.Rows(np.arange(3), lens, page_table=pt, page_size=P)
        paged = oracle.indexer("bf16", q, w, kp, rows, ld=max(lens))
        assert np.array_equal(np.isnan(paged), np.isnan(contig))
        assert np.array_equal(paged[~np.isnan(paged)], contig[~np.isnan(contig)])
        assert rows.cache_row(0, 65) == pt[0, 1] * P + 1


# --------------------------------------------------------------------------- top-k

def _beats(x, a, b):
    return x[a] > x[b] or (x[a] == x[b] and a < b)


def test_topk_brute_force_pairwise(oracle_lib):
    """Every selected position beats every unselected one under (score desc, position asc)."""
    rng = np.random.default_rng(7)
    for trial in range(200):
        n = int(rng.integers(1, 14))
        k = int(rng.integers(1, 10))
        x = rng.integers(-3, 4, size=n).astype(np.float64)      # many ties
        x[x == 0] *= rng.choice([-1.0, 1.0], size=int((x == 0).sum()))   # mix -0 and +0
        sel = oracle.topk(x[None], np.array([n]), k)[0]
        keff = min(n, k)
        chosen = sel[:keff].tolist()
        assert all(v == -1 for v in sel[keff:])
        assert chosen == sorted(chosen) and len(set(chosen)) == keff
        rest = [s for s in range(n) if s not in chosen]
        for a in chosen:
            for b in rest:
                assert _beats(x, a, b), (x, chosen)


def test_topk_special_cases(oracle_lib):
    n, k = 50, 8
    equal = np.full((1, n), 3.25)
    assert oracle.topk(equal, [n], k)[0].tolist() == list(range(k))
    inc = np.arange(n, dtype=np.float64)[None]
    assert oracle.topk(inc, [n], k)[0].tolist() == list(range(n - k, n))
    short = oracle.topk(inc, [5], k)[0].tolist()
    assert short == [0, 1, 2, 3, 4, -1, -1, -1]
    # -0 and +0 tie: the lower position wins whatever the sign bit
    z = np.array([[-0.0, 0.0, -0.0, 0.0, -1.0]])
    assert oracle.topk(z, [5], 2)[0].tolist() == [0, 1]
    # ties straddling the boundary: 3 values of 9 above, 4 tied at 5, k = 5
    x = np.array([[5, 9, 5, 1, 9, 5, 9, 5, 0]], dtype=np.float64)
    assert oracle.topk(x, [9], 5)[0].tolist() == [0, 1, 2, 4, 6]
    # float32 input is widened exactly
    assert oracle.topk(x.astype(np.float32), [9], 5)[0].tolist() == [0, 1, 2, 4, 6]


def test_topk_matches_torch_topk_on_distinct_values(oracle_lib):
    """Library cross-check: with distinct values the set equals torch.topk's."""
    g = torch.Generator().manual_seed(11)
    for n, k in [(100, 10), (4096, 2048), (5000, 2048), (3, 2048)]:
        x = torch.randperm(n, generator=g).to(torch.float64) * 0.5 - 7.0
        ours = oracle.topk(x[None].numpy(), [n], k)[0]
        ref = torch.topk(x, min(n, k)).indices.sort().values.numpy()
        assert np.array_equal(ours[:min(n, k)], ref)


def test_topk_permutation_equivariant(oracle_lib):
    """Permuting a row with distinct values permutes the selected set accordingly."""
    rng = np.random.default_rng(13)
    x = rng.permutation(300).astype(np.float64)
    perm = rng.permutation(300)
    a = set(oracle.topk(x[None], [300], 40)[0].tolist())
    b = set(oracle.topk(x[perm][None], [300], 40)[0].tolist())
    assert {int(perm[i]) for i in b} == a


# --------------------------------------------------------------------------- sparse MLA

def test_mla_hand_fixture(oracle_lib):
    g = _read_golden("mla_hand.txt")
    q = np.array([[_nums(g["q"])]], dtype=np.float32)            # [1, 1, 2]
    kv = np.array([_nums(g[f"C_s{s}"]) for s in range(3)], dtype=np.float32)
    out, lse = oracle.sparse_mla("f32", q, kv, np.array([[0, 1, 2]]), _rows_contig([3]), 1.0, 1)
    e = math.e
    assert abs(out[0, 0, 0] - (1 + e * e) / (1 + e + e * e)) < 1e-15
    assert abs(lse[0, 0] - (1 + math.log(1 + e + e * e))) < 1e-14


def test_mla_single_entry_is_its_value(oracle_lib):
    rng = np.random.default_rng(17)
    q = _bf16_bits(rng.standard_normal((1, 4, 24)))
    kv = _bf16_bits(rng.standard_normal((10, 24)))
    idx = np.array([[-1, 6, -1, 40]], dtype=np.int32)             # -1 and out-of-range skipped
    out, lse = oracle.sparse_mla("bf16", q, kv, idx, _rows_contig([10]), 0.3, 16)
    val = oracle.bf16_to_f64(kv[6, :16])
    for h in range(4):
        assert np.array_equal(out[0, h], val)
        z = 0.3 * float(np.dot(oracle.bf16_to_f64(q[0, h]), oracle.bf16_to_f64(kv[6])))
        assert abs(lse[0, h] - z) < 1e-12


def test_mla_identical_keys_or_zero_scale_give_mean(oracle_lib):
    rng = np.random.default_rng(19)
    n, D, Dv = 7, 12, 8
    q = rng.standard_normal((1, 3, D)).astype(np.float32)
    kv = rng.standard_normal((n, D)).astype(np.float32)
    idx = np.arange(n, dtype=np.int32)[None]
    out, lse = oracle.sparse_mla("f32", q, kv, idx, _rows_contig([n]), 0.0, Dv)
    mean = kv[:, :Dv].astype(np.float64).mean(0)
    np.testing.assert_allclose(out[0], np.broadcast_to(mean, (3, Dv)), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse[0], math.log(n), rtol=1e-14)
    # identical key parts, distinct values (keys only read dims >= Dv here via one-hot q)
    kv2 = kv.copy()
    kv2[:, Dv:] = kv[0, Dv:]
    q2 = np.zeros((1, 1, D), dtype=np.float32)
    q2[0, 0, Dv:] = rng.standard_normal(D - Dv)
    out2, lse2 = oracle.sparse_mla("f32", q2, kv2, idx, _rows_contig([n]), 1.0, Dv)
    np.testing.assert_allclose(out2[0, 0], mean, rtol=1e-13, atol=1e-14)
    z = float(np.dot(q2[0, 0].astype(np.float64), kv2[0].astype(np.float64)))
    assert abs(lse2[0, 0] - (z + math.log(n))) < 1e-12


def test_mla_empty_selection(oracle_lib):
    q = np.ones((1, 2, 4), dtype=np.float32)
    kv = np.ones((3, 4), dtype=np.float32)
    out, lse = oracle.sparse_mla("f32", q, kv, np.array([[-1, -1, 5]]), _rows_contig([3]), 1.0, 2)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_mla_dense_equivalence_and_torch_sdpa(oracle_lib):
    """Short context (len <= k): sparse over every position == dense causal MQA ==
    torch scaled_dot_product_attention in fp64 on the CPU (a library routine)."""
    wl = workloads.config(1)
    L, H, Dqk, Dv = 256, wl.H, wl.D_qk, wl.D_v
    q, kv = workloads.raw_numpy(wl.q), workloads.raw_numpy(wl.kv)
    rows = _rows_prefill(L)
    which = [0, 1, 2, 31, 63, 64, 128, 200, 255]
    idx = np.full((L, 256), -1, dtype=np.int32)
    for t in range(L):
        idx[t, :t + 1] = np.arange(t + 1)[::-1]                   # any order of the entries
    sp, sp_lse = oracle.sparse_mla("f32", q, kv, idx, rows, wl.scale, Dv, which=which)
    de, de_lse = oracle.dense_mqa("f32", q, kv, rows, wl.scale, Dv, which=which)
    np.testing.assert_allclose(sp, de, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(sp_lse, de_lse, rtol=1e-13, atol=1e-14)
    qt = torch.from_numpy(q).double().transpose(0, 1)[None]      # [1, H, L, Dqk]
    kt = torch.from_numpy(kv).double()[None, None].expand(1, H, L, Dqk)
    vt = kt[..., :Dv]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                           scale=wl.scale)[0].transpose(0, 1)
    err = oracle.max_abs_rel(de, ref.numpy()[which])
    assert err < 1e-12


def test_mla_mqa_equals_absorbed_mha(oracle_lib):
    """MQA over 576-d entries == per-head MHA with 192-d q/k (128 nope + 64 rope) and 128-d v
    after absorbing random up-projections W_UK, W_UV (pins value = first 512 dims, key = all 576)."""
    rng = np.random.default_rng(23)
    H, R, C, dn, dr, dv = 4, 64, 512, 128, 64, 128
    n = 37
    c = rng.standard_normal((n, C)) * 0.05
    kr = rng.standard_normal((n, dr)) * 0.05
    W_UK = rng.standard_normal((H, dn, C)) * 0.05
    W_UV = rng.standard_normal((H, dv, C)) * 0.05
    qn = rng.standard_normal((H, dn))
    qr = rng.standard_normal((H, dr))
    scale = 1.0 / math.sqrt(dn + dr)
    # MHA reference per head with torch SDPA in fp64
    k_mha = torch.from_numpy(np.concatenate([np.einsum("hdc,nc->hnd", W_UK, c),
                                             np.broadcast_to(kr, (H, n, dr))], axis=-1))
    v_mha = torch.from_numpy(np.einsum("hdc,nc->hnd", W_UV, c))
    q_mha = torch.from_numpy(np.concatenate([qn, qr], axis=-1))[:, None]
    o_mha = torch.nn.functional.scaled_dot_product_attention(q_mha, k_mha, v_mha, scale=scale)[:, 0]
    # absorbed query and MQA entries, in fp32 storage (error ~1e-7)
    q_abs = np.concatenate([np.einsum("hd,hdc->hc", qn, W_UK), qr], axis=-1)[None].astype(np.float32)
    entries = np.concatenate([c, kr], axis=-1).astype(np.float32)
    out, _ = oracle.sparse_mla("f32", q_abs, entries, np.arange(n)[None], _rows_contig([n]), scale, C)
    o_mqa = np.einsum("hdc,hc->hd", W_UV, out[0])
    assert oracle.max_abs_rel(o_mqa, o_mha.numpy()) < 1e-5


def test_mla_paged_permutation_bit_identical(oracle_lib):
    rng = np.random.default_rng(29)
    lens, P, H, D, Dv = [100, 70], 64, 2, 16, 8
    q = _bf16_bits(rng.standard_normal((2, H, D)))
    kv = _bf16_bits(rng.standard_normal((sum(lens), D)))
    idx = np.stack([rng.permutation(100)[:32], rng.permutation(70)[:32]]).astype(np.int32)
    ref, ref_lse = oracle.sparse_mla("bf16", q, kv, idx, _rows_contig(lens), 0.2, Dv)
    npages = [math.ceil(n / P) for n in lens]
    starts = [0, lens[0]]
    for trial in range(3):
        perm = rng.permutation(sum(npages))
        pt = np.full((2, max(npages)), -1, dtype=np.int32)
        kvp = np.zeros((sum(npages), P, D), dtype=np.uint16)
        off = 0
        for b, n in enumerate(lens):
            for j in range(npages[b]):
                pt[b, j] = perm[off + j]
                lo, hi = j * P, min(n, j * P + P)
                kvp[perm[off + j], :hi - lo] = kv[starts[b] + lo:starts[b] + hi]
            off += npages[b]
        out, lse = oracle.sparse_mla("bf16", q, kvp, idx, oracle.Rows([0, 1], lens, page_table=pt), 0.2, Dv)
        assert np.array_equal(out, ref) and np.array_equal(lse, ref_lse)


def test_oracle_thread_count_does_not_change_results(oracle_lib):
    wl = workloads.config(1)
    q, k, w = (workloads.raw_numpy(t) for t in (wl.q_idx, wl.k_idx, wl.w))
    rows = _rows_prefill(256)
    a = oracle.indexer("f32", q, w, k, rows, which=range(0, 256, 5), n_threads=1)
    b = oracle.indexer("f32", q, w, k, rows, which=range(0, 256, 5), n_threads=7)
    assert np.array_equal(np.nan_to_num(a, nan=-1), np.nan_to_num(b, nan=-1))
