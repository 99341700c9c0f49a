"""Pins for the oracle's indexer-input and cache-write prep, against facts that do not come from
the oracle itself.

Sources: the "DeepSeek-V3.2-Exp" README, section "更新" (the 2025-11-17 update: the indexer's
RoPE takes the non-interleaved layout, the MLA's RoPE the interleaved one); the FP8 indexer of
"DeepSeek-V3.2 技术报告摘要" (section 1, DSA ①); the bf16 latent cache of the "DeepSeek-V3.2"
model docs (section 5.3).  The rotation, format and quantisation definitions are in
oracle/dsa_oracle.h.
"""
import math

import numpy as np
import torch

import oracle


def _table(max_pos, base=10000.0):
    """A textbook RoPE frequency schedule: angle i of position p is p * base^(-i/32)."""
    i = np.arange(32, dtype=np.float64)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * base ** (-i / 32.0)[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _bf16_val(bits):
    return oracle.bf16_to_f64(bits)


def _keys(idx_dtype, pos, cs, k_in, kv_in, n_rows=None, rows_out=None):
    T = len(pos)
    n_rows = T if n_rows is None else n_rows
    rows_out = np.arange(T, dtype=np.int64) if rows_out is None else rows_out
    kc = np.zeros((n_rows, 128), dtype=np.uint16 if idx_dtype == "bf16" else np.uint8)
    kvc = np.zeros((n_rows, 576), dtype=np.uint16)
    ks = np.zeros(n_rows, dtype=np.float32) if idx_dtype == "fp8" else None
    return oracle.prep_keys(idx_dtype, pos, rows_out, cs, k_in, kv_in, kc, kvc, ks)


# ------------------------------------------------------------------------ number formats

def test_bf16_codes_match_torch_rounding():
    """The bf16 code is the round-to-nearest-even conversion torch implements (random values,
    exact halfway cases of both parities, signed zeros, subnormals)."""
    g = np.random.default_rng(1)
    x = (g.standard_normal(20000) * np.exp(g.uniform(-30, 30, 20000))).astype(np.float32)
    base = _bf16_val(_bf16_bits(g.standard_normal(2000))).astype(np.float32)
    halves = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)   # exactly halfway
    x = np.concatenate([x, halves, np.array([0.0, -0.0, 1e-40, -3e-39], np.float32)])
    assert np.array_equal(oracle.bf16_codes(x), _bf16_bits(x))


def test_e4m3_codes_match_torch_rounding():
    """The e4m3 code is torch's float8_e4m3fn conversion for |x| <= 448 (nearest, ties to even),
    incl. exact halfway points between neighbouring codes and the subnormal range."""
    g = np.random.default_rng(2)
    x = (g.uniform(-1, 1, 20000) * np.exp2(g.uniform(-12, 8.8, 20000))).astype(np.float32)
    x = x[np.abs(x) <= 448]
    vals = oracle.e4m3_to_f64(np.arange(0, 0x7F, dtype=np.uint8))      # finite magnitudes
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)               # exactly representable
    x = np.concatenate([x, mids, -mids, np.array([0.0, -0.0, 448.0, -448.0], np.float32)])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_codes(x), ref)
    # beyond the largest finite value the code saturates to 448
    assert list(oracle.e4m3_codes(np.array([449.0, 470.0, 1e6, -1e6], np.float32))) == \
        [0x7E, 0x7E, 0x7E, 0xFE]


# ------------------------------------------------------------------------ rotation layouts

def test_position_zero_is_identity():
    """At position 0 every angle is 0 (cos 1, sin 0): the bf16 outputs are the inputs, bit for
    bit, for the indexer key, the latent entry and both query kinds."""
    g = np.random.default_rng(3)
    cs = _table(4)
    k_in = _bf16_bits(g.standard_normal((5, 128)))
    kv_in = _bf16_bits(g.standard_normal((5, 576)))
    kc, kvc, _ = _keys("bf16", np.zeros(5, np.int32), cs, k_in, kv_in)
    assert np.array_equal(kc, k_in) and np.array_equal(kvc, kv_in)
    qi = _bf16_bits(g.standard_normal((2, 64, 128)))
    q = _bf16_bits(g.standard_normal((2, 4, 576)))
    qo, qs, q2 = oracle.prep_queries("bf16", np.zeros(2, np.int32), cs, qi, q)
    assert qs is None and np.array_equal(qo, qi) and np.array_equal(q2, q)


def test_indexer_rotation_is_non_interleaved_and_mla_interleaved():
    """One-hot inputs show which dims form a pair and the sign of the rotation: the indexer pairs
    dim i with i + 32 inside its first 64 dims, the latent entry pairs 512 + 2i with 513 + 2i;
    (a, b) -> (a cos - b sin, b cos + a sin).  Every pair gets cos 0.6 and sin 0.8, so the
    two outputs of a one-hot pair are distinct and signed."""
    cs = np.zeros((1, 64), np.float32)
    cs[0, :32], cs[0, 32:] = 0.6, 0.8
    for i in (0, 5, 31):
        for src, part in ((i, "a"), (i + 32, "b")):
            k_in = np.zeros((1, 128), np.float32)
            k_in[0, src] = 1.0
            kc, _, _ = _keys("bf16", np.zeros(1, np.int32), cs, _bf16_bits(k_in),
                             np.zeros((1, 576), np.uint16))
            got = _bf16_val(kc[0])
            exp = np.zeros(128)
            if part == "a":                    # (1, 0) -> (cos, sin)
                exp[i], exp[i + 32] = 0.6, 0.8
            else:                              # (0, 1) -> (-sin, cos)
                exp[i], exp[i + 32] = -0.8, 0.6
            assert np.allclose(got, _bf16_val(_bf16_bits(exp))), (i, part)
        for src, part in ((512 + 2 * i, "a"), (513 + 2 * i, "b")):
            kv_in = np.zeros((1, 576), np.float32)
            kv_in[0, src] = 1.0
            _, kvc, _ = _keys("bf16", np.zeros(1, np.int32), cs, np.zeros((1, 128), np.uint16),
                              _bf16_bits(kv_in))
            got = _bf16_val(kvc[0])
            exp = np.zeros(576)
            if part == "a":
                exp[512 + 2 * i], exp[513 + 2 * i] = 0.6, 0.8
            else:
                exp[512 + 2 * i], exp[513 + 2 * i] = -0.8, 0.6
            assert np.allclose(got, _bf16_val(_bf16_bits(exp))), (i, part)


def test_rotation_keeps_pair_norms_and_relative_positions():
    """A rotation keeps each pair's length, and the dot product of a rotated query and key
    depends only on the distance of their positions (within the bf16 rounding of the
    outputs): the pair index used for the angle matches on both sides."""
    g = np.random.default_rng(4)
    cs = _table(4096)
    x = g.standard_normal((1, 128))
    k_bits = _bf16_bits(x)
    xv = _bf16_val(k_bits)
    for p in (1, 17, 4000):
        kc, _, _ = _keys("bf16", np.array([p], np.int32), cs, k_bits, np.zeros((1, 576), np.uint16))
        y = _bf16_val(kc[0])
        for i in range(32):
            n0 = math.hypot(xv[0, i], xv[0, i + 32])
            n1 = math.hypot(y[i], y[i + 32])
            assert abs(n1 - n0) <= 2 ** -7 * n0 + 1e-30
        assert np.array_equal(y[64:], xv[0, 64:])              # the rest is untouched
    qb = _bf16_bits(g.standard_normal((1, 1, 128)))
    kb = _bf16_bits(g.standard_normal((1, 128)))

    def dot(m, n):
        qo, _, _ = oracle.prep_queries("bf16", np.array([m], np.int32), cs, qb,
                                       np.zeros((1, 1, 576), np.uint16))
        kc, _, _ = _keys("bf16", np.array([n], np.int32), cs, kb, np.zeros((1, 576), np.uint16))
        return float(np.dot(_bf16_val(qo[0, 0]), _bf16_val(kc[0])))

    ref = dot(100, 37)
    scale = float(np.linalg.norm(_bf16_val(qb)) * np.linalg.norm(_bf16_val(kb)))
    for d in (1, 500, 3000):
        assert abs(dot(100 + d, 37 + d) - ref) <= 2e-2 * scale
    assert abs(dot(100, 36) - ref) > 1e-3 * scale            # a different distance differs


# ------------------------------------------------------------------------ fp8 quantisation

def test_fp8_key_quantisation_per_token():
    """Per token: the largest rotated magnitude maps to +-448 (code 0x7E / 0xFE), the scale is
    that magnitude / 448, and every code decodes to within half a step of the rotated value
    (computed here in fp64 from the same rotation)."""
    g = np.random.default_rng(5)
    cs = _table(64)
    T = 6
    k_bits = _bf16_bits(g.standard_normal((T, 128)) * np.exp(g.uniform(-3, 3, (T, 1))))
    pos = np.array([0, 1, 9, 33, 62, 63], np.int32)
    kc, _, ks = _keys("fp8", pos, cs, k_bits, np.zeros((T, 576), np.uint16))
    x = _bf16_val(k_bits)
    c, s = cs[pos, :32].astype(np.float64), cs[pos, 32:].astype(np.float64)
    y = x.copy()
    y[:, :32] = x[:, :32] * c - x[:, 32:64] * s
    y[:, 32:64] = x[:, 32:64] * c + x[:, :32] * s
    amax = np.abs(y).max(axis=1)
    assert np.allclose(ks, amax / 448.0, rtol=1e-6)
    for t in range(T):
        assert np.max(kc[t] & 0x7F) == 0x7E
        deq = oracle.e4m3_to_f64(kc[t]) * float(ks[t])
        step = np.where(np.abs(y[t]) / ks[t] >= 2 ** -6, np.abs(y[t]) * 2 ** -3, 2 ** -9 * ks[t])
        assert np.all(np.abs(deq - y[t]) <= 0.5 * step + 1e-6 * amax[t])
        assert np.all(np.sign(deq[deq != 0]) == np.sign(y[t][deq != 0]))


def test_fp8_query_scales_per_head_and_zero_vector():
    """Query heads are quantised independently (one scale per row and head); an all-zero head
    gets scale 1 and codes of zero (signed as the rotation's zero products are)."""
    g = np.random.default_rng(6)
    cs = _table(8)
    qi = g.standard_normal((2, 64, 128))
    qi[1, 7] = 0.0
    qb = _bf16_bits(qi)
    qo, qs, _ = oracle.prep_queries("fp8", np.array([3, 5], np.int32), cs, qb,
                                    np.zeros((2, 1, 576), np.uint16))
    assert qs.shape == (2, 64) and qs[1, 7] == 1.0 and not (qo[1, 7] & 0x7F).any()
    for r in range(2):
        for h in range(64):
            if (r, h) != (1, 7):
                assert np.max(qo[r, h] & 0x7F) == 0x7E


def test_skipped_tokens_leave_the_cache_untouched():
    """Tokens with a position outside the table or a cache row outside the cache write
    nothing; the others land in the rows they name."""
    g = np.random.default_rng(7)
    cs = _table(16)
    k_bits = _bf16_bits(g.standard_normal((4, 128)))
    kv_bits = _bf16_bits(g.standard_normal((4, 576)))
    pos = np.array([2, 16, -1, 5], np.int32)
    rows = np.array([9, 1, 2, 3], np.int64)
    kc, kvc, _ = _keys("bf16", pos, cs, k_bits, kv_bits, n_rows=8, rows_out=rows)
    # token 0 names row 9 (beyond 8 rows), tokens 1 and 2 have bad positions: only row 3 is set
    assert not kc[[0, 1, 2, 4, 5, 6, 7]].any() and not kvc[[0, 1, 2, 4, 5, 6, 7]].any()
    one, one_kv, _ = _keys("bf16", pos[3:], cs, k_bits[3:], kv_bits[3:])
    assert np.array_equal(kc[3], one[0]) and np.array_equal(kvc[3], one_kv[0])
