"""The seeded input generator: determinism, encodings, structure of the five workloads."""
import math

import numpy as np
import torch

import workloads


def test_same_seed_same_bytes_and_different_seed_differs():
    a = workloads.decode([100, 37], H_I=4, D_I=16, H=2, D_qk=24, D_v=16, topk=8, seed=5)
    b = workloads.decode([100, 37], H_I=4, D_I=16, H=2, D_qk=24, D_v=16, topk=8, seed=5)
    c = workloads.decode([100, 37], H_I=4, D_I=16, H=2, D_qk=24, D_v=16, topk=8, seed=6)
    for f in ("q_idx", "k_idx", "w", "q", "kv"):
        assert np.array_equal(workloads.raw_numpy(getattr(a, f)), workloads.raw_numpy(getattr(b, f)))
    assert not np.array_equal(workloads.raw_numpy(a.kv), workloads.raw_numpy(c.kv))


def test_fp8_codes_finite_and_scales_positive():
    wl = workloads.decode([300, 5], idx_dtype="fp8", H_I=8, D_I=64, H=2, D_qk=16, D_v=8, topk=8, seed=9)
    for t in (wl.q_idx, wl.k_idx):
        codes = workloads.raw_numpy(t)
        assert not np.any((codes & 0x7F) == 0x7F)            # no NaN code
        assert float(t.to(torch.float32).abs().max()) == 448.0   # amax lands on the top code
    assert torch.all(wl.q_scale > 0) and torch.all(wl.k_scale > 0)
    assert wl.q_scale.shape == (2, 8) and wl.k_scale.shape == (305,)
    # per-token scale: every head of a query token shares it
    assert torch.all(wl.q_scale == wl.q_scale[:, :1])


def test_paged_layout_is_a_permutation_of_pages():
    lens = [130, 64, 1, 700]
    wl = workloads.decode(lens, paged=True, H_I=2, D_I=8, H=2, D_qk=16, D_v=8, topk=8, seed=4)
    npages = [math.ceil(n / 64) for n in lens]
    pt = wl.page_table.numpy()
    used = np.concatenate([pt[b, :n] for b, n in enumerate(npages)])
    assert sorted(used.tolist()) == list(range(sum(npages)))
    for b, n in enumerate(npages):
        assert np.all(pt[b, n:] == -1)
    assert wl.kv.shape == (sum(npages), 64, 16) and wl.k_idx.shape == (sum(npages), 64, 8)


def test_named_configs_shapes():
    c1 = workloads.config(1)
    assert (c1.H_I, c1.D_I, c1.H, c1.D_qk, c1.D_v, c1.topk) == (4, 32, 8, 80, 64, 64)
    assert c1.row_len.tolist() == list(range(1, 257))
    assert abs(c1.scale - 1 / math.sqrt(80)) < 1e-15
    lens = workloads.c5_lengths(1005)
    assert len(lens) == 32 and min(lens) >= 1024 and max(lens) <= 65536
    assert sum(1 for n in lens if n < 2048) >= 2                  # some rows select everything


def test_bf16_rounding_is_nearest_even():
    x = torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], dtype=torch.float32)
    assert workloads._round(x, "bf16").float().tolist() == [1.0, 1.0 + 2 ** -6]
