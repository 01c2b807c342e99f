"""The seeded input generator: C library against its numpy mirror, and its statistics."""
import math

import numpy as np
import pytest

import synth


def test_c_matches_numpy_mirror_normal():
    for t in (synth.tid(synth.K_WQKV, 3), synth.tid(synth.K_K_CACHE, 7), 12345):
        for start in (0, 1, 999_983):
            a = synth.normal_bf16(synth.SEED_WEIGHTS, t, start, 4099, 0.02)
            b = synth.normal_bf16_np(synth.SEED_WEIGHTS, t, start, 4099, 0.02)
            assert np.array_equal(a, b)


def test_c_matches_numpy_mirror_gain_uniform_perm():
    t = synth.tid(synth.K_ATTN_NORM, 1)
    assert np.array_equal(synth.gain_bf16(0, t, 17, 3000, 0.02), synth.gain_bf16_np(0, t, 17, 3000, 0.02))
    for n in (1, 7, 1024, 151936):
        assert np.array_equal(synth.uniform_u32(1, 99, 5, 2000, n), synth.uniform_u32_np(1, 99, 5, 2000, n))
    for n in (1, 2, 17, 4096):
        assert np.array_equal(synth.permutation(2, 31, n), synth.permutation_np(2, 31, n))


def test_splitmix64_published_sequence():
    # SplitMix64 seeded with 0 (Steele, Lea & Flood 2014; the reference
    # sequence Vigna distributes with splitmix64.c starts with these words).
    k = 0
    got = [synth._mix64_int(k + (i + 1) * synth.GOLDEN) for i in range(3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_normal_statistics():
    a = synth.normal_bf16(0, 1, 0, 1 << 20, 1.0)
    x = (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert abs(x.mean()) < 5e-3
    assert abs(x.std() - 1.0) < 5e-3
    # Irwin-Hall(4) has excess kurtosis -1.2/4 = -0.3
    kurt = np.mean(x ** 4) / np.mean(x ** 2) ** 2 - 3.0
    assert abs(kurt + 0.3) < 0.05
    s = synth.normal_bf16(0, 1, 0, 1 << 16, 0.02)
    y = (s.astype(np.uint32) << 16).view(np.float32)
    assert abs(float(y.std()) - 0.02) < 5e-4


def test_normal_scale_is_unit_variance_constant():
    sd = math.sqrt(4 * (65536 ** 2 - 1) / 12)
    assert abs(float(synth.normal_scale_np(1.0)) * sd - 1.0) < 1e-7


def test_uniform_and_permutation_valid():
    u = synth.uniform_u32(1, 3, 0, 100000, 1024)
    assert u.min() >= 0 and u.max() < 1024
    assert abs(u.mean() - 511.5) < 5
    p = synth.permutation(2, 4, 10000)
    assert np.array_equal(np.sort(p), np.arange(10000))
    assert not np.array_equal(p, np.arange(10000))


def test_streams_are_distinct_and_subranges_consistent():
    a = synth.normal_bf16(0, 1, 0, 1000, 0.02)
    b = synth.normal_bf16(0, 2, 0, 1000, 0.02)
    c = synth.normal_bf16(1, 1, 0, 1000, 0.02)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)
    assert np.array_equal(synth.normal_bf16(0, 1, 300, 200, 0.02), a[300:500])


def test_expert_slice_is_range_of_full_tensor():
    s = synth.TINY
    full = synth.weight_bits(s, synth.K_W_GATE, 1)
    for e in (0, 5, 7):
        assert np.array_equal(full[e], synth.weight_bits(s, synth.K_W_GATE, 1, e))


def test_workloads_page_tables():
    for name in synth.WORKLOADS:
        w = synth.workload(name)
        pt = w.page_table()
        used = pt[pt >= 0]
        assert len(np.unique(used)) == len(used) == w.num_pages - w.spare_pages
        assert used.max() < w.num_pages
    r = synth.workload("moe30b_bs8_ragged")
    assert all(1024 <= c <= 32768 for c in r.context) and len(set(r.context)) > 1
