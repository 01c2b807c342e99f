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


def test_fp8_codes_and_scales_c_equals_numpy():
    for kind, idx, start, n in ((synth.K_WQKV, 0, 0, 70001), (synth.K_W_GATE, 5, 123457, 50000)):
        t = synth.tid(kind, idx)
        assert np.array_equal(synth.fp8_codes(0, t, start, n), synth.fp8_codes_np(0, t, start, n))
        ts = synth.tid(synth.FP8_SCALE_KIND + kind, idx)
        assert np.array_equal(synth.fp8_scales(0, ts, start, 999), synth.fp8_scales_np(0, ts, start, 999))


def test_e4m3_encoder_picks_the_nearest_code_ties_to_even():
    """Brute force over every finite code (decoded by torch): the encoder's code is nearest, and an
    exact midpoint goes to the code with an even mantissa; beyond 464 it saturates to 448."""
    import torch
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    rng = np.random.default_rng(5)
    mids = (vals[1:] + vals[:-1]) / 2
    x = np.concatenate([rng.uniform(0, 470, 20000), rng.uniform(0, 0.03, 5000), mids,
                        [0.0, 448.0, 463.99, 464.0, 1e4]]).astype(np.float32)
    for sgn in (1.0, -1.0):
        xs = (sgn * x).astype(np.float32)
        got = synth.e4m3_rne_np(xs)
        # the C encoder agrees with the mirror (on every midpoint and a sample of the rest)
        pick = np.concatenate([np.arange(0, len(xs), 17), np.arange(25000, len(xs))])
        assert np.array_equal(got[pick], np.array([synth.lib().synth_e4m3_rne(float(v)) for v in xs[pick]],
                                                  dtype=np.uint8))
        mag = np.abs(xs.astype(np.float64))
        d = np.abs(mag[:, None] - vals[None, :])
        best = d.min(1)
        cand = d == best[:, None]
        want = np.where(cand.sum(1) == 1, cand.argmax(1),
                        np.where(cand & ((codes[None, :] & 1) == 0), codes[None, :], 255).min(1))
        want = np.where(mag >= 464.0, 0x7E, want)
        assert np.array_equal(got & 0x7F, want.astype(np.uint8))
        assert np.all((got >> 7)[mag > 0] == (1 if sgn < 0 else 0))


def test_fp8_weight_slices_and_workloads():
    from dataclasses import replace
    s = replace(synth.TINY, weights="fp8")
    codes, scales = synth.weight_fp8(s, synth.K_W_DOWN, 1)
    assert codes.shape == s.weight_shape(synth.K_W_DOWN) and codes.dtype == np.uint8
    assert scales.shape == (s.n_experts * s.hidden,) and scales.dtype == np.float32
    for e in (0, 5):
        c, sc = synth.weight_fp8(s, synth.K_W_DOWN, 1, e)
        assert np.array_equal(c, codes[e]) and np.array_equal(sc, scales[e * s.hidden:(e + 1) * s.hidden])
    assert s.weight_nbytes(synth.K_W_DOWN) == codes.size + 4 * scales.size
    assert s.weight_nbytes(synth.K_ROUTER) == 2 * s.n_experts * s.hidden
    w = synth.workload("moe30b_8k_fp8")
    assert w.shape.weights == "fp8" and w.context == [8192] and w.name == "moe30b_8k_fp8"
    assert synth.workload("moe30b_8k").shape.weights == "bf16"
    # codes never saturate and use both signs; scales sit near sigma / 32
    assert (codes & 0x7F).max() < 0x7E and (codes >> 7).min() == 0 and (codes >> 7).max() == 1
    assert np.all(np.abs(scales / (synth.WEIGHT_SIGMA / 32) - 1) < 0.2)


def test_fp4_codes_c_equals_numpy_and_encoder_is_nearest():
    for kind, idx, start, n in ((synth.K_WQKV, 0, 0, 70002), (synth.K_W_DOWN, 5, 123456, 50000)):
        t = synth.tid(kind, idx)
        assert np.array_equal(synth.fp4_codes(0, t, start, n), synth.fp4_codes_np(0, t, start, n))
        ts = synth.tid(synth.FP8_SCALE_KIND + kind, idx)
        assert np.array_equal(synth.fp4_scales(0, ts, start, 999), synth.fp4_scales_np(0, ts, start, 999))
    vals = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.uniform(-7, 7, 20000), (vals[1:] + vals[:-1]) / 2, -(vals[1:] + vals[:-1]) / 2]).astype(np.float32)
    got = synth.e2m1_rne_np(x)
    assert np.array_equal(got[::50], np.array([synth.lib().synth_e2m1_rne(float(v)) for v in x[::50]], dtype=np.uint8))
    mag = np.abs(x.astype(np.float64))
    d = np.abs(mag[:, None] - vals[None, :])
    cand = d == d.min(1)[:, None]
    want = np.where(cand.sum(1) == 1, cand.argmax(1), np.where(cand & (np.arange(8)[None, :] % 2 == 0), np.arange(8)[None, :], 99).min(1))
    assert np.array_equal(got & 7, want.astype(np.uint8))
    assert np.all((got >> 3)[x < 0] == 1) and np.all((got >> 3)[x > 0] == 0)
