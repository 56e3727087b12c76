"""Checks of the seeded input generator (CPU only)."""

import numpy as np
import torch

import gen as G

MASK = (1 << 64) - 1


def test_splitmix64_published_sequence():
    # First outputs of SplitMix64 seeded with 0 (Steele, Lea & Flood 2014;
    # the values every reference implementation reproduces).
    gamma = 0x9E3779B97F4A7C15
    assert G.splitmix64(0) == 0xE220A8397B1DCDAF
    assert G.splitmix64(gamma) == 0x6E789E6AA1B965F4
    assert G.splitmix64((2 * gamma) & MASK) == 0x06C45D188009454F


def test_counter_construction():
    seed, stream = 1234, 3
    bits = G.raw_bits(seed, stream, 5)
    mix = G.splitmix64(seed)
    for k in range(5):
        assert int(bits[k]) == G.splitmix64(mix ^ (stream << 56) ^ k)


def test_thread_count_independence():
    a = G.normal(5, 1, 37, 129, G.BF16, nthreads=1)
    b = G.normal(5, 1, 37, 129, G.BF16, nthreads=4)
    assert np.array_equal(a, b)
    u1 = G.uniform(5, 4, 1000, 0.5, 1.5, G.F32, nthreads=1)
    u2 = G.uniform(5, 4, 1000, 0.5, 1.5, G.F32, nthreads=3)
    assert np.array_equal(u1, u2)


def test_streams_and_seeds_differ():
    a = G.normal(5, 1, 4, 64, G.F64)
    assert not np.array_equal(a, G.normal(5, 2, 4, 64, G.F64))
    assert not np.array_equal(a, G.normal(6, 1, 4, 64, G.F64))


def test_distributions():
    z = G.normal(21, 1, 1000, 1000, G.F64)
    n = z.size
    assert abs(z.mean()) < 5 / np.sqrt(n)
    assert abs(z.var() - 1) < 5 * np.sqrt(2 / n)
    assert abs((z > 1.0).mean() - 0.15865525393145707) < 5e-3   # normal tail
    u = G.uniform(21, 4, 200000, 0.5, 1.5, G.F64)
    assert u.min() >= 0.5 and u.max() < 1.5
    assert abs(u.mean() - 1.0) < 5 * np.sqrt(1 / 12 / u.size)


def test_outlier_rows_scaled():
    base = G.normal(33, 1, 300, 50, G.F64)
    sc = G.normal(33, 1, 300, 50, G.F64, row_scale=200.0, scale_every=97)
    rows = np.arange(300)
    hit = rows % 97 == 0
    assert hit.sum() == 4
    assert np.array_equal(sc[hit], base[hit] * 200.0)
    assert np.array_equal(sc[~hit], base[~hit])


def test_encodings_match_libraries():
    v = G.normal(44, 1, 100, 1000, G.F64, row_scale=300.0, scale_every=7)
    f16 = G.normal(44, 1, 100, 1000, G.F16, row_scale=300.0, scale_every=7)
    assert np.array_equal(f16, v.astype(np.float16).view(np.uint16))
    bf = G.normal(44, 1, 100, 1000, G.BF16, row_scale=300.0, scale_every=7)
    want = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
    assert np.array_equal(bf, want.numpy().view(np.uint16))
    f32 = G.normal(44, 1, 100, 1000, G.F32, row_scale=300.0, scale_every=7)
    assert np.array_equal(f32, v.astype(np.float32))


def test_workload_table():
    names = [w.name for w in G.WORKLOADS]
    assert len(names) == 5 and len(set(names)) == 5
    w = G.WORKLOADS_BY_NAME["fwd_bf16_m4096_n8192_rstd"]
    assert w.algorithmic_bytes() == 134_250_496
    assert G.WORKLOADS[0].algorithmic_bytes() == 528_384
    assert G.WORKLOADS[2].algorithmic_bytes() == 536_887_296
    assert G.WORKLOADS[3].algorithmic_bytes() == 402_735_104
    assert G.WORKLOADS[4].algorithmic_bytes() == 655_370_000
