"""The seeded input generator (host side; the GPU suite checks device == host)."""
import numpy as np
import pytest
from scipy import stats

import zsgen
from zsgen.workloads import WORKLOADS, llama_block_params


def test_deterministic_and_split_independent():
    a = zsgen.host_f32(3, 1, 0, 0, 0.02, 12345, 100_001, threads=8)
    b = zsgen.host_f32(3, 1, 0, 0, 0.02, 12345, 100_001, threads=1)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    c = np.concatenate([zsgen.host_f32(3, 1, 0, 0, 0.02, 12345, 7),
                        zsgen.host_f32(3, 1, 0, 0, 0.02, 12352, 100_001 - 7)])
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))
    idx = np.array([12345, 12346, 50_000, 112_345], np.int64)
    assert np.array_equal(zsgen.host_f32_at(3, 1, 0, 0, 0.02, idx).view(np.uint32),
                          a[idx - 12345].view(np.uint32))
    g = zsgen.host_bf16(1, 4, 2, 5, 1e-3, 999, 50_000, p_out=0.01, sigma_out=0.1)
    gi = zsgen.host_bf16_at(1, 4, 2, 5, 1e-3, np.arange(999, 50_999), p_out=0.01, sigma_out=0.1)
    assert np.array_equal(g, gi)


def test_streams_differ():
    base = zsgen.host_f32(0, 1, 0, 0, 1.0, 0, 10_000)
    for args in ((1, 1, 0, 0), (0, 2, 0, 0), (0, 1, 1, 0), (0, 1, 0, 1)):
        other = zsgen.host_f32(*args, 1.0, 0, 10_000)
        assert abs(np.corrcoef(base, other)[0, 1]) < 0.05


@pytest.mark.parametrize("sigma", [0.02, 1e-3, 1e-6])
def test_normal_distribution(sigma):
    x = zsgen.host_f32(7, 1, 0, 0, sigma, 0, 1_000_000).astype(np.float64) / sigma
    assert abs(x.mean()) < 0.005 and abs(x.std() - 1) < 0.005
    assert stats.kstest(x, "norm").pvalue > 1e-4


def test_bf16_values_and_outliers():
    g = zsgen.host_bf16(1, 4, 0, 1, 1e-3, 0, 2_000_000)
    f = (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert abs(f.std() / 1e-3 - 1) < 0.01          # truncation to 8 bits shrinks by < 0.4%
    o = zsgen.host_bf16(1, 4, 0, 1, 1e-3, 0, 2_000_000, p_out=0.01, sigma_out=0.1)
    fo = (o.astype(np.uint32) << 16).view(np.float32)
    changed = np.count_nonzero(o != g) / o.size
    assert 0.009 < changed < 0.011
    big = np.abs(fo) > 0.01
    assert 0.0085 < big.mean() < 0.0100


def test_abs_stream_is_nonnegative():
    v = zsgen.host_f32(2, 3, 0, 0, 1e-6, 0, 100_000, absval=True)
    assert (v >= 0).all() and v.max() > 0


def test_workload_shapes():
    assert llama_block_params() == 218_112_000
    assert WORKLOADS["fsdp_llama_units"].psi == llama_block_params()
    assert WORKLOADS["zero2_7b"].psi // WORKLOADS["zero2_7b"].n_d == 875_000_000
    assert WORKLOADS["zero3_70b"].psi // WORKLOADS["zero3_70b"].n_d == 1_093_750_000
