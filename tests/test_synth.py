"""Host generator: determinism, counter addressing and the distribution of the synthetic workloads."""
import numpy as np
import pytest

from synth import gen, workloads as W


def test_splitmix64_reference_values():
    # SplitMix64 with seed 0: the first outputs are mix64(GAMMA), mix64(2*GAMMA), ...
    # (published test vector of the reference implementation, seed 0)
    out = gen.uniform_u64(np.uint64(0), np.arange(3, dtype=np.uint64))
    assert [hex(int(v)) for v in out] == ["0xe220a8397b1dcdaf", "0x6e789e6aa1b965f4", "0x6c45d188009454f"]


def test_normals_are_counter_addressed():
    key = gen.stream_key(W.TINY, gen.S_DATA)
    j = np.arange(1000, dtype=np.uint64)
    a = gen.normals(key, j)
    b = gen.normals(key, j[::-1])[::-1]
    assert np.array_equal(a, b)
    assert np.array_equal(gen.normals(key, j[500:]), a[500:])


def test_normal_table_moments():
    t = gen.normal_table()
    assert abs(t.mean()) < 1e-12
    assert t.var() == pytest.approx(1.0, abs=2e-4)
    assert np.all(np.diff(t) > 0)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 1.0 + 2**-9, 65504.0])
    bits = gen.to_bf16_bits(x)
    back = gen.bf16_to_f64(bits)
    assert back.tolist() == [1.0, 1.0, 1.0 + 2**-6, -2.5, 1.0, 65536.0]


def test_kv_windows_agree_with_full_rows():
    wl = W.TINY
    full = gen.kv_tokens(wl, 1, 0, 0, 0, 0, 64, 0, 4)
    part = gen.kv_tokens(wl, 1, 0, 0, 0, 10, 20, 2, 4)
    assert np.array_equal(part, full[10:20, 2:4])


def test_kv_distribution_loop_correlation_and_scales():
    wl = W.LAYER_4K
    sc = gen.scales(wl)
    v = gen.bf16_to_f64(gen.kv_tokens(wl, 1, 0, 0, 3, 0, 4000, 0, 4, sc))   # values: no outliers
    z = v / sc[0, 3, 1][None, None, :]
    assert abs(z.mean()) < 0.02
    assert z.var() == pytest.approx(1.0, rel=0.03)
    rho = np.mean(z[:, 1:, :] * z[:, :-1, :]) / np.mean(z * z)
    assert rho == pytest.approx(0.9, abs=0.01)
    # lognormal(0, 0.5) scales and 4 outlier key channels per head at 10x
    s_v = np.log(sc[:, :, 1, :]).ravel()
    assert s_v.std() == pytest.approx(0.5, rel=0.2)
    # exactly 4 key channels per head carry the 10x factor: their log-scale sits ~log(10) high
    z_k = np.log(sc[:, :, 0, :])
    n_out = (z_k > np.log(10.0) - 4 * 0.5).sum(axis=-1)
    assert (n_out >= 4).all()


def test_queries_are_standard_normal_bf16():
    q = gen.bf16_to_f64(gen.queries(W.LAYER_4K, 0, 1))
    assert q.shape == (32, 16, 128)
    assert abs(q.mean()) < 0.02 and q.std() == pytest.approx(1.0, rel=0.02)


def test_random_indices_range_and_shape():
    wl = W.LAYER_4K
    i = gen.random_indices(wl, 0, 0, 0, 3, 2, 500)
    assert i.shape == (500, 32) and i.min() >= 0 and i.max() < 256
    assert len(np.unique(i)) == 256


def test_ragged_lengths():
    n = gen.context_lengths(W.LAYER_4K, ragged=True, seed=1)
    assert n[0] == 4096 and n.min() >= 1 and n.max() <= 4096 and len(n) == 32


def test_sample_weights_range_zero_share_and_exactness():
    w = gen.sample_weights(W.LAYER_4K, 4000)
    assert w.shape == (4000, W.LAYER_4K.kv_heads, W.LAYER_4K.groups) and w.dtype == np.float32
    assert (w >= 0).all() and (w <= 2).all()
    assert abs((w == 0).mean() - 1 / 16) < 0.01
    nz = w[w > 0].astype(np.float64)
    assert np.array_equal(nz * 2 ** 23, np.round(nz * 2 ** 23)), "weights are multiples of 2^-23"
    assert np.array_equal(gen.sample_weights(W.LAYER_4K, 100), w[:100]), "counter-addressed"
    assert not np.array_equal(gen.sample_weights(W.LAYER_4K, 100, salt=1), w[:100])
