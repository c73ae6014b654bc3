"""The seeded input generator: determinism, chunking, bf16 rounding, skew shape."""
import numpy as np
import pytest
import torch

from synth import WORKLOADS, gen


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100_000).astype(np.float32) * 50,
                        np.array([0.0, -0.0, 1.0, -1.0, 1.00390625, 1.01171875, 3e-39],
                                 dtype=np.float32)])
    ours = gen.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(gen.bf16_bits_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("name", ["tiny_fp32", "opt6.7b", "llama7b_stream"])
def test_chunked_generation_equals_whole(name):
    wl = WORKLOADS[name]
    n = min(wl.n_positions, 9000)
    whole = gen.unit_storage(wl, 0, 1, 0, n)
    for a, b in [(0, 100), (4000, 4200), (4095, 8193), (n - 5, n)]:
        if b > n:
            continue
        part = gen.unit_storage(wl, 0, 1, a, b)
        for w, p in zip(whole, part):
            np.testing.assert_array_equal(w[a:b], p)


def test_determinism_and_distinct_streams():
    wl = WORKLOADS["opt6.7b"]
    a = gen.unit_storage(wl, 1, 2, 0, 64)
    b = gen.unit_storage(wl, 1, 2, 0, 64)
    c = gen.unit_storage(wl, 2, 1, 0, 64)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a[1], c[1])
    assert not np.array_equal(a[0], a[1])


def test_batch_storage_matches_units():
    wl = WORKLOADS["opt6.7b"]
    q, k, v = gen.batch_storage(wl, 10, 20)
    assert q.shape == (wl.batch, wl.heads, 10, wl.head_dim) and q.dtype == np.uint16
    for b, h in [(0, 0), (3, 17), (7, 31)]:
        uq, uk, uv = gen.unit_storage(wl, b, h, 10, 20)
        np.testing.assert_array_equal(q[b, h], uq)
        np.testing.assert_array_equal(k[b, h], uk)
        np.testing.assert_array_equal(v[b, h], uv)
    sub = gen.batch_storage(wl, 10, 20, units=[(3, 17)])
    np.testing.assert_array_equal(sub[1][0], k[3, 17])


def test_skew_shapes():
    c1 = WORKLOADS["tiny_fp32"]
    a = gen.skew_amplitudes(c1, 0, 0)
    assert (a > 0).sum() == round(0.08 * c1.n_positions) and set(np.unique(a)) == {0.0, 3.0}
    c4 = WORKLOADS["neox20b"]
    a = gen.skew_amplitudes(c4, 0, 0)
    hot = np.flatnonzero(a)
    assert len(hot) == 19 * 16
    assert all((hot.reshape(19, 16)[:, 0] % 16) == 0)
    c3 = WORKLOADS["opt30b"]
    a = gen.skew_amplitudes(c3, 0, 0)
    ranks = np.sort(a)[::-1]
    # logit boost alpha*ln(N/rho): top rank and the rank-ratio law
    boost = ranks * 1.5 * c3.scale
    assert boost[0] == pytest.approx(1.1 * np.log(c3.n_positions), rel=1e-5)
    assert boost[0] - boost[9] == pytest.approx(1.1 * np.log(10), rel=1e-5)
    c5 = WORKLOADS["llama7b_stream"]
    a = gen.skew_amplitudes(c5, 0, 3)
    np.testing.assert_array_equal(a[:5000], a[5000:10000])
    u = gen.skew_direction(c1, 1)
    assert np.linalg.norm(u) == pytest.approx(1.0, rel=1e-6)


def test_query_offset_and_value_no_skew():
    wl = WORKLOADS["tiny_fp32"]
    q, k, v = gen.unit_raw(wl, 0, 0, 0, wl.n_positions)
    u = gen.skew_direction(wl, 0)
    # the planted direction is visible in the query mean, not in the values
    assert float(q.mean(0) @ u) == pytest.approx(1.5, abs=0.3)
    assert abs(float(v.mean(0) @ u)) < 0.3
