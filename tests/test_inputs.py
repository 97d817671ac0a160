"""The seeded input generator: determinism, per-head streams, laws, row samples (CPU)."""
import numpy as np

from flashattention_tiling_online_amd import inputs


def test_deterministic_and_per_head_independent():
    w = inputs.custom("t", 2, 3, 33, 17, 8, "bf16", False, seed=12)
    a = inputs.make_tensor(w, "k")
    b = inputs.make_tensor(w, "k")
    np.testing.assert_array_equal(a, b)
    # any head regenerates alone
    one = inputs.round_fp32(inputs.head_values(12, "k", 1, 2, 17, 8, 1.0), "bf16")
    np.testing.assert_array_equal(a[1, 2], one)
    # different tensors / heads / seeds differ
    assert not np.array_equal(a, inputs.make_tensor(w, "v"))
    assert not np.array_equal(a[0, 0], a[0, 1])


def test_value_law_sigma():
    w = inputs.custom("t", 1, 2, 4096, 4096, 64, "f32", False, seed=3, sigma_q=3.0)
    q = inputs.make_tensor(w, "q").astype(np.float64)
    v = inputs.make_tensor(w, "v").astype(np.float64)
    assert abs(q.std() - 3.0) < 0.02 and abs(q.mean()) < 0.02
    assert abs(v.std() - 1.0) < 0.01


def test_workloads_table():
    w = inputs.WORKLOADS
    assert (w["self_8k_causal"].flops == 0.5 * 4 * 16 * 8192 * 8192 * 128)
    assert w["cross_1k_8k"].Nq == 1024 and w["cross_1k_8k"].Nk == 8192
    assert w["ctx_32k_causal"].sigma_q == 3.0 and w["ctx_32k_causal"].sigma_v == 1.0
    assert w["single_head_fp32"].dtype == "f32"
    assert np.float32(w["long_4k"].scale) == np.float32(1 / np.sqrt(128))


def test_sample_rows():
    w = inputs.WORKLOADS["ctx_32k_causal"]
    bh, rows = inputs.sample_rows(w, 4, 256)
    assert bh.size == rows.size == 1024
    assert len(np.unique(bh)) == 4
    for h in np.unique(bh):
        r = rows[bh == h]
        assert len(np.unique(r)) == 256 and r.min() >= 0 and r.max() < w.Nq
    bh2, rows2 = inputs.sample_rows(w, 4, 256)
    np.testing.assert_array_equal(bh, bh2)
    np.testing.assert_array_equal(rows, rows2)
    # all rows when the sample asks for at least Nq
    w2 = inputs.custom("t", 1, 2, 10, 10, 8, "bf16", False, seed=1)
    bh3, rows3 = inputs.sample_rows(w2, 5, 100)
    assert bh3.size == 20 and set(rows3.tolist()) == set(range(10))


def test_round_fp32_to_bf16_matches_fp64_path():
    """The in-place bit rounding equals the general fp64 rounding on fp32 inputs,
    including ties, carries into the exponent, overflow and subnormals."""
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        (rng.standard_normal(1000) * 1e-39).astype(np.float32),
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 3.3895314e38, -3.4e38, 0.0, -0.0,
                                  np.inf, -np.inf], dtype=np.float32)])
    got = inputs.round_fp32(x.copy(), "bf16")
    want = inputs.round_fp64(x.astype(np.float64), "bf16")
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(inputs.round_fp32(x, "f16"),
                                  inputs.round_fp64(x.astype(np.float64), "f16"))
