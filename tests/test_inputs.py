"""The seeded generator is a pure function of (seed, stream, index)."""
import numpy as np
import torch

from quantized_kv_cache_seal_amd import inputs


def test_splitmix64_reference_values():
    # splitmix64 with state 0: the generator's first outputs as published with the algorithm
    state = 0
    outs = []
    for _ in range(3):
        state = (state + 0x9E3779B97F4A7C15) & inputs.MASK64
        outs.append(inputs.mix64((state - 0x9E3779B97F4A7C15) & inputs.MASK64))
    assert outs[0] == 0xE220A8397B1DCDAF
    assert outs[1] == 0x6E789E6AA1B965F4
    assert outs[2] == 0x06C45D188009454F


def test_slices_are_independent_of_offset():
    a = inputs.normal_np(3, 9, 0, 1001)
    b = inputs.normal_np(3, 9, 37, 500)
    assert np.array_equal(a[37:537], b)
    assert abs(a.mean()) < 0.1 and abs(a.std() - 1) < 0.1


def test_torch_backend_same_words_and_values():
    w_np = inputs.words_np(5, 77, 10, 300)
    w_t = inputs.words_t(5, 77, 10, 300, "cpu")
    assert np.array_equal(w_np.view(np.int64), w_t.numpy())
    z_np = inputs.normal_np(5, 77, 11, 299)
    z_t = inputs.normal_t(5, 77, 11, 299, "cpu").numpy()
    assert np.max(np.abs(z_np - z_t)) < 1e-13


def test_kv_recipe_outliers_and_heavy_tail():
    spec = inputs.KVSpec(2, 2, 256, 4, outliers=5, outlier_scale=15.0)
    k = spec.tokens(1, "k", 0, 2000).astype(np.float64)
    ch = inputs.outlier_channels(4, 1, 0, 256, 5)
    assert len(ch) == 5 and len(set(ch.tolist())) == 5
    s = k[:, 0].std(axis=0)
    assert np.all(s[ch] > 10) and np.median(s) < 1.2
    t = inputs.KVSpec(1, 1, 512, 3, k_dist="student_t3").tokens(0, "k", 0, 400).astype(np.float64)
    kurt = np.mean(t ** 4) / np.mean(t ** 2) ** 2
    assert kurt > 5           # a Gaussian has 3
    signs = inputs.rotation_signs(8)
    assert signs.shape == (2, 128) and set(np.unique(signs)) == {-1, 1}
    words = inputs.signs_to_words(signs)
    assert len(words) == 4 and all(0 <= w < 2 ** 64 for w in words)
