"""The seeded input generator (workloads/): same seed -> same bytes, and the
documented structure of the synthetic Llama-shaped inputs.

The stored SHA-256 digests were taken with numpy 2.2 (PCG64 through
default_rng); a numpy release that changed the generator's stream would
change every input of the parity tests and the benchmark, and this test
says so before anything else does."""
import hashlib

import numpy as np

import workloads as wl

W_SHA = "0f9ec4be067f13c25db9fffb99165461fc969287b5890a004e289cca866e9779"
X_SHA = "2c6a301c63c1aa0c909fc15657e200ec84c07ccea9c97a3bdad4577c03b0d8c7"


def test_same_seed_same_bytes():
    w = wl.gen_weights(64, 512, wl.seed_w(wl.TINY))
    x = wl.gen_activations(16, 512, wl.seed_x(wl.TINY), wl.seed_outliers(wl.TINY))
    assert hashlib.sha256(w.tobytes()).hexdigest() == W_SHA
    assert hashlib.sha256(x.tobytes()).hexdigest() == X_SHA
    assert np.array_equal(w, wl.gen_weights(64, 512, wl.seed_w(wl.TINY)))
    assert not np.array_equal(w, wl.gen_weights(64, 512, wl.seed_w(wl.TINY) + 1))


def test_row_prefix_property():
    """A draw of fewer rows with the same seed is exactly the leading rows of
    a larger draw (the benchmark's CPU baseline samples channels this way)."""
    big = wl.gen_weights(256, 1024, 5)
    small = wl.gen_weights(64, 1024, 5)
    assert np.array_equal(small, big[:64])
    xb = wl.gen_activations(64, 1024, 6, 7)
    xs = wl.gen_activations(10, 1024, 6, 7)
    assert np.array_equal(xs, xb[:10])


def test_distributions_and_outliers():
    """Weights ~ N(0, 0.02); activations ~ N(0, 1) with round(1 % of K)
    channels, the same for every token, scaled by 20."""
    w = wl.gen_weights(512, 4096, 11)
    assert w.dtype == np.float32
    assert abs(float(w.std()) - 0.02) < 5e-4 and abs(float(w.mean())) < 5e-4
    K = 8192
    ch = wl.outlier_channels(K, 3)
    assert len(ch) == round(0.01 * K) and len(set(ch.tolist())) == len(ch)
    x = wl.gen_activations(64, K, 2, 3)
    rng = np.random.default_rng(2)
    base = rng.standard_normal((64, K), dtype=np.float32)
    mask = np.zeros(K, bool)
    mask[ch] = True
    np.testing.assert_array_equal(x[:, ~mask], base[:, ~mask])
    np.testing.assert_array_equal(x[:, mask], base[:, mask] * np.float32(20.0))
    # every Llama config's K gets its documented outlier count
    for k, n in ((512, 5), (4096, 41), (8192, 82), (11008, 110), (28672, 287)):
        assert len(wl.outlier_channels(k, 1)) == n
