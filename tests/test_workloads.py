"""The seeded input generator: rounding to the 16-bit element types and
thread-count independence of the draws (CPU only)."""

import numpy as np

from segmented_varlen_attention_amd import workloads as W


def test_round_to_bf16_ties_to_even():
    u = 2.0 ** -7  # spacing of bf16 values in [1, 2)
    x = np.array([1.0, 1 + u / 2, 1 + 3 * u / 2, 1 + u / 2 + 2 ** -20, -(1 + u / 2), 3.0e38],
                 np.float32)
    r = W.round_to_bf16(x)
    assert r[0] == 1.0
    assert r[1] == 1.0                      # tie -> even significand
    assert r[2] == np.float32(1 + 2 * u)    # tie -> even significand
    assert r[3] == np.float32(1 + u)        # above the midpoint
    assert r[4] == -1.0
    assert np.isfinite(r[5]) or np.isinf(r[5])
    assert np.isnan(W.round_to_bf16(np.array([np.nan], np.float32)))[0]


def test_round_to_fp16_ties_overflow_subnormals():
    u = 2.0 ** -10  # spacing of fp16 values in [1, 2)
    x = np.array([1 + u / 2, 1 + 3 * u / 2, 65504.0, 65519.0, 65520.0,
                  2.0 ** -25, 3 * 2.0 ** -25], np.float32)
    r = W.round_to_fp16(x)
    assert r[0] == 1.0
    assert r[1] == np.float32(1 + 2 * u)
    assert r[2] == 65504.0 and r[3] == 65504.0
    assert np.isinf(r[4])                   # halfway to 2^16 rounds to infinity
    assert r[5] == 0.0                      # tie between 0 and 2^-24 -> 0
    assert r[6] == np.float32(2.0 ** -23)   # tie between 2^-24 and 2^-23 -> 2^-23


def test_round_to_dispatch_and_exactness():
    x = np.random.default_rng(3).standard_normal(4096, dtype=np.float32)
    for dt, fn in ((W.BF16, W.round_to_bf16), (W.FP16, W.round_to_fp16)):
        r = W.round_to(dt, x)
        assert np.array_equal(r, fn(x))
        assert np.array_equal(W.round_to(dt, r), r)  # idempotent
    assert np.array_equal(W.round_to(W.FP32, x), x)


def test_normal_tensor_thread_independent():
    shape = (3 * W.CHUNK // 1024 + 5, 1024)
    for dt in (W.FP32, W.BF16, W.FP16):
        a = W.normal_tensor(11, 2, shape, 1.0, dt, threads=1)
        b = W.normal_tensor(11, 2, shape, 1.0, dt, threads=4)
        assert np.array_equal(a, b)
        assert np.array_equal(W.round_to(dt, a), a)
