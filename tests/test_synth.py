"""The seeded input generator: published splitmix64 output, C == numpy, moments."""
import numpy as np

from synth import gen, presets


def test_splitmix64_published_first_output():
    # splitmix64 seeded with state 0: first output is 0xE220A8397B1DCDAF.
    assert gen.mix64(0x9E3779B97F4A7C15) == 0xE220A8397B1DCDAF
    h = gen.hashes_np(0, 0, 0, 1)
    base = gen.stream_base(0, 0)
    assert int(h[0]) == gen.mix64(base + 0x9E3779B97F4A7C15)


def test_c_matches_numpy_bits():
    for (seed, tid, start, n, std, mean) in [(0, 17, 12345, 100000, 0.02, 0.0), (5, 2, 0, 70001, 0.1, 1.0),
                                              (0, 1296, 10 ** 9, 5000, 0.02, 0.0)]:
        a = gen.bf16_normal_np(seed, tid, start, n, std, mean)
        b = gen.bf16_normal(seed, tid, start, n, std, mean)
        assert np.array_equal(a, b)
    assert np.array_equal(gen.tokens_np(1002, 3, 0, 4096, 128256), gen.tokens(1002, 3, 0, 4096, 128256))


def test_moments_and_range():
    w = gen.bf16_bits_to_f32(gen.bf16_normal(0, 20, 0, 4_000_000)).astype(np.float64)
    assert abs(w.mean()) < 1e-4
    assert abs(w.std() / 0.02 - 1.0) < 0.01
    assert np.abs(w).max() <= 2 * np.sqrt(3) * 0.02 * 1.001


def test_tokens_uniform_range():
    t = gen.tokens(1, 3, 0, 200000, 1000)
    assert t.min() >= 0 and t.max() < 1000
    counts = np.bincount(t, minlength=1000)
    assert counts.min() > 100 and counts.max() < 320


def test_streams_are_distinct_and_deterministic():
    a = gen.bf16_normal(0, presets.layer_tid(0, "wq"), 0, 1000)
    b = gen.bf16_normal(0, presets.layer_tid(0, "wk"), 0, 1000)
    assert not np.array_equal(a, b)
    assert np.array_equal(a, gen.bf16_normal(0, presets.layer_tid(0, "wq"), 0, 1000))


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    assert list(gen.f32_to_bf16_bits(f)) == [0x3F80, 0x3F80, 0x3F82, 0x3F81]


def test_workload_prompts():
    wl = presets.WORKLOADS["llama8b"]
    p = gen.gen_prompt(wl)
    assert p.shape == (1, 39) and p.dtype == np.int32
    assert p.min() >= 0 and p.max() < 128256
