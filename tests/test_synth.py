"""The seeded input generator: published SplitMix64 outputs, counter-based
reproducibility, and the moments of the normal deviates."""
import numpy as np

import synth


def test_splitmix64_published_outputs():
    # First two outputs of SplitMix64 seeded with 0 (Steele, Lea, Flood 2014;
    # the reference implementation's state advances by 0x9E3779B97F4A7C15).
    assert synth.splitmix64(0) == 0xE220A8397B1DCDAF
    assert synth.splitmix64(0x9E3779B97F4A7C15) == 0x6E789E6AA1B965F4


def test_counter_based_offsets_and_threads():
    a = synth.normal_bf16(3, 2, (50_001,), threads=1)
    b = synth.normal_bf16(3, 2, (50_001,), threads=7)
    assert np.array_equal(a, b)
    for off in (0, 1, 2, 17, 4095):
        c = synth.normal_bf16(3, 2, (1001,), offset=off, threads=3)
        assert np.array_equal(a[off:off + 1001], c)
    assert not np.array_equal(a[:1000], synth.normal_bf16(3, 1, (1000,)))
    assert not np.array_equal(a[:1000], synth.normal_bf16(4, 2, (1000,)))


def test_normal_moments():
    z = synth.normal_f64(0, 0, (2_000_000,))
    assert abs(z.mean()) < 3e-3 and abs(z.std() - 1) < 3e-3
    assert abs((z ** 4).mean() - 3.0) < 3e-2
    b = synth.bf16_bits_to_f32(synth.normal_bf16(0, 0, (1000,), std=0.02)).astype(np.float64)
    assert np.allclose(b, synth.f32_to_bf16_bits(np.float32(0.02) * z[:1000].astype(np.float32))
                       .astype(np.uint32).__lshift__(16).view(np.float32), rtol=1e-2, atol=1e-4)
