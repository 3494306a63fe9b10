"""The seeded generators are deterministic and draw the stated distributions (CPU only)."""
import numpy as np

import synth


def test_generators_are_deterministic():
    a = synth.small_linear(3, 64, 256, 4, 1e-4)
    b = synth.small_linear(3, 64, 256, 4, 1e-4)
    assert all(synth.sha256(u) == synth.sha256(v) for u, v in zip(a, b))


def test_distributions():
    rng = np.random.default_rng(0)
    q = synth.draw_codes(rng, 256, 4096)
    assert q.min() == -127 and q.max() == 127
    s = synth.draw_scales(rng, 256, 4096, 1e-4).view(np.float16).astype(np.float64)
    assert s.shape == (256, 128) and s.min() >= 1e-4 * 0.999 and abs(s.mean() - 0.016) < 0.001
    x = synth.bf16_bits_to_f32(synth.draw_acts(rng, 64, 4096))
    assert abs(float(x.mean())) < 0.01 and abs(float(x.std()) - 1.0) < 0.01


def test_bf16_packing_is_round_to_nearest_even():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.0 ** -130], dtype=np.float32)
    b = synth.f32_to_bf16_bits(v)
    assert list(b) == [0x3F80, 0x3F80, 0x3F82, 0x8000 | 0x0008]  # 2^-130 = 8 * 2^-133
