"""The seeded input generator (no GPU)."""
import numpy as np

from mixture_experts_layer_38_amd import datagen
from mixture_experts_layer_38_amd.configs import CONFIGS


def setup_module():
    datagen.build()


def test_splitmix64_reference_outputs():
    # First outputs of SplitMix64 started from state 0 (Vigna's reference code).
    got = datagen.splitmix64(0, 3)
    assert [int(v) for v in got] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_slices_regenerate_identically():
    full = datagen.normal(0, 3, (1001,), 0.5, "f32")
    part = datagen.normal(0, 3, (300,), 0.5, "f32", offset=401)
    assert np.array_equal(full[401:701], part)
    fb = datagen.normal(0, 3, (1001,), 0.5, "bf16")
    assert np.array_equal(fb, datagen.f32_to_bf16_bits(full))


def test_normal_moments():
    z = datagen.normal(7, 1, (1 << 20,), 1.0, "f32").astype(np.float64)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    assert abs((z ** 4).mean() - 3) < 0.05


def test_streams_differ_and_repeat():
    a = datagen.normal(0, 1, (64,), 1.0, "f32")
    b = datagen.normal(0, 2, (64,), 1.0, "f32")
    c = datagen.normal(1, 1, (64,), 1.0, "f32")
    assert not np.array_equal(a, b) and not np.array_equal(a, c)
    assert np.array_equal(a, datagen.normal(0, 1, (64,), 1.0, "f32"))


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.00390625, 1.005859375, 1.0078125, -2.5, 3.0e-3], np.float32)
    bits = datagen.f32_to_bf16_bits(vals)
    back = datagen.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-9 rounds up
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0078125 and back[3] == 1.0078125
    assert np.all(np.abs(back - vals) <= np.abs(vals) * 2.0 ** -8)


def test_logit_offsets():
    z = datagen.logit_offset(CONFIGS["mixtral_prefill"])
    p = np.exp(z.astype(np.float64))
    assert abs(p.sum() - 1) < 1e-6 and np.all(np.diff(z) < 0)
    np.testing.assert_allclose(p[0] / p[1], 2 ** 1.2, rtol=1e-5)
    u = datagen.logit_offset(CONFIGS["dsv3_routed"])
    assert u.shape == (256,) and u.min() >= -0.5 and u.max() < 0.5
    assert datagen.logit_offset(CONFIGS["mixtral_decode"]) is None
    assert CONFIGS["capacity_top2"].capacity == 512
