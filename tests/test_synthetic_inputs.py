"""The seeded input generator: bfloat16 rounding, determinism, moments."""
import numpy as np

import synthetic_inputs as si


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, 1.0 + 2 ** -7 + 2 ** -8, -2.5,
                  np.inf, -np.inf, 3.3895313892515355e38, 1e-45], dtype=np.float32)
    bits = si.f32_to_bf16_bits(x)
    # tie at 1 + 2^-8 goes to the even neighbour 1.0; 1 + 3*2^-9 rounds up to 1 + 2^-7;
    # tie at 1 + 2^-7 + 2^-8 goes to the even neighbour 1 + 2^-6
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F81, 0x3F82, 0xC020, 0x7F80, 0xFF80, 0x7F7F, 0x0000]
    assert si.f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))[0] == 0x7FC0


def test_bf16_roundtrip_of_representable_values():
    bits = np.arange(0, 0x7F80, 37, dtype=np.uint16)
    assert np.array_equal(si.f32_to_bf16_bits(si.bf16_bits_to_f32(bits)), bits)


def test_draw_is_deterministic_and_chunk_independent():
    a = si.normal_bf16((3, 1000, 7), 42, 1)
    b = si.normal_bf16((3, 1000, 7), 42, 1)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, si.normal_bf16((3, 1000, 7), 42, 2))
    big = si.normal_bf16((si.CHUNK + 1000,), 42, 1)
    small = si.normal_bf16((si.CHUNK,), 42, 1)
    assert np.array_equal(big[:si.CHUNK], small)


def test_moments_and_sigma():
    x = si.bf16_bits_to_f32(si.normal_bf16((1 << 20,), 1, 0)).astype(np.float64)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1.0) < 5e-3
    y = si.bf16_bits_to_f32(si.normal_bf16((1 << 20,), 1, 0, sigma=0.5)).astype(np.float64)
    assert np.array_equal(y, 0.5 * x)


def test_key_length_range_and_rows():
    L = [si.key_length(s) for s in range(200)]
    assert min(L) >= 64 and max(L) <= 512 and len(set(L)) > 50
    rows = si.sample_rows(75600, 4096, 1003, si.tile_edge_rows(75600))
    assert len(rows) >= 4096 and np.all(np.diff(rows) > 0) and rows[-1] == 75599 and rows[0] == 0
    assert si.sample_rows(100, 4096, 1).tolist() == list(range(100))
