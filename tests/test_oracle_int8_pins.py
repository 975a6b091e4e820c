"""Pins of the int8 per-block oracle (oracle/int8_qk.py) against things other
than itself: hand-computed codes with ties, degenerate blocks, the quantization
error bound, a lossless closed form that reduces to the exact oracle, and the
masking rule. Mutations planted on the CPU show that the pins catch them.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import int8_qk
import synthetic_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def golden():
    with open(os.path.join(ROOT, "tests", "golden", "int8_block_quantization.json")) as f:
        return json.load(f)["cases"]


def scale_of(expr):
    a, _, b = expr.partition("/")
    return np.float32(np.float32(float(a)) / np.float32(float(b))) if b else np.float32(float(a))


@pytest.mark.parametrize("case", golden(), ids=lambda c: c["name"])
def test_hand_computed_codes(case):
    x = np.array(case["x"], dtype=np.float32)
    codes, scales = oracle.quantize_blocks(x, 128)
    assert codes.tolist() == case["codes"]
    assert scales.shape == (1,) and scales[0] == scale_of(case["scale_expr"])


def _quantize_half_away(x, block):
    """Mutation: ties rounded away from zero."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.abs(x).max())
    s = np.float32(amax / np.float32(127.0)) or np.float32(1.0)
    return np.clip(np.sign(x) * np.floor(np.abs(x / s) + np.float32(0.5)), -127, 127).astype(np.int8)


def _quantize_by_128(x, block):
    """Mutation: 128 levels instead of 127."""
    x = np.asarray(x, dtype=np.float32)
    s = np.float32(np.float32(np.abs(x).max()) / np.float32(128.0)) or np.float32(1.0)
    return np.clip(np.rint(x / s), -127, 127).astype(np.int8)


@pytest.mark.parametrize("mutant", [_quantize_half_away, _quantize_by_128])
def test_mutated_quantizers_fail_the_hand_codes(mutant):
    bad = 0
    for case in golden():
        x = np.array(case["x"], dtype=np.float32)
        if mutant(x, 128).tolist() != case["codes"]:
            bad += 1
    assert bad >= 1


def test_tiny_block_codes_are_zero():
    for amax in (1e-35, 3e-39, 1e-44):
        x = np.array([[amax, -amax / 2]], dtype=np.float32)
        codes, scales = oracle.quantize_blocks(x, 64)
        assert scales[0] == 1.0 and not codes.any()


def test_error_bound_and_full_range():
    rng = np.random.default_rng(7)
    for sigma in (1.0, 1e-3, 300.0):
        x = (rng.standard_normal((300, 128)) * sigma).astype(np.float32)
        codes, scales = oracle.quantize_blocks(x, 64)
        for b in range(len(scales)):
            xb = x[b * 64:(b + 1) * 64].astype(np.float64)
            cb = codes[b * 64:(b + 1) * 64].astype(np.float64)
            s = float(scales[b])
            assert np.abs(cb).max() == 127                      # the block maximum maps to +-127
            # |dequantized - x| <= half a step, up to float32 rounding of x / s
            assert np.all(np.abs(cb * s - xb) <= 0.5 * s * (1 + 1e-6) + np.abs(xb) * 2.0 ** -23)
        assert len(scales) == 5                                  # ragged last block of 44 rows


def _grid_values(shape, seed, step):
    """bf16 bit patterns of integer codes in [-127, 127] times ``step`` (a power of 2),
    every block of 64 rows holding a +-127."""
    rng = np.random.default_rng(seed)
    c = rng.integers(-126, 127, size=shape).astype(np.float32)
    c[::64, ..., 0] = 127.0
    x = (c * np.float32(step)).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16), c


def test_lossless_blocks_reduce_to_the_exact_oracle():
    # q * 0.125 and k are exact multiples of their block scale: quantization is
    # lossless and the int8 attention equals plain attention with scale 0.125
    n, nk, ht, d, L = 300, 200, 2, 64, 150
    q_bits, _ = _grid_values((n, ht, d), 1, 2.0 ** -4)
    k_bits, _ = _grid_values((nk, ht, d), 2, 2.0 ** -5)
    v_bits = si.normal_bf16((nk, ht, d), 3, si.STREAM_V)
    rows = np.array([0, 1, 127, 128, 200, 299])
    got = oracle.mha_reference_qk_int8(q_bits, k_bits, v_bits, rows=rows, key_len=L, scale=0.125)
    ref = oracle.mha_reference(q_bits, k_bits, v_bits, rows=rows, key_len=L, scale=0.125)
    assert np.abs(got - ref).max() < 1e-12


def test_unscaled_q_mutation_breaks_the_closed_form():
    n, nk, ht, d = 130, 100, 1, 64
    q_bits, _ = _grid_values((n, ht, d), 4, 2.0 ** -4)
    k_bits, _ = _grid_values((nk, ht, d), 5, 2.0 ** -5)
    v_bits = si.normal_bf16((nk, ht, d), 6, si.STREAM_V)
    ref = oracle.mha_reference(q_bits, k_bits, v_bits, scale=0.125)
    # quantizing q without the softmax scale is the same as using scale 1
    mutant = oracle.mha_reference_qk_int8(q_bits, k_bits, v_bits, scale=1.0)
    assert np.abs(mutant - ref).max() > 1e-3


def test_masked_keys_change_nothing():
    n, nk, ht, d, L = 200, 192, 2, 128, 100
    q = si.normal_bf16((n, ht, d), 11, si.STREAM_Q)
    k = si.normal_bf16((nk, ht, d), 11, si.STREAM_K)
    v = si.normal_bf16((nk, ht, d), 11, si.STREAM_V)
    a = oracle.mha_reference_qk_int8(q, k, v, key_len=L)
    k2, v2 = k.copy(), v.copy()
    k2[L:] = 0x4700        # bf16 32768: would dominate the block scale if it were counted
    v2[L:] = 0x4700
    b = oracle.mha_reference_qk_int8(q, k2, v2, key_len=L)
    assert np.array_equal(a, b)


def test_quantization_error_is_small_against_exact_attention():
    # the int8 result stays close to exact attention (order 1e-2 relative at d = 128)
    n, ht, d = 256, 2, 128
    q = si.normal_bf16((n, ht, d), 21, si.STREAM_Q)
    k = si.normal_bf16((n, ht, d), 21, si.STREAM_K)
    v = si.normal_bf16((n, ht, d), 21, si.STREAM_V)
    a = oracle.mha_reference_qk_int8(q, k, v)
    b = oracle.mha_reference(q, k, v)
    rel = np.abs(a - b).sum() / np.abs(b).sum()
    assert 1e-4 < rel < 5e-2
