"""Pins for the float64 oracle, independent of the oracle's own code.

Each pin is a brute-force loop, a library routine, a closed form, an invariant or
a value the pages state. The ``*_pins`` helpers return the list of failed checks
for a given implementation so that the mutation tests at the bottom can show
that plausible mistakes planted in a copy of the oracle are caught.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oa
import synthetic_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# Brute force: pure-Python loops over Python floats, no numpy arithmetic.
# ---------------------------------------------------------------------------

def brute_attention(q, k, v, scale, key_len):
    out = []
    for qi in q:
        s = []
        for j in range(key_len):
            acc = 0.0
            for c in range(len(qi)):
                acc += float(qi[c]) * float(k[j][c])
            s.append(scale * acc)
        m = max(s)
        w = [math.exp(x - m) for x in s]
        l = sum(w)
        row = []
        for c in range(len(v[0])):
            acc = 0.0
            for j in range(key_len):
                acc += w[j] * float(v[j][c])
            row.append(acc / l)
        out.append(row)
    return np.array(out)


def brute_rope_1d(vec, pos, base):
    """Textbook 1-D rotary embedding via complex multiplication, pairs (2i, 2i+1)."""
    D = len(vec)
    out = []
    for i in range(D // 2):
        z = complex(vec[2 * i], vec[2 * i + 1]) * complex(math.cos(pos * base ** (-2 * i / D)),
                                                          math.sin(pos * base ** (-2 * i / D)))
        out += [z.real, z.imag]
    return out


# ---------------------------------------------------------------------------
# Pin collections, parametrised by the implementation under test.
# ---------------------------------------------------------------------------

def attention_pins(attn_rows):
    """Checks of a single-head attention function attn_rows(q, k, v, scale, key_len)."""
    fails = []
    rng = np.random.default_rng(7)
    # brute force on tiny inputs, several lengths and masks
    for n, d, L in [(1, 4, 1), (2, 4, 2), (3, 8, 2), (5, 4, 5), (17, 8, 9), (8, 3, 8)]:
        q = rng.standard_normal((n, d)); k = rng.standard_normal((n, d)); v = rng.standard_normal((n, d))
        got = attn_rows(q, k, v, 0.37, L)
        ref = brute_attention(q.tolist(), k.tolist(), v.tolist(), 0.37, L)
        if not np.allclose(got, ref, rtol=1e-12, atol=1e-13):
            fails.append(f"brute force n={n} d={d} L={L}")
    # torch CPU float64 scaled_dot_product_attention with a boolean key mask
    for n, d, L in [(64, 64, 64), (300, 128, 177), (1024, 128, 1000)]:
        q = rng.standard_normal((n, d)); k = rng.standard_normal((n, d)); v = rng.standard_normal((n, d))
        mask = torch.zeros((n, n), dtype=torch.bool)
        mask[:, :L] = True
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
            attn_mask=mask[None], is_causal=False, scale=1.0 / math.sqrt(d))[0].numpy()
        got = attn_rows(q, k, v, 1.0 / math.sqrt(d), L)
        if not np.allclose(got, ref, rtol=1e-10, atol=1e-12):
            fails.append(f"torch sdpa n={n} d={d} L={L}")
    # closed forms
    q = rng.standard_normal((6, 16)); k = rng.standard_normal((40, 16)); v = rng.standard_normal((40, 16))
    if not np.allclose(attn_rows(q, k, v, 0.25, 1), np.repeat(v[:1], 6, 0), rtol=0, atol=1e-15):
        fails.append("key_len=1 returns v0")
    if not np.allclose(attn_rows(np.zeros_like(q), k, v, 0.25, 23), np.repeat(v[:23].mean(0, keepdims=True), 6, 0),
                       rtol=1e-13, atol=1e-14):
        fails.append("q=0 gives the mean of the valid values")
    vc = np.tile(rng.standard_normal((1, 16)), (40, 1))
    if not np.allclose(attn_rows(q, k, vc, 0.25, 40), np.repeat(vc[:1], 6, 0), rtol=1e-13, atol=1e-14):
        fails.append("constant V gives a constant output")
    # invariants: joint permutation of keys and values; masked keys have no effect
    perm = rng.permutation(40)
    if not np.allclose(attn_rows(q, k[perm], v[perm], 0.25, 40), attn_rows(q, k, v, 0.25, 40), rtol=1e-12, atol=1e-14):
        fails.append("joint key/value permutation")
    k2 = k.copy(); v2 = v.copy()
    k2[30:] = np.nan; v2[30:] = 1e300
    got = attn_rows(q, k2, v2, 0.25, 30)
    if not (np.all(np.isfinite(got)) and np.array_equal(got, attn_rows(q, k, v, 0.25, 30))):
        fails.append("masked keys have no effect")
    # hand-worked example (tests/golden/attention_hand_example.json)
    with open(os.path.join(GOLDEN, "attention_hand_example.json")) as f:
        g = json.load(f)
    qg = np.array(g["q"]); vg = np.array(g["v"])
    kg = np.array([[math.log(j + 1), 0.0] for j in range(3)])
    for case in g["cases"]:
        got = attn_rows(qg, kg, vg, case["scale"], case["key_len"])[0]
        if not np.allclose(got, case["out"], rtol=1e-14, atol=1e-14):
            fails.append(f"hand example scale={case['scale']} L={case['key_len']}")
    return fails


def rope_pins(rope_apply):
    """Checks of a 3D RoPE function rope_apply(u [R, d], tokens, grid, dims, base)."""
    fails = []
    rng = np.random.default_rng(11)
    dims = (44, 42, 42)
    grid = (3, 5, 7)
    tokens = np.arange(105)
    u = rng.standard_normal((105, 128))
    r = rope_apply(u, tokens, grid, dims, 10000.0)
    if not np.array_equal(r[0], u[0]):
        fails.append("position 0 is the identity")
    if not np.allclose(r[:, 0::2] ** 2 + r[:, 1::2] ** 2, u[:, 0::2] ** 2 + u[:, 1::2] ** 2, rtol=1e-13, atol=0):
        fails.append("pair norms are preserved")
    # a 1x1xW grid is textbook 1-D RoPE on the w band, identity elsewhere
    W = 9
    u1 = rng.standard_normal((W, 128))
    r1 = rope_apply(u1, np.arange(W), (1, 1, W), dims, 10000.0)
    for x in range(W):
        want = list(u1[x, :86]) + brute_rope_1d(list(u1[x, 86:]), x, 10000.0)
        if not np.allclose(r1[x], want, rtol=1e-13, atol=1e-14):
            fails.append(f"1x1xW grid, token {x}")
            break
    # a Tx1x1 grid is 1-D RoPE on the t band
    u2 = rng.standard_normal((4, 128))
    r2 = rope_apply(u2, np.arange(4), (4, 1, 1), dims, 10000.0)
    for t in range(4):
        want = brute_rope_1d(list(u2[t, :44]), t, 10000.0) + list(u2[t, 44:])
        if not np.allclose(r2[t], want, rtol=1e-13, atol=1e-14):
            fails.append(f"Tx1x1 grid, token {t}")
            break
    # relative position: <R(p) a, R(p') b> depends on p - p' only (check on the h band)
    a = rng.standard_normal((1, 128)); b = rng.standard_normal((1, 128))
    g = (1, 12, 1)
    dots = []
    for p, pp in [(3, 1), (7, 5), (11, 9)]:
        ra = rope_apply(a, [p], g, dims, 10000.0)[0]
        rb = rope_apply(b, [pp], g, dims, 10000.0)[0]
        dots.append(float(ra @ rb))
    if not np.allclose(dots, dots[0], rtol=1e-12, atol=1e-12):
        fails.append("relative position property")
    # closed-form worked example: grid 2x3x4, token 23 = (t, y, x) = (1, 2, 3); d = 8, bands (4, 2, 2)
    e = np.array([[1.0, 0.0] * 4])
    got = rope_apply(e, [23], (2, 3, 4), (4, 2, 2), 10000.0)[0]
    want = [math.cos(1.0), math.sin(1.0), math.cos(0.01), math.sin(0.01),
            math.cos(2.0), math.sin(2.0), math.cos(3.0), math.sin(3.0)]
    if not np.allclose(got, want, rtol=1e-14, atol=1e-15):
        fails.append("worked example token 23")
    # a pure second component rotates the other way round: (0, 1) -> (-sin, cos)
    e2 = np.array([[0.0, 1.0] * 4])
    got2 = rope_apply(e2, [23], (2, 3, 4), (4, 2, 2), 10000.0)[0]
    want2 = [-math.sin(1.0), math.cos(1.0), -math.sin(0.01), math.cos(0.01),
             -math.sin(2.0), math.cos(2.0), -math.sin(3.0), math.cos(3.0)]
    if not np.allclose(got2, want2, rtol=1e-14, atol=1e-15):
        fails.append("worked example token 23, second component")
    return fails


# ---------------------------------------------------------------------------
# The oracle passes every pin.
# ---------------------------------------------------------------------------

def test_attention_pins():
    assert attention_pins(oa.attention_rows) == []


def test_attention_rejects_empty_key_set():
    q = np.zeros((1, 4)); k = np.zeros((3, 4))
    with pytest.raises(ValueError):
        oracle.attention_rows(q, k, k, 1.0, 0)
    with pytest.raises(ValueError):
        oracle.attention_rows(q, k, k, 1.0, 4)


def test_rope_pins():
    assert rope_pins(oa.rope_apply) == []


def test_rope_index_table_hand_values():
    # grid (T, H, W) = (2, 3, 4), w fastest: token n -> (n // 12, (n // 4) % 3, n % 4)
    tab = oracle.rope_index_table([0, 5, 12, 23], (2, 3, 4), 8, (4, 2, 2))
    assert tab.shape == (4, 4, 5)
    assert tab[:, 0, :3].tolist() == [[0, 0, 0], [0, 1, 1], [1, 0, 0], [1, 2, 3]]
    # pairs -> (band, i): t band holds pairs 0, 1; h band pair 2; w band pair 3
    assert tab[0, :, 3:].tolist() == [[0, 0], [0, 1], [1, 0], [2, 0]]
    full = oracle.rope_index_table(np.arange(21 * 45 * 80), (21, 45, 80), 128, (44, 42, 42))
    assert full[-1, 0, :3].tolist() == [20, 44, 79]
    assert full[80, 0, :3].tolist() == [0, 1, 0]
    assert full[45 * 80, 0, :3].tolist() == [1, 0, 0]
    assert [int(x) for x in np.bincount(full[0, :, 3])] == [22, 21, 21]


def test_rope_rejects_bad_bands():
    with pytest.raises(ValueError):
        oracle.rope_pair_bands(128, (43, 43, 42))
    with pytest.raises(ValueError):
        oracle.rope_pair_bands(128, (44, 42, 40))


def test_ulysses_golden():
    with open(os.path.join(GOLDEN, "ulysses_head_shares.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        if c["valid"]:
            shares = [oracle.ulysses_head_range(c["heads_total"], c["degree"], r) for r in range(c["degree"])]
            assert all(cnt == c["heads_per_rank"] for _, cnt in shares)
            assert [b for b, _ in shares] == [r * c["heads_per_rank"] for r in range(c["degree"])]
        else:
            with pytest.raises(ValueError):
                oracle.ulysses_head_range(c["heads_total"], c["degree"], 0)


def _bits(shape, seed, stream, sigma=1.0):
    return si.normal_bf16(shape, seed, stream, sigma)


def test_mha_head_range_is_a_slice_of_all_heads():
    q = _bits((96, 8, 32), 5, 0); k = _bits((96, 8, 32), 5, 1); v = _bits((96, 8, 32), 5, 2)
    full = oracle.mha_reference(q, k, v)
    part = oracle.mha_reference(q, k, v, head_begin=2, head_count=4)
    assert np.array_equal(part, full[:, 2:6])
    rows = np.array([0, 17, 95])
    assert np.array_equal(oracle.mha_reference(q, k, v, rows=rows), full[rows])


def test_mha_packed_equals_separate():
    qkv = _bits((80, 3, 4, 64), 9, 0, 0.5)
    rope = {"grid": (5, 4, 4), "dims": (24, 20, 20), "base": 10000.0}
    a = oracle.mha_reference(qkv, layout="N3HD", rope=rope)
    b = oracle.mha_reference(qkv[:, 0].copy(), qkv[:, 1].copy(), qkv[:, 2].copy(), rope=rope)
    assert np.array_equal(a, b)


def test_mha_matches_torch_sdpa_multihead_with_mask():
    q = _bits((200, 6, 64), 4, 0); k = _bits((120, 6, 64), 4, 1); v = _bits((120, 6, 64), 4, 2)
    got = oracle.mha_reference(q, k, v, head_begin=1, head_count=4, key_len=77)
    qt = torch.from_numpy(oa.bf16_bits_to_f64(q)).permute(1, 0, 2)[1:5]
    kt = torch.from_numpy(oa.bf16_bits_to_f64(k)).permute(1, 0, 2)[1:5]
    vt = torch.from_numpy(oa.bf16_bits_to_f64(v)).permute(1, 0, 2)[1:5]
    mask = torch.zeros((200, 120), dtype=torch.bool); mask[:, :77] = True
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask).permute(1, 0, 2).numpy()
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_bf16_widening_is_exact():
    bits = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x4049, 0x7F7F, 0x0001], dtype=np.uint16)
    want = [0.0, -0.0, 1.0, -1.0, 3.140625, 3.3895313892515355e38, 9.183549615799121e-41]
    assert oracle.bf16_bits_to_f64(bits).tolist() == want


# ---------------------------------------------------------------------------
# Mutation tests: plausible mistakes planted in copies of the oracle must fail a pin.
# ---------------------------------------------------------------------------

def _attn_no_max(q, k, v, scale, L):
    s = (q @ k[:L].T) * scale
    e = np.exp(s)                                   # fine mathematically, kept as a control
    return (e @ v[:L]) / e.sum(1, keepdims=True)


def _attn_dropped_scale(q, k, v, scale, L):
    return oa.attention_rows(q, k, v, 1.0, L)


def _attn_wrong_value_operand(q, k, v, scale, L):
    return oa.attention_rows(q, k, k, scale, L)


def _attn_mask_off_by_one(q, k, v, scale, L):
    return oa.attention_rows(q, k, v, scale, min(L + 1, k.shape[0]))


def _attn_normalise_by_max(q, k, v, scale, L):
    s = (q @ k[:L].T) * scale
    e = np.exp(s - s.max(1, keepdims=True))
    return (e @ v[:L]) / e.max(1, keepdims=True)


def _attn_transposed_scores(q, k, v, scale, L):
    s = (k[:L] @ q.T).T * scale if q.shape[0] == L else (q @ k[:L].T) * scale
    s = s.T if s.shape[0] == s.shape[1] else s
    e = np.exp(s - s.max(1, keepdims=True))
    return (e @ v[:L]) / e.sum(1, keepdims=True)


def test_attention_pins_accept_equivalent_form():
    # dropping the max subtraction is exact in real arithmetic: a control that must pass
    assert attention_pins(_attn_no_max) == []


@pytest.mark.parametrize("mutant", [_attn_dropped_scale, _attn_wrong_value_operand, _attn_mask_off_by_one,
                                    _attn_normalise_by_max, _attn_transposed_scores])
def test_attention_pins_catch_mutants(mutant):
    assert attention_pins(mutant) != []


def _rope_mutant(kind):
    def f(u, tokens, grid, dims, base):
        u = np.asarray(u, dtype=np.float64)
        pos = oa.rope_grid_position(tokens, grid).astype(np.float64)
        if kind == "hw_swapped":
            pos = pos[:, [0, 2, 1]]
        out = u.copy()
        off = 0
        for band, width in enumerate(dims):
            i = np.arange(width // 2)
            expo = (-2.0 * i / width) if kind != "half_width" else (-2.0 * i / (width // 2))
            theta = pos[:, band][:, None] * float(base) ** expo[None, :]
            c, s = np.cos(theta), np.sin(theta)
            if kind == "sign":
                s = -s
            if kind == "rotate_half":
                a = u[:, off:off + width // 2]; b = u[:, off + width // 2:off + width]
                out[:, off:off + width // 2] = a * c - b * s
                out[:, off + width // 2:off + width] = a * s + b * c
            else:
                a = u[:, off:off + width:2]; b = u[:, off + 1:off + width:2]
                out[:, off:off + width:2] = a * c - b * s
                out[:, off + 1:off + width:2] = a * s + b * c
            off += width
        return out
    return f


@pytest.mark.parametrize("kind", ["sign", "hw_swapped", "half_width", "rotate_half"])
def test_rope_pins_catch_mutants(kind):
    assert rope_pins(_rope_mutant(kind)) != []


def test_rope_mutant_control_passes():
    assert rope_pins(_rope_mutant("none")) == []
