"""Attention with q and k quantized to int8 per block — test infrastructure only
(see the package docstring).

Source: ComfyUI issue "MultiGPU Work Units". Its traceback of the WAN forward
pass runs SageAttention, whose first step quantizes q and k to int8 per block,
taking the softmax scale as an argument (``per_block_int8(q, k, sm_scale=...)``
returns int8 q, q scales, int8 k, k scales). The pages say nothing else about
the method; the reading implemented here (the plainest one) is:

  * symmetric quantization, one scale per block of consecutive tokens of one
    head (all d elements of each token): 128 query tokens, 64 key tokens;
  * q is multiplied by the softmax scale before it is quantized; k is not;
  * only valid keys (j < key length) belong to a key block;
  * the scores are s_ij = q_scale(i) * k_scale(j) * sum_c qcode[i, c] kcode[j, c],
    followed by the same exact softmax and weighted sum of v as ``attention_rows``.

A quantized code is an integer decided by floating point, so this file takes
each decision in float32, in the order the library takes it:

  x     = float32(bfloat16 value), times float32(softmax scale) for q
  amax  = max |x| over the block
  scale = float32(amax / 127)          (float32 division, round to nearest even)
          replaced by 1 when below 2^-100 (a block of zeros, or one so small that
          every code would be 0 anyway: then denormals, flushing and overflow of
          127 / amax cannot change any code)
  code  = clip(rint(x / scale), -127, 127)   (float32 division, ties to even)

Everything after the codes is float64. Parity of the quantizer is pinned by
hand-computed codes (including ties), a lossless closed form and an error bound
in tests/test_oracle_int8_pins.py.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import _split_inputs

Q_BLOCK = 128
K_BLOCK = 64
_TINY = np.float32(2.0 ** -100)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize_blocks(x: np.ndarray, block: int) -> tuple[np.ndarray, np.ndarray]:
    """Symmetric int8 codes of float32 rows x [n, d], one scale per ``block`` rows.

    Returns (codes int8 [n, d], scales float32 [ceil(n / block)]).
    """
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[0]
    nb = (n + block - 1) // block
    codes = np.empty(x.shape, dtype=np.int8)
    scales = np.empty(nb, dtype=np.float32)
    for b in range(nb):
        xb = x[b * block:(b + 1) * block]
        amax = np.float32(np.max(np.abs(xb))) if xb.size else np.float32(0.0)
        scale = np.float32(amax / np.float32(127.0))
        if not scale >= _TINY:
            scale = np.float32(1.0)
        q = np.rint(xb / scale)            # float32 / float32, then ties to even
        codes[b * block:(b + 1) * block] = np.clip(q, -127, 127).astype(np.int8)
        scales[b] = scale
    return codes, scales


def quantize_head(q_bits_h, k_bits_h, key_len: int, sm_scale: float):
    """Codes and scales of one head: q [Nq, d] (scaled by sm_scale), k [:key_len, d]."""
    qx = bf16_bits_to_f32(q_bits_h) * np.float32(sm_scale)
    kx = bf16_bits_to_f32(k_bits_h[:key_len])
    qc, qs = quantize_blocks(qx, Q_BLOCK)
    kc, ks = quantize_blocks(kx, K_BLOCK)
    return qc, qs, kc, ks


def dequantized_scores(qc, qs, kc, ks, rows) -> np.ndarray:
    """s [R, L] = q_scale * k_scale * (integer dot product), in float64."""
    rows = np.asarray(rows, dtype=np.int64)
    # every partial sum is an integer below 128 * 127^2 < 2^53, so this float64
    # product is the exact integer dot product whatever the summation order
    dot = qc[rows].astype(np.float64) @ kc.astype(np.float64).T
    qsc = qs[rows // Q_BLOCK].astype(np.float64)[:, None]
    ksc = ks[np.arange(kc.shape[0]) // K_BLOCK].astype(np.float64)[None, :]
    return qsc * ksc * dot


def mha_reference_qk_int8(q_bits, k_bits=None, v_bits=None, *, layout: str = "NHD",
                          head_begin: int = 0, head_count: int | None = None, rows=None,
                          key_len: int | None = None, scale: float | None = None) -> np.ndarray:
    """Float64 output [R, head_count, d] of attention on int8 per-block q and k.

    Arguments as for ``mha_reference`` (no RoPE). The softmax scale is folded into
    q before quantization, so the scores below carry it already.
    """
    qb, kb, vb = _split_inputs(q_bits, k_bits, v_bits, layout)
    Nq, Ht, d = qb.shape
    hc = Ht - head_begin if head_count is None else int(head_count)
    if not (0 <= head_begin and hc >= 1 and head_begin + hc <= Ht):
        raise ValueError("head range out of bounds")
    sm = np.float32(1.0 / math.sqrt(d) if scale is None else scale)
    rows = np.arange(Nq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    L = kb.shape[0] if key_len is None else int(key_len)
    if not 1 <= L <= kb.shape[0]:
        raise ValueError("key length must be in [1, Nk]")
    out = np.empty((rows.shape[0], hc, d), dtype=np.float64)
    for j, h in enumerate(range(head_begin, head_begin + hc)):
        qc, qs, kc, ks = quantize_head(qb[:, h, :], kb[:, h, :], L, sm)
        v = bf16_bits_to_f32(vb[:L, h, :]).astype(np.float64)
        for r0 in range(0, rows.shape[0], 256):
            s = dequantized_scores(qc, qs, kc, ks, rows[r0:r0 + 256])
            m = s.max(axis=1, keepdims=True)            # exact two-pass softmax
            e = np.exp(s - m)
            out[r0:r0 + 256, j, :] = (e @ v) / e.sum(axis=1, keepdims=True)
    return out
