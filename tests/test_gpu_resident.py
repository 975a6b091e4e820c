"""GPU: attention with the keys resident in LDS (short key sequences).

A call whose key lengths all fit the LDS array (256 keys at d = 128, 512 at
d = 64) and that has at least one 256-query tile per compute unit runs the
kernel that stages K and V^T once per head and streams query tiles against
them (256 CUs here: the shapes below have 300-400 tiles). A single-head call on
the same data has fewer tiles than CUs and runs the streaming kernel. Per row
the two do the same arithmetic, so the rows must agree bit for bit; both are
checked against the float64 oracle as well. The exact-maximum retry is decided
per wave in the resident kernel and per workgroup in the streaming one, so a
case that takes it is checked against the oracle only.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from test_gpu_batch import entries, stack
from test_gpu_parity import as_f64, check, down, nhd_inputs, note, run_nhd, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this environment")
    import long_sequence_attention_amd as vd
    vd.load_library()
    return torch.device("cuda:0")


def vdm():
    import long_sequence_attention_amd as vd
    return vd


CASES = [(128, 12000, 256, L) for L in (1, 2, 63, 64, 65, 129, 200, 255, 256)] + \
        [(64, 20000, 512, L) for L in (1, 64, 300, 511, 512)]


@pytest.mark.parametrize("d,nq,nk,L", CASES)
def test_resident_rows_match_oracle_and_streaming_kernel(dev, d, nq, nk, L):
    ht = 8 if d == 128 else 4
    seed = 7000 + d + L
    note(f"resident cross-attention nq={nq} nk={nk} L={L} Ht={ht} d={d} seed {seed}")
    q, k, v = nhd_inputs(nq, nk, ht, d, seed)
    out = run_nhd(dev, q, k, v, key_len=L)
    rows = si.sample_rows(nq, 384, seed, si.tile_edge_rows(nq))
    got = as_f64(out[torch.from_numpy(rows).to(dev)])
    check(got, oracle.mha_reference(q, k, v, rows=rows, key_len=L), f"resident d={d} L={L}")
    for h in (0, ht - 1):
        single = run_nhd(dev, q, k, v, head_begin=h, head_count=1, key_len=L)
        assert np.array_equal(down(single[:, 0]), down(out[:, h])), f"head {h}: resident and streaming rows differ"


def test_resident_self_attention_short_sequence(dev):
    # self-attention over 250 tokens with many heads: keys fit, query tiles fill the CUs
    n, ht, d = 250, 300, 64
    note(f"resident self-attention n={n} Ht={ht} d={d}")
    q, k, v = nhd_inputs(n, n, ht, d, 7400)
    out = run_nhd(dev, q, k, v)
    heads = [0, 1, 150, 299]
    check(as_f64(out[:, heads]), oracle.mha_reference(q, k, v)[:, heads], "resident self-attention")
    single = run_nhd(dev, q, k, v, head_begin=150, head_count=1)
    assert np.array_equal(down(single[:, 0]), down(out[:, 150]))


def test_resident_batch_entries_with_their_own_key_lengths(dev):
    # entries of different key lengths: each workgroup restages K/V^T (and the tile
    # count) when its range of query tiles crosses into the next (entry, head)
    vd = vdm()
    B, nq, nk, ht, d = 2, 12000, 256, 8, 128
    lens = [256, 37]
    note(f"resident batch cross-attention B={B} nq={nq} key_lens={lens}")
    es = entries(B, nq, nk, ht, d, 7500)
    attn = vd.Attention(nq, nk, ht, d, use_key_mask=True, batch=B)
    out = attn.forward(*(stack(dev, [e[j] for e in es]) for j in range(3)), key_lens=lens)
    torch.cuda.synchronize()
    for i, ((q, k, v), L) in enumerate(zip(es, lens)):
        single = vd.Attention(nq, nk, ht, d, use_key_mask=True).forward(up(q, dev), up(k, dev), up(v, dev),
                                                                        key_len=L)
        torch.cuda.synchronize()
        assert np.array_equal(down(out[i]), down(single)), f"entry {i} (key_len {L}) differs from its single call"
        rows = si.sample_rows(nq, 256, 7500 + i, si.tile_edge_rows(nq))
        got = as_f64(out[i][torch.from_numpy(rows).to(dev)])
        check(got, oracle.mha_reference(q, k, v, rows=rows, key_len=L), f"resident batch entry {i} L={L}")


def test_resident_masked_keys_have_no_effect(dev):
    nq, nk, ht, d, L = 12000, 256, 8, 128, 150
    q, k, v = nhd_inputs(nq, nk, ht, d, 7600)
    base = run_nhd(dev, q, k, v, key_len=L)
    k2, v2 = k.copy(), v.copy()
    v2[L:] = 0x7FC0  # NaN
    k2[L:] = 0x7F80  # +inf
    other = run_nhd(dev, q, k2, v2, key_len=L)
    assert torch.equal(base.view(torch.int16), other.view(torch.int16))


@pytest.mark.parametrize("L", [None, 230])
def test_resident_scores_growing_past_first_tile_max(dev, L):
    # key j has k[j, 0] ~ j / 8 and queries q[:, 0] = 8: the scores of the last key
    # tiles exceed the first tile's maximum by far more than the float16 range, so
    # the waves of those rows recompute with the exact maximum; every seventh row
    # of head 1 stays tame
    nq, nk, ht, d = 12000, 256, 8, 128
    q, k, v = nhd_inputs(nq, nk, ht, d, 7700, 0.25)
    q[:, :, 0] = si.f32_to_bf16_bits(np.full((nq, ht), 8.0, dtype=np.float32))
    ramp = (np.arange(nk, dtype=np.float32) / 8.0)[:, None]
    k[:, :, 0] = si.f32_to_bf16_bits(np.broadcast_to(ramp, (nk, ht)))
    q[::7, 1, 0] = si.f32_to_bf16_bits(np.zeros(len(range(0, nq, 7)), dtype=np.float32))
    out = run_nhd(dev, q, k, v, key_len=L)
    rows = si.sample_rows(nq, 256, 7700, si.tile_edge_rows(nq))
    got = as_f64(out[torch.from_numpy(rows).to(dev)])
    check(got, oracle.mha_reference(q, k, v, rows=rows, key_len=L), f"resident growing scores L={L}")
