"""GPU: q.k on int8 per-block codes (descriptor qk_int8).

The codes and scales that the quantize pre-pass writes into the workspace must
equal the oracle's bit for bit (integer work decided in float32 on both sides);
the attention output must match the int8 oracle (oracle/int8_qk.py) to the same
tolerances as the bfloat16 path, on both kernel configurations (key lengths up
to 1024 and beyond), with masks, ragged tiles, batches and a block of zero queries.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import int8_qk
import synthetic_inputs as si
from test_gpu_parity import as_f64, check, note, up, workspace_layout

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


def ws_regions(B, hc, nq, nk, d=128):
    """Byte offsets of the int8 regions, as the header lays the workspace out."""
    return workspace_layout(B, hc, nq, nk, d, int8=True)


def test_codes_and_scales_are_bit_exact(dev):
    vd = vdm()
    B, nq, nk, ht, h0, hc, d = 2, 300, 200, 3, 1, 2, 128
    lens = [150, 200]
    note(f"int8 codes B={B} nq={nq} nk={nk} heads {h0}-{h0 + hc - 1} key_lens={lens}")
    es = [(si.normal_bf16((nq, ht, d), 5100 + i, si.STREAM_Q, 2.0), si.normal_bf16((nk, ht, d), 5100 + i, si.STREAM_K),
           si.normal_bf16((nk, ht, d), 5100 + i, si.STREAM_V)) for i in range(B)]
    attn = vd.Attention(nq, nk, ht, d, head_begin=h0, head_count=hc, use_key_mask=True, batch=B, qk_int8=True)
    r = ws_regions(B, hc, nq, nk)
    assert attn.workspace_bytes == r["end"]
    qb, kb, vb = (up(np.stack([e[j] for e in es]), dev) for j in range(3))
    ws = attn.prepare(qb, kb, vb, key_lens=lens)
    torch.cuda.synchronize()
    w = ws.cpu().numpy()
    sm = np.float32(1.0 / np.sqrt(d))
    for b in range(B):
        for j, h in enumerate(range(h0, h0 + hc)):
            sl = b * hc + j
            qc, qs, kc, ks = int8_qk.quantize_head(es[b][0][:, h, :], es[b][1][:, h, :], lens[b], sm)
            gq = w[r["qc"] + sl * r["nq_pad"] * d:][:nq * d].view(np.int8).reshape(nq, d)
            gk = w[r["kc"] + sl * r["nk_pad"] * d:][:lens[b] * d].view(np.int8).reshape(lens[b], d)
            gqs = w[r["qs"] + sl * (r["nq_pad"] // 128) * 4:][:len(qs) * 4].view(np.float32)
            gks = w[r["ks"] + sl * (r["nk_pad"] // 64) * 4:][:len(ks) * 4].view(np.float32)
            assert np.array_equal(gq, qc), f"q codes entry {b} head {h}"
            assert np.array_equal(gk, kc), f"k codes entry {b} head {h}"
            assert np.array_equal(gqs.view(np.uint32), qs.view(np.uint32)), f"q scales entry {b} head {h}"
            assert np.array_equal(gks.view(np.uint32), ks.view(np.uint32)), f"k scales entry {b} head {h}"


@pytest.mark.parametrize("n,ht,h0,hc", [(1000, 4, 1, 2), (2300, 2, 0, 2)])
def test_self_attention_matches_int8_oracle(dev, n, ht, h0, hc):
    vd = vdm()
    note(f"int8 self-attention n={n} Ht={ht} heads {h0}-{h0 + hc - 1} ({'short' if n <= 1024 else 'long'} keys)")
    q = si.normal_bf16((n, ht, 128), 5200 + n, si.STREAM_Q)
    k = si.normal_bf16((n, ht, 128), 5200 + n, si.STREAM_K)
    v = si.normal_bf16((n, ht, 128), 5200 + n, si.STREAM_V)
    out = vd.Attention(n, n, ht, 128, head_begin=h0, head_count=hc, qk_int8=True).forward(up(q, dev), up(k, dev),
                                                                                         up(v, dev))
    torch.cuda.synchronize()
    got = as_f64(out)
    check(got, oracle.mha_reference_qk_int8(q, k, v, head_begin=h0, head_count=hc), f"int8 n={n}")
    exact = oracle.mha_reference(q, k, v, head_begin=h0, head_count=hc)
    note(f"  against exact attention: relL1={np.abs(got - exact).sum() / np.abs(exact).sum():.3e}")


@pytest.mark.parametrize("key_len", [77, 512])
def test_cross_attention_masked_matches_int8_oracle(dev, key_len):
    vd = vdm()
    nq, nk, ht = 600, 512, 4
    note(f"int8 cross-attention nq={nq} nk={nk} key_len={key_len}")
    q = si.normal_bf16((nq, ht, 128), 5300, si.STREAM_Q)
    k = si.normal_bf16((nk, ht, 128), 5300, si.STREAM_K)
    v = si.normal_bf16((nk, ht, 128), 5300, si.STREAM_V)
    k2, v2 = k.copy(), v.copy()
    k2[key_len:] = 0x7FC0   # NaN past the valid keys: never read, never in a scale
    v2[key_len:] = 0x7FC0
    out = vd.Attention(nq, nk, ht, 128, use_key_mask=True, qk_int8=True).forward(up(q, dev), up(k2, dev), up(v2, dev),
                                                                                  key_len=key_len)
    torch.cuda.synchronize()
    check(as_f64(out), oracle.mha_reference_qk_int8(q, k, v, key_len=key_len), f"int8 cross L={key_len}")


def test_batch_with_key_lengths_and_zero_query_block(dev):
    vd = vdm()
    B, nq, nk, ht = 2, 400, 300, 2
    lens = [300, 65]
    note(f"int8 batch B={B} nq={nq} nk={nk} key_lens={lens}, zero queries 128-255 in entry 1")
    es = []
    for i in range(B):
        q = si.normal_bf16((nq, ht, 128), 5400 + i, si.STREAM_Q)
        if i == 1:
            q[128:256] = 0     # one whole quantization block of zeros: scale 1, codes 0
        es.append((q, si.normal_bf16((nk, ht, 128), 5400 + i, si.STREAM_K),
                   si.normal_bf16((nk, ht, 128), 5400 + i, si.STREAM_V)))
    attn = vd.Attention(nq, nk, ht, 128, use_key_mask=True, batch=B, qk_int8=True)
    out = attn.forward(*(up(np.stack([e[j] for e in es]), dev) for j in range(3)), key_lens=lens)
    torch.cuda.synchronize()
    for i, ((q, k, v), L) in enumerate(zip(es, lens)):
        ref = oracle.mha_reference_qk_int8(q, k, v, key_len=L)
        check(as_f64(out[i]), ref, f"int8 batch entry {i} L={L}")
    # zero queries: uniform weights over the valid keys only
    vmean = int8_qk.bf16_bits_to_f32(es[1][2][:lens[1]]).astype(np.float64).mean(axis=0)
    got = as_f64(out[1, 128:256])
    assert np.abs(got - vmean[None]).max() < 2e-2


@pytest.mark.timeout(900)
def test_ulysses_share_n75600_sampled_rows(dev):
    vd = vdm()
    n = 21 * 45 * 80
    note(f"int8 N={n} Ht=40 heads 0-9 seed 1003 (sampled rows)")
    q = si.normal_bf16((n, 40, 128), 1003, si.STREAM_Q)
    k = si.normal_bf16((n, 40, 128), 1003, si.STREAM_K)
    v = si.normal_bf16((n, 40, 128), 1003, si.STREAM_V)
    out = vd.Attention(n, n, 40, 128, head_begin=0, head_count=10, qk_int8=True).forward(up(q, dev), up(k, dev),
                                                                                       up(v, dev))
    torch.cuda.synchronize()
    rows = si.sample_rows(n, 4096, 1003, si.tile_edge_rows(n))
    got = as_f64(out[torch.from_numpy(rows).to(dev)])
    ref = oracle.mha_reference_qk_int8(q, k, v, head_begin=0, head_count=10, rows=rows)
    check(got, ref, f"int8 N={n} ({len(rows)} rows x 10 heads)")


def test_scores_growing_past_first_tile_max_four_stage(dev):
    # more than 1024 keys and 256 workgroups of 256 queries: the eight-wave,
    # four-stage int8 kernel; the last keys overflow the first tile's reference,
    # so its exact-maximum retry runs
    from test_gpu_parity import growing_score_inputs
    vd = vdm()
    nq = nk = 4096
    ht = 16
    note(f"int8 growing scores, four-stage kernel: nq=nk={nq} heads={ht}")
    q, k, v = growing_score_inputs(nq, nk, ht, 128, 9500)
    out = vd.Attention(nq, nk, ht, 128, qk_int8=True).forward(up(q, dev), up(k, dev), up(v, dev))
    torch.cuda.synchronize()
    check(as_f64(out), oracle.mha_reference_qk_int8(q, k, v), "int8 growing scores 4-stage")
