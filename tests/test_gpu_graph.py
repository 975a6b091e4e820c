"""GPU: the compute calls only enqueue kernels (no allocation, memset or host
synchronisation), so a serving loop can capture them in a HIP graph once and
replay it. Each replay must equal the eager call bit for bit, also after the
captured input buffers were refilled between replays; eager work runs between the
replays. Scalar arguments (key length, keep) are fixed at capture.
"""
import numpy as np
import pytest
import torch

import synthetic_inputs as si
from test_gpu_parity import down, note, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this environment")
    import long_sequence_attention_amd as vd
    vd.load_library()
    return torch.device("cuda:0")


def capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replay_checks(g, out, eager_of, q_buf, q_new):
    """Replay three times against the eager result, then once more after new q."""
    want = eager_of()
    for i in range(3):
        out.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(down(out), want), f"replay {i}"
        _ = (q_buf.float() * 2.0).sum().item()   # unrelated eager work between replays
    q_buf.copy_(q_new)
    want2 = eager_of()
    out.fill_(7.0)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert np.array_equal(down(out), want2), "replay after refilling q"
    assert not np.array_equal(want, want2)


@pytest.mark.parametrize("masked", [False, True])
def test_dense_attention_graph_replay(dev, masked):
    import long_sequence_attention_amd as vd
    n, ht, d = 2000, 4, 128
    note(f"graph replay dense n={n} masked={masked}")
    q = up(si.normal_bf16((n, ht, d), 4400, si.STREAM_Q), dev)
    k = up(si.normal_bf16((n, ht, d), 4400, si.STREAM_K), dev)
    v = up(si.normal_bf16((n, ht, d), 4400, si.STREAM_V), dev)
    q_new = up(si.normal_bf16((n, ht, d), 4401, si.STREAM_Q), dev)
    attn = vd.Attention(n, n, ht, d, head_begin=1, head_count=2, use_key_mask=masked)
    L = 1234 if masked else 0
    out = torch.empty(attn.out_shape, dtype=torch.bfloat16, device=dev)
    ws = attn.new_workspace(dev)
    g = capture(lambda: attn.forward(q, k, v, key_len=L, out=out, workspace=ws))

    def eager():
        o = attn.forward(q, k, v, key_len=L)
        torch.cuda.synchronize()
        return down(o)
    replay_checks(g, out, eager, q, q_new)


@pytest.mark.parametrize("cubes", [None, (5, 9, 57)])
def test_block_sparse_graph_replay(dev, cubes):
    import long_sequence_attention_amd as vd
    n, ht, d = (64 * 40 + 9 if cubes is None else int(np.prod(cubes))), 2, 128
    note(f"graph replay block-sparse n={n} cubes={cubes}")
    q = up(si.normal_bf16((n, ht, d), 4410, si.STREAM_Q), dev)
    k = up(si.normal_bf16((n, ht, d), 4410, si.STREAM_K), dev)
    v = up(si.normal_bf16((n, ht, d), 4410, si.STREAM_V), dev)
    q_new = up(si.normal_bf16((n, ht, d), 4411, si.STREAM_Q), dev)
    attn = vd.Attention(n, n, ht, d, vsa_cubes=cubes)
    keep = attn.vsa_keep(0.8)
    out = torch.empty(attn.out_shape, dtype=torch.bfloat16, device=dev)
    ws = attn.new_vsa_workspace(keep, dev)
    g = capture(lambda: attn.vsa_forward(q, k, v, keep=keep, out=out, workspace=ws))

    def eager():
        o = attn.vsa_forward(q, k, v, keep=keep)
        torch.cuda.synchronize()
        return down(o)
    replay_checks(g, out, eager, q, q_new)


def test_resident_cross_attention_graph_replay(dev):
    # short text keys with query tiles for every CU: the keys-resident kernel (its
    # persistent grid is sized at capture)
    import long_sequence_attention_amd as vd
    nq, nk, ht, d, L = 12000, 256, 8, 128, 200
    note(f"graph replay resident cross-attention nq={nq} nk={nk} L={L}")
    q = up(si.normal_bf16((nq, ht, d), 4420, si.STREAM_Q), dev)
    k = up(si.normal_bf16((nk, ht, d), 4420, si.STREAM_K), dev)
    v = up(si.normal_bf16((nk, ht, d), 4420, si.STREAM_V), dev)
    q_new = up(si.normal_bf16((nq, ht, d), 4421, si.STREAM_Q), dev)
    attn = vd.Attention(nq, nk, ht, d, use_key_mask=True)
    out = torch.empty(attn.out_shape, dtype=torch.bfloat16, device=dev)
    ws = attn.new_workspace(dev)
    g = capture(lambda: attn.forward(q, k, v, key_len=L, out=out, workspace=ws))

    def eager():
        o = attn.forward(q, k, v, key_len=L)
        torch.cuda.synchronize()
        return down(o)
    replay_checks(g, out, eager, q, q_new)


def test_retry_list_graph_replay(dev):
    # q[:, :, 0] = 8 and keys whose first dimension ramps up: most rows overflow the
    # first tile's reference, so every replay lists rows (the list counters are cleared
    # by the captured prepare and again by the retry launch) and recomputes them
    import long_sequence_attention_amd as vd
    nq, nk, ht, d = 1500, 2600, 2, 128
    note(f"graph replay with the retry list nq={nq} nk={nk}")
    q = si.normal_bf16((nq, ht, d), 4430, si.STREAM_Q, 0.25)
    k = si.normal_bf16((nk, ht, d), 4430, si.STREAM_K, 0.25)
    v = si.normal_bf16((nk, ht, d), 4430, si.STREAM_V, 1.0)
    q[:, :, 0] = si.f32_to_bf16_bits(np.full((nq, ht), 8.0, dtype=np.float32))
    k[:, :, 0] = si.f32_to_bf16_bits(np.broadcast_to((np.arange(nk, dtype=np.float32) / 8.0)[:, None], (nk, ht)))
    q_new = q.copy()
    q_new[::3, :, 0] = 0
    qd, kd, vd_ = up(q, dev), up(k, dev), up(v, dev)
    attn = vd.Attention(nq, nk, ht, d)
    out = torch.empty(attn.out_shape, dtype=torch.bfloat16, device=dev)
    ws = attn.new_workspace(dev)
    g = capture(lambda: attn.forward(qd, kd, vd_, out=out, workspace=ws))

    def eager():
        o = attn.forward(qd, kd, vd_)
        torch.cuda.synchronize()
        return down(o)
    replay_checks(g, out, eager, qd, up(q_new, dev))
