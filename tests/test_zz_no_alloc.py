"""GPU: vdit_attn_fwd_noalloc (workspace in the library's fixed per-GPU array)
against vdit_attn_fwd with a caller workspace, through the raw C ABI.

Both run the same kernels on the same inputs, so the outputs must be equal bit
for bit. Calls follow each other on one stream, each smaller than the one
before, so a later call runs over what the earlier one left in the array.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from test_gpu_parity import as_f64, check, note, up

pytestmark = pytest.mark.gpu

ROPE = {"grid": (4, 8, 30), "dims": (44, 42, 42), "base": 10000.0}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this environment")
    import long_sequence_attention_amd as vd
    vd.load_library()
    return torch.device("cuda:0")


def p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def both(dev, attn, q, k, v, key_len):
    """(vdit_attn_fwd output, vdit_attn_fwd_noalloc output), both raw C calls on one stream."""
    from long_sequence_attention_amd import _lib
    lib = _lib.load()
    s = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    ref = torch.full(attn.out_shape, 7.0, dtype=torch.bfloat16, device=dev)
    got = torch.full(attn.out_shape, -3.0, dtype=torch.bfloat16, device=dev)
    ws = attn.new_workspace(dev)
    st = lib.vdit_attn_fwd(attn._h, p(q), p(k), p(v), key_len, p(ref), p(ws), ws.numel(), s)
    assert st == 0, st
    st = lib.vdit_attn_fwd_noalloc(attn._h, p(q), p(k), p(v), key_len, p(got), s)
    assert st == 0, st
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_equals_fwd_on_shrinking_calls(dev):
    import long_sequence_attention_amd as vd
    # 1: N=4096, 10 heads, d=128 (workspace ~10.5 MB)
    note("no-alloc call 1: N=4096 H=10 d=128")
    q, k, v = (si.normal_bf16((4096, 10, 128), 1002, s) for s in (0, 1, 2))
    a1 = vd.Attention(4096, 4096, 10, 128)
    ref, got = both(dev, a1, up(q, dev), up(k, dev), up(v, dev), 0)
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))
    check(as_f64(got), oracle.mha_reference(q, k, v), "no-alloc N=4096 H=10")
    # 2: smaller, masked, head share, d=64
    note("no-alloc call 2: nq=1000 nk=900 L=700 heads 1-2 of 4 d=64")
    q, k, v = (si.normal_bf16(sh, 9900, s) for sh, s in (((1000, 4, 64), 0), ((900, 4, 64), 1), ((900, 4, 64), 2)))
    a2 = vd.Attention(1000, 900, 4, 64, head_begin=1, head_count=2, use_key_mask=True)
    ref, got = both(dev, a2, up(q, dev), up(k, dev), up(v, dev), 700)
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))
    check(as_f64(got), oracle.mha_reference(q, k, v, head_begin=1, head_count=2, key_len=700), "no-alloc masked")
    # 3: smaller still, packed with RoPE (rotated keys in the array too)
    n = 4 * 8 * 30
    note(f"no-alloc call 3: packed RoPE n={n} H=2 d=128")
    qkv = si.normal_bf16((n, 3, 2, 128), 9901, 0, 0.5)
    a3 = vd.Attention(n, n, 2, 128, layout="N3HD", rope=ROPE)
    ref, got = both(dev, a3, up(qkv, dev), None, None, 0)
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))
    check(as_f64(got), oracle.mha_reference(qkv, layout="N3HD", rope=ROPE), "no-alloc packed RoPE")


def test_noalloc_rejects_plans_beyond_the_array(dev):
    import long_sequence_attention_amd as vd
    from long_sequence_attention_amd import _lib
    big = vd.Attention(64, 131072, 40, 128)   # 1.3 GB of float16 V^T
    assert big.workspace_bytes > (256 << 20)
    st = _lib.load().vdit_attn_fwd_noalloc(big._h, None, None, None, 0, None, None)
    assert st == 2  # VDIT_ERR_UNSUPPORTED, before any pointer is looked at
    with pytest.raises(vd.VditError):
        big.forward_noalloc(torch.empty((64, 40, 128), dtype=torch.bfloat16, device=dev),
                            torch.empty((131072, 40, 128), dtype=torch.bfloat16, device=dev),
                            torch.empty((131072, 40, 128), dtype=torch.bfloat16, device=dev))
