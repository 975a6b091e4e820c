"""The C ABI without a GPU: symbols, host-side validation, status strings.

Every call here returns before the library touches the HIP runtime.
"""
import ctypes
import json
import os
import re

import pytest

import long_sequence_attention_amd as vd
from long_sequence_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vdit_attn.h")

INVALID, UNSUPPORTED, ALIGNMENT, WORKSPACE = 1, 2, 3, 6


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from long_sequence_attention_amd import build
        build.build()
    return _lib.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(vdit_\w+)\s*\(", text, flags=re.M)


def test_library_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) == 20
    assert sorted(names) == sorted(_lib.SIGNATURES)
    for n in names:
        assert hasattr(lib, n), n


def test_desc_struct_matches_header_field_order():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct \{(.*?)\} vdit_attn_desc_t;", text, flags=re.S).group(1)
    fields = []
    for decl in body.split(";"):
        decl = decl.strip()
        if not decl:
            continue
        names = decl.split(None, 1)[1]
        fields += [x.strip() for x in names.split(",")]
    assert fields == [f for f, _ in _lib.Desc._fields_]


def test_status_strings(lib):
    for code, name in _lib.STATUS_NAMES.items():
        assert vd.status_string(code).startswith(name)
    assert vd.status_string(99).startswith("VDIT_ERR_UNKNOWN")


def test_ulysses_heads_golden(lib):
    with open(os.path.join(ROOT, "tests", "golden", "ulysses_head_shares.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        if c["valid"]:
            for r in range(c["degree"]):
                assert vd.ulysses_heads(c["heads_total"], c["degree"], r) == (r * c["heads_per_rank"],
                                                                                c["heads_per_rank"])
        else:
            with pytest.raises(vd.VditError) as e:
                vd.ulysses_heads(c["heads_total"], c["degree"], 0)
            assert e.value.code == INVALID
    for bad in [(40, 4, 4), (40, 4, -1), (40, 0, 0), (0, 1, 0)]:
        with pytest.raises(vd.VditError):
            vd.ulysses_heads(*bad)


def _desc(**kw):
    base = dict(nq=4096, nk=4096, heads_total=40, head_dim=128)
    base.update(kw)
    extra = {k: base.pop(k) for k in list(base) if k not in ("nq", "nk", "heads_total", "head_dim")}
    return vd.make_desc(base["nq"], base["nk"], base["heads_total"], base["head_dim"], **extra)


ROPE = {"grid": (4, 32, 32), "dims": (44, 42, 42), "base": 10000.0}


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), UNSUPPORTED),
    (dict(head_dim=256), UNSUPPORTED),
    (dict(nq=0), INVALID),
    (dict(nk=-1), INVALID),
    (dict(heads_total=0, head_count=1), INVALID),
    (dict(head_begin=35, head_count=10), INVALID),
    (dict(head_begin=-1, head_count=4), INVALID),
    (dict(head_count=0), INVALID),
    (dict(layout="N3HD", nk=512), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(rope=dict(ROPE, grid=(4, 32, 31))), INVALID),
    (dict(rope=dict(ROPE, dims=(43, 43, 42))), INVALID),
    (dict(rope=dict(ROPE, dims=(44, 42, 40))), INVALID),
    (dict(rope=dict(ROPE, dims=(0, 64, 64))), INVALID),
    (dict(rope=dict(ROPE, base=0.0)), INVALID),
    (dict(rope=dict(ROPE, base=float("inf"))), INVALID),
    (dict(nk=512, rope=ROPE), INVALID),
    (dict(batch=-1), INVALID),
    (dict(batch=65), UNSUPPORTED),
    (dict(batch=64, head_count=1025, heads_total=2048), UNSUPPORTED),
    (dict(qk_int8=True, head_dim=64), UNSUPPORTED),
    (dict(qk_int8=True, rope=ROPE), UNSUPPORTED),
    (dict(qk_int8=True, nq=64, nk=262145), UNSUPPORTED),
    (dict(vsa_cubes=(4, 32, 31)), INVALID),                  # the grid does not hold nq tokens
    (dict(vsa_cubes=(0, 64, 64)), INVALID),
    (dict(vsa_cubes=(4, 32, 32), nk=2048), INVALID),         # nq != nk
    (dict(vsa_cubes=(8, 256, 260), nq=532480, nk=532480), UNSUPPORTED),  # 8320 cubes > 8192
    # a 64-key tile's row offsets must fit 32-bit byte offsets: 64 * token stride * 2 < 2^31
    (dict(nq=64, nk=64, heads_total=131072, head_count=1), UNSUPPORTED),
    (dict(nq=64, nk=64, heads_total=43691, head_count=1, layout="N3HD"), UNSUPPORTED),
])
def test_create_rejects_bad_descriptors(lib, kw, code):
    st, h = vd.create_raw(_desc(**kw))
    assert st == code and h == 0


def test_largest_token_stride_is_accepted(lib):
    for kw in (dict(heads_total=131071), dict(heads_total=43690, layout="N3HD")):
        # validation passes; without a device, create then reports DEVICE
        st, h = vd.create_raw(_desc(nq=64, nk=64, head_count=1, **kw))
        assert st in (0, 5), kw
        if h:
            assert lib.vdit_attn_destroy(ctypes.c_void_p(h)) == 0


def test_batch_zero_reads_as_one():
    # the field defaults to 0 in a zero-initialised descriptor; the binding passes 1
    assert _lib.Desc().batch == 0 and _desc().batch == 1 and _desc(batch=2).batch == 2


def test_create_rejects_null_arguments(lib):
    h = ctypes.c_void_p()
    assert lib.vdit_attn_create(None, ctypes.byref(h)) == INVALID
    d = _desc()
    assert lib.vdit_attn_create(ctypes.byref(d), None) == INVALID


def test_handle_checks_without_device(lib):
    assert lib.vdit_attn_destroy(None) == 0
    bogus = ctypes.c_void_p(0x1000)
    assert lib.vdit_attn_destroy(bogus) == INVALID
    n = ctypes.c_size_t()
    assert lib.vdit_attn_workspace_bytes(bogus, ctypes.byref(n)) == INVALID
    assert lib.vdit_attn_fwd(bogus, None, None, None, 1, None, None, 0, None) == INVALID
    assert lib.vdit_attn_prepare(bogus, None, None, None, 1, None, 0, None) == INVALID
    assert lib.vdit_attn_attend(bogus, None, None, None, 1, None, None, 0, None) == INVALID
    assert lib.vdit_attn_fwd_noalloc(bogus, None, None, None, 1, None, None) == INVALID
    lens = (ctypes.c_int32 * 2)(5, 7)
    assert lib.vdit_attn_fwd_lens(bogus, None, None, None, lens, None, None, 0, None) == INVALID
    assert lib.vdit_attn_prepare_lens(bogus, None, None, None, lens, None, 0, None) == INVALID
    assert lib.vdit_attn_attend_lens(bogus, None, None, None, lens, None, None, 0, None) == INVALID
    assert lib.vdit_attn_rope_probe(bogus, None, None) == INVALID
    k = ctypes.c_int32()
    assert lib.vdit_vsa_keep(bogus, 0.8, ctypes.byref(k)) == INVALID
    assert lib.vdit_vsa_workspace_bytes(bogus, 3, ctypes.byref(n)) == INVALID
    assert lib.vdit_vsa_select(bogus, None, None, 3, None, None, 0, None) == INVALID
    assert lib.vdit_vsa_attend(bogus, None, None, None, 3, None, None, None, 0, None) == INVALID
    assert lib.vdit_vsa_fwd(bogus, None, None, None, 3, None, None, 0, None) == INVALID


def test_pack_validation_without_device(lib):
    p = ctypes.c_void_p(0x10000)
    q = ctypes.c_void_p(0x20000000)
    assert lib.vdit_pack_heads(None, q, 10, 40, 128, 4, None) == INVALID
    assert lib.vdit_pack_heads(p, q, 10, 40, 128, 3, None) == INVALID
    assert lib.vdit_pack_heads(p, q, 0, 40, 128, 4, None) == INVALID
    assert lib.vdit_unpack_heads(p, ctypes.c_void_p(0x20000008), 10, 40, 128, 4, None) == ALIGNMENT
    assert lib.vdit_pack_heads(p, q, 10, 40, 4, 4, None) == ALIGNMENT
    assert lib.vdit_pack_heads(p, ctypes.c_void_p(0x10000 + 64), 10, 40, 128, 4, None) == INVALID


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load()
