"""Thin Python binding over the C ABI (include/vdit_attn.h).

Argument marshalling only: torch tensors are checked for device, dtype, shape
and contiguity, and their device pointers and the current HIP stream are handed
to the library. Every computation runs in the library's HIP kernels; there is
no fallback path.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib


class VditError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = int(code)
        self.status = _lib.STATUS_NAMES.get(self.code, f"status {code}")
        super().__init__(f"{what}: {self.status}")


def _check(code: int, what: str) -> None:
    if code != _lib.VDIT_OK:
        raise VditError(code, what)


def status_string(code: int) -> str:
    return _lib.load().vdit_status_string(code).decode()


def _stream_ptr(t: torch.Tensor, stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return int(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, shape, dtype, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def ulysses_heads(heads_total: int, degree: int, rank: int) -> tuple[int, int]:
    """Head share (begin, count) of ``rank`` at Ulysses degree ``degree``."""
    b, c = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.load().vdit_attn_ulysses_heads(heads_total, degree, rank, ctypes.byref(b), ctypes.byref(c)),
           "vdit_attn_ulysses_heads")
    return b.value, c.value


def make_desc(nq: int, nk: int, heads_total: int, head_dim: int, *, layout: str = "NHD", head_begin: int = 0,
              head_count: int | None = None, scale: float = 0.0, use_key_mask: bool = False,
              rope: dict | None = None, batch: int = 1, qk_int8: bool = False,
              vsa_cubes: tuple | None = None) -> _lib.Desc:
    d = _lib.Desc()
    d.batch = batch
    d.qk_int8 = 1 if qk_int8 else 0
    d.nq, d.nk, d.heads_total, d.head_dim = nq, nk, heads_total, head_dim
    d.layout = {"NHD": _lib.LAYOUT_NHD, "N3HD": _lib.LAYOUT_N3HD}[layout]
    d.head_begin = head_begin
    d.head_count = heads_total - head_begin if head_count is None else head_count
    d.scale = scale
    d.use_key_mask = 1 if use_key_mask else 0
    if rope is not None:
        d.use_rope = 1
        d.grid_t, d.grid_h, d.grid_w = (int(g) for g in rope["grid"])
        d.rope_dim_t, d.rope_dim_h, d.rope_dim_w = (int(x) for x in rope["dims"])
        d.rope_base = float(rope.get("base", 10000.0))
    if vsa_cubes is not None:
        d.vsa_cubes = 1
        d.grid_t, d.grid_h, d.grid_w = (int(g) for g in vsa_cubes)
    return d


def create_raw(desc: _lib.Desc) -> tuple[int, int]:
    """Call vdit_attn_create; returns (status, handle or 0). For tests of the validation."""
    h = ctypes.c_void_p()
    st = _lib.load().vdit_attn_create(ctypes.byref(desc), ctypes.byref(h))
    return st, (h.value or 0)


class Attention:
    """One attention plan (vdit_attn_t) and its calls on torch tensors.

    With ``batch`` = B > 1 every tensor has a leading [B] dimension; the calls take
    either one ``key_len`` for all entries or ``key_lens`` (B values). ``qk_int8``
    selects q.k on int8 per-block codes (d = 128, no RoPE). ``vsa_cubes`` = (T, H, W):
    the block-sparse calls tile q and k as 4x4x4 cubes of that latent grid instead of
    runs of 64 tokens.
    """

    def __init__(self, nq: int, nk: int, heads_total: int, head_dim: int, *, layout: str = "NHD",
                 head_begin: int = 0, head_count: int | None = None, scale: float = 0.0,
                 use_key_mask: bool = False, rope: dict | None = None, batch: int = 1,
                 qk_int8: bool = False, vsa_cubes: tuple | None = None):
        self._lib = _lib.load()
        self.desc = make_desc(nq, nk, heads_total, head_dim, layout=layout, head_begin=head_begin,
                              head_count=head_count, scale=scale, use_key_mask=use_key_mask, rope=rope,
                              batch=batch, qk_int8=qk_int8, vsa_cubes=vsa_cubes)
        self.vsa_cubes = None if vsa_cubes is None else tuple(int(g) for g in vsa_cubes)
        self.layout = layout
        self.batch = int(batch)
        h = ctypes.c_void_p()
        _check(self._lib.vdit_attn_create(ctypes.byref(self.desc), ctypes.byref(h)), "vdit_attn_create")
        self._h = h
        n = ctypes.c_size_t()
        _check(self._lib.vdit_attn_workspace_bytes(self._h, ctypes.byref(n)), "vdit_attn_workspace_bytes")
        self.workspace_bytes = int(n.value)

    # -- shapes
    def _lead(self):
        return (self.batch,) if self.batch > 1 else ()

    @property
    def out_shape(self):
        d = self.desc
        return self._lead() + (d.nq, d.head_count, d.head_dim)

    def _check_inputs(self, q, k, v):
        d = self.desc
        b = self._lead()
        if self.layout == "N3HD":
            _need(q, b + (d.nq, 3, d.heads_total, d.head_dim), torch.bfloat16, "qkv")
            if k is not None or v is not None:
                raise ValueError("the packed layout takes the [N, 3, H, d] tensor alone")
        else:
            _need(q, b + (d.nq, d.heads_total, d.head_dim), torch.bfloat16, "q")
            _need(k, b + (d.nk, d.heads_total, d.head_dim), torch.bfloat16, "k")
            _need(v, b + (d.nk, d.heads_total, d.head_dim), torch.bfloat16, "v")

    def _lens(self, key_lens):
        if key_lens is None:
            return None
        lens = [int(x) for x in key_lens]
        if len(lens) != self.batch:
            raise ValueError(f"key_lens needs {self.batch} values, got {len(lens)}")
        return (ctypes.c_int32 * len(lens))(*lens)

    def new_workspace(self, device) -> torch.Tensor:
        return torch.empty(max(self.workspace_bytes, 16), dtype=torch.uint8, device=device)

    def _ws(self, workspace, device):
        if workspace is None:
            workspace = self.new_workspace(device)
        if workspace.device.type != "cuda" or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous GPU tensor")
        return workspace

    # -- calls
    def forward(self, q, k=None, v=None, *, key_len: int = 0, key_lens=None, out=None, workspace=None,
                stream=None):
        self._check_inputs(q, k, v)
        if out is None:
            out = torch.empty(self.out_shape, dtype=torch.bfloat16, device=q.device)
        _need(out, self.out_shape, torch.bfloat16, "out")
        ws = self._ws(workspace, q.device)
        nbytes, sp = ws.numel() * ws.element_size(), _stream_ptr(q, stream)
        lens = self._lens(key_lens)
        if lens is None:
            _check(self._lib.vdit_attn_fwd(self._h, _ptr(q), _ptr(k), _ptr(v), int(key_len), _ptr(out), _ptr(ws),
                                           nbytes, sp), "vdit_attn_fwd")
        else:
            _check(self._lib.vdit_attn_fwd_lens(self._h, _ptr(q), _ptr(k), _ptr(v), lens, _ptr(out), _ptr(ws),
                                                nbytes, sp), "vdit_attn_fwd_lens")
        return out

    __call__ = forward

    def forward_noalloc(self, q, k=None, v=None, *, key_len: int = 0, out=None, stream=None):
        """forward without a workspace: the library's fixed per-GPU array holds it
        (vdit_attn_fwd_noalloc; calls overlapping in time on one GPU race)."""
        self._check_inputs(q, k, v)
        if out is None:
            out = torch.empty(self.out_shape, dtype=torch.bfloat16, device=q.device)
        _need(out, self.out_shape, torch.bfloat16, "out")
        _check(self._lib.vdit_attn_fwd_noalloc(self._h, _ptr(q), _ptr(k), _ptr(v), int(key_len), _ptr(out),
                                               _stream_ptr(q, stream)), "vdit_attn_fwd_noalloc")
        return out

    def prepare(self, q, k=None, v=None, *, key_len: int = 0, key_lens=None, workspace=None, stream=None):
        self._check_inputs(q, k, v)
        ws = self._ws(workspace, q.device)
        nbytes, sp = ws.numel() * ws.element_size(), _stream_ptr(q, stream)
        lens = self._lens(key_lens)
        if lens is None:
            _check(self._lib.vdit_attn_prepare(self._h, _ptr(q), _ptr(k), _ptr(v), int(key_len), _ptr(ws), nbytes,
                                               sp), "vdit_attn_prepare")
        else:
            _check(self._lib.vdit_attn_prepare_lens(self._h, _ptr(q), _ptr(k), _ptr(v), lens, _ptr(ws), nbytes,
                                                    sp), "vdit_attn_prepare_lens")
        return ws

    def attend(self, q, k=None, v=None, *, key_len: int = 0, key_lens=None, out=None, workspace=None,
               stream=None):
        self._check_inputs(q, k, v)
        if workspace is None:
            raise ValueError("attend needs the workspace filled by prepare")
        if out is None:
            out = torch.empty(self.out_shape, dtype=torch.bfloat16, device=q.device)
        _need(out, self.out_shape, torch.bfloat16, "out")
        nbytes, sp = workspace.numel() * workspace.element_size(), _stream_ptr(q, stream)
        lens = self._lens(key_lens)
        if lens is None:
            _check(self._lib.vdit_attn_attend(self._h, _ptr(q), _ptr(k), _ptr(v), int(key_len), _ptr(out),
                                              _ptr(workspace), nbytes, sp), "vdit_attn_attend")
        else:
            _check(self._lib.vdit_attn_attend_lens(self._h, _ptr(q), _ptr(k), _ptr(v), lens, _ptr(out),
                                                   _ptr(workspace), nbytes, sp), "vdit_attn_attend_lens")
        return out

    # -- block-sparse attention over 64-token tiles or latent-grid cubes (vdit_vsa_*)
    def _cubes(self) -> int:
        t, h, w = self.vsa_cubes
        return ((t + 3) // 4) * ((h + 3) // 4) * ((w + 3) // 4)

    @property
    def q_tiles(self) -> int:
        return self._cubes() if self.vsa_cubes else (self.desc.nq + 63) // 64

    @property
    def k_tiles(self) -> int:
        return self._cubes() if self.vsa_cubes else (self.desc.nk + 63) // 64

    def vsa_keep(self, sparsity: float) -> int:
        """Key tiles kept per query tile at ``sparsity``: ceil((1 - sparsity) * Tk), >= 1."""
        k = ctypes.c_int32()
        _check(self._lib.vdit_vsa_keep(self._h, float(sparsity), ctypes.byref(k)), "vdit_vsa_keep")
        return int(k.value)

    def vsa_workspace_bytes(self, keep: int) -> int:
        n = ctypes.c_size_t()
        _check(self._lib.vdit_vsa_workspace_bytes(self._h, int(keep), ctypes.byref(n)), "vdit_vsa_workspace_bytes")
        return int(n.value)

    def new_vsa_workspace(self, keep: int, device) -> torch.Tensor:
        return torch.empty(max(self.vsa_workspace_bytes(keep), 16), dtype=torch.uint8, device=device)

    def tiles_shape(self, keep: int):
        return self._lead() + (self.desc.head_count, self.q_tiles, int(keep))

    def _keep(self, keep, sparsity):
        if (keep is None) == (sparsity is None):
            raise ValueError("give exactly one of keep and sparsity")
        return int(keep) if keep is not None else self.vsa_keep(sparsity)

    def vsa_select(self, q, k=None, *, keep: int | None = None, sparsity: float | None = None, tiles=None,
                   workspace=None, stream=None) -> torch.Tensor:
        """Kept key tiles, int32 [B?, head_count, Tq, keep], ascending per query tile."""
        keep = self._keep(keep, sparsity)
        d = self.desc
        b = self._lead()
        if self.layout == "N3HD":
            _need(q, b + (d.nq, 3, d.heads_total, d.head_dim), torch.bfloat16, "qkv")
            if k is not None:
                raise ValueError("the packed layout takes the [N, 3, H, d] tensor alone")
        else:
            _need(q, b + (d.nq, d.heads_total, d.head_dim), torch.bfloat16, "q")
            _need(k, b + (d.nk, d.heads_total, d.head_dim), torch.bfloat16, "k")
        if tiles is None:
            tiles = torch.empty(self.tiles_shape(keep), dtype=torch.int32, device=q.device)
        _need(tiles, self.tiles_shape(keep), torch.int32, "tiles")
        if workspace is None:
            workspace = self.new_vsa_workspace(keep, q.device)
        _check(self._lib.vdit_vsa_select(self._h, _ptr(q), _ptr(k), keep, _ptr(tiles), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream_ptr(q, stream)),
               "vdit_vsa_select")
        return tiles

    def vsa_attend(self, q, k=None, v=None, *, tiles, out=None, workspace=None, stream=None) -> torch.Tensor:
        """Block-sparse attention over the key tiles in ``tiles`` [B?, head_count, Tq, keep]."""
        self._check_inputs(q, k, v)
        keep = int(tiles.shape[-1]) if isinstance(tiles, torch.Tensor) else 0
        _need(tiles, self.tiles_shape(keep), torch.int32, "tiles")
        if out is None:
            out = torch.empty(self.out_shape, dtype=torch.bfloat16, device=q.device)
        _need(out, self.out_shape, torch.bfloat16, "out")
        ws = self._ws(workspace, q.device)
        _check(self._lib.vdit_vsa_attend(self._h, _ptr(q), _ptr(k), _ptr(v), keep, _ptr(tiles), _ptr(out), _ptr(ws),
                                         ws.numel() * ws.element_size(), _stream_ptr(q, stream)), "vdit_vsa_attend")
        return out

    def vsa_forward(self, q, k=None, v=None, *, keep: int | None = None, sparsity: float | None = None, out=None,
                    workspace=None, stream=None) -> torch.Tensor:
        """Coarse selection then block-sparse attention (vdit_vsa_fwd)."""
        keep = self._keep(keep, sparsity)
        self._check_inputs(q, k, v)
        if out is None:
            out = torch.empty(self.out_shape, dtype=torch.bfloat16, device=q.device)
        _need(out, self.out_shape, torch.bfloat16, "out")
        if workspace is None:
            workspace = self.new_vsa_workspace(keep, q.device)
        _check(self._lib.vdit_vsa_fwd(self._h, _ptr(q), _ptr(k), _ptr(v), keep, _ptr(out), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream_ptr(q, stream)),
               "vdit_vsa_fwd")
        return out

    def rope_probe(self, device, stream=None) -> torch.Tensor:
        d = self.desc
        out = torch.empty((d.nq, d.head_dim // 2, 5), dtype=torch.int32, device=device)
        _check(self._lib.vdit_attn_rope_probe(self._h, _ptr(out), _stream_ptr(out, stream)), "vdit_attn_rope_probe")
        return out

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            _check(self._lib.vdit_attn_destroy(self._h), "vdit_attn_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _pack_call(fn_name: str, src: torch.Tensor, out: torch.Tensor, n: int, ht: int, d: int, groups: int, stream):
    _check(getattr(_lib.load(), fn_name)(_ptr(src), _ptr(out), n, ht, d, groups, _stream_ptr(src, stream)), fn_name)
    return out


def pack_heads(src: torch.Tensor, groups: int, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """[n, Ht, d] -> [groups, n, Ht/groups, d] (bit-exact permutation)."""
    if src.dim() != 3:
        raise ValueError("src must be [n, Ht, d]")
    n, ht, d = src.shape
    if groups <= 0 or ht % groups:
        raise ValueError("groups must divide the head count")
    shape = (groups, n, ht // groups, d)
    if out is None:
        out = torch.empty(shape, dtype=src.dtype, device=src.device)
    _need(src, (n, ht, d), src.dtype, "src")
    _need(out, shape, src.dtype, "out")
    if src.element_size() != 2:
        raise ValueError("pack moves 2-byte elements")
    return _pack_call("vdit_pack_heads", src, out, n, ht, d, groups, stream)


def unpack_heads(src: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """[groups, n, Ht/groups, d] -> [n, Ht, d] (inverse of pack_heads)."""
    if src.dim() != 4:
        raise ValueError("src must be [groups, n, Ht/groups, d]")
    g, n, hg, d = src.shape
    shape = (n, g * hg, d)
    if out is None:
        out = torch.empty(shape, dtype=src.dtype, device=src.device)
    _need(src, (g, n, hg, d), src.dtype, "src")
    _need(out, shape, src.dtype, "out")
    if src.element_size() != 2:
        raise ValueError("unpack moves 2-byte elements")
    return _pack_call("vdit_unpack_heads", src, out, n, g * hg, d, g, stream)
