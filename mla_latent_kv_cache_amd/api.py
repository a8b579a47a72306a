"""Python binding of the latent-cache library: argument marshalling only.

Every step of append / decode / prefill runs in the library's gfx950 kernels; this module builds the
C structs from torch device tensors, passes the current HIP stream, and raises on a non-zero status.
There is no fallback: without the built library or a GPU the calls raise.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import _lib
from ._lib import (MLA_BF16, MLA_CACHE_DENSE, MLA_CACHE_INT2_G32_WIN, MLA_CACHE_INT4_G32, MLA_CACHE_INT4_G32_WIN,
                   MLA_F32, MlaCache, MlaConfig, MlaWeights)

_FMT = {"dense": MLA_CACHE_DENSE, "int4_g32": MLA_CACHE_INT4_G32, "int2_g32_win": MLA_CACHE_INT2_G32_WIN,
        "int4_g32_win": MLA_CACHE_INT4_G32_WIN}
WINDOWED = ("int2_g32_win", "int4_g32_win")


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = _lib.load().mla_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise MlaError(fn, rc)


@dataclass(frozen=True)
class LayerShape:
    """Shape of one converted layer and its cache format (mirrors mla_config)."""

    d_model: int
    n_heads: int
    d_head: int
    r_pairs: int
    d_kv: int
    dtype: str = "bf16"  # "bf16" or "f32"
    cache_fmt: str = "dense"  # "dense", "int4_g32", "int2_g32_win" or "int4_g32_win"
    # RoPE key heads: 0 (= n_heads, keys per query head) or a divisor of n_heads -- query head h uses key
    # head h // (n_heads // rope_heads), the layout of a layer converted from a grouped-query source
    rope_heads: int = 0

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def n_rope_heads(self) -> int:
        return self.rope_heads or self.n_heads

    def c(self) -> MlaConfig:
        return MlaConfig(
            self.d_model,
            self.n_heads,
            self.d_head,
            self.r_pairs,
            self.d_kv,
            MLA_BF16 if self.dtype == "bf16" else MLA_F32,
            _FMT[self.cache_fmt],
            self.rope_heads,
        )


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _expect(*specs) -> None:
    """Each spec is (tensor, name, dtype, shape, device) (None: not checked).  Raise ValueError unless every
    tensor has its dtype and shape (checked for all of them first), and then unless every one is a contiguous
    GPU tensor on its device.  The library reads raw device pointers, so a host tensor, a wrong element type
    or a short buffer would be read or written past its end rather than rejected."""
    for t, name, dtype, shape, _ in specs:
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name}: expected a torch tensor, got {type(t).__name__}")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    for t, name, _, _, device in specs:
        if not t.is_cuda:
            raise ValueError(f"{name}: on {t.device}, the library takes GPU tensors")
        if device is not None and t.device != device:
            raise ValueError(f"{name}: on {t.device}, the cache is on {device}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: not contiguous")


def _expect_ws(ws, name: str, need: int, device) -> None:
    """A caller workspace: uint8 on the cache's device, at least `need` bytes."""
    _expect((ws, name, torch.uint8, None, device))
    if ws.numel() < need:
        raise ValueError(f"{name}: {ws.numel()} bytes, {need} needed")


def rope_tables(rope_len: int, d_head: int, theta: float = 1e4):
    """cos / sin tables [rope_len, d_head/2] (fp32) of the angle pos * theta^(-2p/d_head): mla_rope_tables."""
    cos = np.empty((rope_len, d_head // 2), dtype=np.float32)
    sin = np.empty_like(cos)
    _check("mla_rope_tables", _lib.load().mla_rope_tables(int(rope_len), int(d_head), float(theta),
                                                          cos.ctypes.data if cos.size else None,
                                                          sin.ctypes.data if sin.size else None))
    return cos, sin


@dataclass
class LayerWeights:
    """Converted weights on the device, in the ABI's [out_features, in_features] layouts."""

    shape: LayerShape
    w_dkv: torch.Tensor  # [d_kv, d_model]
    w_krope: torch.Tensor  # [n_h*2r, d_model]
    w_uk: torch.Tensor  # [n_h, d_h-2r, d_kv]
    w_uv: torch.Tensor  # [n_h, d_h, d_kv]
    pair_idx: torch.Tensor  # [n_h, r] int32
    rope_cos: torch.Tensor  # [rope_len, d_h/2] fp32
    rope_sin: torch.Tensor

    def c(self) -> MlaWeights:
        return MlaWeights(
            _ptr(self.w_dkv),
            _ptr(self.w_krope),
            _ptr(self.w_uk),
            _ptr(self.w_uv),
            _ptr(self.pair_idx),
            _ptr(self.rope_cos),
            _ptr(self.rope_sin),
            self.rope_cos.shape[0],
        )


def pack_weights(shape: LayerShape, conv: dict, rope_len: int, theta: float = 1e4, device="cuda") -> LayerWeights:
    """Move converted weights (math layouts: w_dkv [d, d_kv], w_krope [d, n_rh*2r], w_uk [n_h, d_kv, d_h-2r],
    w_uv [n_h, d_kv, d_h], pair_idx [n_rh, r]; n_rh = shape.n_rope_heads) to the device in the ABI layouts and
    dtype."""
    dt = shape.torch_dtype

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(device=device, dtype=dt).contiguous()

    n_h, dn, dh, D, d = shape.n_heads, shape.d_head - 2 * shape.r_pairs, shape.d_head, shape.d_kv, shape.d_model
    w_krope_m = np.asarray(conv["w_krope"]).reshape(d, -1)
    pair_idx = np.asarray(conv["pair_idx"])
    nrh = shape.n_rope_heads
    if nrh != n_h and pair_idx.shape[0] == n_h:
        # a layer expanded per query head (the GQA conversion): one RoPE key head per group of n_h / nrh heads,
        # which must all carry the same kept pairs and key columns
        hpg = n_h // nrh
        wk3 = w_krope_m.reshape(d, n_h, -1)
        for g in range(nrh):
            heads = range(g * hpg, (g + 1) * hpg)
            if any(not np.array_equal(pair_idx[h], pair_idx[g * hpg]) or not np.array_equal(wk3[:, h], wk3[:, g * hpg])
                   for h in heads):
                raise ValueError(f"query heads of RoPE key head {g} differ in their kept pairs or key columns")
        pair_idx = pair_idx[::hpg]
        w_krope_m = wk3[:, ::hpg, :].reshape(d, -1)
    if pair_idx.shape != (nrh, shape.r_pairs) or w_krope_m.shape != (d, nrh * 2 * shape.r_pairs):
        raise ValueError(f"pair_idx {pair_idx.shape} / w_krope {w_krope_m.shape} do not hold {nrh} RoPE key heads "
                         f"of {shape.r_pairs} pairs")
    w_dkv = dev(np.asarray(conv["w_dkv"]).T)
    w_krope = dev(w_krope_m.T)
    w_uk = dev(np.asarray(conv["w_uk"]).reshape(n_h, D, dn).transpose(0, 2, 1))
    w_uv = dev(np.asarray(conv["w_uv"]).reshape(n_h, D, dh).transpose(0, 2, 1))
    pidx = torch.from_numpy(np.ascontiguousarray(pair_idx, dtype=np.int32)).to(device)
    cos, sin = rope_tables(rope_len, dh, theta)
    return LayerWeights(shape, w_dkv, w_krope, w_uk, w_uv, pidx, torch.from_numpy(cos).to(device),
                        torch.from_numpy(sin).to(device))


@dataclass
class LatentCache:
    """Latent cache for `batch` sequences of up to t_max tokens (layouts of mla_cache).  For the windowed formats
    ckv_window is the bf16 ring of each sequence's last `window` rows, and ckv / ckv_scale hold the older rows'
    codes: 2-bit codes and (s, z) pairs per group of 32 ("int2_g32_win"), or int4 codes and fp16 scales
    ("int4_g32_win")."""

    shape: LayerShape
    ckv: torch.Tensor
    ckv_scale: Optional[torch.Tensor]
    krope: torch.Tensor
    batch: int
    t_max: int
    ckv_window: Optional[torch.Tensor] = None
    window: int = 0
    # paged caches: ckv / ckv_scale / krope are pools [n_pages, page_size, ...] and block_table [batch,
    # pages_per_seq] int32 maps sequence b's page j to a pool page
    block_table: Optional[torch.Tensor] = None
    page_size: int = 0
    n_pages: int = 0

    @staticmethod
    def allocate(shape: LayerShape, batch: int, t_max: int, device="cuda", fill: Optional[float] = None,
                 window: int = 128):
        """`window` (windowed formats only) is the number of recent rows kept in bf16 per sequence."""
        nr = shape.n_rope_heads * 2 * shape.r_pairs
        ring = None
        if shape.cache_fmt in ("int4_g32", "int4_g32_win"):
            ckv = torch.zeros((batch, t_max, shape.d_kv // 2), dtype=torch.uint8, device=device)
            scale = torch.zeros((batch, t_max, shape.d_kv // 32), dtype=torch.float16, device=device)
            if shape.cache_fmt == "int4_g32_win":
                ring = torch.empty((batch, max(window, 1), shape.d_kv), dtype=torch.bfloat16, device=device)
        elif shape.cache_fmt == "int2_g32_win":
            ckv = torch.zeros((batch, t_max, shape.d_kv // 4), dtype=torch.uint8, device=device)
            scale = torch.zeros((batch, t_max, shape.d_kv // 32, 2), dtype=torch.float16, device=device)
            ring = torch.empty((batch, max(window, 1), shape.d_kv), dtype=torch.bfloat16, device=device)
        else:
            ckv = torch.empty((batch, t_max, shape.d_kv), dtype=shape.torch_dtype, device=device)
            scale = None
        krope = torch.empty((batch, t_max, max(nr, 1)), dtype=shape.torch_dtype, device=device)
        if fill is not None:
            if scale is None:
                ckv.fill_(fill)
            if ring is not None:
                ring.fill_(fill)
            krope.fill_(fill)
        return LatentCache(shape, ckv, scale, krope, batch, t_max, ring,
                           window if shape.cache_fmt in WINDOWED else 0)

    @staticmethod
    def allocate_paged(shape: LayerShape, block_table: torch.Tensor, page_size: int, n_pages: int, device="cuda",
                       fill: Optional[float] = None, window: int = 128):
        """A paged cache: pools of n_pages pages of page_size rows and the page table block_table [batch,
        pages_per_seq] (int32, device); each sequence holds up to pages_per_seq * page_size tokens.  The windowed
        formats page their codes, scales and RoPE keys; the bf16 ring of each sequence's last `window` rows
        stays one block per sequence."""
        batch, pps = block_table.shape
        nr = shape.n_rope_heads * 2 * shape.r_pairs
        ring = None
        if shape.cache_fmt in ("int4_g32", "int4_g32_win"):
            ckv = torch.zeros((n_pages, page_size, shape.d_kv // 2), dtype=torch.uint8, device=device)
            scale = torch.zeros((n_pages, page_size, shape.d_kv // 32), dtype=torch.float16, device=device)
        elif shape.cache_fmt == "int2_g32_win":
            ckv = torch.zeros((n_pages, page_size, shape.d_kv // 4), dtype=torch.uint8, device=device)
            scale = torch.zeros((n_pages, page_size, shape.d_kv // 32, 2), dtype=torch.float16, device=device)
        else:
            ckv = torch.empty((n_pages, page_size, shape.d_kv), dtype=shape.torch_dtype, device=device)
            scale = None
        if shape.cache_fmt in WINDOWED:
            ring = torch.empty((batch, max(window, 1), shape.d_kv), dtype=torch.bfloat16, device=device)
        krope = torch.empty((n_pages, page_size, max(nr, 1)), dtype=shape.torch_dtype, device=device)
        if fill is not None:
            if scale is None:
                ckv.fill_(fill)
            if ring is not None:
                ring.fill_(fill)
            krope.fill_(fill)
        return LatentCache(shape, ckv, scale, krope, batch, pps * page_size, ring,
                           window if shape.cache_fmt in WINDOWED else 0,
                           block_table.to(device=device, dtype=torch.int32).contiguous(), page_size, n_pages)

    def view(self, b0: int, b1: int) -> "LatentCache":
        """The cache of sequences b0 .. b1-1 (views of the same memory; a paged cache keeps its pools and
        takes those sequences' page-table rows)."""
        sl = slice(b0, b1)
        if self.block_table is not None:
            return LatentCache(self.shape, self.ckv, self.ckv_scale, self.krope, b1 - b0, self.t_max,
                               None if self.ckv_window is None else self.ckv_window[sl], self.window,
                               self.block_table[sl], self.page_size, self.n_pages)
        return LatentCache(self.shape, self.ckv[sl], None if self.ckv_scale is None else self.ckv_scale[sl],
                           self.krope[sl], b1 - b0, self.t_max, None if self.ckv_window is None else self.ckv_window[sl],
                           self.window)

    def c(self) -> MlaCache:
        pps = 0 if self.block_table is None else self.block_table.shape[1]
        return MlaCache(_ptr(self.ckv), _ptr(self.ckv_scale), _ptr(self.krope), self.batch, self.t_max,
                        _ptr(self.ckv_window), self.window, _ptr(self.block_table), self.page_size, pps,
                        self.n_pages)

    def nbytes_per_token(self) -> int:
        """Bytes per cached position (the ring of a windowed cache is a fixed extra per sequence)."""
        n = self.ckv[0, 0].numel() * self.ckv.element_size() + self.krope[0, 0].numel() * self.krope.element_size()
        if self.ckv_scale is not None:
            n += self.ckv_scale[0, 0].numel() * 2
        return n


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _weight_specs(w: LayerWeights, cache: LatentCache):
    if w.shape != cache.shape:
        raise ValueError(f"weights are for {w.shape}, the cache for {cache.shape}")
    dev, s = cache.ckv.device, w.shape
    rope = (w.rope_cos.shape[0], s.d_head // 2)
    dn, nrh = s.d_head - 2 * s.r_pairs, s.n_rope_heads
    shapes = {"w_dkv": (s.d_kv, s.d_model), "w_krope": (nrh * 2 * s.r_pairs, s.d_model),
              "w_uk": (s.n_heads, dn, s.d_kv), "w_uv": (s.n_heads, s.d_head, s.d_kv)}
    return ([(getattr(w, n), n, s.torch_dtype, shp, dev) for n, shp in shapes.items()] +
            [(w.pair_idx, "pair_idx", torch.int32, (nrh, s.r_pairs), dev),
             (w.rope_cos, "rope_cos", torch.float32, rope, dev), (w.rope_sin, "rope_sin", torch.float32, rope, dev)])


def _append_specs(w: LayerWeights, cache: LatentCache, x, start_pos):
    if not isinstance(x, torch.Tensor) or x.dim() != 3:
        raise ValueError("x: expected a [batch, t_new, d_model] tensor")
    dev, s = cache.ckv.device, w.shape
    return [(x, "x", s.torch_dtype, (cache.batch, x.shape[1], s.d_model), dev),
            (start_pos, "start_pos", torch.int32, (cache.batch,), dev)]


def _decode_specs(w: LayerWeights, cache: LatentCache, q, seq_lens, out, q_len: Optional[int] = None):
    dev, s = cache.ckv.device, w.shape
    qs = (cache.batch, s.n_heads, s.d_head) if q_len is None else (cache.batch, q_len, s.n_heads, s.d_head)
    return [(q, "q", s.torch_dtype, qs, dev), (seq_lens, "seq_lens", torch.int32, (cache.batch,), dev),
            (out, "out", s.torch_dtype, qs, dev)]


def _check_append_args(w: LayerWeights, cache: LatentCache, x, start_pos) -> None:
    _expect(*_append_specs(w, cache, x, start_pos), *_weight_specs(w, cache))


def _check_decode_args(w: LayerWeights, cache: LatentCache, q, seq_lens, out, q_len: Optional[int] = None) -> None:
    _expect(*_decode_specs(w, cache, q, seq_lens, out, q_len), *_weight_specs(w, cache))


def _check_step_args(w: LayerWeights, cache: LatentCache, x, start_pos, q, seq_lens, out) -> None:
    _expect(*_append_specs(w, cache, x, start_pos), *_decode_specs(w, cache, q, seq_lens, out),
            *_weight_specs(w, cache))


def append(w: LayerWeights, cache: LatentCache, x: torch.Tensor, start_pos: torch.Tensor, max_start_pos: int,
           stream=None) -> None:
    """mla_cache_append: x [batch, t_new, d_model] at positions start_pos[b] + i."""
    _check_append_args(w, cache, x, start_pos)
    lib = _lib.load()
    cfg, cw, cc = w.shape.c(), w.c(), cache.c()
    t_new = x.shape[1]
    _check("mla_cache_append", lib.mla_cache_append(ctypes.byref(cfg), ctypes.byref(cw), ctypes.byref(cc), _ptr(x),
                                                    _ptr(start_pos), t_new, int(max_start_pos), _stream(stream)))


def append_workspace_bytes(shape: LayerShape, batch: int, t_new: int) -> int:
    cfg = shape.c()
    return _lib.load().mla_cache_append_workspace_bytes(ctypes.byref(cfg), batch, t_new)


def append_ws(w: LayerWeights, cache: LatentCache, x: torch.Tensor, start_pos: torch.Tensor, max_start_pos: int,
              workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """mla_cache_append_ws: the same append, with a workspace that spreads few-token appends over the GPU."""
    _check_append_args(w, cache, x, start_pos)
    lib = _lib.load()
    cfg, cw, cc = w.shape.c(), w.c(), cache.c()
    t_new = x.shape[1]
    need = lib.mla_cache_append_workspace_bytes(ctypes.byref(cfg), cache.batch, t_new)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if workspace is not None:
        _expect_ws(workspace, "workspace", need, x.device)
    _check("mla_cache_append_ws", lib.mla_cache_append_ws(
        ctypes.byref(cfg), ctypes.byref(cw), ctypes.byref(cc), _ptr(x), _ptr(start_pos), t_new, int(max_start_pos),
        _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(stream)))


def decode_workspace_bytes(shape: LayerShape, batch: int, max_seq_len: int) -> int:
    cfg = shape.c()
    return _lib.load().mla_decode_workspace_bytes(ctypes.byref(cfg), batch, max_seq_len)


def decode(w: LayerWeights, cache: LatentCache, q: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """mla_decode: q [batch, n_h, d_h] -> out [batch, n_h, d_h]."""
    if out is None and isinstance(q, torch.Tensor):
        out = torch.empty_like(q)
    _check_decode_args(w, cache, q, seq_lens, out)
    lib = _lib.load()
    cfg, cw, cc = w.shape.c(), w.c(), cache.c()
    nbytes = lib.mla_decode_workspace_bytes(ctypes.byref(cfg), cache.batch, int(max_seq_len))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _expect_ws(workspace, "workspace", nbytes, q.device)
    _check("mla_decode", lib.mla_decode(ctypes.byref(cfg), ctypes.byref(cw), ctypes.byref(cc), _ptr(q),
                                        _ptr(seq_lens), int(max_seq_len), _ptr(out), _ptr(workspace),
                                        workspace.numel(), _stream(stream)))
    return out


def decode_multi(w: LayerWeights, cache: LatentCache, q: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                 out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """mla_decode_multi: q [batch, q_len, n_h, d_h] (query i of sequence b at position L_b - q_len + i) -> out."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q: expected a [batch, q_len, n_heads, d_head] tensor")
    q_len = q.shape[1]
    if out is None:
        out = torch.empty_like(q)
    _check_decode_args(w, cache, q, seq_lens, out, q_len=q_len)
    lib = _lib.load()
    cfg, cw, cc = w.shape.c(), w.c(), cache.c()
    nbytes = lib.mla_decode_multi_workspace_bytes(ctypes.byref(cfg), cache.batch, q_len, int(max_seq_len))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _expect_ws(workspace, "workspace", nbytes, q.device)
    _check("mla_decode_multi", lib.mla_decode_multi(ctypes.byref(cfg), ctypes.byref(cw), ctypes.byref(cc), _ptr(q),
                                                    q_len, _ptr(seq_lens), int(max_seq_len), _ptr(out), _ptr(workspace),
                                                    workspace.numel(), _stream(stream)))
    return out


def decode_phase(phase: int, w: LayerWeights, cache: LatentCache, q: torch.Tensor, seq_lens: torch.Tensor,
                 max_seq_len: int, out: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    """mla_decode_phase: one of the three launches of mla_decode (1 q-prep, 2 attention, 3 combine)."""
    _check_decode_args(w, cache, q, seq_lens, out)
    lib = _lib.load()
    cfg, cw, cc = w.shape.c(), w.c(), cache.c()
    _check("mla_decode_phase", lib.mla_decode_phase(phase, ctypes.byref(cfg), ctypes.byref(cw), ctypes.byref(cc),
                                                    _ptr(q), _ptr(seq_lens), int(max_seq_len), _ptr(out),
                                                    _ptr(workspace), workspace.numel(), _stream(stream)))


def decode_step_workspace_bytes(shape: LayerShape, batch: int, t_new: int, max_seq_len: int) -> int:
    cfg = shape.c()
    return _lib.load().mla_decode_step_workspace_bytes(ctypes.byref(cfg), batch, t_new, max_seq_len)


def decode_step(w: LayerWeights, cache: LatentCache, x_new: torch.Tensor, start_pos: torch.Tensor, max_start_pos: int,
                q: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """mla_decode_step: append x_new [batch, t_new, d_model] at start_pos, then decode q -> out."""
    if out is None and isinstance(q, torch.Tensor):
        out = torch.empty_like(q)
    _check_step_args(w, cache, x_new, start_pos, q, seq_lens, out)
    lib = _lib.load()
    cfg, cw, cc = w.shape.c(), w.c(), cache.c()
    t_new = x_new.shape[1]
    nbytes = lib.mla_decode_step_workspace_bytes(ctypes.byref(cfg), cache.batch, t_new, int(max_seq_len))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _expect_ws(workspace, "workspace", nbytes, q.device)
    _check("mla_decode_step", lib.mla_decode_step(
        ctypes.byref(cfg), ctypes.byref(cw), ctypes.byref(cc), _ptr(x_new), _ptr(start_pos), t_new, int(max_start_pos),
        _ptr(q), _ptr(seq_lens), int(max_seq_len), _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


STATIC_SCRATCH_BYTES = 64 << 20  # MLA_STATIC_SCRATCH_BYTES


def decode_step_static(w: LayerWeights, cache: LatentCache, x_new: torch.Tensor, start_pos: torch.Tensor,
                       max_start_pos: int, q: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                       out: torch.Tensor, stream=None) -> torch.Tensor:
    """mla_decode_step_static: the decode step with the library's static per-GPU workspace (no workspace
    argument, no allocation in the call; `out` must be given)."""
    _check_step_args(w, cache, x_new, start_pos, q, seq_lens, out)
    lib = _lib.load()
    cfg, cw, cc = w.shape.c(), w.c(), cache.c()
    _check("mla_decode_step_static", lib.mla_decode_step_static(
        ctypes.byref(cfg), ctypes.byref(cw), ctypes.byref(cc), _ptr(x_new), _ptr(start_pos), x_new.shape[1],
        int(max_start_pos), _ptr(q), _ptr(seq_lens), int(max_seq_len), _ptr(out), _stream(stream)))
    return out


def prefill_workspace_bytes(shape: LayerShape, batch: int, seq_len: int) -> int:
    cfg = shape.c()
    return _lib.load().mla_prefill_workspace_bytes(ctypes.byref(cfg), batch, seq_len)


def prefill(w: LayerWeights, cache: LatentCache, q: torch.Tensor, out: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """mla_prefill: q [batch, S, n_h, d_h] at positions 0..S-1 -> out [batch, S, n_h, d_h]."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q: expected a [batch, seq_len, n_heads, d_head] tensor")
    seq_len = q.shape[1]
    s = w.shape
    qs = (cache.batch, seq_len, s.n_heads, s.d_head)
    if out is None:
        out = torch.empty_like(q)
    dev = cache.ckv.device
    _expect((q, "q", s.torch_dtype, qs, dev), (out, "out", s.torch_dtype, qs, dev), *_weight_specs(w, cache))
    lib = _lib.load()
    cfg, cw, cc = w.shape.c(), w.c(), cache.c()
    nbytes = lib.mla_prefill_workspace_bytes(ctypes.byref(cfg), cache.batch, seq_len)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _expect_ws(workspace, "workspace", nbytes, q.device)
    _check("mla_prefill", lib.mla_prefill(ctypes.byref(cfg), ctypes.byref(cw), ctypes.byref(cc), _ptr(q), seq_len,
                                          _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def quantize_int4(x: torch.Tensor, stream=None):
    """mla_quantize_int4 on fp32 x [..., 32*g] -> (codes uint8 [..., 16*g], scales float16 [..., g])."""
    if isinstance(x, torch.Tensor) and (x.dim() < 1 or x.shape[-1] % 32 != 0):
        raise ValueError("x: the last dim must be a multiple of 32")
    _expect((x, "x", torch.float32, None, None))
    lib = _lib.load()
    n_groups = x.numel() // 32
    codes = torch.empty(x.shape[:-1] + (x.shape[-1] // 2,), dtype=torch.uint8, device=x.device)
    scales = torch.empty(x.shape[:-1] + (x.shape[-1] // 32,), dtype=torch.float16, device=x.device)
    _check("mla_quantize_int4", lib.mla_quantize_int4(_ptr(x), n_groups, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def quantize_int2(x: torch.Tensor, stream=None):
    """mla_quantize_int2 on fp32 x [..., 32*g] -> (codes uint8 [..., 8*g], meta float16 [..., g, 2] = (s, z))."""
    if isinstance(x, torch.Tensor) and (x.dim() < 1 or x.shape[-1] % 32 != 0):
        raise ValueError("x: the last dim must be a multiple of 32")
    _expect((x, "x", torch.float32, None, None))
    lib = _lib.load()
    n_groups = x.numel() // 32
    codes = torch.empty(x.shape[:-1] + (x.shape[-1] // 4,), dtype=torch.uint8, device=x.device)
    meta = torch.empty(x.shape[:-1] + (x.shape[-1] // 32, 2), dtype=torch.float16, device=x.device)
    _check("mla_quantize_int2", lib.mla_quantize_int2(_ptr(x), n_groups, _ptr(codes), _ptr(meta), _stream(stream)))
    return codes, meta


class BoundDecode:
    """A decode step whose C structs are built once: append of the new token(s) (with its workspace)
    followed by the three decode launches, for serving loops and timing where per-call marshalling would
    dominate."""

    def __init__(self, w: LayerWeights, cache: LatentCache, x_new: torch.Tensor, start_pos: torch.Tensor,
                 max_start_pos: int, q: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                 out: torch.Tensor, workspace: Optional[torch.Tensor] = None):
        _check_step_args(w, cache, x_new, start_pos, q, seq_lens, out)
        self.lib = _lib.load()
        self.cfg, self.cw, self.cc = w.shape.c(), w.c(), cache.c()
        nbytes = self.lib.mla_decode_workspace_bytes(ctypes.byref(self.cfg), cache.batch, int(max_seq_len))
        if workspace is None:
            workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
        na = self.lib.mla_cache_append_workspace_bytes(ctypes.byref(self.cfg), cache.batch, x_new.shape[1])
        append_ws_buf = torch.empty(max(na, 16), dtype=torch.uint8, device=q.device)
        ns = self.lib.mla_decode_step_workspace_bytes(ctypes.byref(self.cfg), cache.batch, x_new.shape[1],
                                                      int(max_seq_len))
        step_ws = torch.empty(max(ns, 16), dtype=torch.uint8, device=q.device)
        self.args_step = (ctypes.byref(self.cfg), ctypes.byref(self.cw), ctypes.byref(self.cc), _ptr(x_new),
                          _ptr(start_pos), x_new.shape[1], int(max_start_pos), _ptr(q), _ptr(seq_lens),
                          int(max_seq_len), _ptr(out), _ptr(step_ws), step_ws.numel())
        self._keep = (w, cache, x_new, start_pos, q, seq_lens, out, append_ws_buf, step_ws, workspace)
        self.args_append = (ctypes.byref(self.cfg), ctypes.byref(self.cw), ctypes.byref(self.cc), _ptr(x_new),
                            _ptr(start_pos), x_new.shape[1], int(max_start_pos), _ptr(append_ws_buf),
                            append_ws_buf.numel())
        self.args_decode = (ctypes.byref(self.cfg), ctypes.byref(self.cw), ctypes.byref(self.cc), _ptr(q),
                            _ptr(seq_lens), int(max_seq_len), _ptr(out), _ptr(workspace), workspace.numel())
        self.out = out

    def append(self, stream=None):
        _check("mla_cache_append_ws", self.lib.mla_cache_append_ws(*self.args_append, _stream(stream)))

    def decode(self, stream=None):
        _check("mla_decode", self.lib.mla_decode(*self.args_decode, _stream(stream)))

    def step(self, stream=None):
        """mla_decode_step: the append and the decode in one call (prologue launches fused)."""
        _check("mla_decode_step", self.lib.mla_decode_step(*self.args_step, _stream(stream)))

    def phase(self, p: int, stream=None):
        _check("mla_decode_phase", self.lib.mla_decode_phase(p, *self.args_decode, _stream(stream)))

    def step_phase(self, p: int, stream=None):
        """mla_decode_step_phase: one of the step's three launches (1 append + q-prep, 2 attention with the
        append's reduction, 3 combine)."""
        _check("mla_decode_step_phase", self.lib.mla_decode_step_phase(p, *self.args_step, _stream(stream)))
