"""Host-only checks of the C ABI: the library loads, exports every function include/mla.h declares, sizes
workspaces, and rejects bad arguments before enqueueing anything (no GPU needed: every call here fails
validation, so no kernel is ever launched)."""

import ctypes
import os
import re

import pytest

from mla_latent_kv_cache_amd import _lib
from mla_latent_kv_cache_amd._lib import MlaCache, MlaConfig, MlaWeights

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mla.h")

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE, CAPACITY = 0, -1, -2, -3, -4, -5
FAKE = 0x10000  # a 16-byte aligned, non-null address that is never dereferenced (calls fail first)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*)\s*\*?\s*(mla_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert names, "no declarations parsed"
    assert set(names) == set(_lib.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def cfg(**kw):
    base = dict(d_model=4096, n_heads=32, d_head=128, r_pairs=4, d_kv=512, dtype=1, cache_fmt=0)
    base.update(kw)
    return MlaConfig(**base)


def weights(**kw):
    base = dict(w_dkv=FAKE, w_krope=FAKE, w_uk=FAKE, w_uv=FAKE, pair_idx=FAKE, rope_cos=FAKE, rope_sin=FAKE,
                rope_len=4096)
    base.update(kw)
    return MlaWeights(**base)


def cache(**kw):
    base = dict(ckv=FAKE, ckv_scale=FAKE, krope=FAKE, batch=32, t_max=4096, ckv_window=FAKE, window=128)
    base.update(kw)
    return MlaCache(**base)


def decode_call(lib, c=None, w=None, k=None, q=FAKE, lens=FAKE, max_len=4096, out=FAKE, ws=FAKE, ws_bytes=None):
    c = c or cfg()
    w = w or weights()
    k = k or cache()
    if ws_bytes is None:
        ws_bytes = lib.mla_decode_workspace_bytes(ctypes.byref(c), k.batch, max_len)
    return lib.mla_decode(ctypes.byref(c), ctypes.byref(w), ctypes.byref(k), q, lens, max_len, out, ws, ws_bytes, None)


def test_shared_rope_heads_accepted(lib):
    # 0 (one key head per query head) and every divisor of n_heads pass validation: the call then fails
    # only on the deliberately short workspace
    for nrh in (0, 1, 2, 8, 16, 32):
        assert decode_call(lib, c=cfg(rope_heads=nrh), ws_bytes=16) == WORKSPACE, nrh


def test_workspace_sizes(lib):
    c = cfg()
    n = lib.mla_decode_workspace_bytes(ctypes.byref(c), 32, 4096)
    # latent queries + rotated pairs + per-split (m, l) + per-split latent outputs
    assert n >= 32 * 32 * 512 * 2 + 32 * 32 * 512 * 4
    assert lib.mla_decode_workspace_bytes(ctypes.byref(c), 64, 4096) > n
    assert lib.mla_decode_workspace_bytes(ctypes.byref(c), 1, 1 << 20) > lib.mla_decode_workspace_bytes(ctypes.byref(c), 1, 4096)
    bad = cfg(d_head=7)
    assert lib.mla_decode_workspace_bytes(ctypes.byref(bad), 32, 4096) == 0
    assert lib.mla_decode_workspace_bytes(ctypes.byref(c), -1, 4096) == 0


@pytest.mark.parametrize(
    "kw,expected",
    [
        (dict(d_head=127), INVALID),
        (dict(r_pairs=65), INVALID),
        (dict(r_pairs=-1), INVALID),
        (dict(d_kv=0), INVALID),
        (dict(dtype=7), INVALID),
        (dict(cache_fmt=9), INVALID),
        (dict(d_head=512, r_pairs=4), UNSUPPORTED),
        (dict(cache_fmt=1, dtype=0), UNSUPPORTED),
        (dict(cache_fmt=1, d_kv=48), UNSUPPORTED),
        (dict(cache_fmt=2, dtype=0), UNSUPPORTED),
        (dict(cache_fmt=2, d_kv=48), UNSUPPORTED),
        (dict(cache_fmt=3, dtype=0), UNSUPPORTED),
        (dict(cache_fmt=3, d_kv=48), UNSUPPORTED),
        (dict(cache_fmt=4), INVALID),
        (dict(rope_heads=-1), INVALID),
        (dict(rope_heads=5), INVALID),  # not a divisor of the 32 query heads
        (dict(rope_heads=64), INVALID),
    ],
)
def test_decode_rejects_bad_config(lib, kw, expected):
    c = cfg(**kw)
    assert decode_call(lib, c=c, ws_bytes=1 << 40) == expected


def test_decode_rejects_bad_pointers_and_sizes(lib):
    assert decode_call(lib, q=None) == INVALID
    assert decode_call(lib, lens=None) == INVALID
    assert decode_call(lib, out=None) == INVALID
    assert decode_call(lib, q=FAKE + 4) == ALIGN
    assert decode_call(lib, w=weights(w_uv=None)) == INVALID
    assert decode_call(lib, w=weights(w_uk=FAKE + 2)) == ALIGN
    assert decode_call(lib, w=weights(rope_len=0)) == INVALID
    assert decode_call(lib, k=cache(ckv=None)) == INVALID
    assert decode_call(lib, k=cache(t_max=0)) == INVALID
    assert decode_call(lib, max_len=-1) == INVALID
    assert decode_call(lib, max_len=4097) == CAPACITY  # beyond t_max
    assert decode_call(lib, k=cache(t_max=8192), w=weights(rope_len=100), max_len=200) == CAPACITY
    assert decode_call(lib, ws=None) == WORKSPACE
    c = cfg()
    need = lib.mla_decode_workspace_bytes(ctypes.byref(c), 32, 4096)
    assert decode_call(lib, ws_bytes=need - 1) == WORKSPACE
    assert decode_call(lib, ws=FAKE + 8, ws_bytes=need) == ALIGN
    # int4 cache needs its scale buffer
    c4 = cfg(cache_fmt=1)
    assert decode_call(lib, c=c4, k=cache(ckv_scale=None), ws_bytes=1 << 40) == INVALID
    # the 2-bit cache needs its (s, z) buffer, a window >= 0 and, for a window > 0, the bf16 ring
    c2 = cfg(cache_fmt=2)
    assert decode_call(lib, c=c2, k=cache(ckv_scale=None), ws_bytes=1 << 40) == INVALID
    assert decode_call(lib, c=c2, k=cache(window=-1), ws_bytes=1 << 40) == INVALID
    assert decode_call(lib, c=c2, k=cache(ckv_window=None), ws_bytes=1 << 40) == INVALID
    assert decode_call(lib, c=c2, k=cache(ckv_window=FAKE + 2), ws_bytes=1 << 40) == ALIGN
    assert decode_call(lib, c=c2, k=cache(ckv_window=None, window=0), q=None, ws_bytes=1 << 40) == INVALID  # fails on q
    # the ring is not read for the other formats
    assert decode_call(lib, k=cache(ckv_window=None, window=-1), q=None) == INVALID  # fails on q
    # zero batch is a no-op
    assert decode_call(lib, k=cache(batch=0), q=None, lens=None, out=None) == OK


def test_append_checks(lib):
    c, w, k = cfg(), weights(), cache()

    def call(x=FAKE, sp=FAKE, t_new=1, max_start=4095, c=c, w=w, k=k):
        return lib.mla_cache_append(ctypes.byref(c), ctypes.byref(w), ctypes.byref(k), x, sp, t_new, max_start, None)

    assert call(t_new=2, max_start=4095) == CAPACITY
    assert call(x=None) == INVALID
    assert call(sp=FAKE + 1) == ALIGN
    assert call(t_new=-1) == INVALID
    assert call(max_start=-5) == INVALID
    assert call(w=weights(w_dkv=None)) == INVALID
    assert call(w=weights(w_krope=None)) == INVALID
    assert call(t_new=0, x=None, sp=None) == OK
    # no RoPE pairs: RoPE pointers may be absent
    c0 = cfg(r_pairs=0)
    w0 = weights(w_krope=None, pair_idx=None, rope_cos=None, rope_sin=None, rope_len=0)
    assert call(c=c0, w=w0, x=None) == INVALID  # fails on x, not on the absent RoPE pointers


def test_append_ws_checks(lib):
    c, w, k = cfg(), weights(), cache()
    need = lib.mla_cache_append_workspace_bytes(ctypes.byref(c), 32, 1)
    assert need > 0  # a few-token append on this shape splits the model width
    assert lib.mla_cache_append_workspace_bytes(ctypes.byref(c), 32, 4096) == 0  # large appends need none
    assert lib.mla_cache_append_workspace_bytes(ctypes.byref(cfg(dtype=0)), 32, 1) == 0

    def call(ws=FAKE, nbytes=need):
        return lib.mla_cache_append_ws(ctypes.byref(c), ctypes.byref(w), ctypes.byref(k), FAKE, FAKE, 1, 4095, ws,
                                       nbytes, None)

    assert call(ws=None) == WORKSPACE
    assert call(nbytes=need - 1) == WORKSPACE
    assert call(ws=FAKE + 4) == ALIGN


def test_decode_step_checks(lib):
    c, w, k = cfg(), weights(), cache()
    na = lib.mla_cache_append_workspace_bytes(ctypes.byref(c), 32, 1)
    nd = lib.mla_decode_workspace_bytes(ctypes.byref(c), 32, 4096)
    need = lib.mla_decode_step_workspace_bytes(ctypes.byref(c), 32, 1, 4096)
    assert need == ((na + 255) // 256) * 256 + nd  # the append's partial sums, then the decode workspace
    assert lib.mla_decode_step_workspace_bytes(ctypes.byref(c), -1, 1, 4096) == 0
    assert lib.mla_decode_step_workspace_bytes(ctypes.byref(cfg(d_kv=0)), 32, 1, 4096) == 0

    def call(x=FAKE, sp=FAKE, t_new=1, max_start=4095, q=FAKE, lens=FAKE, max_len=4096, out=FAKE, ws=FAKE,
             nbytes=need, c=c, w=w, k=k):
        return lib.mla_decode_step(ctypes.byref(c), ctypes.byref(w), ctypes.byref(k), x, sp, t_new, max_start, q, lens,
                                   max_len, out, ws, nbytes, None)

    assert call(ws=None) == WORKSPACE
    assert call(nbytes=need - 1) == WORKSPACE
    assert call(ws=FAKE + 4) == ALIGN
    assert call(x=None) == INVALID
    assert call(q=None) == INVALID
    assert call(lens=None) == INVALID
    assert call(out=FAKE + 2) == ALIGN
    assert call(t_new=2, max_start=4095) == CAPACITY
    assert call(max_len=4097) == CAPACITY
    assert call(t_new=-1) == INVALID
    assert call(w=weights(w_dkv=None)) == INVALID  # the append half needs the down-projection
    assert call(w=weights(w_uv=None)) == INVALID   # the decode half needs the up-projection
    assert call(k=cache(batch=0), x=None, q=None, lens=None, out=None, ws=None) == OK


def test_prefill_checks(lib):
    c, w, k = cfg(), weights(), cache()

    def call(q=FAKE, s=4096, out=FAKE, ws=FAKE, nbytes=1 << 40, c=c, k=k):
        return lib.mla_prefill(ctypes.byref(c), ctypes.byref(w), ctypes.byref(k), q, s, out, ws, nbytes, None)

    assert call(c=cfg(dtype=0)) == UNSUPPORTED
    assert call(c=cfg(d_head=64)) == UNSUPPORTED
    assert call(s=-1) == INVALID
    # quantised latents are accepted; their workspace also holds the dequantised latent rows [batch, S, d_kv]
    dense = lib.mla_prefill_workspace_bytes(ctypes.byref(c), 4, 4096)
    for fmt in (1, 2):
        cq = cfg(cache_fmt=fmt)
        need = lib.mla_prefill_workspace_bytes(ctypes.byref(cq), 4, 4096)
        assert need == dense + 4 * 4096 * 512 * 2
        assert call(c=cq, k=cache(batch=4), nbytes=need - 1) == WORKSPACE
    assert call(c=cfg(cache_fmt=1), k=cache(batch=4, ckv_scale=None), nbytes=1 << 40) == INVALID


def test_quantize_checks(lib):
    assert lib.mla_quantize_int4(FAKE, -1, FAKE, FAKE, None) == INVALID
    assert lib.mla_quantize_int4(None, 4, FAKE, FAKE, None) == INVALID
    assert lib.mla_quantize_int4(FAKE, 4, FAKE + 1, FAKE, None) == ALIGN
    assert lib.mla_quantize_int4(None, 0, None, None, None) == OK
    assert lib.mla_quantize_int2(FAKE, -1, FAKE, FAKE, None) == INVALID
    assert lib.mla_quantize_int2(FAKE, 4, None, FAKE, None) == INVALID
    assert lib.mla_quantize_int2(FAKE, 4, FAKE, FAKE + 2, None) == ALIGN
    assert lib.mla_quantize_int2(None, 0, None, None, None) == OK


def test_window_format_workspace(lib):
    """The 2-bit format's window rides on each sequence's last work item, so it needs no more split
    results than the int4 format."""
    for batch, ctx in ((64, 8192), (1, 100), (8, 32768)):
        n1 = lib.mla_decode_workspace_bytes(ctypes.byref(cfg(cache_fmt=1)), batch, ctx)
        n2 = lib.mla_decode_workspace_bytes(ctypes.byref(cfg(cache_fmt=2)), batch, ctx)
        assert n2 == n1 > 0


def test_status_strings(lib):
    for s in range(-6, 1):
        assert lib.mla_status_string(s)
    assert lib.mla_status_string(-99) == b"unknown status"


def test_paged_cache_checks(lib):
    """A paged cache: page size a multiple of 64, t_max = pages_per_seq * page_size, a 4-byte aligned table,
    a pool of at most 2^31 - 1 rows, any latent format."""
    def paged(**kw):
        base = dict(block_table=FAKE, page_size=64, pages_per_seq=64, n_pages=2048, t_max=4096)
        base.update(kw)
        return cache(**base)

    big = 1 << 40
    assert decode_call(lib, k=paged(page_size=32, t_max=2048), ws_bytes=big, q=None) == INVALID
    assert decode_call(lib, k=paged(t_max=4000), ws_bytes=big, max_len=4000, q=None) == INVALID
    assert decode_call(lib, k=paged(pages_per_seq=0), ws_bytes=big, q=None) == INVALID
    assert decode_call(lib, k=paged(n_pages=0), ws_bytes=big, q=None) == INVALID
    assert decode_call(lib, k=paged(block_table=FAKE + 2), ws_bytes=big) == ALIGN
    assert decode_call(lib, k=paged(block_table=FAKE + 4), ws_bytes=big, q=None) == INVALID  # 4-byte aligned is fine
    assert decode_call(lib, k=paged(n_pages=1 << 26), ws_bytes=big) == UNSUPPORTED
    # the windowed formats page their codes too: such a cache passes the cache checks and the call stops at the
    # missing query pointer
    assert decode_call(lib, c=cfg(cache_fmt=2), k=paged(), ws_bytes=big, q=None) == INVALID
    assert decode_call(lib, c=cfg(cache_fmt=3), k=paged(), ws_bytes=big, q=None) == INVALID
    # a contiguous cache with more than 2^31 - 1 rows
    assert decode_call(lib, k=cache(batch=1 << 17, t_max=1 << 15), max_len=1, ws_bytes=big) == UNSUPPORTED


def test_decode_multi_checks(lib):
    c, w, k = cfg(), weights(), cache()
    n1 = lib.mla_decode_workspace_bytes(ctypes.byref(c), 32 * 4, 4096)
    assert lib.mla_decode_multi_workspace_bytes(ctypes.byref(c), 32, 4, 4096) == n1  # 4 queries = 4x the sequences
    assert lib.mla_decode_multi_workspace_bytes(ctypes.byref(c), 32, 0, 4096) == 0

    def call(q=FAKE, q_len=4, lens=FAKE, out=FAKE, ws=FAKE, nbytes=n1, c=c, k=k):
        return lib.mla_decode_multi(ctypes.byref(c), ctypes.byref(w), ctypes.byref(k), q, q_len, lens, 4096, out, ws,
                                    nbytes, None)

    assert call(q_len=0) == INVALID
    assert call(q=None) == INVALID
    assert call(nbytes=n1 - 1) == WORKSPACE
    # windowed formats take several queries too: the call passes the format checks and stops at the query
    assert call(c=cfg(cache_fmt=2), nbytes=1 << 40, q=None) == INVALID
    assert call(k=cache(batch=0), q=None, lens=None, out=None) == OK


def test_static_step_rejects_oversized_request_on_the_host(lib):
    """mla_decode_step_static refuses a step whose workspace exceeds its static buffer before touching the
    device (here there is none): 256 sequences x 4096 positions of the Llama-2-7B-shaped layer."""
    c, w, k = cfg(), weights(), cache(batch=256)
    assert lib.mla_decode_step_workspace_bytes(ctypes.byref(c), 256, 1, 4096) > (64 << 20)
    rc = lib.mla_decode_step_static(ctypes.byref(c), ctypes.byref(w), ctypes.byref(k), FAKE, FAKE, 1, 4095, FAKE,
                                    FAKE, 4096, FAKE, None)
    assert rc == WORKSPACE
    # invalid arguments are reported as for mla_decode_step, before the size
    assert lib.mla_decode_step_static(ctypes.byref(cfg(d_head=7)), ctypes.byref(w), ctypes.byref(k), FAKE, FAKE, 1,
                                      4095, FAKE, FAKE, 4096, FAKE, None) == INVALID


def test_rope_tables_through_the_abi(lib):
    """mla_rope_tables fills host buffers with cos / sin of pos * theta^(-2p/d_head) rounded to fp32: within
    half an fp32 step of the fp64 values (a value in [-1, 1] rounds by at most 2^-25), exactly cos 0 = 1 and
    sin 0 = 0 at position 0 and subspace 0 turning by one radian per position."""
    import numpy as np

    L, dh, theta = 300, 64, 1e4
    cos = np.full((L, dh // 2), np.nan, dtype=np.float32)
    sin = np.full_like(cos, np.nan)
    assert lib.mla_rope_tables(L, dh, theta, cos.ctypes.data, sin.ctypes.data) == OK
    ang = np.arange(L)[:, None] * theta ** (-2.0 * np.arange(dh // 2) / dh)
    assert np.max(np.abs(cos - np.cos(ang))) <= 2.0 ** -25 * (1 + 1e-9)
    assert np.max(np.abs(sin - np.sin(ang))) <= 2.0 ** -25 * (1 + 1e-9)
    assert np.all(cos[0] == 1.0) and np.all(sin[0] == 0.0)
    assert np.all(cos[:, 0] == np.cos(np.arange(L)).astype(np.float32))
    # the binding's tables are the library's
    from mla_latent_kv_cache_amd import rope_tables

    c2, s2 = rope_tables(L, dh, theta)
    assert np.array_equal(c2, cos) and np.array_equal(s2, sin)
    for args in ((-1, dh, theta), (L, 7, theta), (L, 0, theta), (L, dh, 0.0), (L, dh, float("inf"))):
        assert lib.mla_rope_tables(*args, cos.ctypes.data, sin.ctypes.data) == INVALID
    assert lib.mla_rope_tables(L, dh, theta, None, sin.ctypes.data) == INVALID
    assert lib.mla_rope_tables(0, dh, theta, None, None) == OK


def test_decode_step_phase_rejects_bad_phase(lib):
    c, w, k = cfg(), weights(), cache()
    ws = lib.mla_decode_step_workspace_bytes(ctypes.byref(c), 32, 1, 4096)
    for phase in (0, 4, -1):
        assert lib.mla_decode_step_phase(phase, ctypes.byref(c), ctypes.byref(w), ctypes.byref(k), FAKE, FAKE, 1, 4095,
                                         FAKE, FAKE, 4096, FAKE, FAKE, ws, None) == INVALID
    # argument errors as for mla_decode_step
    assert lib.mla_decode_step_phase(1, ctypes.byref(c), ctypes.byref(w), ctypes.byref(k), FAKE, FAKE, 1, 4095,
                                     FAKE, FAKE, 4096, FAKE, FAKE, ws - 16, None) == WORKSPACE
