"""The Python binding rejects tensors of the wrong dtype, shape or device with ValueError before any library
call (the library reads raw device pointers: an int64 length array would be read as int32 halves, a short
activation buffer read past its end, a host tensor faulted on).  Runs without a GPU: every case fails in the
binding's checks."""

import numpy as np
import pytest
import torch

from mla_latent_kv_cache_amd import (LatentCache, LayerShape, append, append_ws, decode, decode_multi, decode_step,
                                     pack_weights, prefill, quantize_int2, quantize_int4)

SHAPE = LayerShape(64, 2, 16, 2, 32, "bf16", "dense")


def _layer(shape=SHAPE):
    rng = np.random.default_rng(0)
    d, n_h, d_h, r, D = shape.d_model, shape.n_heads, shape.d_head, shape.r_pairs, shape.d_kv
    conv = {"w_dkv": rng.standard_normal((d, D)), "w_krope": rng.standard_normal((d, n_h * 2 * r)),
            "w_uk": rng.standard_normal((n_h, D, d_h - 2 * r)), "w_uv": rng.standard_normal((n_h, D, d_h)),
            "pair_idx": np.tile(np.arange(r), (n_h, 1))}
    w = pack_weights(shape, conv, rope_len=16, device="cpu")
    cache = LatentCache.allocate(shape, 3, 16, device="cpu")
    return w, cache


def _q(B=3):
    return torch.zeros((B, SHAPE.n_heads, SHAPE.d_head), dtype=torch.bfloat16)


def test_int64_lengths_rejected():
    w, cache = _layer()
    with pytest.raises(ValueError, match="seq_lens: dtype"):
        decode(w, cache, _q(), torch.tensor([4, 4, 4]), 4)  # torch.tensor defaults to int64
    with pytest.raises(ValueError, match="start_pos: dtype"):
        append(w, cache, torch.zeros((3, 1, 64), dtype=torch.bfloat16), torch.tensor([0, 0, 0]), 0)


def test_wrong_shapes_rejected():
    w, cache = _layer()
    lens = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError, match="x: shape"):
        append(w, cache, torch.zeros((2, 1, 64), dtype=torch.bfloat16), lens, 0)  # fewer rows than the cache
    with pytest.raises(ValueError, match="x: shape"):
        append_ws(w, cache, torch.zeros((3, 1, 32), dtype=torch.bfloat16), lens, 0)
    with pytest.raises(ValueError, match="seq_lens: shape"):
        decode(w, cache, _q(), torch.zeros(2, dtype=torch.int32), 4)
    with pytest.raises(ValueError, match="q: shape"):
        decode(w, cache, _q(2), lens, 4)
    with pytest.raises(ValueError, match="out: shape"):
        decode(w, cache, _q(), lens, 4, out=_q(2))
    with pytest.raises(ValueError, match="q: shape"):
        prefill(w, cache, torch.zeros((3, 5, 2, 8), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="q: expected"):
        decode_multi(w, cache, _q(), lens, 4)


def test_wrong_dtypes_rejected():
    w, cache = _layer()
    lens = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError, match="q: dtype"):
        decode(w, cache, _q().float(), lens, 4)  # an fp32 query under a bf16 layer
    with pytest.raises(ValueError, match="x: dtype"):
        decode_step(w, cache, torch.zeros((3, 1, 64)), lens, 0, _q(), lens, 4)
    with pytest.raises(ValueError, match="x: dtype"):
        quantize_int4(torch.zeros((4, 32), dtype=torch.float64))
    with pytest.raises(ValueError, match="multiple of 32"):
        quantize_int2(torch.zeros((4, 30), dtype=torch.float32))


def test_host_tensors_rejected():
    """Correct dtypes and shapes but host memory: rejected, never handed to a kernel."""
    w, cache = _layer()
    lens = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensors"):
        decode(w, cache, _q(), lens, 4)
    with pytest.raises(ValueError, match="GPU tensors"):
        append(w, cache, torch.zeros((3, 1, 64), dtype=torch.bfloat16), lens, 0)
    with pytest.raises(ValueError, match="GPU tensors"):
        quantize_int4(torch.zeros((4, 32), dtype=torch.float32))
