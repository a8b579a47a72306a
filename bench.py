#!/usr/bin/env python3
"""Throughput of the MHA2MLA latent-cache hot path on one MI355X (gfx950).

One step of the headline workload (Llama-2-7B-shaped layer, bf16, d_kv 512, r 4, batch 32, every
sequence at context 4096) is one decode step of serving, mla_decode_step: the append of the new token of
every sequence (position 4095) and the decode over the 4096 cached tokens.  `value` is the latent-cache
bytes one decode must read (batch x context x bytes per cache row) divided by the step time.

Timing: inputs are resident in HBM before the timed region; three independent cache copies are used in
rotation so that the 256 MB last-level cache cannot serve a step's reads from the previous step.  Each copy's
step is captured in a HIP graph (the library records no memset), and a graph of 10 consecutive steps over the
copies is replayed `max(50, --steps)` times after `--warmup` replays, each replay bracketed by HIP events on the
launch stream: ms_per_step is the median replay time / 10.  One step alone (a single-step graph, the graph
launch included) and the mean of `--steps` eager back-to-back steps are reported beside it; a graph's first
replay is checked bit for bit against the eager step.

The roofline object is the step's dominant launch, the split-K attention with the append's reduction inside
it (phase 2 of mla_decode_step), timed as `--steps` back-to-back launches between two HIP events; the same
attention without the append (phase 2 of mla_decode) and the whole step's fraction are given beside it, and the
rate of an in-tree streaming-read kernel over a 2 GiB buffer (libmla_bandwidth.so, the practical HBM ceiling).

The cpu_baseline object times the oracle (plain fp64 numpy; the library never uses it) on the host's cores:
its conversion of the layer, then the cache fill + unabsorbed decode of whole sequences of the same workload
(a bounded sample), each timed apart.  Secondary workloads (long-context variable-length decode, int4-latent
decode, 2-bit- and int4-latent decode with a 128-row bf16 window, the headline decode on a paged cache of
64-token pages in random order, a 4-query multi-query decode, a grouped-query source whose RoPE keys are
stored once per KV head, the headline layer at the shape of the pages' LongBench runs (batch 16 x 2048
tokens), causal prefill) are reported in `secondary`.

`roofline.traffic` is the HBM traffic of one launch of that kernel from FETCH_SIZE / WRITE_SIZE counter
runs (profiles/pmc_traffic.json, scaled by the counters of a plain copy of known size, see
--copy-calibration); it is null when those counters were taken on different decode sources.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--only bw,c1,c3,c4,c5,c8,c6,c7,c9,c10,c2] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode latent-cache GB/s (% of HBM peak); prefill MFMA TFLOP/s"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure (no sparsity)
DOMINANT_KERNEL = "decode_attn_dma<128, 8, 3, false, false>"
FUSED_KEY = DOMINANT_KERNEL + " in mla_decode_step"  # the same kernel launched with the append's reduction


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", default="bw,c1,c3,c4,c5,c8,c6,c7,c9,c10,c2")
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--replays", type=int, default=50, help="graph replays the median step time is taken over (>= 50 "
                                                             "for a reported figure; fewer for profiler runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 10 plain device copies of 256 MiB (reference kernel for byte counters)")
    return ap.parse_args()


# ---------------------------------------------------------------- traffic from byte counters

DECODE_SOURCES = ("mla_latent_kv_cache_amd/csrc/decode.hip", "mla_latent_kv_cache_amd/csrc/common.h",
                  "mla_latent_kv_cache_amd/csrc/kernels.h", "mla_latent_kv_cache_amd/csrc/step.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")


def decode_source_digest():
    import hashlib

    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed byte-counter summary, or None when the summary is
    missing or was taken on other kernel sources (the digest of the decode sources no longer matches)."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != decode_source_digest():
        return None
    return int(rec["traffic_bytes"])


def copy_calibration():
    """A plain device-to-device copy of known size: the byte counters of this kernel give the scale
    factors between FETCH_SIZE / WRITE_SIZE and the bytes actually moved."""
    import torch

    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: 10 copies of {n} bytes")
    del src, dst


def stream_read_ceiling(reps=10, nbytes=2 << 30):
    """The best rate of the in-tree streaming-read kernels (libmla_bandwidth.so: 16-byte loads, grid-stride, or
    1 KB direct-to-LDS requests with the non-temporal hint; nothing written) over launch shapes, reading a 2 GiB
    buffer (far past the 256 MB last-level cache): the practical ceiling of a kernel that reads HBM once,
    reported beside the vendor peak."""
    import ctypes

    import torch

    from mla_latent_kv_cache_amd import build as _b

    lib = ctypes.CDLL(_b.BW_LIB)
    lib.mla_bw_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_void_p]
    lib.mla_bw_stream_read.restype = ctypes.c_int
    lib.mla_bw_stream_dma.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p]
    lib.mla_bw_stream_dma.restype = ctypes.c_int
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").random_()
    shapes = [(256 * k, u, nt) for k in (1, 4, 8, 16, 32) for u in (2, 4, 8) for nt in (0, 1)]
    # LDS DMA with the non-temporal hint (the decode kernels' load path): one workgroup of 4 waves per CU
    shapes += [(256, f, "dma") for f in (4, 8, 16)]
    sink = torch.zeros(max(b for b, _, _ in shapes), dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch(b, u, nt):
        if nt == "dma":
            rc = lib.mla_bw_stream_dma(src.data_ptr(), nbytes // 1024, sink.data_ptr(), b, u, stream)
        else:
            rc = lib.mla_bw_stream_read(src.data_ptr(), nbytes // 16, sink.data_ptr(), b, u, nt, stream)
        if rc != 0:
            raise RuntimeError(f"mla_bw_stream_read failed ({rc})")

    best = (0.0, None)
    for b, u, nt in shapes:
        for _ in range(2):
            launch(b, u, nt)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            launch(b, u, nt)
        t1.record()
        torch.cuda.synchronize()
        gbs = nbytes * reps / (t0.elapsed_time(t1) * 1e-3) / 1e9
        if gbs > best[0]:
            best = (gbs, dict(workgroups=b, loads_in_flight=u, nontemporal=True, lds_dma=True) if nt == "dma" else
                    dict(workgroups=b, loads_in_flight=u, nontemporal=bool(nt), lds_dma=False))
    del src, sink
    torch.cuda.empty_cache()
    log(f"[bench] streaming-read ceiling: {best[0]:.0f} GB/s ({100 * best[0] / HBM_PEAK_GBS:.1f}% of {HBM_PEAK_GBS:.0f}) "
        f"at {best[1]}")
    return {"gbs": round(best[0], 1), "frac_of_peak": round(best[0] / HBM_PEAK_GBS, 4), "bytes": nbytes,
            "launch": best[1], "kernel": "stream_dma (libmla_bandwidth.so)" if best[1].get("lds_dma") else "stream_read (libmla_bandwidth.so)"}


# ---------------------------------------------------------------- workloads

def converted(family, r, d_kv):
    import synth
    from mla_latent_kv_cache_amd import convert_layer

    d, n_h, d_h, _ = synth.FAMILIES[family]
    wq, wk, wv, xc = synth.layer_weights(family)
    t = time.time()
    conv = convert_layer(wq, wk, wv, xc, n_h, d_h, r, d_kv)
    log(f"[bench] converted {family} r={r} d_kv={d_kv} in {time.time() - t:.1f}s")
    conv["w_q"] = wq
    return conv


def converted_gqa(family, r, d_kv):
    """The library converter on a seeded grouped-query layer (synth.GQA_FAMILIES), RoPE part kept per KV head."""
    import synth
    from mla_latent_kv_cache_amd import convert_layer

    d, n_h, n_kv, d_h, _ = synth.GQA_FAMILIES[family]
    wq, wk, wv, xc = synth.gqa_layer_weights(family)
    t = time.time()
    conv = convert_layer(wq, wk, wv, xc, n_h, d_h, r, d_kv, n_kv_heads=n_kv, compact_rope=True)
    log(f"[bench] converted {family} (GQA, {n_kv} KV heads) r={r} d_kv={d_kv} in {time.time() - t:.1f}s")
    conv["w_q"] = wq
    return conv


def make_decode_workload(cfg, conv, lens, copies, seed, page_size=0, rope_heads=0):
    """Weights, `copies` filled caches (through mla_cache_append), the step's new-token activations, queries
    and one BoundDecode per copy.  Activations are seeded N(0,1) generated on the device.  page_size > 0:
    paged caches whose pages are a random permutation of the pool; rope_heads > 0: RoPE keys stored per key
    head (LayerShape.rope_heads)."""
    import torch

    from mla_latent_kv_cache_amd import BoundDecode, LatentCache, LayerShape, append, pack_weights

    shape = LayerShape(cfg.d_model, cfg.n_heads, cfg.d_head, cfg.r_pairs, cfg.d_kv, cfg.dtype, cfg.cache_fmt,
                       rope_heads=rope_heads)
    B = len(lens)
    t_max = int(max(lens))
    w = pack_weights(shape, conv, rope_len=t_max, theta=cfg.theta)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    caches = []
    for c in range(copies):
        if page_size:
            pps = (t_max + page_size - 1) // page_size
            perm = torch.randperm(B * pps, generator=g, device="cuda").to(torch.int32).reshape(B, pps)
            cache = LatentCache.allocate_paged(shape, perm, page_size, B * pps)
        else:
            cache = LatentCache.allocate(shape, B, t_max)
        for b in range(B):
            L = int(lens[b])
            x = torch.randn((1, L, cfg.d_model), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
            view = cache.view(b, b + 1)
            append(w, view, x, torch.zeros(1, dtype=torch.int32, device="cuda"), 0)
            del x
        caches.append(cache)
    torch.cuda.synchronize()
    x_new = torch.randn((B, 1, cfg.d_model), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    wq = torch.from_numpy(conv["w_q"].astype(np.float32)).cuda()
    q = (x_new[:, 0].float() @ wq).to(torch.bfloat16).reshape(B, cfg.n_heads, cfg.d_head).contiguous()
    del wq
    lens_t = torch.tensor(np.asarray(lens, dtype=np.int32), device="cuda")
    start = (lens_t - 1).contiguous()
    out = torch.empty_like(q)
    ws = None
    bound = []
    for cache in caches:
        bd = BoundDecode(w, cache, x_new, start, t_max - 1, q, lens_t, t_max, out, ws)
        ws = bd._keep[-1]
        bound.append(bd)
    bytes_per_row = caches[0].nbytes_per_token()
    total = bytes_per_row * int(np.sum(lens))
    if caches[0].window:
        # the last min(L, W) rows of each sequence are read from the bf16 ring instead of the code store
        ring_row = cfg.d_kv * 2
        code_row = caches[0].ckv[0, 0].numel() + caches[0].ckv_scale[0, 0].numel() * 2
        total += sum(min(int(L), caches[0].window) for L in lens) * (ring_row - code_row)
    return dict(w=w, caches=caches, bound=bound, lens=lens, bytes=int(total), bytes_per_row=bytes_per_row)


STEPS_PER_GRAPH = 10


def capture_steps(bound, check=True):
    """HIP graphs of the decode step (mla_decode_step: its three launches; the library records no memset):
    one single-step graph per cache copy, and one graph of STEPS_PER_GRAPH consecutive steps rotating over the
    copies.  With `check`, the first replay of each is compared bit for bit with the same step run eagerly
    (not for the windowed 2-bit cache, whose step is not idempotent: a repeated step re-codes the row that
    left the window from a ring slot the first run has already overwritten)."""
    import torch

    out = bound[0].out
    n = len(bound)

    def checked(g, bd):
        if not check:
            return
        bd.step()
        torch.cuda.synchronize()
        ref = out.clone()
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, ref):
            raise RuntimeError("a graph replay of the decode step differs from the eager step")

    single = []
    for bd in bound:
        bd.step()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            bd.step()
        checked(g, bd)
        single.append(g)
    multi = torch.cuda.CUDAGraph()
    with torch.cuda.graph(multi):
        for i in range(STEPS_PER_GRAPH):
            bound[i % n].step()
    checked(multi, bound[(STEPS_PER_GRAPH - 1) % n])
    return single, multi


def median_replay_ms(graphs, replays, warmup):
    """Median over `replays` graph replays (rotating over `graphs`) of each replay's own duration, bracketed by
    HIP events on the launch stream."""
    import torch

    n = len(graphs)
    for i in range(warmup):
        graphs[i % n].replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(replays)]
    for i, (e0, e1) in enumerate(ev):
        e0.record()
        graphs[i % n].replay()
        e1.record()
    torch.cuda.synchronize()
    return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))


REPLAYS = 50


def time_decode(wl, steps, warmup, check=True):
    """Step time: the median over >= 50 replays of a graph of STEPS_PER_GRAPH consecutive steps, per step;
    the median of single-step graph replays (one step in isolation, the graph launch included); the mean of
    `steps` back-to-back eager steps; and the attention kernel's average launch duration."""
    import torch

    bound = wl["bound"]
    n = len(bound)
    single, multi = capture_steps(bound, check)
    step_ms = median_replay_ms([multi], max(REPLAYS, steps), warmup) / STEPS_PER_GRAPH
    lat_ms = median_replay_ms(single, max(REPLAYS, steps), warmup)
    del single, multi
    for i in range(warmup):
        bound[i % n].step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        bound[i % n].step()
    t1.record()
    torch.cuda.synchronize()
    eager_ms = t0.elapsed_time(t1) / steps
    # the step's attention launch (phase 2 of mla_decode_step: the split-K attention with the append's reduction
    # inside it): phase 1 once per copy, then back-to-back launches of phase 2 over the rotating copies,
    # bracketed by two events on the launch stream (repeating it rewrites the same rows with the same values)
    fused_ms = None
    if check:
        for i in range(n):
            bound[i].step_phase(1)
        fused_ms = _time_launches(lambda i: bound[i % n].step_phase(2), steps, warmup)
    # the attention alone (phase 2 of mla_decode), the same way
    for i in range(n):
        bound[i].phase(1)
    k_ms = _time_launches(lambda i: bound[i % n].phase(2), steps, warmup)
    return dict(step_ms=step_ms, latency_ms=lat_ms, eager_ms=eager_ms, kernel_ms=k_ms, fused_ms=fused_ms)


def _time_launches(launch, steps, warmup):
    import torch

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record()
    for i in range(steps):
        launch(i)
    k1.record()
    torch.cuda.synchronize()
    return k0.elapsed_time(k1) / steps


def multi_query_result(cfg, wl, q_len, steps, warmup):
    """mla_decode_multi with q_len queries per sequence over the workload's caches (rotating copies), each
    query causal: whole-call time (q-prep, attention, combine) and the cache bytes it covers once."""
    import torch

    from mla_latent_kv_cache_amd import decode_multi, decode_workspace_bytes

    B = len(wl["lens"])
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    q = (torch.randn((B, q_len, cfg.n_heads, cfg.d_head), generator=g, device="cuda") * 2).to(torch.bfloat16)
    lens_t = torch.tensor(np.asarray(wl["lens"], dtype=np.int32), device="cuda")
    t_max = int(max(wl["lens"]))
    out = torch.empty_like(q)
    ws = torch.empty(decode_workspace_bytes(wl["w"].shape, B * q_len, t_max), dtype=torch.uint8, device="cuda")
    n = len(wl["caches"])
    for i in range(warmup):
        decode_multi(wl["w"], wl["caches"][i % n], q, lens_t, t_max, out=out, workspace=ws)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        decode_multi(wl["w"], wl["caches"][i % n], q, lens_t, t_max, out=out, workspace=ws)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    gbs = wl["bytes"] / (ms * 1e-3) / 1e9
    log(f"[bench] multi-query decode, {q_len} queries x {B} sequences: {ms * 1e3:.1f} us per call -> {gbs:.0f} GB/s "
        f"of cache covered once ({q_len * B / (ms * 1e-3):.0f} queries/s)")
    return dict(call_ms=ms, q_len=q_len, gbs_cache_once=gbs, queries_per_s=q_len * B / (ms * 1e-3), bytes=wl["bytes"])


def decode_result(name, cfg, wl, steps, warmup, check=True):
    t = time_decode(wl, steps, warmup, check)
    step_ms, k_ms, f_ms = t["step_ms"], t["kernel_ms"], t["fused_ms"]
    gbs = wl["bytes"] / (step_ms * 1e-3) / 1e9
    kgbs = wl["bytes"] / (k_ms * 1e-3) / 1e9
    fused = "" if f_ms is None else (f"; the step's attention launch {f_ms * 1e3:.1f} us -> "
                                     f"{wl['bytes'] / (f_ms * 1e-3) / 1e9:.0f} GB/s")
    log(f"[bench] {name}: step {step_ms * 1e3:.1f} us (median of graph replays, {STEPS_PER_GRAPH} steps each; one "
        f"step alone {t['latency_ms'] * 1e3:.1f} us; eager back-to-back {t['eager_ms'] * 1e3:.1f} us) -> {gbs:.0f} GB/s "
        f"({100 * gbs / HBM_PEAK_GBS:.1f}% of HBM peak){fused}; attention alone {k_ms * 1e3:.1f} us -> {kgbs:.0f} GB/s "
        f"({100 * kgbs / HBM_PEAK_GBS:.1f}%)")
    r = dict(step_ms=step_ms, step_latency_ms=t["latency_ms"], step_eager_ms=t["eager_ms"], kernel_ms=k_ms,
             gbs=gbs, kernel_gbs=kgbs, bytes=wl["bytes"], step_frac=gbs / HBM_PEAK_GBS)
    if f_ms is not None:
        r.update(fused_kernel_ms=f_ms, fused_kernel_gbs=wl["bytes"] / (f_ms * 1e-3) / 1e9)
    return r


def prefill_result(cfg, conv, steps, warmup):
    """Causal prefill of the whole prompt: mla_cache_append of every token followed by mla_prefill."""
    import torch

    from mla_latent_kv_cache_amd import LatentCache, LayerShape, append, pack_weights, prefill, prefill_workspace_bytes

    shape = LayerShape(cfg.d_model, cfg.n_heads, cfg.d_head, cfg.r_pairs, cfg.d_kv, cfg.dtype, cfg.cache_fmt)
    B, S = cfg.batch, cfg.context
    w = pack_weights(shape, conv, rope_len=S, theta=cfg.theta)
    cache = LatentCache.allocate(shape, B, S)
    g = torch.Generator(device="cuda")
    g.manual_seed(1002)
    x = torch.randn((B, S, cfg.d_model), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    wq = torch.from_numpy(conv["w_q"].astype(np.float32)).cuda().to(torch.bfloat16)
    q = (x.reshape(B * S, -1) @ wq).reshape(B, S, cfg.n_heads, cfg.d_head).contiguous()
    del wq
    out = torch.empty_like(q)
    ws = torch.empty(prefill_workspace_bytes(shape, B, S), dtype=torch.uint8, device="cuda")
    start = torch.zeros(B, dtype=torch.int32, device="cuda")

    def step():
        append(w, cache, x, start, 0)
        prefill(w, cache, q, out, ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ref = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    out.zero_()
    graph.replay()
    torch.cuda.synchronize()
    if not torch.equal(out, ref):
        raise RuntimeError("a graph replay of the prefill differs from the eager call")
    ms = median_replay_ms([graph], max(min(20, REPLAYS), steps), warmup)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    mean_ms = t0.elapsed_time(t1) / steps
    del graph
    flop_append = 2.0 * B * S * cfg.d_model * (cfg.d_kv + cfg.n_heads * 2 * cfg.r_pairs)
    flop_rec = 2.0 * B * S * cfg.d_kv * cfg.n_heads * (2 * cfg.d_head - 2 * cfg.r_pairs)
    flop_attn = 4.0 * cfg.d_head * S * (S + 1) / 2 * B * cfg.n_heads
    total = flop_append + flop_rec + flop_attn
    tfs = total / (ms * 1e-3) / 1e12
    log(f"[bench] llama_bf16_prefill: {ms * 1e3:.1f} us per append+prefill (median of graph replays; back-to-back "
        f"mean {mean_ms * 1e3:.1f} us) -> {tfs:.0f} TFLOP/s ({100 * tfs / BF16_PEAK_TFLOPS:.1f}% of bf16 dense peak)")
    return dict(step_ms=ms, step_mean_ms=mean_ms, tflops=tfs, mfma_frac=tfs / BF16_PEAK_TFLOPS, flop=total,
                flop_parts={"append": flop_append, "reconstruction": flop_rec, "attention": flop_attn})


# ---------------------------------------------------------------- cpu baseline

def _blas_info():
    """BLAS library behind numpy and its thread count, as threadpoolctl reports them."""
    try:
        from threadpoolctl import threadpool_info

        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return f"{i.get('internal_api')} {i.get('version')}", int(i.get("num_threads", 1))
    except Exception:  # pragma: no cover
        pass
    return "unknown", 1


def cpu_baseline(cfg, seconds):
    """The oracle on the host: its conversion of the workload's layer (pair ranking + joint SVD), then its cache
    fill + unabsorbed decode for whole sequences of the workload, each timed separately.  BLAS threads are set to
    the host CPUs this process may run on (the affinity mask), capped by OMP_NUM_THREADS when that is set."""
    import oracle
    import synth

    avail = len(os.sched_getaffinity(0))
    cap = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = min(avail, cap) if cap > 0 else avail
    try:
        from threadpoolctl import threadpool_limits

        limiter = threadpool_limits(limits=threads, user_api="blas")
    except Exception:  # pragma: no cover
        limiter = None
    blas, used = _blas_info()
    d, n_h, d_h, _ = synth.FAMILIES[cfg.family]
    wq, wk, wv, xc = synth.layer_weights(cfg.family)
    t = time.perf_counter()
    conv = oracle.convert_layer(wq, wk, wv, xc, n_h, d_h, cfg.r_pairs, cfg.d_kv)
    t_conv = time.perf_counter() - t
    L = cfg.context
    w = {k: synth.round_to_device(conv[k], cfg.dtype) for k in ("w_dkv", "w_krope", "w_uk", "w_uv")}
    done, t_fill, t_attn = 0, 0.0, 0.0
    while done < cfg.batch and (t_fill + t_attn < seconds or done == 0):
        x = synth.context_x(cfg, done, L)
        q = synth.query_rows(x[-1:], wq, cfg.dtype).reshape(cfg.n_heads, cfg.d_head)
        t = time.perf_counter()
        c, kr = oracle.append_ref(x, w["w_dkv"], w["w_krope"], conv["pair_idx"], np.arange(L), cfg.d_head, cfg.theta)
        t_fill += time.perf_counter() - t
        t = time.perf_counter()
        oracle.decode_ref(q, c, kr, w["w_uk"], w["w_uv"], conv["pair_idx"], cfg.d_head, cfg.theta)
        t_attn += time.perf_counter() - t
        done += 1
    if limiter is not None:
        limiter.restore_original_limits()
    row = cfg.d_kv * 2 + cfg.n_heads * 2 * cfg.r_pairs * 2
    gbs = done * L * row / (t_fill + t_attn) / 1e9
    log(f"[bench] cpu oracle ({blas}, {used} threads of {avail} CPUs): conversion {t_conv:.1f}s; {done} sequence(s) "
        f"fill {t_fill:.1f}s + attention {t_attn:.1f}s -> {gbs:.5f} GB/s")
    return {"value": gbs, "unit": "GB/s", "cores": used, "kind": "oracle",
            "sample": f"{done} of {cfg.batch} sequences (context {L}) of the same workload: oracle cache fill "
                      f"(down-projection + partial RoPE) and unabsorbed decode, fp64, timed apart from the "
                      f"conversion; {t_fill + t_attn:.1f} s",
            "blas": blas, "affinity_cpus": avail, "conversion_s": round(t_conv, 2), "fill_s": round(t_fill, 2),
            "attention_s": round(t_attn, 2)}


# ---------------------------------------------------------------- main

def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (decode shards by sequence with no "
              "exchange; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    import synth
    from mla_latent_kv_cache_amd import _lib

    _lib.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    only = set(args.only.split(","))
    global REPLAYS
    REPLAYS = args.replays
    C = synth.CONFIGS
    if args.copy_calibration:
        copy_calibration()

    ceiling = stream_read_ceiling() if "bw" in only else None
    conv_main = converted("llama", 4, 512)
    cfg1 = C[1]
    wl1 = make_decode_workload(cfg1, conv_main, synth.seq_lens(cfg1), args.copies, seed=1001)
    main_res = decode_result("llama_bf16_decode", cfg1, wl1, args.steps, args.warmup)
    secondary = {}
    if "c7" in only:
        secondary["llama_bf16_multiquery4"] = multi_query_result(cfg1, wl1, 4, args.steps, args.warmup)
    del wl1
    torch.cuda.empty_cache()
    if "c6" in only:
        wl6 = make_decode_workload(cfg1, conv_main, synth.seq_lens(cfg1), args.copies, seed=1006, page_size=64)
        r6 = decode_result("llama_bf16_decode_paged64", cfg1, wl6, args.steps, args.warmup)
        r6.update(hbm_frac=r6["kernel_gbs"] / HBM_PEAK_GBS, page_size=64,
                  kernel="decode_attn_dma<128, 8, 3, true, false>")
        secondary["llama_bf16_decode_paged64"] = r6
        del wl6
        torch.cuda.empty_cache()

    if "c3" in only:
        cfg3 = C[3]
        conv3 = converted("llama", 2, 256)
        lens3 = synth.seq_lens(cfg3)
        wl3 = make_decode_workload(cfg3, conv3, lens3, args.copies, seed=1003)
        r3 = decode_result("llama_bf16_longctx_decode", cfg3, wl3, args.steps, args.warmup)
        k3 = "decode_attn_wave<256, 4, 0, 3, false>"
        r3.update(lens=[int(v) for v in lens3], hbm_frac=r3["kernel_gbs"] / HBM_PEAK_GBS, kernel=k3,
                  traffic=measured_traffic(k3 + " in mla_decode_step"), traffic_alone=measured_traffic(k3))
        secondary["llama_bf16_longctx_decode"] = r3
        del wl3, conv3
        torch.cuda.empty_cache()
    if "c4" in only:
        cfg4 = C[4]
        wl4 = make_decode_workload(cfg4, conv_main, synth.seq_lens(cfg4), args.copies, seed=1004)
        r4 = decode_result("llama_int4_decode", cfg4, wl4, args.steps, args.warmup)
        k4 = "decode_attn_mfma<128, 8, 1, false>"
        r4.update(hbm_frac=r4["kernel_gbs"] / HBM_PEAK_GBS, kernel=k4,
                  traffic=measured_traffic(k4 + " in mla_decode_step"), traffic_alone=measured_traffic(k4))
        secondary["llama_int4_decode"] = r4
        del wl4
        torch.cuda.empty_cache()

    if "c5" in only:
        # the int4 workload's shape with the 2-bit latent and a bf16 window of the last 128 rows
        cfg5 = synth.scaled(C[4], name="llama_int2w_decode", cache_fmt="int2_g32_win")
        wl5 = make_decode_workload(cfg5, conv_main, synth.seq_lens(cfg5), args.copies, seed=1005)
        r5 = decode_result("llama_int2w_decode", cfg5, wl5, args.steps, args.warmup, check=False)
        r5.update(hbm_frac=r5["kernel_gbs"] / HBM_PEAK_GBS, window=wl5["caches"][0].window,
                  kernel="decode_attn_mfma<128, 8, 2>")
        secondary["llama_int2w_decode"] = r5
        del wl5
        torch.cuda.empty_cache()

    if "c8" in only:
        # the int4 workload's shape with a bf16 window of the last 128 rows (older rows int4 codes of their bf16
        # values), as the README page's quantised-cache evaluation keeps its most recent tokens unquantised
        cfg8 = synth.scaled(C[4], name="llama_int4w_decode", cache_fmt="int4_g32_win")
        wl8 = make_decode_workload(cfg8, conv_main, synth.seq_lens(cfg8), args.copies, seed=1008)
        r8 = decode_result("llama_int4w_decode", cfg8, wl8, args.steps, args.warmup, check=False)
        r8.update(hbm_frac=r8["kernel_gbs"] / HBM_PEAK_GBS, window=wl8["caches"][0].window,
                  kernel="decode_attn_mfma<128, 8, 3>")
        secondary["llama_int4w_decode"] = r8
        del wl8
        torch.cuda.empty_cache()

    if "c10" in only:
        # the shape of the pages' LongBench evaluation (batch 16, 2048 tokens per sequence) on the main
        # workload's layer: seeded synthetic inputs stand in for the benchmark's items
        cfg10 = synth.scaled(C[1], name="longbench_shape_decode", batch=16, context=2048)
        wl10 = make_decode_workload(cfg10, conv_main, synth.seq_lens(cfg10), args.copies, seed=1010)
        r10 = decode_result("longbench_shape_decode", cfg10, wl10, args.steps, args.warmup)
        r10.update(hbm_frac=r10["kernel_gbs"] / HBM_PEAK_GBS, batch=16, context=2048)
        secondary["longbench_shape_decode"] = r10
        del wl10
        torch.cuda.empty_cache()

    if "c9" in only:
        # a grouped-query source (Llama-3-8B-shaped attention: 32 query heads, 8 KV heads) converted at r 4,
        # d_kv 512, its RoPE keys stored once per KV head: 1152 cache bytes per token instead of 1536; the
        # batch and context of the main workload
        cfg9 = synth.scaled(C[1], name="llama3_gqa_compact_decode")
        conv9 = converted_gqa("llama3", 4, 512)
        wl9 = make_decode_workload(cfg9, conv9, synth.seq_lens(cfg9), args.copies, seed=1009, rope_heads=8)
        r9 = decode_result("llama3_gqa_compact_decode", cfg9, wl9, args.steps, args.warmup)
        k9 = "decode_attn_dma<128, 8, 3, false, true>"
        r9.update(hbm_frac=r9["kernel_gbs"] / HBM_PEAK_GBS, rope_heads=8, bytes_per_token=wl9["bytes_per_row"],
                  kernel=k9, traffic=measured_traffic(k9 + " in mla_decode_step"), traffic_alone=measured_traffic(k9))
        secondary["llama3_gqa_compact_decode"] = r9
        del wl9, conv9
        torch.cuda.empty_cache()

    if "c2" in only:
        secondary["llama_bf16_prefill"] = prefill_result(C[2], conv_main, max(2, args.steps // 5), max(1, args.warmup // 5))
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg1, args.cpu_seconds)

    fgbs = main_res["fused_kernel_gbs"]
    roof = {"bound": "hbm", "achieved": round(fgbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(fgbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(FUSED_KEY),
            "kernel": DOMINANT_KERNEL + " with the append's reduction (mla_decode_step phase 2)",
            "kernel_us": round(main_res["fused_kernel_ms"] * 1e3, 2),
            "algorithmic_bytes": main_res["bytes"],
            "step_frac": round(main_res["step_frac"], 4),
            "attention_alone_us": round(main_res["kernel_ms"] * 1e3, 2),
            "attention_alone_frac": round(main_res["kernel_gbs"] / HBM_PEAK_GBS, 4),
            "attention_alone_traffic": measured_traffic(DOMINANT_KERNEL)}
    if ceiling is not None:
        roof.update(stream_read_ceiling_gbs=ceiling["gbs"], frac_of_stream_ceiling=round(fgbs / ceiling["gbs"], 4))
    line = {
        "metric": METRIC,
        "value": round(main_res["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama_bf16_decode: Llama-2-7B-shaped layer (d_model 4096, 32 heads x 128), r 4 pairs/head, "
                               "d_kv 512, bf16 latent cache, batch 32, every sequence at context 4096; step = "
                               "mla_decode_step (append of the new token + decode)",
                   "batch": 32, "context": 4096, "d_kv": 512, "r_pairs": 4, "cache_bytes_per_step": main_res["bytes"],
                   "parallelism": "single GPU",
                   "timing": f"median over {max(REPLAYS, args.steps)} replays of a HIP graph of {STEPS_PER_GRAPH} "
                             f"consecutive steps (3 cache copies in rotation), per step"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    if ceiling is not None:
        line["secondary"]["stream_read_ceiling"] = ceiling
    line["secondary"]["llama_bf16_decode"] = {k: v for k, v in main_res.items() if k != "bytes"}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
