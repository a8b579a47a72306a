#!/usr/bin/env python3
"""Throughput of the MHA2MLA latent-cache hot path on one MI355X (gfx950).

One step of the headline workload (Llama-2-7B-shaped layer, bf16, d_kv 512, r 4, batch 32, every
sequence at context 4096) is one decode step of serving, mla_decode_step: the append of the new token of
every sequence (position 4095) and the decode over the 4096 cached tokens.  `value` is the latent-cache
bytes one decode must read (batch x context x bytes per cache row) divided by the step time.

Timing: inputs are resident in HBM before the timed region; `--warmup` untimed steps, then `--steps`
timed steps bracketed by device synchronisation and HIP events on the launch stream.  Three independent
cache copies are used in rotation so that the 256 MB last-level cache cannot serve a step's reads from
the previous step.  The roofline object times the dominant kernel (the split-K attention launch, phase 2
of mla_decode) separately: `--steps` back-to-back launches of it between two HIP events.

The cpu_baseline object times the oracle (plain fp64 numpy; the library never uses it) on a bounded
sample of the same workload on the host's cores.  Secondary workloads (long-context variable-length
decode, int4-latent decode, 2-bit-latent decode with a 128-row bf16 window, the headline decode on a
paged cache of 64-token pages in random order, a 4-query multi-query decode, causal prefill) are reported
in `secondary`.

`roofline.traffic` is the HBM traffic of one launch of that kernel from FETCH_SIZE / WRITE_SIZE counter
runs (profiles/pmc_traffic.json, scaled by the counters of a plain copy of known size, see
--copy-calibration); it is null when those counters were taken on different decode sources.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--only c1,c3,c4,c5,c6,c7,c2] [--no-cpu-baseline]
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
DOMINANT_KERNEL = "decode_attn_dma<128, 8, 3, false>"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", default="c1,c3,c4,c5,c6,c7,c2")
    ap.add_argument("--copies", type=int, default=3)
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


def make_decode_workload(cfg, conv, lens, copies, seed, page_size=0):
    """Weights, `copies` filled caches (through mla_cache_append), the step's new-token activations, queries
    and one BoundDecode per copy.  Activations are seeded N(0,1) generated on the device.  page_size > 0:
    paged caches whose pages are a random permutation of the pool."""
    import torch

    from mla_latent_kv_cache_amd import BoundDecode, LatentCache, LayerShape, append, pack_weights

    shape = LayerShape(cfg.d_model, cfg.n_heads, cfg.d_head, cfg.r_pairs, cfg.d_kv, cfg.dtype, cfg.cache_fmt)
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


def time_decode(wl, steps, warmup):
    """Whole-step time (append + decode) and the attention kernel's average launch duration."""
    import torch

    bound = wl["bound"]
    n = len(bound)
    for i in range(warmup):
        bound[i % n].step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        bound[i % n].step()
    t1.record()
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / steps
    # dominant kernel: phase 1 (query preparation) once, then back-to-back launches of phase 2 (the split-K
    # attention) over the rotating cache copies, bracketed by two events on the launch stream
    for i in range(n):
        bound[i].phase(1)
    for i in range(warmup):
        bound[i % n].phase(2)
    torch.cuda.synchronize()
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record()
    for i in range(steps):
        bound[i % n].phase(2)
    k1.record()
    torch.cuda.synchronize()
    k_ms = k0.elapsed_time(k1) / steps
    return step_ms, k_ms


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


def decode_result(name, cfg, wl, steps, warmup):
    step_ms, k_ms = time_decode(wl, steps, warmup)
    gbs = wl["bytes"] / (step_ms * 1e-3) / 1e9
    kgbs = wl["bytes"] / (k_ms * 1e-3) / 1e9
    log(f"[bench] {name}: step {step_ms * 1e3:.1f} us -> {gbs:.0f} GB/s; attention kernel {k_ms * 1e3:.1f} us -> "
        f"{kgbs:.0f} GB/s ({100 * kgbs / HBM_PEAK_GBS:.1f}% of HBM peak)")
    return dict(step_ms=step_ms, kernel_ms=k_ms, gbs=gbs, kernel_gbs=kgbs, bytes=wl["bytes"])


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
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    flop_append = 2.0 * B * S * cfg.d_model * (cfg.d_kv + cfg.n_heads * 2 * cfg.r_pairs)
    flop_rec = 2.0 * B * S * cfg.d_kv * cfg.n_heads * (2 * cfg.d_head - 2 * cfg.r_pairs)
    flop_attn = 4.0 * cfg.d_head * S * (S + 1) / 2 * B * cfg.n_heads
    total = flop_append + flop_rec + flop_attn
    tfs = total / (ms * 1e-3) / 1e12
    log(f"[bench] llama_bf16_prefill: {ms * 1e3:.1f} us per append+prefill -> {tfs:.0f} TFLOP/s "
        f"({100 * tfs / BF16_PEAK_TFLOPS:.1f}% of bf16 dense peak)")
    return dict(step_ms=ms, tflops=tfs, mfma_frac=tfs / BF16_PEAK_TFLOPS, flop=total,
                flop_parts={"append": flop_append, "reconstruction": flop_rec, "attention": flop_attn})


# ---------------------------------------------------------------- cpu baseline

def cpu_baseline(cfg, conv, seconds):
    """The oracle's cache fill + unabsorbed decode for whole sequences of the workload, on the host."""
    import oracle
    import synth

    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    L = cfg.context
    w = {k: synth.round_to_device(conv[k], cfg.dtype) for k in ("w_dkv", "w_krope", "w_uk", "w_uv")}
    done, t_all = 0, 0.0
    while done < cfg.batch and (t_all < seconds or done == 0):
        x = synth.context_x(cfg, done, L)
        q = synth.query_rows(x[-1:], conv["w_q"], cfg.dtype).reshape(cfg.n_heads, cfg.d_head)
        t = time.perf_counter()
        c, kr = oracle.append_ref(x, w["w_dkv"], w["w_krope"], conv["pair_idx"], np.arange(L), cfg.d_head, cfg.theta)
        oracle.decode_ref(q, c, kr, w["w_uk"], w["w_uv"], conv["pair_idx"], cfg.d_head, cfg.theta)
        t_all += time.perf_counter() - t
        done += 1
    row = cfg.d_kv * 2 + cfg.n_heads * 2 * cfg.r_pairs * 2
    gbs = done * L * row / t_all / 1e9
    log(f"[bench] cpu oracle: {done} sequence(s) in {t_all:.1f}s -> {gbs:.5f} GB/s on {threads} threads")
    return {"value": gbs, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {cfg.batch} sequences (context {L}) of the same workload: oracle cache fill "
                      f"(down-projection + partial RoPE) and unabsorbed decode, fp64, conversion excluded; "
                      f"{t_all:.1f} s"}


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
    C = synth.CONFIGS
    if args.copy_calibration:
        copy_calibration()

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
                  kernel="decode_attn_dma<128, 8, 3, true>")
        secondary["llama_bf16_decode_paged64"] = r6
        del wl6
        torch.cuda.empty_cache()

    if "c3" in only:
        cfg3 = C[3]
        conv3 = converted("llama", 2, 256)
        lens3 = synth.seq_lens(cfg3)
        wl3 = make_decode_workload(cfg3, conv3, lens3, args.copies, seed=1003)
        r3 = decode_result("llama_bf16_longctx_decode", cfg3, wl3, args.steps, args.warmup)
        r3.update(lens=[int(v) for v in lens3], hbm_frac=r3["kernel_gbs"] / HBM_PEAK_GBS)
        secondary["llama_bf16_longctx_decode"] = r3
        del wl3, conv3
        torch.cuda.empty_cache()
    if "c4" in only:
        cfg4 = C[4]
        wl4 = make_decode_workload(cfg4, conv_main, synth.seq_lens(cfg4), args.copies, seed=1004)
        r4 = decode_result("llama_int4_decode", cfg4, wl4, args.steps, args.warmup)
        r4.update(hbm_frac=r4["kernel_gbs"] / HBM_PEAK_GBS)
        secondary["llama_int4_decode"] = r4
        del wl4
        torch.cuda.empty_cache()

    if "c5" in only:
        # the int4 workload's shape with the 2-bit latent and a bf16 window of the last 128 rows
        cfg5 = synth.scaled(C[4], name="llama_int2w_decode", cache_fmt="int2_g32_win")
        wl5 = make_decode_workload(cfg5, conv_main, synth.seq_lens(cfg5), args.copies, seed=1005)
        r5 = decode_result("llama_int2w_decode", cfg5, wl5, args.steps, args.warmup)
        r5.update(hbm_frac=r5["kernel_gbs"] / HBM_PEAK_GBS, window=wl5["caches"][0].window,
                  kernel="decode_attn_mfma<128, 8, 2>")
        secondary["llama_int2w_decode"] = r5
        del wl5
        torch.cuda.empty_cache()

    if "c2" in only:
        secondary["llama_bf16_prefill"] = prefill_result(C[2], conv_main, max(2, args.steps // 5), max(1, args.warmup // 5))
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg1, conv_main, args.cpu_seconds)

    kgbs = main_res["kernel_gbs"]
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
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(kgbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kgbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(DOMINANT_KERNEL),
                     "kernel": DOMINANT_KERNEL + " (mla_decode phase 2)",
                     "kernel_us": round(main_res["kernel_ms"] * 1e3, 2)},
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
