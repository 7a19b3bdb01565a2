#!/usr/bin/env python3
"""Throughput benchmark of the block-hybrid attention hot path on one MI355X.

One step is one block cycle of the model's block-hybrid layers on a
continuous-batching decode batch: for each of the 32 denoising steps of the
active block every layer runs ``bha_block_forward`` over all requests and heads;
the last step is ``bha_block_forward_commit``, which also folds the finished
block into the states in the same pass (``--separate-commit``: 32 plain
forwards, then ``bha_state_commit``). Each layer instance has its own state pool, W and gate,
as the model's six block-hybrid layers do, so consecutive forwards of one layer
do not find its 270 MB state in the 256 MB Infinity Cache.

Default workload (decode256): 256 requests x 16 heads, d = 128, FW = 64
(F = 128), B = 32, ragged prefixes of UniformInt{8..256} blocks (256..8,192
tokens) folded into the states before timing (one ragged prefill launch per
layer, itself timed and reported), bf16 Q/K/V/W/O, fp32 states.

Prints ONE JSON line: value = active-block tokens per second through
block-hybrid attention (each forward moves R * B tokens through one layer),
the roofline of the dominant kernel (the forward; algorithmic bytes per launch
divided by its HIP-event-timed average launch duration, against 8 TB/s), and
the fp64 CPU oracle timed on a bounded sample of the same workload. Beside
it, outside the timed region: exact softmax attention of the same batch over the
whole prefixes (``bha_prefix_attention``), the per-step cost the hybrid layer
removes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "active-block tokens/s through block-hybrid attn; achieved HBM GB/s vs peak"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published

# What the pages report for the whole method, printed beside the measurement as
# context only: end-to-end serving ratios of the 16B model with 6 of its 20
# layers linearised, on hardware the pages mostly leave unstated (the
# gist.science explainer, "Technical Summary", Experimental Results, names an
# NVIDIA H200), and a kernel-level ratio with no hardware given. None of them
# is a per-layer kernel rate, so vs_baseline stays null.
PAGES_FIGURES = {
    "decode_throughput_gain": "up to 1.73x over the softmax model (1.50x-1.73x, largest at high concurrency), "
                              "continuous batching",
    "concurrent_requests_gain": "about 1.3x more requests before memory runs out, fixed memory budget",
    "kernel_speedup_at_long_prefixes": "about 30x for the hybrid kernel against softmax prefix attention",
    "sources": "gist.science explainer, Technical Summary: Experimental Results (Throughput and Concurrency); "
               "pith.science review: The reading, Editorial extensions (If this is right)",
    "measured_here": "softmax_prefix_attention.launch_time_over_hybrid_step (this batch) and bench.py "
                     "--prefix-sweep (one 32-token block over 1K-32K-token prefixes)",
}
# streaming-probe configurations reported as context (include/bha_probe.h):
# 16-byte loads per lane per trip, trips in flight per wave, non-temporal
# loads, work-groups per CU, KiB written per wave per trip
PROBE_CONFIGS = (
    ("read_only_forward_shape", dict(loads_per_lane=16, buffers=1, nontemporal=1, wgs_per_cu=1, store_kb_per_wave=0)),
    ("read_only_deep", dict(loads_per_lane=32, buffers=1, nontemporal=0, wgs_per_cu=3, store_kb_per_wave=0)),
    ("read_write_11_to_1", dict(loads_per_lane=32, buffers=1, nontemporal=1, wgs_per_cu=1, store_kb_per_wave=3)),
)
KERNEL_SOURCES = tuple(f"linear_attention_block_amd/csrc/{f}" for f in (
    "mfma_common.hpp", "mfma_forward.hip", "mfma_gqa.hip", "mfma_gqa8.hip", "mfma_commit.hip", "mfma_fused.hip",
    "mfma_prefill.hip", "mfma_feature_map.hip", "bha_device.hpp", "bha_internal.hpp", "bha_mfma.hpp"))


def forward_kernel_name(d, FW, B, npairs, dev):
    """The matrix-core kernel bha_block_forward runs for B <= 32 (one query
    head per K/V head), as the launcher chooses it: the split-slice kernel at
    d = 128, FW = 128; otherwise the persistent one-tile kernel, compiled for
    one wave per SIMD at d = 64, FW <= 64 when it runs that grid (from 8 pairs
    per CU, blocks of more than 16 tokens)."""
    import torch

    if d == 128 and FW == 128:
        return "forward_split_kernel<128>"
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    one = d == 64 and FW <= 64 and B > 16 and npairs >= 8 * cus
    return f"forward_mfma_kernel<{d},{FW},1,{'true' if one else 'false'}>"


def state_store_scope(FW, npairs, dev) -> str:
    """The template flag the commit and fused-step launchers choose for the
    state write-back: device-scope non-temporal stores at F <= 128 from 16
    pairs per CU, non-temporal alone otherwise."""
    import torch

    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    return "true" if FW <= 64 and npairs >= 16 * cus else "false"


def fmap_store_scope(d, FW, ntok, H, dev) -> str:
    """The template flag the feature-map launcher chooses: device-scope
    stores at d = 128, FW = 64 for up to 4 units (128 tokens x head) per CU."""
    import torch

    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    units = (ntok + 127) // 128 * H
    return "true" if d == 128 and FW == 64 and units <= 4 * cus else "false"


def forward_bytes(R, H, d, FW, B, es=2):
    """Algorithmic HBM bytes of one bha_block_forward launch: per (request, head)
    the fp32 S tiles and Z (read), Q, K, V (read) and O (written); W once per head."""
    F = 2 * FW
    return R * H * (d * F * 4 + F * 4 + 4 * B * d * es) + H * FW * d * es


def commit_bytes(R, H, d, FW, B, es=2):
    """Algorithmic HBM bytes of one bha_state_commit launch: per (request, head)
    the state record read and written back, K and V read; W once per head."""
    F = 2 * FW
    return R * H * (2 * (d * F * 4 + F * 4) + 2 * B * d * es) + H * FW * d * es


def forward_commit_bytes(R, H, d, FW, B, es=2):
    """Algorithmic HBM bytes of one bha_block_forward_commit launch: the
    forward's bytes plus the state record written back (every request commits)."""
    F = 2 * FW
    return forward_bytes(R, H, d, FW, B, es) + R * H * (d * F * 4 + F * 4)


def prefill_bytes(T, R, H, d, FW, es=2):
    """Algorithmic HBM bytes of one bha_state_prefill launch over T packed tokens:
    K and V of every token and head read once, each (request, head) state record
    read and written once, W once per head, the offsets and slot ids."""
    F = 2 * FW
    return T * H * 2 * d * es + R * H * 2 * (d * F * 4 + F * 4) + H * FW * d * es + (2 * R + 1) * 4


def forward_gqa_bytes(R, H, HK, d, FW, B, es=2):
    """Algorithmic HBM bytes of one bha_block_forward_gqa launch: per
    (request, K/V head) the state record (S, Z) and K, V read; per (request,
    query head) Q read and O written; W once per K/V head."""
    F = 2 * FW
    return R * HK * (d * F * 4 + F * 4 + 2 * B * d * es) + R * H * 2 * B * d * es + HK * FW * d * es


def prefix_attention_bytes(T, R, H, d, B, es=2):
    """Algorithmic HBM bytes of one bha_prefix_attention launch: K and V of
    every packed prefix token and head read once, the block's Q, K, V read and
    O written, the offsets."""
    return T * H * 2 * d * es + R * H * 4 * B * d * es + (R + 1) * 4


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(config: str):
    """HBM bytes per forward launch measured with rocprofv3 counters, if the
    summary in profiles/ was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"forward_{config}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def record_to_plain(rec, d, F):
    """State records [..., (d+1)F] -> (S [..., F, d], Z [..., F]) in float64,
    following the record layout of include/bha.h (S in 32 x 4 tiles, then Z)."""
    import numpy as np

    f = np.arange(F)[:, None]
    c = np.arange(d)[None, :]
    idx = ((c // 32) * (F // 4) + f // 4) * 128 + (c % 32) * 4 + (f % 4)
    rec = np.asarray(rec, dtype=np.float64)
    return np.ascontiguousarray(rec[..., idx]), np.ascontiguousarray(rec[..., d * F:(d + 1) * F])


def cpu_baseline(layer, case, denoise, n_req, log):
    """Time the fp64 oracle on one block cycle of the first n_req requests,
    median of three runs, on the host's cores (at most 16 threads: the host
    share of one GPU on the box), and the same cycle for n_req / 16 requests on
    one thread."""
    import numpy as np
    import torch

    import oracle

    R, H, d, FW, B = case.R, case.H, case.d, case.FW, case.B
    n_req = min(n_req, R)
    host_cpus = os.cpu_count() or 1
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = host_cpus
    nthreads = max(1, min(16, usable))

    def host(t):
        return np.ascontiguousarray(
            t[:n_req].float().cpu().numpy().astype(np.float64).transpose(0, 2, 1, 3))

    q, k, v = host(layer["q"]), host(layer["k"]), host(layer["v"])
    w = layer["w"].float().cpu().numpy().astype(np.float64)
    g = layer["gamma"].cpu().numpy().astype(np.float64)
    rec = layer["state"].cpu().numpy()[case.slot_ids[:n_req]]
    S, Z = record_to_plain(rec, d, 2 * FW)
    torch.cuda.synchronize()

    def cycle(n, threads):
        S_, Z_ = S[:n].copy(), Z[:n].copy()
        t0 = time.perf_counter()
        for _ in range(denoise):
            oracle.block_forward_batch(q[:n], k[:n], v[:n], w, g, S_, Z_, nthreads=threads)
        oracle.state_commit_batch(S_, Z_, k[:n], v[:n], w, nthreads=threads)
        return time.perf_counter() - t0

    dts = [cycle(n_req, nthreads) for _ in range(3)]
    dt = float(np.median(dts))
    n1 = max(1, n_req // 16)
    dts1 = [cycle(n1, 1) for _ in range(3)]
    dt1 = float(np.median(dts1))
    log(f"cpu oracle: {n_req} requests x {H} heads, {denoise} forwards + 1 commit: median {dt:.2f} s of "
        f"{', '.join(f'{x:.2f}' for x in dts)} on {nthreads} threads ({host_cpus} logical CPUs on the host, "
        f"{usable} usable); {n1} requests on 1 thread: median {dt1:.2f} s")
    return {
        "value": denoise * n_req * B / dt,
        "unit": "tokens/s",
        "cores": nthreads,
        "threads": nthreads,
        "host_logical_cpus": host_cpus,
        "usable_cpus": usable,
        "thread_cap": "16 threads at most: the host CPU share of one GPU on the box",
        "kind": "oracle",
        "sample": (f"one block cycle ({denoise} forwards + 1 commit, one layer) of the first {n_req} "
                   f"of {R} requests, all {H} heads, same workload and state; fp64 C oracle; median of "
                   f"3 runs ({', '.join(f'{x:.2f}' for x in dts)} s wall)"),
        "value_1thread": denoise * n1 * B / dt1,
        "sample_1thread": (f"the same cycle for the first {n1} requests on one thread, median of 3 runs "
                           f"({', '.join(f'{x:.2f}' for x in dts1)} s wall)"),
    }


def feature_map_bytes(R, H, d, FW, B, es=2):
    """Algorithmic HBM bytes of one bha_feature_map launch: every token row read
    (d elements), phi written (2 FW float32 per token and head), W once per head."""
    return R * B * H * (d * es + 2 * FW * 4) + H * FW * d * es


def probe_context(fwd_read, fwd_write, log):
    """The HBM streaming probe (libbha_probe.so) at the forward's byte count:
    read only, and the forward's read/write mix. Median of 10 launches each,
    on rotating regions of the source so no launch finds its bytes cached."""
    from linear_attention_block_amd import probe

    out = {}
    for tag, c in PROBE_CONFIGS:
        cfg = probe.cfg(**c)
        moved, t, gbps = probe.stream_gbps(cfg, fwd_read)
        out[tag] = {"GBps": gbps, "frac": gbps / PEAK_HBM_GBS, "us": t * 1e6, "bytes": moved, "config": c}
        log(f"probe {tag}: {moved / 1e6:.0f} MB in {t * 1e6:.1f} us = {gbps:.0f} GB/s ({gbps / PEAK_HBM_GBS:.1%})")
    return out


def gqa_cycle(args, log) -> dict:
    """The block cycle of the default workload with grouped K/V heads: the H
    query heads share args.kv_heads K/V heads (states, W, K and V per K/V
    head). Per layer: states built by one prefill over the K/V heads, then per
    step 32 bha_block_forward_gqa launches and one bha_state_commit per layer
    (the fused last step exists for one K/V head per query head only)."""
    import numpy as np
    import torch

    import linear_attention_block_amd as bha
    import synth

    dev = torch.device("cuda:0")
    case = synth.make_case(args.config, R=args.requests or None, with_prefix=False, with_qkv=False)
    R, H, d, FW, B = case.R, case.H, case.d, case.FW, case.B
    HK = args.kv_heads
    if HK < 1 or H % HK:
        raise SystemExit(f"--kv-heads {HK} must divide the {H} query heads")
    G = H // HK
    nl, nd = args.layers, args.denoise
    slots = torch.from_numpy(case.slot_ids).to(dev)
    layers = []
    for L in range(nl):
        w, _ = synth.device_layer_params(args.config, L, dev, H=HK)
        _, gamma = synth.device_layer_params(args.config, L, dev)
        state = bha.new_state(case.num_slots, HK, d, FW, dev)
        pk, pv, offs = synth.device_packed_prefix(args.config, case.n_blocks, dev, layer=L, H=HK)
        bha.state_prefill(pk, pv, offs, w, state, slots)
        del pk, pv, offs
        q = synth.device_step_qkv(args.config, 0, R, dev, layer=L)[0]
        _, k, v = synth.device_step_qkv(args.config, 0, R, dev, layer=L, H=HK)
        out = torch.empty_like(q)
        layers.append(dict(fwd=bha.prepare_forward_gqa(q, k, v, w, gamma, state, slots, out),
                           com=bha.prepare_commit(k, v, w, state, slots), keep=(q, k, v, w, gamma, state, out)))
    torch.cuda.synchronize()
    # one event pair around each step's forwards and one around its commits
    def ev_pair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def step(evs=None):
        if evs is not None:
            evs[0][0].record()
        for _ in range(nd):
            for lay in layers:
                lay["fwd"]()
        if evs is not None:
            evs[0][1].record()
            evs[1][0].record()
        for lay in layers:
            lay["com"]()
        if evs is not None:
            evs[1][1].record()

    ev = [(ev_pair(), ev_pair()) for _ in range(args.steps)]
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for st in range(args.steps):
        step(ev[st])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    fwd_avg = sum(f0.elapsed_time(f1) for (f0, f1), _ in ev) * 1e-3 / (args.steps * nd * nl)
    com_avg = sum(c0.elapsed_time(c1) for _, (c0, c1) in ev) * 1e-3 / (args.steps * nl)
    fb = forward_gqa_bytes(R, H, HK, d, FW, B)
    cb = commit_bytes(R, HK, d, FW, B)
    value = args.steps * nd * nl * R * B / elapsed
    log(f"gqa forward (H={H}, {HK} K/V heads): avg {fwd_avg * 1e6:.1f} us/launch, {fb / fwd_avg / 1e9:.0f} GB/s "
        f"algorithmic ({fb / 1e6:.1f} MB/launch); commit: avg {com_avg * 1e6:.1f} us, {cb / com_avg / 1e9:.0f} GB/s")
    log(f"step: {elapsed / args.steps * 1e3:.2f} ms; {value / 1e6:.1f} M tokens/s")
    return {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": elapsed / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": (f"{args.config} with grouped K/V heads: {R} requests x {H} query heads over {HK} "
                                f"K/V heads (G={G}), d={d}, FW={FW}, B={B}; per step {nd} forwards in each of {nl} "
                                f"layers, then a commit per layer"),
                   "requests": R, "heads": H, "kv_heads": HK, "head_dim": d, "feat_half": FW, "block": B,
                   "denoise_steps": nd, "layers": nl},
        "roofline": {"bound": "hbm", "achieved": fb / fwd_avg / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": fb / fwd_avg / 1e9 / PEAK_HBM_GBS, "traffic": None,
                     "kernel": ("bha_block_forward_gqa: " +
                                (f"forward_mfma_kernel<{d},{FW},{(B + 31) // 32}>" if G == 1 and B <= 64 else
                                 f"forward_gqa_mfma_kernel<{d},{FW},{G}>" if G in (2, 4) and B <= 32 else
                                 f"forward_gqa8_kernel<{d},{FW}>" if G == 8 and FW <= 64 and B <= 32 else
                                 "forward_generic_kernel")),
                     "bytes_per_launch": fb, "avg_launch_us": fwd_avg * 1e6},
        "commit": {"kernel": "bha_state_commit over the K/V heads", "avg_launch_us": com_avg * 1e6,
                   "bytes_per_launch": cb, "achieved_GBps": cb / com_avg / 1e9},
        "cpu_baseline": None,
    }


def prefix_sweep(requests, prefixes, log) -> dict:
    """Kernel-level comparison of one block-hybrid step with exact softmax
    attention over the prefix: a 32-token block (16 heads, d = 128, FW = 64)
    of each of ``requests`` requests over a prefix of P tokens, for every P in
    ``prefixes``. Each launch is timed with HIP events on its stream, cold (a
    1 GiB buffer is read between launches, outside the events, so the
    256 MB Infinity Cache and L2 start without the operands; a read leaves no
    dirty lines whose write-back would be charged to the timed launch) and warm
    (back to back); medians of 10 and 20 launches."""
    import numpy as np
    import torch

    import linear_attention_block_amd as bha
    import synth

    dev = torch.device("cuda:0")
    name = "longctx2k"  # 16 heads, d = 128, FW = 64, B = 32, bf16
    H, d, FW, B = 16, 128, 64, 32
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    flush_sink = torch.empty((), dtype=torch.float32, device=dev)

    def timed(fn, n, cold):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for _ in range(3):
            fn()
        for e0, e1 in evs:
            if cold:
                torch.sum(flush, dim=0, out=flush_sink)
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3

    rows = []
    for R in requests:
        w, gamma = synth.device_layer_params(name, 0, dev)
        q, k, v = synth.device_step_qkv(name, 0, R, dev, layer=0)
        slots = torch.arange(R, dtype=torch.int32, device=dev)
        for P in prefixes:
            pk, pv, offs = synth.device_packed_prefix(name, np.full(R, P // B), dev, layer=0)
            state = bha.new_state(R, H, d, FW, dev)
            bha.state_prefill(pk, pv, offs, w, state, slots)
            out_h, out_s = torch.empty_like(q), torch.empty_like(q)
            hyb = bha.prepare_forward(q, k, v, w, gamma, state, slots, out_h)
            sm = bha.prepare_prefix_attention(q, k, v, pk, pv, offs, out_s)
            fb = forward_bytes(R, H, d, FW, B)
            sb = prefix_attention_bytes(R * P, R, H, d, B)
            row = {"requests": R, "prefix": P,
                   "splits": bha.prefix_attention_workspace(R, H, d, B, R * P) // (R * H * (32 * d + 64) * 4) or 1}
            for tag, cold, n in (("cold", True, 10), ("warm", False, 20)):
                th, ts = timed(hyb, n, cold), timed(sm, n, cold)
                row[f"hybrid_us_{tag}"] = th
                row[f"softmax_us_{tag}"] = ts
                row[f"softmax_over_hybrid_{tag}"] = ts / th
                row[f"hybrid_GBps_{tag}"] = fb / th / 1e3
                row[f"softmax_GBps_{tag}"] = sb / ts / 1e3
            log(f"sweep R={R} P={P}: hybrid {row['hybrid_us_cold']:.1f} us cold / {row['hybrid_us_warm']:.1f} warm, "
                f"softmax {row['softmax_us_cold']:.1f} / {row['softmax_us_warm']:.1f} us "
                f"({row['splits']} splits, {row['softmax_GBps_cold']:.0f} GB/s cold); "
                f"ratio {row['softmax_over_hybrid_cold']:.1f}x cold, {row['softmax_over_hybrid_warm']:.1f}x warm")
            rows.append(row)
            del hyb, sm, pk, pv, offs, state, out_h, out_s
            torch.cuda.empty_cache()
    return {"comparison": "one block-hybrid forward vs exact softmax attention over the prefix "
                          f"(B={B}, H={H}, d={d}, FW={FW}, bf16; per-launch medians)", "rows": rows}


def shape_sweep(log) -> dict:
    """Latency and bandwidth of one forward and one commit launch as the block
    size B and the feature width FW vary: 256 requests x 16 heads, d = 128,
    bf16, states built by one prefill over 1,024-token prefixes. Each launch is
    timed with HIP events, cold (a 1 GiB buffer is read before it so the
    Infinity Cache does not hold the state), median of 10."""
    import numpy as np
    import torch

    import linear_attention_block_amd as bha
    import synth

    dev = torch.device("cuda:0")
    R, H, d = 256, 16, 128
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)

    def timed(fn, n=10):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for _ in range(2):
            fn()
        for e0, e1 in evs:
            torch.sum(flush, dim=0, out=sink)
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3

    rows = []
    for FW in (32, 64, 128):
        over = dict(H=H, d=d, FW=FW, B=32)
        w, gamma = synth.device_layer_params("decode256", 0, dev, **over)
        slots = torch.arange(R, dtype=torch.int32, device=dev)
        state = bha.new_state(R, H, d, FW, dev)
        pk, pv, offs = synth.device_packed_prefix("decode256", np.full(R, 32), dev, **over)
        bha.state_prefill(pk, pv, offs, w, state, slots)
        del pk, pv, offs
        for B in (8, 16, 32, 48, 64):
            q, k, v = synth.device_step_qkv("decode256", 0, R, dev, **dict(over, B=B))
            out = torch.empty_like(q)
            fwd = bha.prepare_forward(q, k, v, w, gamma, state, slots, out)
            snap = state.clone()
            com = bha.prepare_commit(k, v, w, state, slots)
            tf, tc = timed(fwd), timed(com)
            state.copy_(snap)
            del snap
            fb, cb = forward_bytes(R, H, d, FW, B), commit_bytes(R, H, d, FW, B)
            row = {"B": B, "FW": FW, "F": 2 * FW, "state_MB": R * H * (d + 1) * 2 * FW * 4 / 1e6,
                   "forward_us": tf, "forward_GBps": fb / tf / 1e3, "forward_tokens_per_s": R * B / tf * 1e6,
                   "commit_us": tc, "commit_GBps": cb / tc / 1e3,
                   "path": ("mfma, one query tile; commit kernel" if B <= 32 else
                            "mfma, two query tiles; commit through the prefill kernel")}
            log(f"shape B={B} FW={FW}: forward {tf:.1f} us ({row['forward_GBps']:.0f} GB/s, "
                f"{row['forward_tokens_per_s'] / 1e6:.1f} M tok/s), commit {tc:.1f} us ({row['commit_GBps']:.0f} GB/s) "
                f"[{row['path']}]")
            rows.append(row)
            del fwd, com, q, k, v, out
        del state
        torch.cuda.empty_cache()
    return {"sweep": "forward and commit per launch vs block size B and feature width FW "
                     f"(R={R}, H={H}, d={d}, bf16, cold)", "rows": rows}


def probe_sweep(read_bytes, log) -> dict:
    """The HBM streaming probe (libbha_probe.so) over its configurations at
    read_bytes per launch: read-only streams (slice size, slices in flight,
    non-temporal loads, work-groups per CU), then streams with writes mixed in
    at 2:1 to 16:1 under each store mode of include/bha_probe.h. Medians of 10
    launches on rotating source regions."""
    from linear_attention_block_amd import probe

    rows = []

    def run(**c):
        moved, t, gbps = probe.stream_gbps(probe.cfg(**c), read_bytes)
        row = dict(c, us=t * 1e6, bytes=moved, GBps=gbps, frac=gbps / PEAK_HBM_GBS)
        rows.append(row)
        log(f"probe {c}: {moved / 1e6:.0f} MB in {t * 1e6:.1f} us = {gbps:.0f} GB/s ({gbps / PEAK_HBM_GBS:.1%})")

    for nsl in (8, 16, 32):
        for nbuf in (1, 2):
            for nt in (0, 1):
                for wpe in (1, 2, 4, 8):
                    if nsl * nbuf * 4 * wpe <= 512:  # register file: slices of every resident wave
                        run(loads_per_lane=nsl, buffers=nbuf, nontemporal=nt, wgs_per_cu=wpe, store_kb_per_wave=0)
    for nsl, wkb in ((16, 1), (8, 1), (32, 3), (16, 2), (16, 8), (8, 8)):
        for sm in (0, 1, 2, 3, 4):
            for wpe in (1, 2):
                run(loads_per_lane=nsl, buffers=1, nontemporal=1, wgs_per_cu=wpe, store_kb_per_wave=wkb,
                    store_mode=sm)
    return {"probe_sweep": f"streaming probe at {read_bytes / 1e6:.0f} MB read per launch", "rows": rows}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="decode256",
                    choices=["decode256", "b16", "longctx2k", "longctx16k", "longctx32k", "wide2048"])
    ap.add_argument("--requests", type=int, default=0,
                    help="override the workload's request count (the first R requests of its seeded draw)")
    ap.add_argument("--layers", type=int, default=6, help="block-hybrid layer instances (default 6)")
    ap.add_argument("--denoise", type=int, default=32, help="denoising forwards per block")
    ap.add_argument("--cpu-sample-requests", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--io", choices=("bf16", "f32"), default="bf16",
                    help="token dtype of the block cycle (default bf16; f32: the same draws widened, the "
                         "fp32-arithmetic kernels)")
    ap.add_argument("--separate-commit", action="store_true",
                    help="run every denoising step as a plain forward and commit with bha_state_commit "
                         "(default: the last step of the block is bha_block_forward_commit)")
    ap.add_argument("--staggered", action="store_true",
                    help="continuous batching with staggered blocks: request r finishes its block at denoising "
                         "step r mod 32, so every step is one bha_block_forward_commit whose mask commits "
                         "1/32 of the requests")
    ap.add_argument("--prefix-sweep", action="store_true",
                    help="instead of the block cycle: the kernel-level comparison of one block-hybrid forward "
                         "with softmax attention over prefixes of 1K..32K tokens (prints its own JSON line)")
    ap.add_argument("--sweep-requests", default="1,64")
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="grouped K/V heads: the query heads share this many K/V heads (states, W, K, V per "
                         "K/V head); runs the block cycle with bha_block_forward_gqa (prints its own JSON line)")
    ap.add_argument("--shape-sweep", action="store_true",
                    help="instead of the block cycle: forward and commit latency over block sizes 8..64 and "
                         "feature widths FW 32..128 (prints its own JSON line)")
    ap.add_argument("--probe-sweep", action="store_true",
                    help="instead of the block cycle: the HBM streaming probe over its configurations at the "
                         "forward's read bytes (prints its own JSON line)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB (counter scaling)")
    args = ap.parse_args()

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this library's hot path runs on one GPU; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported. Every (request, head) pair is independent, "
              "so requests or heads shard across GPUs with no exchange; run one process per GPU.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import linear_attention_block_amd as bha
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bha.load_library()
    if args.prefix_sweep:
        reqs = [int(x) for x in args.sweep_requests.split(",")]
        print(json.dumps(prefix_sweep(reqs, [1024, 2048, 4096, 8192, 16384, 32768], log)), flush=True)
        return 0
    if args.shape_sweep:
        print(json.dumps(shape_sweep(log)), flush=True)
        return 0
    if args.probe_sweep:
        c = synth.make_case(args.config, R=args.requests or None, with_prefix=False, with_qkv=False)
        fb = forward_bytes(c.R, c.H, c.d, c.FW, c.B)
        print(json.dumps(probe_sweep(fb - c.R * c.B * c.H * c.d * 2, log)), flush=True)
        return 0
    if args.kv_heads:
        print(json.dumps(gqa_cycle(args, log)), flush=True)
        return 0
    io = dict(io=args.io)  # every draw in the chosen token dtype (bf16 values, widened for f32)
    es = 2 if args.io == "bf16" else 4
    case = synth.make_case(args.config, R=args.requests or None, with_prefix=False, with_qkv=False, **io)
    R, H, d, FW, B = case.R, case.H, case.d, case.FW, case.B
    nl, nd = args.layers, args.denoise
    slots = torch.from_numpy(case.slot_ids).to(dev)
    max_blocks = int(case.n_blocks.max())
    T = int(case.n_blocks.sum()) * B

    # each layer's states are built from its whole ragged prefix by one prefill
    # launch (timed); the first launch goes into a scratch pool as a warm-up
    t_setup = time.perf_counter()
    layers, prefill_ms = [], []
    for L in range(nl):
        w, gamma = synth.device_layer_params(args.config, L, dev, **io)
        state = bha.new_state(case.num_slots, H, d, FW, dev)
        pk, pv, offs = synth.device_packed_prefix(args.config, case.n_blocks, dev, layer=L, **io)
        if L == 0:
            bha.state_prefill(pk, pv, offs, w, bha.new_state(case.num_slots, H, d, FW, dev), slots)
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        p0.record()
        bha.state_prefill(pk, pv, offs, w, state, slots)
        p1.record()
        torch.cuda.synchronize()
        prefill_ms.append(p0.elapsed_time(p1))
        if L == 0:
            prefix0 = (pk, pv, offs)  # for the softmax prefix-attention comparison
        del pk, pv
        q, k, v = synth.device_step_qkv(args.config, 0, R, dev, layer=L, **io)
        out = torch.empty_like(q)
        masks = [torch.from_numpy((np.arange(R) % nd == i).astype(np.uint8)).to(dev) for i in range(nd)]
        layers.append(dict(w=w, gamma=gamma, state=state, q=q, k=k, v=v, out=out,
                           stag=[bha.prepare_forward_commit(q, k, v, w, gamma, state, slots, out, commit_mask=m)
                                 for m in masks] if args.staggered else None,
                           fwd=bha.prepare_forward(q, k, v, w, gamma, state, slots, out),
                           com=(bha.prepare_commit(k, v, w, state, slots) if args.separate_commit else
                                bha.prepare_forward_commit(q, k, v, w, gamma, state, slots, out))))
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    pre_avg = sum(prefill_ms) / len(prefill_ms) * 1e-3
    pb = prefill_bytes(T, R, H, d, FW, es)
    log(f"setup: {nl} layers x {R} requests, prefixes {int(case.n_blocks.min()) * B}.."
        f"{max_blocks * B} tokens ({T} total), {time.perf_counter() - t_setup:.1f} s")
    log(f"prefill: avg {pre_avg * 1e6:.1f} us/launch over {nl} layers, {T / pre_avg / 1e6:.1f} M tokens/s, "
        f"{pb / pre_avg / 1e9:.0f} GB/s algorithmic ({pb / 1e9:.2f} GB/launch)")

    # a block cycle: nd denoising steps in every layer; the last one either is
    # the fused forward + commit, or a plain forward followed by a commit
    nd_plain = nd if args.separate_commit else nd - 1
    n_fwd, n_com = nd_plain * nl, nl
    if args.staggered:
        nd_plain, n_fwd, n_com = nd, nd * nl, 0
    # Each step is timed by one event pair around its forwards and one around
    # its commits (per-launch events would add their own cost to the step);
    # a launch's average duration is its group's time over its launches, gaps
    # between back-to-back launches included.
    def ev_pair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def step(evs=None, per_launch=None):
        def run(fn):
            if per_launch is None:
                fn()
            else:
                e0, e1 = ev_pair()
                e0.record()
                fn()
                e1.record()
                per_launch.append((e0, e1))

        if evs is not None:
            evs[0][0].record()
        if args.staggered:
            for i in range(nd):
                for lay in layers:
                    run(lay["stag"][i])
        else:
            for _ in range(nd_plain):
                for lay in layers:
                    run(lay["fwd"])
        if evs is not None:
            evs[0][1].record()
            evs[1][0].record()
        if not args.staggered:
            for lay in layers:
                run(lay["com"])
        if evs is not None:
            evs[1][1].record()

    ev = [(ev_pair(), ev_pair()) for _ in range(args.steps)]
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    fwd_avg = sum(f0.elapsed_time(f1) for (f0, f1), _ in ev) * 1e-3 / (args.steps * n_fwd)
    com_avg = (sum(c0.elapsed_time(c1) for _, (c0, c1) in ev) * 1e-3 / (args.steps * n_com)) if n_com else None
    # the spread of single launches: one more step with an event pair around
    # every launch, outside the timed region
    per_launch = []
    step(per_launch=per_launch)
    torch.cuda.synchronize()
    fwd_ms = [a.elapsed_time(b) for a, b in per_launch[:n_fwd]]
    fb = forward_bytes(R, H, d, FW, B, es)
    if args.staggered:
        # every launch writes back the records of the 1/nd of requests it commits
        F_ = 2 * FW
        fb += sum(1 for r in range(R) if r % nd == 0) * H * (d * F_ * 4 + F_ * 4)
    cb = commit_bytes(R, H, d, FW, B, es) if args.separate_commit else forward_commit_bytes(R, H, d, FW, B, es)
    com_name = "commit" if args.separate_commit else "forward+commit"
    tokens = args.steps * nd * nl * R * B
    value = tokens / elapsed
    if args.staggered:
        log(f"staggered forward+commit: avg {fwd_avg * 1e6:.1f} us/launch, {fb / fwd_avg / 1e9:.0f} GB/s "
            f"algorithmic ({fb / 1e6:.1f} MB/launch)")
        log(f"step: {elapsed / args.steps * 1e3:.2f} ms ({nd} x {nl} launches); {value / 1e6:.1f} M tokens/s")
    else:
        log(f"forward: avg {fwd_avg * 1e6:.1f} us/launch, {fb / fwd_avg / 1e9:.0f} GB/s algorithmic "
            f"({fb / 1e6:.1f} MB/launch); {com_name}: avg {com_avg * 1e6:.1f} us/launch, "
            f"{cb / com_avg / 1e9:.0f} GB/s ({cb / 1e6:.1f} MB/launch)")
        log(f"step: {elapsed / args.steps * 1e3:.2f} ms ({nd_plain} x {nl} forwards + {nl} {com_name}); "
            f"{value / 1e6:.1f} M tokens/s")

    # comparison: exact softmax attention of the same batch over each request's
    # whole prefix and block (what the hybrid forward replaces), layer 0's
    # tokens, timed outside the timed region above
    pk, pv, offs = prefix0
    l0 = layers[0]
    sm_out = torch.empty_like(l0["q"])
    sm = bha.prepare_prefix_attention(l0["q"], l0["k"], l0["v"], pk, pv, offs, sm_out)
    sm()
    sm_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
    for e0, e1 in sm_ev:
        e0.record()
        sm()
        e1.record()
    torch.cuda.synchronize()
    sm_avg = sum(a.elapsed_time(b) for a, b in sm_ev) / len(sm_ev) * 1e-3
    smb = prefix_attention_bytes(T, R, H, d, B, es)
    del sm, sm_out, pk, pv, offs, prefix0
    torch.cuda.empty_cache()
    log(f"softmax prefix attention (same batch, whole prefixes): avg {sm_avg * 1e6:.1f} us/launch, "
        f"{smb / sm_avg / 1e9:.0f} GB/s algorithmic ({smb / 1e9:.2f} GB/launch); "
        f"{sm_avg / fwd_avg:.1f}x the hybrid step's launch")

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 x {args.copy_calibration_mib} MiB device copies")

    # the standalone commit (bha_state_commit), on copies of the states: one
    # event pair around 5 rounds over the layers (consecutive commits touch
    # different layers' pools, as in the cycle)
    com_ms = None
    if not args.staggered:
        snaps = [lay["state"].clone() for lay in layers]
        coms = [bha.prepare_commit(lay["k"], lay["v"], lay["w"], st, slots) for lay, st in zip(layers, snaps)]
        for c in coms:
            c()
        s0, s1 = ev_pair()
        s0.record()
        for _ in range(5):
            for c in coms:
                c()
        s1.record()
        torch.cuda.synchronize()
        com_ms = s0.elapsed_time(s1) / (5 * len(coms))
        del coms, snaps
        torch.cuda.empty_cache()
    scb = commit_bytes(R, H, d, FW, B, es)
    if com_ms is not None:
        log(f"standalone commit: avg {com_ms * 1e3:.1f} us/launch, {scb / com_ms / 1e6:.0f} GB/s algorithmic "
            f"({scb / 1e6:.1f} MB/launch)")

    # the feature map of each layer's queries (bha_feature_map), 5 rounds over the layers
    phi_out = torch.empty((R, B, H, 2 * FW), dtype=torch.float32, device=dev)
    fms = [bha.prepare_feature_map(lay["q"], lay["w"], phi_out) for lay in layers]
    fms[0]()
    f0, f1 = ev_pair()
    f0.record()
    for _ in range(5):
        for fm in fms:
            fm()
    f1.record()
    torch.cuda.synchronize()
    fm_ms = f0.elapsed_time(f1) / (5 * len(fms))
    fmb = feature_map_bytes(R, H, d, FW, B, es)
    del phi_out, fms
    log(f"feature map: avg {fm_ms * 1e3:.1f} us/launch, {fmb / fm_ms / 1e6:.0f} GB/s algorithmic "
        f"({fmb / 1e6:.1f} MB/launch, {R * B * H} token-heads)")

    # context: a plain device-to-device copy of the forward's byte count (read + write)
    ctx_src = torch.empty(fb // 4, dtype=torch.float32, device=dev)
    ctx_dst = torch.empty_like(ctx_src)
    ctx_dst.copy_(ctx_src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        ctx_dst.copy_(ctx_src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * ctx_src.numel() * 4 * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    # and a plain streaming read of the same bytes: sums of 4096-float rows
    # (of torch's reductions the one that streams fastest here)
    ctx_rows = ctx_src[: ctx_src.numel() // 4096 * 4096].view(-1, 4096)
    ctx_sum = torch.empty(ctx_rows.shape[0], dtype=torch.float32, device=dev)
    torch.sum(ctx_rows, dim=1, out=ctx_sum)
    c0.record()
    for _ in range(5):
        torch.sum(ctx_rows, dim=1, out=ctx_sum)
    c1.record()
    torch.cuda.synchronize()
    read_gbps = ctx_rows.numel() * 4 * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del ctx_src, ctx_dst, ctx_sum, ctx_rows
    log(f"context: torch device copy of {fb / 1e6:.0f} MB runs at {copy_gbps:.0f} GB/s (read + write); "
        f"row sums over the same bytes read at {read_gbps:.0f} GB/s")
    out_bytes = R * B * H * d * es
    probes = probe_context(fb - out_bytes, out_bytes, log)

    achieved = fb / fwd_avg / 1e9
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.io,
        "data": "synthetic",
        "config": {
            "workload": (f"{args.config}: continuous-batching decode, {R} requests x {H} heads, d={d}, "
                         f"FW={FW} (F={2 * FW}), B={B}, ragged prefixes {int(case.n_blocks.min()) * B}-"
                         f"{max_blocks * B} tokens; per step {nd} denoising forwards in each of {nl} "
                         f"block-hybrid layers, the block committed "
                         + ("by a separate commit" if args.separate_commit else
                            "with staggered blocks (1/32 of requests per step)" if args.staggered else
                            "within the last forward")),
            "requests": R, "heads": H, "head_dim": d, "feat_half": FW, "block": B,
            "denoise_steps": nd, "layers": nl, "state_dtype": "f32", "io_dtype": args.io,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": (None if args.staggered or args.io != "bf16" or args.requests
                        else read_traffic(args.config)),
            "kernel": ((f"bha_block_forward_commit: forward_commit_mfma_kernel<{d},{FW},"
                        f"{state_store_scope(FW, R * H, dev)}> (1/{nd} of requests "
                        f"commit per launch)" if args.io == "bf16" else
                        f"bha_block_forward_commit: forward_generic_kernel<float,{d},{FW}> then "
                        f"commit_generic_kernel<float,{d},{FW}> (1/{nd} of requests commit per launch)")
                       if args.staggered else
                       f"bha_block_forward: {forward_kernel_name(d, FW, B, R * H, dev)} (persistent, bf16 MFMA)"
                       if args.io == "bf16" else
                       f"bha_block_forward: forward_generic_kernel<float,{d},{FW}> (fp32 MFMA)"),
            "bytes_per_launch": fb,
            "avg_launch_us": fwd_avg * 1e6,
            "launches": args.steps * n_fwd,
            "timing": "one event pair around each step's forwards; average over its launches, gaps included",
            "single_launch_us_p10_median_p90": [float(x) * 1e3 for x in np.percentile(fwd_ms, [10, 50, 90])],
        },
        "context": {"torch_copy_GBps": copy_gbps, "torch_row_sum_read_GBps": read_gbps,
                    "stream_probe": probes,
                    "forward_over_probe": {k_: achieved / p_["GBps"] for k_, p_ in probes.items()},
                    "pages_figures": PAGES_FIGURES},
        "commit": None if args.staggered else {
            "kernel": ("bha_state_commit" if args.separate_commit
                       else "bha_block_forward_commit (last denoising step and commit, one pass)" if args.io == "bf16"
                       else "bha_block_forward_commit (fp32: the forward, then the commit kernel)"),
            "avg_launch_us": com_avg * 1e6,
            "bytes_per_launch": cb,
            "achieved_GBps": cb / com_avg / 1e9,
            "frac": cb / com_avg / 1e9 / PEAK_HBM_GBS,
        },
        "standalone_commit": None if com_ms is None else {
            "kernel": (f"bha_state_commit: commit_mfma_kernel<{d},{FW},{state_store_scope(FW, R * H, dev)}>"
                       if args.io == "bf16" and B <= 32
                       else "bha_state_commit"),
            "avg_launch_us": com_ms * 1e3,
            "bytes_per_launch": scb,
            "achieved_GBps": scb / com_ms / 1e6,
            "frac": scb / com_ms / 1e6 / PEAK_HBM_GBS,
            "committed_tokens_per_s": R * B / (com_ms * 1e-3),
            "timing": "on copies of the states, one event pair around 5 rounds over the layers",
        },
        "feature_map": {
            "kernel": (f"bha_feature_map: feature_map_mfma_kernel<{d},{FW},{fmap_store_scope(d, FW, R * B, H, dev)}>"
                       if args.io == "bf16"
                       else "bha_feature_map: feature_map_generic_kernel<float>"),
            "avg_launch_us": fm_ms * 1e3,
            "bytes_per_launch": fmb,
            "achieved_GBps": fmb / fm_ms / 1e6,
            "frac": fmb / fm_ms / 1e6 / PEAK_HBM_GBS,
        },
        "prefill": {
            "workload": f"one bha_state_prefill launch per layer over all {R} requests' packed prefixes "
                        f"({T} tokens x {H} heads)",
            "avg_launch_us": pre_avg * 1e6,
            "tokens_per_s": T / pre_avg,
            "bytes_per_launch": pb,
            "achieved_GBps": pb / pre_avg / 1e9,
            "frac": pb / pre_avg / 1e9 / PEAK_HBM_GBS,
        },
        "softmax_prefix_attention": {
            "workload": f"bha_prefix_attention on layer 0's batch: the {R * B} block queries attend to their "
                        f"request's whole prefix and block ({T} prefix tokens x {H} heads)",
            "avg_launch_us": sm_avg * 1e6,
            "bytes_per_launch": smb,
            "achieved_GBps": smb / sm_avg / 1e9,
            "frac": smb / sm_avg / 1e9 / PEAK_HBM_GBS,
            "launch_time_over_hybrid_step": sm_avg / fwd_avg,
        },
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(layers[0], case, nd,
                                                                          args.cpu_sample_requests, log),
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
