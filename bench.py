#!/usr/bin/env python3
"""Throughput of the gfx950 Qwen3 attention block on one MI355X.

A step is one prefill forward of the block (q/k/v projection with fused
QK-Norm + RoPE + cache write, causal GQA flash attention, o_proj) over the
Qwen3-0.6B-shaped batch B=2, T=2048 (d=1024, 16 query heads, 8 KV heads,
head dim 128, bf16 storage, fp32 accumulation) on synthetic seeded inputs
already resident in HBM.  The decode path (64 sequences, caches of
1024..32768 tokens) is timed beside it and reported in "decode".

Prints ONE JSON line (the last line of stdout).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention-block tokens/s and TFLOP/s (% MFMA/HBM peak), 0.6B-shape B=2 T=2048"
PEAK_BF16_FLOPS = 2.5e15      # MI355X dense bf16 MFMA
PEAK_HBM_BYTES = 8.0e12       # MI355X HBM3E

# Measured HBM traffic of the roofline kernels (rocprofv3 FETCH_SIZE / WRITE_SIZE,
# calibrated on a plain copy), written by --summarize-pmc; used only while the
# kernel sources still hash to the value recorded with it.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_prefill_B2_T2048_decode_N64.txt")
CSRC = os.path.join(ROOT, "qwen3_gqa_attention_amd", "csrc")
COPY_BYTES = 512 << 20        # bytes read (and written) by one calibration copy
PMC_KERNELS = {               # roofline entry -> kernel-name substrings summed per launch
    "prefill_attention": ["flash_prefill_kernel"],
    # the headline shape's q/k/v (256x256 tiles) and o_proj (128x128, K groups)
    # GEMMs: the flash kernel and the q/k/v GEMM do the same FLOPs, so either
    # can be the dominant kernel of a run
    "prefill_qkv": ["gemm_nt_kernel<unsigned short, 4, 2, 2, 4, true, false, 2, false, 1>"],
    "prefill_oproj": ["gemm_nt_kernel<unsigned short, 2, 2, 2, 2, false, false, 2, false, 2>"],
    "decode_attention": ["decode_attn_kernel", "decode_combine_kernel"],
}
KERNEL_SOURCES = {            # roofline entry -> the sources its kernels are built from
    "prefill_attention": ["flash_prefill.hip", "device_common.hpp", "kernels.hpp"],
    "prefill_qkv": ["gemm.hip", "device_common.hpp", "kernels.hpp"],
    "prefill_oproj": ["gemm.hip", "device_common.hpp", "kernels.hpp"],
    "decode_attention": ["decode.hip", "device_common.hpp", "kernels.hpp"],
}
PREFILL_TRAFFIC_KEY = {"attention": "prefill_attention", "qkv_norm_rope_gemm": "prefill_qkv",
                       "o_proj_gemm": "prefill_oproj"}


def code_only(text):
    """C++ source without its comments, trailing blanks and blank lines (an
    edit to comments alone does not change a kernel)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def kernel_source_hash(key):
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[key]:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + code_only(f.read()).encode())
    return h.hexdigest()[:16]


def load_traffic():
    """Per-launch HBM bytes of the roofline kernels whose sources are unchanged
    since the counters were taken ({} entries are dropped otherwise)."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = [l for l in f if l.startswith("TRAFFIC_JSON ")]
        rec = json.loads(lines[-1][len("TRAFFIC_JSON "):])
    except (OSError, IndexError, ValueError):
        return {}
    hashes = rec.get("source_hash", {})
    return {k: v for k, v in rec.get("bytes_per_launch", {}).items()
            if isinstance(hashes, dict) and hashes.get(k) == kernel_source_hash(k)}


def copy_calibration():
    """A plain device copy of known size (the PMC runs scale their counters by it)."""
    import torch
    n = COPY_BYTES // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def summarize_pmc(fetch_csv, write_csv, commands):
    """Turn two rocprofv3 counter CSVs into the traffic file."""
    import csv
    import statistics

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")

    def avg(vals, subs):
        tot = 0.0
        for sub in subs:
            ks = [k for k in vals if sub in k]
            if not ks:
                raise SystemExit(f"no dispatches of {sub} in the counter CSV")
            tot += statistics.mean(v for k in ks for v in vals[k])
        return tot

    copy_kib = COPY_BYTES / 1024
    cf, cw = avg(fetch, ["neg_kernel"]), avg(write, ["neg_kernel"])
    sf, sw = copy_kib / cf, copy_kib / cw
    out = {}
    lines = ["HBM traffic per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch),",
             "each scaled by what the counter reads for a plain copy of known size",
             f"(torch.neg over {COPY_BYTES >> 20} MiB of bf16: {copy_kib:.0f} KiB read, {copy_kib:.0f} KiB written).",
             "", "Commands (from /tmp, TMPDIR=/tmp, one MI355X):"] + [f"    {c}" for c in commands] + [
             "", f"copy kernel: FETCH_SIZE {cf:.0f} KiB -> fetch scale {sf:.4f}; "
                 f"WRITE_SIZE {cw:.0f} KiB -> write scale {sw:.4f}", "",
             "| kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | scaled traffic (MB) |", "|---|---|---|---|"]
    for key, subs in PMC_KERNELS.items():
        f_, w_ = avg(fetch, subs), avg(write, subs)
        b = (f_ * sf + w_ * sw) * 1024
        out[key] = b
        lines.append(f"| {key} ({' + '.join(subs)}) | {f_:.0f} | {w_:.0f} | {b / 1e6:.2f} |")
    rec = {"source_hash": {k: kernel_source_hash(k) for k in PMC_KERNELS}, "bytes_per_launch": out,
           "copy_scale": {"fetch": sf, "write": sw}}
    lines += ["", "TRAFFIC_JSON " + json.dumps(rec)]
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def prefill_flops(B, T, d, n_q, n_kv, dh=128):
    """Algorithmic FLOPs per kernel of one prefill call."""
    M = B * T
    return {
        "qkv_norm_rope_gemm": 2.0 * M * (n_q + 2 * n_kv) * dh * d,
        "attention": 2.0 * B * n_q * dh * T * (T + 1),   # causal QK^T and PV incl. diagonal
        "o_proj_gemm": 2.0 * M * d * n_q * dh,
    }


MIN_TIMED_S = 0.2      # duration-timed entries run at least this long ...
MIN_TIMED_STEPS = 50   # ... and at least this many steps


def steps_for_duration(step_s):
    """Steps for a timed region of at least MIN_TIMED_S and MIN_TIMED_STEPS steps."""
    import math
    return max(MIN_TIMED_STEPS, int(math.ceil(MIN_TIMED_S / max(step_s, 1e-9))))


def decode_timing(args, fn):
    """Warm-up, then the timed step count of a decode workload: --decode-steps
    if given, else by duration (as the prefill shapes)."""
    import torch
    for _ in range(max(args.warmup, 10)):
        fn()
    torch.cuda.synchronize()
    return args.decode_steps if args.decode_steps > 0 else steps_for_duration(estimate_step_s(fn))


def estimate_step_s(fn, n=5):
    """Mean time of n back-to-back calls (after the caller's warm-up)."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / n


def prepare_prefill(layer=False, idx=2):
    """Handle, resident inputs, caches and workspace of the prefill of workload idx."""
    import numpy as np
    import torch

    import qwen3_gqa_attention_amd as q3
    from workloads import EPS, ROPE_THETA, WORKLOADS, prefill_inputs

    w = WORKLOADS[idx]
    B, T = w.B, w.T
    inp = prefill_inputs(w)
    bf = torch.bfloat16
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(bf)
    g_in = None
    if layer:
        g_in = d(1 + 0.1 * np.random.default_rng(w.seed + 2).standard_normal(w.d))
    blk = q3.Qwen3Attention(d(inp["Wq"]), d(inp["Wk"]), d(inp["Wv"]), d(inp["Wo"]), d(inp["gq"]),
                            d(inp["gk"]), n_q=w.n_q, n_kv=w.n_kv, eps=EPS, rope_theta=ROPE_THETA,
                            input_norm=g_in)
    x = d(inp["X"])
    pos = torch.from_numpy(inp["positions"]).cuda()
    kc = torch.empty((B, w.n_kv, T, 128), dtype=bf, device="cuda")
    vc = torch.empty_like(kc)
    out = torch.empty_like(x)
    ws = torch.empty(blk.workspace_size(False, B, T), dtype=torch.uint8, device="cuda")
    return w, blk, x, pos, kc, vc, out, ws


def bench_prefill(args, layer=False, idx=2, steps=None, prepared=None):
    """The prefill of workload idx (default: the 0.6B shape, B=2, T=2048); with
    layer=True the block carries the fused input RMSNorm and residual add (the
    attention half of a decoder layer).  steps=None: args.steps (the headline);
    steps="duration": enough steps for MIN_TIMED_S and MIN_TIMED_STEPS.
    prepared: the result of prepare_prefill(layer, idx), made earlier."""
    import torch

    import qwen3_gqa_attention_amd as q3

    w, blk, x, pos, kc, vc, out, ws = prepared or prepare_prefill(layer, idx)
    B, T = w.B, w.T
    for _ in range(args.warmup):
        blk.prefill(x, pos, kc, vc, out=out, workspace=ws)
    torch.cuda.synchronize()
    if steps == "duration":
        steps = steps_for_duration(estimate_step_s(
            lambda: blk.prefill(x, pos, kc, vc, out=out, workspace=ws)))
    steps = steps or args.steps

    # timed region 1: K plain steps -> the reported throughput
    t0 = time.perf_counter()
    for _ in range(steps):
        blk.prefill(x, pos, kc, vc, out=out, workspace=ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # timed region 2: K more steps with HIP events recorded by the library
    # between its kernels, on the stream it launches on -> per-kernel
    # durations (the events add a few microseconds per step, so this pass is
    # not the one `value` comes from)
    blk.enable_stage_timing(steps)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(steps):
        blk.prefill(x, pos, kc, vc, out=out, workspace=ws)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    stage_ms, ncalls = blk.stage_times()
    blk.enable_stage_timing(0)

    step_s = (t1 - t0) / steps
    step_events_s = (t3 - t2) / steps
    flops = prefill_flops(B, T, w.d, w.n_q, w.n_kv)
    kernels = {}
    for name, tot in zip(q3.STAGES, stage_ms):
        avg = tot / max(ncalls, 1) / 1e3
        kernels[name] = {"avg_ms": avg * 1e3, "gflop": flops[name] / 1e9,
                         "tflops": flops[name] / avg / 1e12 if avg > 0 else None,
                         "frac_mfma_peak": flops[name] / avg / PEAK_BF16_FLOPS if avg > 0 else None}
    dom = max(kernels, key=lambda k: kernels[k]["avg_ms"])
    total_flops = sum(flops.values())
    blk.close()
    return dict(B=B, T=T, w=w, step_s=step_s, step_events_s=step_events_s, kernels=kernels,
                dominant=dom, flops=flops, total_flops=total_flops, ncalls=ncalls, steps=steps)


def chunk_flops(B, T, P, d, n_q, n_kv, dh=128):
    """Algorithmic FLOPs per kernel of one chunked-prefill call (T new tokens
    over P cached ones: token t sees P + t + 1 keys)."""
    M = B * T
    return {
        "qkv_norm_rope_gemm": 2.0 * M * (n_q + 2 * n_kv) * dh * d,
        "attention": 4.0 * B * n_q * dh * (T * P + T * (T + 1) / 2),
        "o_proj_gemm": 2.0 * M * d * n_q * dh,
    }


def bench_chunk(args, P=1536, T=512):
    """Chunked prefill: the 0.6B shape, B=2, a T-token chunk over P cached tokens."""
    import numpy as np
    import torch

    import qwen3_gqa_attention_amd as q3
    from workloads import EPS, ROPE_THETA, WORKLOADS, prefill_inputs

    w = WORKLOADS[2]
    B = w.B
    inp = prefill_inputs(w, B=B, T=T)
    bf = torch.bfloat16
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(bf)
    blk = q3.Qwen3Attention(d(inp["Wq"]), d(inp["Wk"]), d(inp["Wv"]), d(inp["Wo"]), d(inp["gq"]),
                            d(inp["gk"]), n_q=w.n_q, n_kv=w.n_kv, eps=EPS, rope_theta=ROPE_THETA)
    x = d(inp["X"])
    pos = (torch.arange(T, dtype=torch.int32, device="cuda") + P).repeat(B, 1).contiguous()
    past = torch.full((B,), P, dtype=torch.int32, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 1)
    kc = torch.randn((B, w.n_kv, P + T, 128), generator=gen, device="cuda").to(bf)
    vc = torch.randn((B, w.n_kv, P + T, 128), generator=gen, device="cuda").to(bf)
    out = torch.empty_like(x)
    ws = torch.empty(blk.workspace_size(False, B, T), dtype=torch.uint8, device="cuda")
    for _ in range(args.warmup):
        blk.prefill_chunk(x, pos, past, kc, vc, out=out, workspace=ws)
    torch.cuda.synchronize()
    steps = steps_for_duration(estimate_step_s(
        lambda: blk.prefill_chunk(x, pos, past, kc, vc, out=out, workspace=ws)))
    t0 = time.perf_counter()
    for _ in range(steps):
        blk.prefill_chunk(x, pos, past, kc, vc, out=out, workspace=ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    blk.enable_stage_timing(steps)
    for _ in range(steps):
        blk.prefill_chunk(x, pos, past, kc, vc, out=out, workspace=ws)
    torch.cuda.synchronize()
    stage_ms, ncalls = blk.stage_times()
    blk.enable_stage_timing(0)
    blk.close()
    step_s = (t1 - t0) / steps
    flops = chunk_flops(B, T, P, w.d, w.n_q, w.n_kv)
    kernels = {}
    for name, tot in zip(q3.STAGES, stage_ms):
        avg = tot / max(ncalls, 1) / 1e3
        kernels[name] = {"avg_ms": avg * 1e3, "tflops": flops[name] / avg / 1e12,
                         "frac_mfma_peak": flops[name] / avg / PEAK_BF16_FLOPS}
    total = sum(flops.values())
    return {"workload": f"{w.name}-chunk-T{T}-past{P}", "B": B, "T": T, "past": P,
            "steps": steps, "ms_per_step": step_s * 1e3, "tokens_per_s": B * T / step_s,
            "tflops": total / step_s / 1e12, "frac_mfma_peak": total / step_s / PEAK_BF16_FLOPS,
            "kernels": kernels}


def decode_caches():
    """The 64-sequence decode workload's KV caches (N(0,1) entries, bf16)."""
    import torch

    from workloads import WORKLOADS

    w = WORKLOADS[5]
    bf = torch.bfloat16
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    kc = torch.empty((w.B, w.n_kv, w.cap, 128), dtype=bf, device="cuda")
    vc = torch.empty_like(kc)
    for s in range(w.B):   # drawn per sequence to bound the fp32 temporary
        kc[s] = torch.randn((w.n_kv, w.cap, 128), generator=gen, device="cuda").to(bf)
        vc[s] = torch.randn((w.n_kv, w.cap, 128), generator=gen, device="cuda").to(bf)
    return kc, vc


def bench_decode(args, window=0, caches=None):
    """The 64-sequence decode; window > 0 makes it a sliding-window layer.
    caches: (k, v) from decode_caches() to reuse (the full and the windowed
    decode share one allocation, as a server keeps its cache), else drawn
    here and freed at the end."""
    import numpy as np
    import torch

    import qwen3_gqa_attention_amd as q3
    from workloads import EPS, ROPE_THETA, WORKLOADS, decode_inputs

    w = WORKLOADS[5]
    inp = decode_inputs(w)
    L = inp["positions"]
    bf = torch.bfloat16
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(bf)
    blk = q3.Qwen3Attention(d(inp["Wq"]), d(inp["Wk"]), d(inp["Wv"]), d(inp["Wo"]), d(inp["gq"]),
                            d(inp["gk"]), n_q=w.n_q, n_kv=w.n_kv, eps=EPS, rope_theta=ROPE_THETA,
                            sliding_window=window)
    own = caches is None
    kc, vc = decode_caches() if own else caches
    x = d(inp["X"])
    pos = torch.from_numpy(L).cuda()
    out = torch.empty_like(x)
    ws = torch.empty(blk.workspace_size(True, w.B, 1, w.cap), dtype=torch.uint8, device="cuda")
    steps = decode_timing(args, lambda: blk.decode(x, pos, kc, vc, out=out, workspace=ws))
    t0 = time.perf_counter()
    for _ in range(steps):
        blk.decode(x, pos, kc, vc, out=out, workspace=ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    blk.enable_stage_timing(steps)   # second pass: per-kernel durations from HIP events
    torch.cuda.synchronize()
    for _ in range(steps):
        blk.decode(x, pos, kc, vc, out=out, workspace=ws)
    torch.cuda.synchronize()
    stage_ms, ncalls = blk.stage_times()
    blk.enable_stage_timing(0)
    blk.close()
    step_s = (t1 - t0) / steps
    # algorithmic bytes: each cached key/value row read once (bf16), plus the
    # new token's q/k/v/o weights and the small activations; a window of W
    # reads the W - 1 most recent cached rows
    seen = L.astype(np.int64) if window == 0 else np.minimum(L.astype(np.int64), window - 1)
    kv_read = float(np.sum(seen)) * 2 * w.n_kv * 128 * 2
    weights = (w.n_q + 2 * w.n_kv) * 128 * w.d * 2 + w.d * w.n_q * 128 * 2
    attn_ms = stage_ms[1] / max(ncalls, 1)
    attn_bytes = kv_read + w.B * w.n_kv * 2 * 128 * 2 + 2 * w.B * w.n_q * 128 * 2
    if own:
        del kc, vc
        torch.cuda.empty_cache()
    return dict(step_s=step_s, kv_read=kv_read, weights=weights, stage_ms=[m / max(ncalls, 1) for m in stage_ms],
                attn_ms=attn_ms, attn_bytes=attn_bytes, N=w.B, mean_len=float(L.mean()), w=w,
                steps=steps)


def bench_decode_paged(args, bs=64):
    """Decode over a paged cache: the same 64 sequences, their keys/values in
    64-token blocks of one pool, the blocks of all sequences shuffled."""
    import numpy as np
    import torch

    import qwen3_gqa_attention_amd as q3
    from workloads import EPS, ROPE_THETA, WORKLOADS, decode_inputs

    w = WORKLOADS[5]
    inp = decode_inputs(w)
    L = inp["positions"]
    bf = torch.bfloat16
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(bf)
    blk = q3.Qwen3Attention(d(inp["Wq"]), d(inp["Wk"]), d(inp["Wv"]), d(inp["Wo"]), d(inp["gq"]),
                            d(inp["gk"]), n_q=w.n_q, n_kv=w.n_kv, eps=EPS, rope_theta=ROPE_THETA)
    need = (L.astype(np.int64) + bs) // bs          # blocks for L + 1 tokens
    mb, nb = int(need.max()), int(need.sum())
    perm = np.random.default_rng(w.seed + 11).permutation(nb).astype(np.int32)
    table = np.zeros((w.B, mb), np.int32)
    off = 0
    for s in range(w.B):
        table[s, : need[s]] = perm[off: off + need[s]]
        table[s, need[s]:] = perm[off + need[s] - 1]
        off += need[s]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 12)
    kp = torch.empty((nb, w.n_kv, bs, 128), dtype=bf, device="cuda")
    vp = torch.empty_like(kp)
    for lo in range(0, nb, 4096):   # N(0,1) blocks, drawn in slices to bound the fp32 temporary
        hi = min(nb, lo + 4096)
        kp[lo:hi] = torch.randn((hi - lo, w.n_kv, bs, 128), generator=gen, device="cuda").to(bf)
        vp[lo:hi] = torch.randn((hi - lo, w.n_kv, bs, 128), generator=gen, device="cuda").to(bf)
    x = d(inp["X"])
    pos = torch.from_numpy(L).cuda()
    tab = torch.from_numpy(table).cuda()
    out = torch.empty_like(x)
    ws = torch.empty(blk.workspace_size(True, w.B, 1, mb * bs), dtype=torch.uint8, device="cuda")
    steps = decode_timing(args, lambda: blk.decode_paged(x, pos, tab, kp, vp, out=out,
                                                          workspace=ws))
    t0 = time.perf_counter()
    for _ in range(steps):
        blk.decode_paged(x, pos, tab, kp, vp, out=out, workspace=ws)
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / steps
    blk.close()
    del kp, vp
    torch.cuda.empty_cache()
    nbytes = float(np.sum(L.astype(np.int64))) * 2 * w.n_kv * 128 * 2 + \
        ((w.n_q + 2 * w.n_kv) * 128 * w.d * 2 + w.d * w.n_q * 128 * 2)
    return {"workload": f"{w.name}-paged-bs{bs}", "block_size": bs, "blocks": nb, "steps": steps,
            "ms_per_step": step_s * 1e3, "tokens_per_s": w.B / step_s,
            "GBps": nbytes / step_s / 1e9, "frac_hbm_peak": nbytes / step_s / PEAK_HBM_BYTES}


def bench_prefill_cold(args, calls=50, flush_mb=512):
    """Per-call HIP-event times of the 0.6B-shaped prefill, hot (back to back)
    and cold (a 512 MB buffer rewritten before each call evicts the block's
    ~80 MB working set from L2 and the Infinity Cache); median and minimum."""
    import numpy as np
    import torch

    import qwen3_gqa_attention_amd as q3
    from workloads import EPS, ROPE_THETA, WORKLOADS, prefill_inputs

    w = WORKLOADS[2]
    B, T = w.B, w.T
    inp = prefill_inputs(w)
    bf = torch.bfloat16
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(bf)
    blk = q3.Qwen3Attention(d(inp["Wq"]), d(inp["Wk"]), d(inp["Wv"]), d(inp["Wo"]), d(inp["gq"]),
                            d(inp["gk"]), n_q=w.n_q, n_kv=w.n_kv, eps=EPS, rope_theta=ROPE_THETA)
    x = d(inp["X"])
    pos = torch.from_numpy(inp["positions"]).cuda()
    kc = torch.empty((B, w.n_kv, T, 128), dtype=bf, device="cuda")
    vc = torch.empty_like(kc)
    out = torch.empty_like(x)
    ws = torch.empty(blk.workspace_size(False, B, T), dtype=torch.uint8, device="cuda")
    flush = torch.empty(flush_mb << 20, dtype=torch.uint8, device="cuda")
    res = {}
    for mode in ("hot", "cold"):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(calls)]
        for _ in range(5):
            blk.prefill(x, pos, kc, vc, out=out, workspace=ws)
        for e0, e1 in ev:
            if mode == "cold":
                flush.fill_(1)
            e0.record()
            blk.prefill(x, pos, kc, vc, out=out, workspace=ws)
            e1.record()
        torch.cuda.synchronize()
        ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
        res[mode] = {"median_ms": ms[len(ms) // 2], "min_ms": ms[0]}
    blk.close()
    del flush
    torch.cuda.empty_cache()
    return res


def cpu_info():
    """The host CPU's model name and logical CPU count, and the BLAS threads numpy uses."""
    from threadpoolctl import threadpool_info
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return model, os.cpu_count(), int(threads)


def cpu_baseline():
    """The oracle (its own code, run in float32) on the host's cores: the
    headline prefill (median of 3), the 4B prefill (one run), the wide-GQA
    shape over its first 2048 tokens (one run), and one decode step of 8 of the
    64 decode sequences at their own cache lengths.  About 20-40 s of CPU."""
    import statistics

    import numpy as np

    import oracle
    from workloads import (EPS, ROPE_THETA, WORKLOADS, decode_cache_host, decode_inputs,
                           prefill_inputs)

    def prefill_time(idx, T=None):
        w = WORKLOADS[idx]
        inp = prefill_inputs(w, T=T)
        a = [inp[k] for k in ("X", "Wq", "Wk", "Wv", "Wo", "gq", "gk", "positions")]
        t0 = time.perf_counter()
        oracle.prefill(*a, n_q=w.n_q, n_kv=w.n_kv, eps=EPS, theta=ROPE_THETA, dtype=np.float32)
        return time.perf_counter() - t0, w, inp["X"].shape[0] * inp["X"].shape[1]

    runs = [prefill_time(2) for _ in range(3)]
    head_s = statistics.median(r[0] for r in runs)
    tokens = runs[0][2]
    other = {}
    for idx, T, note in ((3, None, "one run, full size"), (4, 2048, "one run, first 2048 tokens")):
        t, w, n = prefill_time(idx, T)
        other[w.name] = {"sample": note, "tokens": n, "seconds": t, "tokens_per_s": n / t}
    # decode: 8 of the 64 sequences (the first 8 of the seeded draw), their caches on the host
    w = WORKLOADS[5]
    full = decode_inputs(w)
    lens = full["lengths"][:8].astype(np.int32)
    inp = decode_inputs(w, N=8)
    kc, vc = decode_cache_host(w, lens, int(lens.max()) + 1)
    t0 = time.perf_counter()
    oracle.decode(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], inp["gq"], inp["gk"], lens,
                  kc, vc, n_q=w.n_q, n_kv=w.n_kv, eps=EPS, theta=ROPE_THETA, dtype=np.float32)
    dt = time.perf_counter() - t0
    nbytes = float(lens.astype(np.int64).sum()) * 2 * w.n_kv * 128 * 2   # bf16 cache rows read
    other[w.name] = {"sample": "one step of 8 of the 64 sequences", "cache_tokens": int(lens.sum()),
                     "seconds": dt, "tokens_per_s": 8 / dt, "GBps_bf16_cache_bytes": nbytes / dt / 1e9}
    model, ncpu, threads = cpu_info()
    return {"value": tokens / head_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"median of 3 oracle.prefill (float32) runs of the full B=2, T=2048 0.6B-shaped "
                      f"batch ({', '.join(f'{r[0]:.2f}' for r in runs)} s); host: {model}, "
                      f"{ncpu} logical CPUs, numpy BLAS on {threads} threads",
            "cpu_model": model, "logical_cpus": ncpu, "other": other}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=0,
                    help="timed steps of each decode workload (0: by duration, at least "
                         f"{MIN_TIMED_S} s and {MIN_TIMED_STEPS} steps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="run only the prefill step and the full-attention decode (the two "
                         "roofline kernels), e.g. under a profiler")
    ap.add_argument("--only", choices=["4b", "wide-gqa", "chunk", "decode", "decode-window",
                                       "decode-paged"],
                    help="time one secondary workload alone and print its own JSON line "
                         "(for profiling it by itself; not the headline line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain copy of known size (for PMC traffic calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic file from two rocprofv3 counter CSVs and exit")
    ap.add_argument("--pmc-command", action="append", default=[],
                    help="command line recorded in the traffic file (repeatable)")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.pmc_command)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the block's multi-GPU sharding is a design note, not a measured path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import qwen3_gqa_attention_amd as q3
    if not os.path.exists(q3.LIB_PATH):
        from qwen3_gqa_attention_amd.build import build
        build()
    torch.cuda.set_device(0)

    if args.only:
        if args.only == "chunk":
            r = bench_chunk(args)
        elif args.only == "decode-paged":
            r = bench_decode_paged(args)
        elif args.only.startswith("decode"):
            W = 4096 if args.only == "decode-window" else 0
            dd = bench_decode(args, window=W)
            nbytes = dd["kv_read"] + dd["weights"]
            r = {"workload": dd["w"].name + (f"-window{W}" if W else ""), "window": W,
                 "steps": dd["steps"], "ms_per_step": dd["step_s"] * 1e3,
                 "GBps": nbytes / dd["step_s"] / 1e9,
                 "frac_hbm_peak": nbytes / dd["step_s"] / PEAK_HBM_BYTES,
                 "kernel_ms": dict(zip(q3.STAGES, dd["stage_ms"]))}
        else:
            pc = bench_prefill(args, idx=3 if args.only == "4b" else 4, steps="duration")
            r = {"workload": pc["w"].name, "B": pc["B"], "T": pc["T"], "steps": pc["steps"],
                 "ms_per_step": pc["step_s"] * 1e3,
                 "tokens_per_s": pc["B"] * pc["T"] / pc["step_s"],
                 "frac_mfma_peak": pc["total_flops"] / pc["step_s"] / PEAK_BF16_FLOPS,
                 "kernels": pc["kernels"]}
        print(json.dumps(r), flush=True)
        return
    if args.copy_calibration:
        copy_calibration()
    traffic = load_traffic()

    def headline(prepared=None):
        log("bench: prefill 0.6B-shape B=2 T=2048 bf16")
        hp = bench_prefill(args, prepared=prepared)
        log(f"bench: prefill {hp['step_s'] * 1e3:.4f} ms/step; kernels " +
            ", ".join(f"{k} {v['avg_ms']:.4f} ms" for k, v in hp["kernels"].items()))
        return hp

    layer = chunk = dec_window = dec_paged = cold = dec = p = pl = None
    other = {}
    extras = not args.headline_only
    # With the other workloads the headline prefill is measured last, its
    # inputs prepared beforehand so that its W warm-up steps follow the
    # chunked prefill with no idle gap: they start on a GPU already at working
    # clocks, as in service.  (After an idle gap for input generation, a
    # 5-step warm-up left the 20 timed steps up to 10% slower than 200 warm-up
    # steps did on the same box.)  Alone (--headline-only, e.g. under a
    # profiler) it runs first.
    if not extras:
        p = headline()
    else:
        prep = prepare_prefill()
        prep_layer = prepare_prefill(layer=True)
    dcache = None
    if not args.no_decode:
        log("bench: decode 64 sequences, caches 1024..32768")
        dcache = decode_caches()
        dd = bench_decode(args, caches=dcache)
        log(f"bench: decode {dd['step_s'] * 1e3:.4f} ms/step, attention kernels {dd['attn_ms']:.4f} ms")
        dec = {
            "workload": dd["w"].name, "sequences": dd["N"], "mean_cache_len": dd["mean_len"],
            "steps": dd["steps"],
            "ms_per_step": dd["step_s"] * 1e3, "tokens_per_s": dd["N"] / dd["step_s"],
            "bytes_per_step": dd["kv_read"] + dd["weights"],
            "GBps": (dd["kv_read"] + dd["weights"]) / dd["step_s"] / 1e9,
            "frac_hbm_peak": (dd["kv_read"] + dd["weights"]) / dd["step_s"] / PEAK_HBM_BYTES,
            "kernel_ms": dict(zip(q3.STAGES, dd["stage_ms"])),
            "roofline": {"bound": "hbm", "kernel": "attention (split-K + combine)",
                         "achieved": dd["attn_bytes"] / (dd["attn_ms"] / 1e3) / 1e9,
                         "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                         "frac": dd["attn_bytes"] / (dd["attn_ms"] / 1e3) / PEAK_HBM_BYTES,
                         "traffic": traffic.get("decode_attention")},
        }
    if extras and not args.no_decode:
        W = 4096
        log(f"bench: decode, the same 64 sequences in a sliding-window layer (W={W})")
        dw = bench_decode(args, window=W, caches=dcache)
        nbytes = dw["kv_read"] + dw["weights"]
        dec_window = {"workload": f"{dw['w'].name}-window{W}", "window": W, "steps": dw["steps"],
                      "ms_per_step": dw["step_s"] * 1e3, "tokens_per_s": dw["N"] / dw["step_s"],
                      "bytes_per_step": nbytes, "GBps": nbytes / dw["step_s"] / 1e9,
                      "frac_hbm_peak": nbytes / dw["step_s"] / PEAK_HBM_BYTES,
                      "kernel_ms": dict(zip(q3.STAGES, dw["stage_ms"]))}
        log(f"bench: window decode {dec_window['ms_per_step']:.4f} ms/step, "
            f"{dec_window['frac_hbm_peak'] * 100:.1f}% of HBM peak")
        log("bench: decode over a paged cache (64-token blocks, shuffled pool)")
        dec_paged = bench_decode_paged(args)
        log(f"bench: paged decode {dec_paged['ms_per_step']:.4f} ms/step, "
            f"{dec_paged['frac_hbm_peak'] * 100:.1f}% of HBM peak")
    if dcache is not None:
        # freed only now, so that no decode workload runs on memory just
        # released by another (a freshly re-allocated 8.6 GB cache measured
        # 3-5% slower than the first allocation)
        del dcache
        torch.cuda.empty_cache()
    if extras:
        log("bench: prefill per-call times, hot and with the caches flushed")
        cold = bench_prefill_cold(args)
        log(f"bench: prefill per call: hot median {cold['hot']['median_ms']:.4f} ms, "
            f"cold median {cold['cold']['median_ms']:.4f} ms")
        for idx in (3, 4):
            pc = bench_prefill(args, idx=idx, steps="duration")
            wc = pc["w"]
            other[wc.name] = {
                "B": pc["B"], "T": pc["T"], "steps": pc["steps"], "ms_per_step": pc["step_s"] * 1e3,
                "tokens_per_s": pc["B"] * pc["T"] / pc["step_s"],
                "tflops": pc["total_flops"] / pc["step_s"] / 1e12,
                "frac_mfma_peak": pc["total_flops"] / pc["step_s"] / PEAK_BF16_FLOPS,
                "kernels": pc["kernels"]}
            log(f"bench: prefill {wc.name}: {pc['step_s'] * 1e3:.4f} ms/step, "
                f"{other[wc.name]['frac_mfma_peak'] * 100:.1f}% of MFMA peak")
        log("bench: chunked prefill 0.6B-shape B=2, 512 tokens over 1536 cached")
        chunk = bench_chunk(args)
        p = headline(prep)
        log("bench: the same prefill with the fused input RMSNorm + residual add")
        pl = bench_prefill(args, layer=True, prepared=prep_layer)
        log(f"bench: layer prefill {pl['step_s'] * 1e3:.4f} ms/step")
        log(f"bench: chunked prefill {chunk['ms_per_step']:.4f} ms/step, "
            f"{chunk['frac_mfma_peak'] * 100:.1f}% of MFMA peak")
        layer = {"workload": f"{pl['w'].name}-input-norm-residual",
                 "ms_per_step": pl["step_s"] * 1e3,
                 "tokens_per_s": pl["B"] * pl["T"] / pl["step_s"],
                 "overhead_vs_block": pl["step_s"] / p["step_s"] - 1.0,
                 "kernel_ms": {k: v["avg_ms"] for k, v in pl["kernels"].items()}}
        log(f"bench: layer prefill {layer['overhead_vs_block'] * 100:+.1f}% vs the block alone")
    cpu = None
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle, float32)")
        cpu = cpu_baseline()

    w = p["w"]
    dom = p["dominant"]
    dk = p["kernels"][dom]
    tokens = p["B"] * p["T"]
    line = {
        "metric": METRIC,
        "value": tokens / p["step_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": p["step_s"] * 1e3,
        "ms_per_step_with_stage_events": p["step_events_s"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": p["B"], "T": p["T"], "d": w.d, "n_q": w.n_q,
                   "n_kv": w.n_kv, "d_head": w.dh, "parallelism": "none (1 GPU)"},
        "tflops": p["total_flops"] / p["step_s"] / 1e12,
        "frac_mfma_peak": p["total_flops"] / p["step_s"] / PEAK_BF16_FLOPS,
        "kernels": p["kernels"],
        "roofline": {"bound": "mfma", "kernel": dom,
                     "achieved": p["flops"][dom] / (dk["avg_ms"] / 1e3) / 1e12,
                     "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                     "frac": p["flops"][dom] / (dk["avg_ms"] / 1e3) / PEAK_BF16_FLOPS,
                     "traffic": traffic.get(PREFILL_TRAFFIC_KEY[dom])},
        "prefill_per_call": cold,
        "prefill_other_shapes": other,
        "layer_prefill": layer,
        "chunked_prefill": chunk,
        "decode": dec,
        "decode_paged": dec_paged,
        "decode_window": dec_window,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
