"""Benchmark: one decode step of the 2-bit MLA cache at the serving shape.

A step is one pass of the whole hot path over one batch: quantize-append of
the new token of each request (rotate, standardize, threshold, pack, RoPE
copy) followed by absorbed-MLA decode attention over the paged 2-bit cache
(split-KV + merge).  Default workload: 4 requests x 262,144 context tokens,
16 heads, latent 512 + RoPE 64, group 128 (DeepSeek-V2-Lite MLA shapes at the
pages' 256K-input, 4-concurrent-request serving point).

Prints one JSON line.  `value` is context tokens per second of the whole step
with every input already resident in HBM; `roofline` reports the decode call
against MI355X's 8 TB/s HBM; `cpu_baseline` times the CPU oracle on the same
step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "2-bit MLA decode context tokens/s and HBM GB/s (% peak) at B=4, 256K ctx"
HBM_PEAK_GBPS = 8000.0
BYTES_PER_TOKEN = 288          # 128 B codes + 32 B fp32 stats + 128 B bf16 RoPE key
BYTES_PER_PROTECTED = 1152     # 1024 B bf16 latent + 128 B RoPE key
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic_v2lite_256k.json")
KERNEL_SOURCES = ["decode_attention_rlq_amd/csrc/rlq_decode.hip",
                  "decode_attention_rlq_amd/csrc/rlq_internal.h"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_decode_bytes(batch, heads, ctx_lens, n_sink=0, n_recent=0):
    prot = sum(min(int(c), n_sink + n_recent) for c in ctx_lens)
    toks = int(sum(int(c) for c in ctx_lens))
    return ((toks - prot) * BYTES_PER_TOKEN + prot * BYTES_PER_PROTECTED
            + batch * heads * (512 + 64) * 2 + batch * heads * 512 * 4)


def measured_traffic():
    """Per-launch HBM bytes from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    return t.get("traffic_bytes_per_launch")


def cpu_baseline(prob, new_idx):
    """Time the oracle on the same decode step (append of the new tokens +
    decode over the full contexts) on the host cores."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    log("cpu baseline: oracle setup (quantize the whole cache)")
    oc = oracle.new_cache(prob.num_pages)
    oracle.quantize_append(oc, prob.tau, prob.k_rope_bits, prob.cu_seqlens, prob.start_pos,
                           prob.block_table, latent_bf16=prob.latent_bits,
                           rotation_bf16=prob.rotation_bits)
    log("cpu baseline: timed oracle step")
    t0 = time.perf_counter()
    oracle.quantize_append(oc, prob.tau, prob.k_rope_bits[new_idx], np.arange(prob.batch + 1),
                           prob.ctx_lens - 1, prob.block_table,
                           latent_bf16=prob.latent_bits[new_idx], rotation_bf16=prob.rotation_bits)
    oracle.decode(oc, prob.q_c_bits, prob.q_r_bits, prob.sm_scale, prob.block_table, prob.ctx_lens,
                  prob.gain, prob.level_inner, prob.level_outer)
    dt = time.perf_counter() - t0
    toks = int(prob.ctx_lens.sum())
    return {"value": toks / dt, "unit": "context tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one full step of the same workload ({prob.batch} x {int(prob.ctx_lens[0])} "
                      f"context tokens: append {prob.batch} tokens + decode), fp64 numpy, "
                      f"{dt:.2f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="v2lite_256k")
    ap.add_argument("--replicas", type=int, default=2,
                    help="cache copies cycled per step so no step reads a cache the MALL still holds")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 3}))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is described in DESIGN.md but not built.", file=sys.stderr)
        sys.exit(2)

    import torch
    from decode_attention_rlq_amd import rlq, workloads

    torch.cuda.set_device(0)
    log(f"generating workload {args.config}")
    prob = workloads.make_problem(args.config)
    B, H = prob.batch, prob.heads
    ctx = prob.ctx_lens.astype(np.int32)

    def dev(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    p = rlq.params(prob.tau, prob.gain, prob.level_inner, prob.level_outer)
    latent = dev(prob.latent_bits)
    rot = dev(prob.rotation_bits)
    k_rope = dev(prob.k_rope_bits)
    bt = dev(prob.block_table)
    ctx_d = dev(ctx)
    caches = []
    for r in range(args.replicas):
        log(f"prefill replica {r}: quantize-append {prob.n_tokens} tokens")
        c = rlq.PagedCache.allocate(prob.num_pages, max_batch=B, n_sink=prob.n_sink, n_recent=prob.n_recent)
        rlq.quantize_append(p, c, k_rope, dev(prob.cu_seqlens), dev(prob.start_pos), bt,
                            latent=latent, rotation=rot)
        caches.append(c)
    torch.cuda.synchronize()
    del latent

    # The step's new tokens: the last position of each request is re-appended
    # (so the context length stays fixed from step to step).
    new_idx = (prob.cu_seqlens[1:] - 1).astype(np.int64)
    new_lat = dev(prob.latent_bits[new_idx])
    new_kr = dev(prob.k_rope_bits[new_idx])
    new_cu = dev(np.arange(B + 1, dtype=np.int32))
    new_start = dev(ctx - 1)
    q_c, q_r = dev(prob.q_c_bits), dev(prob.q_r_bits)
    max_ctx = int(ctx.max())
    out = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = torch.zeros(rlq.decode_workspace_size(B, H, max_ctx), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    n_ev = args.steps
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]

    def step(i, timed):
        c = caches[i % len(caches)]
        rlq.quantize_append(p, c, new_kr, new_cu, new_start, bt, latent=new_lat, rotation=rot,
                            n_tokens=B, stream=stream)
        if timed:
            ev_a[i].record(stream)
        rlq.mla_decode(p, c, q_c, q_r, prob.sm_scale, bt, ctx_d, max_ctx, out=out, lse=lse,
                       workspace=ws, stream=stream)
        if timed:
            ev_b[i].record(stream)

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(i, True)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    dec_ms = np.array([a.elapsed_time(b) for a, b in zip(ev_a, ev_b)])
    dec_avg = float(dec_ms.mean())
    log(f"step {ms_step * 1e3:.1f} us, decode avg {dec_avg * 1e3:.1f} us "
        f"(p10 {np.percentile(dec_ms, 10) * 1e3:.1f}, p90 {np.percentile(dec_ms, 90) * 1e3:.1f})")

    toks = int(ctx.sum())
    alg_bytes = algorithmic_decode_bytes(B, H, ctx, prob.n_sink, prob.n_recent)
    achieved = alg_bytes / (dec_avg * 1e-3) / 1e9
    traffic = measured_traffic()
    res = {
        "metric": METRIC,
        "value": toks / (ms_step * 1e-3),
        "unit": "context tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: decode step, B={B} x {int(ctx[0])} context tokens, "
                               f"{H} heads, latent 512 + RoPE 64, 2-bit codes, group 128, page 64",
                   "batch": B, "ctx_per_request": int(ctx[0]), "heads": H,
                   "cache_replicas": args.replicas, "tau": prob.tau, "gain": prob.gain},
        "decode_us": dec_avg * 1e3,
        "decode_hbm_gbps": achieved,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": "rlq_mla_decode (split-KV kernel + merge kernel)",
                     "algorithmic_bytes_per_launch": alg_bytes},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(prob, new_idx)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
