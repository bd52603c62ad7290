"""Benchmark of the 2-bit MLA cache hot path on one MI355X.

Default workload (v2lite_256k): one decode step at the serving shape, i.e.
quantize-append of the new token of each request (rotate, standardize,
threshold, pack, RoPE copy) followed by absorbed-MLA decode attention over the
paged 2-bit cache (split-KV + merge); 4 requests x 262,144 context tokens, 16
heads, latent 512 + RoPE 64, group 128 (DeepSeek-V2-Lite MLA shapes at the
pages' 256K-input, 4-concurrent-request serving point).

Other workloads (each prints its own line with its own metric):
  --config v2lite_32k      the same step at 4 x 32,768 tokens (16 cache replicas)
  --config ragged_protect  32 requests of log-uniform 1K..64K tokens, 128 heads,
                           4 sink + 64 recent BF16 tokens per request (MFMA-bound)
  --config append_bulk     bulk quantize-append of 4 x 65,536 new tokens
  --config extend_32k      prefill / extend attention of a 512-token chunk per
                           request over 4 x 32,768 cached tokens (the chunk's own
                           positions included, causal), 16 heads (MFMA-bound)
  --config long_input      the long-input serving flow: 4 requests prefill
                           --input-tokens prompt tokens in --prefill-chunk chunks
                           (append + extend), then decode 128 tokens each;
                           reports decode tokens/s after prefill and prefill tokens/s
  --config long_output     the per-step decode loop of a long generation: 4
                           requests from 128-token prompts generate --gen-tokens
                           tokens each (append the new token, decode over the grown
                           cache, 4 sink + 64 recent BF16 tokens), 16 heads;
                           reports generated tokens/s over successive intervals

Prints one JSON line.  For the decode workloads `value` is context tokens per
second of the whole step with every input already resident in HBM; `roofline`
reports the decode call against MI355X's 8 TB/s HBM (or 2.5 PFLOP/s fp16 MFMA
for 128 heads); `cpu_baseline` times the CPU oracle on a bounded sample of the
same work.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]

Tools beside the benchmark (each prints one JSON line and exits):
  --ceilings               measured ceilings of this GPU: read-only HBM stream and
                           device copy, MFMA rates of the instruction shapes the
                           kernels use (one wave per SIMD, with the shader clock),
                           LDS read / write / transposed-read rates per CU
  --copy-calibration MIB   a plain device copy, the reference for the
                           FETCH_SIZE / WRITE_SIZE counter scale
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

DECODE_METRIC = "2-bit MLA decode context tokens/s and HBM GB/s (% peak) at B=4, 256K ctx"
APPEND_METRIC = "2-bit MLA quantize-append tokens/s, HBM GB/s and MFMA TFLOP/s (% peak), 4 x 65,536 new tokens"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0      # dense fp16 / bf16
BYTES_PER_TOKEN = 288          # 128 B codes + 32 B fp32 stats + 128 B bf16 RoPE key
BYTES_PER_PROTECTED = 1152     # 1024 B bf16 latent + 128 B RoPE key
APPEND_BYTES_PER_TOKEN = 1024 + 128 + 288   # latent + RoPE key read, cache record written
APPEND_FLOP_PER_TOKEN = 2 * 512 * 512       # z = R c
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic_v2lite_256k.json")
KERNEL_SOURCES = ["decode_attention_rlq_amd/csrc/rlq_decode.hip",
                  "decode_attention_rlq_amd/csrc/rlq_decode_common.h",
                  "decode_attention_rlq_amd/csrc/rlq_internal.h"]
DEFAULT_REPLICAS = {"v2lite_256k": 2, "v2lite_32k": 16, "ragged_protect": 3}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def protected_count(ctx_lens, n_sink, n_recent):
    return sum(min(int(c), n_sink + n_recent) for c in ctx_lens)


def algorithmic_decode_bytes(batch, heads, ctx_lens, n_sink=0, n_recent=0):
    prot = protected_count(ctx_lens, n_sink, n_recent)
    toks = int(sum(int(c) for c in ctx_lens))
    return ((toks - prot) * BYTES_PER_TOKEN + prot * BYTES_PER_PROTECTED
            + batch * heads * (512 + 64) * 2 + batch * heads * 512 * 4)


def decode_flops(heads, ctx_lens):
    # scores over 576 dims + value product over 512 dims, per head and token
    return 2.0 * heads * (576 + 512) * float(sum(int(c) for c in ctx_lens))


def measured_traffic(config):
    """Per-launch HBM bytes from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source and this workload."""
    if config != "v2lite_256k":
        return None
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    return t.get("traffic_bytes_per_launch")


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def copy_peak_gbps(torch, mib=1024, reps=5):
    """Device-to-device copy rate (bytes read + written per second): the
    practical HBM peak the decode is also compared against."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    del src, dst
    return 2.0 * n / min(ts) / 1e9


def per_call_us(torch, stream, fn, n):
    """fn(0) .. fn(n-1), each bracketed by its own pair of HIP events on
    `stream`; returns (median, p10, p90) of the per-call times in us."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        evs[i][0].record(stream)
        fn(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    return float(np.median(t)), float(np.percentile(t, 10)), float(np.percentile(t, 90))


# --------------------------------------------------------------------------- measured ceilings

def ceilings_lib():
    import ctypes
    path = os.path.join(ROOT, "decode_attention_rlq_amd", "librlq_ceilings.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build with `python -m decode_attention_rlq_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.rlq_ceiling_read.argtypes = [i32, vp, i64, vp, i32, vp]
    L.rlq_ceiling_mfma.argtypes = [i32, i32, i32, vp, vp, vp]
    L.rlq_ceiling_lds.argtypes = [i32, i32, i32, vp, vp]
    return L


def read_peak_gbps(torch, mib=1024, reps=5):
    """HBM read-only streaming rate with 16-byte loads (a HIP kernel reading
    `mib` MiB once per call; best of `reps` for each of a few grid sizes)."""
    L = ceilings_lib()
    n = mib << 20
    buf = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    best = 0.0
    for mode in (0, 1, 2):
        for blocks in (1024, 2048, 4096, 8192):
            for _ in range(reps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                assert L.rlq_ceiling_read(mode, buf.data_ptr(), n, sink.data_ptr(), blocks, stream.cuda_stream) == 0
                b.record(stream)
                torch.cuda.synchronize()
                best = max(best, n / (a.elapsed_time(b) * 1e-3) / 1e9)
    del buf
    return best


def measure_ceilings(torch):
    """Read stream, copy, MFMA rates with the shader clock, LDS rates."""
    L = ceilings_lib()
    stream = torch.cuda.current_stream()
    res = {"hbm_read_gbps": read_peak_gbps(torch), "hbm_copy_gbps": copy_peak_gbps(torch)}
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    blocks, iters = 1024, 2000                      # 4 workgroups of 4 waves per CU
    waves = blocks * 4
    clk = torch.zeros(2 * waves, dtype=torch.int64, device="cuda")
    names = {0: ("mfma_f32_16x16x32_f16", 2 * 16 * 16 * 32), 1: ("mfma_f32_16x16x32_bf16", 2 * 16 * 16 * 32),
             2: ("mfma_f32_16x16x32_bf8_fp8", 2 * 16 * 16 * 32), 3: ("mfma_f32_16x16x128_f8f6f4 (fp8)",
                                                                      2 * 16 * 16 * 128),
             4: ("mfma_f32_32x32x16_f16", 2 * 32 * 32 * 16),
             5: ("mfma_f32_32x32x16_f16 + 8 independent v_fma_f32 per MFMA", 2 * 32 * 32 * 16)}
    for kind, (name, flop) in names.items():
        L.rlq_ceiling_mfma(kind, blocks, 10, sink.data_ptr(), clk.data_ptr(), stream.cuda_stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        assert L.rlq_ceiling_mfma(kind, blocks, iters, sink.data_ptr(), clk.data_ptr(), stream.cuda_stream) == 0
        b.record(stream)
        torch.cuda.synchronize()
        t = a.elapsed_time(b) * 1e-3
        c = clk.view(-1, 2).cpu().numpy().astype(np.float64)
        ghz = float(np.median(c[:, 0] / c[:, 1]) * 0.1)   # shader cycles per 100 MHz tick
        # One workgroup of 4 waves per CU (256 workgroups): one wave per
        # SIMD, so a wave's own clock gives the SIMD's cycles per MFMA with
        # eight independent accumulators, and the rate follows from the clock.
        assert L.rlq_ceiling_mfma(kind, 256, iters, sink.data_ptr(), clk.data_ptr(), stream.cuda_stream) == 0
        torch.cuda.synchronize()
        c1 = clk.view(-1, 2)[:1024].cpu().numpy().astype(np.float64)
        cyc1 = float(np.median(c1[:, 0])) / (iters * 8)
        ghz1 = float(np.median(c1[:, 0] / c1[:, 1]) * 0.1)
        res[name] = {"tflops_event_timed": waves * iters * 8 * flop / t / 1e12,
                     "cycles_per_mfma_one_wave_per_simd": cyc1,
                     "tflops_at_that_rate": flop * 1024 * ghz1 * 1e9 / cyc1 / 1e12,
                     "shader_clock_ghz": ghz1}
    isink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for kind, (name, nbytes) in {0: ("lds_read_b128", 16), 1: ("lds_write_b128", 16),
                                 2: ("lds_read_b64_tr_b16", 8)}.items():
        L.rlq_ceiling_lds(kind, 256, 10, isink.data_ptr(), stream.cuda_stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        assert L.rlq_ceiling_lds(kind, 256, 1000, isink.data_ptr(), stream.cuda_stream) == 0
        b.record(stream)
        torch.cuda.synchronize()
        t = a.elapsed_time(b) * 1e-3
        res[name + "_gbps_per_cu"] = 1024 * 16 * 1000 * nbytes / t / 1e9
    return res


def timed_loop(torch, stream, fn, n, chunks=1):
    """fn(0) .. fn(n-1) on `stream` with HIP events only at chunk boundaries
    (an event record idles the GPU for a few microseconds, so none goes
    between calls).  Returns (mean ms per call, per-chunk means in ms)."""
    k = max(1, min(chunks, n))
    bounds = [round(j * n / k) for j in range(k + 1)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(k + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for j in range(k):
        for i in range(bounds[j], bounds[j + 1]):
            fn(i)
        evs[j + 1].record(stream)
    torch.cuda.synchronize()
    per_chunk = [evs[j].elapsed_time(evs[j + 1]) / (bounds[j + 1] - bounds[j]) for j in range(k)]
    return evs[0].elapsed_time(evs[k]) / n, per_chunk


def spread(chunk_ms):
    return {"chunks": len(chunk_ms), "chunk_mean_min_us": min(chunk_ms) * 1e3,
            "chunk_mean_max_us": max(chunk_ms) * 1e3}


def dev_of(torch):
    def dev(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()
    return dev


# --------------------------------------------------------------------------- CPU oracle baselines

def cpu_baseline_decode(prob, new_idx, sample_requests):
    """The oracle on the same decode step (append of the new tokens + decode
    over the full contexts) for `sample_requests` of the batch."""
    import oracle
    reqs = list(range(min(sample_requests, prob.batch)))
    log(f"cpu baseline: oracle setup (quantize the cache of {len(reqs)} request(s))")
    oc = oracle.new_cache(prob.num_pages, max_batch=prob.batch, n_sink=prob.n_sink, n_recent=prob.n_recent)
    cu = prob.cu_seqlens
    sel = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in reqs])
    sub_cu = np.zeros(len(reqs) + 1, np.int32)
    sub_cu[1:] = np.cumsum([cu[b + 1] - cu[b] for b in reqs])
    bt = prob.block_table[reqs]
    oracle.quantize_append(oc, prob.tau, prob.k_rope_bits[sel], sub_cu, np.zeros(len(reqs), np.int32), bt,
                           latent_bf16=prob.latent_bits[sel], rotation_bf16=prob.rotation_bits)
    ctx = prob.ctx_lens[reqs]
    log("cpu baseline: timed oracle steps (about 10 s)")
    t0 = time.perf_counter()
    steps = 0
    while steps < 8 and (steps == 0 or time.perf_counter() - t0 < 10.0):
        # Re-appending the last position leaves the cache as it was.
        oracle.quantize_append(oc, prob.tau, prob.k_rope_bits[new_idx[reqs]], np.arange(len(reqs) + 1),
                               ctx - 1, bt, latent_bf16=prob.latent_bits[new_idx[reqs]],
                               rotation_bf16=prob.rotation_bits)
        oracle.decode(oc, prob.q_c_bits[reqs], prob.q_r_bits[reqs], prob.sm_scale, bt, ctx,
                      prob.gain, prob.level_inner, prob.level_outer)
        steps += 1
    dt = time.perf_counter() - t0
    toks = int(ctx.sum())
    return {"value": toks * steps / dt, "unit": "context tokens/s", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"{steps} step(s) (append + fp64 decode) for {len(reqs)} of {prob.batch} requests, "
                      f"{toks} context tokens, {prob.heads} heads: {dt:.2f} s"}


def cpu_baseline_append(prob, n_sample):
    import oracle
    n = min(n_sample, int(prob.cu_seqlens[-1]))
    oc = oracle.new_cache(prob.num_pages)
    cu = np.array([0, n], np.int32)
    log(f"cpu baseline: timed oracle quantize-append of {n} tokens")
    t0 = time.perf_counter()
    oracle.quantize_append(oc, prob.tau, prob.k_rope_bits[:n], cu, np.zeros(1, np.int32), prob.block_table[:1],
                           latent_bf16=prob.latent_bits[:n], rotation_bf16=prob.rotation_bits)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"quantize-append of the first {n} new tokens (fp64 rotation): {dt:.2f} s"}


# --------------------------------------------------------------------------- decode step

def bench_decode(args, torch, rlq, workloads):
    dev = dev_of(torch)
    log(f"generating workload {args.config}")
    prob = workloads.make_problem(args.config)
    B, H = prob.batch, prob.heads
    ctx = prob.ctx_lens.astype(np.int32)
    prot = prob.n_sink > 0 or prob.n_recent > 0
    p = rlq.params(prob.tau, prob.gain, prob.level_inner, prob.level_outer)
    latent, rot, k_rope = dev(prob.latent_bits), dev(prob.rotation_bits), dev(prob.k_rope_bits)
    bt, ctx_d = dev(prob.block_table), dev(ctx)
    replicas = args.replicas or DEFAULT_REPLICAS.get(args.config, 2)
    caches = []
    for r in range(replicas):
        log(f"prefill replica {r}: quantize-append {prob.n_tokens} tokens")
        c = rlq.PagedCache.allocate(prob.num_pages, max_batch=B, n_sink=prob.n_sink, n_recent=prob.n_recent)
        rlq.quantize_append(p, c, k_rope, dev(prob.cu_seqlens), dev(prob.start_pos), bt, latent=latent, rotation=rot)
        caches.append(c)
    torch.cuda.synchronize()
    del latent

    # The step's new tokens: the last position of each request is re-appended
    # (so the context length stays fixed from step to step).
    new_idx = (prob.cu_seqlens[1:] - 1).astype(np.int64)
    new_lat, new_kr = dev(prob.latent_bits[new_idx]), dev(prob.k_rope_bits[new_idx])
    new_cu, new_start = dev(np.arange(B + 1, dtype=np.int32)), dev(ctx - 1)
    q_c, q_r = dev(prob.q_c_bits), dev(prob.q_r_bits)
    max_ctx = int(ctx.max())
    out = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = torch.zeros(rlq.decode_workspace_size(B, H, max_ctx), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def append(i):
        rlq.quantize_append(p, caches[i % len(caches)], new_kr, new_cu, new_start, bt, latent=new_lat,
                            rotation=rot, n_tokens=B, stream=stream)

    def decode(i):
        rlq.mla_decode(p, caches[i % len(caches)], q_c, q_r, prob.sm_scale, bt, ctx_d, max_ctx, out=out, lse=lse,
                       workspace=ws, stream=stream)

    def step(i):
        append(i)
        decode(i)

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    ms_step, _ = timed_loop(torch, stream, step, args.steps)
    # The decode call alone over the same caches, for the roofline: the mean
    # over args.steps back-to-back calls, events only every fifth of them.
    log(f"timing {args.steps} decode calls")
    dec_avg, dec_chunks = timed_loop(torch, stream, decode, args.steps, chunks=5)
    # Distribution: every call bracketed by its own events (at least 50 calls).
    n_dist = max(50, args.steps)
    dec_med, dec_p10, dec_p90 = per_call_us(torch, stream, decode, n_dist)
    # The step loop once more after the decode loops: the two step figures
    # bracket any drift of the clock over the run.
    ms_step2, _ = timed_loop(torch, stream, step, args.steps)
    log(f"step {ms_step * 1e3:.1f} us (again after the decode loops: {ms_step2 * 1e3:.1f} us), decode call "
        f"{dec_avg * 1e3:.1f} us (chunk means {min(dec_chunks) * 1e3:.1f} .. {max(dec_chunks) * 1e3:.1f}; "
        f"per call median {dec_med:.1f}, p10 {dec_p10:.1f}, p90 {dec_p90:.1f})")
    copy_gbps = copy_peak_gbps(torch)
    read_gbps = read_peak_gbps(torch)
    log(f"device copy rate {copy_gbps:.0f} GB/s, read-only stream {read_gbps:.0f} GB/s")

    toks = int(ctx.sum())
    alg_bytes = algorithmic_decode_bytes(B, H, ctx, prob.n_sink if prot else 0, prob.n_recent if prot else 0)
    gbps = alg_bytes / (dec_avg * 1e-3) / 1e9
    tflops = decode_flops(H, ctx) / (dec_avg * 1e-3) / 1e12
    hbm = {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
           "frac": gbps / HBM_PEAK_GBPS, "traffic": measured_traffic(args.config),
           "kernel": "rlq_mla_decode (many-head kernel + merge kernel)" if H % 64 == 0 else
                     "rlq_mla_decode (split-KV kernel + merge kernel)",
           "algorithmic_bytes_per_launch": alg_bytes, "copy_peak_gbps": copy_gbps,
           "frac_of_copy_peak": gbps / copy_gbps, "read_peak_gbps": read_gbps,
           "frac_of_read_peak": gbps / read_gbps}
    mfma = {"bound": "mfma", "achieved": tflops, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": tflops / MFMA_PEAK_TFLOPS, "traffic": None,
            "kernel": "rlq_mla_decode (many-head kernel + merge kernel)" if H % 64 == 0 else
                      "rlq_mla_decode (split-KV kernel + merge kernel)",
            "algorithmic_flop_per_launch": decode_flops(H, ctx)}
    # 16 heads: 121 flop per byte, HBM-bound; 128 heads: 967 flop per byte, MFMA-bound.
    roofline, other = (mfma, hbm) if H >= 64 else (hbm, mfma)
    roofline = dict(roofline)
    roofline["other_bound"] = {k: other[k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    workload = (f"{args.config}: decode step, B={B}, {toks} context tokens "
                f"({'ragged ' if len(set(ctx.tolist())) > 1 else ''}{int(ctx.min())}..{int(ctx.max())} per request), "
                f"{H} heads, latent 512 + RoPE 64, 2-bit codes, group 128, page 64"
                + (f", {prob.n_sink} sink + {prob.n_recent} recent BF16 tokens" if prot else ""))
    res = {
        "metric": DECODE_METRIC if args.config == "v2lite_256k" else
        f"2-bit MLA decode context tokens/s ({args.config})",
        "value": toks / (ms_step * 1e-3),
        "unit": "context tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": workload, "batch": B, "context_tokens": toks, "heads": H,
                   "cache_replicas": replicas, "tau": prob.tau, "gain": prob.gain},
        "decode_us": dec_avg * 1e3, "decode_spread": spread(dec_chunks),
        "decode_call_us": {"median": dec_med, "p10": dec_p10, "p90": dec_p90, "calls": n_dist},
        "step_us_repeat": ms_step2 * 1e3,
        "decode_hbm_gbps": gbps,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decode(prob, new_idx, args.cpu_sample_requests or
                                                  (prob.batch if H <= 16 else 2))
    return res


# --------------------------------------------------------------------------- bulk append

def bench_append(args, torch, rlq, workloads):
    dev = dev_of(torch)
    log(f"generating workload {args.config}")
    prob = workloads.make_problem(args.config)
    n = int(prob.cu_seqlens[-1])
    p = rlq.params(prob.tau, prob.gain, prob.level_inner, prob.level_outer)
    c = rlq.PagedCache.allocate(prob.num_pages, max_batch=prob.batch)
    lat, rot, kr = dev(prob.latent_bits), dev(prob.rotation_bits), dev(prob.k_rope_bits)
    cu, sp, bt = dev(prob.cu_seqlens), dev(prob.start_pos), dev(prob.block_table)
    stream = torch.cuda.current_stream()

    def call():
        rlq.quantize_append(p, c, kr, cu, sp, bt, latent=lat, rotation=rot, n_tokens=n, stream=stream)

    log(f"warmup {args.warmup} calls")
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    log(f"timing {args.steps} calls")
    ms, chunks = timed_loop(torch, stream, lambda i: call(), args.steps, chunks=5)
    t = ms * 1e-3
    log(f"append avg {t * 1e6:.1f} us (chunk means {min(chunks) * 1e3:.1f} .. {max(chunks) * 1e3:.1f})")
    copy_gbps = copy_peak_gbps(torch)
    tflops = n * APPEND_FLOP_PER_TOKEN / t / 1e12
    gbps = n * APPEND_BYTES_PER_TOKEN / t / 1e9
    roofline = {"bound": "mfma", "achieved": tflops, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": tflops / MFMA_PEAK_TFLOPS, "traffic": None,
                "kernel": "rlq_quantize_append (bulk kernel)",
                "algorithmic_flop_per_launch": n * APPEND_FLOP_PER_TOKEN,
                "other_bound": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                "frac": gbps / HBM_PEAK_GBPS},
                "algorithmic_bytes_per_launch": n * APPEND_BYTES_PER_TOKEN, "copy_peak_gbps": copy_gbps}
    res = {
        "metric": APPEND_METRIC, "value": n / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.config}: quantize-append of {prob.batch} x {n // prob.batch} new tokens "
                               f"(bf16 latent 512 + RoPE 64, Haar rotation, 1% Student-t coordinates)",
                   "batch": prob.batch, "new_tokens": n, "tau": prob.tau},
        "append_us": t * 1e6, "append_spread": spread(chunks),
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_append(prob, args.cpu_sample_tokens)
    return res


# --------------------------------------------------------------------------- long output

LONG_OUTPUT_METRIC = "2-bit MLA long-output decode loop: generated tokens/s (4 requests, 128-token prompts)"


def bench_long_output(args, torch, rlq, workloads):
    """Successive-interval throughput of the generation loop.  One step =
    quantize-append of the new token of every request (bf16 latent, MFMA
    rotation) + decode over the cache grown by it; `unroll` steps are captured
    in one HIP graph that also advances the device-side positions, and the
    graph is replayed until every request has generated --gen-tokens tokens."""
    dev = dev_of(torch)
    B, H, prompt, gen = 4, 16, 128, args.gen_tokens
    unroll, interval = 32, max(args.interval // 32 * 32, 32)
    gen = (gen + interval - 1) // interval * interval
    log(f"generating workload long_output: {B} x {prompt}-token prompts, {gen} generated tokens each")
    prob = workloads.make_problem("v2lite_32k", ctx_lens=[prompt] * B, heads=H, n_sink=4, n_recent=64)
    # The cache and the decode grid are sized for --gen-capacity tokens (the
    # whole generation by default), as a server sizes them before it starts.
    total = prompt + max(gen, args.gen_capacity)
    ppr = (total + 63) // 64
    perm = np.random.default_rng(7).permutation(B * ppr).astype(np.int32)
    bt_np = perm.reshape(B, ppr)
    p = rlq.params(prob.tau, prob.gain, prob.level_inner, prob.level_outer)
    cache = rlq.PagedCache.allocate(B * ppr, max_batch=B, n_sink=prob.n_sink, n_recent=prob.n_recent)
    bt, rot = dev(bt_np), dev(prob.rotation_bits)
    rlq.quantize_append(p, cache, dev(prob.k_rope_bits), dev(prob.cu_seqlens), dev(prob.start_pos), bt,
                        latent=dev(prob.latent_bits), rotation=rot)
    # Step k of a replay appends the latents of prompt position k of every
    # request again (values do not change the work); one int32 [2][B] tensor
    # holds the append positions (row 0) and the context lengths (row 1).
    rows = np.asarray([[int(prob.cu_seqlens[b]) + t for b in range(B)] for t in range(unroll)]).reshape(-1)
    lat_pool = dev(prob.latent_bits[rows]).view(unroll, B, 512)
    kr_pool = dev(prob.k_rope_bits[rows]).view(unroll, B, 64)
    q_c, q_r = dev(prob.q_c_bits), dev(prob.q_r_bits)
    cu_d = dev(np.arange(B + 1, dtype=np.int32))
    pos_d = torch.tensor([[prompt] * B, [prompt + 1] * B], dtype=torch.int32, device="cuda")
    out = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = torch.zeros(rlq.decode_workspace_size(B, H, total), dtype=torch.uint8, device="cuda")

    def step(st, k):
        rlq.quantize_append(p, cache, kr_pool[k], cu_d, pos_d[0], bt, latent=lat_pool[k], rotation=rot,
                            n_tokens=B, stream=st)
        rlq.mla_decode(p, cache, q_c, q_r, prob.sm_scale, bt, pos_d[1], total, out=out, lse=lse, workspace=ws,
                       stream=st)
        pos_d.add_(1)

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for k in range(unroll):
            step(cap, k)
    torch.cuda.synchronize()

    def reset():
        pos_d[0].fill_(prompt)
        pos_d[1].fill_(prompt + 1)

    log(f"warmup {args.warmup} replays of {unroll} steps")
    reset()
    for _ in range(max(args.warmup, 1)):
        g.replay()
    torch.cuda.synchronize()
    reset()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(gen // interval + 1)]
    log(f"timing {gen} steps ({gen // unroll} replays), events every {interval} steps")
    ev[0].record(stream)
    for k in range(gen // interval):
        for _ in range(interval // unroll):
            g.replay()
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    assert int(pos_d[0, 0].item()) == prompt + gen
    dts = [ev[k].elapsed_time(ev[k + 1]) * 1e-3 for k in range(gen // interval)]
    t_all = sum(dts)
    intervals = [{"context_end": prompt + (k + 1) * interval, "generated_tokens_per_s": B * interval / dt,
                  "ms_per_step": dt * 1e3 / interval} for k, dt in enumerate(dts)]
    ctx_sum = B * sum(prompt + t + 1 for t in range(gen))          # context tokens attended over the run
    prot = B * sum(min(prompt + t + 1, 68) for t in range(gen))    # of which BF16 sink/recent
    alg_bytes = (ctx_sum - prot) * BYTES_PER_TOKEN + prot * BYTES_PER_PROTECTED
    gbps = alg_bytes / t_all / 1e9
    log(f"{gen} steps in {t_all * 1e3:.1f} ms: {B * gen / t_all:.3g} generated tokens/s; first interval "
        f"{intervals[0]['ms_per_step'] * 1e3:.1f} us/step, last {intervals[-1]['ms_per_step'] * 1e3:.1f} us/step")
    return {
        "metric": LONG_OUTPUT_METRIC, "value": B * gen / t_all, "unit": "generated tokens/s", "n_gpus": 1,
        "steps": gen, "warmup": args.warmup, "ms_per_step": t_all * 1e3 / gen, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp16", "data": "synthetic",
        "config": {"workload": f"long_output: {B} requests, {prompt}-token prompts, {gen} generated tokens each, "
                               f"{H} heads, 4 sink + 64 recent BF16 tokens; one step = append 1 token per request "
                               f"+ decode (the grid sized for the final length), {unroll} steps per HIP graph",
                   "batch": B, "heads": H, "prompt_tokens": prompt, "generated_tokens": gen},
        "intervals": intervals,
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "whole step (append + decode), cache bytes attended per second",
                     "algorithmic_bytes_per_run": alg_bytes},
    }


# --------------------------------------------------------------------------- long input (prefill + decode)

def bench_long_input(args, torch, rlq, workloads):
    """The long-input serving flow: 4 requests each prefill --input-tokens
    prompt tokens in --prefill-chunk chunks (bulk quantize-append of the chunk,
    then extend attention of its queries over the cache built so far), then
    generate 128 tokens (append + decode per step).  Reports decode
    throughput after prefill, and the prefill rate."""
    dev = dev_of(torch)
    B, H, n_in, n_out = 4, 16, args.input_tokens, 128
    chunk = min(args.prefill_chunk, n_in)
    log(f"generating workload long_input: {B} x {n_in}-token prompts, chunks of {chunk}, {n_out} output tokens")
    prob = workloads.make_problem("v2lite_32k", ctx_lens=[n_in] * B, heads=H)
    total = n_in + n_out
    ppr = (total + 63) // 64
    bt_np = np.random.default_rng(11).permutation(B * ppr).astype(np.int32).reshape(B, ppr)
    p = rlq.params(prob.tau, prob.gain, prob.level_inner, prob.level_outer)
    cache = rlq.PagedCache.allocate(B * ppr, max_batch=B)
    bt, rot = dev(bt_np), dev(prob.rotation_bits)
    lat, kr = dev(prob.latent_bits), dev(prob.k_rope_bits)
    rng = np.random.default_rng(3)
    qc = dev(workloads.to_bf16_bits(rng.standard_normal((B * chunk, H, 512), dtype=np.float32)))
    qr = dev(workloads.to_bf16_bits(rng.standard_normal((B * chunk, H, 64), dtype=np.float32)))
    e_out = torch.empty((B * chunk, H, 512), dtype=torch.float32, device="cuda")
    e_lse = torch.empty((B * chunk, H), dtype=torch.float32, device="cuda")
    e_ws = torch.zeros(rlq.extend_workspace_size(B, H, chunk, total), dtype=torch.uint8, device="cuda")
    chunks = []
    for c0 in range(0, n_in, chunk):
        n = min(chunk, n_in - c0)
        # Token rows of the chunk in the workload's latent array (request-major).
        rows = np.concatenate([np.arange(b * n_in + c0, b * n_in + c0 + n) for b in range(B)])
        cu = np.arange(0, B * n + 1, n, dtype=np.int32)
        chunks.append((n, dev(prob.latent_bits[rows]), dev(prob.k_rope_bits[rows]), dev(cu),
                       dev(np.full(B, c0, np.int32)), dev(np.full(B, c0 + n, np.int32)), c0 + n))
    del lat, kr
    stream = torch.cuda.current_stream()

    def prefill():
        for n, cl, ck, cu, start, ctx, c_end in chunks:
            rlq.quantize_append(p, cache, ck, cu, start, bt, latent=cl, rotation=rot, n_tokens=B * n, stream=stream)
            rlq.mla_extend(p, cache, qc[:B * n], qr[:B * n], cu, n, prob.sm_scale, bt, ctx, c_end,
                           out=e_out[:B * n], lse=e_lse[:B * n], workspace=e_ws, stream=stream)

    new_lat = dev(prob.latent_bits[np.arange(B) * n_in])
    new_kr = dev(prob.k_rope_bits[np.arange(B) * n_in])
    cu1 = dev(np.arange(B + 1, dtype=np.int32))
    q_c, q_r = dev(prob.q_c_bits), dev(prob.q_r_bits)
    out = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    d_ws = torch.zeros(rlq.decode_workspace_size(B, H, total), dtype=torch.uint8, device="cuda")
    starts = [dev(np.full(B, n_in + k, np.int32)) for k in range(n_out)]
    ctxs = [dev(np.full(B, n_in + k + 1, np.int32)) for k in range(n_out)]

    def decode_step(k):
        rlq.quantize_append(p, cache, new_kr, cu1, starts[k], bt, latent=new_lat, rotation=rot, n_tokens=B,
                            stream=stream)
        rlq.mla_decode(p, cache, q_c, q_r, prob.sm_scale, bt, ctxs[k], total, out=out, lse=lse, workspace=d_ws,
                       stream=stream)

    log("warmup: one prefill and the decode steps")
    prefill()
    for k in range(n_out):
        decode_step(k)
    torch.cuda.synchronize()
    log(f"timing the prefill ({len(chunks)} chunks)")
    ms_pre, _ = timed_loop(torch, stream, lambda i: prefill(), 1)
    log(f"timing {n_out} decode steps")
    ms_dec, _ = timed_loop(torch, stream, decode_step, n_out)
    log(f"prefill {ms_pre:.1f} ms ({B * n_in / (ms_pre * 1e-3):.3g} tokens/s), decode step {ms_dec * 1e3:.1f} us")
    ctx_end = n_in + n_out
    alg = algorithmic_decode_bytes(B, H, [ctx_end - n_out // 2] * B)
    gbps = alg / (ms_dec * 1e-3) / 1e9
    return {
        "metric": "2-bit MLA long-input serving flow: decode tokens/s after a chunked prefill "
                  "(also prefill tokens/s)",
        "value": B / (ms_dec * 1e-3), "unit": "generated tokens/s",
        "n_gpus": 1, "steps": n_out, "warmup": 1, "ms_per_step": ms_dec, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp16", "data": "synthetic",
        "config": {"workload": f"long_input: {B} requests x {n_in}-token prompts prefilled in chunks of {chunk} "
                               f"(bulk append + extend attention), then {n_out} output tokens each (append + "
                               f"decode), {H} heads, latent 512 + RoPE 64, 2-bit codes",
                   "batch": B, "input_tokens": n_in, "prefill_chunk": chunk, "output_tokens": n_out, "heads": H},
        "prefill_ms": ms_pre, "prefill_tokens_per_s": B * n_in / (ms_pre * 1e-3),
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "decode step (few-token append + rlq_mla_decode) after the prefill",
                     "algorithmic_bytes_per_launch": alg},
    }


# --------------------------------------------------------------------------- extend (prefill chunk)

def extend_flops(heads, ctx, n_q):
    """2 (576 + 512) flop per (query, visible position, head): query i of a
    request with ctx positions and n_q queries sees ctx - n_q + i + 1."""
    vis = sum(int(c) * n - n * (n - 1) // 2 for c, n in zip(ctx, n_q))
    return 2.0 * (RLQ_DC_R + 512) * heads * vis


RLQ_DC_R = 576  # score contraction: 512 latent + 64 RoPE


def cpu_baseline_extend(prob, oc_builder, qc, qr, cuq, n_sample):
    """The oracle's extend for the first n_sample queries of request 0."""
    import oracle
    log("cpu baseline: oracle setup (quantize request 0's cache)")
    oc, ctx0 = oc_builder()
    n = min(n_sample, int(cuq[1]))
    nq0 = int(cuq[1])
    # Queries 0 .. n-1 of request 0 (positions ctx0 - nq0 .. ctx0 - nq0 + n - 1).
    log(f"cpu baseline: timed oracle extend of {n} queries")
    t0 = time.perf_counter()
    sub_ctx = ctx0 - nq0 + n  # the same positions as the first n queries of the chunk
    oracle.extend(oc, qc[:n], qr[:n], prob.sm_scale, prob.block_table[:1], [sub_ctx], [0, n],
                  prob.gain, prob.level_inner, prob.level_outer)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "query tokens/s", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"fp64 extend of the first {n} of {nq0} chunk queries of one request "
                      f"({ctx0} cached tokens, {prob.heads} heads): {dt:.2f} s"}


def bench_extend(args, torch, rlq, workloads):
    dev = dev_of(torch)
    log("generating workload extend_32k (cache of v2lite_32k)")
    prob = workloads.make_problem("v2lite_32k")
    B, H = prob.batch, prob.heads
    ctx = prob.ctx_lens.astype(np.int32)
    chunk = min(args.chunk, int(ctx.min()))
    n_q = [chunk] * B
    p = rlq.params(prob.tau, prob.gain, prob.level_inner, prob.level_outer)
    c = rlq.PagedCache.allocate(prob.num_pages, max_batch=B)
    bt, ctx_d = dev(prob.block_table), dev(ctx)
    log(f"prefill: quantize-append {prob.n_tokens} tokens")
    rlq.quantize_append(p, c, dev(prob.k_rope_bits), dev(prob.cu_seqlens), dev(prob.start_pos), bt,
                        latent=dev(prob.latent_bits), rotation=dev(prob.rotation_bits))
    rng = np.random.default_rng(7)
    total = chunk * B
    qc = workloads.to_bf16_bits(rng.standard_normal((total, H, 512), dtype=np.float32))
    qr = workloads.to_bf16_bits(rng.standard_normal((total, H, 64), dtype=np.float32))
    cuq = np.arange(0, total + 1, chunk, dtype=np.int32)
    q_c, q_r, cuq_d = dev(qc), dev(qr), dev(cuq)
    max_ctx = int(ctx.max())
    out = torch.empty((total, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((total, H), dtype=torch.float32, device="cuda")
    ws = torch.zeros(rlq.extend_workspace_size(B, H, chunk, max_ctx), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def call(i):
        rlq.mla_extend(p, c, q_c, q_r, cuq_d, chunk, prob.sm_scale, bt, ctx_d, max_ctx, out=out, lse=lse,
                       workspace=ws, stream=stream)

    log(f"warmup {args.warmup} calls")
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    steps = max(1, args.steps // 5)
    log(f"timing {steps} calls")
    ms, chunks = timed_loop(torch, stream, call, steps, chunks=min(5, steps))
    log(f"extend call {ms * 1e3:.1f} us (chunk means {min(chunks) * 1e3:.1f} .. {max(chunks) * 1e3:.1f})")
    flops = extend_flops(H, ctx, n_q)
    tflops = flops / (ms * 1e-3) / 1e12
    # Cache once, queries in, outputs and LSE out.
    cache_bytes = int(ctx.sum()) * BYTES_PER_TOKEN + total * H * ((512 + 64) * 2 + 512 * 4 + 4)
    gbps = cache_bytes / (ms * 1e-3) / 1e9
    workload = (f"extend_32k: prefill chunk of {chunk} new tokens per request attending causally to "
                f"{B} x {max_ctx} cached tokens (chunk included), {H} heads, latent 512 + RoPE 64, "
                f"2-bit codes, group 128, page 64")
    res = {
        "metric": "2-bit MLA extend (prefill chunk) query tokens/s and MFMA TFLOP/s (% peak)",
        "value": total / (ms * 1e-3), "unit": "query tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp16", "data": "synthetic",
        "config": {"workload": workload, "batch": B, "chunk": chunk, "context_tokens": int(ctx.sum()), "heads": H},
        "extend_us": ms * 1e3, "extend_spread": spread(chunks),
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_PEAK_TFLOPS, "traffic": None,
                     "kernel": "rlq_mla_extend (many-head kernel over (query, head) rows + merge kernel)",
                     "algorithmic_flop_per_launch": flops,
                     "other_bound": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                     "frac": gbps / HBM_PEAK_GBPS}},
    }
    if not args.no_cpu_baseline:
        def build_request0():
            import oracle
            oc = oracle.new_cache(prob.num_pages)
            n0 = int(prob.cu_seqlens[1])
            oracle.quantize_append(oc, prob.tau, prob.k_rope_bits[:n0], np.array([0, n0], np.int32),
                                   np.zeros(1, np.int32), prob.block_table[:1],
                                   latent_bf16=prob.latent_bits[:n0], rotation_bf16=prob.rotation_bits)
            return oc, n0
        res["cpu_baseline"] = cpu_baseline_extend(prob, build_request0, qc, qr, cuq, chunk)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="v2lite_256k",
                    choices=["v2lite_256k", "v2lite_32k", "ragged_protect", "append_bulk", "long_output",
                             "extend_32k", "long_input"])
    ap.add_argument("--input-tokens", type=int, default=32768, help="long_input: prompt tokens per request")
    ap.add_argument("--prefill-chunk", type=int, default=4096, help="long_input: prefill chunk (tokens)")
    ap.add_argument("--chunk", type=int, default=512, help="extend_32k: new (query) tokens per request")
    ap.add_argument("--gen-tokens", type=int, default=262144,
                    help="long_output: tokens generated per request")
    ap.add_argument("--gen-capacity", type=int, default=0,
                    help="long_output: size the cache and decode grid for this many generated tokens")
    ap.add_argument("--interval", type=int, default=8192,
                    help="long_output: steps per reported interval (a multiple of 32)")
    ap.add_argument("--replicas", type=int, default=0,
                    help="cache copies cycled per step so no step reads a cache the MALL still holds")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-requests", type=int, default=0)
    ap.add_argument("--cpu-sample-tokens", type=int, default=16384)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (counter calibration)")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure the GPU's ceilings (HBM read / copy, MFMA, LDS, shader clock)")
    args = ap.parse_args()
    if args.ceilings:
        import torch
        torch.cuda.set_device(0)
        print(json.dumps(measure_ceilings(torch)), flush=True)
        return
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
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): sharding this path "
              "across GPUs is designed but not built.", file=sys.stderr)
        sys.exit(2)

    import torch
    from decode_attention_rlq_amd import rlq, workloads

    torch.cuda.set_device(0)
    if args.config == "append_bulk":
        res = bench_append(args, torch, rlq, workloads)
    elif args.config == "long_output":
        res = bench_long_output(args, torch, rlq, workloads)
    elif args.config == "extend_32k":
        res = bench_extend(args, torch, rlq, workloads)
    elif args.config == "long_input":
        res = bench_long_input(args, torch, rlq, workloads)
    else:
        res = bench_decode(args, torch, rlq, workloads)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
