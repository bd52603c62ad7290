"""Chunked prefill followed by decode steps, the serving flow of the pages'
long-input tests ([RoLaQ] §D: prefill, then decode over the cache):

* each prompt is appended in chunks (rlq_quantize_append) and every chunk's
  queries attend causally to the cache built so far (rlq_mla_extend);
* then a few decode steps append one token per request and decode.

Sink and recent BF16 rows are on, so the recent ring is rewritten by every
chunk.  The oracle runs the same sequence on its own cache from the same
pre-rotated latents: pools stay bit-exact and every extend / decode output is
within tolerance.
"""

import numpy as np
import pytest
import torch

import oracle
from decode_attention_rlq_amd import rlq, workloads
from gpu_helpers import check_decode, dev, host_bits, params_of

pytestmark = pytest.mark.gpu

PROMPTS = [300, 1000, 77]
CHUNK = 256
DECODE_STEPS = 4


def compare_pools(dc, oc):
    assert np.array_equal(host_bits(dc.codes), oc.codes), "codes differ"
    assert np.array_equal(host_bits(dc.meta).view(np.uint32), oc.meta.view(np.uint32)), "meta differ"
    assert np.array_equal(host_bits(dc.rope), oc.rope), "rope differ"
    assert np.array_equal(host_bits(dc.sink), oc.sink), "sink differ"
    assert np.array_equal(host_bits(dc.recent), oc.recent), "recent ring differs"


@pytest.mark.parametrize("heads", [16, 128])
def test_chunked_prefill_then_decode(heads):
    print(f"prefill flow: heads {heads}, prompts {PROMPTS}, chunk {CHUNK}", flush=True)
    prob = workloads.make_problem("ragged_protect", ctx_lens=[n + DECODE_STEPS for n in PROMPTS], heads=heads,
                                  n_sink=4, n_recent=16)
    B = prob.batch
    z = (prob.latent_bits.astype(np.uint32) << 16).view(np.float32)  # latents taken as already rotated
    base = [int(prob.cu_seqlens[b]) for b in range(B)]
    p = params_of(prob)
    bt_np = prob.block_table
    bt = dev(bt_np)
    oc = oracle.new_cache(prob.num_pages, max_batch=B, n_sink=prob.n_sink, n_recent=prob.n_recent)
    dc = rlq.PagedCache.allocate(prob.num_pages, max_batch=B, n_sink=prob.n_sink, n_recent=prob.n_recent)
    rng = np.random.default_rng(77 + heads)
    done = [0] * B
    worst = [0.0, 0.0]
    while any(done[b] < PROMPTS[b] for b in range(B)):
        n_new = [min(CHUNK, PROMPTS[b] - done[b]) for b in range(B)]
        rows = np.concatenate([np.arange(base[b] + done[b], base[b] + done[b] + n_new[b]) for b in range(B)])
        cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
        start = np.asarray(done, np.int32)
        oracle.quantize_append(oc, prob.tau, prob.k_rope_bits[rows], cu, start, bt_np, latent_rot_f32=z[rows])
        rlq.quantize_append(p, dc, dev(prob.k_rope_bits[rows]), dev(cu), dev(start), bt, latent_rot=dev(z[rows]))
        ctx = np.asarray([done[b] + n_new[b] for b in range(B)], np.int32)
        total = int(cu[-1])
        qc = workloads.to_bf16_bits(rng.standard_normal((total, heads, 512), dtype=np.float32))
        qr = workloads.to_bf16_bits(rng.standard_normal((total, heads, 64), dtype=np.float32))
        ref_o, ref_l = oracle.extend(oc, qc, qr, prob.sm_scale, bt_np, ctx, cu, prob.gain, prob.level_inner,
                                     prob.level_outer)
        out, lse = rlq.mla_extend(p, dc, dev(qc), dev(qr), dev(cu), max(n_new), prob.sm_scale, bt, dev(ctx),
                                  int(ctx.max()))
        torch.cuda.synchronize()
        rows_ctx = np.ones(total, np.int64)
        e = check_decode(out, lse, ref_o, ref_l, rows_ctx)
        worst = [max(worst[0], e[0]), max(worst[1], e[1])]
        compare_pools(dc, oc)
        done = [done[b] + n_new[b] for b in range(B)]
    print(f"prefill: worst extend out err {worst[0]:.2e}, lse err {worst[1]:.2e}")

    cur = list(PROMPTS)
    q_c, q_r = dev(prob.q_c_bits), dev(prob.q_r_bits)
    for step in range(DECODE_STEPS):
        rows = np.asarray([base[b] + cur[b] for b in range(B)])
        cu = np.arange(B + 1, dtype=np.int32)
        start = np.asarray(cur, np.int32)
        oracle.quantize_append(oc, prob.tau, prob.k_rope_bits[rows], cu, start, bt_np, latent_rot_f32=z[rows])
        rlq.quantize_append(p, dc, dev(prob.k_rope_bits[rows]), dev(cu), dev(start), bt, latent_rot=dev(z[rows]))
        ctx = start + 1
        ref_o, ref_l = oracle.decode(oc, prob.q_c_bits, prob.q_r_bits, prob.sm_scale, bt_np, ctx, prob.gain,
                                     prob.level_inner, prob.level_outer)
        out, lse = rlq.mla_decode(p, dc, q_c, q_r, prob.sm_scale, bt, dev(ctx), int(ctx.max()))
        torch.cuda.synchronize()
        check_decode(out, lse, ref_o, ref_l, ctx)
        cur = [c + 1 for c in cur]
    compare_pools(dc, oc)
