"""The per-step decode loop of a long generation: every step appends one new
token per request (the few-token append) and decodes over the grown cache.

The cache starts from short prompts and grows one token per step; with a
16-token recent ring it wraps several times, so the BF16 ring has to follow
the newest tokens ([RoLaQ] §4.1, §A.3: sink and recent tokens stay in BF16).
The oracle runs the same sequence of appends and decodes; the pools stay
bit-exact (pre-rotated latents) and every step's output is within tolerance.
The same loop captured once as a HIP graph (append, decode, advance the device
counters) and replayed gives the same result."""

import numpy as np
import pytest
import torch

import oracle
from decode_attention_rlq_amd import rlq, workloads
from gpu_helpers import check_decode, dev, host_bits, params_of

pytestmark = pytest.mark.gpu

PROMPTS = [5, 40, 100]
STEPS = 45


def loop_problem(heads):
    # Latents for prompt + generated tokens of each request (in request order).
    return workloads.make_problem("ragged_protect", ctx_lens=[n + STEPS for n in PROMPTS], heads=heads,
                                  n_sink=4, n_recent=16)


def token_rows(prob):
    """Row of each request's position p in the problem's latent arrays."""
    return [int(prob.cu_seqlens[b]) for b in range(prob.batch)]


def compare_pools(dc, oc):
    assert np.array_equal(host_bits(dc.codes), oc.codes), "codes differ"
    assert np.array_equal(host_bits(dc.meta).view(np.uint32), oc.meta.view(np.uint32)), "meta differ"
    assert np.array_equal(host_bits(dc.rope), oc.rope), "rope differ"
    assert np.array_equal(host_bits(dc.sink), oc.sink), "sink differ"
    assert np.array_equal(host_bits(dc.recent), oc.recent), "recent ring differs"


def setup(heads):
    prob = loop_problem(heads)
    B = prob.batch
    z = oracle.rotate(prob.latent_bits, prob.rotation_bits)
    base = token_rows(prob)
    prompt_rows = np.concatenate([np.arange(base[b], base[b] + PROMPTS[b]) for b in range(B)])
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(PROMPTS)
    oc = oracle.new_cache(prob.num_pages, max_batch=B, n_sink=prob.n_sink, n_recent=prob.n_recent)
    oracle.quantize_append(oc, prob.tau, prob.k_rope_bits[prompt_rows], cu, np.zeros(B, np.int32),
                           prob.block_table, latent_rot_f32=z[prompt_rows])
    dc = rlq.PagedCache.allocate(prob.num_pages, max_batch=B, n_sink=prob.n_sink, n_recent=prob.n_recent)
    p = params_of(prob)
    rlq.quantize_append(p, dc, dev(prob.k_rope_bits[prompt_rows]), dev(cu), dev(np.zeros(B, np.int32)),
                        dev(prob.block_table), latent_rot=dev(z[prompt_rows]))
    return prob, z, base, oc, dc, p


def oracle_step(prob, z, base, oc, cur):
    """Append the token at position cur[b] of each request, then decode."""
    B = prob.batch
    rows = np.asarray([base[b] + cur[b] for b in range(B)])
    oracle.quantize_append(oc, prob.tau, prob.k_rope_bits[rows], np.arange(B + 1, dtype=np.int32),
                           np.asarray(cur, np.int32), prob.block_table, latent_rot_f32=z[rows])
    ctx = np.asarray(cur, np.int32) + 1
    out, lse = oracle.decode(oc, prob.q_c_bits, prob.q_r_bits, prob.sm_scale, prob.block_table, ctx,
                             prob.gain, prob.level_inner, prob.level_outer)
    return ctx, out, lse


@pytest.mark.parametrize("heads", [16, 128])
def test_decode_loop_eager(heads):
    prob, z, base, oc, dc, p = setup(heads)
    B = prob.batch
    bt = dev(prob.block_table)
    q_c, q_r = dev(prob.q_c_bits), dev(prob.q_r_bits)
    max_ctx = max(PROMPTS) + STEPS
    cur = list(PROMPTS)
    worst = (0.0, 0.0)
    for step in range(STEPS):
        rows = np.asarray([base[b] + cur[b] for b in range(B)])
        rlq.quantize_append(p, dc, dev(prob.k_rope_bits[rows]), dev(np.arange(B + 1, dtype=np.int32)),
                            dev(np.asarray(cur, np.int32)), bt, latent_rot=dev(z[rows]))
        ctx, ref_out, ref_lse = oracle_step(prob, z, base, oc, cur)
        out, lse = rlq.mla_decode(p, dc, q_c, q_r, prob.sm_scale, bt, dev(ctx), max_ctx)
        torch.cuda.synchronize()
        err = check_decode(out, lse, ref_out, ref_lse, ctx)
        worst = tuple(max(a, b) for a, b in zip(worst, err))
        if step in (0, 11, STEPS - 1):
            compare_pools(dc, oc)
        cur = [c + 1 for c in cur]
    print(f"heads {heads}: {STEPS} steps, worst out err {worst[0]:.2e}, lse err {worst[1]:.2e}")


@pytest.mark.parametrize("heads", [16, 128])
def test_decode_loop_graph(heads):
    """One captured step advances its own device counters; replays walk the
    generation.  Checked against the oracle after 1, 17 and STEPS replays."""
    prob, z, base, oc, dc, p = setup(heads)
    B = prob.batch
    bt = dev(prob.block_table)
    q_c, q_r = dev(prob.q_c_bits), dev(prob.q_r_bits)
    max_ctx = max(PROMPTS) + STEPS
    # The new tokens of every step, laid out [step][request] so the captured
    # append reads row block `step` through a device offset.
    rows = np.asarray([[base[b] + PROMPTS[b] + s for b in range(B)] for s in range(STEPS)])
    z_steps = dev(z[rows.reshape(-1)])
    kr_steps = dev(prob.k_rope_bits[rows.reshape(-1)])
    cur_d = dev(np.asarray(PROMPTS, np.int32))
    ctx_d = cur_d + 1
    step_d = torch.zeros(1, dtype=torch.int64, device="cuda")
    new_z = torch.empty((B, 512), dtype=torch.float32, device="cuda")
    new_kr = torch.empty((B, 64), dtype=torch.bfloat16, device="cuda")
    cu_d = dev(np.arange(B + 1, dtype=np.int32))
    ws = torch.zeros(rlq.decode_workspace_size(B, heads, max_ctx), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, heads, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, heads), dtype=torch.float32, device="cuda")
    zs = z_steps.view(STEPS, B, 512)
    ks = kr_steps.view(STEPS, B, 64)

    def step(st):
        s = step_d.clamp(max=STEPS - 1)
        new_z.copy_(zs.index_select(0, s).view(B, 512))
        new_kr.copy_(ks.index_select(0, s).view(B, 64))
        rlq.quantize_append(p, dc, new_kr, cu_d, cur_d, bt, latent_rot=new_z, n_tokens=B, stream=st)
        rlq.mla_decode(p, dc, q_c, q_r, prob.sm_scale, bt, ctx_d, max_ctx, out=out, lse=lse, workspace=ws,
                       stream=st)
        cur_d.add_(1)
        ctx_d.add_(1)
        step_d.add_(1)

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step(cap)
    torch.cuda.synchronize()
    cur = list(PROMPTS)
    for s in range(STEPS):
        g.replay()
        ctx, ref_out, ref_lse = oracle_step(prob, z, base, oc, cur)
        cur = [c + 1 for c in cur]
        if s in (0, 16, STEPS - 1):
            torch.cuda.synchronize()
            assert np.array_equal(cur_d.cpu().numpy(), np.asarray(cur, np.int32))
            check_decode(out, lse, ref_out, ref_lse, ctx)
            compare_pools(dc, oc)
