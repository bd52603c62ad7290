"""Extend (prefill over the cache) parity: rlq_mla_extend against oracle.extend.

Each request's cache holds ctx tokens; its n_q queries are the last n_q
positions and attend causally to the cache as decode reads it ([RoLaQ] §D,
§2.1, §3.3).  The caches are written by the oracle from the workloads'
latents taken as already rotated, so no GPU value enters an oracle input.
Cases cover 16, 32 and 128 heads (head groups that end inside a request's
rows), ragged query counts including none, a full prefill from position 0,
and sink / recent BF16 rows.
"""

import numpy as np
import pytest
import torch

import oracle
from decode_attention_rlq_amd import rlq, workloads
from gpu_helpers import check_decode, dev, device_cache_from, oracle_cache_for, params_of

pytestmark = pytest.mark.gpu

CASES = {
    # name: (heads, ctx_lens, n_q per request, n_sink, n_recent)
    "h16_ragged_protect": (16, [200, 1000, 3000], [1, 5, 37], 4, 16),
    "h128_protect": (128, [300, 2500], [3, 12], 4, 64),
    "h16_full_prefill": (16, [700], [700], 0, 0),
    "h32_partial_group": (32, [500, 90], [9, 90], 2, 8),
    "h16_no_queries_in_one": (16, [100, 200, 64], [0, 6, 64], 0, 0),
    "h64_single_query": (64, [4097], [1], 4, 16),
}


def latents_as_z(prob):
    return (prob.latent_bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("name", list(CASES))
def test_extend_matches_oracle(name):
    heads, lens, n_q, n_sink, n_recent = CASES[name]
    print(f"extend case {name}: heads {heads}, ctx {lens}, queries {n_q}", flush=True)
    prob = workloads.make_problem("ragged_protect", ctx_lens=lens, heads=heads, n_sink=n_sink, n_recent=n_recent)
    oc, _ = oracle_cache_for(prob, z=latents_as_z(prob), protect=n_sink + n_recent > 0)
    rng = np.random.default_rng(1000 + len(name))
    cuq = np.concatenate([[0], np.cumsum(n_q)]).astype(np.int32)
    total = int(cuq[-1])
    qc = workloads.to_bf16_bits(rng.standard_normal((total, heads, 512), dtype=np.float32))
    qr = workloads.to_bf16_bits(rng.standard_normal((total, heads, 64), dtype=np.float32))
    ref_out, ref_lse = oracle.extend(oc, qc, qr, prob.sm_scale, prob.block_table, prob.ctx_lens, cuq,
                                     prob.gain, prob.level_inner, prob.level_outer)
    dc = device_cache_from(oc)
    out, lse = rlq.mla_extend(params_of(prob), dc, dev(qc), dev(qr), dev(cuq), max(n_q), prob.sm_scale,
                              dev(prob.block_table), dev(prob.ctx_lens.astype(np.int32)), int(max(lens)))
    torch.cuda.synchronize()
    rows_ctx = np.ones(total, np.int64)  # every query row sees at least position 0
    err, lerr = check_decode(out, lse, ref_out, ref_lse, rows_ctx)
    print(f"{name}: out err {err:.2e}, lse err {lerr:.2e}")


@pytest.mark.parametrize("heads", [16, 128])
def test_extend_peaked_scores(heads):
    """Queries three times wider than the workload's (scores peaked on a few
    tokens, near ties common), 1 sink + 16 recent rows: the score correction
    keeps every row within the bar."""
    lens, n_q = [900, 3000], [40, 9]
    print(f"extend peaked scores: heads {heads}, ctx {lens}, queries {n_q}", flush=True)
    prob = workloads.make_problem("ragged_protect", ctx_lens=lens, heads=heads, n_sink=1, n_recent=16, seed=79)
    oc, _ = oracle_cache_for(prob, z=latents_as_z(prob))
    rng = np.random.default_rng(2024 + heads)
    cuq = np.concatenate([[0], np.cumsum(n_q)]).astype(np.int32)
    total = int(cuq[-1])
    qc = workloads.to_bf16_bits(3.0 * rng.standard_normal((total, heads, 512), dtype=np.float32))
    qr = workloads.to_bf16_bits(rng.standard_normal((total, heads, 64), dtype=np.float32))
    ref_out, ref_lse = oracle.extend(oc, qc, qr, prob.sm_scale, prob.block_table, prob.ctx_lens, cuq,
                                     prob.gain, prob.level_inner, prob.level_outer)
    dc = device_cache_from(oc)
    out, lse = rlq.mla_extend(params_of(prob), dc, dev(qc), dev(qr), dev(cuq), max(n_q), prob.sm_scale,
                              dev(prob.block_table), dev(prob.ctx_lens.astype(np.int32)), int(max(lens)))
    torch.cuda.synchronize()
    err, lerr = check_decode(out, lse, ref_out, ref_lse, np.ones(total, np.int64))
    print(f"extend peaked, {heads} heads: out err {err:.2e}, lse err {lerr:.2e}")


def test_extend_of_one_query_equals_decode():
    """One query per request is the decode of the last position: both entry
    points on the same cache agree to rounding (different kernels for 16
    heads, the same many-head kernel for 64)."""
    for heads in (16, 64):
        prob = workloads.make_problem("ragged_protect", ctx_lens=[333, 2048, 1], heads=heads, n_sink=4,
                                      n_recent=16)
        oc, _ = oracle_cache_for(prob, z=latents_as_z(prob))
        dc = device_cache_from(oc)
        p = params_of(prob)
        bt, ctx = dev(prob.block_table), dev(prob.ctx_lens.astype(np.int32))
        qc, qr = dev(prob.q_c_bits), dev(prob.q_r_bits)
        mcl = int(prob.ctx_lens.max())
        o_d, l_d = rlq.mla_decode(p, dc, qc, qr, prob.sm_scale, bt, ctx, mcl)
        o_e, l_e = rlq.mla_extend(p, dc, qc, qr, dev(np.arange(4, dtype=np.int32)), 1, prob.sm_scale, bt, ctx, mcl)
        torch.cuda.synchronize()
        d = (o_d - o_e).abs().max().item() / o_d.abs().max().item()
        assert d < 2e-3, d
        assert (l_d - l_e).abs().max().item() < 2e-3
