"""The boundary reports what it cannot trust.

* RLQ_DEBUG: the decode, extend and append calls check their device-resident
  tables on the host first and refuse out-of-range values (RLQ_EINVAL ->
  ValueError) with nothing launched; in-range calls give the same results as
  without the checks.
* The 16-head kernel's bounded exchange wait: when a poll gives up, the
  affected rows come out NaN (output and LSE) rather than silently wrong.
  The give-up is forced from the host (RLQ_TEST_EXCHANGE_TIMEOUT: every poll
  finds its slot empty and stops after two tries), so every kernel still runs
  to its end.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from decode_attention_rlq_amd import rlq, workloads
from gpu_helpers import check_decode, dev, device_cache_from, oracle_cache_for, oracle_decode, params_of

pytestmark = pytest.mark.gpu


@pytest.fixture
def env():
    saved = {k: os.environ.get(k) for k in ("RLQ_DEBUG", "RLQ_TEST_EXCHANGE_TIMEOUT")}
    yield os.environ
    for k, v in saved.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v


def problem(heads):
    prob = workloads.make_problem("v2lite_32k", ctx_lens=[700, 129, 2000], heads=heads, seed=55)
    oc, _ = oracle_cache_for(prob, z=oracle.rotate(prob.latent_bits, prob.rotation_bits))
    return prob, oc, device_cache_from(oc)


@pytest.mark.parametrize("heads", [16, 128])
def test_debug_checks_refuse_bad_tables(env, heads):
    print(f"debug checks: heads {heads}", flush=True)
    prob, oc, dc = problem(heads)
    p, qc, qr = params_of(prob), dev(prob.q_c_bits), dev(prob.q_r_bits)
    ctx = prob.ctx_lens.astype(np.int32)
    mcl = int(ctx.max())
    o_plain, l_plain = rlq.mla_decode(p, dc, qc, qr, prob.sm_scale, dev(prob.block_table), dev(ctx), mcl)
    torch.cuda.synchronize()
    env["RLQ_DEBUG"] = "1"
    o_dbg, l_dbg = rlq.mla_decode(p, dc, qc, qr, prob.sm_scale, dev(prob.block_table), dev(ctx), mcl)
    torch.cuda.synchronize()
    assert torch.equal(o_plain, o_dbg) and torch.equal(l_plain, l_dbg)
    bad_bt = prob.block_table.copy()
    bad_bt[1, 1] = prob.num_pages          # page id out of the pool, used by request 1 (129 tokens)
    out = torch.full_like(o_plain, 3.0)
    with pytest.raises(ValueError):
        rlq.mla_decode(p, dc, qc, qr, prob.sm_scale, dev(bad_bt), dev(ctx), mcl, out=out)
    bad_ctx = ctx.copy()
    bad_ctx[2] = mcl + 1                   # above the max_ctx_len hint
    with pytest.raises(ValueError):
        rlq.mla_decode(p, dc, qc, qr, prob.sm_scale, dev(prob.block_table), dev(bad_ctx), mcl, out=out)
    with pytest.raises(ValueError):
        rlq.mla_decode_noalloc(p, dc, qc, qr, prob.sm_scale, dev(bad_bt), dev(ctx), mcl, out=out)
    # Extend: more queries than the request has tokens.
    cuq = np.array([0, 1, 131, 132], np.int32)
    eq = dev(np.repeat(prob.q_c_bits[:1], 132, axis=0))
    er = dev(np.repeat(prob.q_r_bits[:1], 132, axis=0))
    with pytest.raises(ValueError):
        rlq.mla_extend(p, dc, eq, er, dev(cuq), 130, prob.sm_scale, dev(prob.block_table), dev(ctx), mcl)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)           # nothing ran


def test_debug_checks_refuse_bad_append(env):
    prob = workloads.make_problem("tiny")
    dc = rlq.PagedCache.allocate(prob.num_pages)
    z = dev(oracle.rotate(prob.latent_bits, prob.rotation_bits))
    p = params_of(prob)
    env["RLQ_DEBUG"] = "1"
    bad_bt = prob.block_table.copy()
    bad_bt[0, 3] = -1
    with pytest.raises(ValueError):
        rlq.quantize_append(p, dc, dev(prob.k_rope_bits), dev(prob.cu_seqlens), dev(prob.start_pos),
                            dev(bad_bt), latent_rot=z)
    bad_cu = prob.cu_seqlens.copy()
    bad_cu[1] += 1                         # does not end at n_tokens
    with pytest.raises(ValueError):
        rlq.quantize_append(p, dc, dev(prob.k_rope_bits), dev(bad_cu), dev(prob.start_pos),
                            dev(prob.block_table), latent_rot=z)
    torch.cuda.synchronize()
    assert int(dc.codes.abs().sum().item()) == 0   # nothing written
    rlq.quantize_append(p, dc, dev(prob.k_rope_bits), dev(prob.cu_seqlens), dev(prob.start_pos),
                        dev(prob.block_table), latent_rot=z)
    torch.cuda.synchronize()
    oc = oracle.new_cache(prob.num_pages)
    oracle.quantize_append(oc, prob.tau, prob.k_rope_bits, prob.cu_seqlens, prob.start_pos, prob.block_table,
                           latent_rot_f32=oracle.rotate(prob.latent_bits, prob.rotation_bits))
    assert np.array_equal(dc.codes.cpu().numpy().view(np.uint32), oc.codes)


def test_exchange_timeout_marks_rows_nan(env):
    print("forced exchange timeout, 16 heads", flush=True)
    prob, oc, dc = problem(16)
    p, qc, qr = params_of(prob), dev(prob.q_c_bits), dev(prob.q_r_bits)
    ctx = prob.ctx_lens.astype(np.int32)
    mcl = int(ctx.max())
    env["RLQ_TEST_EXCHANGE_TIMEOUT"] = "1"
    o_bad, l_bad = rlq.mla_decode(p, dc, qc, qr, prob.sm_scale, dev(prob.block_table), dev(ctx), mcl)
    torch.cuda.synchronize()
    assert torch.isnan(l_bad).all().item()
    assert torch.isnan(o_bad).any(dim=-1).all().item()
    env.pop("RLQ_TEST_EXCHANGE_TIMEOUT")
    out, lse = rlq.mla_decode(p, dc, qc, qr, prob.sm_scale, dev(prob.block_table), dev(ctx), mcl)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_decode(prob, oc)
    check_decode(out, lse, ref_o, ref_l, ctx)
