"""Parity at the full sizes of the benchmarked workloads, in the launch
configurations bench.py times (same batch, heads and context lengths, so the
same split grid or work-item plan).

* 4 x 32,768- and 4 x 262,144-token decode, 16 heads: every output row and
  LSE against the oracle.
* 32-request ragged decode, 128 heads, 4 sink + 64 recent BF16 tokens,
  log-uniform lengths in [1,024, 65,536]: every output row and LSE.
* 4 x 65,536-token bulk append through the bf16 MFMA rotation: z, group
  statistics and codes of every token.
* Extend of a 512-query chunk per request over 4 x 32,768 cached tokens,
  16 heads: every output finite, sampled rows against the oracle.

The decode caches are written by the oracle from the workloads' latents taken
as already rotated (decode computes on whatever the cache holds), so no value
computed on the GPU enters an oracle input or an expected value.
"""

import types

import numpy as np
import pytest
import torch

import oracle
from decode_attention_rlq_amd import rlq, workloads
from gpu_helpers import (check_decode, check_rotated_append, dev, device_cache_from, empty_device_cache,
                         oracle_cache_for, oracle_decode, params_of, run_decode)

pytestmark = pytest.mark.gpu


def latents_as_z(prob):
    """The bf16 latents widened exactly to fp32."""
    return (prob.latent_bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("name", ["v2lite_32k", "v2lite_256k", "ragged_protect"])
def test_decode_full_size(name):
    prob = workloads.make_problem(name)
    print(f"{name}: batch {prob.batch}, heads {prob.heads}, tokens {int(prob.ctx_lens.sum())}", flush=True)
    oc, _ = oracle_cache_for(prob, z=latents_as_z(prob))
    dc = device_cache_from(oc)
    out, lse = run_decode(prob, dc)
    del dc
    torch.cuda.empty_cache()
    ref_out, ref_lse = oracle_decode(prob, oc)
    err, lerr = check_decode(out, lse, ref_out, ref_lse, prob.ctx_lens)
    print(f"{name}: out err {err:.2e}, lse err {lerr:.2e}")


def test_append_full_size_bulk():
    prob = workloads.make_problem("append_bulk")
    n = prob.n_tokens
    print(f"append_bulk: {prob.batch} x {n // prob.batch} new tokens", flush=True)
    dc = empty_device_cache(prob)
    zdbg = torch.empty((n, 512), dtype=torch.float32, device="cuda")
    rlq.quantize_append(params_of(prob), dc, dev(prob.k_rope_bits), dev(prob.cu_seqlens),
                        dev(prob.start_pos), dev(prob.block_table), latent=dev(prob.latent_bits),
                        rotation=dev(prob.rotation_bits), z_debug=zdbg)
    torch.cuda.synchronize()
    flips = check_rotated_append(prob, dc, zdbg.cpu().numpy())
    print(f"append_bulk: {flips} codes at a cut point differ from the oracle's")


def test_extend_full_size_sampled():
    """The extend call bench.py times: a 512-query chunk per request over
    4 x 32,768 cached tokens, 16 heads, same launch.  Every output is finite,
    and sampled rows (both ends of the chunk and around its middle) match the
    oracle.  This cache has no sink or recent rows, so query position p is
    exactly the one-query extend over the first p + 1 positions."""
    prob = workloads.make_problem("v2lite_32k")
    assert prob.n_sink == 0 and prob.n_recent == 0
    B, H, n, chunk = prob.batch, prob.heads, int(prob.ctx_lens[0]), 512
    print(f"extend full size: {B} x {chunk} queries over {n} tokens, {H} heads", flush=True)
    oc, _ = oracle_cache_for(prob, z=latents_as_z(prob))
    dc = device_cache_from(oc)
    rng = np.random.default_rng(7)
    qc = workloads.to_bf16_bits(rng.standard_normal((B * chunk, H, 512), dtype=np.float32))
    qr = workloads.to_bf16_bits(rng.standard_normal((B * chunk, H, 64), dtype=np.float32))
    cuq = np.arange(0, B * chunk + 1, chunk, dtype=np.int32)
    out, lse = rlq.mla_extend(params_of(prob), dc, dev(qc), dev(qr), dev(cuq), chunk, prob.sm_scale,
                              dev(prob.block_table), dev(prob.ctx_lens.astype(np.int32)), n)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item() and torch.isfinite(lse).all().item()
    one = np.array([0, 1], np.int32)
    worst = [0.0, 0.0]
    for b in range(B):
        view = types.SimpleNamespace(sm_scale=prob.sm_scale, block_table=prob.block_table[b:b + 1],
                                     gain=prob.gain, level_inner=prob.level_inner, level_outer=prob.level_outer)
        for i in (0, 1, chunk // 2 - 1, chunk // 2, chunk - 2, chunk - 1):
            r, pos = b * chunk + i, n - chunk + i
            ref_o, ref_l = oracle.extend(oc, qc[r:r + 1], qr[r:r + 1], prob.sm_scale, view.block_table, [pos + 1],
                                         one, prob.gain, prob.level_inner, prob.level_outer)
            e = check_decode(out[r:r + 1], lse[r:r + 1], ref_o, ref_l, [1])
            worst = [max(worst[0], e[0]), max(worst[1], e[1])]
    print(f"extend full size: sampled out err {worst[0]:.2e}, lse err {worst[1]:.2e}")
