"""Parity at the full sizes of the benchmarked workloads, in the launch
configurations bench.py times (same batch, heads and context lengths, so the
same split grid or work-item plan).

* 4 x 262,144-token decode, 16 heads: every output row and LSE against the
  oracle.
* 32-request ragged decode, 128 heads, 4 sink + 64 recent BF16 tokens,
  log-uniform lengths in [1,024, 65,536]: every output row and LSE.
* 4 x 65,536-token bulk append through the bf16 MFMA rotation: z, group
  statistics and codes of every token.

The decode caches are written by the oracle from the workloads' latents taken
as already rotated (decode computes on whatever the cache holds), so no value
computed on the GPU enters an oracle input or an expected value.
"""

import numpy as np
import pytest
import torch

import oracle
from decode_attention_rlq_amd import rlq, workloads
from gpu_helpers import (check_decode, lse_tolerance, check_rotated_append, dev, device_cache_from, empty_device_cache,
                         oracle_cache_for, oracle_decode, params_of, run_decode)

pytestmark = pytest.mark.gpu


def latents_as_z(prob):
    """The bf16 latents widened exactly to fp32."""
    return (prob.latent_bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("name", ["v2lite_256k", "ragged_protect"])
def test_decode_full_size(name):
    prob = workloads.make_problem(name)
    print(f"{name}: batch {prob.batch}, heads {prob.heads}, tokens {int(prob.ctx_lens.sum())}", flush=True)
    oc, _ = oracle_cache_for(prob, z=latents_as_z(prob))
    dc = device_cache_from(oc)
    out, lse = run_decode(prob, dc)
    del dc
    torch.cuda.empty_cache()
    ref_out, ref_lse = oracle_decode(prob, oc)
    err, lerr = check_decode(out, lse, ref_out, ref_lse, prob.ctx_lens, lse_tolerance(prob, oc))
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
