"""GPU parity of rlq_quantize_append against the oracle (codes bit-exact)."""

import numpy as np
import pytest
import torch

import oracle
from decode_attention_rlq_amd import rlq, workloads
from gpu_helpers import check_rotated_append, dev, empty_device_cache, host_bits, oracle_cache_for, params_of

pytestmark = pytest.mark.gpu


def appended(prob, new_lens, start_pos):
    """Keep only positions start_pos[b] .. start_pos[b]+new_lens[b]-1 of each request as new tokens."""
    lat, kr, cu = [], [], [0]
    for b in range(prob.batch):
        lo = int(prob.cu_seqlens[b]) + int(start_pos[b])
        lat.append(prob.latent_bits[lo:lo + new_lens[b]])
        kr.append(prob.k_rope_bits[lo:lo + new_lens[b]])
        cu.append(cu[-1] + int(new_lens[b]))
    prob.latent_bits = np.concatenate(lat)
    prob.k_rope_bits = np.concatenate(kr)
    prob.cu_seqlens = np.asarray(cu, np.int32)
    prob.start_pos = np.asarray(start_pos, np.int32)
    return prob


def compare_pools(dc, oc):
    assert np.array_equal(host_bits(dc.codes), oc.codes), "codes differ"
    assert np.array_equal(host_bits(dc.meta).view(np.uint32), oc.meta.view(np.uint32)), "meta differ"
    assert np.array_equal(host_bits(dc.rope), oc.rope), "rope differ"
    if oc.sink is not None:
        assert np.array_equal(host_bits(dc.sink), oc.sink), "sink differ"
    if oc.recent is not None:
        assert np.array_equal(host_bits(dc.recent), oc.recent), "recent differ"


def gpu_append(prob, dc, *, z=None, rotation_bits=None):
    kw = dict(latent_rot=dev(z)) if z is not None else dict(
        latent=dev(prob.latent_bits), rotation=dev(prob.rotation_bits if rotation_bits is None else rotation_bits))
    rlq.quantize_append(params_of(prob), dc, dev(prob.k_rope_bits), dev(prob.cu_seqlens),
                        dev(prob.start_pos), dev(prob.block_table), **kw)
    torch.cuda.synchronize()


CASES = {
    "tiny": dict(name="tiny"),
    "ragged_offsets": dict(name="tiny", ctx_lens=[37, 6, 130, 128, 200], start=[0, 5, 27, 64, 3],
                           n_sink=4, n_recent=16),
    "protect_4_64": dict(name="ragged_protect", ctx_lens=[70, 1, 300], start=[0, 0, 100],
                         heads=16, n_sink=4, n_recent=64),
    # Requests with no new token between ones that have some (the request
    # search must skip empty requests).
    "empty_requests": dict(name="tiny", ctx_lens=[5, 9, 5, 70, 3], start=[5, 0, 5, 60, 3],
                           n_sink=2, n_recent=4),
    # 70 requests: more than one wave's worth of cu_seqlens entries.
    "many_requests": dict(name="tiny", ctx_lens=[1 + (7 * b) % 11 for b in range(70)],
                          start=[(3 * b) % 2 for b in range(70)], n_sink=1, n_recent=3),
    # More than 4096 new tokens: the persistent bulk kernel, with ragged
    # requests, start offsets and protection.
    "bulk_ragged": dict(name="tiny", ctx_lens=[1500, 3070, 7, 900, 2100], start=[0, 60, 0, 33, 64],
                        n_sink=4, n_recent=16),
    # The bulk kernel with more requests than its LDS request table holds
    # (2047): the request search runs on global memory; every ninth request
    # has no new token.
    "bulk_many_requests": dict(name="tiny", ctx_lens=[1 + (5 * b + b // 7) % 6 for b in range(2100)],
                               start=[(1 + (5 * b + b // 7) % 6) if b % 9 == 0 else
                                      (b % 2) * min(1, (5 * b + b // 7) % 6) for b in range(2100)],
                               n_sink=1, n_recent=3),
}


def build(case):
    c = dict(CASES[case])
    start = c.pop("start", None)
    prob = workloads.make_problem(c.pop("name"), **c)
    if start is not None:
        new = [int(n) - int(s) for n, s in zip(prob.ctx_lens, start)]
        prob = appended(prob, new, start)
    return prob


@pytest.mark.parametrize("case", list(CASES))
def test_append_prerotated_bitexact(case):
    prob = build(case)
    z = oracle.rotate(prob.latent_bits, prob.rotation_bits)
    oc, _ = oracle_cache_for(prob, z=z)
    dc = empty_device_cache(prob)
    gpu_append(prob, dc, z=z)
    compare_pools(dc, oc)


@pytest.mark.parametrize("case", ["tiny", "ragged_offsets"])
def test_append_signed_permutation_exact_end_to_end(case):
    prob = build(case)
    perm = workloads.signed_permutation(np.random.default_rng(5), 512)
    prob.rotation_bits = workloads.to_bf16_bits(perm)
    oc, _ = oracle_cache_for(prob)
    dc = empty_device_cache(prob)
    gpu_append(prob, dc)
    compare_pools(dc, oc)


@pytest.mark.parametrize("case", list(CASES))
def test_append_haar_rotation(case):
    """Haar rotation through bf16 MFMA: z within the fp32 accumulation bound of
    the exact product, statistics and codes as the oracle's up to what that
    bound allows; RoPE keys and protected rows bit-exact where z is."""
    prob = build(case)
    n = prob.n_tokens
    dc = empty_device_cache(prob)
    zdbg = torch.empty((n, 512), dtype=torch.float32, device="cuda")
    rlq.quantize_append(params_of(prob), dc, dev(prob.k_rope_bits), dev(prob.cu_seqlens),
                        dev(prob.start_pos), dev(prob.block_table), latent=dev(prob.latent_bits),
                        rotation=dev(prob.rotation_bits), z_debug=zdbg)
    torch.cuda.synchronize()
    check_rotated_append(prob, dc, zdbg.cpu().numpy())
    oc, _ = oracle_cache_for(prob)
    assert np.array_equal(host_bits(dc.rope), oc.rope), "rope differ"


def test_append_empty_is_noop():
    prob = workloads.make_problem("tiny")
    dc = empty_device_cache(prob, fill=0x5A5A)
    before = host_bits(dc.codes).copy()
    rlq.quantize_append(params_of(prob), dc, dev(prob.k_rope_bits), dev(prob.cu_seqlens),
                        dev(prob.start_pos), dev(prob.block_table), latent=dev(prob.latent_bits),
                        rotation=dev(prob.rotation_bits), n_tokens=0)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(dc.codes), before)


def test_append_invalid_arguments_raise():
    prob = workloads.make_problem("tiny")
    dc = empty_device_cache(prob)
    p = params_of(prob)
    with pytest.raises(ValueError):  # both latent forms given
        rlq.quantize_append(p, dc, dev(prob.k_rope_bits), dev(prob.cu_seqlens), dev(prob.start_pos),
                            dev(prob.block_table), latent=dev(prob.latent_bits),
                            latent_rot=torch.zeros((256, 512), device="cuda"),
                            rotation=dev(prob.rotation_bits))
    with pytest.raises(ValueError):  # latent without rotation
        rlq.quantize_append(p, dc, dev(prob.k_rope_bits), dev(prob.cu_seqlens), dev(prob.start_pos),
                            dev(prob.block_table), latent=dev(prob.latent_bits))
