"""rlq_mla_decode_noalloc: the decode with the library's static scratch array
(for callers that cannot allocate) gives the same output as rlq_mla_decode
with a caller workspace, call after call, and refuses a call whose scratch
need exceeds the array."""

import numpy as np
import pytest
import torch

import oracle
from decode_attention_rlq_amd import rlq, workloads
from gpu_helpers import check_decode, dev, device_cache_from, oracle_cache_for, oracle_decode, params_of

pytestmark = pytest.mark.gpu


def decode_both(prob, dc, ctx):
    p, bt, cl = params_of(prob), dev(prob.block_table), dev(np.asarray(ctx, np.int32))
    qc, qr = dev(prob.q_c_bits), dev(prob.q_r_bits)
    mcl = int(max(ctx))
    ref_o, ref_l = rlq.mla_decode(p, dc, qc, qr, prob.sm_scale, bt, cl, mcl)
    out = torch.empty_like(ref_o)
    lse = torch.empty_like(ref_l)
    rlq.mla_decode_noalloc(p, dc, qc, qr, prob.sm_scale, bt, cl, mcl, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse, ref_o, ref_l


@pytest.mark.parametrize("heads", [16, 128])
def test_noalloc_matches_workspace_decode(heads):
    print(f"noalloc decode: heads {heads}", flush=True)
    prob = workloads.make_problem("ragged_protect", ctx_lens=[3000, 700, 4100], heads=heads, seed=91)
    oc, _ = oracle_cache_for(prob, z=oracle.rotate(prob.latent_bits, prob.rotation_bits))
    dc = device_cache_from(oc)
    # Two calls in a row, the second on a smaller input (shorter contexts, so
    # a smaller split grid over the same scratch, which keeps the first
    # call's contents).
    for ctx in ([3000, 700, 4100], [100, 700, 37]):
        out, lse, ref_o, ref_l = decode_both(prob, dc, ctx)
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
        ro, rl = oracle_decode(prob, oc, ctx_lens=np.asarray(ctx))
        err, lerr = check_decode(out, lse, ro, rl, ctx)
        print(f"ctx {ctx}: identical to rlq_mla_decode; vs oracle out {err:.2e}, lse {lerr:.2e}")


def test_noalloc_rejects_oversized_call():
    batch, heads, mcl = 1024, 128, 65536
    assert rlq.decode_workspace_size(batch, heads, mcl) > rlq.NOALLOC_SCRATCH_BYTES
    prob = workloads.make_problem("tiny")
    dc = rlq.PagedCache.allocate(1)
    q = torch.zeros((batch, heads, 512), dtype=torch.bfloat16, device="cuda")
    qr = torch.zeros((batch, heads, 64), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((batch, mcl // 64), dtype=torch.int32, device="cuda")
    ctx = torch.zeros(batch, dtype=torch.int32, device="cuda")
    out = torch.full((batch, heads, 512), 7.0, device="cuda")
    with pytest.raises(rlq.RlqError) as e:
        rlq.mla_decode_noalloc(params_of(prob), dc, q, qr, 0.1, bt, ctx, mcl, out=out)
    assert e.value.status == rlq.RLQ_ENOSPC
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)  # nothing ran
