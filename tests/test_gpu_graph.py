"""The decode step (quantize-append of the new tokens + decode) captured in a
HIP graph: every replay, with eager work and synchronizations in between,
gives bit-for-bit the eager result."""

import numpy as np
import pytest
import torch

from decode_attention_rlq_amd import rlq, workloads
from gpu_helpers import dev, params_of

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,kw", [("tiny", dict(batch=3, ctx_lens=[700, 64, 1500])),
                                     ("ragged_protect", dict(batch=2, heads=32, ctx_lens=[300, 2100]))])
def test_step_graph_replays_match_eager(name, kw):
    prob = workloads.make_problem(name, **kw)
    B, H = prob.batch, prob.heads
    p = params_of(prob)
    ctx = prob.ctx_lens.astype(np.int32)
    cache = rlq.PagedCache.allocate(prob.num_pages, max_batch=B, n_sink=prob.n_sink, n_recent=prob.n_recent)
    bt = dev(prob.block_table)
    rlq.quantize_append(p, cache, dev(prob.k_rope_bits), dev(prob.cu_seqlens), dev(prob.start_pos), bt,
                        latent=dev(prob.latent_bits), rotation=dev(prob.rotation_bits))
    new_idx = (prob.cu_seqlens[1:] - 1).astype(np.int64)
    new_lat, new_kr = dev(prob.latent_bits[new_idx]), dev(prob.k_rope_bits[new_idx])
    new_cu, new_start = dev(np.arange(B + 1, dtype=np.int32)), dev(ctx - 1)
    q_c, q_r, ctx_d, rot = dev(prob.q_c_bits), dev(prob.q_r_bits), dev(ctx), dev(prob.rotation_bits)
    max_ctx = int(ctx.max())
    ws = torch.zeros(rlq.decode_workspace_size(B, H, max_ctx), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")

    def step(o, l, st):
        rlq.quantize_append(p, cache, new_kr, new_cu, new_start, bt, latent=new_lat, rotation=rot,
                            n_tokens=B, stream=st)
        rlq.mla_decode(p, cache, q_c, q_r, prob.sm_scale, bt, ctx_d, max_ctx, out=o, lse=l, workspace=ws,
                       stream=st)

    step(out, lse, torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    out.zero_()
    with torch.cuda.graph(g, stream=cap):
        step(out, lse, cap)
    o2 = torch.empty_like(out)
    l2 = torch.empty_like(lse)
    for r in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), f"replay {r}: output differs from the eager step"
        assert torch.equal(lse, ref_l), f"replay {r}: lse differs from the eager step"
        # Eager work on the same cache and workspace between replays.
        step(o2, l2, torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert torch.equal(o2, ref_o)
