"""Decode and extend at the longest context one call accepts (RLQ_MAX_CTX =
4,194,304 tokens), checked through a property that holds at any length.

Every block-table entry of a request names the same 64-token page, so its
context is that page repeated: n positions are R = n // 64 whole copies of the
page plus its first t = n % 64 tokens.  Softmax attention over a repeated
multiset follows in closed form from the attention over one copy (out_64,
lse_64) and over the t-token prefix (out_t, lse_t), both small oracle calls:

    lse = log(R exp(lse_64) + exp(lse_t))           (second term absent if t = 0)
    out = (R exp(lse_64 - lse) out_64 + exp(lse_t - lse) out_t)

This reaches the maximum split plan of the 16-head kernel (256 splits of 256
pages), the item cap of the many-head kernel (86 items of at most 1534 tiles
per request) and extend rows at the last positions, with a ragged tail; and,
at shapes with enough row groups to need no splitting, requests whose
contexts still span two or three items.  No sink /
recent rows (a repeated page has no single recent window).
"""

import types

import numpy as np
import pytest
import torch

import oracle
from decode_attention_rlq_amd import rlq, workloads
from gpu_helpers import (LSE_TOL, OUT_TOL, dev, device_cache_from, oracle_cache_for, params_of,
                         row_rel_err)

pytestmark = pytest.mark.gpu

MAX_CTX = 4194304
PAGES = MAX_CTX // 64


def one_page_problem(heads):
    prob = workloads.make_problem("v2lite_32k", ctx_lens=[64, 64], heads=heads)
    z = (prob.latent_bits.astype(np.uint32) << 16).view(np.float32)
    oc, _ = oracle_cache_for(prob, z=z, protect=False)
    # Request b's whole block table names its one page.
    bt = np.repeat(np.asarray(prob.block_table)[:, :1], PAGES, axis=1).astype(np.int32)
    return prob, oc, bt


def repeated_reference(prob, oc, b, qc, qr, n):
    """(out [H][512], lse [H]) of one query over the first n positions of
    request b's repeated page, from the oracle over one copy and the tail."""
    one = np.array([0, 1], np.int32)
    bt = np.asarray(prob.block_table)[b:b + 1]

    def attend(m):
        o, l = oracle.extend(oc, qc[None], qr[None], prob.sm_scale, bt, [m], one, prob.gain,
                             prob.level_inner, prob.level_outer)
        return o[0], l[0]

    reps, tail = divmod(n, 64)
    o64, l64 = attend(64)
    big = l64 + np.log(reps)
    if tail == 0:
        return o64, big
    ot, lt = attend(tail)
    lse = np.logaddexp(big, lt)
    out = np.exp(big - lse)[:, None] * o64 + np.exp(lt - lse)[:, None] * ot
    return out, lse


def check_row(out, lse, ref_out, ref_lse):
    out, lse = out.astype(np.float64), lse.astype(np.float64)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    err = row_rel_err(out, ref_out)
    lerr = np.abs(lse - ref_lse)
    assert err <= OUT_TOL, f"output row-relative error {err:.3e}"
    assert (lerr <= LSE_TOL).all(), f"lse error {lerr.max():.3e} > {LSE_TOL}"
    return err, float(lerr.max())


@pytest.mark.parametrize("heads", [16, 128])
def test_decode_at_max_context(heads):
    ctx = np.array([MAX_CTX, MAX_CTX - 17], np.int32)
    print(f"max-context decode: heads {heads}, ctx {ctx.tolist()}", flush=True)
    prob, oc, bt = one_page_problem(heads)
    out, lse = rlq.mla_decode(params_of(prob), device_cache_from(oc), dev(prob.q_c_bits), dev(prob.q_r_bits),
                              prob.sm_scale, dev(bt), dev(ctx), MAX_CTX)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for b in range(2):
        ref_o, ref_l = repeated_reference(prob, oc, b, prob.q_c_bits[b], prob.q_r_bits[b], int(ctx[b]))
        e = check_row(out[b], lse[b], ref_o, ref_l)
        print(f"request {b}: out err {e[0]:.2e}, lse err {e[1]:.2e}")


def test_extend_at_max_context():
    heads, n_q = 16, [3, 2]
    ctx = np.array([MAX_CTX, MAX_CTX - 17], np.int32)
    print(f"max-context extend: heads {heads}, ctx {ctx.tolist()}, queries {n_q}", flush=True)
    prob, oc, bt = one_page_problem(heads)
    cuq = np.array([0, n_q[0], n_q[0] + n_q[1]], np.int32)
    rng = np.random.default_rng(4242)
    qc = workloads.to_bf16_bits(rng.standard_normal((int(cuq[-1]), heads, 512), dtype=np.float32))
    qr = workloads.to_bf16_bits(rng.standard_normal((int(cuq[-1]), heads, 64), dtype=np.float32))
    out, lse = rlq.mla_extend(params_of(prob), device_cache_from(oc), dev(qc), dev(qr), dev(cuq), max(n_q),
                              prob.sm_scale, dev(bt), dev(ctx), MAX_CTX)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for b in range(2):
        for i in range(n_q[b]):
            r = int(cuq[b]) + i
            n = int(ctx[b]) - n_q[b] + i + 1
            ref_o, ref_l = repeated_reference(prob, oc, b, qc[r], qr[r], n)
            e = check_row(out[r], lse[r], ref_o, ref_l)
            print(f"request {b} query {i} (positions {n}): out err {e[0]:.2e}, lse err {e[1]:.2e}")


# The plan without context splitting: when (request, 64-row group) workgroups
# alone fill the GPU (at least 512 of them), every request gets one work item
# of up to 1534 tiles (49,088 tokens), and only longer contexts span several
# items (then merged through partials).  The same repeated-page property
# checks both paths at their real shapes.

def test_decode_many_requests_spanning_two_items():
    """256 requests x 128 heads (512 row-group workgroups: no splitting) with
    contexts of 49,089 .. 74,374 tokens: two work items each, merged."""
    heads, B = 128, 256
    prob, oc, bt2 = one_page_problem(heads)
    ctx = (49089 + 99 * np.arange(B)).astype(np.int32)
    max_ctx = int(ctx.max())
    pages = (max_ctx + 63) // 64
    page_of = np.asarray(prob.block_table)[:, 0]
    bt = np.repeat(page_of[np.arange(B) % 2][:, None], pages, axis=1).astype(np.int32)
    rng = np.random.default_rng(515)
    qc = workloads.to_bf16_bits(rng.standard_normal((B, heads, 512), dtype=np.float32))
    qr = workloads.to_bf16_bits(rng.standard_normal((B, heads, 64), dtype=np.float32))
    print(f"decode, {B} requests x {heads} heads, ctx {ctx.min()}..{ctx.max()}", flush=True)
    out, lse = rlq.mla_decode(params_of(prob), device_cache_from(oc), dev(qc), dev(qr), prob.sm_scale, dev(bt),
                              dev(ctx), max_ctx)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    worst = (0.0, 0.0)
    for b in list(range(0, B, 17)) + [B - 1]:
        ref_o, ref_l = repeated_reference(prob, oc, b % 2, qc[b], qr[b], int(ctx[b]))
        e = check_row(out[b], lse[b], ref_o, ref_l)
        worst = (max(worst[0], e[0]), max(worst[1], e[1]))
    print(f"sampled requests: worst out err {worst[0]:.2e}, lse err {worst[1]:.2e}")


def test_extend_many_rows_spanning_items():
    """2 requests x 2048 queries x 16 heads (1024 row-group workgroups: no
    splitting) over contexts of 100,000 and 99,937 tokens: three work items
    per request, merged; sampled (query, head) rows."""
    heads, n_q = 16, 2048
    prob, oc, bt2 = one_page_problem(heads)
    ctx = np.array([100000, 99937], np.int32)
    pages = (int(ctx.max()) + 63) // 64
    bt = np.repeat(np.asarray(prob.block_table)[:, :1], pages, axis=1).astype(np.int32)
    cuq = np.array([0, n_q, 2 * n_q], np.int32)
    rng = np.random.default_rng(2049)
    qc = workloads.to_bf16_bits(rng.standard_normal((2 * n_q, heads, 512), dtype=np.float32))
    qr = workloads.to_bf16_bits(rng.standard_normal((2 * n_q, heads, 64), dtype=np.float32))
    print(f"extend, 2 x {n_q} queries x {heads} heads, ctx {ctx.tolist()}", flush=True)
    out, lse = rlq.mla_extend(params_of(prob), device_cache_from(oc), dev(qc), dev(qr), dev(cuq), n_q,
                              prob.sm_scale, dev(bt), dev(ctx), int(ctx.max()))
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    worst = (0.0, 0.0)
    for b in range(2):
        for i in [0, 1, 777, 1500, n_q - 2, n_q - 1]:
            r = int(cuq[b]) + i
            n = int(ctx[b]) - n_q + i + 1
            ref_o, ref_l = repeated_reference(prob, oc, b, qc[r], qr[r], n)
            e = check_row(out[r], lse[r], ref_o, ref_l)
            worst = (max(worst[0], e[0]), max(worst[1], e[1]))
    print(f"sampled rows: worst out err {worst[0]:.2e}, lse err {worst[1]:.2e}")
