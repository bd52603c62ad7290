"""Shared helpers for the GPU parity tests: move seeded inputs to the device,
build oracle caches, compare results.  The oracle side and the HIP side only
meet here, on the same seeded inputs."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from decode_attention_rlq_amd import rlq

OUT_TOL = 2e-3   # row-normalised max relative error of the decode output
LSE_TOL = 2e-3   # absolute error of the natural-log LSE


def dev(x: np.ndarray, dtype=None) -> torch.Tensor:
    """numpy -> cuda tensor; uint16 arrays are bf16 bit patterns, uint32 are code words."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    if x.dtype == np.uint32:
        return torch.from_numpy(x.view(np.int32)).cuda()
    t = torch.from_numpy(x)
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    """cuda tensor -> numpy with the bit patterns of include/rlq.h."""
    a = t.detach().cpu()
    if a.dtype == torch.bfloat16:
        return a.view(torch.int16).numpy().view(np.uint16)
    if a.dtype == torch.int32:
        return a.numpy().view(np.uint32)
    return a.numpy()


def params_of(prob) -> rlq.LayerParams:
    return rlq.params(prob.tau, prob.gain, prob.level_inner, prob.level_outer)


def oracle_cache_for(prob, *, z=None, protect=True):
    """Cache written by the oracle from the problem's latents (or a given z)."""
    cache = oracle.new_cache(prob.num_pages, max_batch=prob.batch,
                             n_sink=prob.n_sink if protect else 0,
                             n_recent=prob.n_recent if protect else 0)
    kw = dict(latent_rot_f32=z) if z is not None else dict(
        latent_bf16=prob.latent_bits, rotation_bf16=prob.rotation_bits)
    zz = oracle.quantize_append(cache, prob.tau, prob.k_rope_bits, prob.cu_seqlens,
                                prob.start_pos, prob.block_table, **kw)
    return cache, zz


def device_cache_from(cache: oracle.Cache) -> rlq.PagedCache:
    return rlq.PagedCache(codes=dev(cache.codes), meta=dev(cache.meta), rope=dev(cache.rope),
                          sink=None if cache.sink is None else dev(cache.sink),
                          recent=None if cache.recent is None else dev(cache.recent))


def empty_device_cache(prob, protect=True, fill=None) -> rlq.PagedCache:
    c = rlq.PagedCache.allocate(prob.num_pages, max_batch=prob.batch,
                                n_sink=prob.n_sink if protect else 0,
                                n_recent=prob.n_recent if protect else 0)
    if fill is not None:
        for t in (c.codes, c.meta, c.rope, c.sink, c.recent):
            if t is not None:
                t.view(torch.int16 if t.element_size() == 2 else torch.int32).fill_(fill)
    return c


def row_rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """max over (request, head) of max_j |out - ref| / max_j |ref|."""
    num = np.abs(out - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return float((num / den).max())


def check_decode(out, lse, ref_out, ref_lse, ctx_lens):
    """Output within OUT_TOL (row-normalised) and LSE within LSE_TOL of the
    oracle; empty contexts give 0 and -inf."""
    out = out.detach().cpu().numpy().astype(np.float64)
    lse = lse.detach().cpu().numpy().astype(np.float64)
    ctx = np.asarray(ctx_lens)
    empty = ctx == 0
    if empty.any():
        assert np.all(out[empty] == 0)
        assert np.all(np.isneginf(lse[empty]))
    full = ~empty
    err = row_rel_err(out[full], ref_out[full]) if full.any() else 0.0
    lerr = float(np.abs(lse[full] - ref_lse[full]).max()) if full.any() else 0.0
    assert np.isfinite(out).all()
    assert err <= OUT_TOL, f"output row-relative error {err:.3e} > {OUT_TOL}"
    assert lerr <= LSE_TOL, f"lse error {lerr:.3e} > {LSE_TOL}"
    return err, lerr


def run_decode(prob, cache: rlq.PagedCache, max_ctx_len=None, ctx_lens=None):
    ctx = prob.ctx_lens if ctx_lens is None else np.asarray(ctx_lens, np.int32)
    mcl = int(ctx.max()) if max_ctx_len is None else max_ctx_len
    out, lse = rlq.mla_decode(params_of(prob), cache, dev(prob.q_c_bits), dev(prob.q_r_bits),
                              prob.sm_scale, dev(prob.block_table), dev(ctx.astype(np.int32)), mcl)
    torch.cuda.synchronize()
    return out, lse


def oracle_decode(prob, cache: oracle.Cache, ctx_lens=None, heads=None):
    ctx = prob.ctx_lens if ctx_lens is None else ctx_lens
    return oracle.decode(cache, prob.q_c_bits, prob.q_r_bits, prob.sm_scale, prob.block_table,
                         ctx, prob.gain, prob.level_inner, prob.level_outer, heads=heads)


def gathered_pools(prob, dc):
    """GPU codes [n][32] (uint32) and meta [n][8] (fp32) of the appended tokens, in
    cu_seqlens order (request b, positions start_pos[b] ...)."""
    pages, slots = [], []
    for b in range(prob.batch):
        new = int(prob.cu_seqlens[b + 1] - prob.cu_seqlens[b])
        pos = int(prob.start_pos[b]) + np.arange(new)
        pages.append(np.asarray(prob.block_table[b])[pos // 64])
        slots.append(pos % 64)
    pages, slots = np.concatenate(pages), np.concatenate(slots)
    codes = host_bits(dc.codes)[pages, slots]
    meta = host_bits(dc.meta)[pages, slots]
    return codes, meta


def unpacked(words: np.ndarray) -> np.ndarray:
    """2-bit codes [n][512] from words [n][32], 16 per word, least significant first."""
    shifts = (2 * np.arange(16)).astype(np.uint32)
    return ((words[..., None] >> shifts) & np.uint32(3)).reshape(words.shape[0], -1).astype(np.int8)


def check_rotated_append(prob, dc, z_gpu):
    """Append through the bf16 MFMA rotation against the oracle's exact rotation.

    The oracle encodes fl32(c R^T) taken in fp64; the GPU accumulates in fp32,
    so (RoLaQ §3.3 puts the rotation before the quantizer) its z is checked
    against the fp32 accumulation bound gamma_512 * |c| |R|^T of the exact
    product, its group statistics against the oracle's within what that bound
    allows, and any code that differs from the oracle's must sit within that
    slack of a cut point (-t, 0, +t).  Nothing computed on the GPU is fed to
    the oracle."""
    c = oracle.bf16_bits_to_f64(prob.latent_bits)
    r = oracle.bf16_bits_to_f64(prob.rotation_bits)
    z_exact = c @ r.T
    gamma = 512 * 2.0 ** -24 / (1 - 512 * 2.0 ** -24)
    bound = gamma * (np.abs(c) @ np.abs(r).T) + np.abs(z_exact) * 2.0 ** -24
    assert np.all(np.abs(z_gpu - z_exact) <= bound), "z outside the fp32 accumulation bound"
    z_or = z_exact.astype(np.float32)
    w_o, m_o = oracle.encode_tokens(z_or, prob.tau)
    w_g, m_g = gathered_pools(prob, dc)
    # Group statistics: a shift of at most B in every coordinate moves the mean
    # by at most B and the population std by at most 2B (both up to fp32
    # rounding of the sums).
    bg = bound.reshape(bound.shape[0], 4, 128).max(axis=2) + 1e-6 * np.abs(z_or).reshape(-1, 4, 128).max(axis=2)
    assert np.all(np.abs(m_g[:, :4] - m_o[:, :4]) <= bg), "group means differ beyond the bound"
    assert np.all(np.abs(m_g[:, 4:] - m_o[:, 4:]) <= 2 * bg), "group scales differ beyond the bound"
    co, cg = oracle.unpack_codes(w_o), unpacked(w_g)
    diff = co != cg
    assert diff.mean() < 1e-3, f"{diff.sum()} codes differ"
    if diff.any():
        mu, s, d = oracle.group_stats(z_or)
        t = (np.float32(prob.tau) * s).repeat(128, axis=1)
        dist = np.minimum(np.minimum(np.abs(d - t), np.abs(d + t)), np.abs(d))
        slack = (4 * bound.max(axis=1, keepdims=True) +
                 np.abs(m_o - m_g).max(axis=1, keepdims=True) * (1 + float(prob.tau)))
        assert np.all(dist[diff] <= np.broadcast_to(slack, d.shape)[diff])
    return int(diff.sum())
