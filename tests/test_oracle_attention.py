"""Pins for the oracle's read side: dequant, decode, split merge (CPU only)."""

import math

import mpmath
import numpy as np
import pytest
import torch

import oracle
from decode_attention_rlq_amd import workloads


def rand_bf16(rng, shape, scale=1.0):
    return workloads.to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * scale)


def build_cache(rng, n_tokens, d_c=32, d_r=4, page=4, group=8, tau=0.9, n_sink=0,
                n_recent=0, perm=None):
    num_pages = (n_tokens + page - 1) // page
    cache = oracle.new_cache(num_pages, d_c, d_r, page, group, max_batch=1,
                             n_sink=n_sink, n_recent=n_recent)
    z = (rng.standard_normal((n_tokens, d_c)) * 1.3 + 0.2).astype(np.float32)
    kr = rand_bf16(rng, (n_tokens, d_r))
    bt = (np.arange(num_pages)[None, :] if perm is None else perm[None, :]).astype(np.int32)
    oracle.quantize_append(cache, tau, kr, [0, n_tokens], [0], bt, latent_rot_f32=z)
    return cache, z, kr, bt


def test_dequant_formula_and_degenerate_cases():
    words = oracle.pack_codes(np.array([[0, 1, 2, 3] * 4], np.uint8))
    meta = np.array([[0.25, -1.0, 2.0, 0.5]], np.float32)  # mu0, mu1, s0, s1; groups of 8
    c = oracle.dequant(words, meta, 1.5, 0.5, 1.25, group=8)
    g0 = [0.25 - 3.0 * 1.25, 0.25 - 3.0 * 0.5, 0.25 + 3.0 * 0.5, 0.25 + 3.0 * 1.25]
    g1 = [-1.0 - 0.75 * 1.25, -1.0 - 0.75 * 0.5, -1.0 + 0.75 * 0.5, -1.0 + 0.75 * 1.25]
    assert np.array_equal(c[0], g0 * 2 + g1 * 2)
    assert np.array_equal(oracle.dequant(words, meta, 0.0, 0.5, 1.25, group=8)[0], [0.25] * 8 + [-1.0] * 8)
    meta0 = np.array([[0.25, -1.0, 0.0, 0.0]], np.float32)
    assert np.array_equal(oracle.dequant(words, meta0, 1.5, 0.5, 1.25, group=8)[0], [0.25] * 8 + [-1.0] * 8)


def test_single_token_returns_its_latent():
    rng = np.random.default_rng(1)
    cache, z, kr, bt = build_cache(rng, 1)
    qc = rand_bf16(rng, (1, 3, 32))
    qr = rand_bf16(rng, (1, 3, 4))
    out, lse = oracle.decode(cache, qc, qr, 0.3, bt, [1], 1.1, 0.4528, 1.51)
    c_hat = oracle.dequant(cache.codes[0, 0], cache.meta[0, 0], 1.1, 0.4528, 1.51, group=8)
    assert np.allclose(out[0], c_hat[None, :], rtol=0, atol=1e-14)
    s = float(np.float32(0.3)) * (oracle.bf16_bits_to_f64(qc[0]) @ c_hat + oracle.bf16_bits_to_f64(qr[0]) @ oracle.bf16_bits_to_f64(kr[0]))
    assert np.allclose(lse[0], s, atol=1e-13)


def test_zero_query_returns_mean_latent():
    rng = np.random.default_rng(2)
    cache, z, kr, bt = build_cache(rng, 37)
    qc = np.zeros((1, 2, 32), np.uint16)
    qr = np.zeros((1, 2, 4), np.uint16)
    out, lse = oracle.decode(cache, qc, qr, 0.1, bt, [37], 1.0, 0.4528, 1.51)
    c_hat, _ = oracle.gather_request(cache, bt[0], 37, 1.0, 0.4528, 1.51)
    assert np.allclose(out[0], c_hat.mean(axis=0)[None, :], atol=1e-13)
    assert np.allclose(lse[0], math.log(37), atol=1e-13)


def test_two_tokens_follow_the_logistic():
    rng = np.random.default_rng(3)
    cache, z, kr, bt = build_cache(rng, 2)
    qc = rand_bf16(rng, (1, 1, 32))
    qr = rand_bf16(rng, (1, 1, 4))
    out, lse = oracle.decode(cache, qc, qr, 0.2, bt, [2], 1.0, 0.4528, 1.51)
    c_hat, k = oracle.gather_request(cache, bt[0], 2, 1.0, 0.4528, 1.51)
    q = oracle.bf16_bits_to_f64(qc[0, 0])
    r = oracle.bf16_bits_to_f64(qr[0, 0])
    s = [float(np.float32(0.2)) * (q @ c_hat[t] + r @ k[t]) for t in range(2)]
    p1 = 1 / (1 + math.exp(-(s[0] - s[1])))
    assert np.allclose(out[0, 0], p1 * c_hat[0] + (1 - p1) * c_hat[1], atol=1e-13)


def test_token_permutation_invariance():
    rng = np.random.default_rng(4)
    n = 40
    cache, z, kr, bt = build_cache(rng, n)
    order = rng.permutation(n)
    cache2 = oracle.new_cache(10, 32, 4, 4, 8)
    oracle.quantize_append(cache2, 0.9, kr[order], [0, n], [0], np.arange(10)[None, :],
                           latent_rot_f32=z[order])
    qc = rand_bf16(rng, (1, 4, 32))
    qr = rand_bf16(rng, (1, 4, 4))
    o1, l1 = oracle.decode(cache, qc, qr, 0.25, bt, [n], 1.05, 0.4528, 1.51)
    o2, l2 = oracle.decode(cache2, qc, qr, 0.25, np.arange(10)[None, :], [n], 1.05, 0.4528, 1.51)
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(l1, l2, atol=1e-12)


def test_page_order_does_not_matter():
    rng = np.random.default_rng(5)
    perm = np.array([3, 0, 4, 1, 2])
    cache, z, kr, bt = build_cache(rng, 19, perm=perm)
    cache2, _, _, bt2 = build_cache(np.random.default_rng(5), 19)
    qc = rand_bf16(rng, (1, 2, 32))
    qr = rand_bf16(rng, (1, 2, 4))
    o1, _ = oracle.decode(cache, qc, qr, 0.25, bt, [19], 1.0, 0.4528, 1.51)
    o2, _ = oracle.decode(cache2, qc, qr, 0.25, bt2, [19], 1.0, 0.4528, 1.51)
    assert np.array_equal(o1, o2)


def test_mpmath_bruteforce_tiny_cache():
    rng = np.random.default_rng(6)
    mpmath.mp.dps = 50
    d_c, d_r, group, n = 16, 2, 4, 7
    cache = oracle.new_cache(2, d_c, d_r, 4, group)
    z = rng.standard_normal((n, d_c)).astype(np.float32)
    kr = rand_bf16(rng, (n, d_r))
    oracle.quantize_append(cache, 0.93, kr, [0, n], [0], [[0, 1]], latent_rot_f32=z)
    qc = rand_bf16(rng, (1, 2, d_c))
    qr = rand_bf16(rng, (1, 2, d_r))
    g, a, b, sm = 1.15, 0.4528, 1.51, 0.37
    out, lse = oracle.decode(cache, qc, qr, sm, [[0, 1]], [n], g, a, b)
    A, B, G, SM = (mpmath.mpf(float(np.float32(x))) for x in (a, b, g, sm))
    lv = [-B, -A, A, B]
    for h in range(2):
        q = [mpmath.mpf(float(x)) for x in oracle.bf16_bits_to_f64(qc[0, h])]
        r = [mpmath.mpf(float(x)) for x in oracle.bf16_bits_to_f64(qr[0, h])]
        rows, scores = [], []
        for t in range(n):
            pg, sl = divmod(t, 4)
            w = int(cache.codes[pg, sl, 0])
            mu = [mpmath.mpf(float(x)) for x in cache.meta[pg, sl, :4]]
            sc = [mpmath.mpf(float(x)) for x in cache.meta[pg, sl, 4:]]
            row = [mu[j // group] + sc[j // group] * G * lv[(w >> (2 * j)) & 3] for j in range(d_c)]
            k = [mpmath.mpf(float(x)) for x in oracle.bf16_bits_to_f64(cache.rope[pg, sl])]
            rows.append(row)
            scores.append(SM * (sum(q[j] * row[j] for j in range(d_c)) + sum(r[j] * k[j] for j in range(d_r))))
        den = sum(mpmath.exp(s) for s in scores)
        for j in range(d_c):
            o = sum(mpmath.exp(scores[t]) * rows[t][j] for t in range(n)) / den
            assert abs(float(o) - out[0, h, j]) < 1e-13
        assert abs(float(mpmath.log(den)) - lse[0, h]) < 1e-13


def test_all_protected_equals_library_attention():
    # Every token protected: decode is plain softmax(q k^T) v over bf16 latents.
    rng = np.random.default_rng(7)
    n, d_c, d_r = 12, 32, 4
    cache, z, kr, bt = build_cache(rng, n, n_sink=4, n_recent=8)
    qc = rand_bf16(rng, (1, 3, d_c))
    qr = rand_bf16(rng, (1, 3, d_r))
    sm = 0.31
    out, lse = oracle.decode(cache, qc, qr, sm, bt, [n], 1.0, 0.4528, 1.51)
    c = torch.tensor(oracle.bf16_bits_to_f64(oracle.f32_to_bf16_bits(z)))
    k = torch.cat([c, torch.tensor(oracle.bf16_bits_to_f64(kr))], dim=1)
    q = torch.cat([torch.tensor(oracle.bf16_bits_to_f64(qc[0])), torch.tensor(oracle.bf16_bits_to_f64(qr[0]))], dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], c[None], scale=float(np.float32(sm)))[0]
    assert np.allclose(out[0], ref.numpy(), atol=1e-12)
    lse_ref = torch.logsumexp(float(np.float32(sm)) * (q @ k.T), dim=1).numpy()
    assert np.allclose(lse[0], lse_ref, atol=1e-12)


def test_protection_reads_bf16_and_ignores_codes():
    rng = np.random.default_rng(8)
    n = 30
    cache, z, kr, bt = build_cache(rng, n, n_sink=4, n_recent=8)
    qc = rand_bf16(rng, (1, 2, 32))
    qr = rand_bf16(rng, (1, 2, 4))
    o1, l1 = oracle.decode(cache, qc, qr, 0.25, bt, [n], 1.0, 0.4528, 1.51)
    # Garbage in the codes/meta of protected positions changes nothing.
    for t in list(range(4)) + list(range(n - 8, n)):
        pg, sl = bt[0, t // 4], t % 4
        cache.codes[pg, sl] = rng.integers(0, 2 ** 32, size=cache.codes.shape[-1], dtype=np.uint32)
        cache.meta[pg, sl] = rng.standard_normal(cache.meta.shape[-1]) * 100
    o2, l2 = oracle.decode(cache, qc, qr, 0.25, bt, [n], 1.0, 0.4528, 1.51)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # And protected rows really are the bf16 latents: compare with a cache
    # where those rows are quantized instead.
    c_hat, _ = oracle.gather_request(cache, bt[0], n, 1.0, 0.4528, 1.51)
    zb = oracle.bf16_bits_to_f64(oracle.f32_to_bf16_bits(z))
    assert np.abs(c_hat[:4] - zb[:4]).max() > 1e-3


def test_rotation_invariance_in_all_protected_mode():
    # decode(Rq, Rc) = R decode(q, c) when every token is stored exactly:
    # with a signed permutation R the bf16 values map exactly.
    rng = np.random.default_rng(9)
    n, d_c = 10, 32
    p = workloads.signed_permutation(rng, d_c).astype(np.float64)
    cache, z, kr, bt = build_cache(rng, n, n_sink=4, n_recent=8)
    zr = (z.astype(np.float64) @ p.T).astype(np.float32)
    cache2 = oracle.new_cache(3, d_c, 4, 4, 8, max_batch=1, n_sink=4, n_recent=8)
    oracle.quantize_append(cache2, 0.9, kr, [0, n], [0], bt, latent_rot_f32=zr)
    qc = rand_bf16(rng, (1, 2, d_c))
    qcr = workloads.to_bf16_bits((workloads.bf16_bits_to_f32(qc).astype(np.float64) @ p.T).astype(np.float32))
    qr = rand_bf16(rng, (1, 2, 4))
    o1, l1 = oracle.decode(cache, qc, qr, 0.3, bt, [n], 1.0, 0.4528, 1.51)
    o2, l2 = oracle.decode(cache2, qcr, qr, 0.3, bt, [n], 1.0, 0.4528, 1.51)
    assert np.allclose(o2[0], o1[0] @ p.T, atol=1e-13) and np.allclose(l1, l2, atol=1e-13)


def test_split_merge_equals_whole():
    rng = np.random.default_rng(10)
    n = 50
    cache, z, kr, bt = build_cache(rng, n)
    qc = oracle.bf16_bits_to_f64(rand_bf16(rng, (3, 32)))
    qr = oracle.bf16_bits_to_f64(rand_bf16(rng, (3, 4)))
    c_hat, k = oracle.gather_request(cache, bt[0], n, 1.0, 0.4528, 1.51)
    whole = oracle.attend(qc, qr, c_hat, k, 0.3)
    for cuts in ([0, 50], [0, 17, 50], [0, 1, 2, 30, 49, 50], [0, 0, 25, 25, 50]):
        parts = [oracle.attend_partial(qc, qr, c_hat[a:b], k[a:b], 0.3) for a, b in zip(cuts, cuts[1:])]
        out, lse = oracle.lse_merge(parts)
        assert np.allclose(out, whole[0], atol=1e-13) and np.allclose(lse, whole[1], atol=1e-13)


def test_empty_context():
    rng = np.random.default_rng(11)
    cache, z, kr, bt = build_cache(rng, 4)
    qc = rand_bf16(rng, (1, 2, 32))
    qr = rand_bf16(rng, (1, 2, 4))
    out, lse = oracle.decode(cache, qc, qr, 0.3, bt, [0], 1.0, 0.4528, 1.51)
    assert not out.any() and np.all(np.isneginf(lse))
