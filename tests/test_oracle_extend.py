"""Pins for the oracle's extend (prefill over the cache) attention (CPU only).

Query i of a request with ctx tokens and n_q queries sits at position
p = ctx - n_q + i and attends to positions 0 .. p, each read as decode reads
it with the cache state at ctx ([RoLaQ] §D: prefill and decode both read the
cache; §2.1 / §3.3: the attention).
"""

import math

import mpmath
import numpy as np

import oracle
from decode_attention_rlq_amd import workloads

A_IN, A_OUT = 0.4528, 1.51


def rand_bf16(rng, shape, scale=1.0):
    return workloads.to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * scale)


def build(rng, lens, d_c=32, d_r=4, page=4, group=8, n_sink=0, n_recent=0):
    """A cache with len(lens) requests on disjoint, shuffled pages."""
    ppr = max((n + page - 1) // page for n in lens)
    perm = rng.permutation(ppr * len(lens)).astype(np.int32)
    bt = perm.reshape(len(lens), ppr)
    cache = oracle.new_cache(ppr * len(lens), d_c, d_r, page, group, max_batch=len(lens),
                             n_sink=n_sink, n_recent=n_recent)
    total = int(sum(lens))
    z = (rng.standard_normal((total, d_c)) * 1.3 + 0.2).astype(np.float32)
    kr = rand_bf16(rng, (total, d_r))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    oracle.quantize_append(cache, 0.9, kr, cu, np.zeros(len(lens), np.int32), bt, latent_rot_f32=z)
    return cache, z, cu, bt


def test_single_query_equals_decode():
    rng = np.random.default_rng(21)
    lens = [11, 6]
    cache, _, _, bt = build(rng, lens, n_sink=2, n_recent=3)
    qc = rand_bf16(rng, (2, 3, 32))
    qr = rand_bf16(rng, (2, 3, 4))
    o_d, l_d = oracle.decode(cache, qc, qr, 0.3, bt, lens, 1.1, A_IN, A_OUT)
    o_e, l_e = oracle.extend(cache, qc, qr, 0.3, bt, lens, [0, 1, 2], 1.1, A_IN, A_OUT)
    assert np.array_equal(o_d, o_e) and np.array_equal(l_d, l_e)


def test_unprotected_query_i_equals_decode_over_its_prefix():
    # Without sink / recent rows the cache reads the same at every length, so
    # query i is decode over the first p + 1 positions.
    rng = np.random.default_rng(22)
    lens, n_q = [13, 9], [5, 9]
    cache, _, _, bt = build(rng, lens)
    cuq = np.concatenate([[0], np.cumsum(n_q)]).astype(np.int32)
    qc = rand_bf16(rng, (cuq[-1], 2, 32))
    qr = rand_bf16(rng, (cuq[-1], 2, 4))
    out, lse = oracle.extend(cache, qc, qr, 0.27, bt, lens, cuq, 0.9, A_IN, A_OUT)
    for b in range(2):
        for i in range(n_q[b]):
            p = lens[b] - n_q[b] + i
            r = cuq[b] + i
            o, l = oracle.decode(cache, qc[r:r + 1], qr[r:r + 1], 0.27, bt[b:b + 1], [p + 1], 0.9, A_IN, A_OUT)
            assert np.array_equal(out[r], o[0]) and np.array_equal(lse[r], l[0])


def test_zero_query_is_mean_of_visible_rows_read_at_the_cache_state():
    # q = 0: every visible position weighs the same, so query i returns the
    # mean of rows 0..p and lse = ln(p + 1).  Rows 0..1 are the sink's bf16
    # latents and rows ctx-3..ctx-1 the ring's (the window of the whole
    # cache, not of p + 1); the rest are the dequantized codes.
    rng = np.random.default_rng(23)
    n, n_q, n_sink, n_recent = 12, 6, 2, 3
    cache, z, _, bt = build(rng, [n], n_sink=n_sink, n_recent=n_recent)
    qc = np.zeros((n_q, 2, 32), np.uint16)
    qr = np.zeros((n_q, 2, 4), np.uint16)
    out, lse = oracle.extend(cache, qc, qr, 0.5, bt, [n], [0, n_q], 1.0, A_IN, A_OUT)
    page = cache.page
    rows = []
    for t in range(n):
        if t < n_sink or t >= n - n_recent:
            rows.append(oracle.bf16_bits_to_f64(oracle.f32_to_bf16_bits(z[t])))
        else:
            pg, sl = bt[0, t // page], t % page
            rows.append(oracle.dequant(cache.codes[pg, sl][None], cache.meta[pg, sl][None], 1.0, A_IN, A_OUT,
                                       cache.group)[0])
    rows = np.array(rows)
    for i in range(n_q):
        p = n - n_q + i
        assert np.allclose(out[i], rows[:p + 1].mean(axis=0)[None, :], atol=1e-13)
        assert np.allclose(lse[i], math.log(p + 1), atol=1e-13)
    # The window follows the cache: position 7 (query 1) is read from codes,
    # which differ from its bf16 latent.
    assert np.abs(rows[7] - oracle.bf16_bits_to_f64(oracle.f32_to_bf16_bits(z[7]))).max() > 1e-3


def test_mpmath_bruteforce_causal_tiny_cache():
    rng = np.random.default_rng(24)
    mpmath.mp.dps = 50
    d_c, d_r, group, n, n_q = 16, 2, 4, 7, 3
    cache = oracle.new_cache(2, d_c, d_r, 4, group)
    z = rng.standard_normal((n, d_c)).astype(np.float32)
    kr = rand_bf16(rng, (n, d_r))
    oracle.quantize_append(cache, 0.93, kr, [0, n], [0], [[1, 0]], latent_rot_f32=z)
    qc = rand_bf16(rng, (n_q, 2, d_c))
    qr = rand_bf16(rng, (n_q, 2, d_r))
    g, a, b, sm = 1.15, A_IN, A_OUT, 0.37
    out, lse = oracle.extend(cache, qc, qr, sm, [[1, 0]], [n], [0, n_q], g, a, b)
    A, B, G, SM = (mpmath.mpf(float(np.float32(x))) for x in (a, b, g, sm))
    lv = [-B, -A, A, B]
    for i in range(n_q):
        p = n - n_q + i
        for h in range(2):
            q = [mpmath.mpf(float(x)) for x in oracle.bf16_bits_to_f64(qc[i, h])]
            r = [mpmath.mpf(float(x)) for x in oracle.bf16_bits_to_f64(qr[i, h])]
            rows, scores = [], []
            for t in range(p + 1):
                pg, sl = [1, 0][t // 4], t % 4
                w = int(cache.codes[pg, sl, 0])
                mu = [mpmath.mpf(float(x)) for x in cache.meta[pg, sl, :4]]
                sc = [mpmath.mpf(float(x)) for x in cache.meta[pg, sl, 4:]]
                row = [mu[j // group] + sc[j // group] * G * lv[(w >> (2 * j)) & 3] for j in range(d_c)]
                k = [mpmath.mpf(float(x)) for x in oracle.bf16_bits_to_f64(cache.rope[pg, sl])]
                rows.append(row)
                scores.append(SM * (sum(q[j] * row[j] for j in range(d_c)) + sum(r[j] * k[j] for j in range(d_r))))
            den = sum(mpmath.exp(s) for s in scores)
            for j in range(d_c):
                o = sum(mpmath.exp(scores[t]) * rows[t][j] for t in range(p + 1)) / den
                assert abs(float(o) - out[i, h, j]) < 1e-13
            assert abs(float(mpmath.log(den)) - lse[i, h]) < 1e-13


def test_requests_without_queries_are_skipped():
    rng = np.random.default_rng(25)
    lens = [5, 8, 3]
    cache, _, _, bt = build(rng, lens)
    qc = rand_bf16(rng, (4, 2, 32))
    qr = rand_bf16(rng, (4, 2, 4))
    out, lse = oracle.extend(cache, qc, qr, 0.2, bt, lens, [0, 0, 4, 4], 1.0, A_IN, A_OUT)
    o, l = oracle.extend(cache, qc, qr, 0.2, bt[1:2], lens[1:2], [0, 4], 1.0, A_IN, A_OUT)
    assert np.array_equal(out, o) and np.array_equal(lse, l)


def test_repeated_page_is_one_copy_merged_in_closed_form():
    """A block table that names one page for every position makes the context
    that page repeated.  Softmax over R copies plus a t-token prefix has a
    closed form (the LSE gains log R for the copies, then a two-term log-sum-
    exp merge with the prefix); the oracle must reach it exactly, for every
    query position including the ones on a page boundary."""
    rng = np.random.default_rng(31)
    page = 4
    cache, _, _, bt = build(rng, [page], page=page)
    n_q, reps = 6, 5
    ctx = reps * page + 2
    big_bt = np.zeros((1, (ctx + page - 1) // page), np.int32) + bt[0, 0]
    qc, qr = rand_bf16(rng, (n_q, 2, 32)), rand_bf16(rng, (n_q, 2, 4))
    cu = np.array([0, n_q], np.int32)
    out, lse = oracle.extend(cache, qc, qr, 0.3, big_bt, [ctx], cu, 1.1, A_IN, A_OUT)
    for i in range(n_q):
        n = ctx - n_q + i + 1
        r, t = divmod(n, page)
        one = np.array([0, 1], np.int32)
        o_p, l_p = oracle.extend(cache, qc[i:i + 1], qr[i:i + 1], 0.3, bt, [page], one, 1.1, A_IN, A_OUT)
        want_l, want_o = l_p[0] + math.log(r), o_p[0]
        if t:
            o_t, l_t = oracle.extend(cache, qc[i:i + 1], qr[i:i + 1], 0.3, bt, [t], one, 1.1, A_IN, A_OUT)
            merged = np.logaddexp(want_l, l_t[0])
            want_o = np.exp(want_l - merged)[:, None] * want_o + np.exp(l_t[0] - merged)[:, None] * o_t[0]
            want_l = merged
        np.testing.assert_allclose(lse[i], want_l, rtol=0, atol=1e-12)
        np.testing.assert_allclose(out[i], want_o, rtol=0, atol=1e-12)
