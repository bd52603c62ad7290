"""CPU oracle for RoLaQ-style 2-bit MLA latent caching.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  The product path (the
HIP library and its Python binding) never calls it and shares no code with it.

What it computes, and where that is stated
------------------------------------------
Sources are the pages on the method; each is cited by title and section:

* [RoLaQ] "RoLaQ: Joint Rotation and Range Calibration for 2-Bit KV Caches in
  Multi-Head Latent Attention" (section summary page, arXiv 2610.20686v1).
* [Figs] the figure-caption page of the same paper.
* [Store] the notebook "What does a 2-bit KV cache actually store?" (storage
  accounting for the paper's Appendix A.3 defaults).

Write side (per token, per layer):
  1. rotate the 512-d content latent by the fixed shared rotation
     ([RoLaQ] §3.3: rotated latents are stored as 2-bit codes; rotation,
     thresholds and gains are fixed while serving);
  2. standardize each 128-coordinate group with two fp32 statistics
     ([RoLaQ] §A.3; [Store]: group 128, two FP32 statistics per group);
  3. assign each standardized coordinate to one of four levels with the
     per-layer threshold tau ([RoLaQ] §3.2, §C.3: Lloyd-Max initial threshold);
  4. pack the 2-bit codes (128 B per token: [Store], [RoLaQ] §A.3);
  5. keep the 64-d RoPE key in BF16 ([RoLaQ] §2.1, §4.1);
  6. optionally keep sink / recent tokens' content in BF16 ([RoLaQ] §4.1,
     §5.4, §A.3: protected tokens also store BF16 content).
Read side: absorbed-MLA decode attention; the content latent serves as key and
value, read-side rotation is folded into the absorbed query ([RoLaQ] §2.1,
§3.3; [Figs] Fig. 1a, Fig. 3a).  Reconstruction: group mean + scale * gain *
level ([RoLaQ] §3.2: the gain scales reconstruction around the group mean).

Readings taken where the pages are silent:
  * scale statistic = population standard deviation of the centred group,
    two-pass, divided by the group size;
  * fixed fp32 reduction order: the adjacent-pair binary tree;
  * threshold rule compares the centred value against +-fl32(tau * s), with
    ">=" at all three cut points; code order 0:-b 1:-a 2:+a 3:+b;
  * fixed Lloyd-Max levels a, b (they do not move with tau);
  * 16 codes per little-endian uint32 word, code j at bits 2j..2j+1;
  * metadata per token = [mu_0..mu_{G-1}, s_0..s_{G-1}] in fp32;
  * protected tokens store bf16(rotated latent), decode reads them instead of
    the codes; the RoPE key always comes from the rope pool.

Pins (tests/test_oracle_*.py) and which functions they cover:
  lloyd_max_gaussian    -> Max's published 4-level Gaussian table, the centroid
                           and midpoint conditions, a direct MSE minimisation.
  quantizer_response /
  coupled_gain          -> [RoLaQ] §B.3 "approximately 0.88", Monte Carlo.
  bytes_per_token       -> [Store] / [RoLaQ] §A.3: 288 B, 144 B, 1152 B, 4.000x.
  rotate                -> exact rational brute force on small inputs, signed
                           permutations exact.
  tree_sum_f32 /
  group_stats           -> hand-computable groups, sign and power-of-two
                           symmetries, exact rational brute force.
  assign_codes          -> nearest-level rule at tau=(a+b)/2, antisymmetry,
                           ties, constant groups.
  pack_codes            -> exhaustive 2^16 round trip, hand-built words.
  quantize_append       -> composition of the above on a hand-checked paged
                           layout, protection slots.
  dequant               -> s = 0 / g = 0 reduce to the mean; exact rationals.
  decode                -> T=1, q=0, T=2 closed forms, permutation invariance,
                           mpmath brute force, library softmax attention in the
                           all-protected case.
  extend                -> one query equals decode; without protection query i
                           equals decode over its first p+1 positions; q=0
                           gives the mean of the visible rows (protected rows
                           substituted as the cache holds them) and lse
                           ln(p+1); mpmath brute force of a causal tiny case.
  lse_merge             -> merge of disjoint ranges equals the whole.
No function is "parity unpinned".
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# Dimensions fixed for DeepSeek-V2-Lite-shaped MLA ([Store]: d=512, d_r=64,
# group 128; [RoLaQ] §A.3).  Every function below also accepts other sizes.
D_C = 512
D_R = 64
GROUP = 128
PAGE = 64
CODES_PER_WORD = 16


# ---------------------------------------------------------------------------
# bf16 helpers (the oracle's own; nothing shared with the HIP path)
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns uint16.

    The 16 dropped mantissa bits decide the rounding: above half goes up,
    below half goes down, exactly half goes to the even kept pattern.
    Non-finite inputs are outside the method's domain.
    """
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    upper = (u >> np.uint32(16)).astype(np.uint64)
    lower = (u & np.uint32(0xFFFF)).astype(np.uint64)
    round_up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    return (upper + round_up.astype(np.uint64)).astype(np.uint16)


# ---------------------------------------------------------------------------
# Quantizer constants ([RoLaQ] §3.2, §B.3, §C.3; [Figs] Fig. 8)
# ---------------------------------------------------------------------------

def _phi(x: float) -> float:
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _Phi(x: float) -> float:
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def lloyd_max_gaussian(iters: int = 10000, tol: float = 1e-15):
    """Four-level Lloyd-Max quantizer for a unit Gaussian.

    The pages name the "Lloyd-Max threshold" as the initial threshold
    ([RoLaQ] §C.3, [Figs] Fig. 8) without printing it.  By symmetry the
    quantizer has cut points {-tau, 0, tau} and levels {-b, -a, a, b}.  Lloyd's
    two conditions are alternated until they hold together:
      centroid: a = E[x | 0 < x < tau],  b = E[x | x > tau];
      midpoint: tau = (a + b) / 2.
    Returns (tau, a, b, mse).
    """
    tau = 1.0
    a = b = 0.0
    for _ in range(iters):
        a = (_phi(0.0) - _phi(tau)) / (_Phi(tau) - 0.5)
        b = _phi(tau) / (1.0 - _Phi(tau))
        new_tau = 0.5 * (a + b)
        if abs(new_tau - tau) < tol:
            tau = new_tau
            break
        tau = new_tau
    a = (_phi(0.0) - _phi(tau)) / (_Phi(tau) - 0.5)
    b = _phi(tau) / (1.0 - _Phi(tau))
    mse = quantizer_mse(tau, a, b)
    return tau, a, b, mse


def quantizer_mse(tau: float, a: float, b: float, gain: float = 1.0) -> float:
    """E[(x - g Q(x))^2] for x ~ N(0,1) and the symmetric four-level Q.

    Integrates each cell in closed form:  E[x^2] = 1,
    E[x Q] = 2 (a (phi(0) - phi(tau)) + b phi(tau)),
    E[Q^2] = 2 (a^2 (Phi(tau) - 1/2) + b^2 (1 - Phi(tau))).
    """
    exq = quantizer_response(tau, a, b)
    eq2 = 2.0 * (a * a * (_Phi(tau) - 0.5) + b * b * (1.0 - _Phi(tau)))
    return 1.0 - 2.0 * gain * exq + gain * gain * eq2


def quantizer_response(tau: float, a: float, b: float) -> float:
    """Response E[x Q(x)] / E[x^2] of the four-level quantizer at unit gain.

    For x ~ N(0,1): E[x Q] = 2 (a phi(0) + (b - a) phi(tau)).  [RoLaQ] §B.3
    states that at the official threshold the MSE-optimal response is about
    0.88; the coupled gain of §3.2 scales it back to unit response.
    """
    return 2.0 * (a * _phi(0.0) + (b - a) * _phi(tau))


def coupled_gain(tau: float, a: float, b: float) -> float:
    """Gain linked to tau so that the centred signal has unit response.

    Reading of [RoLaQ] §3.2 / §B.3 (kappa = g * response = 1); the pages print
    no formula.  g(tau) = 1 / response(tau).
    """
    return 1.0 / quantizer_response(tau, a, b)


# ---------------------------------------------------------------------------
# Storage accounting ([Store]; [RoLaQ] §A.3)
# ---------------------------------------------------------------------------

def bytes_per_token(d_c: int = D_C, d_r: int = D_R, bits: int = 2,
                    group: int = GROUP, stats_per_group: int = 2,
                    stat_bytes: int = 4, rope_bytes: int = 2) -> float:
    """Bytes per unprotected token per layer: codes + group stats + BF16 RoPE."""
    codes = d_c * bits / 8
    meta = (d_c / group) * stats_per_group * stat_bytes
    rope = d_r * rope_bytes
    return codes + meta + rope


def bf16_bytes_per_token(d_c: int = D_C, d_r: int = D_R) -> float:
    """Bytes per token per layer of a BF16 MLA cache (content + RoPE key)."""
    return (d_c + d_r) * 2


# ---------------------------------------------------------------------------
# Write side
# ---------------------------------------------------------------------------

def rotate(latent_bf16: np.ndarray, rotation_bf16: np.ndarray) -> np.ndarray:
    """z = R c for each token, returned in fp32 ([RoLaQ] §3.3).

    c and R are the bf16 values actually passed (widened exactly); the sum is
    taken in fp64 and rounded once to fp32.  R is row-major [out][in].
    """
    c = bf16_bits_to_f64(latent_bf16)
    r = bf16_bits_to_f64(rotation_bf16)
    return (c @ r.T).astype(np.float32)


def tree_sum_f32(v: np.ndarray) -> np.ndarray:
    """fp32 sum over the last axis in the adjacent-pair binary tree order.

    S(v[a:b]) = S(v[a:m]) + S(v[m:b]) with m the midpoint, i.e. level by
    level v <- v[0::2] + v[1::2].  The length must be a power of two.
    """
    v = np.asarray(v, dtype=np.float32)
    n = v.shape[-1]
    if n & (n - 1):
        raise ValueError("tree_sum_f32 needs a power-of-two length")
    while v.shape[-1] > 1:
        v = v[..., 0::2] + v[..., 1::2]
    return v[..., 0]


def group_stats(z: np.ndarray, group: int = GROUP):
    """Per-group mean and scale in fp32 ([RoLaQ] §3.2, §A.3).

    mu = S(z_G) / n;  d = z - mu;  s = sqrt(S(d*d) / n), with S the fp32 tree
    sum, n = group (a power of two, so the divisions are exact scalings), the
    square taken as a plain fp32 multiply and sqrt correctly rounded.
    Returns (mu, s, d) with mu, s of shape [..., n_groups] and d like z.
    """
    z = np.asarray(z, dtype=np.float32)
    n_groups = z.shape[-1] // group
    zg = z.reshape(z.shape[:-1] + (n_groups, group))
    inv = np.float32(1.0 / group)
    mu = (tree_sum_f32(zg) * inv).astype(np.float32)
    d = (zg - mu[..., None]).astype(np.float32)
    sq = (d * d).astype(np.float32)
    var = (tree_sum_f32(sq) * inv).astype(np.float32)
    s = np.sqrt(var).astype(np.float32)
    return mu, s, d.reshape(z.shape)


def assign_codes(d: np.ndarray, s: np.ndarray, tau: float,
                 group: int = GROUP) -> np.ndarray:
    """Four-level assignment of centred coordinates ([RoLaQ] §3.2).

    t = fl32(tau * s); code = [d >= -t] + [d >= 0] + [d >= t] in {0,1,2,3},
    meaning levels -b, -a, +a, +b.  Comparing d with tau*s is the standardized
    comparison d/s >= tau written without a division.
    """
    d = np.asarray(d, dtype=np.float32)
    n_groups = d.shape[-1] // group
    dg = d.reshape(d.shape[:-1] + (n_groups, group))
    t = (np.float32(tau) * np.asarray(s, dtype=np.float32))[..., None].astype(np.float32)
    code = (dg >= -t).astype(np.uint8) + (dg >= 0).astype(np.uint8) + (dg >= t).astype(np.uint8)
    return code.reshape(d.shape)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Pack 2-bit codes, 16 per uint32 word, code j of a word at bits 2j..2j+1."""
    c = np.asarray(codes, dtype=np.uint32)
    n = c.shape[-1]
    if n % CODES_PER_WORD:
        raise ValueError("code count must be a multiple of 16")
    cw = c.reshape(c.shape[:-1] + (n // CODES_PER_WORD, CODES_PER_WORD))
    words = np.zeros(cw.shape[:-1], dtype=np.uint32)
    for j in range(CODES_PER_WORD):
        words |= (cw[..., j] & np.uint32(3)) << np.uint32(2 * j)
    return words


def unpack_codes(words: np.ndarray) -> np.ndarray:
    """Inverse of pack_codes."""
    w = np.asarray(words, dtype=np.uint32)
    out = np.empty(w.shape + (CODES_PER_WORD,), dtype=np.uint8)
    for j in range(CODES_PER_WORD):
        out[..., j] = ((w >> np.uint32(2 * j)) & np.uint32(3)).astype(np.uint8)
    return out.reshape(w.shape[:-1] + (w.shape[-1] * CODES_PER_WORD,))


def encode_tokens(z: np.ndarray, tau: float, group: int = GROUP):
    """Standardize, threshold and pack rotated latents z [N][d_c] (fp32).

    Returns (words uint32 [N][d_c/16], meta fp32 [N][2*n_groups]) where meta
    is [mu_0..mu_{G-1}, s_0..s_{G-1}].
    """
    mu, s, d = group_stats(z, group)
    codes = assign_codes(d, s, tau, group)
    meta = np.concatenate([mu, s], axis=-1).astype(np.float32)
    return pack_codes(codes), meta


@dataclass
class Cache:
    """Paged 2-bit cache held as numpy arrays (layout of include/rlq.h).

    codes  uint32 [num_pages][page][d_c/16]
    meta   fp32   [num_pages][page][2*d_c/group]
    rope   uint16 [num_pages][page][d_r]        (bf16 bits)
    sink   uint16 [max_batch][n_sink][d_c]      (bf16 bits) or None
    recent uint16 [max_batch][n_recent][d_c]    (bf16 bits) or None
    """
    codes: np.ndarray
    meta: np.ndarray
    rope: np.ndarray
    sink: np.ndarray | None = None
    recent: np.ndarray | None = None
    group: int = GROUP

    @property
    def page(self) -> int:
        return self.codes.shape[1]

    @property
    def n_sink(self) -> int:
        return 0 if self.sink is None else self.sink.shape[1]

    @property
    def n_recent(self) -> int:
        return 0 if self.recent is None else self.recent.shape[1]


def new_cache(num_pages: int, d_c: int = D_C, d_r: int = D_R, page: int = PAGE,
              group: int = GROUP, max_batch: int = 0, n_sink: int = 0,
              n_recent: int = 0) -> Cache:
    return Cache(
        codes=np.zeros((num_pages, page, d_c // CODES_PER_WORD), np.uint32),
        meta=np.zeros((num_pages, page, 2 * (d_c // group)), np.float32),
        rope=np.zeros((num_pages, page, d_r), np.uint16),
        sink=np.zeros((max_batch, n_sink, d_c), np.uint16) if n_sink else None,
        recent=np.zeros((max_batch, n_recent, d_c), np.uint16) if n_recent else None,
        group=group)


def quantize_append(cache: Cache, tau: float, k_rope_bf16: np.ndarray,
                    cu_seqlens, start_pos, block_table, *,
                    latent_bf16: np.ndarray | None = None,
                    rotation_bf16: np.ndarray | None = None,
                    latent_rot_f32: np.ndarray | None = None) -> np.ndarray:
    """Append new tokens of each request to the paged cache (in place).

    Request b owns new tokens cu_seqlens[b]..cu_seqlens[b+1]-1; its i-th new
    token lands at position p = start_pos[b] + i, page block_table[b][p // page],
    slot p % page.  Every token gets codes, metadata and its BF16 RoPE key
    ([RoLaQ] §A.3 accounting).  With protection, positions p < n_sink also go
    to sink[b][p], and the last n_recent positions of the request after this
    append go to recent[b][p % n_recent] ([RoLaQ] §4.1, §A.3).
    Either latent_bf16 (+ rotation_bf16) or an already rotated latent_rot_f32
    is given.  Returns z (fp32) for inspection.
    """
    if latent_rot_f32 is not None:
        z = np.asarray(latent_rot_f32, dtype=np.float32)
    else:
        z = rotate(latent_bf16, rotation_bf16)
    words, meta = encode_tokens(z, tau, cache.group)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    sp = np.asarray(start_pos, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    page = cache.page
    for b in range(len(sp)):
        lo, hi = int(cu[b]), int(cu[b + 1])
        new_len = int(sp[b]) + (hi - lo)
        for i in range(lo, hi):
            p = int(sp[b]) + (i - lo)
            pg = int(bt[b, p // page])
            cache.codes[pg, p % page] = words[i]
            cache.meta[pg, p % page] = meta[i]
            cache.rope[pg, p % page] = k_rope_bf16[i]
            if cache.sink is not None and p < cache.n_sink:
                cache.sink[b, p] = f32_to_bf16_bits(z[i])
            if cache.recent is not None and p >= new_len - cache.n_recent:
                cache.recent[b, p % cache.n_recent] = f32_to_bf16_bits(z[i])
    return z


# ---------------------------------------------------------------------------
# Read side
# ---------------------------------------------------------------------------

def dequant(words: np.ndarray, meta: np.ndarray, gain: float, level_inner: float,
            level_outer: float, group: int = GROUP) -> np.ndarray:
    """Reconstruct c_hat = mu_G + s_G * g * L[code] in fp64 ([RoLaQ] §3.2).

    L = (-b, -a, +a, +b) indexed by the code; a, b and g enter as the fp32
    values the kernels receive.
    """
    codes = unpack_codes(words).astype(np.int64)
    a = float(np.float32(level_inner))
    b = float(np.float32(level_outer))
    g = float(np.float32(gain))
    levels = np.array([-b, -a, a, b], dtype=np.float64)
    n_groups = codes.shape[-1] // group
    meta = np.asarray(meta, dtype=np.float64)
    mu = meta[..., :n_groups]
    s = meta[..., n_groups:2 * n_groups]
    lv = levels[codes].reshape(codes.shape[:-1] + (n_groups, group))
    out = mu[..., None] + (s * g)[..., None] * lv
    return out.reshape(codes.shape)


def gather_request(cache: Cache, block_table_row, ctx_len: int, gain: float,
                   level_inner: float, level_outer: float):
    """Reconstructed content latents [T][d_c] and RoPE keys [T][d_r] (fp64).

    Position t reads sink[t] if t < n_sink, recent[t % n_recent] if
    t >= ctx_len - n_recent, and the dequantized codes otherwise; the RoPE key
    always comes from the rope pool.
    """
    page = cache.page
    t = np.arange(ctx_len)
    pages = np.asarray(block_table_row, dtype=np.int64)[t // page]
    slots = t % page
    c_hat = dequant(cache.codes[pages, slots], cache.meta[pages, slots], gain,
                    level_inner, level_outer, cache.group)
    k_r = bf16_bits_to_f64(cache.rope[pages, slots])
    return c_hat, k_r


def _protected_rows(cache: Cache, b: int, ctx_len: int, c_hat: np.ndarray) -> np.ndarray:
    c_hat = c_hat.copy()
    if cache.recent is not None and cache.n_recent > 0:
        for t in range(max(0, ctx_len - cache.n_recent), ctx_len):
            c_hat[t] = bf16_bits_to_f64(cache.recent[b, t % cache.n_recent])
    if cache.sink is not None and cache.n_sink > 0:
        for t in range(min(cache.n_sink, ctx_len)):
            c_hat[t] = bf16_bits_to_f64(cache.sink[b, t])
    return c_hat


def attend(q_c: np.ndarray, q_r: np.ndarray, c_hat: np.ndarray, k_r: np.ndarray,
           sm_scale: float):
    """Plain softmax attention over a latent cache, fp64, two passes.

    Scores s[h,t] = sm_scale (q_c[h] . c_hat[t] + q_r[h] . k_r[t]); the output
    is the softmax-weighted average of c_hat in latent space ([RoLaQ] §2.1:
    the latent serves keys and values; §3.3: rotation folded into the
    absorbed projections).  Returns (out [H][d_c], lse [H]) with lse the
    natural-log sum of exp(scores).  An empty cache gives 0 and -inf.
    """
    q_c = np.asarray(q_c, dtype=np.float64)
    q_r = np.asarray(q_r, dtype=np.float64)
    h = q_c.shape[0]
    if c_hat.shape[0] == 0:
        return np.zeros((h, q_c.shape[1])), np.full(h, -np.inf)
    scores = float(np.float32(sm_scale)) * (q_c @ c_hat.T + q_r @ k_r.T)
    m = scores.max(axis=1, keepdims=True)
    p = np.exp(scores - m)
    den = p.sum(axis=1)
    out = (p @ c_hat) / den[:, None]
    lse = m[:, 0] + np.log(den)
    return out, lse


def decode(cache: Cache, q_c_bf16: np.ndarray, q_r_bf16: np.ndarray, sm_scale: float,
           block_table, ctx_lens, gain: float, level_inner: float,
           level_outer: float, heads: slice | None = None):
    """Absorbed-MLA decode over the paged cache for every request.

    q_c_bf16 [B][H][d_c] and q_r_bf16 [B][H][d_r] are bf16 bit patterns.
    Returns (out fp64 [B][H][d_c], lse fp64 [B][H]).  `heads` optionally
    restricts the computation to a slice of heads (for sampled checks).
    """
    qc = bf16_bits_to_f64(q_c_bf16)
    qr = bf16_bits_to_f64(q_r_bf16)
    if heads is not None:
        qc, qr = qc[:, heads], qr[:, heads]
    bsz, h, d_c = qc.shape
    out = np.zeros((bsz, h, d_c))
    lse = np.full((bsz, h), -np.inf)
    bt = np.asarray(block_table)
    for b in range(bsz):
        n = int(ctx_lens[b])
        c_hat, k_r = gather_request(cache, bt[b], n, gain, level_inner, level_outer)
        c_hat = _protected_rows(cache, b, n, c_hat)
        out[b], lse[b] = attend(qc[b], qr[b], c_hat, k_r, sm_scale)
    return out, lse


def extend(cache: Cache, q_c_bf16: np.ndarray, q_r_bf16: np.ndarray, sm_scale: float,
           block_table, ctx_lens, cu_seqlens_q, gain: float, level_inner: float,
           level_outer: float):
    """Prefill / extend attention of each request's newest tokens over the cache.

    [RoLaQ] §D: the method serves prefill as well as decode from its cache;
    the attention is the decode attention of §2.1 / §3.3 with the causal
    limit of a prefill.  Reading taken: the new tokens are already appended,
    so request b holds ctx_lens[b] positions and its n_q = cu[b+1] - cu[b]
    queries are the last n_q of them; query i (row cu[b] + i of q_c [N_q][H]
    [d_c]) sits at position p = ctx_lens[b] - n_q + i and attends to positions
    0 .. p, each reconstructed exactly as decode reconstructs it with the cache
    state at ctx_lens[b] (sink rows, the recent ring of the last n_recent
    positions, codes elsewhere).
    Returns (out fp64 [N_q][H][d_c], lse fp64 [N_q][H]).
    """
    qc = bf16_bits_to_f64(q_c_bf16)
    qr = bf16_bits_to_f64(q_r_bf16)
    n_total, h, d_c = qc.shape
    out = np.zeros((n_total, h, d_c))
    lse = np.full((n_total, h), -np.inf)
    bt = np.asarray(block_table)
    cu = np.asarray(cu_seqlens_q)
    for b in range(len(cu) - 1):
        n = int(ctx_lens[b])
        n_q = int(cu[b + 1] - cu[b])
        if n_q == 0:
            continue
        c_hat, k_r = gather_request(cache, bt[b], n, gain, level_inner, level_outer)
        c_hat = _protected_rows(cache, b, n, c_hat)
        for i in range(n_q):
            p = n - n_q + i
            r = int(cu[b]) + i
            out[r], lse[r] = attend(qc[r], qr[r], c_hat[:p + 1], k_r[:p + 1], sm_scale)
    return out, lse


def attend_partial(q_c, q_r, c_hat, k_r, sm_scale):
    """(m, l, o) of one token range: running max, sum of exp(s - m), and the
    unnormalised sum of exp(s - m) * c_hat.  Used with lse_merge."""
    q_c = np.asarray(q_c, dtype=np.float64)
    q_r = np.asarray(q_r, dtype=np.float64)
    h = q_c.shape[0]
    if c_hat.shape[0] == 0:
        return np.full(h, -np.inf), np.zeros(h), np.zeros((h, q_c.shape[1]))
    s = float(np.float32(sm_scale)) * (q_c @ c_hat.T + q_r @ k_r.T)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    return m, p.sum(axis=1), p @ c_hat


def lse_merge(parts):
    """Merge (m_i, l_i, o_i) partials of disjoint token ranges.

    m = max m_i;  w_i = exp(m_i - m);  out = sum w_i o_i / sum w_i l_i;
    lse = m + ln(sum w_i l_i).  Ranges with no tokens (m_i = -inf) weigh 0.
    """
    ms = np.stack([p[0] for p in parts])
    m = ms.max(axis=0)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    num = 0.0
    den = 0.0
    for mi, li, oi in parts:
        w = np.where(np.isfinite(mi), np.exp(np.where(np.isfinite(mi), mi, 0.0) - safe_m), 0.0)
        num = num + w[:, None] * oi
        den = den + w * li
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(den[:, None] > 0, num / np.where(den > 0, den, 1.0)[:, None], 0.0)
        lse = np.where(den > 0, safe_m + np.log(np.where(den > 0, den, 1.0)), -np.inf)
    return out, lse
