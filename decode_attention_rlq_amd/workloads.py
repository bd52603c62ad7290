"""Seeded synthetic inputs for the 2-bit MLA cache path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no rotation, statistics, thresholds, packing or
attention).  Both the CPU oracle checks and the GPU path consume what it
returns, so neither side can influence the other's inputs.

Workload shapes follow the pages' serving setting for DeepSeek-V2-Lite
(content latent 512, RoPE key 64, group 128; 4 concurrent requests at 256K
input tokens) and these per-configuration recipes:

  tiny            1 request x 256 tokens, 16 heads, tau 0.9816, gain 1.0
  v2lite_32k      4 x 32,768 tokens, 16 heads, paged (64-token pages)
  v2lite_256k     4 x 262,144 tokens, 16 heads (the headline decode shape)
  append_bulk     4 x 65,536 new tokens with 1% Student-t (nu=3) coordinates
  ragged_protect  32 requests, 128 heads, log-uniform lengths in [1024, 65536],
                  4 sink + 64 recent BF16-protected tokens

Draw order (numpy PCG64, seed = 1000 + config index unless given):
  1 per-channel sigma ~ lognormal(0, 0.5) over the 512 content channels
  2 Haar rotation: QR of a 512x512 standard normal matrix, sign-fixed
  3 six RoPE outlier channels (scaled x8)
  4 tau ~ U(0.85, 1.10), gain ~ U(1.0, 1.2) (fixed values for 'tiny')
  5 context lengths (ragged configuration only)
  6 latents, request by request, in chunks
  7 RoPE keys
  8 absorbed queries q_c, q_R
  9 page order (a permutation of the page pool)
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

D_C = 512
D_R = 64
PAGE = 64
SM_SCALE = float(np.float32(1.0 / np.sqrt(192.0)))

CONFIG_NAMES = ("tiny", "v2lite_32k", "v2lite_256k", "append_bulk", "ragged_protect")


def to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 bit patterns (nearest, ties to even)."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Problem:
    """One synthetic layer: inputs for quantize-append and for decode."""
    name: str
    batch: int
    heads: int
    ctx_lens: np.ndarray          # int32 [B] tokens cached per request after the append
    tau: float
    gain: float
    sigma: np.ndarray             # fp32 [d_c]
    rotation_bits: np.ndarray     # uint16 [d_c][d_c] bf16, z = R c
    rotation_f64: np.ndarray      # the unrounded Haar matrix (for diagnostics)
    latent_bits: np.ndarray       # uint16 [N][d_c] bf16, requests concatenated
    k_rope_bits: np.ndarray       # uint16 [N][d_r] bf16
    q_c_bits: np.ndarray          # uint16 [B][H][d_c] bf16
    q_r_bits: np.ndarray          # uint16 [B][H][d_r] bf16
    cu_seqlens: np.ndarray        # int32 [B+1]
    start_pos: np.ndarray         # int32 [B]
    block_table: np.ndarray       # int32 [B][max_pages]
    num_pages: int
    n_sink: int = 0
    n_recent: int = 0
    sm_scale: float = SM_SCALE
    level_inner: float = 0.4528
    level_outer: float = 1.510
    page: int = PAGE
    outlier_channels: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))

    @property
    def n_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def d_c(self) -> int:
        return int(self.latent_bits.shape[1])

    @property
    def d_r(self) -> int:
        return int(self.k_rope_bits.shape[1])


def haar_rotation(rng: np.random.Generator, d: int) -> np.ndarray:
    g = rng.standard_normal((d, d))
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))[None, :]


def _latents(rng, sigma, n, heavy_p, chunk=1 << 16):
    d = sigma.shape[0]
    out = np.empty((n, d), np.uint16)
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        x = rng.standard_normal((hi - lo, d), dtype=np.float32)
        if heavy_p > 0:
            mask = rng.random((hi - lo, d), dtype=np.float32) < heavy_p
            k = int(mask.sum())
            if k:
                x[mask] = rng.standard_t(3.0, size=k).astype(np.float32)
        out[lo:hi] = to_bf16_bits(x * sigma[None, :])
    return out


def make_problem(name: str = "tiny", *, seed: int | None = None, batch: int | None = None,
                 heads: int | None = None, ctx: int | None = None,
                 ctx_lens=None, tau: float | None = None, gain: float | None = None,
                 n_sink: int | None = None, n_recent: int | None = None,
                 heavy_p: float | None = None, d_c: int = D_C, d_r: int = D_R,
                 page: int = PAGE, extra_pages: int = 0) -> Problem:
    """Build a named workload; keyword overrides shrink it for tests.

    All new tokens of a request are appended from position 0, so after the
    append ctx_lens[b] tokens are cached for request b.
    """
    idx = CONFIG_NAMES.index(name)
    rng = np.random.Generator(np.random.PCG64(1000 + idx if seed is None else seed))
    defaults = {
        "tiny": dict(batch=1, heads=16, ctx=256, n_sink=0, n_recent=0, heavy_p=0.0),
        "v2lite_32k": dict(batch=4, heads=16, ctx=32768, n_sink=0, n_recent=0, heavy_p=0.0),
        "v2lite_256k": dict(batch=4, heads=16, ctx=262144, n_sink=0, n_recent=0, heavy_p=0.0),
        "append_bulk": dict(batch=4, heads=16, ctx=65536, n_sink=0, n_recent=0, heavy_p=0.01),
        "ragged_protect": dict(batch=32, heads=128, ctx=None, n_sink=4, n_recent=64, heavy_p=0.0),
    }[name]
    batch = defaults["batch"] if batch is None else batch
    heads = defaults["heads"] if heads is None else heads
    n_sink = defaults["n_sink"] if n_sink is None else n_sink
    n_recent = defaults["n_recent"] if n_recent is None else n_recent
    heavy_p = defaults["heavy_p"] if heavy_p is None else heavy_p

    sigma = rng.lognormal(0.0, 0.5, size=d_c).astype(np.float32)
    rot = haar_rotation(rng, d_c)
    outliers = rng.choice(d_r, size=min(6, d_r), replace=False)
    if name == "tiny":
        t_draw, g_draw = 0.9816, 1.0
    else:
        t_draw = float(rng.uniform(0.85, 1.10))
        g_draw = float(rng.uniform(1.0, 1.2))
    tau = t_draw if tau is None else tau
    gain = g_draw if gain is None else gain

    if ctx_lens is not None:
        lens = np.asarray(ctx_lens, dtype=np.int64)
        batch = len(lens)
    elif name == "ragged_protect" and ctx is None:
        lens = np.floor(np.exp(rng.uniform(np.log(1024), np.log(65536), size=batch))).astype(np.int64)
    else:
        c = defaults["ctx"] if ctx is None else ctx
        lens = np.full(batch, c, dtype=np.int64)

    n_total = int(lens.sum())
    latent = _latents(rng, sigma, n_total, heavy_p)
    kr = rng.standard_normal((n_total, d_r), dtype=np.float32)
    kr[:, outliers] *= 8.0
    k_rope = to_bf16_bits(kr)
    q_c = to_bf16_bits(rng.standard_normal((batch, heads, d_c), dtype=np.float32))
    q_r = to_bf16_bits(rng.standard_normal((batch, heads, d_r), dtype=np.float32))

    pages_per = [(int(n) + page - 1) // page for n in lens]
    max_pages = max(1, max(pages_per) if pages_per else 1)
    num_pages = sum(pages_per) + extra_pages
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.zeros((batch, max_pages), np.int32)
    off = 0
    for b, npg in enumerate(pages_per):
        bt[b, :npg] = perm[off:off + npg]
        off += npg
    cu = np.zeros(batch + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    return Problem(name=name, batch=batch, heads=heads, ctx_lens=lens.astype(np.int32),
                   tau=float(tau), gain=float(gain), sigma=sigma,
                   rotation_bits=to_bf16_bits(rot.astype(np.float32)), rotation_f64=rot,
                   latent_bits=latent, k_rope_bits=k_rope, q_c_bits=q_c, q_r_bits=q_r,
                   cu_seqlens=cu, start_pos=np.zeros(batch, np.int32), block_table=bt,
                   num_pages=max(num_pages, 1), n_sink=n_sink, n_recent=n_recent,
                   page=page, outlier_channels=np.asarray(outliers))


def signed_permutation(rng: np.random.Generator, d: int) -> np.ndarray:
    """A random signed permutation matrix (every product is exact)."""
    p = np.zeros((d, d), np.float32)
    idx = rng.permutation(d)
    p[np.arange(d), idx] = rng.choice(np.array([-1.0, 1.0], np.float32), size=d)
    return p
