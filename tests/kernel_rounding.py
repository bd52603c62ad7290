"""A host model of the decode kernels' roundings (test infrastructure).

This is not the oracle and is never a reference for parity: it reproduces, on
the CPU, the few places where the HIP decode rounds on purpose, so that the
size of the kernels' error on a given input can be explained and the effect
of a change of staging precision can be measured before any GPU run.

What it models (RoLaQ §3.2: reconstruction = group mean + scale x gain x
level, staged per (token, group) as a table of four values):
  * the per-(token, group) table t_c = fl32(mu + fl32(s g) L_c), rounded once
    to fp16 - the score and value operand c_hat16;
  * optionally the score correction: the table's residual r_c = t_c -
    fp16(t_c) rounded to OCP e5m2 (bf8), contracted with the query rounded to
    OCP e4m3 (fp8), added to the same fp32 score;
  * P = 2^(s - m + 7) (log2 units) rounded to fp16, used for the value
    product and the row sum;
  * everything else exactly (fp64): the kernels accumulate in fp32, whose
    rounding is far below the staging error modelled here.
"""

from __future__ import annotations

import numpy as np

import oracle

LN2 = float(np.log(2.0))


def round_to_format(x, man_bits: int, emin: int, max_value: float) -> np.ndarray:
    """Round to the nearest value (ties to even) of a binary floating-point
    format with `man_bits` stored mantissa bits, smallest normal exponent
    `emin` (subnormals below it) and largest finite value `max_value`
    (saturating).  OCP e5m2: (2, -14, 57344); OCP e4m3: (3, -6, 448)."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, emin)
    step = np.exp2(e - man_bits)
    r = np.round(x / step) * step
    return np.clip(r, -max_value, max_value)


def e5m2(x):
    return round_to_format(x, 2, -14, 57344.0)


def e4m3(x):
    return round_to_format(x, 3, -6, 448.0)


def fp16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def tables(meta: np.ndarray, gain: float, level_inner: float, level_outer: float):
    """fp32 tables t [n][groups][4] of mu + s g {-b, -a, +a, +b}."""
    f32 = np.float32
    a, b = f32(level_inner), f32(level_outer)
    g = meta.shape[-1] // 2
    mu = meta[:, :g].astype(f32)
    sg = (meta[:, g:].astype(f32) * f32(gain)).astype(f32)
    lv = np.array([-b, -a, a, b], dtype=np.float64)
    # One fused multiply-add: the product is exact, one rounding to fp32.
    t = (mu.astype(np.float64)[..., None] + sg.astype(np.float64)[..., None] * lv).astype(f32)
    return t.astype(np.float64)


def model_decode(words: np.ndarray, meta: np.ndarray, k_r_bits: np.ndarray, q_c_bits: np.ndarray,
                 q_r_bits: np.ndarray, sm_scale: float, gain: float, level_inner: float,
                 level_outer: float, correct: bool):
    """Decode of one request (unprotected tokens) with the kernels' staging.

    words [T][32] uint32, meta [T][8] fp32, k_r_bits [T][64] and the query
    bit patterns q_c [H][512], q_r [H][64].  Returns (out [H][512], lse [H]).
    """
    codes = oracle.unpack_codes(words).astype(np.int64)          # [T][512]
    t = tables(meta, gain, level_inner, level_outer)              # [T][4][4]
    n_tok, d = codes.shape
    grp = np.repeat(np.arange(4), d // 4)
    tab = t[:, grp, :]                                            # [T][512][4]
    exact = np.take_along_axis(tab, codes[..., None], axis=2)[..., 0]
    c16 = fp16(exact)
    qc = oracle.bf16_bits_to_f64(q_c_bits)
    qr = oracle.bf16_bits_to_f64(q_r_bits)
    kr = oracle.bf16_bits_to_f64(k_r_bits)
    s = qc @ c16.T + qr @ kr.T
    if correct:
        resid = e5m2(exact - c16)
        s = s + e4m3(qc) @ resid.T
    s = s * float(np.float32(sm_scale))
    s2 = s / LN2                                                  # log2 units
    m = s2.max(axis=1, keepdims=True)
    p = fp16(np.exp2(s2 - m + 7.0))
    den = p.sum(axis=1)
    out = (p @ c16) / den[:, None]
    lse = (m[:, 0] - 7.0 + np.log2(den)) * LN2
    return out, lse


def row_rel_err(out: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-row max_j |out - ref| / max_j |ref|."""
    num = np.abs(out - ref).max(axis=-1)
    return num / np.maximum(np.abs(ref).max(axis=-1), 1e-30)
