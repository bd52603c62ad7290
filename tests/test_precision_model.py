"""Host model of the decode kernels' staging precision (tests/kernel_rounding.py).

Why the score needs a correction beyond fp16 c_hat, reproduced on the CPU:
the kernels stage c_hat = mu + s g L (RoLaQ §3.2) as fp16 for both MFMA
products.  When two tokens share the softmax, the output moves with their
score difference, and each score carries the rounding of 512 fp16 values.
These tests show, on the same seeded inputs the GPU tests use, that fp16
alone misses the 2e-3 bar and that the bf8 residual correction of the score
(what the kernels now run) brings the error well inside it.  They measure the
model only; the GPU parity tests measure the kernels.
"""

import numpy as np
import pytest

import kernel_rounding as kr
import oracle
from decode_attention_rlq_amd import workloads

OUT_TOL = 2e-3
LSE_TOL = 2e-3


def test_round_to_format_pins():
    # OCP e4m3: largest finite 448, 3 mantissa bits, ties to even.
    assert kr.e4m3(448.0) == 448.0 and kr.e4m3(1e6) == 448.0 and kr.e4m3(-1e6) == -448.0
    assert kr.e4m3(1.0625) == 1.0 and kr.e4m3(1.1875) == 1.25 and kr.e4m3(1.2) == 1.25
    assert kr.e4m3(2.0 ** -9) == 2.0 ** -9 and kr.e4m3(2.0 ** -10) == 0.0  # smallest subnormal, tie to 0
    # OCP e5m2: 2 mantissa bits, smallest subnormal 2^-16.
    assert kr.e5m2(1.125) == 1.0 and kr.e5m2(1.375) == 1.5 and kr.e5m2(57344.0) == 57344.0
    assert kr.e5m2(2.0 ** -16) == 2.0 ** -16 and kr.e5m2(3 * 2.0 ** -17) == 2.0 ** -15
    # Every representable e5m2 value in [1, 2) is a fixed point, nothing else is.
    grid = 1.0 + np.arange(4) / 4
    assert np.array_equal(kr.e5m2(grid), grid)
    x = np.linspace(1.0, 2.0, 1001)[1:-1]
    on = np.isin(x, grid)
    assert np.all(kr.e5m2(x[~on]) != x[~on])


def request_terms(prob, b):
    lo, hi = int(prob.cu_seqlens[b]), int(prob.cu_seqlens[b + 1])
    z = oracle.rotate(prob.latent_bits[lo:hi], prob.rotation_bits)
    words, meta = oracle.encode_tokens(z, prob.tau)
    c_hat = oracle.dequant(words, meta, prob.gain, prob.level_inner, prob.level_outer)
    k_r = prob.k_rope_bits[lo:hi]
    ref_o, ref_l = oracle.attend(oracle.bf16_bits_to_f64(prob.q_c_bits[b]), oracle.bf16_bits_to_f64(prob.q_r_bits[b]),
                                 c_hat, oracle.bf16_bits_to_f64(k_r), prob.sm_scale)
    model = {}
    for corr in (False, True):
        o, l = kr.model_decode(words, meta, k_r, prob.q_c_bits[b], prob.q_r_bits[b], prob.sm_scale, prob.gain,
                               prob.level_inner, prob.level_outer, corr)
        model[corr] = (float(kr.row_rel_err(o, ref_o).max()), float(np.abs(l - ref_l).max()))
    return model


def test_near_tie_row_of_many_requests_h16():
    """The 300-request, 16-head decode case: request 77, head 8 (two tokens
    hold 0.39 and 0.33 of the softmax) measured 2.2e-3 on the GPU with fp16
    c_hat scores.  The model gives the same, and the corrected score removes
    it."""
    prob = workloads.make_problem("v2lite_32k", ctx_lens=[1 + 7 * b for b in range(300)])
    m = request_terms(prob, 77)
    print(f"request 77: fp16 {m[False]}, corrected {m[True]}")
    assert m[False][0] > OUT_TOL
    assert m[True][0] < 0.3 * OUT_TOL and m[True][1] < 0.2 * LSE_TOL


@pytest.mark.parametrize("b", [0, 2])
def test_peaked_scores_need_the_correction(b):
    """The GPU tests' peaked-score input (queries x3, 128 heads): fp16 c_hat
    alone misses both bars, the corrected score meets them with margin."""
    prob = workloads.make_problem("v2lite_32k", ctx_lens=[700, 2100, 33, 5000], heads=128, seed=77)
    q = oracle.bf16_bits_to_f64(prob.q_c_bits) * 3.0
    prob.q_c_bits = workloads.to_bf16_bits(q.astype(np.float32))
    m = request_terms(prob, b)
    print(f"request {b}: fp16 {m[False]}, corrected {m[True]}")
    assert m[False][0] > OUT_TOL and m[False][1] > LSE_TOL
    assert m[True][0] < 0.4 * OUT_TOL and m[True][1] < 0.3 * LSE_TOL
