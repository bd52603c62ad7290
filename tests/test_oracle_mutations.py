"""Plant plausible mistakes in the oracle (on the CPU) and check a pin catches each.

Each mutation swaps one oracle function for a subtly wrong variant (transposed
operand, wrong reduction order, wrong divisor, strict comparison, wrong bit
order, swapped levels, dropped term, missing scale, an extend that misses its
own position, counts queries from position 0, or reads the sink / recent
window at the query instead of the cache).  The pins must fail.
"""

import numpy as np
import pytest

import oracle
import oracle.rlq_oracle as ro
import test_oracle_attention as ta
import test_oracle_encode as te
import test_oracle_extend as tx


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(ro, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def rotate_transposed(latent_bf16, rotation_bf16):
    return (ro.bf16_bits_to_f64(latent_bf16) @ ro.bf16_bits_to_f64(rotation_bf16)).astype(np.float32)


def tree_sum_sequential(v):
    v = np.asarray(v, dtype=np.float32)
    acc = np.zeros(v.shape[:-1], np.float32)
    for i in range(v.shape[-1]):
        acc = (acc + v[..., i]).astype(np.float32)
    return acc


def group_stats_sample_std(z, group=ro.GROUP):
    mu, s, d = ORIG["group_stats"](z, group)
    return mu, (s * np.float32(np.sqrt(group / (group - 1)))).astype(np.float32), d


def assign_codes_strict(d, s, tau, group=ro.GROUP):
    d = np.asarray(d, dtype=np.float32)
    n_groups = d.shape[-1] // group
    dg = d.reshape(d.shape[:-1] + (n_groups, group))
    t = (np.float32(tau) * np.asarray(s, np.float32))[..., None]
    c = (dg > -t).astype(np.uint8) + (dg > 0).astype(np.uint8) + (dg > t).astype(np.uint8)
    return c.reshape(d.shape)


def pack_msb_first(codes):
    c = np.asarray(codes, dtype=np.uint32)
    cw = c.reshape(c.shape[:-1] + (c.shape[-1] // 16, 16))
    w = np.zeros(cw.shape[:-1], np.uint32)
    for j in range(16):
        w |= (cw[..., j] & 3) << np.uint32(30 - 2 * j)
    return w


def dequant_swapped_levels(words, meta, gain, level_inner, level_outer, group=ro.GROUP):
    return ORIG["dequant"](words, meta, gain, level_outer, level_inner, group)


def attend_without_rope(q_c, q_r, c_hat, k_r, sm_scale):
    return ORIG["attend"](q_c, np.zeros_like(np.asarray(q_r, np.float64)), c_hat, k_r, sm_scale)


def attend_without_scale(q_c, q_r, c_hat, k_r, sm_scale):
    return ORIG["attend"](q_c, q_r, c_hat, k_r, 1.0)


def _extend_variant(limit, window_at_query=False):
    """An extend with a planted mistake: query i attends to positions
    [0, limit(ctx, n_q, i)); with window_at_query the sink / recent rows are
    read as if the cache held only those positions."""
    def extend(cache, q_c_bf16, q_r_bf16, sm_scale, block_table, ctx_lens, cu_seqlens_q, gain, level_inner,
               level_outer):
        qc, qr = ro.bf16_bits_to_f64(q_c_bf16), ro.bf16_bits_to_f64(q_r_bf16)
        out = np.zeros(qc.shape)
        lse = np.full(qc.shape[:2], -np.inf)
        cu = np.asarray(cu_seqlens_q)
        for b in range(len(cu) - 1):
            n, n_q = int(ctx_lens[b]), int(cu[b + 1] - cu[b])
            for i in range(n_q):
                lim = limit(n, n_q, i)
                src = lim if window_at_query else n
                c_hat, k_r = ro.gather_request(cache, np.asarray(block_table)[b], src, gain, level_inner, level_outer)
                c_hat = ro._protected_rows(cache, b, src, c_hat)
                r = int(cu[b]) + i
                out[r], lse[r] = ro.attend(qc[r], qr[r], c_hat[:lim], k_r[:lim], sm_scale)
        return out, lse
    return extend


extend_excludes_own_position = _extend_variant(lambda n, n_q, i: n - n_q + i)
extend_queries_from_position_0 = _extend_variant(lambda n, n_q, i: i + 1)
extend_window_at_query = _extend_variant(lambda n, n_q, i: n - n_q + i + 1, window_at_query=True)
for _f, _n in ((extend_excludes_own_position, "extend_excludes_own_position"),
               (extend_queries_from_position_0, "extend_queries_from_position_0"),
               (extend_window_at_query, "extend_window_at_query")):
    _f.__name__ = _n

ORIG = {n: getattr(ro, n) for n in ("group_stats", "dequant", "attend")}

MUTATIONS = [
    ("rotate", rotate_transposed, [te.test_rotate_matches_exact_rational_sum]),
    ("tree_sum_f32", tree_sum_sequential, [te.test_tree_sum_order_is_not_sequential,
                                           te.test_tree_sum_matches_recursive_emulation]),
    ("group_stats", group_stats_sample_std, [te.test_group_stats_hand_computed,
                                             te.test_group_stats_match_bruteforce]),
    ("assign_codes", assign_codes_strict, [te.test_codes_ties_and_antisymmetry,
                                           te.test_codes_are_nearest_level_at_the_midpoint_threshold]),
    ("pack_codes", pack_msb_first, [te.test_pack_hand_built_words,
                                    te.test_pack_exhaustive_halfword_round_trip]),
    ("dequant", dequant_swapped_levels, [ta.test_dequant_formula_and_degenerate_cases,
                                         ta.test_mpmath_bruteforce_tiny_cache]),
    ("attend", attend_without_rope, [ta.test_mpmath_bruteforce_tiny_cache,
                                     ta.test_all_protected_equals_library_attention]),
    ("attend", attend_without_scale, [ta.test_two_tokens_follow_the_logistic,
                                      ta.test_mpmath_bruteforce_tiny_cache]),
    ("extend", extend_excludes_own_position, [tx.test_single_query_equals_decode,
                                              tx.test_unprotected_query_i_equals_decode_over_its_prefix,
                                              tx.test_zero_query_is_mean_of_visible_rows_read_at_the_cache_state,
                                              tx.test_mpmath_bruteforce_causal_tiny_cache]),
    ("extend", extend_queries_from_position_0, [tx.test_single_query_equals_decode,
                                                tx.test_unprotected_query_i_equals_decode_over_its_prefix,
                                                tx.test_zero_query_is_mean_of_visible_rows_read_at_the_cache_state]),
    # (one query per request cannot tell these windows apart: its position is the last)
    ("extend", extend_window_at_query, [tx.test_zero_query_is_mean_of_visible_rows_read_at_the_cache_state]),
]


@pytest.mark.parametrize("name,fn,pins", MUTATIONS, ids=[f"{m[0]}-{m[1].__name__}" for m in MUTATIONS])
def test_pins_catch_planted_mistake(monkeypatch, name, fn, pins):
    _patch(monkeypatch, name, fn)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()
