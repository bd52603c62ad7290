"""Host model of the many-head kernel's LDS layout and MFMA operand maps.

The kernel (decode_attention_rlq_amd/csrc/rlq_decode_wide.hip) stages the
fp16 c_hat of a 32-token tile in LDS and reads it back in three ways: the fill
writes decode8 chunks, the score reads A operands of v_mfma_f32_32x32x16_f16,
and the value product reads transposed operands with ds_read_b64_tr_b16.  The
offsets of each are written out separately in the kernel; this test models
them with labels (token, coordinate) instead of values and checks that they
agree: every K slot of every product pairs the same coordinate on both
operands, the transposed reads deliver the tokens of P's operand slots, the
output coordinate map is a bijection onto each latent half, and none of the
three access patterns has an LDS bank conflict (64 banks of 4 bytes).  The
merge kernel's output map is checked against the same coordinate map.

Lane maps used (gfx950):
  32x32x16 (f16/bf16): A lane l holds row l % 32, K slots 8 (l // 32) + e;
    B lane l holds column l % 32, the same K slots; C register r of lane l is
    row 8 (r // 4) + 4 (l // 32) + r % 4, column l % 32.
  32x32x64 f8f6f4: as above with K slots 32 (l // 32) + e, e < 32.
  ds_read_b64_tr_b16: lane l receives element l % 4 of the 8-byte reads of
    lanes 16 (l // 16) + 4 j + (l % 16) // 4, j = 0 .. 3.
"""

import numpy as np

ROW = 512 * 2 + 16  # bytes per token row (padded)


def sub_of(jj, e):
    """Code of a word in operand slot jj of decode8 parity e."""
    return 2 * e + (jj >> 2) + 4 * (jj & 3)


def out_coord(mt, r, hl):
    return 128 * (mt >> 2) + 16 * ((mt >> 1) & 1) + 2 * (mt & 1) + 32 * (2 * ((r >> 2) & 1) + hl) + 4 * (r & 3) + (
        r >> 3)


def fill_lds():
    lds = {}
    for wave in range(4):
        for lane in range(64):
            r32, hl = lane & 31, lane >> 5
            fw0 = 8 * wave + 4 * hl
            base = r32 * ROW + 32 * fw0
            for j in range(4):
                for e in range(2):
                    for jj in range(8):
                        b = base + 32 * j + 16 * e + 2 * jj
                        assert b not in lds, "two lanes write one element"
                        lds[b] = (r32, 16 * (fw0 + j) + sub_of(jj, e))
    assert len(lds) == 32 * 512
    return lds


LDS = fill_lds()


def q_coord(c, jj):
    return 16 * (c >> 1) + sub_of(jj, c & 1)


def test_query_staging_matches_chunk_order():
    for w in range(32):
        for e in range(2):
            for bb in range(2):
                for a in range(4):
                    assert q_coord(2 * w + e, 4 * bb + a) == 16 * w + 2 * e + bb + 4 * a


def test_score_k_slots_pair_the_same_coordinate():
    for h in range(2):
        seen = np.zeros(512, int)
        for kk in range(16):
            a_lab, b_lab = {}, {}
            for lane in range(64):
                r32, hl = lane & 31, lane >> 5
                off = r32 * ROW + 16 * (32 * h + hl) + 32 * kk
                for i in range(8):
                    tok, co = LDS[off + 2 * i]
                    assert tok == r32
                    a_lab[(r32, 8 * hl + i)] = co
                    b_lab[(r32, 8 * hl + i)] = q_coord(32 * h + 2 * kk + hl, i)
            for k in range(16):
                col = {a_lab[(m, k)] for m in range(32)} | {b_lab[(n, k)] for n in range(32)}
                assert len(col) == 1
                seen[col.pop()] += 1
        assert np.all(seen[256 * h:256 * h + 256] == 1) and seen.sum() == 256


def test_correction_k_slots_pair_the_same_coordinate():
    for h in range(2):
        seen = np.zeros(512, int)
        for j in range(4):
            for hl in range(2):
                w0 = 16 * h + 8 * hl + 2 * j
                a = [16 * w + sub_of(jj, e) for w in (w0, w0 + 1) for e in range(2) for jj in range(8)]
                c0 = 32 * h + 16 * hl + 4 * j
                b = [q_coord(c, jj) for c in range(c0, c0 + 4) for jj in range(8)]
                assert a == b
                for co in a:
                    seen[co] += 1
        assert np.all(seen[256 * h:256 * h + 256] == 1) and seen.sum() == 256


def p_token(lane, ks, e):
    r = 8 * ks + e
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)


def tr_src(s, h, j, ks, sec):
    hl = s >> 5
    base = (4 * hl + ((s & 15) >> 2)) * ROW + 8 * ((s >> 4) & 1) + 64 * (s & 3) + 512 * h
    return base + 16 * ks * ROW + 16 * (j & 3) + 256 * (j >> 2) + 8 * ROW * sec


def test_value_operands_and_output_map():
    for h in range(2):
        covered = set()
        for j in range(8):
            mt = 8 * h + j
            for ks in range(2):
                a_lab = {}
                for l in range(64):
                    for sec in range(2):
                        for jq in range(4):
                            s = 16 * (l // 16) + 4 * jq + (l % 16) // 4
                            a_lab[(l % 32, 8 * (l // 32) + 4 * sec + jq)] = LDS[tr_src(s, h, j, ks, sec) + 2 * (l % 4)]
                for m in range(32):
                    coords = set()
                    for k in range(16):
                        tok, co = a_lab[(m, k)]
                        assert tok == p_token(32 * (k // 8), ks, k % 8)
                        coords.add(co)
                    assert len(coords) == 1
                    r, hl = 4 * (m >> 3) + (m & 3), (m >> 2) & 1
                    assert 8 * (r >> 2) + 4 * hl + (r & 3) == m
                    assert out_coord(mt, r, hl) == coords.pop()
                    covered.add(out_coord(mt, r, hl))
        assert covered == set(range(256 * h, 256 * h + 256))


def worst_bank_multiplicity(addrs, width):
    banks = {}
    for a in addrs:
        for w in range(0, width, 4):
            banks.setdefault(((a + w) // 4) % 64, set()).add(a + w)
    return max(len(v) for v in banks.values())


def test_no_bank_conflicts():
    worst = 1
    for h in range(2):
        for kk in range(16):
            for g in range(4):  # 16-byte reads: 16 lanes per pass
                addrs = [(l & 31) * ROW + 16 * (32 * h + (l >> 5)) + 32 * kk for l in range(16 * g, 16 * g + 16)]
                worst = max(worst, worst_bank_multiplicity(addrs, 16))
        for j in range(8):
            for ks in range(2):
                for sec in range(2):
                    for g in range(2):  # 8-byte reads: 32 lanes per pass
                        addrs = [tr_src(s, h, j, ks, sec) for s in range(32 * g, 32 * g + 32)]
                        worst = max(worst, worst_bank_multiplicity(addrs, 8))
    for wave in range(4):
        for j in range(4):
            for e in range(2):
                for g in range(4):
                    addrs = [(l & 31) * ROW + 32 * (8 * wave + 4 * (l >> 5)) + 32 * j + 16 * e
                             for l in range(16 * g, 16 * g + 16)]
                    worst = max(worst, worst_bank_multiplicity(addrs, 16))
    assert worst == 1


def test_merge_output_map():
    for cb in range(4):
        for rr in range(32):
            for pc in range(8):
                g = pc >> 1
                ln = rr + 32 * (g & 1)
                for e in range(16):
                    mtl = 2 * (pc & 1) + ((e >> 1) & 1)
                    q = 2 * (e & 1) + (g >> 1)
                    r = 4 * q + (e >> 2)
                    assert out_coord(4 * cb + mtl, r, ln >> 5) == 128 * cb + 16 * pc + e
