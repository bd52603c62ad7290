// Read side: absorbed-MLA decode attention over the paged 2-bit cache.
// RoLaQ paper: §2.1 (one content latent serves keys and values, BF16 RoPE
// key), §3.2 (reconstruction = group mean + scale * gain * level), §3.3
// (read-side rotation folded into the absorbed projections), §4.1 / §A.3
// (sink and recent tokens kept in BF16), Fig. 1a / Fig. 3a.
//
// Split-KV.  Workgroup (split, request, 16-head group) = four wave pairs,
// one workgroup per CU, two waves per SIMD.  Each pair walks its share of the
// split in 32-token tiles (two 16-token sub-tiles); wave h of a pair owns
// latent half h (coordinates of K-steps 8h .. 8h+7):
//  * score - each lane loads, for one token, 16 bytes of code words, the
//    (mean, scale) of the group they belong to and 16 bytes of the RoPE key.
//    A per-(token, group) table of the four fp16 values mu + s*g*{-b,-a,+a,+b}
//    (rounded once from fp32) is applied to the codes with byte permutes
//    (v_perm_b32), giving the fp16 c_hat operand with no per-coordinate
//    arithmetic.  Partial scores S^T[token, head] over the wave's half run on
//    MFMA (16x16x32 fp16 content part, 16x16x32 bf16 RoPE part) in a
//    contraction order chosen so every lane's operand comes straight from the
//    code words it loaded; the absorbed query is laid out in the same order
//    once per workgroup.  c_hat also goes to the wave's LDS region.
//  * exchange - the two partial scores meet in LDS slots that a reader marks
//    empty again (kPoison), so no barrier is needed; both waves run the same
//    lazy online softmax on the full scores.
//  * value - O^T[latent, head] += c_hat^T P^T for the wave's half, reading
//    c_hat^T with the gfx950 LDS transpose load (ds_read_b64_tr_b16); P (fp16,
//    times 2^kBias) never leaves registers.
// Tiles are software-pipelined: the value product of tile i-1 runs inside the
// decode loop of tile i.  The pairs of a workgroup merge through LDS at the
// end; a protected-token kernel covers the BF16 sink/recent tokens, and a
// merge kernel combines the per-split partials (LSE merge) and restores the
// natural coordinate order.

#include "rlq_decode_common.h"

namespace rlq {
namespace {

constexpr int kPairs = kDecodeWaves / 2;           // wave pairs per workgroup
constexpr int kChatBytes = kDecodeWaves * kWaveBytes;  // 128 KB
constexpr int kXchBytes = kPairs * 2 * 2 * 2 * 64 * 16;  // [pair][parity][half][sub-tile] scores
constexpr int kLdsBytes = kChatBytes + kXchBytes;      // 160 KB: one workgroup per CU
// Workgroups resident at once: one per CU x 256 CUs.
constexpr int kResidentWorkgroups = 256;
// Partial-score exchange between the two waves of a pair: an empty slot holds
// this NaN pattern (no partial score of finite inputs is NaN); a reader polls
// at most A.spin_limit times, then gives up and marks the workgroup's partial
// NaN, so the call's output and LSE for those rows come out NaN.
constexpr uint32_t kPoison = 0x7fbadbadu;

// What one lane loads for its tokens of a wave tile (32 consecutive tokens as
// two 16-token sub-tiles), for the latent half h of its wave (K-steps 8h ..
// 8h+7 and RoPE K-step h).  Code words with the (mean, scale) of their group
// 2*(g>>1) + h, fetched two tiles ahead; the RoPE key, needed only at the
// end of a tile, is fetched as the tile starts.
struct CodeLoad {
  u4 cw[2];          // code words [4 q0 + 8h, 4 q0 + 8h + 4) of sub-tile 0 / 1
  float mu, sd;      // (mean, scale) of sub-tile g & 1 (lanes g and g ^ 1 share a table)
};
struct RopeLoad {
  u4 rp[2];          // RoPE key elements [16g + 8h, 16g + 8h + 8)
};

// `first` = cache slot (page * 64 + 0 or 32) of the tile's first token, the
// same for the whole wave: the row bases are scalar and the per-lane parts
// 32-bit offsets.
__device__ inline void load_codes(const DecodeArgs &A, int64_t first, int r16, int g4, int h,
                                  CodeLoad &L) {
  const uint32_t q0 = 4 * (g4 >> 1) + (g4 & 1);
  const uint32_t *cw = A.codes + first * RLQ_WORDS;
  const float *mt = A.meta + first * 8;
#pragma unroll
  for (int st = 0; st < 2; ++st)
    L.cw[st] = *(const u4 *)(cw + (uint32_t)((16 * st + r16) * RLQ_WORDS + 4 * q0 + 8 * h));
  const uint32_t m = (16 * (g4 & 1) + r16) * 8 + 2 * (g4 >> 1) + h;
  L.mu = mt[m];
  L.sd = mt[m + 4];
}
__device__ inline void load_rope(const DecodeArgs &A, int64_t first, int r16, int g4, int h,
                                 RopeLoad &L) {
  const uint16_t *rp = A.rope + first * RLQ_DR;
#pragma unroll
  for (int st = 0; st < 2; ++st)
    L.rp[st] = *(const u4 *)(rp + (uint32_t)((16 * st + r16) * RLQ_DR + 16 * g4 + 8 * h));
}


// Tokens per split of a request with ctx tokens: ctx spread over the launch's
// splits in whole pages (at least 4), at most the launch's split size (which
// covers the longest context).
__device__ inline int split_tokens(const DecodeArgs &A, int ctx) {
  const int per = (ctx + A.splits - 1) / A.splits;
  const int t = max(4 * RLQ_PAGE, (per + RLQ_PAGE - 1) / RLQ_PAGE * RLQ_PAGE);
  return min(t, A.tokens_per_split);
}

// kProt = false: the ordinary splits (partials prot .. prot + splits - 1 of a
// request); kProt = true: the BF16 sink/recent tokens (partial 0).
//
// Workgroup = kPairs wave pairs (two waves per SIMD); a pair walks its share
// of the workgroup's tiles.
// Wave h of a pair owns latent half h: it decodes K-steps 8h .. 8h+7 (and
// RoPE K-step h) of each tile, so its score accumulator holds a partial sum;
// the two partials are exchanged through LDS (no barrier: see kPoison) and both
// waves run the same online softmax on the full scores.  The value product of
// wave h covers latent half h, whose c_hat it wrote to its own LDS region.
template <bool kProt>
__device__ __attribute__((always_inline)) void split_body(const DecodeArgs &A, const int sp) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int b = blockIdx.y, hg = blockIdx.z;
  const int part = kProt ? 0 : A.prot + sp;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = wave & 1, pr = wave >> 1;  // latent half, pair
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int HG = A.heads >> 4;
  // The absorbed query (converted and staged below) is loaded first: it
  // depends on nothing, and the page-id and code loads then overlap it.
  constexpr int kQChunks = 16 * RLQ_DC / 8 / kDecodeThreads;  // 16-byte chunks per thread
  u4 qv[kQChunks];
  {
    const uint16_t *qsrc = A.q_c + ((int64_t)b * A.heads + hg * 16) * RLQ_DC;
#pragma unroll
    for (int j = 0; j < kQChunks; ++j) qv[j] = *(const u4 *)(qsrc + 8 * (threadIdx.x + j * kDecodeThreads));
  }
  const bf16x8 qrB = __builtin_bit_cast(
      bf16x8, *(const u4 *)(A.q_r + ((int64_t)b * A.heads + hg * 16 + r16) * RLQ_DR + 16 * g4 + 8 * h));
  // Page ids of the pair's tiles in one VGPR: lane l holds page
  // p_first + (tile0 >> 1) + l (a pair's tiles span at most 64 pages), so a
  // tile's loads need one readlane and no memory access for their page.
  // They are fetched first for the launch's split size (right when every
  // context is near the longest) and again below if this request's split
  // size differs.
  auto pid_load = [&](int tb, int ni) -> int32_t {
    const int pf = (tb >> 6) + ((pr * ni) >> 1) + lane;
    return (!kProt && pf < A.max_pages) ? A.block_table[(int64_t)b * A.max_pages + pf] : 0;
  };
  const int tps_h = A.tokens_per_split;
  int32_t pid_pair = pid_load(sp * tps_h, (tps_h / kWaveTok + kPairs - 1) / kPairs);
  const int ctx = A.ctx_lens[b];
  // Split size of this request: its context spread over the launch's splits
  // (so a short request among long ones, or a grid sized for a later, longer
  // context, still uses every split).
  const int tps = kProt ? tps_h : split_tokens(A, ctx);
  // A split past the context (other than split 0) has nothing to add: the
  // merge reads only the splits that hold tokens, so it exits at once.
  if (!kProt && sp > 0 && sp * tps >= ctx) {
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }
  const Protect pr_ = protect_range(A, ctx);
  // Token range of this workgroup: positions for ordinary splits, indices
  // into the protected list (sink positions, then recent positions) for the
  // protected one.
  int t_begin, t_end;
  if (kProt) {
    t_begin = 0;
    t_end = pr_.ns + pr_.nr;
  } else {
    t_begin = sp * tps;
    t_end = min(ctx, t_begin + tps);
  }
  const int u_lo = pr_.ns, u_hi = ctx - pr_.nr;  // unprotected positions

  // Tiles of the workgroup.  An ordinary split deals its nominal tile count
  // (tps / 32) out to the pairs; in a split cut short by the context the last
  // pairs get fewer tiles or none.  The protected workgroup deals its tiles
  // evenly (every pair runs n_iter steps, tiles past the end masked).
  const int n_tiles = t_end > t_begin ? (t_end - t_begin + kWaveTok - 1) / kWaveTok : 0;
  const int n_iter = kProt ? (n_tiles + kPairs - 1) / kPairs : (tps / kWaveTok + kPairs - 1) / kPairs;
  const int tile0 = pr * n_iter;
  const int n_mine = min(max(n_tiles - tile0, 0), n_iter);  // ordinary splits: tiles of this pair
  const int pp0 = tile0 >> 1;
  if (!kProt && tps != tps_h) pid_pair = pid_load(t_begin, n_iter);
  const int last_mine = tile0 + n_mine - 1;
  auto tile_slot = [&](int i) -> int64_t {  // i = pair-local tile index
    // Past the pair's last tile the last one is loaded again (never
    // consumed); a pair without tiles loads cache slot 0 (never consumed).
    const int t = min(tile0 + i, last_mine);
    const int64_t s = (int64_t)__builtin_amdgcn_readlane(pid_pair, (t >> 1) - pp0) * RLQ_PAGE +
                      ((t_begin + kWaveTok * t) & 63);
    return n_mine > 0 ? s : 0;
  };
  // ---- absorbed query of 16 heads, converted to fp16 and scattered through
  // LDS into operand order: row (head) hd, K-step k, lane group g, slot j at
  // qslot(hd, k, g) + 2j.  The first two tiles' code loads go out before
  // it, so their latency overlaps the staging.
  constexpr int kQHead = 16 * 4 * 16 + 16;  // bytes per head row, padded against bank conflicts
  static_assert(16 * kQHead <= kChatBytes, "query staging fits");
  auto qslot = [](int hd, int k, int g) { return hd * kQHead + (k * 4 + g) * 16; };
  CodeLoad c0, c1, c2;
  if constexpr (!kProt) {
    load_codes(A, tile_slot(0), r16, g4, h, c0);
    load_codes(A, tile_slot(1), r16, g4, h, c1);
  }
#pragma unroll
  for (int j = 0; j < kQChunks; ++j) {
    const int c = threadIdx.x + j * kDecodeThreads;
    const int hd = c >> 6;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // Latent coordinate x = 16 word + sub, inverted through coord_of.
      const int x = 8 * (c & 63) + e, word = x >> 4, sub = x & 15, w2 = word >> 2;
      const int k = 8 * ((w2 >> 1) & 1) + 2 * (word & 3) + ((sub >> 1) & 1);
      const int g = ((w2 >> 2) << 1) | (w2 & 1);
      const int jj = 4 * (sub & 1) + (sub >> 2);
      const uint32_t v = (e & 1) ? (qv[j][e >> 1] >> 16) : (qv[j][e >> 1] & 0xFFFFu);
      *(_Float16 *)(smem + qslot(hd, k, g) + 2 * jj) = (_Float16)bf16_to_f32(v);
    }
  }
  __syncthreads();
  half8 qB[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) qB[k] = *(const half8 *)(smem + qslot(r16, 8 * h + k, g4));
  // The query in fp8 for the score correction of decoded tokens (BF16 sink /
  // recent rows convert to fp16 exactly and need none).
  constexpr bool kCorr = !kProt;
  i8v q8B[2];  // K-steps 0-3 and 4-7
  if constexpr (kCorr) {
#pragma unroll
    for (int k = 0; k < 2; ++k)
      q8B[k] = cat4(query_fp8(qB[4 * k]), query_fp8(qB[4 * k + 1]), query_fp8(qB[4 * k + 2]), query_fp8(qB[4 * k + 3]));
  }
  // Exchange slots of partial scores, [pair][parity][half][sub-tile][64 lanes].
  // A slot holding kPoison in any element is empty: the reader re-poisons a
  // slot after consuming it, so readiness needs no flag and no barrier.
  // The slots are accessed as volatile: a store that publishes a partial and
  // the partner's polling loads are not reordered or merged by the compiler.
  volatile lds_f4 *xch = (volatile lds_f4 *)(smem + kChatBytes);
  auto xch_at = [&](int i, int half) -> volatile lds_f4 * {
    return xch + (((pr * 2 + (i & 1)) * 2 + half) * 2) * 64;
  };
  bool xch_lost = false;  // a poll gave up (wave-uniform)
  const f4 poison = __builtin_bit_cast(f4, u4{kPoison, kPoison, kPoison, kPoison});
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    xch_at(par, h)[lane] = poison;
    xch_at(par, h)[64 + lane] = poison;
  }
  __syncthreads();

  float m_run = kNegInf, l_run = 0.f;
  const float pinf = opaque_inf();
  f4 O[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) O[i] = f4{0.f, 0.f, 0.f, 0.f};
  half8 PB = {};  // P of the previous tile: B operand of the value product

  unsigned char *wl = smem + wave * kWaveBytes;  // this wave's c_hat (latent half h)
  // Transposed-read offset of this lane: lane p = r16 of lane group g4 supplies
  // token row 4*g4 + p/4 of each sub-tile and coordinates q = p % 4.
  const int va = (r16 & 3) >> 1;
  const int vrd = 1024 * va + 16 * ((4 * g4 + (r16 >> 2)) ^ (8 * va)) + 8 * (r16 & 1);

  // Tile pipeline.  Step i (pair-local tile index) runs, in program order:
  //   part 1  - own partial scores of tile i-1 (finished in step i-1) out to
  //             the exchange slots and the partner's read back; transposed
  //             reads of tile i-1's K-step pair 0; decode + partial scores of
  //             tile i's K-step pair 0 (its c_hat overwrites those slots: LDS
  //             operations of a wave run in order);
  //   softmax - the partner's partial of tile i-1 (polled if not there yet),
  //             online softmax of tile i-1 -> P;
  //   part 2  - value product O^T += c_hat^T P^T of tile i-1 (pair 0 from
  //             registers, pairs 1..3 read just before tile i overwrites
  //             them), decode + partial scores of tile i's pairs 1..3, RoPE
  //             part, decode tables of tile i+1.
  f4 acc_prev[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};

  // Online softmax of the pair's tile i (partial scores of this wave in
  // acc_prev).  The running max moves only when a tile exceeds it by more
  // than kLazy (log2 units), so O is rescaled rarely; P = 2^(s - m + kBias)
  // stays below 2^15.
  auto softmax = [&](const f4 &o0, const f4 &o1, int c0, int vlo, int vhi) {
    // Full raw scores = own partial + partner's partial (the same sum, in the
    // same order, on both waves of the pair).
    f4 sc[2];
    sc[0] = h == 0 ? acc_prev[0] + o0 : o0 + acc_prev[0];
    sc[1] = h == 0 ? acc_prev[1] + o1 : o1 + acc_prev[1];
    // sc[st][j] = raw score of token c0 + 16*st + 4*g4 + j, head r16.
    if (!(c0 >= vlo && c0 + kWaveTok <= vhi)) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = c0 + 16 * st + 4 * g4 + j;
          sc[st][j] = (t >= vlo && t < vhi) ? sc[st][j] : kNegInf;
        }
    }
    half2v ph[4];
    auto exps = [&]() {
      // While no finite score has been seen the clamp keeps the exponent
      // finite (exp2(-inf) = 0, never NaN).
      const float mb = max_nn(m_run, -1e30f, pinf) - kBias;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        ph[2 * st] = __builtin_convertvector(
            (float2v){__builtin_amdgcn_exp2f(__builtin_fmaf(sc[st][0], A.scale_log2, -mb)),
                      __builtin_amdgcn_exp2f(__builtin_fmaf(sc[st][1], A.scale_log2, -mb))},
            half2v);
        ph[2 * st + 1] = __builtin_convertvector(
            (float2v){__builtin_amdgcn_exp2f(__builtin_fmaf(sc[st][2], A.scale_log2, -mb)),
                      __builtin_amdgcn_exp2f(__builtin_fmaf(sc[st][3], A.scale_log2, -mb))},
            half2v);
      }
    };
    // P against the current running max first: the common case keeps the max
    // reduction off the critical path.  When the tile exceeds the running max
    // by more than kLazy the max moves, O is rescaled and P recomputed.
    exps();
    auto mx = [&](float x, float y) { return max_nn(x, y, pinf); };
    float mt = mx(mx(mx(sc[0][0], sc[0][1]), mx(sc[0][2], sc[0][3])), mx(mx(sc[1][0], sc[1][1]), mx(sc[1][2], sc[1][3])));
    mt = max_over_groups(mt, pinf) * A.scale_log2;
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kLazy) != 0) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int j = 0; j < 16; ++j) O[j] *= alpha;
      m_run = m_new;
      exps();
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) l_run = __builtin_amdgcn_fdot2(ph[j], (half2v){1.0f16, 1.0f16}, l_run, false);
    PB = __builtin_bit_cast(half8, u4{__builtin_bit_cast(uint32_t, ph[0]), __builtin_bit_cast(uint32_t, ph[1]),
                                      __builtin_bit_cast(uint32_t, ph[2]), __builtin_bit_cast(uint32_t, ph[3])});
  };

  auto slot_full = [&](const f4 &a, const f4 &c) -> bool {
    bool empty = false;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      empty |= (__float_as_uint(a[j]) == kPoison) | (__float_as_uint(c[j]) == kPoison);
    return __builtin_amdgcn_ballot_w64(empty) == 0;
  };

  auto tr_pair = [&](int p, half8 (&av)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const unsigned char *base = wl + 2048 * p + 256 * q + vrd;
      const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)base);
      const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(base + kSubBytes));
      av[q] = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto value_pair = [&](int p, const half8 (&av)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      O[4 * p + q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[q], PB, O[4 * p + q], 0, 0, 0);
  };

  // kScore: tile i is new (decode + partial scores); kValue: tile i-1 gets its
  // softmax and value product.  `tail` runs once the step's last code word is
  // decoded (the next tile's tables are built there).
  auto step = [&](auto score_c, auto value_c, auto &&dec, const u4 (&rp)[2], int i, int c0_prev,
                  int vlo, int vhi, auto &&tail) {
    constexpr bool kScore = decltype(score_c)::value;
    constexpr bool kValue = decltype(value_c)::value;
    f4 acc[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
    // Residual operands of the last four K-steps; every second pair of
    // K-steps ends with their correction, chained on the score accumulator.
    i8v res[2];
    auto score_one = [&](int kl, int st) {
      const Dec8 v = dec(kl, st);
      *(u4 *)(wl + st * kSubBytes + kl * 1024 + 16 * chat_slot(kl, g4, r16)) = v.v;
      acc[st] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, v.v), qB[kl], acc[st], 0, 0, 0);
      res[st][2 * (kl & 3)] = (int)v.r[0];
      res[st][2 * (kl & 3) + 1] = (int)v.r[1];
    };
    auto score_pair = [&](int p) {
      if (!kCorr || !(p & 1)) {
#pragma unroll
        for (int kl = 2 * p; kl < 2 * p + 2; ++kl)
#pragma unroll
          for (int st = 0; st < 2; ++st) score_one(kl, st);
      } else {
        // Sub-tile by sub-tile, so sub-tile 0's residuals are consumed (and
        // their registers freed) before sub-tile 1's are made.
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
          for (int kl = 2 * p; kl < 2 * p + 2; ++kl) score_one(kl, st);
          acc[st] = correct_scores4(res[st], q8B[p >> 1], acc[st]);
        }
      }
    };
    half8 av0[4];
    f4 o0, o1;
    volatile lds_f4 *other = xch_at(i - 1, h ^ 1);
    if constexpr (kValue) {
      // This wave's partial of tile i-1, finished in the previous step, is
      // published now rather than at the end of that step, so no wave waits
      // there for its last MFMAs.  The partner does the same; its partial is
      // read here and consumed after part 1.
      volatile lds_f4 *mine = xch_at(i - 1, h);
      mine[lane] = acc_prev[0];
      mine[64 + lane] = acc_prev[1];
      o0 = other[lane];
      o1 = other[64 + lane];
      tr_pair(0, av0);
    }
    if constexpr (kScore) score_pair(0);
    if constexpr (kValue) {
      bool ready = slot_full(o0, o1) && !A.force_xch_timeout;
      if (!ready) {
        // Rare: the partner is behind.  Poll with a bound, so a wave can never
        // wait forever.
        for (int n = 0; n < A.spin_limit; ++n) {
          __builtin_amdgcn_s_sleep(2);
          o0 = other[lane];
          o1 = other[64 + lane];
          if (slot_full(o0, o1) && !A.force_xch_timeout) {
            ready = true;
            break;
          }
        }
        xch_lost |= !ready;
      }
      other[lane] = poison;
      other[64 + lane] = poison;
      softmax(o0, o1, c0_prev, vlo, vhi);
      value_pair(0, av0);
    }
#pragma unroll
    for (int p = 1; p < 4; ++p) {
      half8 av[4];
      if constexpr (kValue) tr_pair(p, av);
      if constexpr (kScore) score_pair(p);
      if constexpr (kValue) value_pair(p, av);
    }
    if constexpr (kScore) {
      mfma_type_switch();  // the accumulator comes from an f8f6f4 product (bf16 then reads it safely; the
                           // fence keeps a gap should an f16 product ever precede it)
#pragma unroll
      for (int st = 0; st < 2; ++st)
        acc[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, rp[st]), qrB, acc[st], 0, 0, 0);
      tail();
      acc_prev[0] = acc[0];
      acc_prev[1] = acc[1];
    }
  };
  auto no_dec = [](int, int) -> Dec8 { return Dec8{u4{0, 0, 0, 0}, u2{0, 0}}; };
  auto no_tail = []() {};
  const u4 no_rp[2] = {};

  if constexpr (!kProt) {
    const int vlo = u_lo, vhi = u_hi < t_end ? u_hi : t_end;
    auto c0_of = [&](int i) { return t_begin + kWaveTok * (tile0 + i); };
    // Decode tables of the tile being decoded; the tail of each step replaces
    // them with the next tile's.
    // Lanes g and g ^ 1 (lane groups 0/1, 2/3) decode the same token and
    // group: the even lane group builds sub-tile 0's table, the odd one
    // sub-tile 1's, and a permlane16 swap hands each its partner's.
    Lut lut[2];
    auto build_lut = [&](const CodeLoad &L, int i) {
      const int t = c0_of(i) + 16 * (g4 & 1) + r16;
      const Lut mine = make_lut(L.mu, L.sd, A.gain, A.level_inner, A.level_outer, t >= vlo && t < vhi);
      auto lo = __builtin_amdgcn_permlane16_swap(mine.lo, mine.lo, false, false);
      auto hi = __builtin_amdgcn_permlane16_swap(mine.hi, mine.hi, false, false);
      auto rs = __builtin_amdgcn_permlane16_swap(mine.rs, mine.rs, false, false);
      lut[0] = Lut{lo[0], hi[0], rs[0]};
      lut[1] = Lut{lo[1], hi[1], rs[1]};
    };
    RopeLoad rb;
    // Step i: `cur` holds tile i's codes, `next` tile i+1's, `far` takes
    // tile i+2's.  The RoPE load goes out before the far codes, so waiting
    // for it at the end of the step does not wait for them.
    auto run = [&](auto value_c, const CodeLoad &cur, const CodeLoad &next, CodeLoad &far, int i) {
      load_rope(A, tile_slot(i), r16, g4, h, rb);
      load_codes(A, tile_slot(i + 2), r16, g4, h, far);
      auto dec = [&](int kl, int st) -> Dec8 {
        return decode8(cur.cw[st][(kl >> 1) & 3], kl & 1, lut[st]);
      };
      auto tail = [&]() { build_lut(next, i + 1); };
      step(bool_c<true>{}, value_c, dec, rb.rp, i, c0_of(i - 1), vlo, vhi, tail);
    };
    if (n_mine > 0) {
      // Three code buffers used in turn: tile i+1's and tile i+2's codes are
      // in flight while tile i is processed.  Loads are issued
      // unconditionally (past the end the last tile is loaded again, from
      // L2) so the loop body has one straight path.
      build_lut(c0, 0);
      run(bool_c<false>{}, c0, c1, c2, 0);
      for (int i = 1; i < n_mine; i += 3) {
        run(bool_c<true>{}, c1, c2, c0, i);
        if (i + 1 >= n_mine) break;
        run(bool_c<true>{}, c2, c0, c1, i + 1);
        if (i + 2 >= n_mine) break;
        run(bool_c<true>{}, c0, c1, c2, i + 2);
      }
      step(bool_c<false>{}, bool_c<true>{}, no_dec, no_rp, n_mine, c0_of(n_mine - 1), vlo, vhi, no_tail);
    }
  } else {
    // Protected list index v -> position and BF16 source row.
    const int q0 = 4 * (g4 >> 1) + (g4 & 1);
    for (int i = 0; i < n_iter; ++i) {
      const int c0 = kWaveTok * (tile0 + i);
      const uint16_t *row[2] = {nullptr, nullptr};
      u4 rp[2] = {};
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int v = c0 + 16 * st + r16;
        if (v < t_end) {
          const int pos = (v < pr_.ns) ? v : (ctx - pr_.nr + (v - pr_.ns));
          row[st] = (v < pr_.ns) ? A.sink + ((int64_t)b * A.n_sink + pos) * RLQ_DC
                                 : A.recent + ((int64_t)b * A.n_recent + pos % A.n_recent) * RLQ_DC;
          const int64_t slot =
              (int64_t)A.block_table[(int64_t)b * A.max_pages + (pos >> 6)] * RLQ_PAGE + (pos & 63);
          rp[st] = *(const u4 *)(A.rope + slot * RLQ_DR + 16 * g4 + 8 * h);
        }
      }
      auto dec = [&](int kl, int st) -> Dec8 {
        if (row[st] == nullptr) return Dec8{u4{0, 0, 0, 0}, u2{0, 0}};
        const int word = 4 * (q0 + 2 * h) + ((kl >> 1) & 3);
        const u4 w0 = *(const u4 *)(row[st] + 16 * word);
        const u4 w1 = *(const u4 *)(row[st] + 16 * word + 8);
        return Dec8{convert8(w0, w1, kl & 1), u2{0, 0}};
      };
      if (i == 0)
        step(bool_c<true>{}, bool_c<false>{}, dec, rp, i, 0, 0, t_end, no_tail);
      else
        step(bool_c<true>{}, bool_c<true>{}, dec, rp, i, c0 - kWaveTok, 0, t_end, no_tail);
    }
    if (n_iter > 0)
      step(bool_c<false>{}, bool_c<true>{}, no_dec, no_rp, n_iter, kWaveTok * (tile0 + n_iter - 1), 0, t_end,
           no_tail);
  }

  // ---- partial of the workgroup: pairs 1 .. kPairs-1 hand their (max, sum,
  // O) to pair 0 through LDS; wave h of pair 0 merges latent half h.
  l_run = sum_over_groups(l_run);
  __syncthreads();  // every wave is done with its c_hat region and the exchange
  float *ml = (float *)(smem + kChatBytes);  // [pair][16 heads][2]
  int *lost = (int *)(ml + kPairs * 32);     // [wave]: a poll of this wave gave up
  if (lane == 0) lost[wave] = xch_lost ? 1 : 0;
  if (pr > 0) {
    if (h == 0 && g4 == 0) {
      ml[(pr * 16 + r16) * 2] = m_run;
      ml[(pr * 16 + r16) * 2 + 1] = l_run;
    }
    f4 *ol = (f4 *)(smem + ((pr - 1) * 2 + h) * kWaveBytes);
#pragma unroll
    for (int j = 0; j < 16; ++j) ol[j * 64 + lane] = O[j];
  }
  __syncthreads();
  if (pr == 0) {
    float mv[kPairs], sc[kPairs];
    mv[0] = m_run;
    float M = m_run;
#pragma unroll
    for (int v = 1; v < kPairs; ++v) {
      mv[v] = ml[(v * 16 + r16) * 2];
      M = fmaxf(M, mv[v]);
    }
    const float Mc = fmaxf(M, -1e30f);  // 0 weights for empty pairs
    float L = 0.f;
#pragma unroll
    for (int v = 0; v < kPairs; ++v) {
      sc[v] = __builtin_amdgcn_exp2f(mv[v] - Mc);
      L += sc[v] * (v == 0 ? l_run : ml[(v * 16 + r16) * 2 + 1]);
    }
    int any_lost = 0;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) any_lost |= lost[w];
    if (any_lost) L = __builtin_nanf("");  // the merge turns it into NaN output and LSE
    const int64_t pidx = ((int64_t)b * HG + hg) * (A.splits + A.prot) + part;
    f4 *po = (f4 *)(A.part_o + pidx * kPartialFloats);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      f4 o = sc[0] * O[j];
#pragma unroll
      for (int v = 1; v < kPairs; ++v)
        o += sc[v] * ((const f4 *)(smem + ((v - 1) * 2 + h) * kWaveBytes))[j * 64 + lane];
      po[(16 * h + j) * 64 + lane] = o;
    }
    if (h == 0 && g4 == 0) {
      A.part_ml[pidx * 32 + 2 * r16] = M;
      A.part_ml[pidx * 32 + 2 * r16 + 1] = L;
    }
  }
}

// The ordinary splits of every (request, head group): partials prot .. prot +
// splits - 1.
__global__ __launch_bounds__(kDecodeThreads, 1) void decode_split_kernel(DecodeArgs A) {
  split_body<false>(A, (int)blockIdx.x);
}

// The BF16 sink/recent tokens of each (request, head group): partial 0,
// launched before the ordinary splits (kept apart from them so each kernel is
// allocated only the registers of its own path).
__global__ __launch_bounds__(kDecodeThreads, 1) void decode_prot_kernel(DecodeArgs A) {
  split_body<true>(A, -1);
}

// The standalone merge: 32 workgroups of 4 waves per (request, head group).
__global__ __launch_bounds__(64 * kMergeWaves) void decode_merge_kernel(DecodeArgs A) {
  __shared__ float wts[kMaxSplits + 1][16];
  __shared__ float red_m[16][16], red_l[16][16];
  __shared__ f4 part[kMergeWaves][64];
  const int HG = A.heads >> 4;
  const int bh = blockIdx.y, S = A.splits + A.prot;
  // Only the splits that hold tokens (at least split 0) were written.
  const int ctx = A.ctx_lens[bh / HG];
  const int tps = split_tokens(A, ctx);
  const int used = A.prot + min(A.splits, max(1, (ctx + tps - 1) / tps));
  const MergeSrc src{(const f4 *)(A.part_o + (int64_t)bh * S * kPartialFloats), kPartialFloats / 4,
                     (const float2 *)(A.part_ml + (int64_t)bh * S * 32), 16, used};
  // Request bh / HG, head tile bh % HG: output rows 16 bh .. 16 bh + 15.
  merge_tiles(A, blockIdx.x, 1, (int64_t)bh * 16, src, wts, red_m, red_l, part);
}

}  // namespace

SplitPlan plan_splits(int32_t batch, int32_t heads, int32_t max_ctx_len) {
  // One round of workgroups that fills the GPU exactly: one per CU (256 CUs,
  // LDS-limited), in whole pages, at most kMaxSplits splits per request.
  const int64_t hg = heads / 16;
  const int64_t ctx = max_ctx_len > 0 ? max_ctx_len : 1;
  int64_t per_req = kResidentWorkgroups / (batch * hg);
  if (per_req < 1) per_req = 1;
  int64_t tps = (ctx + per_req - 1) / per_req;
  tps = ((tps + RLQ_PAGE - 1) / RLQ_PAGE) * RLQ_PAGE;
  if (tps < 4 * RLQ_PAGE) tps = 4 * RLQ_PAGE;
  int64_t splits = (ctx + tps - 1) / tps;
  if (splits > kMaxSplits) {
    tps = ((ctx + kMaxSplits - 1) / kMaxSplits + RLQ_PAGE - 1) / RLQ_PAGE * RLQ_PAGE;
    splits = (ctx + tps - 1) / tps;
  }
  // A split holds at most kMaxSplitPages pages (a wave pair's page ids fit
  // one register); longer splits are cut and the count follows.  Callers
  // reject contexts beyond kMaxSplits * kMaxSplitPages pages, so the count
  // stays within kMaxSplits.
  if (tps > (int64_t)kMaxSplitPages * RLQ_PAGE) {
    tps = (int64_t)kMaxSplitPages * RLQ_PAGE;
    splits = (ctx + tps - 1) / tps;
  }
  return SplitPlan{(int32_t)tps, (int32_t)splits};
}

size_t decode_workspace_bytes(int32_t batch, int32_t heads, const SplitPlan &plan) {
  const size_t parts = (size_t)batch * (heads / 16) * (plan.splits + 1);
  return parts * (kPartialFloats + 32) * sizeof(float);
}

hipError_t launch_decode(const DecodeArgs &a, int32_t batch, hipStream_t stream) {
  static PerDeviceOnce attr;
  hipError_t ea = once_per_device(attr, [] {
    for (const void *f : {(const void *)decode_split_kernel, (const void *)decode_prot_kernel}) {
      hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  });
  if (ea != hipSuccess) return ea;
  const int hg = a.heads / 16;
  if (a.prot) {
    hipLaunchKernelGGL(decode_prot_kernel, dim3(1, batch, hg), dim3(kDecodeThreads), kLdsBytes, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(decode_split_kernel, dim3(a.splits, batch, hg), dim3(kDecodeThreads), kLdsBytes, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(32, batch * hg), dim3(64 * kMergeWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rlq
