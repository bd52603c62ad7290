// Read side for many query heads (a multiple of 64): absorbed-MLA decode in
// which the 2-bit latent of each token is decoded once per 64 heads.
// RoLaQ paper: §2.1 (one content latent serves every head's key and value,
// BF16 RoPE key), §3.2 (reconstruction = group mean + scale * gain * level),
// §3.3 (read-side rotation folded into the absorbed projections), §4.1 / §A.3
// (sink and recent tokens kept in BF16), Fig. 1a / Fig. 3a.
//
// Workgroup = (work item, 64-head group): eight waves in four pairs, pair p
// owning head tile p (16 heads) and wave h of a pair latent half h.  A work
// item is a run of 32-token tiles of one request; the items are sized on the
// device from ctx_lens so that no workgroup holds much more than the average
// work of a ragged batch.  Per tile:
//  * fill - the eight waves decode the tile's 32 tokens x 512 coordinates
//    once (wave w: 16 tokens x one 128-coordinate group) into a shared fp16
//    c_hat buffer in LDS, in the operand layout of the score product, and copy
//    the tile's BF16 RoPE keys next to it; sink / recent tokens are converted
//    from their BF16 rows instead of decoded;
//  * score - wave (p, h) reads its latent half of c_hat from LDS and runs the
//    partial scores S^T[token, head] of head tile p on MFMA (16x16x32 fp16,
//    plus its RoPE K-step in bf16);
//  * exchange + softmax - the two partials of a pair meet in LDS (ordered by
//    the tile's barrier) and both waves run the same lazy online softmax;
//  * value - O^T[latent, head] += c_hat^T P^T for the wave's latent half,
//    c_hat^T read with the LDS transpose load, P in registers.
// Three c_hat buffers rotate: while tile i is scored, tile i-1 gets its value
// product and tile i+1 is filled; one barrier per tile orders the three.
// Each pair writes its own (max, sum, O) partial; the merge kernel combines
// the items of a request (LSE merge).

#include "rlq_decode_common.h"

namespace rlq {
namespace {

constexpr int kWideWaves = kDecodeWaves;            // 8: four pairs
constexpr int kWidePairs = kWideWaves / 2;           // head tiles per workgroup
constexpr int kCBufBytes = 2 * kWaveBytes;           // 32 KB: c_hat of one tile, both halves
constexpr int kRopeBufBytes = kWaveTok * RLQ_DR * 2; // 4 KB: BF16 RoPE keys of one tile
constexpr int kBufs = 3;
constexpr int kXchOff = kBufs * (kCBufBytes + kRopeBufBytes);
constexpr int kWideXchBytes = kWidePairs * 2 * 2 * 2 * 64 * 16;  // [pair][parity][half][sub-tile][lane]
constexpr int kPageOff = kXchOff + kWideXchBytes;
// Code words and bf8 residual tables of a tile, for the score correction:
// token row t holds its 32 code words at t * kCodeRow (rows padded so the 16
// rows of one 16-byte read start in distinct bank groups), then the tables
// [32 tokens][4 groups] (uint32: four bf8 residuals each).
constexpr int kCodeRow = RLQ_WORDS * 4 + 16;
constexpr int kCodeTabOff = kWaveTok * kCodeRow;
constexpr int kCodeBufBytes = kCodeTabOff + kWaveTok * 4 * 4;  // 5 KB
constexpr int kCodeOff = kPageOff + kMaxItemPages * 4;
constexpr int kWideLds = kCodeOff + kBufs * kCodeBufBytes;  // 159 KB: one workgroup per CU
static_assert(kWideLds <= 160 * 1024, "LDS budget");
constexpr int kQHead = 16 * 4 * 16 + 16;  // query staging: bytes per head row (padded)
static_assert(kWideHeads * kQHead <= kXchOff, "query staging fits the c_hat buffers");

__device__ inline int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return __builtin_amdgcn_readfirstlane(v);
}

__device__ inline int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Query rows of request b: first row (in q_c / q_r / out / lse, in rows of
// 512 / 64 / 512 / 1 elements), row count and query count.
struct QueryRows {
  int64_t row0;
  int n_rows, n_q;
};
__device__ inline QueryRows query_rows(const DecodeArgs &A, int b) {
  QueryRows r;
  if (A.cu_q != nullptr) {
    const int q0 = A.cu_q[b];
    r.n_q = A.cu_q[b + 1] - q0;
    r.row0 = (int64_t)q0 * A.q_heads;
    r.n_rows = r.n_q * A.q_heads;
  } else {
    r.n_q = 1;
    r.row0 = (int64_t)b * A.heads;
    r.n_rows = A.heads;
  }
  return r;
}

struct Item {
  int b;       // request
  int tb, te;  // tiles [tb, te) of the request (tile t = positions 32t .. 32t+31)
  int first;   // index of the request's first item
  int count;   // items of the request
};

// Work item x of the balanced plan; false past the last item.  Every wave of
// every workgroup computes the same plan from ctx_lens:
//   tiles_b = ceil(min(ctx_b, max_ctx_len) / 32),
//   items_b = max(1, ceil(tiles_b / K)),  items of request b in order,
// with K the smallest tile count (at least kMinItemTiles) for which the items
// number at most item_target, found by bisection (when batch < item_target;
// otherwise K = kMaxItemTiles).  K = ceil(T / (item_target - batch)) always
// qualifies, since sum(items_b) <= T / K + batch.  K is capped at
// kMaxItemTiles, so an item's page ids fit their LDS table; the launch sizes
// its grid for that case too.
__device__ bool find_item(const DecodeArgs &A, int x, Item &it) {
  const int lane = threadIdx.x & 63;
  const int B = A.batch;
  auto tiles = [&](int b) -> int {
    return b < B ? (min(A.ctx_lens[b], A.max_ctx_len) + kWaveTok - 1) / kWaveTok : 0;
  };
  auto items_of = [](int t, int K) { return max(1, (t + K - 1) / K); };
  int K = kMaxItemTiles;
  if (B < A.item_target) {
    // batch < item_target <= 256: lane l holds requests l, l+64, l+128, l+192.
    const int nu = (B + 63) >> 6;
    int t[4];
    int T = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      t[u] = u < nu ? tiles(lane + 64 * u) : 0;
      T += t[u];
    }
    T = wave_sum(T);
    const int tgt = A.item_target;
    int lo = max((T + tgt - 1) / tgt, kMinItemTiles);
    int hi = max((T + (tgt - B) - 1) / (tgt - B), lo);
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      int n = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (u < nu && lane + 64 * u < B) n += items_of(t[u], mid);
      if (wave_sum(n) <= tgt)
        hi = mid;
      else
        lo = mid + 1;
    }
    K = min(lo, kMaxItemTiles);
  }
  int base = 0;
  for (int c = 0; c < B; c += 64) {
    const int b = c + lane;
    const int t = tiles(b);
    const int n = b < B ? items_of(t, K) : 0;
    const int incl = wave_inclusive_scan(n, lane);
    const int excl = incl - n;
    const uint64_t hit = __ballot(n > 0 && x >= base + excl && x < base + incl);
    if (hit != 0) {
      const int l = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
      it.b = c + l;
      it.first = base + __builtin_amdgcn_readfirstlane(__shfl(excl, l));
      it.count = __builtin_amdgcn_readfirstlane(__shfl(n, l));
      const int tt = __builtin_amdgcn_readfirstlane(__shfl(t, l));
      it.tb = (x - it.first) * K;
      it.te = min(it.tb + K, tt);
      return true;
    }
    base += __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
  }
  return false;
}

// What one lane loads for the fill of one tile: two code words of one token
// with the (mean, scale) of their group, and 8 bytes of a RoPE key.
struct FillLoad {
  u2 cw;
  float mu, sd;
  u2 rp;
};

// LDS offset (within a c_hat buffer) of the 16-byte operand slot that code
// word W, parity e of token row r of sub-tile st decodes to: the slot of
// K-step k = 8*hh + 2*(W & 3) + e, lane group g in the contraction order of
// coord_of (word(k, g) = W).
__device__ inline int fill_slot(int W, int e, int st, int r) {
  const int a = W >> 2, q = W & 3;
  const int hh = (a >> 1) & 1;
  const int q0 = a - 2 * hh;
  const int g = 2 * (q0 >> 2) + (q0 & 1);
  const int kl = 2 * q + e;
  return hh * kWaveBytes + st * kSubBytes + kl * 1024 + 16 * chat_slot(kl, g, r);
}

// RoPE keys of a tile in LDS: token row t (128 bytes), 16-byte chunk c at
// position c ^ ((t >> 1) & 7), so the 16 rows of a score operand read fall in
// distinct bank groups.
__device__ inline int rope_off(int t, int c) { return t * 128 + 16 * (c ^ ((t >> 1) & 7)); }

// kProt: the cache has sink and/or recent BF16 rows.
template <bool kProt>
__global__ __launch_bounds__(kDecodeThreads, 1) void decode_wide_kernel(DecodeArgs A) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int x = blockIdx.x, hq = blockIdx.y;  // work item, 64-row group
  Item it;
  if (!find_item(A, x, it)) return;
  const int b = it.b;
  const int head0 = kWideHeads * hq;
  // Query rows of the request: its heads (decode), or (query, head) rows
  // (extend: query i at position ctx - n_q + i sees positions 0 .. ctx - n_q + i).
  const QueryRows qr = query_rows(A, b);
  if (head0 >= qr.n_rows) return;  // every row of this group is past the request's last
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = wave & 1, pr = wave >> 1;  // latent half, pair = head tile
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int HT = A.heads >> 4;

  // ---- absorbed query of 64 heads, converted to fp16 and scattered through
  // LDS into operand order (row = head hd, K-step k, lane group g, slot j at
  // hd * kQHead + (4k + g) * 16 + 2j), as in the 16-head kernel.
  constexpr int kQChunks = kWideHeads * RLQ_DC / 8 / kDecodeThreads;  // 8 per thread
  u4 qv[kQChunks];
  {
    // Rows past the request's last one read its last row (never used).
#pragma unroll
    for (int j = 0; j < kQChunks; ++j) {
      const int c = threadIdx.x + j * kDecodeThreads;
      const int row = min(head0 + (c >> 6), qr.n_rows - 1);
      qv[j] = *(const u4 *)(A.q_c + (qr.row0 + row) * RLQ_DC + 8 * (c & 63));
    }
  }
  const int qrow = min(head0 + 16 * pr + r16, qr.n_rows - 1);
  const bf16x8 qrB =
      __builtin_bit_cast(bf16x8, *(const u4 *)(A.q_r + (qr.row0 + qrow) * RLQ_DR + 16 * g4 + 8 * h));
  const int ctx = min(A.ctx_lens[b], A.max_ctx_len);
  // Positions this pair's rows attend to: [0, lim).  A head tile never spans
  // two queries (heads is a multiple of 16); tiles past the last row see none.
  int lim = ctx;
  if (A.cu_q != nullptr) {
    const int row_t = head0 + 16 * pr;
    lim = row_t < qr.n_rows ? ctx - qr.n_q + row_t / A.q_heads + 1 : 0;
  }
  const Protect pt = protect_range(A, ctx);
  // Tiles of this item that some row of the group can see: all of them for
  // decode; for extend, up to the last query of the group (later tiles are
  // masked for every pair, so they are not loaded at all).
  int wg_lim = ctx;
  if (A.cu_q != nullptr) wg_lim = ctx - qr.n_q + (min(head0 + kWideHeads, qr.n_rows) - 1) / A.q_heads + 1;
  const int n = max(0, min(it.te, (wg_lim + kWaveTok - 1) / kWaveTok) - it.tb);
  const int pg0 = it.tb >> 1;   // first page (in the request's block table)

  // Page ids of the item, staged once (at most kMaxItemPages).
  int32_t *pg = (int32_t *)(smem + kPageOff);
  {
    const int np = n > 0 ? ((it.tb + n - 1) >> 1) - pg0 + 1 : 0;
    const int32_t *bt = A.block_table + (int64_t)b * A.max_pages + pg0;
    for (int i = threadIdx.x; i < np; i += kDecodeThreads) pg[i] = bt[i];
  }
  auto qslot = [](int hd, int k, int g) { return hd * kQHead + (k * 4 + g) * 16; };
#pragma unroll
  for (int j = 0; j < kQChunks; ++j) {
    const int c = threadIdx.x + j * kDecodeThreads;
    const int hd = c >> 6;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // Latent coordinate x = 16 word + sub, inverted through coord_of.
      const int xc = 8 * (c & 63) + e, word = xc >> 4, sub = xc & 15, w2 = word >> 2;
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
  for (int k = 0; k < 8; ++k) qB[k] = *(const half8 *)(smem + qslot(16 * pr + r16, 8 * h + k, g4));
  __syncthreads();  // query staging done: the buffers below may be overwritten
  // The query in fp8 for the score correction.
  i8v q8B[2];  // K-steps 0-3 and 4-7
#pragma unroll
  for (int k = 0; k < 2; ++k)
    q8B[k] = cat4(query_fp8(qB[4 * k]), query_fp8(qB[4 * k + 1]), query_fp8(qB[4 * k + 2]), query_fp8(qB[4 * k + 3]));

  // ---- fill role of this lane: sub-tile fst, 128-coordinate group fgrp,
  // token row fr, code words W0, W0 + 1 (coordinates 16 W0 .. 16 W0 + 31).
  const int fst = wave >> 2, fgrp = wave & 3;
  const int fr = r16, W0 = 8 * fgrp + 2 * g4;
  const int ftok = 16 * fst + fr;  // token within the tile
  // RoPE copy role: token 4 * wave + (lane >> 4), bytes 8 * (lane & 15) ...
  const int rtok = 4 * wave + (lane >> 4), ru = lane & 15;
  // Cache slot of the tile's first token: the page id is read from the LDS
  // table and kept in a scalar register, so every fill load is a scalar row
  // base plus a 32-bit lane offset.
  auto tile_slot0 = [&](int i) -> int64_t {
    const int tt = it.tb + min(i, n - 1);  // past the end: the last tile again
    const int page = __builtin_amdgcn_readfirstlane(pg[(tt >> 1) - pg0]);
    return (int64_t)page * RLQ_PAGE + 32 * (tt & 1);
  };
  const uint32_t off_cw = (uint32_t)(ftok * RLQ_WORDS + W0);  // words
  const uint32_t off_mt = (uint32_t)(ftok * 8 + fgrp);        // floats
  const uint32_t off_rp = (uint32_t)(rtok * RLQ_DR + 4 * ru); // bf16 elements
  auto load_fill = [&](int i, FillLoad &F) {
    const int64_t s0 = tile_slot0(i);
    const uint32_t *cw = A.codes + s0 * RLQ_WORDS;
    const float *mt = A.meta + s0 * 8;
    const uint16_t *rp = A.rope + s0 * RLQ_DR;
    F.cw = *(const u2 *)(cw + off_cw);
    F.mu = mt[off_mt];
    F.sd = mt[off_mt + 4];
    F.rp = *(const u2 *)(rp + off_rp);
  };
  // c_hat and RoPE buffers of ring slot k (tile i lives in slot i % 3).
  auto cbuf = [&](int k) -> unsigned char * { return smem + k * kCBufBytes; };
  auto rbuf = [&](int k) -> unsigned char * { return smem + kBufs * kCBufBytes + k * kRopeBufBytes; };
  auto codebuf = [&](int k) -> unsigned char * { return smem + kCodeOff + k * kCodeBufBytes; };
  // Fill of tile i (into ring slot k) in parts, so the iteration can
  // interleave its decoding with the MFMAs: the table (fill_lut), the four
  // 16-byte slots (fill_part), then the RoPE copy and, in tiles that hold sink
  // or recent positions, the BF16 latents of those tokens written over the
  // decoded values (fill_end).
  auto fill_lut = [&](int i, const FillLoad &F) -> Lut {
    const int pos = kWaveTok * (it.tb + i) + ftok;
    return make_lut(F.mu, F.sd, A.gain, A.level_inner, A.level_outer, pos < ctx);
  };
  auto fill_part = [&](int k, const FillLoad &F, const Lut &l, int e2) {
    *(u4 *)(cbuf(k) + fill_slot(W0 + (e2 >> 1), e2 & 1, fst, fr)) = decode8(F.cw[e2 >> 1], e2 & 1, l).v;
  };
  auto fill_end = [&](int i, int k, const FillLoad &F, const Lut &l) {
    // RoPE key: 8 bytes of token rtok, chunk ru >> 1.
    *(u2 *)(rbuf(k) + rope_off(rtok, ru >> 1) + 8 * (ru & 1)) = F.rp;
    // Code words and residual table of (token ftok, group fgrp) for the
    // scoring waves' correction; BF16 rows below need none (table 0).
    *(u2 *)(codebuf(k) + ftok * kCodeRow + 4 * W0) = F.cw;
    uint32_t rs = l.rs;
    if constexpr (kProt) {
      const int pos0 = kWaveTok * (it.tb + i);
      if (pos0 < pt.ns || pos0 + kWaveTok > ctx - pt.nr) {
        const int pos = pos0 + ftok;
        const bool sink = pos < pt.ns, rec = pos >= ctx - pt.nr && pos < ctx;
        if (sink || rec) {
          const uint16_t *row = sink ? A.sink + ((int64_t)b * A.n_sink + pos) * RLQ_DC
                                     : A.recent + ((int64_t)b * A.n_recent + pos % A.n_recent) * RLQ_DC;
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            const u4 w0 = *(const u4 *)(row + 16 * (W0 + w));
            const u4 w1 = *(const u4 *)(row + 16 * (W0 + w) + 8);
            *(u4 *)(cbuf(k) + fill_slot(W0 + w, 0, fst, fr)) = convert8(w0, w1, 0);
            *(u4 *)(cbuf(k) + fill_slot(W0 + w, 1, fst, fr)) = convert8(w0, w1, 1);
            __builtin_amdgcn_sched_barrier(0);  // one word's rows in registers at a time
          }
          rs = 0u;
        }
      }
    }
    if (g4 == 0) *(uint32_t *)(codebuf(k) + kCodeTabOff + 4 * (4 * ftok + fgrp)) = rs;
  };
  auto fill = [&](int i, int k, const FillLoad &F) {
    const Lut l = fill_lut(i, F);
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) fill_part(k, F, l, e2);
    fill_end(i, k, F, l);
  };

  // ---- pair state
  f4 *xch = (f4 *)(smem + kXchOff);
  auto xch_at = [&](int i, int half) -> f4 * { return xch + (((pr * 2 + (i & 1)) * 2 + half) * 2) * 64; };
  float m_run = kNegInf, l_run = 0.f;
  const float pinf = opaque_inf();
  f4 O[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) O[i] = f4{0.f, 0.f, 0.f, 0.f};
  half8 PB = {};
  // Transposed-read offset of this lane (see the 16-head kernel): lane p = r16
  // of lane group g4 supplies token row 4*g4 + p/4 of each sub-tile and
  // coordinates q = p % 4.
  const int va = (r16 & 3) >> 1;
  const int vrd = 1024 * va + 16 * ((4 * g4 + (r16 >> 2)) ^ (8 * va)) + 8 * (r16 & 1);
  const int wq0 = 4 * (g4 >> 1) + (g4 & 1);  // this lane's 16-byte run of code words (coord_of)

  // Lazy online softmax of the pair's tile (own partial scores in m0, m1,
  // the partner's in o0, o1); both waves compute the same values.
  auto softmax = [&](const f4 &m0, const f4 &m1, const f4 &o0, const f4 &o1, int c0) {
    f4 sc[2];
    sc[0] = h == 0 ? m0 + o0 : o0 + m0;
    sc[1] = h == 0 ? m1 + o1 : o1 + m1;
    // sc[st][j] = raw score of position c0 + 16*st + 4*g4 + j, head r16.
    // Positions past the context (or, for extend, past the query) score -inf.
    if (c0 + kWaveTok > lim) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = c0 + 16 * st + 4 * g4 + j;
          sc[st][j] = t < lim ? sc[st][j] : kNegInf;
        }
    }
    half2v ph[4];
    auto exps = [&]() {
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
    exps();
    // Tile max with v_med3 (med3(x, y, +inf) = max(x, y)): the scores are
    // finite or -inf here, so no NaN handling is needed.
    auto mx = [&](float x, float y) { return max_nn(x, y, pinf); };
    float mt = mx(mx(mx(sc[0][0], sc[0][1]), mx(sc[0][2], sc[0][3])),
                  mx(mx(sc[1][0], sc[1][1]), mx(sc[1][2], sc[1][3])));
    {
      auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
      mt = mx(__uint_as_float(a[0]), __uint_as_float(a[1]));
      auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
      mt = mx(__uint_as_float(c[0]), __uint_as_float(c[1])) * A.scale_log2;
    }
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

  auto tr_pair = [&](const unsigned char *wl, int p, half8 (&av)[4]) {
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

  // Iteration i (tile i in ring slot k = i % 3, a constant in each unrolled
  // copy): partner's partial of tile i-1 -> softmax -> value product of tile
  // i-1 (slot k+2), partial scores of tile i (slot k), and the fill of tile
  // i+1 (slot k+1) from loads issued three tiles ahead, its four parts placed
  // between the MFMA groups; then this wave's partial of tile i goes to the
  // exchange slots, the loads of tile i+4 are issued and the barrier closes
  // the iteration.  Past the item's end the fill repeats its last tile into a
  // free slot, so every scoring iteration issues the same loads.  kScore /
  // kValue switch off the first and last halves.
  auto iteration = [&](auto score_c, auto value_c, int i, int k, FillLoad &F) {
    constexpr bool kScore = decltype(score_c)::value;
    constexpr bool kValue = decltype(value_c)::value;
    const int kn = k == 2 ? 0 : k + 1, kp = k == 0 ? 2 : k - 1;
    const unsigned char *cw = cbuf(k) + h * kWaveBytes;   // tile i, this wave's half
    const unsigned char *vw = cbuf(kp) + h * kWaveBytes;  // tile i-1
    f4 acc[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
    auto score_pair = [&](int p) {
#pragma unroll
      for (int kl = 2 * p; kl < 2 * p + 2; ++kl)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const u4 v = *(const u4 *)(cw + st * kSubBytes + kl * 1024 + 16 * chat_slot(kl, g4, r16));
          acc[st] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, v), qB[kl], acc[st], 0, 0, 0);
        }
    };
    // Score correction of tile i, after all its f16 products: lane (r16, g4)
    // scores token 16 st + r16 with code words 4 q0 + 8h .. + 3 (K-step kl
    // uses word kl / 2) of group 2 (g4 >> 1) + h and that group's residual
    // table, both read back from the tile's code buffer.
    const unsigned char *cb = codebuf(k);
    auto correct = [&]() {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const u4 wv = *(const u4 *)(cb + (16 * st + r16) * kCodeRow + 4 * (4 * wq0 + 8 * h));
        const uint32_t rt = *(const uint32_t *)(cb + kCodeTabOff + 4 * (4 * (16 * st + r16) + 2 * (g4 >> 1) + h));
#pragma unroll
        for (int k4 = 0; k4 < 2; ++k4)
          acc[st] = correct_scores4(cat4(resid8(wv[2 * k4], 0, rt), resid8(wv[2 * k4], 1, rt),
                                         resid8(wv[2 * k4 + 1], 0, rt), resid8(wv[2 * k4 + 1], 1, rt)),
                                    q8B[k4], acc[st]);
      }
    };
    Lut fl;
    if constexpr (kScore) {
      fl = fill_lut(i + 1, F);
      // The tile's scores start with the RoPE part (bf16, from LDS), then the
      // f16 content products and the f8f6f4 corrections chain on it (an f16
      // product may take its accumulator from a bf16 one, and an f8f6f4 one
      // from an f16 one; not the other way round from f16 to bf16).
      const unsigned char *rb = rbuf(k);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const u4 rp = *(const u4 *)(rb + rope_off(16 * st + r16, 2 * g4 + h));
        acc[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, rp), qrB, acc[st], 0, 0, 0);
      }
    }
    half8 av0[4];
    if constexpr (kValue) {
      // Both partials of tile i-1 come back from the exchange slots (the own
      // one too: the slots of tile i-1 are rewritten only in iteration i+1).
      const f4 *other = xch_at(i - 1, h ^ 1), *own = xch_at(i - 1, h);
      const f4 o0 = other[lane], o1 = other[64 + lane];
      const f4 m0 = own[lane], m1 = own[64 + lane];
      if constexpr (kScore) score_pair(0);
      softmax(m0, m1, o0, o1, kWaveTok * (it.tb + i - 1));
      tr_pair(vw, 0, av0);
      value_pair(0, av0);
    } else if constexpr (kScore) {
      score_pair(0);
    }
#pragma unroll
    for (int p = 1; p < 4; ++p) {
      half8 av[4];
      if constexpr (kValue) tr_pair(vw, p, av);
      if constexpr (kScore) score_pair(p);
      if constexpr (kScore) fill_part(kn, F, fl, p - 1);
      if constexpr (kValue) value_pair(p, av);
    }
    if constexpr (kScore) {
      correct();
      fill_part(kn, F, fl, 3);
      fill_end(i + 1, kn, F, fl);
      f4 *mine = xch_at(i, h);
      mine[lane] = acc[0];
      mine[64 + lane] = acc[1];
      __builtin_amdgcn_sched_barrier(0);
      load_fill(i + 4, F);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
    }
  };

  if (n > 0) {
    // The ring's loads are pinned in issue order (scheduling barriers).
    FillLoad F0, F1, F2;
    load_fill(0, F0);
    __builtin_amdgcn_sched_barrier(0);
    load_fill(1, F1);
    __builtin_amdgcn_sched_barrier(0);
    load_fill(2, F2);
    __builtin_amdgcn_sched_barrier(0);
    fill(0, 0, F0);
    load_fill(3, F0);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    // Iteration i fills tile i+1 from ring entry (i+1) % 3 and reloads it
    // with tile i+4.  Whole rounds of three run in the loop (no exit inside
    // it, which keeps the compiler's load-wait counts exact at its head), the
    // remaining one or two after it.
    iteration(bool_c<true>{}, bool_c<false>{}, 0, 0, F1);
    const int n3 = 1 + (n - 1) / 3 * 3;
    for (int i = 1; i < n3; i += 3) {
      iteration(bool_c<true>{}, bool_c<true>{}, i, 1, F2);
      iteration(bool_c<true>{}, bool_c<true>{}, i + 1, 2, F0);
      iteration(bool_c<true>{}, bool_c<true>{}, i + 2, 0, F1);
    }
    if (n3 < n) iteration(bool_c<true>{}, bool_c<true>{}, n3, 1, F2);
    if (n3 + 1 < n) iteration(bool_c<true>{}, bool_c<true>{}, n3 + 1, 2, F0);
    iteration(bool_c<false>{}, bool_c<true>{}, n, n % kBufs, F0);
  }

  // ---- partial of this pair's head tile: wave h writes latent half h.
  l_run = sum_over_groups(l_run);
  const int64_t pidx = (int64_t)x * HT + (head0 >> 4) + pr;
  f4 *po = (f4 *)(A.part_o + pidx * kPartialFloats);
#pragma unroll
  for (int j = 0; j < 16; ++j) po[(16 * h + j) * 64 + lane] = O[j];
  if (h == 0 && g4 == 0) {
    A.part_ml[pidx * 32 + 2 * r16] = m_run;
    A.part_ml[pidx * 32 + 2 * r16 + 1] = l_run;
  }
  if (x == it.first && hq == 0 && threadIdx.x == 0) {
    A.plan[2 * b] = it.first;
    A.plan[2 * b + 1] = it.count;
  }
}

// Merge of the items of one request: gridDim.x workgroups of 4 waves per
// (request, 16-head tile), each for 32 / gridDim.x of the 32 value tiles (so a
// large batch has fewer, longer workgroups); the request's items are
// consecutive.
__global__ __launch_bounds__(64 * kMergeWaves) void decode_wide_merge_kernel(DecodeArgs A) {
  __shared__ float wts[kMaxSplits + 1][16];
  __shared__ float red_m[16][16], red_l[16][16];
  __shared__ f4 part[kMergeMaxTiles][kMergeWaves][64];
  const int HT = A.heads >> 4;
  // (request, 16-row tile) index over gridDim.y x gridDim.z (the y limit is
  // 65,535; an extend call can have more tiles).
  const int64_t bh = blockIdx.y + (int64_t)gridDim.y * blockIdx.z;
  if (bh >= (int64_t)A.batch * HT) return;
  const int b = (int)(bh / HT), ht = (int)(bh % HT);
  const QueryRows qr = query_rows(A, b);
  if (16 * ht >= qr.n_rows) return;  // no such rows in this request
  const int first = A.plan[2 * b], count = A.plan[2 * b + 1];
  const int64_t p0 = (int64_t)first * HT + ht;
  const MergeSrc src{(const f4 *)(A.part_o + p0 * kPartialFloats), (int64_t)HT * (kPartialFloats / 4),
                     (const float2 *)(A.part_ml + p0 * 32), HT * 16, count};
  const int njp = 32 / gridDim.x;
  const int64_t orow = qr.row0 + 16 * ht;
  if (njp == 1)
    merge_tiles(A, blockIdx.x, 1, orow, src, wts, red_m, red_l, part[0]);
  else
    merge_tiles_multi(A, blockIdx.x * njp, njp, orow, src, wts, red_m, red_l, part);
}

}  // namespace

WidePlan plan_wide(int32_t batch, int32_t heads, int32_t max_ctx_len) {
  WidePlan p;
  // One round of workgroups that fills the GPU: one per CU, two per item
  // for 128 heads.  At least one item per XCD: the row groups of an item
  // share its XCD, so with many row groups (extend) and fewer than 8 items
  // some XCDs would get no work.
  const int hq = heads >= kWideHeads ? heads / kWideHeads : 1;
  p.item_target = kResidentWide / hq > 8 ? kResidentWide / hq : 8;
  const int64_t max_tiles = ((int64_t)max_ctx_len + kWaveTok - 1) / kWaveTok;
  const int64_t per_req = max_tiles > 0 ? (max_tiles + kMaxItemTiles - 1) / kMaxItemTiles : 1;
  int64_t slots = (int64_t)batch * per_req;
  if (slots < p.item_target) slots = p.item_target;
  // A multiple of 8, so the head groups of an item (workgroup ids slots apart)
  // land on the same XCD and share its L2.
  slots = (slots + 7) / 8 * 8;
  p.item_slots = (int32_t)slots;
  return p;
}

int64_t extend_rows(int32_t max_q_len, int32_t heads) {
  return ((int64_t)max_q_len * heads + kWideHeads - 1) / kWideHeads * kWideHeads;
}

size_t wide_workspace_bytes(int32_t batch, int32_t heads, const WidePlan &plan) {
  const size_t parts = (size_t)plan.item_slots * (heads / 16);
  return parts * (kPartialFloats + 32) * sizeof(float) + (size_t)batch * 2 * sizeof(int32_t);
}

hipError_t launch_decode_wide(const DecodeArgs &a, int32_t batch, hipStream_t stream) {
  static PerDeviceOnce attr;
  hipError_t ea = once_per_device(attr, [] {
    for (const void *f : {(const void *)decode_wide_kernel<false>, (const void *)decode_wide_kernel<true>}) {
      hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kWideLds);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  });
  if (ea != hipSuccess) return ea;
  const dim3 grid(a.item_slots, a.heads / kWideHeads);
  if (a.prot)
    hipLaunchKernelGGL(decode_wide_kernel<true>, grid, dim3(kDecodeThreads), kWideLds, stream, a);
  else
    hipLaunchKernelGGL(decode_wide_kernel<false>, grid, dim3(kDecodeThreads), kWideLds, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // About 1024 merge workgroups (at least 4 per request and head tile):
  // value tiles per workgroup 32 / chunks, at most kMergeMaxTiles.
  const int bht = batch * (a.heads / 16);
  int chunks = 32 / kMergeMaxTiles;
  while (chunks < 32 && (int64_t)chunks * bht < 1024) chunks *= 2;
  const int gy = bht < 65535 ? bht : 65535;
  hipLaunchKernelGGL(decode_wide_merge_kernel, dim3(chunks, gy, (bht + gy - 1) / gy), dim3(64 * kMergeWaves), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace rlq
