// Read side for many query rows (heads a multiple of 64, or the (query, head)
// rows of an extend call): absorbed-MLA attention in which the 2-bit latent of
// each token is decoded once per 64 rows.
// RoLaQ paper: §2.1 (one content latent serves every head's key and value,
// BF16 RoPE key), §3.2 (reconstruction = group mean + scale * gain * level),
// §3.3 (read-side rotation folded into the absorbed projections), §4.1 / §A.3
// (sink and recent tokens kept in BF16), Fig. 1a / Fig. 3a.
//
// Workgroup = (work item, 64-row group): four waves, one per SIMD, in two
// pairs; pair p owns rows 32p .. 32p+31 of the group and wave h of a pair the
// latent half h (coordinates 256h .. 256h+255).  A work item is a run of
// 32-token tiles of one request; the items are sized on the device from
// ctx_lens so that no workgroup holds much more than the average work of a
// ragged batch.  Per tile:
//  * fill - wave w decodes latent group w (128 coordinates) of the tile's 32
//    tokens into a shared fp16 c_hat buffer in LDS ([token][coordinate], rows
//    padded by 16 bytes so that consecutive tokens start in consecutive bank
//    groups), and the workgroup
//    copies the tile's BF16 RoPE keys and code words next to it; sink /
//    recent tokens are converted from their BF16 rows instead of decoded;
//  * score - wave (p, h) contracts its latent half of c_hat with its 32 rows
//    of the absorbed query on 32x32x16 fp16 MFMAs (S^T[token, row]), plus
//    half of the RoPE part on 32x32x16 bf16 and the score correction (bf8
//    residuals of the fp16 table values against the fp8 query) on 32x32x64
//    f8f6f4;
//  * exchange + softmax - the two partial scores of a pair meet in LDS and
//    both waves run the same lazy online softmax;
//  * value - O^T[latent, row] += c_hat^T P^T for the wave's latent half on
//    32x32x16 fp16 MFMAs, c_hat^T read with the LDS transpose load, P in
//    registers straight from the score accumulator.
// Three LDS ring slots rotate: while tile i is scored, tile i-1 gets its value
// product and tile i+1 is filled; one barrier per tile orders the three.
// A request covered by one item writes its output rows directly; otherwise
// each pair writes its (max, sum, O) partial and the merge kernel combines the
// items of the request (LSE merge).

#include "rlq_decode_common.h"

namespace rlq {
namespace {

typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int kWideWaves = 4;
constexpr int kWideThreads = 64 * kWideWaves;
constexpr int kRowBytes = RLQ_DC * 2 + 16;            // fp16 c_hat of one token, padded
constexpr int kCBufBytes = kWaveTok * kRowBytes;      // 32.5 KB: c_hat of one tile
constexpr int kRopeBufBytes = kWaveTok * RLQ_DR * 2;  // 4 KB: BF16 RoPE keys of one tile
// Code words and bf8 residual tables of a tile, for the score correction:
// token row t holds its 32 code words at t * kCodeRow (rows padded so the 16
// rows of one 16-byte read start in distinct bank groups), then the tables
// [32 tokens][4 groups] (uint32: four bf8 residuals each).
constexpr int kCodeRow = RLQ_WORDS * 4 + 16;
constexpr int kCodeTabOff = kWaveTok * kCodeRow;
constexpr int kCodeBufBytes = kCodeTabOff + kWaveTok * 4 * 4;  // 5 KB
constexpr int kSlotBytes = kCBufBytes + kRopeBufBytes + kCodeBufBytes;
constexpr int kBufs = 3;
// Partial scores of the pairs: [tile parity][wave][quarter q][lane] f4
// (accumulator registers 4q .. 4q+3).
constexpr int kXchOff = kBufs * kSlotBytes;
constexpr int kXchBytes = 2 * kWideWaves * 4 * 64 * 16;
constexpr int kPageOff = kXchOff + kXchBytes;
constexpr int kWideLds = kPageOff + kMaxItemPages * 4;  // 159 KB: one workgroup per CU
static_assert(kWideLds <= 160 * 1024, "LDS budget");
// Query staging (fp16, operand order): row r at r * kQRow, chunk c (8 values)
// at 16 c; rows padded so 16 rows read at one chunk fall in distinct bank groups.
constexpr int kQRow = RLQ_DC * 2 + 16;
static_assert(kWideHeads * kQRow <= kXchOff, "query staging fits the ring");
constexpr int kPart32 = 32 * RLQ_DC;  // floats in the partial O of 32 rows

__device__ inline int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return __builtin_amdgcn_readfirstlane(v);
}

__device__ inline int wave_min(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o));
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

// c_hat row t: 16-byte chunk c at t * kRowBytes + 16 c.  Chunk c holds code
// word c >> 1 (coordinates 16 (c >> 1) .. +15), parity e = c & 1: codes 2e,
// 2e+4, 2e+8, 2e+12, 2e+1, 2e+5, 2e+9, 2e+13 of the word in that order, the
// order decode8 produces; so element a of 8-byte unit u (= 2c + half) is
// coordinate 16 (u >> 2) + 4a + 2 ((u >> 1) & 1) + (u & 1).  With 65 bank
// groups per row, the 16 tokens of a score read (one chunk each) fall in
// distinct bank groups, and so do the 32 units of a transposed read (4
// consecutive tokens x units u0 + hb + 8G, hb < 2, G < 4; see tr_load).

// RoPE keys of a tile in LDS: token row t (128 bytes), 16-byte chunk c at
// position c ^ ((t >> 1) & 7), so the 16 rows of a score operand read fall in
// distinct bank groups.
__device__ inline int rope_off(int t, int c) { return t * 128 + 16 * (c ^ ((t >> 1) & 7)); }

// The value product's M-tile mt (0..15) reads 8-byte units
// u0(mt) + hb + 8G (hb < 2, G < 4) with u0(mt) = 2 (mt & 3) + 32 (mt >> 2):
// A-operand row m = 16 hb + 4 G + a (a < 4) is coordinate
//   128 (mt >> 2) + 16 ((mt >> 1) & 1) + 2 (mt & 1) + 32 G + 4 a + hb,
// and accumulator register r of lane half hl (lane >> 5) holds row
// 8 (r >> 2) + 4 hl + (r & 3), i.e. hb = r >> 3, G = 2 ((r >> 2) & 1) + hl,
// a = r & 3.  M-tiles 8h .. 8h+7 cover latent half h.
__device__ __host__ constexpr int out_coord(int mt, int r, int hl) {
  return 128 * (mt >> 2) + 16 * ((mt >> 1) & 1) + 2 * (mt & 1) + 32 * (2 * ((r >> 2) & 1) + hl) + 4 * (r & 3) +
         (r >> 3);
}

// Gap between two MFMAs of different types chained on one 32x32 accumulator
// (as for the 16x16 shapes, an MFMA reading its accumulator straight from an
// MFMA of another type needs wait states the compiler does not insert): 24
// wait states.  The accumulator passes through the nops, so data dependence
// alone pins them between the two MFMAs and other work can move around them.
__device__ inline void mfma_type_gap(f16v &acc) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc)); }

// acc *= alpha for a value accumulator that lives in accumulation registers,
// one register at a time through a vector register.  Written out so the
// compiler keeps the accumulators there: a plain multiply would make it move
// them to vector registers for good (and spill the query operands).  Runs
// only when the lazy softmax raises its maximum; no MFMA result is pending
// then (the value product last wrote these registers before the tile's
// barrier, and the next one follows the softmax).
__device__ inline void scale_acc(f16v &o, float alpha) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float t = o[r];
    float tmp;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(t), "=&v"(tmp)
                 : "v"(alpha));
    o[r] = t;
  }
}

// What one lane loads for the fill of one tile: four code words of one token
// with the (mean, scale) of their group, and 16 bytes of a RoPE key.
struct FillLoad {
  u4 cw;
  float mu, sd;
  u4 rp;
};

// kProt: the cache has sink and/or recent BF16 rows.
template <bool kProt>
__global__ __launch_bounds__(kWideThreads, 1) void decode_wide_kernel(DecodeArgs A) {
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
  const int h = wave & 1, pr = wave >> 1;  // latent half, row tile of the pair
  const int lane = threadIdx.x & 63;
  const int r32 = lane & 31, hl = lane >> 5;
  const int T32 = A.heads >> 5;

  // ---- absorbed query of 64 rows, converted to fp16 and staged in LDS in
  // chunk order (row, chunk c = 2 * word + parity, 8 values in decode8's
  // order).  Thread t converts words (t + 256 j) of the 64 x 32 words; rows
  // past the request's last read its last row (never used).
  {
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      u4 w0[4], w1[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int wi = threadIdx.x + kWideThreads * (4 * pass + j);
        const int row = min(head0 + (wi >> 5), qr.n_rows - 1);
        const uint16_t *src = A.q_c + (qr.row0 + row) * RLQ_DC + 16 * (wi & 31);
        w0[j] = *(const u4 *)src;
        w1[j] = *(const u4 *)(src + 8);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int wi = threadIdx.x + kWideThreads * (4 * pass + j);
        auto elem = [&](int e) -> float {
          const uint32_t v = (e < 8) ? w0[j][e >> 1] : w1[j][(e - 8) >> 1];
          return bf16_to_f32((e & 1) ? (v >> 16) : (v & 0xFFFFu));
        };
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int bb = 0; bb < 2; ++bb) {
            // Half bb of chunk (word, e): codes 2e + bb + 4a, a = 0..3.
            const int s0 = 2 * e + bb;
            u2 v;
            v[0] = h16(elem(s0)) | (h16(elem(s0 + 4)) << 16);
            v[1] = h16(elem(s0 + 8)) | (h16(elem(s0 + 12)) << 16);
            *(u2 *)(smem + (wi >> 5) * kQRow + 16 * (2 * (wi & 31) + e) + 8 * bb) = v;
          }
      }
    }
  }
  __syncthreads();
  const unsigned char *qrow_l = smem + (32 * pr + r32) * kQRow;
  // Score operands: K-step k takes chunk 32h + 2k + hl (lane half hl supplies
  // K slots 8hl .. 8hl+7).
  half8 qB[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) qB[k] = *(const half8 *)(qrow_l + 16 * (32 * h + 2 * k + hl));
  // Correction operands (fp8, OCP e4m3): product j covers words
  // W0 = 16h + 8hl + 2j and W0 + 1, i.e. chunks 2 W0 .. 2 W0 + 3.
  i8v q8B[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c0 = 32 * h + 16 * hl + 4 * j;
    q8B[j] = cat4(query_fp8(*(const half8 *)(qrow_l + 16 * c0)), query_fp8(*(const half8 *)(qrow_l + 16 * (c0 + 1))),
                  query_fp8(*(const half8 *)(qrow_l + 16 * (c0 + 2))),
                  query_fp8(*(const half8 *)(qrow_l + 16 * (c0 + 3))));
  }
  // The query operands stay in accumulation registers for the whole item
  // (MFMA reads its A / B operands from them directly), which leaves the
  // vector registers to the fill, the softmax and the operand loads.
#pragma unroll
  for (int k = 0; k < 16; ++k) asm volatile("" : "+a"(qB[k]));
#pragma unroll
  for (int k = 0; k < 4; ++k) asm volatile("" : "+a"(q8B[k]));
  __syncthreads();  // query staging done: the ring may be overwritten
  const int row = head0 + 32 * pr + r32;  // this lane's row (head, or (query, head))
  // RoPE operands: K-step ks takes dimensions 32h + 16ks + 8hl .. + 7.
  bf16x8 qrB[2];
  {
    const uint16_t *qr_row = A.q_r + (qr.row0 + min(row, qr.n_rows - 1)) * RLQ_DR;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qrB[ks] = __builtin_bit_cast(bf16x8, *(const u4 *)(qr_row + 32 * h + 16 * ks + 8 * hl));
  }
  const int ctx = min(A.ctx_lens[b], A.max_ctx_len);
  // Positions this lane's row attends to: [0, lim); rows past the request's
  // last see none.
  int lim = ctx;
  if (A.cu_q != nullptr) lim = row < qr.n_rows ? ctx - qr.n_q + row / A.q_heads + 1 : 0;
  const int lim_min = wave_min(lim);
  const Protect pt = protect_range(A, ctx);
  // Tiles of this item that some row of the group can see: all of them for
  // decode; for extend, up to the last query of the group (later tiles are
  // masked for every row, so they are not loaded at all).
  int wg_lim = ctx;
  if (A.cu_q != nullptr) wg_lim = ctx - qr.n_q + (min(head0 + kWideHeads, qr.n_rows) - 1) / A.q_heads + 1;
  const int n = max(0, min(it.te, (wg_lim + kWaveTok - 1) / kWaveTok) - it.tb);
  const int pg0 = it.tb >> 1;  // first page (in the request's block table)

  // Page ids of the item, staged once (at most kMaxItemPages).
  int32_t *pg = (int32_t *)(smem + kPageOff);
  {
    const int np = n > 0 ? ((it.tb + n - 1) >> 1) - pg0 + 1 : 0;
    const int32_t *bt = A.block_table + (int64_t)b * A.max_pages + pg0;
    for (int i = threadIdx.x; i < np; i += kWideThreads) pg[i] = bt[i];
  }
  __syncthreads();

  // ---- fill role of this lane: token ft, group fg = wave, code words fw0 ..
  // fw0 + 3 (coordinates 16 fw0 .. 16 fw0 + 63); RoPE copy: 16 bytes (chunk
  // rch) of token rtok.
  const int ft = r32, fg = wave, fw0 = 8 * fg + 4 * hl;
  const int rtok = threadIdx.x >> 3, rch = threadIdx.x & 7;
  // Cache slot of the tile's first token: the page id is read from the LDS
  // table and kept in a scalar register, so every fill load is a scalar row
  // base plus a 32-bit lane offset.
  auto tile_slot0 = [&](int i) -> int64_t {
    const int tt = it.tb + min(i, n - 1);  // past the end: the last tile again
    const int page = __builtin_amdgcn_readfirstlane(pg[(tt >> 1) - pg0]);
    return (int64_t)page * RLQ_PAGE + 32 * (tt & 1);
  };
  const uint32_t off_cw = (uint32_t)(ft * RLQ_WORDS + fw0);      // words
  const uint32_t off_mt = (uint32_t)(ft * 8 + fg);               // floats
  const uint32_t off_rp = (uint32_t)(rtok * RLQ_DR + 8 * rch);   // bf16 elements
  auto load_fill = [&](int i, FillLoad &F) {
    const int64_t s0 = tile_slot0(i);
    const uint32_t *cw = A.codes + s0 * RLQ_WORDS;
    const float *mt = A.meta + s0 * 8;
    const uint16_t *rp = A.rope + s0 * RLQ_DR;
    F.cw = *(const u4 *)(cw + off_cw);
    F.mu = mt[off_mt];
    F.sd = mt[off_mt + 4];
    F.rp = *(const u4 *)(rp + off_rp);
  };
  auto cbuf = [&](int k) -> unsigned char * { return smem + k * kSlotBytes; };
  auto rbuf = [&](int k) -> unsigned char * { return smem + k * kSlotBytes + kCBufBytes; };
  auto codebuf = [&](int k) -> unsigned char * { return smem + k * kSlotBytes + kCBufBytes + kRopeBufBytes; };
  // Fill write offsets: chunk 2 (fw0 + j) + e of token ft.
  const int f_base = ft * kRowBytes + 32 * fw0;
  auto fill_off = [&](int j, int e) { return f_base + 32 * j + 16 * e; };
  // Fill of tile i (into ring slot k) in parts, so the iteration can
  // interleave its decoding with the MFMAs: the table (fill_lut), the eight
  // 16-byte chunks (fill_part), then the RoPE and code copies and, in tiles
  // that hold sink or recent positions, the BF16 latents of those tokens
  // written over the decoded values (fill_end).
  auto fill_lut = [&](int i, const FillLoad &F) -> Lut {
    const int pos = kWaveTok * (it.tb + i) + ft;
    return make_lut(F.mu, F.sd, A.gain, A.level_inner, A.level_outer, pos < ctx);
  };
  auto fill_part = [&](int k, const FillLoad &F, const Lut &l, int e2) {
    *(u4 *)(cbuf(k) + fill_off(e2 >> 1, e2 & 1)) = decode8(F.cw[e2 >> 1], e2 & 1, l).v;
  };
  auto fill_end = [&](int i, int k, const FillLoad &F, const Lut &l) {
    *(u4 *)(rbuf(k) + rope_off(rtok, rch)) = F.rp;
    // Code words and residual table of (token ft, group fg) for the scoring
    // waves' correction; BF16 rows below need none (table 0).
    *(u4 *)(codebuf(k) + ft * kCodeRow + 4 * fw0) = F.cw;
    uint32_t rs = l.rs;
    if constexpr (kProt) {
      const int pos0 = kWaveTok * (it.tb + i);
      if (pos0 < pt.ns || pos0 + kWaveTok > ctx - pt.nr) {
        const int pos = pos0 + ft;
        const bool sink = pos < pt.ns, rec = pos >= ctx - pt.nr && pos < ctx;
        if (sink || rec) {
          const uint16_t *src = sink ? A.sink + ((int64_t)b * A.n_sink + pos) * RLQ_DC
                                     : A.recent + ((int64_t)b * A.n_recent + pos % A.n_recent) * RLQ_DC;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const u4 w0 = *(const u4 *)(src + 16 * (fw0 + j));
            const u4 w1 = *(const u4 *)(src + 16 * (fw0 + j) + 8);
            *(u4 *)(cbuf(k) + fill_off(j, 0)) = convert8(w0, w1, 0);
            *(u4 *)(cbuf(k) + fill_off(j, 1)) = convert8(w0, w1, 1);
            __builtin_amdgcn_sched_barrier(0);  // one word's rows in registers at a time
          }
          rs = 0u;
        }
      }
    }
    if (hl == 0) *(uint32_t *)(codebuf(k) + kCodeTabOff + 4 * (4 * ft + fg)) = rs;
  };
  auto fill = [&](int i, int k, const FillLoad &F) {
    const Lut l = fill_lut(i, F);
#pragma unroll
    for (int e2 = 0; e2 < 8; ++e2) fill_part(k, F, l, e2);
    fill_end(i, k, F, l);
  };

  // ---- read offsets of this lane (within a ring slot).
  // Score operand of K-step k: chunk 32h + 2k + hl of token r32.
  const int s_base = r32 * kRowBytes + 16 * (32 * h + hl);
  // Transposed read (value operand) as a source lane: 8 bytes of token
  // T = 16 ks + 8 sec + 4 hl + (lane & 15) / 4, unit u0(mt) + hb + 8 G with
  // hb = (lane >> 4) & 1, G = lane & 3 (mt = 8h + j).
  const int tr_base = (4 * hl + ((lane & 15) >> 2)) * kRowBytes + 8 * ((lane >> 4) & 1) + 64 * (lane & 3) + 512 * h;

  // ---- pair state
  unsigned char *xch = smem + kXchOff;
  auto xch_at = [&](int i, int w) -> f4 * { return (f4 *)(xch + ((i & 1) * kWideWaves + w) * 4096) + lane; };
  float m_run = kNegInf, l_run = 0.f;
  const float pinf = opaque_inf();
  f16v O[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) O[j] = f16v{};
  half8 PB[2];

  // Lazy online softmax of the pair's tile from the two partial scores (both
  // waves compute the same values: a sum of two terms does not depend on
  // their order).  Register r of the accumulator holds token
  // c0 + 8 (r >> 2) + 4 hl + (r & 3) of row r32.
  auto softmax = [&](const f4 (&own)[4], const f4 (&oth)[4], int c0) {
    float sc[16];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[4 * q + j] = own[q][j] + oth[q][j];
    // Positions past the context (or, for extend, past the query) score -inf.
    if (c0 + kWaveTok > lim_min) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = c0 + 8 * (r >> 2) + 4 * hl + (r & 3);
        sc[r] = t < lim ? sc[r] : kNegInf;
      }
    }
    // Tile max with v_med3 (med3(x, y, +inf) = max(x, y)): the scores are
    // finite or -inf here, so no NaN handling is needed.
    auto mx = [&](float u, float v) { return max_nn(u, v, pinf); };
    float m8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) m8[j] = mx(sc[2 * j], sc[2 * j + 1]);
    float mt = mx(mx(mx(m8[0], m8[1]), mx(m8[2], m8[3])), mx(mx(m8[4], m8[5]), mx(m8[6], m8[7])));
    {
      auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
      mt = mx(__uint_as_float(a[0]), __uint_as_float(a[1])) * A.scale_log2;
    }
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kLazy) != 0) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int j = 0; j < 8; ++j) scale_acc(O[j], alpha);
      m_run = m_new;
    }
    const float mb = max_nn(m_run, -1e30f, pinf) - kBias;
    half2v ph[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      ph[j] = __builtin_convertvector((float2v){__builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * j], A.scale_log2, -mb)),
                                                __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * j + 1], A.scale_log2, -mb))},
                                      half2v);
#pragma unroll
    for (int j = 0; j < 8; ++j) l_run = __builtin_amdgcn_fdot2(ph[j], (half2v){1.0f16, 1.0f16}, l_run, false);
    // K-step ks of the value product: registers 8ks .. 8ks+7, i.e. tokens
    // 16ks + 8(e >> 2) + 4hl + (e & 3) in operand slot 8hl + e.
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      PB[ks] = __builtin_bit_cast(half8, u4{__builtin_bit_cast(uint32_t, ph[4 * ks]), __builtin_bit_cast(uint32_t, ph[4 * ks + 1]),
                                            __builtin_bit_cast(uint32_t, ph[4 * ks + 2]),
                                            __builtin_bit_cast(uint32_t, ph[4 * ks + 3])});
  };

  // Value operand of M-tile mt = 8h + j, K-step ks: two transposed reads
  // (tokens 16ks + 4hl' + j' and 16ks + 8 + 4hl' + j' of the source lanes,
  // j' < 4), the operand slots of P's registers 8ks .. 8ks+7.
  auto tr_load = [&](const unsigned char *vb, int j, int ks) -> half8 {
    const int o = 16 * ks * kRowBytes + 16 * (j & 3) + 256 * (j >> 2);
    const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(vb + tr_base + o));
    const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(vb + tr_base + o + 8 * kRowBytes));
    return __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // Iteration i (tile i in ring slot k = i % 3, a constant in each unrolled
  // copy): the pair's partial scores of tile i-1 -> softmax -> value product
  // of tile i-1 (slot k+2), scores of tile i (slot k), and the fill of tile
  // i+1 (slot k+1) from loads issued three tiles ahead, its parts placed
  // between the MFMA groups; then this wave's partial of tile i goes to the
  // exchange slots, the loads of tile i+4 are issued and the barrier closes
  // the iteration.  With one wave per SIMD nothing else hides LDS latency, so
  // every group's operands are read one group ahead (two register sets).
  // Past the item's end the fill repeats its last tile into a free slot, so
  // every scoring iteration issues the same loads.  kScore / kValue switch off
  // the first and last halves.
  // Operands of the first value group of the next iteration (tile i's M-tiles
  // 0 and 1), read in iteration i's tail before the barrier: tile i's ĉ is
  // complete since the barrier that opened iteration i.
  half8 vnext[2][2];
  auto iteration = [&](auto score_c, auto value_c, int i, int k, FillLoad &F) {
    constexpr bool kScore = decltype(score_c)::value;
    constexpr bool kValue = decltype(value_c)::value;
    const int kn = k == 2 ? 0 : k + 1, kp = k == 0 ? 2 : k - 1;
    const unsigned char *cs = cbuf(k);   // tile i
    const unsigned char *vb = cbuf(kp);  // tile i-1
    f16v acc = f16v{};
    Lut fl;
    u4 sop[2][4];         // score operands of four K-steps
    half8 vop[2][2][2];   // value operands of two M-tiles x two K-steps
    auto load_s = [&](int buf, int k4) {
#pragma unroll
      for (int t = 0; t < 4; ++t) sop[buf][t] = *(const u4 *)(cs + s_base + 32 * (4 * k4 + t));
    };
    auto mfma_s = [&](int buf, int k4) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, sop[buf][t]), qB[4 * k4 + t], acc, 0, 0, 0);
    };
    auto load_v = [&](int buf, int g) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) vop[buf][u][ks] = tr_load(vb, 2 * g + u, ks);
    };
    auto mfma_v = [&](int buf, int g) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          O[2 * g + u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop[buf][u][ks], PB[ks], O[2 * g + u], 0, 0, 0);
    };
    // ---- reads of the first group, in the order they are needed.
    u4 rp[2], wv0, wv1;
    uint32_t rt = 0;
    f4 o4[4], m4[4];
    if constexpr (kScore) {
      const unsigned char *rb = rbuf(k);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) rp[ks] = *(const u4 *)(rb + rope_off(r32, 4 * h + 2 * ks + hl));
      // Code words 16h + 8hl .. + 7 of token r32 and the residual table of
      // their group 2h + hl, for the correction.
      const unsigned char *cb = codebuf(k);
      wv0 = *(const u4 *)(cb + r32 * kCodeRow + 4 * (16 * h + 8 * hl));
      wv1 = *(const u4 *)(cb + r32 * kCodeRow + 4 * (16 * h + 8 * hl) + 16);
      rt = *(const uint32_t *)(cb + kCodeTabOff + 4 * (4 * r32 + 2 * h + hl));
      load_s(0, 0);
    }
    if constexpr (kValue) {
      // Both partials of tile i-1 come back from the exchange slots (the own
      // one too: the slots of tile i-1 are rewritten only in iteration i+1).
      const f4 *oth = xch_at(i - 1, wave ^ 1), *own = xch_at(i - 1, wave);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        o4[q] = oth[64 * q];
        m4[q] = own[64 * q];
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) vop[0][u][ks] = vnext[u][ks];
    }
    if constexpr (kScore) {
      fl = fill_lut(i + 1, F);
      // The tile's scores start with the RoPE part (bf16), then the score
      // correction (f8f6f4: bf8 residuals of the fp16 table values against
      // the fp8 query; lane (r32, hl) takes words 2j, 2j + 1 of its eight in
      // product j) and the f16 content products chain on it, with a gap at
      // each change of type.
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, rp[ks]), qrB[ks], acc, 0, 0, 0);
      mfma_type_gap(acc);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w0 = j < 2 ? wv0[2 * j] : wv1[2 * j - 4];
        const uint32_t w1 = j < 2 ? wv0[2 * j + 1] : wv1[2 * j - 3];
        const i8v r = cat4(resid8(w0, 0, rt), resid8(w0, 1, rt), resid8(w1, 0, rt), resid8(w1, 1, rt));
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(r, q8B[j], acc, 1, 0, 0, 0, 0, 0);
      }
      load_s(1, 1);
      mfma_type_gap(acc);
      mfma_s(0, 0);
    }
    if constexpr (kValue) softmax(m4, o4, kWaveTok * (it.tb + i - 1));
    __builtin_amdgcn_sched_barrier(0);
    // Value product of tile i-1 in four groups of two M-tiles; the score
    // products of tile i and the fill parts of tile i+1 ride along in the
    // first three, so the score chain is complete before the last group.
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // Reads for the next group first.
      if constexpr (kValue)
        if (g < 3) load_v((g + 1) & 1, g + 1);
      if constexpr (kScore) {
        if (g < 2) load_s(g & 1, g + 2);
        if (g < 3) mfma_s((g + 1) & 1, g + 1);
        fill_part(kn, F, fl, 2 * g);
        fill_part(kn, F, fl, 2 * g + 1);
      }
      if constexpr (kValue) mfma_v(g & 1, g);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kScore) {
      fill_end(i + 1, kn, F, fl);
      f4 *mine = xch_at(i, wave);
#pragma unroll
      for (int q = 0; q < 4; ++q) mine[64 * q] = f4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
      __builtin_amdgcn_sched_barrier(0);
      load_fill(i + 4, F);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) vnext[u][ks] = tr_load(cs, u, ks);
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

  // ---- this pair's rows: lanes l and l + 32 hold the two token halves of
  // row r32's sum; wave h holds latent half h of O.
  {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    l_run = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  }
  if (it.count == 1) {
    // The request's only item: normalised output rows and LSE, no partial.
    // L = 0: no tokens (out 0, lse -inf).
    if (row < qr.n_rows) {
      const float inv = l_run == 0.f ? 0.f : 1.f / l_run;
      float *o = A.out + (qr.row0 + row) * RLQ_DC;
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[out_coord(8 * h + j, r, hl)] = O[j][r] * inv;
      if (A.lse != nullptr && h == 0 && hl == 0)
        A.lse[qr.row0 + row] = l_run == 0.f ? kNegInf : (m_run + log2f(l_run) - kBias) * 0.69314718055994531f;
    }
  } else {
    const int64_t pidx = (int64_t)x * T32 + 2 * hq + pr;
    f4 *po = (f4 *)(A.part_o + pidx * kPart32) + lane;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        po[((8 * h + j) * 4 + q) * 64] = f4{O[j][4 * q], O[j][4 * q + 1], O[j][4 * q + 2], O[j][4 * q + 3]};
    if (h == 0 && hl == 0) {
      A.part_ml[pidx * 64 + 2 * r32] = m_run;
      A.part_ml[pidx * 64 + 2 * r32 + 1] = l_run;
    }
  }
  if (x == it.first && hq == 0 && threadIdx.x == 0) {
    A.plan[2 * b] = it.first;
    A.plan[2 * b + 1] = it.count;
  }
}

// Merge of the items of one request for one 32-row tile and one 128-coordinate
// block cb (M-tiles 4cb .. 4cb+3, i.e. f4 units 16cb .. 16cb+15: unit
// 4 mt + q holds registers 4q .. 4q+3 of M-tile mt for the 64 lanes), by a
// workgroup of four waves: the (max, sum) statistics are reduced once, wave w
// sums every item's four units of M-tile 4cb + w, and the block of 32 rows x
// 128 coordinates goes out row by row through LDS.  The request's items are
// consecutive; a request with one item wrote its rows itself.
__global__ __launch_bounds__(256) void decode_wide_merge_kernel(DecodeArgs A) {
  __shared__ float wts[kMaxSplits + 1][32];
  __shared__ float red_m[8][32], red_l[8][32];
  __shared__ f4 sums[4][4][64];
  const int T32 = A.heads >> 5;
  // (request, 32-row tile) index over gridDim.y x gridDim.z (the y limit is
  // 65,535; an extend call can have more tiles).
  const int64_t bt = blockIdx.y + (int64_t)gridDim.y * blockIdx.z;
  if (bt >= (int64_t)A.batch * T32) return;
  const int b = (int)(bt / T32), t32 = (int)(bt % T32);
  const QueryRows qr = query_rows(A, b);
  if (32 * t32 >= qr.n_rows) return;  // no such rows in this request
  const int first = A.plan[2 * b], S = A.plan[2 * b + 1];
  if (S == 1) return;
  const int cb = blockIdx.x;
  const int64_t p0 = (int64_t)first * T32 + t32;
  const float *ml = A.part_ml + p0 * 64;
  const int64_t mls = (int64_t)T32 * 64;  // floats between items
  const int tid = threadIdx.x;
  const int hr = tid & 31, st = tid >> 5;
  const int lane = tid & 63, w = tid >> 6, hh = lane & 31;
  const f4 *po = (const f4 *)(A.part_o + p0 * kPart32) + (16 * cb + 4 * w) * 64 + lane;
  const int64_t ps = (int64_t)T32 * (kPart32 / 4);  // f4 between items
  {
    float m = kNegInf;
    for (int s = st; s < S; s += 8) m = fmaxf(m, ml[s * mls + 2 * hr]);
    red_m[st][hr] = m;
  }
  // The first item's units are loaded while the statistics are reduced.
  f4 v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = po[q * 64];
  __syncthreads();
  {
    float M = kNegInf;
#pragma unroll
    for (int i = 0; i < 8; ++i) M = fmaxf(M, red_m[i][hr]);
    const float Mc = fmaxf(M, -1e30f);  // 0 weights for empty items
    float l = 0.f;
    for (int s = st; s < S; s += 8) {
      const float m = ml[s * mls + 2 * hr], ls = ml[s * mls + 2 * hr + 1];
      const float wt = __builtin_amdgcn_exp2f(m - Mc);
      wts[s][hr] = wt;
      l += wt * ls;
    }
    red_l[st][hr] = l;
  }
  __syncthreads();
  f4 acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = f4{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    const float wt = wts[s][hh];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] += wt * v[q];
    if (s + 1 < S) {
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = po[(int64_t)(s + 1) * ps + q * 64];
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) sums[w][q][lane] = acc[q];
  __syncthreads();
  // Thread (row rr, piece pc) writes coordinates 128 cb + 16 pc + e, e < 16:
  // with G = pc >> 1, that is register 4q + a of lane rr + 32 (G & 1) in M-tile
  // 4cb + 2 (pc & 1) + ((e >> 1) & 1), q = 2 (e & 1) + (G >> 1), a = e >> 2.
  const int rr = tid >> 3, pc = tid & 7;
  const int orow = 32 * t32 + rr;
  float L = 0.f, Mh = kNegInf;
#pragma unroll
  for (int i = 0; i < 8; ++i) L += red_l[i][rr];
#pragma unroll
  for (int i = 0; i < 8; ++i) Mh = fmaxf(Mh, red_m[i][rr]);
  if (orow < qr.n_rows) {
    // L = 0: no tokens (out 0, lse -inf).
    const float inv = L == 0.f ? 0.f : 1.f / L;
    const int G = pc >> 1, ln = rr + 32 * (G & 1);
    float *o = A.out + (qr.row0 + orow) * RLQ_DC + 128 * cb + 16 * pc;
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      f4 ov;
#pragma unroll
      for (int e1 = 0; e1 < 4; ++e1) {
        const int e = 4 * e4 + e1;
        ov[e1] = sums[2 * (pc & 1) + ((e >> 1) & 1)][2 * (e & 1) + (G >> 1)][ln][e >> 2] * inv;
      }
      *(f4 *)(o + 4 * e4) = ov;
    }
    if (A.lse != nullptr && cb == 0 && pc == 0)
      A.lse[qr.row0 + orow] = L == 0.f ? kNegInf : (Mh + log2f(L) - kBias) * 0.69314718055994531f;
  }
}

}  // namespace

WidePlan plan_wide(int32_t batch, int32_t heads, int32_t max_ctx_len) {
  WidePlan p;
  const int hq = heads >= kWideHeads ? heads / kWideHeads : 1;
  const int64_t max_tiles = ((int64_t)max_ctx_len + kWaveTok - 1) / kWaveTok;
  const int64_t per_req = max_tiles > 0 ? (max_tiles + kMaxItemTiles - 1) / kMaxItemTiles : 1;
  if ((int64_t)batch * hq >= 2 * kResidentWide) {
    // Enough (request, row group) workgroups without splitting contexts: one
    // item per request (more only past kMaxItemTiles tiles).  The grid is
    // not padded, so the row groups of a request spread over the XCDs.
    p.item_target = batch;
    p.item_slots = (int32_t)(batch * per_req);
    p.partials = per_req > 1 ? 1 : 0;
    return p;
  }
  // One round of workgroups that fills the GPU: one per CU, two per item
  // for 128 heads.  At least one item per XCD: the row groups of an item
  // share its XCD, so with fewer than 8 items some XCDs would get no work.
  p.item_target = kResidentWide / hq > 8 ? kResidentWide / hq : 8;
  int64_t slots = (int64_t)batch * per_req;
  if (slots < p.item_target) slots = p.item_target;
  // A multiple of 8, so the row groups of an item (workgroup ids slots apart)
  // land on the same XCD and share its L2.
  slots = (slots + 7) / 8 * 8;
  p.item_slots = (int32_t)slots;
  p.partials = 1;
  return p;
}

int64_t extend_rows(int32_t max_q_len, int32_t heads) {
  return ((int64_t)max_q_len * heads + kWideHeads - 1) / kWideHeads * kWideHeads;
}

// Workspace: the plan ([batch][2] int32, padded to 256 bytes), then, when a
// request can span several items, the partial O ([slot][32-row tile][32 x
// 512] fp32) and the (max, sum) pairs ([slot][32-row tile][32][2]).
static size_t plan_bytes(int32_t batch) { return ((size_t)batch * 2 * sizeof(int32_t) + 255) / 256 * 256; }

size_t wide_workspace_bytes(int32_t batch, int32_t heads, const WidePlan &plan) {
  const size_t tiles = plan.partials ? (size_t)plan.item_slots * (heads / 32) : 0;
  return plan_bytes(batch) + tiles * (kPart32 + 64) * sizeof(float);
}

void wide_workspace_layout(DecodeArgs &a, void *workspace, int32_t batch, int32_t heads, const WidePlan &plan) {
  const size_t tiles = plan.partials ? (size_t)plan.item_slots * (heads / 32) : 0;
  a.plan = (int32_t *)workspace;
  a.part_o = plan.partials ? (float *)((unsigned char *)workspace + plan_bytes(batch)) : nullptr;
  a.part_ml = plan.partials ? a.part_o + tiles * kPart32 : nullptr;
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
    hipLaunchKernelGGL(decode_wide_kernel<true>, grid, dim3(kWideThreads), kWideLds, stream, a);
  else
    hipLaunchKernelGGL(decode_wide_kernel<false>, grid, dim3(kWideThreads), kWideLds, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.part_o == nullptr) return e;
  // Four workgroups per (request, 32-row tile), one per 128-coordinate block.
  const int64_t bt = (int64_t)batch * (a.heads / 32);
  const int gy = bt < 65535 ? (int)bt : 65535;
  hipLaunchKernelGGL(decode_wide_merge_kernel, dim3(RLQ_DC / 128, gy, (int)((bt + gy - 1) / gy)), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace rlq
