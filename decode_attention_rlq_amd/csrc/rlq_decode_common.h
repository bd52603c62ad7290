// Device helpers shared by the decode kernels (16-head split kernel and the
// many-head kernel): the contraction order of the content coordinates, the
// fp16 c_hat layout in LDS, the decoding of 2-bit codes through a per-token
// table of four values, and the LSE merge of split partials.
// RoLaQ paper: §3.2 (reconstruction = group mean + scale * gain * level),
// §2.1 / §3.3 (absorbed decode over the shared latent), §4.1 / §A.3 (BF16
// sink and recent tokens).
#pragma once

#include <math.h>

#include <type_traits>

#include "rlq_internal.h"

namespace rlq {
namespace {

typedef short s4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s4 lds_s4;
typedef __attribute__((address_space(3))) f4 lds_f4;

constexpr float kNegInf = -__builtin_inff();
constexpr int kPageTok = 64;                        // tokens per page
constexpr int kWaveTok = 32;                        // tokens per tile
constexpr int kSubBytes = kTile * (RLQ_DC / 2) * 2; // 8 KB: fp16 c_hat half of 16 tokens
constexpr int kWaveBytes = 2 * kSubBytes;           // 16 KB: fp16 c_hat half of one tile
// Lazy online softmax: the running max m is raised only when a tile's max
// exceeds it by more than kLazy (log2 units); P = 2^(s - m + kBias) then
// stays at most 2^15, inside fp16's range.
constexpr float kLazy = 8.f;
constexpr float kBias = 15.f - kLazy;

// Contraction order of the content coordinates (shared by the query layout,
// the code decoding, the LDS layout and the output mapping).  K-step k
// (0..15), lane group g (lane / 16) and operand slot j (0..7) of the
// 16x16x32 MFMA cover latent coordinate  16 * word(k, g) + sub(j, k & 1):
//   word(k, g) = 4 * (q0(g) + 2 * (k >> 3)) + ((k >> 1) & 3),
//   q0(g)      = 4 * (g >> 1) + (g & 1)        (16-byte run of code words),
//   sub(j, h)  = 2h + (j >> 2) + 4 * (j & 3)   (code within the word).
// A lane thus reads code words [4 q0, 4 q0 + 4) and [4 q0 + 8, 4 q0 + 12) of
// its token: groups 2*(g>>1) (k < 8) and 2*(g>>1)+1 (k >= 8).
__device__ __host__ constexpr int coord_of(int k, int g, int j) {
  return 16 * (4 * ((4 * (g >> 1) + (g & 1)) + 2 * (k >> 3)) + ((k >> 1) & 3)) +
         2 * (k & 1) + (j >> 2) + 4 * (j & 3);
}

// LDS slot (16 bytes) of token row r written by lane group g at K-step k.
// LDS has 64 four-byte banks (256 bytes per cycle): a 16-byte write serves 16
// lanes per cycle, an 8-byte transposed read 32 lanes.  The xor moves odd
// K-steps to the other 128-byte half of each 256-byte window, so the 32 lanes
// of a transposed read (tokens 0-7 of one writer lane group, K-steps 2p and
// 2p+1, both 8-byte halves) cover all 64 banks once.
__device__ __host__ constexpr int chat_slot(int k, int g, int r) {
  return (16 * g + r) ^ (8 * (k & 1));
}

// Value tile jp (0..31) holds, in row m = 4q + e (q, e in 0..3), the latent
// coordinate in K-step 2*(jp>>2) + (q>>1), lane group jp&3, slot 4*(q&1)+e.
__device__ __host__ constexpr int value_coord(int jp, int m) {
  return coord_of(2 * (jp >> 2) + ((m >> 2) >> 1), jp & 3, 4 * ((m >> 2) & 1) + (m & 3));
}

__device__ inline uint32_t h16(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ inline float bf16_to_f32(uint32_t v) { return __uint_as_float(v << 16); }

// max(x, y) of scores, which are finite or -inf (never NaN): one v_med3 with
// +inf (med3(x, y, +inf) = max(x, y)).  The +inf goes through an empty asm so
// the compiler cannot fold the med3 into maxnum, which it would precede with
// NaN-quieting self-max instructions on every operand.
__device__ inline float opaque_inf() {
  float v = __builtin_inff();
  asm volatile("" : "+v"(v));
  return v;
}
__device__ inline float max_nn(float x, float y, float pinf) { return __builtin_amdgcn_fmed3f(x, y, pinf); }

// Reductions over the 4 lane groups sharing lane & 15 (xor 16, xor 32).
__device__ inline float max_over_groups(float x, float pinf) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max_nn(__uint_as_float(a[0]), __uint_as_float(a[1]), pinf);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nn(__uint_as_float(b[0]), __uint_as_float(b[1]), pinf);
}
__device__ inline float sum_over_groups(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Table of one (token, group): low bytes and high bytes of the four fp16
// values, so v_perm_b32 can look both up with 2-bit selectors, and the four
// residuals t - fp16(t) of the fp32 table entries t, each rounded to bf8
// (OCP e5m2) in one byte.  The fp16 value carries a relative rounding error
// of up to 2^-12, which a score contracting 512 such values over a near tie
// of two tokens can no longer afford; the residual takes it down to ~2^-15
// (bf8 keeps 3 significant bits of it) in a second, 8-bit contraction.  The
// value product uses the fp16 value alone.
struct Lut {
  uint32_t lo, hi, rs;
};
__device__ inline Lut make_lut(float mu, float s, float gain, float a, float b, bool valid) {
  const float sg = s * gain;
  const float t0 = __builtin_fmaf(-sg, b, mu), t1 = __builtin_fmaf(-sg, a, mu);
  const float t2 = __builtin_fmaf(sg, a, mu), t3 = __builtin_fmaf(sg, b, mu);
  const _Float16 h0 = (_Float16)t0, h1 = (_Float16)t1, h2 = (_Float16)t2, h3 = (_Float16)t3;
  const uint32_t p01 = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
  const uint32_t p23 = (uint32_t)__builtin_bit_cast(uint16_t, h2) | ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
  // t - fp16(t) is exact in fp32 (fp16(t) is t cut to 11 significant bits).
  uint32_t rs = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(t0 - (float)h0, t1 - (float)h1, 0, false);
  rs = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(t2 - (float)h2, t3 - (float)h3, (int)rs, true);
  Lut l;
  l.lo = valid ? __builtin_amdgcn_perm(p23, p01, 0x06040200u) : 0u;
  l.hi = valid ? __builtin_amdgcn_perm(p23, p01, 0x07050301u) : 0u;
  l.rs = valid ? rs : 0u;
  return l;
}

// Codes 2h, 2h+4, 2h+8, 2h+12, 2h+1, 2h+5, 2h+9, 2h+13 of word w as eight
// fp16 values (operand slots 0..7) and, in the same slots, their eight bf8
// residuals (the operand of the score correction).
struct Dec8 {
  u4 v;
  u2 r;
};
__device__ inline Dec8 decode8(uint32_t w, int h, const Lut &l) {
  const uint32_t y0 = (w >> (4 * h)) & 0x03030303u;
  const uint32_t y1 = (w >> (4 * h + 2)) & 0x03030303u;
  const uint32_t lo0 = __builtin_amdgcn_perm(0u, l.lo, y0);
  const uint32_t hi0 = __builtin_amdgcn_perm(0u, l.hi, y0);
  const uint32_t lo1 = __builtin_amdgcn_perm(0u, l.lo, y1);
  const uint32_t hi1 = __builtin_amdgcn_perm(0u, l.hi, y1);
  Dec8 d;
  d.v[0] = __builtin_amdgcn_perm(hi0, lo0, 0x05010400u);
  d.v[1] = __builtin_amdgcn_perm(hi0, lo0, 0x07030602u);
  d.v[2] = __builtin_amdgcn_perm(hi1, lo1, 0x05010400u);
  d.v[3] = __builtin_amdgcn_perm(hi1, lo1, 0x07030602u);
  d.r[0] = __builtin_amdgcn_perm(0u, l.rs, y0);
  d.r[1] = __builtin_amdgcn_perm(0u, l.rs, y1);
  return d;
}

// The eight bf8 residuals of decode8(w, h, l) alone (for a wave that scores
// c_hat decoded by another wave).
__device__ inline u2 resid8(uint32_t w, int h, uint32_t rs) {
  u2 r;
  r[0] = __builtin_amdgcn_perm(0u, rs, (w >> (4 * h)) & 0x03030303u);
  r[1] = __builtin_amdgcn_perm(0u, rs, (w >> (4 * h + 2)) & 0x03030303u);
  return r;
}

// Gap between two MFMAs of different types chained on one accumulator.  On
// gfx950 an MFMA that takes its accumulator (srcC) straight from the result
// of an MFMA of another type (f16, bf16, bf8 x fp8) reads a wrong value unless
// about six wait states separate the two (measured: four fail, six suffice);
// the compiler assumes an exactly overlapping srcC is forwarded and inserts
// none.  The nop is fenced so no instruction moves across it.
__device__ inline void mfma_type_switch() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7");
  __builtin_amdgcn_sched_barrier(0);
}

// Score correction of four K-steps at once: acc += r^T q8 on one
// v_mfma_f32_16x16x128_f8f6f4 (A = the bf8 residuals of the four c_hat
// operands, B = the query rounded to fp8, OCP e4m3, in the same order).  The
// 128-deep product sums over every (lane group, slot) pair of A and B alike,
// so placing K-step k's eight values in slots 8k .. 8k+7 of both operands
// contracts the same coordinates as four 16x16x32 products.  (It also runs
// about three times faster than four 16x16x32 bf8 x fp8 products, and on this
// GPU it may take its accumulator straight from an f16 product; the 16x16x32
// bf8 x fp8 instruction may not.)
typedef int i8v __attribute__((ext_vector_type(8)));
__device__ inline i8v cat4(const u2 &a, const u2 &b, const u2 &c, const u2 &d) {
  return i8v{(int)a[0], (int)a[1], (int)b[0], (int)b[1], (int)c[0], (int)c[1], (int)d[0], (int)d[1]};
}
__device__ inline f4 correct_scores4(const i8v &r, const i8v &q8, const f4 &acc) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(r, q8, acc, 1, 0, 0, 0, 0, 0);
}

// Eight fp16 query values of an operand slot as fp8 (OCP e4m3, nearest).
__device__ inline u2 query_fp8(const half8 &q) {
  u2 r;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int v = __builtin_amdgcn_cvt_pk_fp8_f32((float)q[4 * i], (float)q[4 * i + 1], 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32((float)q[4 * i + 2], (float)q[4 * i + 3], v, true);
    r[i] = (uint32_t)v;
  }
  return r;
}

// The same eight coordinates taken from a BF16 latent word (16 values held
// in two 16-byte vectors), converted to fp16.
__device__ inline u4 convert8(const u4 &w0, const u4 &w1, int h) {
  auto elem = [&](int e) -> uint32_t {
    const uint32_t v = (e < 8) ? w0[e >> 1] : w1[(e - 8) >> 1];
    return (e & 1) ? (v >> 16) : (v & 0xFFFFu);
  };
  u4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int j0 = 2 * p, j1 = 2 * p + 1;
    const int e0 = 2 * h + (j0 >> 2) + 4 * (j0 & 3);
    const int e1 = 2 * h + (j1 >> 2) + 4 * (j1 & 3);
    r[p] = h16(bf16_to_f32(elem(e0))) | (h16(bf16_to_f32(elem(e1))) << 16);
  }
  return r;
}

struct Protect {
  int ns, nr;  // protected prefix length and recent length inside [0, ctx)
};

__device__ inline Protect protect_range(const DecodeArgs &A, int ctx) {
  Protect p;
  p.ns = (A.sink != nullptr) ? min(A.n_sink, ctx) : 0;
  p.nr = (A.recent != nullptr) ? min(A.n_recent, ctx - p.ns) : 0;
  return p;
}

template <bool V>
using bool_c = std::integral_constant<bool, V>;

// LSE merge of the split partials of one 16-row tile (output rows orow ..
// orow + 15: one request's 16-head tile, or 16 (query, head) rows of an
// extend call) for
// value tiles jp0 .. jp0 + njp - 1 (each 16 heads x 16 latent coordinates as
// 64 lanes x 4) by a workgroup of four waves.  The (max, sum) statistics are
// reduced once; then, per value tile, wave w sums splits w, w + 4, ..., and
// the four sums are added in a fixed order.  The first kMergePre partial tiles
// of each value tile are loaded ahead (before the statistics pass for the
// first, during the previous tile's reduction for the others).
constexpr int kMergeWaves = 4;
constexpr int kMergePre = 16;

// Where the partials of one (request, head tile) are: S splits, each a
// 16 x 512 fp32 tile in the accumulator's order (po, f4 units) and 16
// (max, sum) pairs (ml), consecutive splits po_stride / ml_stride apart.
struct MergeSrc {
  const f4 *po;
  int64_t po_stride;
  const float2 *ml;
  int ml_stride;
  int S;
};

__device__ void merge_tiles(const DecodeArgs &A, int jp0, int njp, int64_t orow, const MergeSrc &src,
                            float (*wts)[16], float (*red_m)[16], float (*red_l)[16], f4 (*part)[64]) {
  const int S = src.S;
  const float2 *ml = src.ml;
  const int mls = src.ml_stride;
  const int tid = threadIdx.x;
  const int h = tid & 15, st = tid >> 4;
  const int lane = tid & 63, grp = tid >> 6, hh = lane & 15;
  const int64_t ps = src.po_stride;
  // Thread (h, st) takes the (max, sum) of splits st, st + 16, ...; the first
  // kMlKeep of them stay in registers for the second pass.  These loads go
  // out before the partial tiles, so the statistics wait only for them.
  // Indices past the last split load the last one (unused), so no load is
  // followed at once by a select that would wait for it.  S >= 1.
  constexpr int kMlKeep = 4;
  float2 mlv[kMlKeep];
#pragma unroll
  for (int u = 0; u < kMlKeep; ++u) mlv[u] = ml[min(st + 16 * u, S - 1) * mls + h];
  f4 pre[kMergePre];
  auto prefetch = [&](int jp) {
    const f4 *po = src.po + jp * 64 + lane;
#pragma unroll
    for (int u = 0; u < kMergePre; ++u) pre[u] = po[(int64_t)min(grp + kMergeWaves * u, S - 1) * ps];
  };
  prefetch(jp0);
  {
    // Max per head over the splits.
    float m = kNegInf;
#pragma unroll
    for (int u = 0; u < kMlKeep; ++u)
      if (st + 16 * u < S) m = fmaxf(m, mlv[u].x);
    for (int s = st + 16 * kMlKeep; s < S; s += 16) m = fmaxf(m, ml[s * mls + h].x);
    red_m[st][h] = m;
  }
  __syncthreads();
  {
    float M = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) M = fmaxf(M, red_m[i][h]);
    const float Mc = fmaxf(M, -1e30f);  // 0 weights for empty splits
    float l = 0.f;
#pragma unroll
    for (int u = 0; u < kMlKeep; ++u) {
      const int s = st + 16 * u;
      if (s < S) {
        const float w = __builtin_amdgcn_exp2f(mlv[u].x - Mc);
        wts[s][h] = w;
        l += w * mlv[u].y;
      }
    }
    for (int s = st + 16 * kMlKeep; s < S; s += 16) {
      const float2 v = ml[s * mls + h];
      const float w = __builtin_amdgcn_exp2f(v.x - Mc);
      wts[s][h] = w;
      l += w * v.y;
    }
    red_l[st][h] = l;
  }
  __syncthreads();
  float L = 0.f, Mh = kNegInf;
  if (grp == 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) L += red_l[i][hh];
#pragma unroll
    for (int i = 0; i < 16; ++i) Mh = fmaxf(Mh, red_m[i][hh]);
  }
  // L = 0: no tokens (out 0, lse -inf); L NaN: a split's partial is marked
  // lost (out and lse NaN).
  const float inv = L == 0.f ? 0.f : 1.f / L;
  float *o = A.out + (orow + hh) * RLQ_DC;
  for (int t = 0; t < njp; ++t) {
    const int jp = jp0 + t;
    const f4 *po = src.po + jp * 64 + lane;
    f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kMergePre; ++u) {
      const int s = grp + kMergeWaves * u;
      if (s < S) acc += wts[s][hh] * pre[u];
    }
    int s = grp + kMergeWaves * kMergePre;
    for (; s + 7 * kMergeWaves < S; s += 8 * kMergeWaves) {
      f4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = po[(int64_t)(s + kMergeWaves * u) * ps];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += wts[s + kMergeWaves * u][hh] * v[u];
    }
    for (; s < S; s += kMergeWaves) acc += wts[s][hh] * po[(int64_t)s * ps];
    if (t + 1 < njp) prefetch(jp + 1);
    part[grp][lane] = acc;
    __syncthreads();
    if (grp == 0) {
      const f4 sum = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[value_coord(jp, 4 * (lane >> 4) + i)] = sum[i] * inv;
      if (A.lse != nullptr && jp == 0 && lane < 16)
        A.lse[orow + lane] =
            L == 0.f ? kNegInf : (Mh + log2f(L) - kBias) * 0.69314718055994531f;
    }
    if (t + 1 < njp) __syncthreads();  // part is rewritten by the next tile
  }
}

// The same merge for njp (2 .. kMergeMaxTiles) value tiles at once, for few
// splits: wave w sums splits w, w + 4, ... of every tile in one pass (all of
// a split's tile loads in flight together), the four sums meet in LDS once,
// and wave w writes tiles w, w + 4, ...
constexpr int kMergeMaxTiles = 8;

__device__ void merge_tiles_multi(const DecodeArgs &A, int jp0, int njp, int64_t orow, const MergeSrc &src,
                                  float (*wts)[16], float (*red_m)[16], float (*red_l)[16],
                                  f4 (*part)[kMergeWaves][64]) {
  const int S = src.S;
  const float2 *ml = src.ml;
  const int mls = src.ml_stride;
  const int tid = threadIdx.x;
  const int h = tid & 15, st = tid >> 4;
  const int lane = tid & 63, grp = tid >> 6, hh = lane & 15;
  const int64_t ps = src.po_stride;
  const f4 *po = src.po + jp0 * 64 + lane;
  {
    float m = kNegInf;
    for (int s = st; s < S; s += 16) m = fmaxf(m, ml[s * mls + h].x);
    red_m[st][h] = m;
  }
  // The first split's tiles of this wave are loaded while the statistics are
  // reduced.
  f4 v[kMergeMaxTiles];
  const int s0 = min(grp, S - 1);
#pragma unroll
  for (int t = 0; t < kMergeMaxTiles; ++t)
    if (t < njp) v[t] = po[(int64_t)s0 * ps + t * 64];
  __syncthreads();
  {
    float M = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) M = fmaxf(M, red_m[i][h]);
    const float Mc = fmaxf(M, -1e30f);  // 0 weights for empty splits
    float l = 0.f;
    for (int s = st; s < S; s += 16) {
      const float2 x = ml[s * mls + h];
      const float w = __builtin_amdgcn_exp2f(x.x - Mc);
      wts[s][h] = w;
      l += w * x.y;
    }
    red_l[st][h] = l;
  }
  __syncthreads();
  f4 acc[kMergeMaxTiles];
#pragma unroll
  for (int t = 0; t < kMergeMaxTiles; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
  for (int s = grp; s < S; s += kMergeWaves) {
    const float w = wts[s][hh];
#pragma unroll
    for (int t = 0; t < kMergeMaxTiles; ++t)
      if (t < njp) acc[t] += w * v[t];
    const int sn = s + kMergeWaves;
    if (sn < S) {
#pragma unroll
      for (int t = 0; t < kMergeMaxTiles; ++t)
        if (t < njp) v[t] = po[(int64_t)sn * ps + t * 64];
    }
  }
#pragma unroll
  for (int t = 0; t < kMergeMaxTiles; ++t)
    if (t < njp) part[t][grp][lane] = acc[t];
  __syncthreads();
  float L = 0.f, Mh = kNegInf;
#pragma unroll
  for (int i = 0; i < 16; ++i) L += red_l[i][hh];
#pragma unroll
  for (int i = 0; i < 16; ++i) Mh = fmaxf(Mh, red_m[i][hh]);
  // L = 0: no tokens (out 0, lse -inf); L NaN: a split's partial is marked
  // lost (out and lse NaN).
  const float inv = L == 0.f ? 0.f : 1.f / L;
  float *o = A.out + (orow + hh) * RLQ_DC;
  for (int t = grp; t < njp; t += kMergeWaves) {
    const int jp = jp0 + t;
    const f4 sum = (part[t][0][lane] + part[t][1][lane]) + (part[t][2][lane] + part[t][3][lane]);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[value_coord(jp, 4 * (lane >> 4) + i)] = sum[i] * inv;
  }
  if (A.lse != nullptr && jp0 == 0 && tid < 16)
    A.lse[orow + tid] = L == 0.f ? kNegInf : (Mh + log2f(L) - kBias) * 0.69314718055994531f;
}

}  // namespace
}  // namespace rlq
