// Read side: absorbed-MLA decode attention over the paged 2-bit cache.
// RoLaQ paper: §2.1 (one content latent serves keys and values, BF16 RoPE
// key), §3.2 (reconstruction = group mean + scale * gain * level), §3.3
// (read-side rotation folded into the absorbed projections), §4.1 / §A.3
// (sink and recent tokens kept in BF16), Fig. 1a / Fig. 3a.
//
// Split-KV.  Workgroup (split, request, head group) walks a page-aligned
// token range one 64-token page at a time with 4 waves:
//  * score phase - wave w owns token tile w (16 tokens) of the page.  Each
//    lane loads, for one token, two 16-byte runs of code words, the (mean,
//    scale) pairs of the two groups those words belong to, and 32 bytes of
//    the RoPE key.  A per-(token, group) table of the four fp16 values
//    mu + s*g*{-b,-a,+a,+b} (rounded once from fp32) is applied to the codes
//    with byte permutes (v_perm_b32), giving the fp16 c_hat operand with no
//    per-coordinate arithmetic.  Scores S^T[token, head] = c_hat.q_c +
//    k_R.q_R run on MFMA (16x16x32 fp16 content part, 16x16x32 bf16 RoPE
//    part) in a contraction order chosen so every lane's operand comes
//    straight from the code words it loaded; the absorbed query is laid out
//    in the same order once per workgroup.  c_hat also goes to LDS (1 KB per
//    token) and the scores to a small LDS array.
//  * value phase - after one barrier every wave reads the 64 scores of each
//    head, updates the online softmax (identical on all waves), and
//    accumulates O^T[latent, head] += c_hat^T P^T for its own quarter of the
//    512 latent coordinates, reading c_hat^T with the gfx950 LDS transpose
//    load (ds_read_b64_tr_b16).  P (times 2^15, to stay in fp16's normal
//    range) never leaves registers.
// The last split index of a request (when protection buffers are given)
// covers the BF16 sink/recent tokens with the same two phases; the other
// splits mask those tokens out.  A second kernel merges the per-split
// partials (LSE merge) and restores the natural coordinate order.

#include <math.h>

#include "rlq_internal.h"

namespace rlq {
namespace {

typedef short s4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s4 lds_s4;

constexpr float kNegInf = -__builtin_inff();
constexpr int kPageTok = 64;                       // tokens per iteration (one page)
constexpr int kTileBytes = kTile * RLQ_DC * 2;     // 16 KB fp16 c_hat per 16-token tile
constexpr int kChatBytes = 4 * kTileBytes;         // 64 KB per page
constexpr int kScoreBytes = 4 * 64 * 16;           // 4 tiles x 64 lanes x f4 scores
constexpr int kPBytes = 4 * 64 * 8;                // 4 tiles x 64 lanes x 4 fp16 P
constexpr int kLdsBytes = kChatBytes + kScoreBytes + kPBytes + 4 * kMaxSplitPages;
// Workgroups resident at once: 2 per CU (LDS: 2 x 71 KB of 160 KB) x 256 CUs.
constexpr int kResidentWorkgroups = 512;

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
// The xor keeps both the 16-byte writes and the transposed 8-byte reads of
// the value phase free of bank conflicts.
__device__ __host__ constexpr int chat_slot(int k, int g, int r) {
  return (16 * g + r) ^ (4 * (k & 1));
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

// Reductions over the 4 lane groups sharing lane & 15 (xor 16, xor 32).
__device__ inline float max_over_groups(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float sum_over_groups(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Table of one (token, group): low bytes and high bytes of the four fp16
// values, so v_perm_b32 can look both up with 2-bit selectors.
struct Lut {
  uint32_t lo, hi;
};
__device__ inline Lut make_lut(float mu, float s, float gain, float a, float b, bool valid) {
  const float sg = s * gain;
  const uint32_t p01 = h16(mu - sg * b) | (h16(mu - sg * a) << 16);
  const uint32_t p23 = h16(mu + sg * a) | (h16(mu + sg * b) << 16);
  Lut l;
  l.lo = valid ? __builtin_amdgcn_perm(p23, p01, 0x06040200u) : 0u;
  l.hi = valid ? __builtin_amdgcn_perm(p23, p01, 0x07050301u) : 0u;
  return l;
}

// Codes 2h, 2h+4, 2h+8, 2h+12, 2h+1, 2h+5, 2h+9, 2h+13 of word w as eight
// fp16 values (operand slots 0..7).
__device__ inline u4 decode8(uint32_t w, int h, const Lut &l) {
  const uint32_t y0 = (w >> (4 * h)) & 0x03030303u;
  const uint32_t y1 = (w >> (4 * h + 2)) & 0x03030303u;
  const uint32_t lo0 = __builtin_amdgcn_perm(0u, l.lo, y0);
  const uint32_t hi0 = __builtin_amdgcn_perm(0u, l.hi, y0);
  const uint32_t lo1 = __builtin_amdgcn_perm(0u, l.lo, y1);
  const uint32_t hi1 = __builtin_amdgcn_perm(0u, l.hi, y1);
  u4 r;
  r[0] = __builtin_amdgcn_perm(hi0, lo0, 0x05010400u);
  r[1] = __builtin_amdgcn_perm(hi0, lo0, 0x07030602u);
  r[2] = __builtin_amdgcn_perm(hi1, lo1, 0x05010400u);
  r[3] = __builtin_amdgcn_perm(hi1, lo1, 0x07030602u);
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

// What one lane loads for its token of the current page.
struct TileLoad {
  u4 cw0, cw1;       // code words [4q0, 4q0+4) and [4q0+8, 4q0+12)
  float2 mu, sd;     // (mean, scale) of groups 2*(g>>1) and 2*(g>>1)+1
  u4 rp0, rp1;       // RoPE key elements [16g, 16g+16)
};

__device__ inline void load_tile(const DecodeArgs &A, int32_t page, int r16, int g4, int w,
                                 TileLoad &L) {
  const int q0 = 4 * (g4 >> 1) + (g4 & 1);
  const int64_t slot = (int64_t)page * RLQ_PAGE + w * kTile + r16;
  const uint32_t *cw = A.codes + slot * RLQ_WORDS + 4 * q0;
  L.cw0 = *(const u4 *)cw;
  L.cw1 = *(const u4 *)(cw + 8);
  const float *m = A.meta + slot * 8 + 2 * (g4 >> 1);
  L.mu = *(const float2 *)m;
  L.sd = *(const float2 *)(m + 4);
  const uint16_t *rp = A.rope + slot * RLQ_DR + 16 * g4;
  L.rp0 = *(const u4 *)rp;
  L.rp1 = *(const u4 *)(rp + 8);
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

__global__ __launch_bounds__(kDecodeThreads, 2) void decode_split_kernel(DecodeArgs A) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // Grid x: [protected-token workgroup if any] then the ordinary splits, so
  // the short protected workgroups are dispatched first.
  const int part = blockIdx.x, b = blockIdx.y, hg = blockIdx.z;
  const int sp = part - A.prot;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int HG = A.heads >> 4;
  const int ctx = A.ctx_lens[b];
  const Protect pr = protect_range(A, ctx);
  const bool prot_wg = sp < 0;  // the BF16 sink/recent tokens
  // Token index range of this workgroup: positions for ordinary splits,
  // indices into the protected list for the protected one.
  int t_begin, t_end;
  if (prot_wg) {
    t_begin = 0;
    t_end = pr.ns + pr.nr;
  } else {
    t_begin = sp * A.tokens_per_split;
    t_end = min(ctx, t_begin + A.tokens_per_split);
  }
  const int u_lo = pr.ns, u_hi = ctx - pr.nr;  // unprotected positions

  // ---- absorbed query of 16 heads, staged through LDS into operand order.
  {
    const uint16_t *qsrc = A.q_c + ((int64_t)b * A.heads + hg * 16) * RLQ_DC;
    for (int c = threadIdx.x; c < 16 * RLQ_DC / 8; c += kDecodeThreads)
      *(u4 *)(smem + 16 * c) = *(const u4 *)(qsrc + 8 * c);
  }
  __syncthreads();
  half8 qB[16];
  {
    const uint16_t *qs = (const uint16_t *)smem + r16 * RLQ_DC;
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        qB[k][j] = (_Float16)bf16_to_f32(qs[coord_of(k, g4, j)]);
  }
  bf16x8 qrB[2];
  {
    const uint16_t *qr = A.q_r + ((int64_t)b * A.heads + hg * 16 + r16) * RLQ_DR + 16 * g4;
    qrB[0] = __builtin_bit_cast(bf16x8, *(const u4 *)qr);
    qrB[1] = __builtin_bit_cast(bf16x8, *(const u4 *)(qr + 8));
  }
  __syncthreads();

  float m_run = kNegInf, l_run = 0.f;
  f4 O[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) O[i] = f4{0.f, 0.f, 0.f, 0.f};

  // Transposed-read offset of this lane in the value phase: lane p = r16 of
  // lane group g4 supplies token row 4*g4 + p/4 and coordinates q = p % 4.
  const int va = (r16 & 3) >> 1;
  const int vrd = 1024 * va + 16 * ((4 * g4 + (r16 >> 2)) ^ (4 * va)) + 8 * (r16 & 1);
  f4 *score_lds = (f4 *)(smem + kChatBytes);
  u2 *p_lds = (u2 *)(smem + kChatBytes + kScoreBytes);

  auto page_of = [&](int t) -> int32_t {
    return A.block_table[(int64_t)b * A.max_pages + (t >> 6)];
  };
  // Page ids of this split, staged once in LDS so that the loads of a page
  // never wait on a block-table read.
  const int p_first = t_begin >> 6;
  const int n_pages = prot_wg ? 0 : (t_end - t_begin + kPageTok - 1) / kPageTok;
  int32_t *pid_lds = (int32_t *)(smem + kChatBytes + kScoreBytes + kPBytes);
  for (int i = threadIdx.x; i < n_pages; i += kDecodeThreads)
    pid_lds[i] = A.block_table[(int64_t)b * A.max_pages + p_first + i];
  __syncthreads();
  auto pid_at = [&](int n) -> int32_t { return __builtin_amdgcn_readfirstlane(pid_lds[n]); };

  // One page: score phase on tile `wave`, barrier, value phase, barrier.
  auto process_page = [&](const TileLoad &cur, int c0) {
    const int trow = c0 + wave * kTile + r16;  // operand row of this lane
    unsigned char *tl = smem + wave * kTileBytes;
    f4 acc = f4{0.f, 0.f, 0.f, 0.f};
    if (!prot_wg) {
      const bool valid = trow < t_end && trow >= u_lo && trow < u_hi;
      const Lut la = make_lut(cur.mu.x, cur.sd.x, A.gain, A.level_inner, A.level_outer, valid);
      const Lut lb = make_lut(cur.mu.y, cur.sd.y, A.gain, A.level_inner, A.level_outer, valid);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const u4 &run = (k < 8) ? cur.cw0 : cur.cw1;
        const u4 av = decode8(run[(k >> 1) & 3], k & 1, (k < 8) ? la : lb);
        *(u4 *)(tl + k * 1024 + 16 * chat_slot(k, g4, r16)) = av;
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, av), qB[k], acc, 0, 0, 0);
        // Keep each decoded operand's live range to its own K-step.
        __builtin_amdgcn_sched_barrier(0);
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.rp0), qrB[0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.rp1), qrB[1], acc, 0, 0, 0);
    } else {
      // Protected list index v -> position and BF16 source row.
      const bool valid = trow < t_end;
      const int pos = (trow < pr.ns) ? trow : (ctx - pr.nr + (trow - pr.ns));
      const uint16_t *row = nullptr;
      if (valid)
        row = (trow < pr.ns) ? A.sink + ((int64_t)b * A.n_sink + pos) * RLQ_DC
                             : A.recent + ((int64_t)b * A.n_recent + pos % A.n_recent) * RLQ_DC;
      const int q0 = 4 * (g4 >> 1) + (g4 & 1);
      u4 rp0 = u4{0, 0, 0, 0}, rp1 = u4{0, 0, 0, 0};
      if (valid) {
        const int64_t slot = (int64_t)page_of(pos) * RLQ_PAGE + (pos & 63);
        rp0 = *(const u4 *)(A.rope + slot * RLQ_DR + 16 * g4);
        rp1 = *(const u4 *)(A.rope + slot * RLQ_DR + 16 * g4 + 8);
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        u4 av = u4{0, 0, 0, 0};
        if (valid) {
          const int word = 4 * (q0 + 2 * (k >> 3)) + ((k >> 1) & 3);
          const u4 w0 = *(const u4 *)(row + 16 * word);
          const u4 w1 = *(const u4 *)(row + 16 * word + 8);
          av = convert8(w0, w1, k & 1);
        }
        *(u4 *)(tl + k * 1024 + 16 * chat_slot(k, g4, r16)) = av;
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, av), qB[k], acc, 0, 0, 0);
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, rp0), qrB[0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, rp1), qrB[1], acc, 0, 0, 0);
    }
    // acc[i] = score of token row 4*g4 + i of tile `wave`, head r16.
    const int vlo = prot_wg ? 0 : u_lo;
    const int vhi = prot_wg ? t_end : min(t_end, u_hi);
    if (c0 >= vlo && c0 + kPageTok <= vhi) {
      acc *= A.scale_log2;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = c0 + wave * kTile + 4 * g4 + i;
        acc[i] = (t >= vlo && t < vhi) ? acc[i] * A.scale_log2 : kNegInf;
      }
    }
    score_lds[wave * 64 + lane] = acc;
    __syncthreads();

    // ---------------- softmax: all waves agree on the running max; each
    // wave exponentiates its own tile and shares fp16 P through LDS.
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f4 sv = score_lds[t * 64 + lane];
      mx = fmaxf(mx, fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
    }
    mx = max_over_groups(mx);
    const float m_new = fmaxf(m_run, mx);
    if (m_new > m_run) {  // identical on all lanes of a head
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run = -inf
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) O[i] *= alpha;
      m_run = m_new;
    }
    // P carries 2^15 (fp16 headroom); while no finite score has been seen the
    // clamp keeps exp2(-inf - mb) at 0 instead of NaN.
    const float mb = fmaxf(m_run, -1e30f) - 15.f;
    {
      const half2v p01 = __builtin_convertvector(
          (float2v){__builtin_amdgcn_exp2f(acc[0] - mb), __builtin_amdgcn_exp2f(acc[1] - mb)}, half2v);
      const half2v p23 = __builtin_convertvector(
          (float2v){__builtin_amdgcn_exp2f(acc[2] - mb), __builtin_amdgcn_exp2f(acc[3] - mb)}, half2v);
      l_run = __builtin_amdgcn_fdot2(p01, (half2v){1.0f16, 1.0f16}, l_run, false);
      l_run = __builtin_amdgcn_fdot2(p23, (half2v){1.0f16, 1.0f16}, l_run, false);
      p_lds[wave * 64 + lane] = u2{__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)};
    }
    __syncthreads();
    half8 PB[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const u2 a = p_lds[(2 * kk) * 64 + lane];
      const u2 c = p_lds[(2 * kk + 1) * 64 + lane];
      PB[kk] = __builtin_bit_cast(half8, u4{a[0], a[1], c[0], c[1]});
    }
#pragma unroll
    for (int jl = 0; jl < 8; ++jl) {
      const int jp = 8 * wave + jl;
      const int cofs = 2048 * (jp >> 2) + 256 * (jp & 3);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const unsigned char *base = smem + (2 * kk) * kTileBytes + cofs + vrd;
        const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)base);
        const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(base + kTileBytes));
        const half8 av = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        O[jl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, PB[kk], O[jl], 0, 0, 0);
      }
    }
    __syncthreads();
  };

  if (prot_wg) {
    TileLoad none{};
    for (int c0 = t_begin; c0 < t_end; c0 += kPageTok) process_page(none, c0);
  } else {
    // Two load buffers used alternately: the loads of page n+1 are in flight
    // while page n is processed, with no register copies between them.
    // Three load buffers in a ring: while page n is processed the loads of
    // pages n+1 and n+2 are in flight.  Loads are issued unconditionally (past
    // the end the last page is loaded again, from L2) so the loop body has one
    // straight path and the compiler's wait counts cover only the buffer
    // being consumed.
    TileLoad buf0, buf1, buf2;
    const int last = n_pages - 1;
    if (n_pages > 0) {
      load_tile(A, pid_at(0), r16, g4, wave, buf0);
      load_tile(A, pid_at(min(1, last)), r16, g4, wave, buf1);
    }
    for (int n = 0; n < n_pages; n += 3) {
      load_tile(A, pid_at(min(n + 2, last)), r16, g4, wave, buf2);
      process_page(buf0, t_begin + n * kPageTok);
      if (n + 1 >= n_pages) break;
      load_tile(A, pid_at(min(n + 3, last)), r16, g4, wave, buf0);
      process_page(buf1, t_begin + (n + 1) * kPageTok);
      if (n + 2 >= n_pages) break;
      load_tile(A, pid_at(min(n + 4, last)), r16, g4, wave, buf1);
      process_page(buf2, t_begin + (n + 2) * kPageTok);
    }
  }

  // ---- partial of this workgroup: each wave writes its quarter of O; the
  // sum of P is spread over the waves (each summed its own tiles).
  l_run = sum_over_groups(l_run);
  float *l_lds = (float *)(smem + kChatBytes);  // free after the last barrier
  if (g4 == 0) l_lds[wave * 16 + r16] = l_run;
  __syncthreads();
  const int64_t pidx = ((int64_t)b * HG + hg) * (A.splits + A.prot) + part;
  f4 *po = (f4 *)(A.part_o + pidx * kPartialFloats);
#pragma unroll
  for (int jl = 0; jl < 8; ++jl) po[(8 * wave + jl) * 64 + lane] = O[jl];
  if (wave == 0 && g4 == 0) {
    const float l_all = (l_lds[r16] + l_lds[16 + r16]) + (l_lds[32 + r16] + l_lds[48 + r16]);
    A.part_ml[pidx * 32 + 2 * r16] = m_run;
    A.part_ml[pidx * 32 + 2 * r16 + 1] = l_all;
  }
}

// LSE merge of the per-split partials of one (request, head group) for one
// value tile: 4 waves each sum a quarter of the splits with many loads in
// flight, then the quarters are added in a fixed order.
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs A) {
  __shared__ float wts[kMaxSplits + 1][16];
  __shared__ float red_m[16][16], red_l[16][16];
  __shared__ f4 part[4][64];
  const int jp = blockIdx.x;  // value tile 0..31
  const int bh = blockIdx.y;  // b * HG + hg
  const int HG = A.heads >> 4;
  const int b = bh / HG, hg = bh % HG;
  const int S = A.splits + A.prot;
  const float2 *ml = (const float2 *)(A.part_ml + (int64_t)bh * S * 32);
  const int tid = threadIdx.x;
  const int h = tid & 15, st = tid >> 4;
  // Max per head over the splits: thread (h, st) takes splits st, st+16, ...
  {
    float m = kNegInf;
#pragma unroll 4
    for (int s = st; s < S; s += 16) m = fmaxf(m, ml[s * 16 + h].x);
    red_m[st][h] = m;
  }
  __syncthreads();
  float M = kNegInf;
#pragma unroll
  for (int i = 0; i < 16; ++i) M = fmaxf(M, red_m[i][h]);
  {
    float l = 0.f;
#pragma unroll 4
    for (int s = st; s < S; s += 16) {
      const float2 v = ml[s * 16 + h];
      const float w = __builtin_amdgcn_exp2f(v.x - fmaxf(M, -1e30f));  // 0 for empty splits
      wts[s][h] = w;
      l += w * v.y;
    }
    red_l[st][h] = l;
  }
  __syncthreads();
  const int lane = tid & 63, grp = tid >> 6, hh = lane & 15;
  const f4 *po = (const f4 *)(A.part_o + (int64_t)bh * S * kPartialFloats) + jp * 64 + lane;
  f4 acc = f4{0.f, 0.f, 0.f, 0.f};
  constexpr int kStride = kPartialFloats / 4;
  int s = grp;
  for (; s + 28 < S; s += 32) {
    f4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = po[(int64_t)(s + 4 * u) * kStride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += wts[s + 4 * u][hh] * v[u];
  }
  for (; s < S; s += 4) acc += wts[s][hh] * po[(int64_t)s * kStride];
  part[grp][lane] = acc;
  __syncthreads();
  if (grp == 0) {
    float L = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) L += red_l[i][hh];
    float Mh = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) Mh = fmaxf(Mh, red_m[i][hh]);
    const f4 sum = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
    const float inv = L > 0.f ? 1.f / L : 0.f;
    float *o = A.out + ((int64_t)b * A.heads + hg * 16 + hh) * RLQ_DC;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[value_coord(jp, 4 * (lane >> 4) + i)] = sum[i] * inv;
    if (A.lse != nullptr && jp == 0 && lane < 16)
      A.lse[(int64_t)b * A.heads + hg * 16 + lane] =
          L > 0.f ? (Mh + log2f(L) - 15.f) * 0.69314718055994531f : kNegInf;
  }
}

}  // namespace

SplitPlan plan_splits(int32_t batch, int32_t heads, int32_t max_ctx_len) {
  // One round of workgroups that fills the GPU exactly: two per CU (256 CUs,
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
  // Callers reject contexts beyond kMaxSplits * kMaxSplitPages pages.
  if (tps > (int64_t)kMaxSplitPages * RLQ_PAGE) tps = (int64_t)kMaxSplitPages * RLQ_PAGE;
  return SplitPlan{(int32_t)tps, (int32_t)splits};
}

size_t decode_workspace_bytes(int32_t batch, int32_t heads, const SplitPlan &plan) {
  const size_t parts = (size_t)batch * (heads / 16) * (plan.splits + 1);
  return parts * (kPartialFloats + 32) * sizeof(float);
}

hipError_t launch_decode(const DecodeArgs &a, int32_t batch, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)decode_split_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int hg = a.heads / 16;
  hipLaunchKernelGGL(decode_split_kernel, dim3(a.splits + a.prot, batch, hg), dim3(kDecodeThreads),
                     kLdsBytes, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(32, batch * hg), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rlq
