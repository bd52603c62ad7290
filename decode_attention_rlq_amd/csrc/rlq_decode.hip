// Read side: absorbed-MLA decode attention over the paged 2-bit cache.
// RoLaQ paper: §2.1 (one content latent serves keys and values, BF16 RoPE
// key), §3.2 (reconstruction = group mean + scale * gain * level), §3.3
// (read-side rotation folded into the absorbed projections), Fig. 1a/3a.
//
// Split-KV: workgroup (split, request, head group) covers a page-aligned token
// range; its 4 waves take 32-token chunks in turn, each with its own online
// softmax state, merged through LDS at the end into one partial per
// workgroup; a second kernel merges the partials of all splits (LSE merge).
//
// Per chunk and wave:
//  * each lane loads, for one token, two 16-byte runs of code words, the
//    (mean, scale) pairs of the two groups those words belong to, and 32 bytes
//    of the RoPE key (all coalesced 8/16-byte loads);
//  * a per-(token, group) 4-entry fp16 table mu + s*g*{-b,-a,+a,+b} (rounded
//    once from fp32) is applied to the codes with byte permutes (v_perm_b32):
//    no per-coordinate multiply or conversion;
//  * scores S^T[token, head] = c_hat . q_c + k_R . q_R on MFMA
//    (16x16x32 fp16 for the content part, 16x16x32 bf16 for the RoPE part),
//    in an order of the 576 contraction coordinates chosen so that every lane
//    gets its operand straight from the code words it loaded; the absorbed
//    query is laid out in the same order once per workgroup;
//  * the fp16 c_hat tile also goes to LDS (1 KB per token) and is read back
//    transposed as the A operand of the value MFMA O^T[d, head] += c_hat^T P^T;
//    P (scaled by 2^15 to keep fp16 normal) never leaves registers.

#include <math.h>

#include "rlq_internal.h"

namespace rlq {
namespace {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr int kTileBytes = kTile * RLQ_DC * 2;      // 16 KB of fp16 per 16 tokens
constexpr int kWaveLds = 2 * kTileBytes;            // one 32-token chunk per wave
constexpr int kLdsBytes = kDecodeWaves * kWaveLds;  // 128 KB

// Contraction order of the content coordinates (shared by the query layout,
// the code decoding and the output mapping).  K-step k (0..15), lane group g
// (lane / 16) and slot j (0..7) of the 16x16x32 MFMA operand cover latent
// coordinate  16 * word(k, g) + sub(j, k & 1)  where
//   word(k, g) = 4 * (q0(g) + 2 * (k >> 3)) + ((k >> 1) & 3),
//   q0(g)     = 4 * (g >> 1) + (g & 1)          (16-byte run of code words),
//   sub(j, h) = 2h + (j >> 2) + 4 * (j & 3)     (code within the word).
// A lane therefore reads code words [4 q0, 4 q0 + 4) and [4 q0 + 8, 4 q0 + 12)
// of its token: groups 2*(g>>1) (k < 8) and 2*(g>>1)+1 (k >= 8).
__device__ __host__ constexpr int coord_of(int k, int g, int j) {
  return 16 * (4 * ((4 * (g >> 1) + (g & 1)) + 2 * (k >> 3)) + ((k >> 1) & 3)) +
         2 * (k & 1) + (j >> 2) + 4 * (j & 3);
}

// fp16 bit pattern, round to nearest even.
__device__ inline uint32_t h16(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// 4-entry reconstruction table of one (token, group): bytes split into a
// low-byte table and a high-byte table so that v_perm_b32 can index both with
// the 2-bit codes.
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

// Decode codes 2h, 2h+4, 2h+8, 2h+12, 2h+1, 2h+5, 2h+9, 2h+13 of word w into
// eight fp16 values (slot order j = 0..7 of the MFMA operand).
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

__device__ inline float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

struct ChunkLoads {
  u4 cw[2][2];   // [tile][run] code words
  float mu[2][2], sd[2][2];  // [tile][group A/B]
  u4 rp[2][2];   // [tile][k-step] RoPE key (bf16)
};

__device__ inline void load_chunk(const DecodeArgs &A, int b, int c0, int r16, int g4,
                                  ChunkLoads &L) {
  const int32_t page = A.block_table[(int64_t)b * A.max_pages + (c0 >> 6)];
  const int q0 = 4 * (g4 >> 1) + (g4 & 1);
  const int ga = 2 * (g4 >> 1);
#pragma unroll
  for (int tile = 0; tile < 2; ++tile) {
    const int64_t slot = (int64_t)page * RLQ_PAGE + (c0 & 63) + tile * kTile + r16;
    const uint32_t *cw = A.codes + slot * RLQ_WORDS + 4 * q0;
    L.cw[tile][0] = *(const u4 *)cw;
    L.cw[tile][1] = *(const u4 *)(cw + 8);
    const float *m = A.meta + slot * 8;
    const float2 mu = *(const float2 *)(m + ga);
    const float2 sd = *(const float2 *)(m + 4 + ga);
    L.mu[tile][0] = mu.x; L.mu[tile][1] = mu.y;
    L.sd[tile][0] = sd.x; L.sd[tile][1] = sd.y;
    const uint16_t *rp = A.rope + slot * RLQ_DR + 16 * g4;
    L.rp[tile][0] = *(const u4 *)rp;
    L.rp[tile][1] = *(const u4 *)(rp + 8);
  }
}

__global__ __launch_bounds__(kDecodeThreads, 1) void decode_split_kernel(DecodeArgs A) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int sp = blockIdx.x, b = blockIdx.y, hg = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int HG = A.heads >> 4;
  const int ctx = A.ctx_lens[b];
  const int t_begin = sp * A.tokens_per_split;
  const int t_end = min(ctx, t_begin + A.tokens_per_split);

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
      for (int j = 0; j < 8; ++j) qB[k][j] = (_Float16)bf16_to_f32(qs[coord_of(k, g4, j)]);
  }
  bf16x8 qrB[2];
  {
    const uint16_t *qr = A.q_r + ((int64_t)b * A.heads + hg * 16 + r16) * RLQ_DR + 16 * g4;
    qrB[0] = __builtin_bit_cast(bf16x8, *(const u4 *)qr);
    qrB[1] = __builtin_bit_cast(bf16x8, *(const u4 *)(qr + 8));
  }
  __syncthreads();

  unsigned char *wlds = smem + wave * kWaveLds;
  const bool protect = (A.sink != nullptr && A.n_sink > 0) || (A.recent != nullptr && A.n_recent > 0);

  float m_run = kNegInf, l_run = 0.f;
  f4 O[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) O[i] = f4{0.f, 0.f, 0.f, 0.f};

  // Value-pass LDS read offsets (see coord_of): lane (m = r16, tg = g4) reads
  // rows 4 tg + i of both tiles at byte 2 * (m & 7) of slot ((...) ^ a).
  const int va = r16 >> 3;
  const int vbase = 1024 * va + 2 * (r16 & 7) + 64 * g4;
  int voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = vbase + 16 * (i ^ va);

  ChunkLoads cur;
  int c0 = t_begin + wave * kChunk;
  if (c0 < t_end) load_chunk(A, b, c0, r16, g4, cur);
  for (; c0 < t_end; c0 += kDecodeWaves * kChunk) {
    ChunkLoads nxt;
    const int c1 = c0 + kDecodeWaves * kChunk;
    if (c1 < t_end) load_chunk(A, b, c1, r16, g4, nxt);

    const bool prot_chunk = protect && ((A.sink != nullptr && c0 < A.n_sink) ||
                                        (A.recent != nullptr && c0 + kChunk > ctx - A.n_recent));
    f4 S[2];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const int tpos = c0 + tile * kTile + r16;  // this lane's operand row
      const bool valid = tpos < t_end;
      const Lut la = make_lut(cur.mu[tile][0], cur.sd[tile][0], A.gain, A.level_inner, A.level_outer, valid);
      const Lut lb = make_lut(cur.mu[tile][1], cur.sd[tile][1], A.gain, A.level_inner, A.level_outer, valid);
      const uint16_t *prow = nullptr;
      if (prot_chunk && valid) {
        if (A.sink != nullptr && tpos < A.n_sink)
          prow = A.sink + ((int64_t)b * A.n_sink + tpos) * RLQ_DC;
        else if (A.recent != nullptr && tpos >= ctx - A.n_recent)
          prow = A.recent + ((int64_t)b * A.n_recent + tpos % A.n_recent) * RLQ_DC;
      }
      unsigned char *tl = wlds + tile * kTileBytes;
      f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const u4 &run = cur.cw[tile][k >> 3];
        const uint32_t w = run[(k >> 1) & 3];
        u4 av = decode8(w, k & 1, (k < 8) ? la : lb);
        if (prot_chunk && prow != nullptr) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float x0 = bf16_to_f32(prow[coord_of(k, g4, 2 * jj)]);
            const float x1 = bf16_to_f32(prow[coord_of(k, g4, 2 * jj + 1)]);
            av[jj] = h16(x0) | (h16(x1) << 16);
          }
        }
        *(u4 *)(tl + k * 1024 + ((lane ^ (k & 1)) << 4)) = av;
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, av), qB[k], acc, 0, 0, 0);
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.rp[tile][0]), qrB[0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.rp[tile][1]), qrB[1], acc, 0, 0, 0);
      // acc[i] = score of token c0 + 16 tile + 4 g4 + i for head r16.
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = c0 + tile * kTile + 4 * g4 + i;
        acc[i] = (t < t_end) ? acc[i] * A.scale_log2 : kNegInf;
      }
      S[tile] = acc;
    }

    // ---- online softmax for head r16 (all 4 lane groups agree on m).
    float mx = fmaxf(fmaxf(fmaxf(S[0][0], S[0][1]), fmaxf(S[0][2], S[0][3])),
                     fmaxf(fmaxf(S[1][0], S[1][1]), fmaxf(S[1][2], S[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    if (__any(m_new > m_run)) {
      const float alpha = (m_run == kNegInf) ? 0.f : exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 32; ++i) O[i] *= alpha;
      m_run = m_new;
    }
    // P^T operand: slots 0..3 = tile 0 rows 4 g4 + i, slots 4..7 = tile 1.
    const float mb = m_run - 15.f;  // P carries a 2^15 factor (fp16 headroom)
    uint32_t pw[4];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = exp2f(S[tile][i] - mb);
        l_run += p[i];
      }
      pw[2 * tile] = h16(p[0]) | (h16(p[1]) << 16);
      pw[2 * tile + 1] = h16(p[2]) | (h16(p[3]) << 16);
    }
    const half8 PB = __builtin_bit_cast(half8, u4{pw[0], pw[1], pw[2], pw[3]});

    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- value: O^T[16 latent coords of tile jp][head] += c_hat^T P^T.
    const uint16_t *vl = (const uint16_t *)wlds;
#pragma unroll
    for (int jp = 0; jp < 32; ++jp) {
      const int cofs = 2048 * (jp >> 2) + 256 * (jp & 3);
      half8 av;
#pragma unroll
      for (int tile = 0; tile < 2; ++tile)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          av[4 * tile + i] = __builtin_bit_cast(_Float16, vl[(voff[i] + cofs + tile * kTileBytes) >> 1]);
      O[jp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, PB, O[jp], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    if (c1 < t_end) cur = nxt;
  }

  // ---- merge the 4 waves through LDS into one partial per workgroup.
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  __syncthreads();
  float *mls = (float *)smem;  // [wave][16][2]
  if (g4 == 0) {
    mls[(wave * 16 + r16) * 2] = m_run;
    mls[(wave * 16 + r16) * 2 + 1] = l_run;
  }
  __syncthreads();
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, mls[(w * 16 + r16) * 2]);
  const float my_scale = (m_run == kNegInf) ? 0.f : exp2f(m_run - M);
  float Lsum = 0.f;
#pragma unroll
  for (int w = 0; w < kDecodeWaves; ++w) {
    const float mw = mls[(w * 16 + r16) * 2];
    Lsum += (mw == kNegInf) ? 0.f : exp2f(mw - M) * mls[(w * 16 + r16) * 2 + 1];
  }
  __syncthreads();
  f4 *ol = (f4 *)smem;  // [wave][32][64] f4
#pragma unroll
  for (int jp = 0; jp < 32; ++jp) ol[(wave * 32 + jp) * 64 + lane] = O[jp] * my_scale;
  __syncthreads();
  const int64_t pidx = ((int64_t)b * HG + hg) * A.splits + sp;
  f4 *po = (f4 *)(A.part_o + pidx * kPartialFloats);
  for (int e = threadIdx.x; e < 32 * 64; e += kDecodeThreads) {
    f4 s = ol[e];
#pragma unroll
    for (int w = 1; w < kDecodeWaves; ++w) s += ol[w * 32 * 64 + e];
    po[e] = s;
  }
  if (threadIdx.x < 16) {
    A.part_ml[pidx * 32 + 2 * threadIdx.x] = M;
    A.part_ml[pidx * 32 + 2 * threadIdx.x + 1] = Lsum;
  }
}

// Latent coordinate held in element (tile jp, lane l, row i) of a partial.
__device__ inline int out_coord(int jp, int l, int i) {
  const int m = 4 * (l >> 4) + i;
  const int k = 2 * (jp >> 2) + (m >> 3);
  return coord_of(k, jp & 3, m & 7);
}

__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs A) {
  __shared__ float w_s[256][16];
  __shared__ float tot[16], mmax[16];
  const int bh = blockIdx.y;  // b * HG + hg
  const int HG = A.heads >> 4;
  const int b = bh / HG, hg = bh % HG;
  const int S = A.splits;
  const float *ml = A.part_ml + (int64_t)bh * S * 32;
  if (threadIdx.x < 16) {
    const int h = threadIdx.x;
    float M = kNegInf;
    for (int s = 0; s < S; ++s) M = fmaxf(M, ml[s * 32 + 2 * h]);
    float L = 0.f;
    for (int s = 0; s < S; ++s) {
      const float ms = ml[s * 32 + 2 * h];
      const float w = (ms == kNegInf) ? 0.f : exp2f(ms - M);
      w_s[s][h] = w;
      L += w * ml[s * 32 + 2 * h + 1];
    }
    tot[h] = L;
    mmax[h] = M;
  }
  __syncthreads();
  const int e = blockIdx.x * 256 + threadIdx.x;  // f4 element: (jp, lane)
  const int jp = e >> 6, l = e & 63, h = l & 15;
  f4 acc = f4{0.f, 0.f, 0.f, 0.f};
  const f4 *po = (const f4 *)(A.part_o + (int64_t)bh * S * kPartialFloats);
  for (int s = 0; s < S; ++s) acc += w_s[s][h] * po[(int64_t)s * (kPartialFloats / 4) + e];
  const float L = tot[h];
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float *o = A.out + ((int64_t)b * A.heads + hg * 16 + h) * RLQ_DC;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[out_coord(jp, l, i)] = acc[i] * inv;
  if (A.lse != nullptr && e < 16) {
    A.lse[(int64_t)b * A.heads + hg * 16 + e] =
        L > 0.f ? (mmax[e] + log2f(L) - 15.f) * 0.69314718055994531f : kNegInf;
  }
}

}  // namespace

SplitPlan plan_splits(int32_t batch, int32_t heads, int32_t max_ctx_len) {
  // Aim for about two workgroups per CU (256 CUs) over the whole batch, in
  // whole pages, at most 256 splits per request.
  const int64_t hg = heads / 16;
  const int64_t total = (int64_t)batch * hg * (int64_t)(max_ctx_len > 0 ? max_ctx_len : 1);
  int64_t tps = (total + 511) / 512;
  tps = ((tps + RLQ_PAGE - 1) / RLQ_PAGE) * RLQ_PAGE;
  if (tps < 2 * RLQ_PAGE) tps = 2 * RLQ_PAGE;
  int64_t splits = (max_ctx_len + tps - 1) / tps;
  if (splits > 256) {
    tps = ((max_ctx_len + 255) / 256 + RLQ_PAGE - 1) / RLQ_PAGE * RLQ_PAGE;
    splits = (max_ctx_len + tps - 1) / tps;
  }
  if (splits < 1) splits = 1;
  return SplitPlan{(int32_t)tps, (int32_t)splits};
}

size_t decode_workspace_bytes(int32_t batch, int32_t heads, const SplitPlan &plan) {
  const size_t parts = (size_t)batch * (heads / 16) * plan.splits;
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
  hipLaunchKernelGGL(decode_split_kernel, dim3(a.splits, batch, hg), dim3(kDecodeThreads),
                     kLdsBytes, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(kPartialFloats / 4 / 256, batch * hg), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace rlq
