// Write side: rotate -> standardize -> threshold -> pack, plus RoPE copy and
// BF16 sink/recent protection.  RoLaQ paper: §3.3 (rotated latents stored as
// 2-bit codes, rotation fixed while serving), §3.2 (four-level assignment by
// the per-layer threshold), §A.3 (group 128 with two fp32 statistics, BF16
// RoPE key, protected tokens keep BF16 content), §4.1 (sink + recent tokens).
//
// One workgroup handles 64 consecutive new tokens; wave w owns coordinate
// group w (128 outputs).  The rotation z^T = R c^T runs on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16) with fp32 accumulation: A = rows of R (M =
// outputs), B = token latents (N = tokens).  In the accumulator layout each
// lane holds, for one token, outputs 16*mt + 4*(lane/16) + i of every 16-row
// tile mt, which lets the statistics follow the fixed adjacent-pair tree:
// two in-lane levels, two cross-lane levels (xor 16, xor 32), three in-lane
// levels across tiles.

#include "rlq_internal.h"

// The statistics must be plain fp32 adds and multiplies in a fixed order; no
// contraction into FMA anywhere in this file.
#pragma clang fp contract(off)

namespace rlq {
namespace {

constexpr int kAppTokens = 64;
// Up to this many new tokens the few-token kernel is used.
constexpr int64_t kSmallTokens = 4096;

__device__ inline uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ inline int find_request(const int32_t *cu, int batch, int64_t tok) {
  int lo = 0, hi = batch;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if ((int64_t)cu[mid] <= tok) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ inline float tree8(const float (&v)[8]) {
  return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
}

// Sum over one 128-coordinate group held as acc[mt][i] by the 4 lanes
// {n, n+16, n+32, n+48}: the adjacent-pair tree, bit-identical on all 4 lanes.
__device__ inline float group_tree_sum(const float (&x)[8][4]) {
  float s16[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    float s4 = (x[mt][0] + x[mt][1]) + (x[mt][2] + x[mt][3]);
    float s8 = s4 + __shfl_xor(s4, 16, 64);
    s16[mt] = s8 + __shfl_xor(s8, 32, 64);
  }
  return tree8(s16);
}

// Statistics, codes and stores for one token and one group: z[mt][i] is
// output 16*mt + 4*kg + i of group G; the four lanes {n, n+16, n+32, n+48}
// hold the whole group.  All 64 lanes must call it (cross-lane sums).
__device__ inline void finish_group(const AppendArgs &a, const float (&z)[8][4], int64_t tok,
                                    int G, int kg) {
  const bool valid = tok < a.n_tokens;
  const float mu = group_tree_sum(z) * 0.0078125f;
  float d[8][4], sq[8][4];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      d[mt][i] = z[mt][i] - mu;
      sq[mt][i] = d[mt][i] * d[mt][i];
    }
  const float s = sqrtf(group_tree_sum(sq) * 0.0078125f);
  const float t = a.tau * s;

  uint32_t word[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    uint32_t byte = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = d[mt][i];
      const uint32_t c = (uint32_t)(x >= -t) + (uint32_t)(x >= 0.f) + (uint32_t)(x >= t);
      byte |= c << (2 * i);
    }
    uint32_t w = byte << (8 * kg);
    w |= (uint32_t)__shfl_xor((int)w, 16, 64);
    w |= (uint32_t)__shfl_xor((int)w, 32, 64);
    word[mt] = w;
  }
  if (!valid) return;

  const int b = find_request(a.cu_seqlens, a.batch, tok);
  const int64_t pos = (int64_t)a.start_pos[b] + (tok - a.cu_seqlens[b]);
  const int32_t page = a.block_table[(int64_t)b * a.max_pages + (pos >> 6)];
  const int64_t slot = (int64_t)page * RLQ_PAGE + (pos & 63);

  // Lane group kg stores code words 2kg, 2kg+1 of this group.
  *(u2 *)(a.codes + slot * RLQ_WORDS + 8 * G + 2 * kg) = u2{word[2 * kg], word[2 * kg + 1]};
  if (kg == 0) {
    a.meta[slot * 8 + G] = mu;
    a.meta[slot * 8 + 4 + G] = s;
  }
  if (a.z_debug != nullptr) {
    float *dst = a.z_debug + tok * RLQ_DC + G * RLQ_GROUP + 4 * kg;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) *(f4 *)(dst + 16 * mt) = f4{z[mt][0], z[mt][1], z[mt][2], z[mt][3]};
  }
  const int64_t new_len = (int64_t)a.start_pos[b] + (a.cu_seqlens[b + 1] - a.cu_seqlens[b]);
  uint16_t *prot[2] = {nullptr, nullptr};
  if (a.sink != nullptr && pos < a.n_sink)
    prot[0] = a.sink + ((int64_t)b * a.n_sink + pos) * RLQ_DC;
  if (a.recent != nullptr && pos >= new_len - a.n_recent)
    prot[1] = a.recent + ((int64_t)b * a.n_recent + pos % a.n_recent) * RLQ_DC;
#pragma unroll
  for (int pi = 0; pi < 2; ++pi) {
    if (prot[pi] == nullptr) continue;
    uint16_t *dst = prot[pi] + G * RLQ_GROUP + 4 * kg;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const uint32_t lo = bf16_rne(z[mt][0]) | ((uint32_t)bf16_rne(z[mt][1]) << 16);
      const uint32_t hi = bf16_rne(z[mt][2]) | ((uint32_t)bf16_rne(z[mt][3]) << 16);
      *(u2 *)(dst + 16 * mt) = u2{lo, hi};
    }
  }
}

// RoPE key copy of tokens [tok0, tok0 + count): 16 bytes per thread step.
__device__ inline void copy_rope(const AppendArgs &a, int64_t tok0, int count, int tid, int nthreads) {
  for (int c = tid; c < count * 8; c += nthreads) {
    const int64_t tok = tok0 + (c >> 3);
    if (tok >= a.n_tokens) continue;
    const int b = find_request(a.cu_seqlens, a.batch, tok);
    const int64_t pos = (int64_t)a.start_pos[b] + (tok - a.cu_seqlens[b]);
    const int32_t page = a.block_table[(int64_t)b * a.max_pages + (pos >> 6)];
    const int64_t slot = (int64_t)page * RLQ_PAGE + (pos & 63);
    *(u4 *)(a.rope + slot * RLQ_DR + 8 * (c & 7)) = *(const u4 *)(a.k_rope + tok * RLQ_DR + 8 * (c & 7));
  }
}

__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int G = threadIdx.x >> 6;  // coordinate group of this wave
  const int n = lane & 15;
  const int kg = lane >> 4;
  const int64_t tile0 = (int64_t)blockIdx.x * kAppTokens;

  f4 acc[4][8];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[nt][mt] = f4{0.f, 0.f, 0.f, 0.f};

  if (a.latent_rot != nullptr) {
    // Already rotated: load z straight into the accumulator layout.
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t tok = tile0 + nt * 16 + n;
      if (tok < a.n_tokens) {
        const float *src = a.latent_rot + tok * RLQ_DC + G * RLQ_GROUP + 4 * kg;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) acc[nt][mt] = *(const f4 *)(src + 16 * mt);
      }
    }
  } else {
    const uint16_t *rrow = a.rotation + (size_t)(G * RLQ_GROUP + n) * RLQ_DC + 8 * kg;
    const uint16_t *crow[4];
    bool cval[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t tok = tile0 + nt * 16 + n;
      cval[nt] = tok < a.n_tokens;
      crow[nt] = a.latent + (cval[nt] ? tok : 0) * RLQ_DC + 8 * kg;
    }
    u4 ra[8], cb[4];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) ra[mt] = *(const u4 *)(rrow + (size_t)16 * mt * RLQ_DC);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) cb[nt] = cval[nt] ? *(const u4 *)crow[nt] : u4{0, 0, 0, 0};
    for (int k = 0; k < RLQ_DC / 32; ++k) {
      u4 ra_n[8], cb_n[4];
      if (k + 1 < RLQ_DC / 32) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
          ra_n[mt] = *(const u4 *)(rrow + (size_t)16 * mt * RLQ_DC + 32 * (k + 1));
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          cb_n[nt] = cval[nt] ? *(const u4 *)(crow[nt] + 32 * (k + 1)) : u4{0, 0, 0, 0};
      }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, ra[mt]), __builtin_bit_cast(bf16x8, cb[nt]),
              acc[nt][mt], 0, 0, 0);
      if (k + 1 < RLQ_DC / 32) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) ra[mt] = ra_n[mt];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) cb[nt] = cb_n[nt];
      }
    }
  }

#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    float z[8][4];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) z[mt][i] = acc[nt][mt][i];
    finish_group(a, z, tile0 + nt * 16 + n, G, kg);
  }

  copy_rope(a, tile0, kAppTokens, threadIdx.x, 256);
}


// Few-token path (decode steps): workgroup (16-token tile, group G); wave w
// contracts inputs [128w, 128w + 128) so every rotation load of the group is
// in flight at once, then wave 0 adds the four partial products in a fixed
// order and finishes the group.
__global__ __launch_bounds__(256) void append_small_kernel(AppendArgs a) {
  __shared__ f4 part[4][8][64];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int G = blockIdx.y;
  const int n = lane & 15;
  const int kg = lane >> 4;
  const int64_t tile0 = (int64_t)blockIdx.x * 16;
  const int64_t tok = tile0 + n;
  const bool cval = tok < a.n_tokens;
  f4 acc[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) acc[mt] = f4{0.f, 0.f, 0.f, 0.f};
  if (a.latent_rot != nullptr) {
    if (w == 0 && cval) {
      const float *src = a.latent_rot + tok * RLQ_DC + G * RLQ_GROUP + 4 * kg;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) acc[mt] = *(const f4 *)(src + 16 * mt);
    }
  } else {
    const uint16_t *rrow = a.rotation + (size_t)(G * RLQ_GROUP + n) * RLQ_DC + 128 * w + 8 * kg;
    const uint16_t *crow = a.latent + (cval ? tok : 0) * RLQ_DC + 128 * w + 8 * kg;
    u4 ra[4][8], cb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      cb[k] = cval ? *(const u4 *)(crow + 32 * k) : u4{0, 0, 0, 0};
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) ra[k][mt] = *(const u4 *)(rrow + (size_t)16 * mt * RLQ_DC + 32 * k);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ra[k][mt]),
                                                          __builtin_bit_cast(bf16x8, cb[k]), acc[mt], 0, 0, 0);
  }
  if (a.latent_rot == nullptr) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) part[w][mt][lane] = acc[mt];
  }
  __syncthreads();
  if (w == 0) {
    float z[8][4];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      f4 v = acc[mt];
      if (a.latent_rot == nullptr)
        v = (part[0][mt][lane] + part[1][mt][lane]) + (part[2][mt][lane] + part[3][mt][lane]);
#pragma unroll
      for (int i = 0; i < 4; ++i) z[mt][i] = v[i];
    }
    finish_group(a, z, tok, G, kg);
  }
  if (G == 0) copy_rope(a, tile0, 16, threadIdx.x, 256);
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, hipStream_t stream) {
  if (a.n_tokens == 0) return hipSuccess;
  if (a.n_tokens <= kSmallTokens) {
    const int64_t blocks = (a.n_tokens + 15) / 16;
    hipLaunchKernelGGL(append_small_kernel, dim3((unsigned)blocks, RLQ_NGROUPS), dim3(256), 0, stream, a);
  } else {
    const int64_t blocks = (a.n_tokens + kAppTokens - 1) / kAppTokens;
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace rlq
