// Write side: rotate -> standardize -> threshold -> pack, plus RoPE copy and
// BF16 sink/recent protection.  RoLaQ paper: §3.3 (rotated latents stored as
// 2-bit codes, rotation fixed while serving), §3.2 (four-level assignment by
// the per-layer threshold), §A.3 (group 128 with two fp32 statistics, BF16
// RoPE key, protected tokens keep BF16 content), §4.1 (sink + recent tokens).
//
// The rotation z^T = R c^T runs on bf16 MFMA (v_mfma_f32_16x16x32_bf16) with
// fp32 accumulation: A = rows of R (M = outputs of one coordinate group), B =
// token latents (N = tokens).  In the accumulator layout each
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

// Value of lane l ^ 32 (resp. l ^ 16) combined with this lane's by v_permlane
// swaps (no LDS traffic).  Both lanes of a pair get the same bits: the
// operations used (+, |) are commutative.
__device__ inline float add_xor32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ inline float add_xor16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ inline uint32_t or_xor16_32(uint32_t w) {
  const auto p = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  w = p[0] | p[1];
  const auto q = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return q[0] | q[1];
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
    const float s4 = (x[mt][0] + x[mt][1]) + (x[mt][2] + x[mt][3]);
    s16[mt] = add_xor32(add_xor16(s4));
  }
  return tree8(s16);
}

// Where a new token goes: its request, position and cache slot (-1 for
// tokens past the end), and the request's new length (read only when BF16
// protection is on: the recent window is measured from it).
struct Dest {
  int64_t slot;
  int32_t pos;  // position in the request (contexts stay below 2^31)
  int32_t b;
  int32_t new_len;
};

__device__ inline Dest resolve(const AppendArgs &a, int64_t tok) {
  Dest d{-1, 0, 0, 0};
  if (tok >= a.n_tokens) return d;
  d.b = find_request(a.cu_seqlens, a.batch, tok);
  const int32_t start = a.start_pos[d.b], cu_b = a.cu_seqlens[d.b];
  d.pos = start + (int32_t)(tok - cu_b);
  d.slot = (int64_t)a.block_table[(int64_t)d.b * a.max_pages + (d.pos >> 6)] * RLQ_PAGE + (d.pos & 63);
  if (a.sink != nullptr || a.recent != nullptr) d.new_len = start + (a.cu_seqlens[d.b + 1] - cu_b);
  return d;
}

// The same for the 16 tokens tile0 .. tile0+15, computed by one whole wave:
// lane n < 16 gets token tile0 + n.  With fewer than 64 requests the request
// search is one load of cu_seqlens (lane i holds cu_seqlens[i]) and 16
// ballots, and start_pos is loaded alongside, so the dependent chain is two
// loads long.
__device__ inline Dest resolve_wave(const AppendArgs &a, int64_t tile0, int lane) {
  if (a.batch >= 64) return resolve(a, tile0 + (lane & 15));
  const int64_t tok = tile0 + (lane & 15);
  const int32_t cu_l = a.cu_seqlens[lane <= a.batch ? lane : a.batch];
  // start_pos of every request, loaded alongside (lane i holds start_pos[i]).
  const int32_t start_l = a.start_pos[lane < a.batch ? lane : a.batch - 1];
  // Request of token t = number of i in [1, batch) with cu_seqlens[i] <= t.
  int b = 0;
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    const uint64_t m =
        __builtin_amdgcn_ballot_w64(lane >= 1 && lane < a.batch && (int64_t)cu_l <= tile0 + n);
    if ((lane & 15) == n) b = __builtin_popcountll(m);
  }
  const int32_t cu_b = __shfl(cu_l, b), cu_b1 = __shfl(cu_l, b + 1), start = __shfl(start_l, b);
  Dest d{-1, 0, b, 0};
  if (tok >= a.n_tokens) return d;
  d.pos = start + (int32_t)(tok - cu_b);
  d.slot = (int64_t)a.block_table[(int64_t)b * a.max_pages + (d.pos >> 6)] * RLQ_PAGE + (d.pos & 63);
  d.new_len = start + (cu_b1 - cu_b);
  return d;
}

// RoPE key of one token (128 bytes) to its slot.
__device__ inline void copy_rope_token(const AppendArgs &a, int64_t tok, const Dest &d) {
  if (d.slot < 0) return;
  const u4 *src = (const u4 *)(a.k_rope + tok * RLQ_DR);
  u4 *dst = (u4 *)(a.rope + d.slot * RLQ_DR);
#pragma unroll
  for (int c = 0; c < RLQ_DR / 8; ++c) dst[c] = src[c];
}

// Statistics, codes and stores for one token and one group: z[mt][i] is
// output 16*mt + 4*kg + i of group G; the four lanes {n, n+16, n+32, n+48}
// hold the whole group.  All 64 lanes must call it (cross-lane sums).
__device__ inline void finish_group(const AppendArgs &a, const float (&z)[8][4], int64_t tok,
                                    const Dest &dst_tok, int G, int kg) {
  const bool valid = dst_tok.slot >= 0;
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
      // code = [x >= -t] + [x >= 0] + [x >= t]; with t >= 0 (tau >= 0 is
      // checked on the host) the sign decides which threshold still matters:
      // x >= 0 gives 2 + [x >= t], x < 0 gives [x >= -t].
      const float x = d[mt][i];
      const bool nonneg = x >= 0.f;
      const uint32_t c = (nonneg ? 2u : 0u) + (uint32_t)(x >= (nonneg ? t : -t));
      byte |= c << (2 * i);
    }
    word[mt] = or_xor16_32(byte << (8 * kg));
  }
  if (!valid) return;
  const int b = dst_tok.b;
  const int64_t pos = dst_tok.pos, slot = dst_tok.slot;

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
  uint16_t *prot[2] = {nullptr, nullptr};
  if (a.sink == nullptr && a.recent == nullptr) return;
  const int64_t new_len = dst_tok.new_len;
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

// Bulk path: one persistent workgroup per CU.  Workgroup (G, slot) keeps the
// 128 rows of R for coordinate group G in LDS (128 KB) and streams 512-token
// tiles through eight waves of 64 tokens; the K loop needs no barrier.  The
// rotation z^T = R c^T: A = rows of R from LDS (M = outputs), B = latents
// straight from memory (N = tokens), fp32 accumulation.
constexpr int kBulkWaves = 8;
constexpr int kBulkTile = 64 * kBulkWaves;           // tokens per workgroup pass
constexpr int kBulkSlots = 8;                        // workgroups per (XCD, group)
constexpr int kBulkGrid = 8 * RLQ_NGROUPS * kBulkSlots;  // 256: one per CU
constexpr int kRSlice = RLQ_GROUP * 32 * 2;          // 8 KB: 128 rows x 32 K
constexpr int kRBytes = (RLQ_DC / 32) * kRSlice;     // 128 KB
// Request table staged in LDS after R: cu_seqlens[0..B] and start_pos[0..B-1]
// (batches up to kLdsRequests; larger ones search global memory).
constexpr int kLdsRequests = 2047;
constexpr int kBulkLds = kRBytes + (2 * kLdsRequests + 2) * 4;  // 144 KB

__global__ __launch_bounds__(64 * kBulkWaves, 1) void append_kernel(AppendArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char rs[];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n = lane & 15;
  const int kg = lane >> 4;
  // Workgroups are dealt to the 8 XCDs round-robin: the four group
  // workgroups of one slot share an XCD and walk the same tiles, so three of
  // them read each tile's latents from that XCD's L2.
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int G = j & 3, slot = j >> 2;
  // 16-byte chunk c (K 8c .. 8c+7) of row r in K-slice k; the xor spreads the
  // operand reads of 16 consecutive rows over distinct banks.
  auto chunk = [](int k, int r, int c) { return k * kRSlice + 64 * r + 16 * (c ^ ((r >> 2) & 3)); };
  if (a.latent_rot == nullptr) {
    // Consecutive lanes fill consecutive chunks of one K-slice (a wave writes
    // one contiguous 1 KB block, free of bank conflicts).
    for (int i = threadIdx.x; i < RLQ_GROUP * RLQ_DC / 8; i += 64 * kBulkWaves) {
      const int c = i & 3, r = (i >> 2) & (RLQ_GROUP - 1), k = i >> 9;  // chunk, row, K-slice
      *(u4 *)(rs + chunk(k, r, c)) =
          *(const u4 *)(a.rotation + (size_t)(G * RLQ_GROUP + r) * RLQ_DC + 8 * (4 * k + c));
    }
  }
  // The request table, so that finding a token's request and position needs
  // no dependent global loads.
  int32_t *lds_cu = (int32_t *)(rs + kRBytes);
  int32_t *lds_start = lds_cu + kLdsRequests + 1;
  const bool lds_table = a.batch <= kLdsRequests;
  if (lds_table) {
    for (int i = threadIdx.x; i <= a.batch; i += 64 * kBulkWaves) lds_cu[i] = a.cu_seqlens[i];
    for (int i = threadIdx.x; i < a.batch; i += 64 * kBulkWaves) lds_start[i] = a.start_pos[i];
  }
  __syncthreads();

  const int64_t n_tiles = (a.n_tokens + kBulkTile - 1) / kBulkTile;
  for (int64_t tile = xcd + 8 * slot; tile < n_tiles; tile += 8 * kBulkSlots) {
    const int64_t tile0 = tile * kBulkTile + 64 * w;
    // Destinations: request and position from the LDS table now, the page id
    // load issued now and consumed after the contraction.
    int32_t rb[4], rpg[4];
    auto pos_of = [&](int nt) -> int32_t {
      const int64_t tok = tile0 + nt * 16 + n;
      const int64_t t = tok < a.n_tokens ? tok : a.n_tokens - 1;
      return lds_start[rb[nt]] + (int32_t)(t - lds_cu[rb[nt]]);
    };
    auto locate = [&](int nt) {
      const int64_t tok = tile0 + nt * 16 + n;
      const int64_t t = tok < a.n_tokens ? tok : a.n_tokens - 1;
      int lo = 0, hi = a.batch;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)lds_cu[mid] <= t) lo = mid; else hi = mid;
      }
      rb[nt] = lo;
      rpg[nt] = a.block_table[(int64_t)lo * a.max_pages + (pos_of(nt) >> 6)];
    };
    auto dest_of = [&](int nt) -> Dest {
      const int64_t tok = tile0 + nt * 16 + n;
      if (!lds_table) return resolve(a, tok);
      const int32_t pos = pos_of(nt);
      Dest d{-1, pos, rb[nt], 0};
      if (tok >= a.n_tokens) return d;
      d.slot = (int64_t)rpg[nt] * RLQ_PAGE + (pos & 63);
      d.new_len = lds_start[rb[nt]] + (lds_cu[rb[nt] + 1] - lds_cu[rb[nt]]);
      return d;
    };

    f4 acc[4][8];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) acc[nt][mt] = f4{0.f, 0.f, 0.f, 0.f};

    if (a.latent_rot != nullptr) {
      if (lds_table) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) locate(nt);
      }
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
      // Latents of this wave's tokens; tokens past the end read the last
      // token (their results are never stored).
      const uint16_t *crow[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int64_t tok = tile0 + nt * 16 + n;
        crow[nt] = a.latent + (tok < a.n_tokens ? tok : a.n_tokens - 1) * RLQ_DC + 8 * kg;
      }
      // Latent K-slices run kCDepth steps ahead; the loop is fully unrolled so
      // every buffer index is a constant.
      constexpr int kSteps = RLQ_DC / 32;
      constexpr int kCDepth = 3;
      u4 cb[kCDepth][4];
      if (lds_table) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) locate(nt);
      }
#pragma unroll
      for (int k = 0; k < kCDepth; ++k)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) cb[k][nt] = *(const u4 *)(crow[nt] + 32 * k);
#pragma unroll
      for (int k = 0; k < kSteps; ++k) {
        u4 c[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) c[nt] = cb[k % kCDepth][nt];
        if (k + kCDepth < kSteps) {
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) cb[k % kCDepth][nt] = *(const u4 *)(crow[nt] + 32 * (k + kCDepth));
        }
        // All eight A operands of the step are read up front, so one LDS
        // wait covers them.
        u4 ra[8];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) ra[mt] = *(const u4 *)(rs + chunk(k, 16 * mt + n, kg));
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, ra[mt]), __builtin_bit_cast(bf16x8, c[nt]), acc[nt][mt], 0, 0, 0);
      }
    }

    // RoPE keys: the four group workgroups of a tile each copy one 32-byte
    // quarter of every token's key (lane l: token tile0 + l).  The loads go
    // out now and the stores after the statistics, which hide their latency.
    const int64_t rtok = tile0 + lane;
    u4 rq[2] = {};
    if (rtok < a.n_tokens) {
      const u4 *src = (const u4 *)(a.k_rope + rtok * RLQ_DR + 16 * G);
      rq[0] = src[0];
      rq[1] = src[1];
    }
    Dest dst[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) dst[nt] = dest_of(nt);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      float z[8][4];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) z[mt][i] = acc[nt][mt][i];
      finish_group(a, z, tile0 + nt * 16 + n, dst[nt], G, kg);
    }
    // Token tile0 + lane is N-tile kg, column n: its destination is dst[kg]
    // (selected, not indexed, so dst stays in registers).
    const int64_t rslot = kg == 0 ? dst[0].slot : kg == 1 ? dst[1].slot : kg == 2 ? dst[2].slot : dst[3].slot;
    if (rslot >= 0) {
      u4 *dstp = (u4 *)(a.rope + rslot * RLQ_DR + 16 * G);
      dstp[0] = rq[0];
      dstp[1] = rq[1];
    }
  }
}


// Few-token path (decode steps): workgroup (16-token tile, group G) of five
// waves.  Wave w < 4 contracts inputs [128w, 128w + 128), so every rotation
// load of the group is in flight at once; wave 4 looks up the destinations
// (a chain of dependent loads that then waits behind no rotation load).
// Wave 0 adds the four partial products in a fixed order and finishes the
// group.
constexpr int kSmallWaves = 5;

__global__ __launch_bounds__(64 * kSmallWaves) void append_small_kernel(AppendArgs a) {
  __shared__ f4 part[4][8][64];
  __shared__ Dest dests[16];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int G = blockIdx.y;
  const int n = lane & 15;
  const int kg = lane >> 4;
  const int64_t tile0 = (int64_t)blockIdx.x * 16;
  const int64_t tok = tile0 + n;
  // Tokens past the end read the last token (their results are never stored).
  const int64_t tok_c = tok < a.n_tokens ? tok : a.n_tokens - 1;
  f4 acc[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) acc[mt] = f4{0.f, 0.f, 0.f, 0.f};
  if (w == 4) {
    const Dest d = resolve_wave(a, tile0, lane);
    if (lane < 16) dests[lane] = d;
  } else if (a.latent_rot != nullptr) {
    if (w == 0) {
      const float *src = a.latent_rot + tok_c * RLQ_DC + G * RLQ_GROUP + 4 * kg;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) acc[mt] = *(const f4 *)(src + 16 * mt);
    }
  } else {
    const uint16_t *rrow = a.rotation + (size_t)(G * RLQ_GROUP + n) * RLQ_DC + 128 * w + 8 * kg;
    const uint16_t *crow = a.latent + tok_c * RLQ_DC + 128 * w + 8 * kg;
    u4 ra[4][8], cb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      cb[k] = *(const u4 *)(crow + 32 * k);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) ra[k][mt] = *(const u4 *)(rrow + (size_t)16 * mt * RLQ_DC + 32 * k);
    }
    // Keep every load above the products: left to itself the scheduler
    // interleaves them to save registers, which exposes the load latency
    // several times over.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ra[k][mt]),
                                                          __builtin_bit_cast(bf16x8, cb[k]), acc[mt], 0, 0, 0);
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
    finish_group(a, z, tok, dests[n], G, kg);
  }
  if (G == 0 && w == 1 && kg == 0) copy_rope_token(a, tok, dests[n]);
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, hipStream_t stream) {
  if (a.n_tokens == 0) return hipSuccess;
  if (a.n_tokens <= kSmallTokens) {
    const int64_t blocks = (a.n_tokens + 15) / 16;
    hipLaunchKernelGGL(append_small_kernel, dim3((unsigned)blocks, RLQ_NGROUPS), dim3(64 * kSmallWaves), 0,
                       stream, a);
  } else {
    static PerDeviceOnce attr;
    hipError_t ea = once_per_device(attr, [] {
      return hipFuncSetAttribute((const void *)append_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kBulkLds);
    });
    if (ea != hipSuccess) return ea;
    hipLaunchKernelGGL(append_kernel, dim3(kBulkGrid), dim3(64 * kBulkWaves), kBulkLds, stream, a);
  }
  return hipGetLastError();
}

}  // namespace rlq
