// Measured ceilings of one MI355X (gfx950) for the rooflines the benchmark
// reports against: HBM read-only streaming with 16-byte loads, MFMA issue
// rates of the instruction shapes the decode kernels use, LDS read / write /
// transposed-read rates per CU, and the shader clock under load.  Built as
// librlq_ceilings.so, used by bench.py (--ceilings); not part of the
// decode / append path.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i8v __attribute__((ext_vector_type(8)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4 lds_s4;

// Streams n 16-byte words once, kDepth independent loads in flight per
// thread and iteration (non-temporal when kNT); the xor of everything decides
// a store that never happens for the host's data, so no load can be dropped.
template <int kDepth, bool kNT>
__global__ __launch_bounds__(256) void read_kernel(const u4 *__restrict__ src, int64_t n, uint32_t *sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kDepth - 1) * stride < n; i += kDepth * stride) {
    u4 v[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) v[d] = kNT ? __builtin_nontemporal_load(src + i + d * stride) : src[i + d * stride];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) acc ^= v[d];
  }
  for (; i < n; i += stride) acc ^= src[i];
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x9e3779b9u) sink[0] = x;
}

// kind 0: v_mfma_f32_16x16x32_f16, 1: _bf16, 2: _bf8_fp8 (16x16x32), 3:
// v_mfma_f32_16x16x128_f8f6f4 with fp8 operands, 4: v_mfma_f32_32x32x16_f16,
// 5: kind 4 with eight independent fp32 FMAs issued after each MFMA (how much
// VALU work one wave can issue under its own MFMAs).  Eight independent
// accumulators per wave, `iters` rounds.  Lane 0 of each wave records the
// shader-clock counter (s_memtime) and the 100 MHz reference counter
// (s_memrealtime) around the loop.
template <int kKind>
__global__ __launch_bounds__(256) void mfma_kernel(int iters, float *sink, int64_t *clk) {
  const uint32_t seed = threadIdx.x * 2654435761u + blockIdx.x;
  u4 a4 = {seed, seed ^ 0x3c003c00u, seed + 7u, seed * 3u};
  a4 &= u4{0x3b3b3b3bu, 0x3b3b3b3bu, 0x3b3b3b3bu, 0x3b3b3b3bu};  // small finite fp16 / bf16 / fp8 values
  typedef float f16v __attribute__((ext_vector_type(16)));
  f4 acc[8];
  constexpr bool k32 = kKind == 4 || kKind == 5;
  f16v acc16[k32 ? 8 : 1];
  float fv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) fv[j] = (float)(threadIdx.x + j);
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < (k32 ? 8 : 1); ++j) acc16[j] = f16v{};
  const int64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (kKind == 0) {
        const half8 a = __builtin_bit_cast(half8, a4);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, a, acc[j], 0, 0, 0);
      } else if constexpr (kKind == 1) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, a4);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, acc[j], 0, 0, 0);
      } else if constexpr (kKind == 2) {
        const long a = __builtin_bit_cast(long, u2v{a4[0], a4[1]});
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf8_fp8(a, a, acc[j], 0, 0, 0);
      } else if constexpr (kKind == 3) {
        const i8v a = __builtin_bit_cast(i8v, __builtin_shufflevector(a4, a4, 0, 1, 2, 3, 0, 1, 2, 3));
        acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, a, acc[j], 0, 0, 0, 0, 0, 0);
      } else {
        // 32x32x16 f16: four 16x16 accumulators' worth of output per product
        const half8 a = __builtin_bit_cast(half8, a4);
        acc16[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, acc16[j], 0, 0, 0);
        if constexpr (kKind == 5) {
#pragma unroll
          for (int x = 0; x < 8; ++x) fv[x] = __builtin_fmaf(fv[x], 1.0001f, 0.5f);
        }
      }
    }
  }
  const int64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  f4 s = acc[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) s += acc[j];
  if constexpr (k32) {
#pragma unroll
    for (int j = 0; j < 8; ++j) s[0] += acc16[j][0] + acc16[j][15];
  }
  if constexpr (kKind == 5) {
#pragma unroll
    for (int j = 0; j < 8; ++j) s[1] += fv[j];
  }
  if (s[0] == 1234.5f) sink[0] = s[1];
  if ((threadIdx.x & 63) == 0) {
    const int w = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
    clk[2 * w] = t1 - t0;
    clk[2 * w + 1] = r1 - r0;
  }
}

// LDS rate per CU.  kind 0: ds_read_b128, 1: ds_write_b128, 2:
// ds_read_b64_tr_b16; every lane touches a distinct 16-byte slot (8-byte for
// kind 2) of a 64 KB region, 16 waves per CU, `iters` rounds of 16 accesses.
template <int kKind>
__global__ __launch_bounds__(1024) void lds_kernel(int iters, uint32_t *sink) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int t = threadIdx.x;
  for (int i = t; i < 65536 / 16; i += blockDim.x) ((u4 *)lds)[i] = u4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  u4 acc = {0u, 0u, 0u, 0u};
  // Lanes of a wave touch consecutive slots (no bank conflicts); the
  // addresses move with the iteration so no access repeats an earlier one.
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if constexpr (kKind == 0) {
        acc ^= *(const u4 *)(lds + ((16 * t + 4096 * j + 16 * it) & 65535));
      } else if constexpr (kKind == 1) {
        *(u4 *)(lds + ((16 * t + 4096 * j + 16 * it) & 65535)) = u4{(uint32_t)it, (uint32_t)j, (uint32_t)t, 0u};
      } else {
        const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(lds + ((8 * t + 8192 * j + 8 * it) & 65535)));
        acc[0] ^= __builtin_bit_cast(u2v, v)[0];
        acc[1] ^= __builtin_bit_cast(u2v, v)[1];
      }
    }
  }
  if constexpr (kKind == 1) acc = *(const u4 *)(lds + 16 * (t & 4095));
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x9e3779b9u) sink[0] = x;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from `src` once on `stream`; mode 0: 4
// loads in flight per thread, 1: 8, 2: 8 non-temporal.
int rlq_ceiling_read(int32_t mode, const void *src, int64_t bytes, uint32_t *sink, int32_t blocks, void *stream) {
  if (src == nullptr || sink == nullptr || bytes < 16 || bytes % 16 || blocks < 1) return -1;
  hipStream_t s = (hipStream_t)stream;
  const u4 *p = (const u4 *)src;
  switch (mode) {
    case 0: hipLaunchKernelGGL((read_kernel<4, false>), dim3(blocks), dim3(256), 0, s, p, bytes / 16, sink); break;
    case 1: hipLaunchKernelGGL((read_kernel<8, false>), dim3(blocks), dim3(256), 0, s, p, bytes / 16, sink); break;
    case 2: hipLaunchKernelGGL((read_kernel<8, true>), dim3(blocks), dim3(256), 0, s, p, bytes / 16, sink); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// MFMA issue loop (see mfma_kernel); clk gets 2 int64 per wave:
// (shader cycles, 100 MHz ticks).
int rlq_ceiling_mfma(int32_t kind, int32_t blocks, int32_t iters, float *sink, int64_t *clk, void *stream) {
  if (sink == nullptr || clk == nullptr || blocks < 1 || iters < 1) return -1;
  hipStream_t s = (hipStream_t)stream;
  switch (kind) {
    case 0: hipLaunchKernelGGL(mfma_kernel<0>, dim3(blocks), dim3(256), 0, s, iters, sink, clk); break;
    case 1: hipLaunchKernelGGL(mfma_kernel<1>, dim3(blocks), dim3(256), 0, s, iters, sink, clk); break;
    case 2: hipLaunchKernelGGL(mfma_kernel<2>, dim3(blocks), dim3(256), 0, s, iters, sink, clk); break;
    case 3: hipLaunchKernelGGL(mfma_kernel<3>, dim3(blocks), dim3(256), 0, s, iters, sink, clk); break;
    case 4: hipLaunchKernelGGL(mfma_kernel<4>, dim3(blocks), dim3(256), 0, s, iters, sink, clk); break;
    case 5: hipLaunchKernelGGL(mfma_kernel<5>, dim3(blocks), dim3(256), 0, s, iters, sink, clk); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// LDS access loop (see lds_kernel), one 1024-thread workgroup per CU.
int rlq_ceiling_lds(int32_t kind, int32_t blocks, int32_t iters, uint32_t *sink, void *stream) {
  if (sink == nullptr || blocks < 1 || iters < 1) return -1;
  hipStream_t s = (hipStream_t)stream;
  const int lds = 65536;
  switch (kind) {
    case 0:
      hipFuncSetAttribute((const void *)lds_kernel<0>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      hipLaunchKernelGGL(lds_kernel<0>, dim3(blocks), dim3(1024), lds, s, iters, sink);
      break;
    case 1:
      hipFuncSetAttribute((const void *)lds_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      hipLaunchKernelGGL(lds_kernel<1>, dim3(blocks), dim3(1024), lds, s, iters, sink);
      break;
    case 2:
      hipFuncSetAttribute((const void *)lds_kernel<2>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      hipLaunchKernelGGL(lds_kernel<2>, dim3(blocks), dim3(1024), lds, s, iters, sink);
      break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
