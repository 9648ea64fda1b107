// Matrix-core measurements on gfx950: the dense MFMA peak that the attention
// kernels are compared with, and a single-instruction product that shows how
// one MFMA sums its products.
//
// Peak loop.  Every workgroup has 8 wavefronts (two per SIMD, the attention
// kernels' occupancy); each wavefront keeps four independent accumulator
// chains and issues `iters` rounds of four MFMAs with register operands, so
// the matrix cores never wait for memory or for a dependent result.  The
// caller times the launch; FLOP = workgroups * 8 * iters * 4 * FLOP per MFMA.
//
// Single product.  One wavefront computes C = A B for one 32x32 tile with
// K = 64: on the f8f6f4 MFMA (one 32x32x64 instruction, e4m3 operands, unit
// block scales) or on four chained 32x32x16 bf16 / fp16 MFMAs.  e4m3 values
// are exact in bf16 and fp16, so the same products can be compared across
// the three forms and with an exact sum.
#include "common.h"

namespace eta {

constexpr int kProbeThreads = 512;

template <int KIND>
__global__ void __launch_bounds__(kProbeThreads) mfma_peak_kernel(float* out, int iters) {
  const int tid = threadIdx.x;
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = (f32x16){};
  if constexpr (KIND == 0 || KIND == 1) {
    // small values: the sums stay far from overflow for any iteration count used here
    const float x = 1.0f / 4096.0f * (1 + (tid & 7));
    if constexpr (KIND == 0) {
      bf16x8 a, b;
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] = b[j] = (__bf16)(x * (j + 1));
      for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    } else {
      f16x8 a, b;
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] = b[j] = (_Float16)(x * (j + 1));
      for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
    }
  } else if constexpr (KIND == 2) {
    // e4m3 code 0x08 + (tid & 7): small normal values
    const int byte = 0x08 + (tid & 7);
    const int w = byte * 0x01010101;
    const i32x8 a = {w, w, w, w, w, w, w, w};
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, acc[c], 0, 0, 0, 127, 0, 127);
  } else {
    const float a = 1.0f / 4096.0f * (1 + (tid & 7));
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, a, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  out[(int64_t)blockIdx.x * kProbeThreads + tid] = s;
}

double mfma_flop_per_instruction(int kind) {
  switch (kind) {
    case 0:
    case 1: return 2.0 * 32 * 32 * 16;
    case 2: return 2.0 * 32 * 32 * 64;
    case 3: return 2.0 * 32 * 32 * 2;
  }
  return 0.0;
}

hipError_t launch_mfma_peak(int kind, int workgroups, int iters, float* out, hipStream_t s) {
  const dim3 grid((unsigned)workgroups), block(kProbeThreads);
  switch (kind) {
    case 0: hipLaunchKernelGGL(mfma_peak_kernel<0>, grid, block, 0, s, out, iters); break;
    case 1: hipLaunchKernelGGL(mfma_peak_kernel<1>, grid, block, 0, s, out, iters); break;
    case 2: hipLaunchKernelGGL(mfma_peak_kernel<2>, grid, block, 0, s, out, iters); break;
    case 3: hipLaunchKernelGGL(mfma_peak_kernel<3>, grid, block, 0, s, out, iters); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// One 32x32 tile, K = 64.  a: 32 rows x 64 elements, row-major; b: 32 columns
// x 64 elements, one column after another (B transposed, row-major); c: 32 x
// 32 fp32, row-major.  Lane l supplies row / column l % 32.
template <int KIND>
__global__ void __launch_bounds__(64) mfma_dot_kernel(const void* a, const void* b, float* c) {
  const int l = threadIdx.x;
  const int r = l & 31, g = l >> 5;
  f32x16 acc = {};
  if constexpr (KIND == 2) {
    // f8f6f4 32x32x64: lane l holds bytes 32 g .. 32 g + 31 of its row / column
    const u32x4* pa = (const u32x4*)((const uint8_t*)a + r * 64 + 32 * g);
    const u32x4* pb = (const u32x4*)((const uint8_t*)b + r * 64 + 32 * g);
    const u32x4 a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
    const i32x8 av = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    const i32x8 bv = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
  } else {
    // 32x32x16, four k-steps: lane l holds elements 16 kk + 8 g .. +8 of its row / column
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4 av = *(const u32x4*)((const uint16_t*)a + r * 64 + 16 * kk + 8 * g);
      const u32x4 bv = *(const u32x4*)((const uint16_t*)b + r * 64 + 16 * kk + 8 * g);
      if constexpr (KIND == 0)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv),
                                                      acc, 0, 0, 0);
      else
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av), __builtin_bit_cast(f16x8, bv),
                                                     acc, 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) c[(8 * (i >> 2) + 4 * g + (i & 3)) * 32 + r] = acc[i];
}

hipError_t launch_mfma_dot(int kind, const void* a, const void* b, float* c, hipStream_t s) {
  switch (kind) {
    case 0: hipLaunchKernelGGL(mfma_dot_kernel<0>, dim3(1), dim3(64), 0, s, a, b, c); break;
    case 1: hipLaunchKernelGGL(mfma_dot_kernel<1>, dim3(1), dim3(64), 0, s, a, b, c); break;
    case 2: hipLaunchKernelGGL(mfma_dot_kernel<2>, dim3(1), dim3(64), 0, s, a, b, c); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace eta
