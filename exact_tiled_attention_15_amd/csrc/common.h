// Internal declarations shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace eta {

// ---------------------------------------------------------------- vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// -------------------------------------------------------------- tile geometry
// One workgroup = 4 wavefronts = 128 query rows (32 per wavefront); each inner
// iteration consumes 64 keys.
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;
constexpr int kBN = 64;

// What the epilogue of the forward kernels writes.
enum Epilogue : int {
  kEpiFinalBf16 = 0,  // O normalised, bf16; LSE (optional)
  kEpiState = 1,      // O normalised fp32, m (natural units), l
  kEpiFinalF32 = 2,   // O normalised, fp32; LSE (optional)
};

// Parameters of the bf16 / fp8 forward kernels (one (b,h) slice per
// q_stride / kv_stride step; every index is a token index inside a slice).
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const float* q_scale;  // fp8 only: [BH, ceil(Nq/128)]
  const float* k_scale;  // fp8 only
  const float* v_scale;  // fp8 only
  void* o;
  float* lse;    // final epilogues; may be null
  float* m_out;  // state epilogue
  float* l_out;  // state epilogue
  int Nq, Nk;
  int BH;        // B * H
  int nqb;       // ceil(Nq / kBM)
  int diag;      // causal: key j allowed for row i iff j <= i + diag
  float c;       // |scale| * log2(e): raw dot product -> base-2 exponent
  float scale_abs;
  uint32_t q_sign;  // sign mask xor-ed into Q elements when scale < 0
};

// Launchers (host side). Each returns hipGetLastError() after the launch.
hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, int epi, hipStream_t s);
hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, hipStream_t s);
hipError_t launch_fwd_fp8(const FwdParams& p, int d, bool causal, bool qk16, hipStream_t s);

struct MergeParams {
  float* o_acc;
  float* m_acc;
  float* l_acc;
  const float* o_part;
  const float* m_part;
  const float* l_part;
  void* o_final;     // bf16, may be null
  float* lse_final;  // may be null
  int64_t rows;      // B * H * Nq
  int d;
};
hipError_t launch_merge(const MergeParams& p, hipStream_t s);

// ------------------------------------------------------------ device helpers
// Workgroup -> (query block, b*h slice).  Workgroups are dealt to the 8 XCDs
// round-robin (XCD = blockIdx % 8); when the work divides evenly, each XCD is
// given a contiguous range of (b,h) slices so that one slice's K/V stays in one
// XCD's L2.  For causal masks the heaviest query blocks (the last ones) are
// issued first.
__device__ inline void map_block(int g, int nqb, int BH, bool causal, int& qb, int& bh) {
  int qi;
  if ((BH & 7) == 0) {
    const int x = g & 7;
    const int t = g >> 3;
    const int hp = BH >> 3;  // slices per XCD
    bh = x * hp + t % hp;
    qi = t / hp;
  } else {
    bh = g % BH;
    qi = g / BH;
  }
  qb = causal ? (nqb - 1 - qi) : qi;
}

// Value of the other half-wave (lane ^ 32) combined with this lane's, for all
// 64 lanes: permlane32_swap(x, x) yields x[l % 32] and x[l % 32 + 32].
__device__ inline float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace eta
