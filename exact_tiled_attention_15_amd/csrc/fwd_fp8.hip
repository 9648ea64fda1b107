// Block-quantized fp8 (OCP e4m3) attention forward for gfx950.
//
// Inputs are e4m3 codes with one fp32 scale per (b, h, 128-token tile), the
// block quantization of "Scaling FlashAttention, multi-GPU training and weight
// quantization" (itimpress, section 1, FP8 bullet).  The decomposition is the
// bf16 kernel's (query blocks over workgroups, 32 rows per wavefront, online
// softmax in registers, K/V tiles double-buffered through LDS), with:
//   * S^T = K Q^T on the 32x32x64 f8f6f4 MFMA (both operands e4m3, unit block
//     scales), or - the QK16 instantiation - on the 32x32x16 fp16 MFMA with
//     the codes widened exactly to fp16.  The fp8 MFMA sums the products of
//     one instruction with limited alignment precision (measured on gfx950:
//     one 448*448 product among small ones leaves an error of ~34 on a sum of
//     2e5), so channels with large outliers need the rotation of the same
//     passage ("incoherent processing") before quantization; the fp16 form is
//     exact for any codes.  Since a workgroup's 128 rows are exactly one query
//     tile and a 64-key iteration lies inside one key tile, the product of the
//     two fp32 scales is a single scalar per iteration, folded into the
//     softmax FMA: c_t = |scale| * log2(e) * s_q * s_k(t).
//   * P V on the 32x32x16 fp16 MFMA: V codes are converted exactly to fp16
//     while staged into LDS; the probabilities are rounded to fp16 as
//     p * s_v(t) / max_t s_v (the ratio folded into the exponent bias, so the
//     value is <= 1 for any scales), and the normaliser is summed from the
//     unrounded fp32 values with the ratio divided out once per tile.
//   * O accumulates and is written in fp32.
// Layouts of the 32x32 MFMAs are those documented in fwd_bf16.hip; for the
// f8f6f4 form the A/B k-slice of lane l is bytes (l/32)*32 .. +32.
#include "common.h"

namespace eta {

template <int D, bool QK16>
struct Geo8 {
  static constexpr int KS = QK16 ? 2 * D + 16 : D + 16;  // K tile row pitch (bytes)
  static constexpr int K_BYTES = kBN * KS;
  static constexpr int V_BYTES = D * kVtPitch;  // fp16 V^T: one row per column d
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int CPR = D / 16;        // 16-byte code chunks per row
  static constexpr int PER_THREAD = kBN * CPR / kThreads;
  static constexpr int V_THREADS = 16 * (D / 8);  // 16 key groups x D/8 column chunks
  static_assert(PER_THREAD >= 1 && PER_THREAD * kThreads == kBN * CPR, "tile must split evenly");
  static_assert(V_THREADS <= kThreads, "V staging needs at most one thread per 4x8 block");
};

typedef float f32x8 __attribute__((ext_vector_type(8)));

__device__ inline u32x4 widen_lo(const u32x4 w) {  // codes 0..7 of 16 -> fp16
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    r[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, false));
    r[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, true));
  }
  return r;
}
__device__ inline u32x4 widen_hi(const u32x4 w) {  // codes 8..15 of 16 -> fp16
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    r[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[2 + i], 1.0f, false));
    r[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[2 + i], 1.0f, true));
  }
  return r;
}

template <int D, bool CAUSAL, bool QK16>
__global__ void __launch_bounds__(kThreads, 2) fwd_fp8_kernel(FwdParams p) {
  using G = Geo8<D, QK16>;
  constexpr int QT = 128;  // tokens per quantization tile
  __shared__ __attribute__((aligned(16))) char smem[G::LDS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r32 = lane & 31;
  const int g = lane >> 5;

  int qb, bh;
  map_block(blockIdx.x, p.nqb, p.BH, CAUSAL, qb, bh);
  const int q0 = qb * kBM;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + r32;
  const int Nq = p.Nq, Nk = p.Nk;
  const int nqt = (Nq + QT - 1) / QT, nkt = (Nk + QT - 1) / QT;

  const uint8_t* __restrict__ qg = (const uint8_t*)p.q + (int64_t)bh * Nq * D;
  const uint8_t* __restrict__ kg = (const uint8_t*)p.k + (int64_t)bh * Nk * D;
  const uint8_t* __restrict__ vg = (const uint8_t*)p.v + (int64_t)bh * Nk * D;
  const float* __restrict__ ksc = p.k_scale + (int64_t)bh * nkt;
  const float* __restrict__ vsc = p.v_scale + (int64_t)bh * nkt;
  const float c_q = p.c * p.q_scale[(int64_t)bh * nqt + q0 / QT];
  // Largest V scale of this (b,h) slice: probabilities are stored as
  // p * s_v(t) / svmax <= 1, which fp16 holds without overflow.
  float svmax = 0.f;
  for (int t = 0; t < nkt; ++t) svmax = fmaxf(svmax, vsc[t]);
  const float inv_svmax = 1.f / svmax;

  int kend = Nk, wkend = Nk, wmask_from = Nk;
  if (CAUSAL) {
    const int last_row = min(q0 + kBM, Nq) - 1;
    kend = min(Nk, last_row + p.diag + 1);
    wkend = min(Nk, min(qw0 + 31, Nq - 1) + p.diag + 1);
    wmask_from = min(Nk, qw0 + p.diag + 1);
  }
  const int ntiles = kend > 0 ? (kend + kBN - 1) / kBN : 0;
  const bool wave_live = qw0 < Nq;

  // Q fragment (B operand).  fp8 form: row my_q, codes 64*kk + 32*g .. +32.
  // fp16 form: row my_q, d = 16*kk + 8*g .. +8 widened exactly to fp16.
  constexpr int QF = QK16 ? D / 16 : D / 64;
  i32x8 qf8[QK16 ? 1 : QF];
  f16x8 qf16[QK16 ? QF : 1];
  {
    const bool ok = my_q < Nq;
    const uint32_t q_and = p.q_and ? 0xFFFFFFFFu : 0u;
    const uint32_t sgn = p.q_xor ? 0x80808080u : 0u;
    const uint8_t* row = qg + (int64_t)(ok ? my_q : 0) * D;
    if constexpr (QK16) {
#pragma unroll
      for (int kk = 0; kk < QF; ++kk) {
        u32x2 c = ok ? *(const u32x2*)(row + 16 * kk + 8 * g) : (u32x2){0u, 0u};
        c = (c & q_and) ^ sgn;
        const u32x4 w = {c[0], c[1], 0u, 0u};
        qf16[kk] = __builtin_bit_cast(f16x8, widen_lo(w));
      }
    } else {
      const u32x4* src = (const u32x4*)(row + 32 * g);
#pragma unroll
      for (int kk = 0; kk < QF; ++kk) {
        u32x4 a = ok ? src[kk * 4] : (u32x4){0u, 0u, 0u, 0u};
        u32x4 b = ok ? src[kk * 4 + 1] : (u32x4){0u, 0u, 0u, 0u};
        a = (a & q_and) ^ sgn;
        b = (b & q_and) ^ sgn;
        qf8[kk] = (i32x8){(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
      }
    }
  }

  // K: 16-byte code chunks of rows.  V: thread (dc, kgrp) takes keys
  // 4*kgrp .. +3 of columns 8*dc .. +7 (8 codes each), widens them to fp16 and
  // stores them transposed (common.h).
  const int v_dc = tid >> 4, v_kg = tid & 15;
  const bool v_stager = tid < G::V_THREADS;
  u32x4 kreg[G::PER_THREAD];
  u32x2 vreg[4];
  auto gload = [&](int t) {
    const int k0 = t * kBN;
#pragma unroll
    for (int u = 0; u < G::PER_THREAD; ++u) {
      const int ch = u * kThreads + tid;
      const int row = ch / G::CPR, col = ch % G::CPR;
      const int key = k0 + row;
      kreg[u] = key < Nk ? *(const u32x4*)(kg + (int64_t)key * D + col * 16) : (u32x4){0u, 0u, 0u, 0u};
    }
    if (v_stager) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 4 * v_kg + r;
        vreg[r] = key < Nk ? *(const u32x2*)(vg + (int64_t)key * D + v_dc * 8) : (u32x2){0u, 0u};
      }
    }
  };
  auto lstore = [&](int stage) {
    char* kb = smem + stage * G::STAGE;
#pragma unroll
    for (int u = 0; u < G::PER_THREAD; ++u) {
      const int ch = u * kThreads + tid;
      const int row = ch / G::CPR, col = ch % G::CPR;
      if constexpr (QK16) {
        *(u32x4*)(kb + row * G::KS + col * 32) = widen_lo(kreg[u]);
        *(u32x4*)(kb + row * G::KS + col * 32 + 16) = widen_hi(kreg[u]);
      } else {
        *(u32x4*)(kb + row * G::KS + col * 16) = kreg[u];
      }
    }
    if (v_stager) {
      u32x4 w[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = widen_lo((u32x4){vreg[r][0], vreg[r][1], 0u, 0u});
      store_vt(kb + G::K_BYTES, kVtPitch, 8 * v_dc, v_kg, w);
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = (f32x16){};
  float m2 = -INFINITY;  // running max of c_t * raw, base-2 units
  float l_lane = 0.f;

  const int k_off = r32 * G::KS + g * (QK16 ? 16 : 32);
  const int v_off = r32 * kVtPitch + g * 16;

  if (ntiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int stage = t & 1;
    const bool more = t + 1 < ntiles;
    if (more) gload(t + 1);
    const int k0 = t * kBN;
    if (wave_live && k0 < wkend) {
      const char* kb = smem + stage * G::STAGE;
      const char* vb = kb + G::K_BYTES;
      const float c = c_q * ksc[k0 / QT];
      const float sv = vsc[k0 / QT];
      const float vfold = __log2f(sv * inv_svmax);  // <= 0
      const float vunfold = svmax / sv;

      f32x16 s[2];
      s[0] = (f32x16){};
      s[1] = (f32x16){};
      __builtin_amdgcn_s_setprio(1);
      if constexpr (QK16) {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const f16x8 a = *(const f16x8*)(kb + k_off + h * 32 * G::KS + kk * 32);
            s[h] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf16[kk], s[h], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < D / 64; ++kk) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const char* ap = kb + k_off + h * 32 * G::KS + kk * 64;
            const u32x4 a0 = *(const u32x4*)ap;
            const u32x4 a1 = *(const u32x4*)(ap + 16);
            const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                             (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
            s[h] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf8[kk], s[h], 0, 0, 0, 127, 0, 127);
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);

      const bool need_mask = k0 + kBN > wmask_from;
      if (need_mask) {
        const int lim = CAUSAL ? min(my_q + p.diag, Nk - 1) : Nk - 1;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + 32 * h + 8 * (i >> 2) + 4 * g + (i & 3);
            if (key > lim) s[h][i] = -INFINITY;
          }
      }

      float mx = s[0][0];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[h][i]);
      mx = halves_max(mx);
      const float mx2 = mx == -INFINITY ? -INFINITY : mx * c;
      const float m_new = fmaxf(m2, mx2);
      const float alpha = (m2 == -INFINITY) ? 0.f : fast_exp2(m2 - m_new);
      const float bias = (m_new == -INFINITY) ? 0.f : -m_new;
      // P' = p * s_v(t) / s_v_max: the tile's V scale rides in the exponent
      // bias; the normaliser gets p back through one multiply per tile.
      const float bias_v = bias + vfold;
      float rs = 0.f;
      f16x8 pb[2][2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          f32x8 pv;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float x = s[h][half * 8 + j];
            const float e = fast_exp2(fmaf(x, c, bias_v));  // masked: exp2(-inf) = 0 as c > 0
            pv[j] = e;
            rs += e;
          }
          pb[h][half] = __builtin_convertvector(pv, f16x8);
        }
      rs *= vunfold;
      l_lane = alpha * l_lane + rs;
      m2 = m_new;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
      }

      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const f16x8 a = *(const f16x8*)(vb + v_off + db * 32 * kVtPitch + (32 * h + 16 * half) * 2);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[h][half], oacc[db], 0, 0, 0);
          }
      __builtin_amdgcn_s_setprio(0);
    }
    if (more) lstore(stage ^ 1);
    __syncthreads();
  }

  const float l_tot = halves_sum(l_lane);
  const float inv = l_tot > 0.f ? svmax / l_tot : 0.f;  // O = oacc * svmax / l
  if (my_q < Nq) {
    const int64_t row = (int64_t)bh * Nq + my_q;
    float* og = (float*)p.o + row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 v = {oacc[db][4 * r] * inv, oacc[db][4 * r + 1] * inv, oacc[db][4 * r + 2] * inv,
                   oacc[db][4 * r + 3] * inv};
        *(f32x4*)(og + 32 * db + 8 * r + 4 * g) = v;
      }
    if (p.lse && g == 0)
      p.lse[row] = l_tot > 0.f ? (m2 + __log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
  }
}

template <int D, bool QK16>
static hipError_t launch_fp8_d(const FwdParams& p, bool causal, hipStream_t s) {
  const dim3 grid((unsigned)(p.nqb * p.BH));
  if (causal)
    hipLaunchKernelGGL((fwd_fp8_kernel<D, true, QK16>), grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<D, false, QK16>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const FwdParams& p, int d, bool causal, bool qk16, hipStream_t s) {
  if (d == 128) return qk16 ? launch_fp8_d<128, true>(p, causal, s) : launch_fp8_d<128, false>(p, causal, s);
  if (d == 64) return qk16 ? launch_fp8_d<64, true>(p, causal, s) : launch_fp8_d<64, false>(p, causal, s);
  return hipErrorInvalidValue;
}

}  // namespace eta
