// fp32 attention forward for gfx950 on 32x32x2 fp32 MFMA.  Same decomposition
// as the bf16 kernel (query blocks across workgroups, 32 rows per wavefront,
// S^T = K Q^T so each lane holds one row's scores, online softmax with one
// deferred division), but every operand and the probabilities stay fp32.
// The tile loop is single-buffered: this path serves small fp32 problems where
// launch latency, not bandwidth, bounds the time.
//
// 32x32x2 fp32 MFMA layout (lane l, accumulator element i): A holds
// row l%32, k = l/32; B holds column l%32, k = l/32; C/D element i is
// row 8*(i/4) + 4*(l/32) + i%4, column l%32.
#include "common.h"

namespace eta {

constexpr int kBN32 = 32;  // keys per tile

template <int D>
__global__ void __launch_bounds__(kThreads, 1) fwd_f32_kernel(FwdParams p, int causal) {
  constexpr int PITCH = D + 1;  // floats per LDS row (odd pitch: no bank conflicts)
  __shared__ float ks[kBN32 * PITCH];
  __shared__ float vs[kBN32 * PITCH];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r32 = lane & 31;
  const int g = lane >> 5;

  int qb, bh;
  map_block(blockIdx.x, p.nqb, p.BH, causal != 0, qb, bh);
  const int q0 = qb * kBM;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + r32;
  const int Nq = p.Nq, Nk = p.Nk;

  const float* __restrict__ qg = (const float*)p.q + (int64_t)bh * Nq * D;
  const float* __restrict__ kg = (const float*)p.k + (int64_t)bh * Nk * D;
  const float* __restrict__ vg = (const float*)p.v + (int64_t)bh * Nk * D;

  int kend = Nk, wkend = Nk, wmask_from = Nk;
  if (causal) {
    const int last_row = min(q0 + kBM, Nq) - 1;
    kend = min(Nk, last_row + p.diag + 1);
    wkend = min(Nk, min(qw0 + 31, Nq - 1) + p.diag + 1);
    wmask_from = min(Nk, qw0 + p.diag + 1);
  }
  const int ntiles = kend > 0 ? (kend + kBN32 - 1) / kBN32 : 0;
  const bool wave_live = qw0 < Nq;
  const float qsgn = p.q_and == 0u ? 0.f : (p.q_xor ? -1.f : 1.f);

  // Q fragment: B operand, row my_q, element kk holds d = 2*kk + g.
  float qf[D / 2];
  {
    const bool ok = my_q < Nq;
    const float* src = qg + (int64_t)(ok ? my_q : 0) * D + g;
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) qf[kk] = ok ? qsgn * src[2 * kk] : 0.f;
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = (f32x16){};
  float m_raw = -INFINITY, l_lane = 0.f;
  const float c = p.c;

  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * kBN32;
    // Stage the tile: 32 rows x D floats of K and of V, zero past Nk.
    for (int e = tid; e < kBN32 * D; e += kThreads) {
      const int row = e / D, col = e % D;
      const int key = k0 + row;
      const bool ok = key < Nk;
      ks[row * PITCH + col] = ok ? kg[(int64_t)key * D + col] : 0.f;
      vs[row * PITCH + col] = ok ? vg[(int64_t)key * D + col] : 0.f;
    }
    __syncthreads();
    if (wave_live && k0 < wkend) {
      f32x16 s = (f32x16){};
#pragma unroll
      for (int kk = 0; kk < D / 2; ++kk)
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[r32 * PITCH + 2 * kk + g], qf[kk], s, 0, 0, 0);

      const bool need_mask = k0 + kBN32 > wmask_from;
      if (need_mask) {
        const int lim = causal ? min(my_q + p.diag, Nk - 1) : Nk - 1;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + 8 * (i >> 2) + 4 * g + (i & 3);
          if (key > lim) s[i] = -INFINITY;
        }
      }
      float mx = s[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
      mx = halves_max(mx);
      const float m_new = fmaxf(m_raw, mx);
      const float alpha = (m_raw == -INFINITY) ? 0.f : fast_exp2((m_raw - m_new) * c);
      const float bias = (m_new == -INFINITY) ? 0.f : -m_new * c;
      float pr[16];
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(fmaf(s[i], c, bias));  // masked: exp2(-inf) = 0 as c > 0
        pr[i] = e;
        rs += e;
      }
      l_lane = alpha * l_lane + rs;
      m_raw = m_new;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
      // O^T += V^T P^T: MFMA i pairs key 8*(i/4) + 4*g + i%4 of both operands.
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 8 * (i >> 2) + 4 * g + (i & 3);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * PITCH + 32 * db + r32], pr[i], oacc[db], 0, 0, 0);
        }
    }
    __syncthreads();
  }

  const float l_tot = halves_sum(l_lane);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
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
      p.lse[row] = l_tot > 0.f ? m_raw * p.scale_abs + __log2f(l_tot) * 0.69314718055994530942f : -INFINITY;
  }
}

hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, hipStream_t s) {
  const dim3 grid((unsigned)(p.nqb * p.BH));
  if (d == 128)
    hipLaunchKernelGGL((fwd_f32_kernel<128>), grid, dim3(kThreads), 0, s, p, causal ? 1 : 0);
  else if (d == 64)
    hipLaunchKernelGGL((fwd_f32_kernel<64>), grid, dim3(kThreads), 0, s, p, causal ? 1 : 0);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace eta
