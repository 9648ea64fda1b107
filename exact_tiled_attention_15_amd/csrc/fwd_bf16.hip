// bf16 attention forward for gfx950: S^T = K Q^T and O^T += V^T P^T on
// 32x32x16 bf16 MFMA, online softmax in registers, K/V tiles double-buffered
// through LDS.
//
// Structure follows "FlashAttention-2" (Systems analysis wiki, "Technical
// architecture and working principles"): the outer loop is over query blocks
// (one workgroup each, all spread over the compute units, item 2), the inner
// loop streams K/V tiles; O stays unnormalised in registers and is divided by
// the running normaliser once after the loop (item 1); each wavefront owns 32
// whole query rows, so row statistics need no exchange between wavefronts
// (item 3).  The running max / normaliser update is the online softmax of
// "Sequence parallelism and ring attention" ("Technical insight").
//
// Register layouts (32x32xK MFMA on gfx950, lane l, accumulator element i):
//   A operand: row l%32, k-slice (l/32)*8 .. +8      B operand: column l%32
//   C/D:       row 8*(i/4) + 4*(l/32) + i%4, column l%32
// Computing S^T (rows = keys, columns = queries) leaves each lane with one
// query's scores for 16 keys of a 32-key block, so row max / sum are in-lane
// plus one permlane32 swap, and the scores feed O^T = V^T P^T as the B
// operand without any data movement.  V^T fragments come from the row-major V
// tile through ds_read_b64_tr_b16.
#include "common.h"

namespace eta {

template <int D>
struct Geo {
  static constexpr int ROW = D * 2;             // bytes in one bf16 row
  static constexpr int KS = ROW + 16;           // K tile row pitch (bytes)
  static constexpr int VS = ROW + 64;           // V tile row pitch (bytes)
  static constexpr int K_BYTES = kBN * KS;
  static constexpr int V_BYTES = kBN * VS;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int LDS = 2 * STAGE;         // double buffered
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int PER_THREAD = kBN * CPR / kThreads;
  static_assert(PER_THREAD * kThreads == kBN * CPR, "tile must split evenly");
};

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ inline bf16x8 pack_bf16(const float* x) {
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  return __builtin_convertvector(v, bf16x8);
}

template <int D, bool CAUSAL, int EPI>
__global__ void __launch_bounds__(kThreads, 2) fwd_bf16_kernel(FwdParams p) {
  using G = Geo<D>;
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

  const uint16_t* __restrict__ qg = (const uint16_t*)p.q + (int64_t)bh * Nq * D;
  const uint16_t* __restrict__ kg = (const uint16_t*)p.k + (int64_t)bh * Nk * D;
  const uint16_t* __restrict__ vg = (const uint16_t*)p.v + (int64_t)bh * Nk * D;

  // Key range of the workgroup (kend) and of this wavefront (wkend); tiles at
  // or beyond kend are skipped wholesale.
  int kend = Nk, wkend = Nk, wmask_from = Nk;
  if (CAUSAL) {
    const int last_row = min(q0 + kBM, Nq) - 1;
    kend = min(Nk, last_row + p.diag + 1);
    wkend = min(Nk, min(qw0 + 31, Nq - 1) + p.diag + 1);
    wmask_from = min(Nk, qw0 + p.diag + 1);  // first key hidden from row qw0
  }
  const int ntiles = kend > 0 ? (kend + kBN - 1) / kBN : 0;
  const bool wave_live = qw0 < Nq;

  // Q fragment (B operand of S^T = K Q^T): row my_q, d = kk*16 + g*8 .. +8.
  bf16x8 qf[D / 16];
  {
    const bool ok = my_q < Nq;
    const u32x4* src = (const u32x4*)(qg + (int64_t)(ok ? my_q : 0) * D + g * 8);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 x = ok ? src[kk * 2] : (u32x4){0u, 0u, 0u, 0u};
      x ^= p.q_sign;
      qf[kk] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // Global -> register -> LDS staging of one K/V tile.
  u32x4 kreg[G::PER_THREAD], vreg[G::PER_THREAD];
  auto gload = [&](int t) {
    const int k0 = t * kBN;
#pragma unroll
    for (int u = 0; u < G::PER_THREAD; ++u) {
      const int ch = u * kThreads + tid;
      const int row = ch / G::CPR, col = ch % G::CPR;
      const int key = k0 + row;
      if (key < Nk) {
        kreg[u] = *(const u32x4*)(kg + (int64_t)key * D + col * 8);
        vreg[u] = *(const u32x4*)(vg + (int64_t)key * D + col * 8);
      } else {
        kreg[u] = (u32x4){0u, 0u, 0u, 0u};
        vreg[u] = (u32x4){0u, 0u, 0u, 0u};
      }
    }
  };
  auto lstore = [&](int stage) {
    char* kb = smem + stage * G::STAGE;
    char* vb = kb + G::K_BYTES;
#pragma unroll
    for (int u = 0; u < G::PER_THREAD; ++u) {
      const int ch = u * kThreads + tid;
      const int row = ch / G::CPR, col = ch % G::CPR;
      *(u32x4*)(kb + row * G::KS + col * 16) = kreg[u];
      *(u32x4*)(vb + row * G::VS + col * 16) = vreg[u];
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = (f32x16){};
  float m_raw = -INFINITY;  // running max of the raw dot product q.k
  float l_lane = 0.f;       // this lane's share of the running normaliser
  const float c = p.c;

  // Per-lane LDS byte offsets. K: row r32, 16-byte slice g.  V (transposed
  // read): source lane s = lane%16 addresses key 4g + s/4, columns
  // 16*((lane/16)%2) + 4*(s%4) .. +4, so result lane r of each 16-lane group
  // receives 4 consecutive keys of column r.
  const int k_off = r32 * G::KS + g * 16;
  const int s16 = lane & 15;
  const int v_off = (4 * g + (s16 >> 2)) * G::VS + (16 * ((lane >> 4) & 1) + 4 * (s16 & 3)) * 2;

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

      // S^T for two 32-key blocks h.
      f32x16 s[2];
      s[0] = (f32x16){};
      s[1] = (f32x16){};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bf16x8 a = *(const bf16x8*)(kb + k_off + h * 32 * G::KS + kk * 32);
          s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[h], 0, 0, 0);
        }
      }

      // Mask keys beyond the causal limit or the end of K (diagonal / tail
      // tiles only).
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

      // Online softmax update (base-2 exponent, scale folded into one FMA).
      float mx = s[0][0];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[h][i]);
      mx = halves_max(mx);
      const float m_new = fmaxf(m_raw, mx);
      const float alpha = (m_raw == -INFINITY) ? 0.f : fast_exp2((m_raw - m_new) * c);
      const float bias = (m_new == -INFINITY) ? 0.f : -m_new * c;
      float rs = 0.f;
      bf16x8 pb[2][2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          float pv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float x = s[h][half * 8 + j];
            float e = fast_exp2(fmaf(x, c, bias));
            if (need_mask && x == -INFINITY) e = 0.f;
            pv[j] = e;
            rs += e;
          }
          pb[h][half] = pack_bf16(pv);
        }
      l_lane = alpha * l_lane + rs;
      m_raw = m_new;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
      }

      // O^T += V^T P^T.
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int key_off = (32 * h + 16 * half) * G::VS;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const char* base = vb + v_off + key_off + db * 64;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 8 * G::VS));
            const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[h][half], oacc[db], 0, 0, 0);
          }
        }
    }
    if (more) lstore(stage ^ 1);
    __syncthreads();
  }

  // Epilogue: one division by the normaliser, one write of O.
  const float l_tot = halves_sum(l_lane);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (my_q < Nq) {
    const int64_t row = (int64_t)bh * Nq + my_q;
    if (EPI == kEpiFinalBf16) {
      uint16_t* og = (uint16_t*)p.o + row * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          f32x4 v = {oacc[db][4 * r] * inv, oacc[db][4 * r + 1] * inv, oacc[db][4 * r + 2] * inv,
                     oacc[db][4 * r + 3] * inv};
          *(bf16x4*)(og + 32 * db + 8 * r + 4 * g) = __builtin_convertvector(v, bf16x4);
        }
      if (p.lse && g == 0)
        p.lse[row] = l_tot > 0.f ? m_raw * p.scale_abs + __log2f(l_tot) * 0.69314718055994530942f : -INFINITY;
    } else {
      float* og = (float*)p.o + row * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          f32x4 v = {oacc[db][4 * r] * inv, oacc[db][4 * r + 1] * inv, oacc[db][4 * r + 2] * inv,
                     oacc[db][4 * r + 3] * inv};
          *(f32x4*)(og + 32 * db + 8 * r + 4 * g) = v;
        }
      if (g == 0) {
        if (EPI == kEpiState) {
          p.m_out[row] = l_tot > 0.f ? m_raw * p.scale_abs : -INFINITY;
          p.l_out[row] = l_tot;
        } else if (p.lse) {
          p.lse[row] = l_tot > 0.f ? m_raw * p.scale_abs + __log2f(l_tot) * 0.69314718055994530942f : -INFINITY;
        }
      }
    }
  }
}

template <int D, bool CAUSAL, int EPI>
static hipError_t launch_one(const FwdParams& p, hipStream_t s) {
  const dim3 grid((unsigned)(p.nqb * p.BH));
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, EPI>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int D, int EPI>
static hipError_t launch_d(const FwdParams& p, bool causal, hipStream_t s) {
  return causal ? launch_one<D, true, EPI>(p, s) : launch_one<D, false, EPI>(p, s);
}

hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, int epi, hipStream_t s) {
  if (d == 128) {
    if (epi == kEpiFinalBf16) return launch_d<128, kEpiFinalBf16>(p, causal, s);
    if (epi == kEpiState) return launch_d<128, kEpiState>(p, causal, s);
  } else if (d == 64) {
    if (epi == kEpiFinalBf16) return launch_d<64, kEpiFinalBf16>(p, causal, s);
    if (epi == kEpiState) return launch_d<64, kEpiState>(p, causal, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace eta
