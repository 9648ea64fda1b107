// bf16 attention backward for gfx950: dQ, dK, dV of L = sum(dO * O) from the
// saved log-sum-exp, with P recomputed tile by tile (never stored).  The pages
// report training throughput for FlashAttention-2 ("FlashAttention-2",
// Systems analysis wiki, "Performance and efficiency") and a training backward
// for FlashAttention-4 ("Hardware-Aware FP4 FlashAttention-4"), which
// presuppose this pass; they give no formula, so it is the chain rule applied
// to the forward's definition:
//   P_ij = exp(scale q_i.k_j - LSE_i)      dV_j = sum_i P_ij dO_i
//   dP_ij = dO_i . v_j    D_i = dO_i . O_i = sum_j P_ij dP_ij
//   dS_ij = P_ij (dP_ij - D_i)   dQ_i = scale sum_j dS_ij k_j
//   dK_j = scale sum_i dS_ij q_i
//
// Three kernels:
//   bwd_delta_kernel  D_i = dO_i . O_i (fp32), one pass over dO and O.
//   bwd_dq_kernel     query rows stationary (8 wavefronts x 32 rows); K and V
//                     rows stream through LDS in 64-key tiles by buffer->LDS
//                     transfers.  S^T = K Q^T and dP^T = V dO^T put one query
//                     per lane, so LSE_i and D_i are per-lane scalars;
//                     dQ^T += K^T dS^T takes dS^T straight from the
//                     accumulators as the B operand, its K^T fragments read
//                     from the K row tile by transposing reads.
//   bwd_dkdv_kernel   key rows stationary (4 wavefronts x 32 keys, one per
//                     SIMD, so the two fp32 accumulators fit); Q and dO rows
//                     stream through LDS in 64-query tiles by buffer->LDS
//                     transfers (no registers on the way), LSE and D beside
//                     them.  S = Q K^T and dP = dO V^T put one key per lane;
//                     dV^T += dO^T P and dK^T += Q^T dS take P and dS from the
//                     accumulators, their dO^T and Q^T fragments read from the
//                     same row tiles by transposing reads (ds_read_b64_tr_b16).
// Probabilities and dS are rounded to bf16 for the products, accumulations are
// fp32.  Masked (query, key) pairs get p = 0 by selection, so any finite
// scale works.  Rows past the tensor ends read as zero through the range-
// checked transfers (LSE and D: the last row); every (query, key) pair they
// form is masked, so its P and dS are exactly 0.
#include <mutex>
#include <type_traits>

#include "common.h"

namespace eta {

namespace {

constexpr float kLog2e = 1.4426950408889634074f;


__device__ inline bf16x8 pack8(const float* x) {
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  return __builtin_convertvector(v, bf16x8);
}

}  // namespace

// ------------------------------------------------------------------ delta
// 16 threads per row for d = 128 (8 for d = 64), 8 bf16 each, xor-shuffle sum.
template <int D>
__global__ void __launch_bounds__(256) bwd_delta_kernel(BwdParams p, int64_t rows) {
  constexpr int TPR = D / 8;
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *(const u32x4*)((const uint16_t*)p.dout + row * D + c * 8);
    const u32x4 b = *(const u32x4*)((const uint16_t*)p.o + row * D + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc += __uint_as_float(a[e] << 16) * __uint_as_float(b[e] << 16);
      acc += __uint_as_float(a[e] & 0xffff0000u) * __uint_as_float(b[e] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int m = TPR / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m, TPR);
  if (row < rows && c == 0) p.delta[row] = acc;
}

// Slot permutation of the row tiles that both kernels stage (K and V for dQ,
// Q and dO for dK/dV): 16-byte chunk c of row r sits at slot
// c ^ qslot(r).  Even values only, distinct over 8 consecutive rows (16-byte
// row reads of 8 lanes at one chunk hit 8 bank groups) and over the 4 rows of
// a transposing read's 16 lanes, whose two chunks c, c + 1 then land on 8
// distinct slots.  d = 64 packs two rows per 256 bytes, so its rows pair up.
template <int D>
__device__ constexpr int qslot(int r) { return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); }

// --------------------------------------------------------------------- dQ
template <int D>
struct DqGeo {
  static constexpr int W = 8, THREADS = 64 * W, BM = 32 * W, BN = 64, KB = BN / 32;
  static constexpr int KS = D * 2;                      // K / V row pitch (unpadded, chunks permuted)
  static constexpr int K_BYTES = BN * KS, V_BYTES = BN * KS;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int CPR = D / 8;                     // 16-byte chunks per row
  static constexpr int RPT = 64 / CPR;                  // rows per wave-wide 1 KiB transfer
  static constexpr int TPW = K_BYTES / 1024 / W;        // transfers per tensor and wavefront
  static_assert(TPW >= 1 && TPW * W * 1024 == K_BYTES, "K / V tile must be whole transfers per wavefront");
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(512, 1) bwd_dq_kernel(BwdParams p, int nqb) {
  using G = DqGeo<D>;
  __shared__ __attribute__((aligned(16))) char smem[G::LDS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r32 = lane & 31, g = lane >> 5;
  int qb, bh;
  map_block(blockIdx.x, nqb, p.BH, CAUSAL, qb, bh);
  const int Nq = p.Nq, Nk = p.Nk;
  const int q0 = qb * G::BM, qw0 = q0 + wave * 32, my_q = qw0 + r32;
  const uint16_t* __restrict__ qg = (const uint16_t*)p.q + (int64_t)bh * Nq * D;
  const uint16_t* __restrict__ dog = (const uint16_t*)p.dout + (int64_t)bh * Nq * D;
  const uint16_t* __restrict__ kg = (const uint16_t*)p.k + (int64_t)bh * Nk * D;
  const uint16_t* __restrict__ vg = (const uint16_t*)p.v + (int64_t)bh * Nk * D;

  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(q0 + G::BM, Nq) - 1 + p.diag + 1);
  const int ntiles = kend > 0 ? (kend + G::BN - 1) / G::BN : 0;

  // Stationary: Q and dO of this lane's query row (B operands), LSE and D.
  bf16x8 qf[D / 16], dof[D / 16];
  const bool row_ok = my_q < Nq;
  {
    const int64_t rq = (int64_t)min(my_q, Nq - 1) * D + g * 8;
    u32x4 rawq[D / 16], rawd[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      rawq[kk] = *(const u32x4*)(qg + rq + kk * 16);
      rawd[kk] = *(const u32x4*)(dog + rq + kk * 16);
    }
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      qf[kk] = __builtin_bit_cast(bf16x8, row_ok ? rawq[kk] : z);
      dof[kk] = __builtin_bit_cast(bf16x8, row_ok ? rawd[kk] : z);
    }
  }
  const int64_t grow = (int64_t)bh * Nq + my_q;
  const float lse_raw = row_ok ? p.lse[grow] : -INFINITY;
  const bool has_keys = lse_raw != -INFINITY;
  const float lse2 = has_keys ? lse_raw * kLog2e : 0.f;
  const float dlt = row_ok ? p.delta[grow] : 0.f;
  const float c = p.c;
  // every query of this wavefront exists and has a finite LSE
  const bool rows_live = __builtin_amdgcn_readfirstlane(__all(row_ok && has_keys));

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = (f32x16){};

  // Staging: K and V rows go straight from global memory into LDS (range-
  // checked buffer transfers: keys past Nk read as zero and are masked), rows
  // whole, chunks permuted by qslot; wavefront w issues transfers w + W n, so
  // each lane's permuted source chunk is one constant.
  const unsigned kv_lane = [&]() {
    const int row = G::RPT * wave + lane / G::CPR, j = lane % G::CPR;
    return (unsigned)((lane / G::CPR) * G::KS + 16 * (j ^ qslot<D>(row)));
  }();
  const unsigned lds0 = lds_offset(smem);
  auto stage_base = [&](int t) { return smem + (t & 1) * G::STAGE; };
  auto gload = [&](int t) {
    const int k0t = t * G::BN;
    const unsigned nbytes = (unsigned)(max(0, min(G::BN, Nk - k0t)) * G::KS);
    const i32x4 rk = buffer_rsrc_n(kg + (int64_t)k0t * D, nbytes);
    const i32x4 rv = buffer_rsrc_n(vg + (int64_t)k0t * D, nbytes);
    const unsigned sb = lds0 + (unsigned)((t & 1) * G::STAGE);
    unsigned soff = __builtin_amdgcn_readfirstlane(1024u * wave);
    unsigned lds = __builtin_amdgcn_readfirstlane(sb + 1024u * wave);
#pragma unroll
    for (int n = 0; n < G::TPW; ++n) buf_lds16<1024 * G::W, 1024 * G::W>(rk, kv_lane, soff, lds);
    soff = __builtin_amdgcn_readfirstlane(1024u * wave);
    lds = __builtin_amdgcn_readfirstlane(sb + (unsigned)G::K_BYTES + 1024u * wave);
#pragma unroll
    for (int n = 0; n < G::TPW; ++n) buf_lds16<1024 * G::W, 1024 * G::W>(rv, kv_lane, soff, lds);
  };

  // Row fragment (S^T = K Q^T, dP^T = V dO^T; A operand): row r32 of a 32-key
  // block, chunk 2kk + g at slot 2kk ^ (g ^ qslot(r32)).
  const int r_off = r32 * G::KS;
  const int r_x = 16 * (g ^ qslot<D>(r32));
  // K^T fragment (dQ^T += K^T dS^T; A operand: row d = 32 db + l % 32, keys
  // 4g .. 4g+3 and 8+4g .. 8+4g+3 of a 16-key half in dS's order) by two
  // transposing reads, addressed as in the dK/dV kernel below.
  const unsigned t_lane = [&]() {
    const int vq = (lane >> 4) & 1, vm = (lane & 15) >> 2, ve = lane & 3;
    const int row = 4 * g + vm, x = qslot<D>(row), y = 2 * vq + (ve >> 1);
    return (unsigned)(row * G::KS + 16 * (x & ~3) + 16 * (y ^ (x & 3)) + 8 * (ve & 1));
  }();

  if (ntiles > 0) gload(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const bool more = t + 1 < ntiles;
    if (more) gload(t + 1);
    const char* kb = stage_base(t);
    const char* vb = kb + G::K_BYTES;
    const unsigned kb_lds = lds0 + (unsigned)((t & 1) * G::STAGE);
    // Tiles in which every (query, key) pair of this wavefront is live skip
    // the per-element mask; only the probabilities sit under the branch.
    const bool full = __builtin_amdgcn_readfirstlane(
        rows_live && (t + 1) * G::BN <= Nk && (!CAUSAL || (t + 1) * G::BN - 1 <= qw0 + p.diag));
#pragma unroll
    for (int h = 0; h < G::KB; ++h) {
      f32x16 s = (f32x16){}, dp = (f32x16){};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 a = *(const bf16x8*)(kb + h * 32 * G::KS + r_off + ((kk * 32) ^ r_x));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s, 0, 0, 0);
        const bf16x8 b = *(const bf16x8*)(vb + h * 32 * G::KS + r_off + ((kk * 32) ^ r_x));
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, dof[kk], dp, 0, 0, 0);
      }
      float pr[16], ds[16];
      if (full) {
#pragma unroll
        for (int i = 0; i < 16; ++i) pr[i] = fast_exp2(fmaf(s[i], c, -lse2));
      } else {
        const int kbase = t * G::BN + 32 * h + 4 * g;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kbase + 8 * (i >> 2) + (i & 3);
          const bool ok = has_keys && key < Nk && (!CAUSAL || key <= my_q + p.diag);
          pr[i] = ok ? fast_exp2(fmaf(s[i], c, -lse2)) : 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) ds[i] = pr[i] * (dp[i] - dlt);
      const bf16x8 pd[2] = {pack8(ds), pack8(ds + 8)};
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const unsigned ad = ((kb_lds + t_lane) ^ (unsigned)(64 * db)) + (unsigned)((32 * h + 16 * half) * G::KS);
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)ad);
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(ad + 8 * G::KS));
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pd[half], acc[db], 0, 0, 0);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // tile t + 1's transfers: counted by vmcnt only, not covered by the barrier
    __syncthreads();
  }

  if (!row_ok) return;
  uint16_t* out = (uint16_t*)p.dq + grow * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      f32x4 v = {acc[db][4 * r] * p.scale, acc[db][4 * r + 1] * p.scale, acc[db][4 * r + 2] * p.scale,
                 acc[db][4 * r + 3] * p.scale};
      *(bf16x4*)(out + 32 * db + 8 * r + 4 * g) = __builtin_convertvector(v, bf16x4);
    }
}

// ----------------------------------------------------------------- dK, dV
template <int D>
struct DkvGeo {
  static constexpr int W = 4, THREADS = 64 * W, BK = 32 * W, BM = 64, QB = BM / 32;
  static constexpr int KS = D * 2;                      // Q / dO row pitch (unpadded, chunks permuted)
  static constexpr int R_BYTES = BM * KS;
  static constexpr int STAGE = 2 * R_BYTES + 2 * BM * 4;  // Q, dO, LSE2, D
  static constexpr int LDS = 2 * STAGE;
  static constexpr int CPR = D / 8;                     // 16-byte chunks per row
  static constexpr int RPT = 64 / CPR;                  // rows per wave-wide 1 KiB transfer
  static constexpr int TPW = R_BYTES / 1024 / W;        // transfers per tensor and wavefront
  static_assert(TPW * W * 1024 == R_BYTES, "Q / dO tile must be whole transfers per wavefront");
  static_assert(2 * BM <= THREADS, "LSE and D loaded by one thread each");
};


template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 1) bwd_dkdv_kernel(BwdParams p, int nkb) {
  using G = DkvGeo<D>;
  __shared__ __attribute__((aligned(16))) char smem[G::LDS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r32 = lane & 31, g = lane >> 5;
  int kb_idx, bh;
  // key blocks in ascending order come first: under a causal mask the first
  // keys are seen by the most queries
  map_block(blockIdx.x, nkb, p.BH, false, kb_idx, bh);
  const int Nq = p.Nq, Nk = p.Nk;
  const int k0 = kb_idx * G::BK, kw0 = k0 + wave * 32, my_k = kw0 + r32;
  const uint16_t* __restrict__ qg = (const uint16_t*)p.q + (int64_t)bh * Nq * D;
  const uint16_t* __restrict__ dog = (const uint16_t*)p.dout + (int64_t)bh * Nq * D;
  const uint16_t* __restrict__ kg = (const uint16_t*)p.k + (int64_t)bh * Nk * D;
  const uint16_t* __restrict__ vg = (const uint16_t*)p.v + (int64_t)bh * Nk * D;
  const float* __restrict__ lseg = p.lse + (int64_t)bh * Nq;
  const float* __restrict__ dltg = p.delta + (int64_t)bh * Nq;

  // Queries that see some key of this block: i >= k0 - diag under the mask.
  const int q_first = CAUSAL ? max(0, k0 - p.diag) : 0;
  const int t0 = q_first / G::BM;
  const int ntiles = q_first < Nq ? (Nq + G::BM - 1) / G::BM : 0;

  // Stationary: K and V of this lane's key (B operands).
  bf16x8 kf[D / 16], vf[D / 16];
  const bool key_ok = my_k < Nk;
  {
    const int64_t rk = (int64_t)min(my_k, Nk - 1) * D + g * 8;
    u32x4 rawk[D / 16], rawv[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      rawk[kk] = *(const u32x4*)(kg + rk + kk * 16);
      rawv[kk] = *(const u32x4*)(vg + rk + kk * 16);
    }
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      kf[kk] = __builtin_bit_cast(bf16x8, key_ok ? rawk[kk] : z);
      vf[kk] = __builtin_bit_cast(bf16x8, key_ok ? rawv[kk] : z);
    }
  }
  const float c = p.c;
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dk[db] = dv[db] = (f32x16){};

  // Staging.  Q and dO rows go straight from global memory into LDS (buffer
  // loads with an LDS destination, range-checked: rows past Nq read as zero
  // and every pair they form is masked), rows whole, chunks permuted by
  // qslot.  Wavefront w issues transfers w + W n, so each lane's row within a
  // transfer, and with it its permuted source chunk, is one constant.
  // Threads 0 .. BM-1 fetch LSE2, BM .. 2BM-1 fetch D, through registers.
  const unsigned q_lane = [&]() {
    const int row = G::RPT * wave + lane / G::CPR, j = lane % G::CPR;
    return (unsigned)((lane / G::CPR) * G::KS + 16 * (j ^ qslot<D>(row)));
  }();
  const unsigned lds0 = lds_offset(smem);
  float sval = 0.f;
  const float* __restrict__ sbase = (tid < G::BM ? lseg : dltg) + (tid % G::BM);
  const float* sptr = sbase;
  auto stage_base = [&](int t) { return smem + (t & 1) * G::STAGE; };
  auto gload = [&](int t) {
    const int q0t = t * G::BM;
    const unsigned nbytes = (unsigned)(max(0, min(G::BM, Nq - q0t)) * G::KS);
    const i32x4 rq = buffer_rsrc_n(qg + (int64_t)q0t * D, nbytes);
    const i32x4 rd = buffer_rsrc_n(dog + (int64_t)q0t * D, nbytes);
    const unsigned sb = lds0 + (unsigned)((t & 1) * G::STAGE);
    unsigned soff = __builtin_amdgcn_readfirstlane(1024u * wave);
    unsigned lds = __builtin_amdgcn_readfirstlane(sb + 1024u * wave);
#pragma unroll
    for (int n = 0; n < G::TPW; ++n) buf_lds16<1024 * G::W, 1024 * G::W>(rq, q_lane, soff, lds);
    soff = __builtin_amdgcn_readfirstlane(1024u * wave);
    lds = __builtin_amdgcn_readfirstlane(sb + (unsigned)G::R_BYTES + 1024u * wave);
#pragma unroll
    for (int n = 0; n < G::TPW; ++n) buf_lds16<1024 * G::W, 1024 * G::W>(rd, q_lane, soff, lds);
    if (tid < 2 * G::BM) {  // raw LSE or D; converted when staged
      // Full tiles read through a pointer carried across the tile loop, so
      // its registers are never recycled while the load is in flight (that
      // would cost a wait for every outstanding load); the last, ragged tile
      // clamps its row.
      if (q0t + G::BM <= Nq) sval = *(sptr + q0t);
      else sval = sbase[min(q0t + (tid % G::BM), Nq - 1) - (tid % G::BM)];
    }
  };
  auto lstore = [&](int t) {
    char* b = stage_base(t);
    if (tid < 2 * G::BM) {
      // LSE in base 2 (rows without keys, LSE = -inf, are masked anyway), or D
      const float v = tid < G::BM ? (sval == -INFINITY ? 0.f : sval * kLog2e) : sval;
      ((float*)(b + 2 * G::R_BYTES))[tid] = v;
    }
  };

  // Row fragment (S = Q K^T, dP = dO V^T; A operand): row r32 of a 32-row
  // block, chunk 2kk + g at slot (2kk + g) ^ qslot(r32) = 2kk ^ (g ^ qslot(r32)).
  const int r_off = r32 * G::KS;
  const int r_x = 16 * (g ^ qslot<D>(r32));
  // Transposed fragment (dV^T += dO^T P, dK^T += Q^T dS; A operand: row d =
  // 32 db + l % 32, queries 4g .. 4g+3 and 8+4g .. 8+4g+3 of a 16-query half
  // in P's order) by two transposing reads: lane (q, m, e) = ((l / 16) % 2,
  // (l % 16) / 4, l % 4) addresses query 4g + m (and 8 on), columns 32 db +
  // 16 q + 4 e, i.e. chunk 4 db + 2 q + e / 2, byte 8 (e % 2).  The slot
  // permutation is even and the row's part of it is the same 8 rows on, so
  // chunk (4 db + y) ^ x = (4 db ^ (x & ~3)) + (y ^ (x & 3)): the column block
  // enters as an XOR of 64 db on the byte address.
  const unsigned t_lane = [&]() {
    const int vq = (lane >> 4) & 1, vm = (lane & 15) >> 2, ve = lane & 3;
    const int row = 4 * g + vm, x = qslot<D>(row), y = 2 * vq + (ve >> 1);
    return (unsigned)(row * G::KS + 16 * (x & ~3) + 16 * (y ^ (x & 3)) + 8 * (ve & 1));
  }();

  if (ntiles > t0) {
    gload(t0);
    lstore(t0);
  }
  // All loads so far (the stationary K and V too) have landed: said
  // explicitly, so that no wait for them is left inside the tile loop.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // One query tile.  ALL_LIVE: every (query, key) pair of the workgroup is
  // live, so the body has no mask and no branch, and the scheduler may
  // overlap one block's P/dS with the other block's products.
  auto step = [&](int t, auto live_tag) __attribute__((always_inline)) {
    constexpr bool ALL_LIVE = decltype(live_tag)::value;
    const bool more = t + 1 < ntiles;
    if (more) gload(t + 1);
    const char* qb = stage_base(t);
    const char* dob = qb + G::R_BYTES;
    const float* l2 = (const float*)(qb + 2 * G::R_BYTES);
    const float* dl = l2 + G::BM;
    const unsigned qb_lds = lds0 + (unsigned)((t & 1) * G::STAGE);
    // The tile's 64 MFMAs, in issue order (h: 32-query block):
    //   0 .. 31   S[h] and dP[h], h = i / 16, k-slice (i / 2) % 8, S / dP
    //   32 .. 63  dV^T and dK^T, h = (i - 32) / 16, then half, column block,
    //             dV / dK
    // Each needs one A fragment from LDS; the reads run RA MFMAs ahead.  The
    // P and dS of block 0 are formed between block 1's S / dP products, those
    // of block 1 between block 0's dV / dK products (16 / (D / 8) elements
    // per MFMA).
    // The source order is the schedule.
    constexpr int NSD = G::QB * (D / 16) * 2;  // S and dP products
    constexpr int NKV = G::QB * 2 * (D / 32) * 2;  // dV and dK products
    constexpr int NM = NSD + NKV;
    constexpr int PER = NSD / G::QB;  // products per block in each phase (D / 8)
    constexpr int EPS = 16 / PER;     // elements of P / dS per MFMA slot
    constexpr int RA = 8;
    static_assert(NKV / G::QB == PER && EPS * PER == 16, "P / dS elements spread evenly over a phase");
    f32x4 lv[G::QB][4], dv4[G::QB][4];
#pragma unroll
    for (int h = 0; h < G::QB; ++h)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        lv[h][blk] = *(const f32x4*)(l2 + 32 * h + 8 * blk + 4 * g);
        dv4[h][blk] = *(const f32x4*)(dl + 32 * h + 8 * blk + 4 * g);
      }
    auto frag = [&](int i) {
      if (i < NSD) {
        const int h = i / PER, kk = (i / 2) % (D / 16), w = i % 2;
        return *(const bf16x8*)((w ? dob : qb) + h * 32 * G::KS + r_off + ((kk * 32) ^ r_x));
      }
      const int j = i - NSD, h = j / PER, half = (j / 2) / (D / 32) % 2, db = (j / 2) % (D / 32), w = j % 2;
      // w = 0: dO^T (dV), w = 1: Q^T (dK)
      const unsigned a = ((qb_lds + (unsigned)(w ? 0 : G::R_BYTES) + t_lane) ^ (unsigned)(64 * db)) +
                         (unsigned)((32 * h + 16 * half) * G::KS);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(a + 8 * G::KS));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    f32x16 s[G::QB], dp[G::QB];
    float pr[16], ds[16];
    bf16x8 pp[G::QB][2], pd[G::QB][2];
    // element e of block h: query 32h + 8(e/4) + 4g + e%4 of the tile, key my_k
    auto elem = [&](int h, int e) {
      float v = fast_exp2(fmaf(s[h][e], c, -lv[h][e / 4][e % 4]));
      if constexpr (!ALL_LIVE) {
        const int q = t * G::BM + 32 * h + 8 * (e / 4) + 4 * g + e % 4;
        if (!(key_ok && q < Nq && (!CAUSAL || my_k <= q + p.diag))) v = 0.f;
      }
      pr[e] = v;
      ds[e] = v * (dp[h][e] - dv4[h][e / 4][e % 4]);
      if (e == 7) {
        pp[h][0] = pack8(pr);
        pd[h][0] = pack8(ds);
      } else if (e == 15) {
        pp[h][1] = pack8(pr + 8);
        pd[h][1] = pack8(ds + 8);
      }
    };
    bf16x8 fa[RA];
#pragma unroll
    for (int i = 0; i < RA; ++i) fa[i] = frag(i);
    // Unrolled at compile time (every array index below is a constant).
    static_for<0, NM>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      const bf16x8 a = fa[i % RA];
      if (i < NSD) {
        const int h = i / PER, kk = (i / 2) % (D / 16);
        if (i % 2 == 0)
          s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[kk], kk == 0 ? (f32x16){} : s[h], 0, 0, 0);
        else
          dp[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vf[kk], kk == 0 ? (f32x16){} : dp[h], 0, 0, 0);
      } else {
        const int j = i - NSD, h = j / PER, half = (j / 2) / (D / 32) % 2, db = (j / 2) % (D / 32);
        if (j % 2 == 0)
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pp[h][half], dv[db], 0, 0, 0);
        else
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pd[h][half], dk[db], 0, 0, 0);
      }
      if (i + RA < NM) fa[i % RA] = frag(i + RA);
      // P / dS of block 0 during block 1's S / dP, of block 1 during block 0's dV / dK
#pragma unroll
      for (int u = 0; u < EPS; ++u) {
        if (i >= PER && i < 2 * PER) elem(0, (i - PER) * EPS + u);
        if (i >= NSD && i < NSD + PER) elem(1, (i - NSD) * EPS + u);
      }
      // Keep this order: with one wavefront per SIMD nothing else hides the
      // LDS latency, and the scheduler would otherwise sink the reads to
      // their MFMAs to save registers.
      __builtin_amdgcn_sched_barrier(0);
    });
    if (more) lstore(t + 1);
    __builtin_amdgcn_s_waitcnt(0);  // tile t + 1's transfers: counted by vmcnt only, not covered by the barrier
    __syncthreads();
  };
  // Tiles t_lo .. t_hi-1 are all-live: every key of the block exists, the
  // tile is whole and, under the causal mask, lies wholly below the diagonal.
  int t_lo = ntiles, t_hi = ntiles;
  if (k0 + G::BK <= Nk) {
    t_hi = max(t0, Nq / G::BM);
    t_lo = t0;
    const int need = k0 + G::BK - 1 - p.diag;  // first query that sees every key
    if (CAUSAL && need > 0) t_lo = max(t0, (need + G::BM - 1) / G::BM);
    t_lo = min(t_lo, t_hi);
  }
  int t = t0;
  for (; t < t_lo; ++t) step(t, std::false_type{});
  for (; t < t_hi; ++t) step(t, std::true_type{});
  for (; t < ntiles; ++t) step(t, std::false_type{});

  if (!key_ok) return;
  const int64_t grow = (int64_t)bh * Nk + my_k;
  uint16_t* outk = (uint16_t*)p.dk + grow * D;
  uint16_t* outv = (uint16_t*)p.dv + grow * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      f32x4 a = {dk[db][4 * r] * p.scale, dk[db][4 * r + 1] * p.scale, dk[db][4 * r + 2] * p.scale,
                 dk[db][4 * r + 3] * p.scale};
      f32x4 b = {dv[db][4 * r], dv[db][4 * r + 1], dv[db][4 * r + 2], dv[db][4 * r + 3]};
      *(bf16x4*)(outk + 32 * db + 8 * r + 4 * g) = __builtin_convertvector(a, bf16x4);
      *(bf16x4*)(outv + 32 * db + 8 * r + 4 * g) = __builtin_convertvector(b, bf16x4);
    }
}

// --------------------------------------------------------------- launcher
// The dQ and dK/dV kernels read the same inputs and write disjoint outputs, so
// dQ runs on a second stream, concurrently with dK/dV: each kernel's last,
// partly empty round of workgroups then shares the chip with the other's
// work.  Per device: that stream and the fork / join events, created on the
// first call and kept until the process ends.  The mutex makes each call's
// record / wait sequence atomic, so concurrent callers cannot interleave on
// the shared events.
namespace {
struct BwdSide {
  std::mutex mu;
  bool ready = false;
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kBwdMaxDevices = 64;
BwdSide g_bwd_side[kBwdMaxDevices];

hipError_t side_init(BwdSide& c) {
  if (c.ready) return hipSuccess;
  if (hipError_t e = hipStreamCreateWithFlags(&c.stream, hipStreamNonBlocking)) return e;
  if (hipError_t e = hipEventCreateWithFlags(&c.fork, hipEventDisableTiming)) return e;
  if (hipError_t e = hipEventCreateWithFlags(&c.join, hipEventDisableTiming)) return e;
  c.ready = true;
  return hipSuccess;
}
}  // namespace

template <int D>
static hipError_t launch_bwd_d(const BwdParams& p, bool causal, hipStream_t s) {
  const int64_t rows = (int64_t)p.BH * p.Nq;
  const int64_t dblocks = (rows * (D / 8) + 255) / 256;
  hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)dblocks), dim3(256), 0, s, p, rows);
  if (hipError_t e = hipGetLastError()) return e;
  const int nkb = (p.Nk + DkvGeo<D>::BK - 1) / DkvGeo<D>::BK;
  const int nqb = (p.Nq + DqGeo<D>::BM - 1) / DqGeo<D>::BM;
  const dim3 gkv((unsigned)(nkb * p.BH)), gq((unsigned)(nqb * p.BH));
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (dev < 0 || dev >= kBwdMaxDevices) return hipErrorInvalidDevice;
  BwdSide& c = g_bwd_side[dev];
  std::lock_guard<std::mutex> lock(c.mu);
  if (hipError_t e = side_init(c)) return e;
  // dQ on the side stream once D is written; the caller's stream waits for it.
  if (hipError_t e = hipEventRecord(c.fork, s)) return e;
  if (hipError_t e = hipStreamWaitEvent(c.stream, c.fork, 0)) return e;
  if (causal)
    hipLaunchKernelGGL((bwd_dq_kernel<D, true>), gq, dim3(DqGeo<D>::THREADS), 0, c.stream, p, nqb);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, false>), gq, dim3(DqGeo<D>::THREADS), 0, c.stream, p, nqb);
  if (hipError_t e = hipGetLastError()) return e;
  if (hipError_t e = hipEventRecord(c.join, c.stream)) return e;
  if (causal)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), gkv, dim3(DkvGeo<D>::THREADS), 0, s, p, nkb);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), gkv, dim3(DkvGeo<D>::THREADS), 0, s, p, nkb);
  if (hipError_t e = hipGetLastError()) return e;
  return hipStreamWaitEvent(s, c.join, 0);
}

hipError_t launch_bwd(const BwdParams& p, int d, bool causal, hipStream_t s) {
  if (d == 128) return launch_bwd_d<128>(p, causal, s);
  if (d == 64) return launch_bwd_d<64>(p, causal, s);
  return hipErrorInvalidValue;
}

}  // namespace eta
