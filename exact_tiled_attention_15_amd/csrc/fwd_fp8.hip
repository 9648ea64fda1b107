// Block-quantized fp8 (OCP e4m3) attention forward for gfx950.
//
// Inputs are e4m3 codes with one fp32 scale per (b, h, 128-token tile), the
// block quantization of "Scaling FlashAttention, multi-GPU training and weight
// quantization" (itimpress, section 1, FP8 bullet).  The decomposition is the
// bf16 kernel's (fwd_bf16.hip: 256-row workgroups of 8 wavefronts, 128-key
// tiles double-buffered through LDS, online softmax in registers, V stored
// transposed), with:
//   * S^T = K Q^T on the 32x32x64 f8f6f4 MFMA (both operands e4m3, unit block
//     scales), or - the QK16 instantiation - on the 32x32x16 fp16 MFMA with
//     the codes widened exactly to fp16.  The fp8 MFMA sums the products of
//     one instruction with limited alignment precision (measured on gfx950:
//     one 448*448 product among small ones leaves an error of ~34 on a sum of
//     2e5), so channels with large outliers need the rotation of the same
//     passage ("incoherent processing") before quantization; the fp16 form is
//     exact for any codes.  A wavefront's 32 rows lie in one query scale tile
//     and a 128-key iteration is exactly one key scale tile, so the product of
//     the two fp32 scales is one scalar per (wavefront, iteration), folded into
//     the softmax FMA: c_t = |scale| * log2(e) * s_q * s_k(t).
//   * P V on the 32x32x16 fp16 MFMA: V codes are converted exactly to fp16
//     while staged into LDS; the probabilities are rounded to fp16 as
//     p * s_v(t) / max_t s_v (the ratio folded into the exponent bias), with
//     p taken against a reference maximum that moves only when the row's
//     maximum passes it by more than 2^8, so the value is <= 2^8 for any
//     scales and O is rarely rescaled; the normaliser is summed from the
//     unrounded fp32 values with the ratio divided out once per tile.
//   * PV8 instantiation (the FlashAttention-3 FP8 form of the same passage,
//     probabilities in fp8 too): P V on the 32x32x64 f8f6f4 MFMA with V's
//     codes used as they are.  A lane's 32 scores of a 64-key group are
//     exactly the 32 bytes its B operand needs, so P goes from the
//     accumulators into e4m3 bytes with no data movement; V^T is stored in
//     LDS as codes, keys permuted so that the A operand's k order matches
//     (common slot formula in vt8_slot below).  P is quantized as
//     p * s_v(t) / max s_v * 2^8 (<= 256 < 448, and small probabilities stay
//     representable) and the MFMA's E8M0 block scale 2^-8 on P undoes the
//     factor exactly; the normaliser sums the rounded values.  e4m3 keeps 3
//     mantissa bits, so this trades accuracy for speed: the result drifts from
//     exact attention by the rounding of P (measured, not held to the parity
//     bar).
//   * PV4 instantiations (the FP4 probabilities of "Hardware-Aware FP4
//     FlashAttention-4", gist.science summary): P.V on the same f8f6f4 MFMA
//     with P as 4-bit e2m1 codes (B operand) against V's e4m3 codes (A).  P
//     is quantized as 4 p s_v(t) / max s_v (<= 4) and the block scale 2^-2
//     on P undoes the factor.  Either the exponential is rounded by the
//     hardware conversion (nearest even), or - Direct-P - the score's base-2
//     exponent relative to the running maximum is mapped straight to the code
//     index with no exponential (index = clamp(round(2 log2(4 p) + 2), 0, 6),
//     which matches nearest-even rounding of 4p from 0.59 up and flushes
//     smaller values to 0).  With a 4-bit B operand the instruction takes k
//     = 16g .. 16g+15 and 32+16g .. 32+16g+15 from lane half g (measured), so
//     V^T uses its own key order (vt4_slot).  The normaliser sums the decoded
//     codes.  One mantissa bit: a speed-for-accuracy mode, drift measured.
//   * O accumulates and is written in fp32.
// For the f8f6f4 MFMA the A/B k-slice of lane l is bytes (l/32)*32 .. +32.
#include "common.h"

namespace eta {

constexpr int kQuantTile = 128;  // tokens per quantization tile
// fp16 probabilities are taken against a reference maximum that moves only
// when a row's maximum passes it by more than this many powers of two.
constexpr float kLazyLog2 = 8.f;

// How P.V runs: fp16 P against fp16-widened V codes, or P in e4m3 / e2m1
// against V's e4m3 codes on the f8f6f4 MFMA (e2m1 by rounding the exponential,
// or by mapping the score straight to the code: Direct-P).
enum PvMode : int { kPvF16 = 0, kPvFp8 = 1, kPvFp4 = 2, kPvFp4Direct = 3 };

template <int D, bool QK16, bool PV8, int W, int BN>
struct Geo8 {
  static constexpr int THREADS = 64 * W;
  static constexpr int BM = 32 * W;
  static constexpr int KB = BN / 32;
  static constexpr int VTP = vt_pitch(BN);
  static constexpr int KROW = QK16 ? 2 * D : D;   // bytes of one staged K row
  static constexpr int KS = KROW + 16;            // K tile row pitch (bytes)
  static constexpr int K_BYTES = BN * KS;
  static constexpr int VTP8 = BN + 16;            // fp8 V^T row pitch (bytes)
  static constexpr int V_BYTES = PV8 ? D * VTP8 : D * VTP;  // V^T: one row per column d
  static constexpr int LDS = 2 * K_BYTES + 2 * V_BYTES;
  static constexpr int CPR = D / 16;              // 16-byte code chunks per row
  static constexpr int K_SLOTS = KS / 16;         // 16-byte LDS slots per K row (pad included)
  static constexpr int K_LOADS = BN * K_SLOTS / 64;  // direct-load form: wave-wide loads per tile
  static constexpr int K_PER_THREAD = BN * CPR / THREADS;  // widened form: chunks per thread
  static constexpr int KG = BN / 4;
  static constexpr int V_THREADS = KG * (D / 8);
  static_assert(BN <= kQuantTile && kQuantTile % BN == 0, "a tile must sit inside one scale tile");
  static_assert(!PV8 || (BN % 64 == 0 && !QK16), "fp8 P.V works on 64-key groups, with fp8 QK^T");
  static_assert(QK16 ? (K_PER_THREAD >= 1 && K_PER_THREAD * THREADS == BN * CPR)
                     : (K_LOADS * 64 == BN * K_SLOTS), "K tile must split evenly");
  static_assert(V_THREADS <= THREADS, "V staging needs at most one thread per 4x8 block");
};

typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));

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

// Byte slot of key k within its 64-key group in the fp8 V^T tile: the order in
// which a lane's S^T accumulator elements of two 32-key blocks become the 32
// bytes of the f8f6f4 B operand (block b = k / 32, element i of the block
// with k % 32 = 8 (i / 4) + 4 g + i % 4, byte 32 g + 16 b + i).
__host__ __device__ constexpr int vt8_slot(int k) {
  return 64 * (k >> 6) + 32 * ((k >> 2) & 1) + 16 * ((k >> 5) & 1) + 4 * ((k >> 3) & 3) + (k & 3);
}

// Two fp32 values into e2m1 codes (nearest even) at byte `sel` of old, and
// the two codes of byte `sel` back to fp32 (sel is a constant once unrolled).
__device__ inline uint32_t pk_fp4(uint32_t old, float a, float b, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 3);
  }
}
__device__ inline float2_t unpk_fp4(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  }
}

// The same for a 4-bit P operand: lane half g of the B operand holds keys
// 32b + 8(i/4) + 4g + i%4 (element i of block b) at k = 32b + 16g + i.
__host__ __device__ constexpr int vt4_slot(int k) {
  return 64 * (k >> 6) + 32 * ((k >> 5) & 1) + 16 * ((k >> 2) & 1) + 4 * ((k >> 3) & 3) + (k & 3);
}

// Four keys x 8 codes (w[r] = codes of key 4kg + r, columns d0 .. d0+7) into
// fp8 V^T rows d0 .. d0+7: one 4-byte word per row (bytes = keys 4kg .. +3).
template <bool P4>
__device__ inline void store_vt8(char* vt, int pitch, int d0, int kg, const u32x2 (&w)[4]) {
  const int col = P4 ? vt4_slot(4 * kg) : vt8_slot(4 * kg);
#pragma unroll
  for (int hw = 0; hw < 2; ++hw) {  // codes 0..3 / 4..7 of each key
    const uint32_t k0 = w[0][hw], k1 = w[1][hw], k2 = w[2][hw], k3 = w[3][hw];
    const uint32_t t0 = __builtin_amdgcn_perm(k1, k0, 0x05010400u);  // k0.b0 k1.b0 k0.b1 k1.b1
    const uint32_t t1 = __builtin_amdgcn_perm(k1, k0, 0x07030602u);  // k0.b2 k1.b2 k0.b3 k1.b3
    const uint32_t t2 = __builtin_amdgcn_perm(k3, k2, 0x05010400u);
    const uint32_t t3 = __builtin_amdgcn_perm(k3, k2, 0x07030602u);
    const uint32_t r[4] = {__builtin_amdgcn_perm(t2, t0, 0x05040100u), __builtin_amdgcn_perm(t2, t0, 0x07060302u),
                           __builtin_amdgcn_perm(t3, t1, 0x05040100u), __builtin_amdgcn_perm(t3, t1, 0x07060302u)};
#pragma unroll
    for (int e = 0; e < 4; ++e) *(uint32_t*)(vt + (d0 + 4 * hw + e) * pitch + col) = r[e];
  }
}

// Non-causal grids of one workgroup per block: block g runs on XCD g % 8 (the
// dispatcher's round robin) and the workgroups an XCD holds at a time are
// consecutive in g / 8, so taking the query blocks of one slice in a row
// (slice-major) keeps few slices' K/V in that XCD's L2 at once.  Every block
// has the same length, so the order costs no balance.  BH a multiple of 8.
__device__ inline void map_block_slices(int g, int nqb, int BH, int& qb, int& bh) {
  const int x = g & 7, t = g >> 3, hp = BH >> 3;
  bh = x * hp + t / nqb;
  qb = t % nqb;
}

template <int D, bool CAUSAL, bool QK16, int PVM, int W, int BN>
__global__ void __launch_bounds__(64 * W, 8 / W) fwd_fp8_kernel(FwdParams p) {
  constexpr bool PV8 = PVM != kPvF16;  // P.V on the f8f6f4 MFMA with V's codes
  constexpr bool P4 = PVM == kPvFp4 || PVM == kPvFp4Direct;
  using G = Geo8<D, QK16, PV8, W, BN>;
  constexpr int QT = kQuantTile;
  constexpr int OPF = D * 4 + 16;  // LDS row pitch of the fp32 O block in the epilogue
  // fp8 Q.K: the workgroup's Q codes (BM rows of D bytes) sit after the K/V
  // stages for the whole kernel.
  constexpr int QLDS = QK16 ? 0 : G::BM * D;
  constexpr int SMEM = G::LDS + QLDS > G::BM * OPF ? G::LDS + QLDS : G::BM * OPF;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r32 = lane & 31;
  const int g = lane >> 5;

  int qb, bh;
  if (!CAUSAL && (p.BH & 7) == 0)
    map_block_slices(tile_index(p), p.nqb, p.BH, qb, bh);
  else
    map_block(tile_index(p), p.nqb, p.BH, CAUSAL, qb, bh);
  const int q0 = qb * G::BM;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + r32;
  const int Nq = p.Nq, Nk = p.Nk;
  const int nqt = (Nq + QT - 1) / QT, nkt = (Nk + QT - 1) / QT;

  const uint8_t* __restrict__ qg = (const uint8_t*)p.q + (int64_t)bh * Nq * D;
  const uint8_t* __restrict__ kg = (const uint8_t*)p.k + (int64_t)bh * Nk * D;
  const uint8_t* __restrict__ vg = (const uint8_t*)p.v + (int64_t)bh * Nk * D;
  const float* __restrict__ ksc = p.k_scale + (int64_t)bh * nkt;
  const float* __restrict__ vsc = p.v_scale + (int64_t)bh * nkt;
  // this wavefront's query scale tile (its 32 rows never straddle two)
  const float c_q = p.c * p.q_scale[(int64_t)bh * nqt + min(qw0, Nq - 1) / QT];
  // Largest V scale of this (b,h) slice: probabilities are stored as
  // p * s_v(t) / svmax, at most 2^8 in fp16 (2^8 in e4m3, 4 in e2m1 after
  // their fixed factors), which holds without overflow.
  float svmax = 0.f;
  for (int t = 0; t < nkt; ++t) svmax = fmaxf(svmax, vsc[t]);
  const float inv_svmax = 1.f / svmax;

  int kend = Nk, wkend = Nk, wmask_from = Nk;
  if (CAUSAL) {
    const int last_row = min(q0 + G::BM, Nq) - 1;
    kend = min(Nk, last_row + p.diag + 1);
    wkend = min(Nk, min(qw0 + 31, Nq - 1) + p.diag + 1);
    wmask_from = min(Nk, qw0 + p.diag + 1);
  }
  const int ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;
  const int wtiles = (qw0 < Nq && wkend > 0) ? min(ntiles, (wkend + BN - 1) / BN) : 0;

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
        u32x2 cw = ok ? *(const u32x2*)(row + 16 * kk + 8 * g) : (u32x2){0u, 0u};
        cw = (cw & q_and) ^ sgn;
        qf16[kk] = __builtin_bit_cast(f16x8, widen_lo((u32x4){cw[0], cw[1], 0u, 0u}));
      }
    } else {
      // The Q block arrives by contiguous 1 KiB transfers into LDS (rows of D
      // bytes; a row's 16-byte chunk c sits at slot c ^ ((r / (256 / D)) mod
      // D/16), so the fragment reads of 16 consecutive rows at one chunk hit
      // distinct banks); the fragments are read after the prologue's barrier.
      // Transfer j covers rows (1024 / D) j ..; wavefront w issues j = w + 8n,
      // which fixes each lane's row and chunk permutation.
      constexpr int QR = 1024 / D, CPQ = D / 16, RPW = 256 / D;
      const int rin = lane / CPQ, jc = lane % CPQ;
      const int swz = ((QR * (wave & 1) + rin) / RPW) & (CPQ - 1);
      const unsigned q_lane = (unsigned)(rin * D + 16 * (jc ^ swz));
      const i32x4 rsrc = buffer_rsrc(qg + (int64_t)q0 * D);
      unsigned lds = __builtin_amdgcn_readfirstlane(lds_offset(smem + G::LDS) + 1024u * wave);
      if (q0 + G::BM <= Nq) {
        unsigned soff = __builtin_amdgcn_readfirstlane(1024u * wave);
#pragma unroll
        for (int n = 0; n < G::BM * D / 1024 / W; ++n) buf_lds16<1024 * W, 1024 * W>(rsrc, q_lane, soff, lds);
      } else {  // last block of a slice: rows past Nq read the last row
        unsigned soff = 0;
#pragma unroll 1
        for (int j = wave; j < G::BM * D / 1024; j += W) {
          const int r = min(q0 + QR * j + rin, Nq - 1) - q0;
          buf_lds16<0, 1024 * W>(rsrc, (unsigned)(r * D) + (q_lane - (unsigned)(rin * D)), soff, lds);
        }
      }
    }
  }

  // ---- staging.  K codes go straight into LDS (fp8 form; the pad slot of a
  // row re-reads chunk 0) or through registers, widened to fp16 (fp16 form).
  // V: thread (dc, kgrp) takes keys 4*kgrp .. +3 of columns 8*dc .. +7
  // (8 codes each), widens them to fp16 and stores them transposed.  In the
  // fp8 form V runs two tiles ahead: tile t+1's codes, loaded during
  // iteration t-1, are widened and stored right after iteration t's Q.K
  // products (where the SIMD's other wavefront keeps the matrix cores busy),
  // and tile t+2's loads go out then and stay in flight across the tile
  // barrier (vmcnt(4)), so they have a whole iteration to arrive.
  const int v_dc = tid / G::KG, v_kg = tid % G::KG;
  const bool v_stager = tid < G::V_THREADS;
  u32x2 vreg[4];
  u32x4 kreg[QK16 ? G::K_PER_THREAD : 1];
  auto kstage = [&](int t) { return smem + (t & 1) * G::K_BYTES; };
  auto vstage = [&](int t) { return smem + 2 * G::K_BYTES + (t & 1) * G::V_BYTES; };
  // Direct-load form: this wavefront's loads are j = wave + W * jj; each
  // lane's row and column offset within a tile are fixed, so they are
  // computed once here and each tile only adds its first key.
  constexpr int NJ = (G::K_LOADS + W - 1) / W;
  int k_row[NJ], k_col[NJ];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
    const int slot = (wave + W * jj) * 64 + lane;
    const int ch = slot % G::K_SLOTS;
    k_row[jj] = slot / G::K_SLOTS;
    k_col[jj] = (ch < G::CPR ? ch : 0) * 16;
  }
  auto load_k = [&](int t) {
    const int k0 = t * BN;
    if constexpr (QK16) {
#pragma unroll
      for (int u = 0; u < G::K_PER_THREAD; ++u) {
        const int ch = u * G::THREADS + tid;
        const int row = ch / G::CPR, col = ch % G::CPR;
        const int key = min(k0 + row, Nk - 1);
        kreg[u] = *(const u32x4*)(kg + (int64_t)key * D + col * 16);
      }
    } else {
      char* kb = kstage(t);
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        const int j = wave + W * jj;
        if (j < G::K_LOADS) {  // wave-uniform
          const int key = min(k0 + k_row[jj], Nk - 1);
          const uint8_t* src = kg + (int64_t)key * D + k_col[jj];
          const unsigned base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)(kb + j * 1024);
          load_lds16(src, __builtin_amdgcn_readfirstlane(base));
        }
      }
    }
  };
  auto store_k = [&](int t) {
    if constexpr (QK16) {
      char* kb = kstage(t);
#pragma unroll
      for (int u = 0; u < G::K_PER_THREAD; ++u) {
        const int ch = u * G::THREADS + tid;
        const int row = ch / G::CPR, col = ch % G::CPR;
        *(u32x4*)(kb + row * G::KS + col * 32) = widen_lo(kreg[u]);
        *(u32x4*)(kb + row * G::KS + col * 32 + 16) = widen_hi(kreg[u]);
      }
    }
  };
  const int v_off_lane = 4 * v_kg * D + v_dc * 8;  // this thread's keys and columns within a tile
  auto gload_v = [&](int t) {
    if (!v_stager) return;
    const int k0 = t * BN;
    const uint8_t* src = vg + (int64_t)k0 * D + v_off_lane;
    if (k0 + BN <= Nk) {  // wave-uniform: the whole tile lies inside V
#pragma unroll
      for (int r = 0; r < 4; ++r) vreg[r] = *(const u32x2*)(src + r * D);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 4 * v_kg + r;
        const u32x2 x = *(const u32x2*)(vg + (int64_t)min(key, Nk - 1) * D + v_dc * 8);
        vreg[r] = key < Nk ? x : (u32x2){0u, 0u};
      }
    }
  };
  auto lstore_v = [&](int t) {
    if (!v_stager) return;
    if constexpr (PV8) {
      store_vt8<P4>(vstage(t), G::VTP8, 8 * v_dc, v_kg, vreg);
      return;
    }
    u32x4 w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) w[r] = widen_lo((u32x4){vreg[r][0], vreg[r][1], 0u, 0u});
    store_vt(vstage(t), G::VTP, 8 * v_dc, v_kg, w);
  };
  auto publish = [&]() {
    __builtin_amdgcn_s_waitcnt(0);  // direct loads are counted by vmcnt only
    __syncthreads();
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = (f32x16){};
  float m2 = -INFINITY;  // reference maximum of c_t * raw, base-2 units
  float l_lane = 0.f;

  const int k_off = r32 * G::KS + g * (QK16 ? 16 : 32);
  const int v_off = r32 * G::VTP + g * 16;

  auto qk = [&](const char* kb, f32x16 (&s)[G::KB]) {
#pragma unroll
    for (int h = 0; h < G::KB; ++h) s[h] = (f32x16){};
    // Fragment i = (k-slice i / KB, block i % KB); the LDS reads run RA
    // fragments ahead of the MFMAs, in source order, pinned (left to itself
    // the scheduler reads each fragment right before its MFMA).
    if constexpr (QK16) {
      constexpr int NF = G::KB * (D / 16), RA = 4;
      auto frag = [&](int i) { return *(const f16x8*)(kb + k_off + (i % G::KB) * 32 * G::KS + (i / G::KB) * 32); };
      f16x8 fa[RA];
#pragma unroll
      for (int i = 0; i < RA; ++i) fa[i] = frag(i);
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        const int kk = i / G::KB, h = i % G::KB;
        s[h] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i % RA], qf16[kk], kk == 0 ? (f32x16){} : s[h], 0, 0, 0);
        if (i + RA < NF) fa[i % RA] = frag(i + RA);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      constexpr int NF = G::KB * (D / 64), RA = 2;
      auto frag = [&](int i) {
        const char* ap = kb + k_off + (i % G::KB) * 32 * G::KS + (i / G::KB) * 64;
        const u32x4 a0 = *(const u32x4*)ap;
        const u32x4 a1 = *(const u32x4*)(ap + 16);
        return (i32x8){(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
      };
      i32x8 fa[RA];
#pragma unroll
      for (int i = 0; i < RA; ++i) fa[i] = frag(i);
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        const int kk = i / G::KB, h = i % G::KB;
        s[h] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i % RA], qf8[kk], kk == 0 ? (f32x16){} : s[h], 0, 0,
                                                               0, 127, 0, 127);
        if (i + RA < NF) fa[i % RA] = frag(i + RA);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto mask = [&](f32x16 (&s)[G::KB], int k0) {
    const int lim = CAUSAL ? min(my_q + p.diag, Nk - 1) : Nk - 1;
#pragma unroll
    for (int h = 0; h < G::KB; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 32 * h + 8 * (i >> 2) + 4 * g + (i & 3);
        if (key > lim) s[h][i] = -INFINITY;
      }
  };

  if (ntiles > 0) {
    load_k(0);
    gload_v(0);
    store_k(0);
    lstore_v(0);
  }
  if (!QK16 && ntiles > 0) gload_v(min(1, ntiles - 1));
  publish();
  if constexpr (!QK16) {
    // Q fragment (B operand): row my_q, bytes 64 kk + 32 g .. +32 = chunks
    // 4 kk + 2 g and 4 kk + 2 g + 1 of block row r = 32 wave + r32.
    constexpr int CPQ = D / 16, RPW = 256 / D;
    const int r = wave * 32 + r32;
    const char* qrow = smem + G::LDS + r * D;
    const int swz = (r / RPW) & (CPQ - 1);
    const bool ok = my_q < Nq;
    const uint32_t q_and = p.q_and ? 0xFFFFFFFFu : 0u;
    const uint32_t sgn = p.q_xor ? 0x80808080u : 0u;
#pragma unroll
    for (int kk = 0; kk < QF; ++kk) {
      u32x4 a = *(const u32x4*)(qrow + 16 * ((4 * kk + 2 * g) ^ swz));
      u32x4 b = *(const u32x4*)(qrow + 16 * ((4 * kk + 2 * g + 1) ^ swz));
      a = (a & q_and) ^ sgn;
      b = (b & q_and) ^ sgn;
      if (!ok) a = b = (u32x4){0u, 0u, 0u, 0u};
      qf8[kk] = (i32x8){(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    }
  }

  // The K and V scales of a tile are fetched one tile ahead with vector
  // loads (the offset is opaque to the compiler, so it cannot turn them into
  // scalar loads): an outstanding scalar load shares the LDS wait counter and
  // would make every LDS wait of the tile a full drain.
  auto scale_pair = [&](int t, float& ks, float& vs) {
    int z = 0;
    asm volatile("" : "+v"(z));
    const int i = (t * BN) / QT + z;
    ks = ksc[i];
    vs = vsc[i];
  };
  float ks_next = 0.f, vs_next = 0.f;
  if (ntiles > 0) scale_pair(0, ks_next, vs_next);
  for (int t = 0; t < ntiles; ++t) {
    const bool more = t + 1 < ntiles;
    const float ks_t = ks_next, vs_t = vs_next;
    if (more) {
      load_k(t + 1);
      if (QK16) gload_v(t + 1);
      scale_pair(t + 1, ks_next, vs_next);
    }
    f32x16 s[G::KB];
    if (t < wtiles) qk(kstage(t), s);
    // fp8 form: tile t+1's V (buffer (t+1) & 1, last read in iteration t-1)
    // from registers to LDS, then tile t+2's loads (the last tile again at
    // the end of the slice, unused).  The next tile's scales are consumed
    // first, so that the V loads are the only ones in flight at the barrier.
    const int v_next = min(t + 2, ntiles - 1);
    if constexpr (!QK16) {
      if (more) lstore_v(t + 1);
      asm volatile("" ::"v"(ks_next), "v"(vs_next));
      gload_v(v_next);
    }
    if (t < wtiles) {
      const int k0 = t * BN;
      const float c = c_q * ks_t;
      const float sv = vs_t;
      const float vfold = __log2f(sv * inv_svmax);  // <= 0
      const float vunfold = svmax * __builtin_amdgcn_rcpf(sv);

      if (k0 + BN > wmask_from) mask(s, k0);

      float mx = s[0][0];
#pragma unroll
      for (int h = 0; h < G::KB; ++h)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[h][i]);
      mx = halves_max(mx);
      const float mx2 = mx == -INFINITY ? -INFINITY : mx * c;
      // fp16 probabilities: the reference moves only when the maximum passes
      // it by more than kLazyLog2 (P' then stays below 2^8, which fp16 holds
      // with its full 11-bit precision), so O and l are rarely rescaled.  The
      // fp8 and fp4 probabilities keep the exact maximum (their scaled range
      // is fixed).
      const bool need = mx2 > m2 + (PV8 ? 0.f : kLazyLog2);
      if (__ballot(need)) {
        const float m_new = need ? mx2 : m2;
        const float alpha = (m2 == -INFINITY) ? 0.f : fast_exp2(m2 - m_new);
        l_lane *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
        m2 = m_new;
      }
      // P' = p * s_v(t) / s_v_max: the tile's V scale rides in the exponent
      // bias; the normaliser gets p back through one multiply per tile.
      const float bias_v = ((m2 == -INFINITY) ? 0.f : -m2) + vfold;
      if constexpr (P4) {
        // 4 P' in e2m1 and O^T += V^T P'^T on the f8f6f4 MFMA (B operand
        // 4-bit), one 64-key group at a time.  Nibble t of the lane's B
        // operand is element t % 16 of block 2 grp + t / 16 (k = 32 (t / 16)
        // + 16 g + t % 16).  The normaliser sums the decoded codes.
        float rs[4] = {0.f, 0.f, 0.f, 0.f};
        const float bias4 = bias_v + 2.f;               // exp path: 4 P'
        const float zc = 2.f * c, zb = 2.f * bias_v + 6.f;  // Direct-P: 2 log2(4 P') + 2
#pragma unroll
        for (int grp = 0; grp < G::KB / 2; ++grp) {
          i32x8 pb4 = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int d2 = 0; d2 < 2; ++d2) {  // dword 2b + d2 = elements 8 d2 .. 8 d2 + 7 of block 2 grp + b
              const f32x16& sv = s[2 * grp + b];
              uint32_t w = 0;
#pragma unroll
              for (int pr = 0; pr < 4; ++pr) {
                const int i0 = 8 * d2 + 2 * pr;
                if constexpr (PVM == kPvFp4) {
                  const float e0 = fast_exp2(fmaf(sv[i0], c, bias4)), e1 = fast_exp2(fmaf(sv[i0 + 1], c, bias4));
                  w = pk_fp4(w, e0, e1, pr);
                } else {
                  const float z0 = __builtin_amdgcn_fmed3f(__builtin_rintf(fmaf(sv[i0], zc, zb)), 0.f, 6.f);
                  const float z1 = __builtin_amdgcn_fmed3f(__builtin_rintf(fmaf(sv[i0 + 1], zc, zb)), 0.f, 6.f);
                  w |= ((uint32_t)z0 | ((uint32_t)z1 << 4)) << (8 * pr);
                }
              }
              pb4[2 * b + d2] = (int)w;
#pragma unroll
              for (int pr = 0; pr < 4; ++pr) {
                const float2_t dv = unpk_fp4(w, pr);
                rs[pr] += dv[0] + dv[1];
              }
            }
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const char* ap = vstage(t) + (32 * db + r32) * G::VTP8 + 64 * grp + 32 * g;
            const u32x4 a0 = *(const u32x4*)ap;
            const u32x4 a1 = *(const u32x4*)(ap + 16);
            const i32x8 av = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                              (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
            oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pb4, oacc[db], 0, 4, 0, 127, 0, 125);
          }
        }
        l_lane += ((rs[0] + rs[1]) + (rs[2] + rs[3])) * (vunfold * 0.25f);
      } else if constexpr (PV8) {
        // P' * 2^8 in e4m3 and O^T += V^T P'^T on the f8f6f4 MFMA, one 64-key
        // group at a time (4 MFMAs per group at d = 128).  The normaliser
        // sums the rounded values (2^-8 applied once per tile).
        float rs[4] = {0.f, 0.f, 0.f, 0.f};
        const float bias8 = bias_v + 8.f;  // * 2^8
#pragma unroll
        for (int grp = 0; grp < G::KB / 2; ++grp) {
          i32x8 pb8;
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) {  // dword 4b + j = elements 4j .. 4j+3 of block 2 grp + b
              const f32x16& sv = s[2 * grp + b];
              const float e0 = fast_exp2(fmaf(sv[4 * j], c, bias8)), e1 = fast_exp2(fmaf(sv[4 * j + 1], c, bias8));
              const float e2 = fast_exp2(fmaf(sv[4 * j + 2], c, bias8)), e3 = fast_exp2(fmaf(sv[4 * j + 3], c, bias8));
              int w = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
              w = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, w, true);
              pb8[4 * b + j] = w;
              const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
              const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
              rs[0] += lo[0];
              rs[1] += lo[1];
              rs[2] += hi[0];
              rs[3] += hi[1];
            }
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const char* ap = vstage(t) + (32 * db + r32) * G::VTP8 + 64 * grp + 32 * g;
            const u32x4 a0 = *(const u32x4*)ap;
            const u32x4 a1 = *(const u32x4*)(ap + 16);
            const i32x8 av = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                              (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
            oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pb8, oacc[db], 0, 0, 0, 127, 0, 119);
          }
        }
        l_lane += ((rs[0] + rs[1]) + (rs[2] + rs[3])) * (vunfold * 0.00390625f);
      } else {
        // P' = exp2(...) in fp16 and O^T += V^T P'^T, one 32-key block h at a
        // time: block h's MFMAs need only block h's probabilities, so the
        // exponentials of block h+1 issue between them.  Four partial sums.
        float rs[4] = {0.f, 0.f, 0.f, 0.f};
  #pragma unroll
        for (int h = 0; h < G::KB; ++h) {
          f16x8 pb[2];
  #pragma unroll
          for (int half = 0; half < 2; ++half) {
            f32x8 pv;
  #pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float e = fast_exp2(fmaf(s[h][half * 8 + j], c, bias_v));  // masked: exp2(-inf) = 0
              pv[j] = e;
              rs[j & 3] += e;
            }
            pb[half] = __builtin_convertvector(pv, f16x8);
          }
  #pragma unroll
          for (int db = 0; db < D / 32; ++db)
  #pragma unroll
            for (int half = 0; half < 2; ++half) {
              const f16x8 a = *(const f16x8*)(vstage(t) + v_off + db * 32 * G::VTP + (32 * h + 16 * half) * 2);
              oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[half], oacc[db], 0, 0, 0);
            }
        }
        l_lane += ((rs[0] + rs[1]) + (rs[2] + rs[3])) * vunfold;
        {
          constexpr int NM = (D / 32) * G::KB * 2;
          constexpr int VPB = 56;  // vector instructions of one block's probabilities
          constexpr int VPM = (VPB + 2 * (D / 32) - 1) / (2 * (D / 32));
          __builtin_amdgcn_sched_group_barrier(0x002, VPB, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
  #pragma unroll
          for (int i = 0; i < NM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i + 4 < NM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
          }
        }
      }
      }
    if (QK16 && more) {
      store_k(t + 1);
      lstore_v(t + 1);
    }
    // A whole tile's V loads are four unconditional instructions, issued
    // after every other vector memory access of the iteration, so vmcnt(4)
    // covers this iteration's K transfers; a partial tile's loads are
    // predicated per key (a wavefront may issue fewer), so they are waited
    // for in full, as are the other forms' stages.
    if (!QK16 && v_stager && (v_next + 1) * BN <= Nk)
      asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
      publish();
  }

  const float l_tot = halves_sum(l_lane);
  const float inv = l_tot > 0.f ? svmax / l_tot : 0.f;  // O = oacc * svmax / l
  // O in fp32 through LDS (free after the loop's last barrier): each lane
  // writes its row's 4-column pieces, then every store to memory is 16
  // contiguous bytes of one row, D/4 lanes per row.
  {
    char* orow = smem + (wave * 32 + r32) * OPF;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 v = {oacc[db][4 * r] * inv, oacc[db][4 * r + 1] * inv, oacc[db][4 * r + 2] * inv,
                   oacc[db][4 * r + 3] * inv};
        *(f32x4*)(orow + 4 * (32 * db + 8 * r + 4 * g)) = v;
      }
  }
  if (p.lse && g == 0 && my_q < Nq)
    p.lse[(int64_t)bh * Nq + my_q] = l_tot > 0.f ? (m2 + __log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
  __syncthreads();
  constexpr int CPO = D / 4;  // 16-byte chunks per O row
  float* ob = (float*)p.o + ((int64_t)bh * Nq + q0) * D;
#pragma unroll
  for (int n = 0; n < G::BM * CPO / G::THREADS; ++n) {
    const int idx = n * G::THREADS + tid;
    const int r = idx / CPO, ch = idx % CPO;
    const f32x4 v = *(const f32x4*)(smem + r * OPF + 16 * ch);
    if (q0 + r < Nq) *(f32x4*)(ob + (int64_t)r * D + 4 * ch) = v;
  }
}

template <int D, bool QK16, int PVM>
static hipError_t launch_fp8_d(FwdParams p, bool causal, hipStream_t s) {
  constexpr int W = kWavesBf16, BN = kTileBf16;
  p.nqb = (p.Nq + 32 * W - 1) / (32 * W);
  const dim3 grid((unsigned)(p.nqb * p.BH));
  if (causal)
    hipLaunchKernelGGL((fwd_fp8_kernel<D, true, QK16, PVM, W, BN>), grid, dim3(64 * W), 0, s, p);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<D, false, QK16, PVM, W, BN>), grid, dim3(64 * W), 0, s, p);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_fp8_mode(const FwdParams& p, bool causal, int mode, hipStream_t s) {
  switch (mode) {
    case kFp8QkFp8: return launch_fp8_d<D, false, kPvF16>(p, causal, s);
    case kFp8QkFp16: return launch_fp8_d<D, true, kPvF16>(p, causal, s);
    case kFp8AllFp8: return launch_fp8_d<D, false, kPvFp8>(p, causal, s);
    case kFp8PvFp4: return launch_fp8_d<D, false, kPvFp4>(p, causal, s);
    case kFp8PvFp4Direct: return launch_fp8_d<D, false, kPvFp4Direct>(p, causal, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_fp8(const FwdParams& p, int d, bool causal, int mode, hipStream_t s) {
  if (d == 128) return launch_fp8_mode<128>(p, causal, mode, s);
  if (d == 64) return launch_fp8_mode<64>(p, causal, mode, s);
  return hipErrorInvalidValue;
}

}  // namespace eta
