// bf16 attention forward for gfx950: S^T = K Q^T and O^T += V^T P^T on
// 32x32x16 bf16 MFMA, online softmax in registers, K/V tiles double-buffered
// through LDS, and a software-pipelined tile loop.
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
// operand without any data movement.  The V^T fragments are single 16-byte
// LDS reads from the transposed, key-permuted V tile (common.h).
//
// Issue order.  The probabilities of each 32-key block are formed right
// before that block's P.V products, so the exponentials of the next block
// issue between the current block's MFMAs: on gfx950 vector and matrix
// instructions overlap when they are interleaved in one wavefront's
// instruction stream.
//
// Staging.  A workgroup of W wavefronts owns 32*W query rows (W = 8: one
// workgroup per compute unit, two wavefronts per SIMD), so every K/V tile read
// from memory serves 256 rows.  K tiles go straight from global memory into LDS
// (global_load_lds); V goes through registers so it can be stored transposed.
// Tile t+1 is in flight while tile t is computed; one barrier per tile.
//
// Rescaling.  O and l are multiplied by alpha only on tiles where some row of
// the wavefront raised its maximum (one ballot per tile).  The exponent always
// uses the current maximum, so the dominant probability of a row is exp2 of a
// rounding residual and rounds to exactly 1.0 in bf16.
#include "common.h"

namespace eta {

template <int D, int W, int BN>
struct Geo {
  static constexpr int THREADS = 64 * W;
  static constexpr int BM = 32 * W;           // query rows per workgroup
  static constexpr int KB = BN / 32;          // 32-key blocks per tile
  static constexpr int VTP = vt_pitch(BN);    // V^T row pitch (bytes)
  static constexpr int KS = D * 2 + 16;         // K tile row pitch (bytes)
  static constexpr int K_BYTES = BN * KS;
  static constexpr int V_BYTES = D * VTP;     // V^T: one row per column d
  static constexpr int LDS = 2 * K_BYTES + 2 * V_BYTES;  // two K stages, two V stages
  static constexpr int CPR = D / 8;             // 16-byte chunks per K row
  static constexpr int K_SLOTS = CPR + 1;       // ... plus one pad slot
  static constexpr int K_LOADS = BN * K_SLOTS / 64;  // wave-wide 1 KiB direct loads per tile
  static constexpr int KG = BN / 4;           // 4-key groups per tile
  static constexpr int V_THREADS = KG * (D / 8);  // key groups x D/8 column chunks
  static_assert(K_LOADS * 64 == BN * K_SLOTS, "K tile must be whole 1 KiB loads");
  static_assert(V_THREADS <= THREADS, "V staging needs at most one thread per 4x8 block");
};

__device__ inline bf16x8 pack_bf16(const float* x) {
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  return __builtin_convertvector(v, bf16x8);
}

template <int D, bool CAUSAL, int EPI, int W, int BN>
__global__ void __launch_bounds__(64 * W, 8 / W) fwd_bf16_kernel(FwdParams p) {
  using G = Geo<D, W, BN>;
  __shared__ __attribute__((aligned(16))) char smem[G::LDS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r32 = lane & 31;
  const int g = lane >> 5;

  int qb, bh;
  map_block(tile_index(p), p.nqb, p.BH, CAUSAL, qb, bh);
  const int q0 = qb * G::BM;
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
    const int last_row = min(q0 + G::BM, Nq) - 1;
    kend = min(Nk, last_row + p.diag + 1);
    wkend = min(Nk, min(qw0 + 31, Nq - 1) + p.diag + 1);
    wmask_from = min(Nk, qw0 + p.diag + 1);  // first key hidden from row qw0
  }
  const int ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;
  const int wtiles = (qw0 < Nq && wkend > 0) ? min(ntiles, (wkend + BN - 1) / BN) : 0;


  bf16x8 qf[D / 16];  // Q fragments, loaded in the prologue below

  // ---- staging.  K: direct global -> LDS loads; each wave-wide load fills 64
  // consecutive 16-byte slots of the padded tile (slot s = row s / K_SLOTS,
  // chunk s % K_SLOTS; the pad chunk re-reads chunk 0).  Keys past Nk read the
  // last row: such tiles are always masked.  V: through registers, thread
  // (dc, kgrp) takes keys 4*kgrp .. +3 of columns 8*dc .. +7 and stores them
  // transposed (common.h).
  const int v_dc = tid / G::KG, v_kg = tid % G::KG;
  const bool v_stager = tid < G::V_THREADS;
  u32x4 vreg[4];
  auto kstage = [&](int t) { return smem + (t & 1) * G::K_BYTES; };
  auto vstage = [&](int t) { return smem + 2 * G::K_BYTES + (t & 1) * G::V_BYTES; };
  // This wavefront's direct loads are j = wave + W * jj; each lane's row and
  // column offset within a tile are fixed, so they are computed once here and
  // each tile only adds its first key.
  constexpr int NJ = (G::K_LOADS + W - 1) / W;
  int k_row[NJ], k_col[NJ];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
    const int slot = (wave + W * jj) * 64 + lane;
    const int ch = slot % G::K_SLOTS;
    k_row[jj] = slot / G::K_SLOTS;
    k_col[jj] = (ch < G::CPR ? ch : 0) * 8;
  }
  auto load_k = [&](int t) {
    char* kb = kstage(t);
    const int k0 = t * BN;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int j = wave + W * jj;
      if (j < G::K_LOADS) {  // wave-uniform
        const int key = min(k0 + k_row[jj], Nk - 1);
        const uint16_t* src = kg + (int64_t)key * D + k_col[jj];
        const unsigned base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)(kb + j * 1024);
        load_lds16(src, __builtin_amdgcn_readfirstlane(base));
      }
    }
  };
  // V keys past Nk read the last row instead: their probabilities are exactly
  // 0, so every load is unconditional (no load waits for another).
  const uint16_t* __restrict__ v_col = vg + v_dc * 8;
  auto gload_v = [&](int t) {
    if (!v_stager) return;
    const int kfirst = t * BN + 4 * v_kg;
    if (t * BN + BN <= Nk) {  // workgroup-uniform: the whole tile lies inside V
      const uint16_t* src = v_col + (int64_t)kfirst * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) vreg[r] = *(const u32x4*)(src + r * D);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) vreg[r] = *(const u32x4*)(v_col + (int64_t)min(kfirst + r, Nk - 1) * D);
    }
  };
  auto lstore_v = [&](int t) {
    if (v_stager) store_vt(vstage(t), G::VTP, 8 * v_dc, v_kg, vreg);
  };
  // Direct loads are counted by vmcnt only: drain them before the barrier that
  // publishes the stage.
  auto publish = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  // ---- per-row state
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = (f32x16){};
  float m_run = -INFINITY;  // running maximum of the raw dot product q.k
  float l_lane = 0.f;       // this lane's share of sum exp2(c (s - m_run))
  const float c = p.c;

  const int k_off = r32 * G::KS + g * 16;     // K row r32, 16-byte slice g
  const int v_off = r32 * G::VTP + g * 16;   // V^T row r32 of a 32-column block, slot 8g

  auto qk = [&](const char* kb, f32x16 (&s)[G::KB]) {
#pragma unroll
    for (int h = 0; h < G::KB; ++h) s[h] = (f32x16){};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int h = 0; h < G::KB; ++h) {
        const bf16x8 a = *(const bf16x8*)(kb + k_off + h * 32 * G::KS + kk * 32);
        s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[h], 0, 0, 0);
      }
    // LDS reads run 4 fragments ahead of the MFMAs (the default schedule
    // waits for each fragment right before its MFMA)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < G::KB * (D / 16) - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };
  // Keys beyond the causal limit or the end of K; exp2(-inf * c) = 0 as c > 0.
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
  auto tile_needs_mask = [&](int t) { return t * BN + BN > wmask_from; };
  auto rowmax = [&](const f32x16 (&s)[G::KB]) {
    float mx = s[0][0];
#pragma unroll
    for (int h = 0; h < G::KB; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[h][i]);
    return halves_max(mx);
  };
  // Raise the running maximum; where some row raised it, rescale O and l by
  // alpha = exp2(c (m_old - m_new)).
  auto rebase = [&](float mx) {
    const bool need = mx > m_run;
    if (__ballot(need)) {
      const float m_new = need ? mx : m_run;
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2((m_run - m_new) * c);
      l_lane *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
  };
  // P = exp2(c s - c m) (bf16) and O^T += V^T P^T, one 32-key block h at a
  // time: block h's eight MFMAs need only block h's probabilities, so the
  // exponentials of block h+1 issue between them (the scheduling pattern
  // below asks for that order).  The row sum runs in four partial sums.
  auto softmax_pv = [&](const f32x16 (&s)[G::KB], const char* vb) {
    const float bias = (m_run == -INFINITY) ? 0.f : -m_run * c;
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < G::KB; ++h) {
      bf16x8 pb[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pv[j] = fast_exp2(fmaf(s[h][half * 8 + j], c, bias));
          rs[j & 3] += pv[j];
        }
        pb[half] = pack_bf16(pv);
      }
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const bf16x8 a = *(const bf16x8*)(vb + v_off + db * 32 * G::VTP + (32 * h + 16 * half) * 2);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[half], oacc[db], 0, 0, 0);
        }
    }
    l_lane += (rs[0] + rs[1]) + (rs[2] + rs[3]);
    constexpr int NM = (D / 32) * G::KB * 2;  // MFMAs
    constexpr int VPB = 56;                   // vector instructions per block's probabilities
    constexpr int VPM = (VPB + 2 * (D / 32) - 1) / (2 * (D / 32));  // per MFMA: one block's worth per block's MFMAs
    __builtin_amdgcn_sched_group_barrier(0x002, VPB, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + 4 < NM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
    }
  };

  // ---- tile loop: stage t%2 holds K(t) and V(t); tile t+1 is in flight
  // while tile t is computed.
  // Prologue: the first K/V tile's loads go out first, then Q's, so the
  // transfers overlap.  Q fragment (B operand of S^T = K Q^T): row my_q,
  // d = kk*16 + g*8 .. +8; rows past Nq load the last row (unconditionally,
  // so no load waits for another) and are zeroed.
  if (ntiles > 0) {
    load_k(0);
    gload_v(0);
  }
  // Q block: contiguous 1 KiB transfers straight into the second K/V stage
  // (rows 0..127 into the K stage, 128..255 into the V stage), each row's
  // 16-byte chunks permuted (chunk c of block row r at slot c ^ (r mod d/8))
  // so the fragment reads below, 32 rows at one column, hit distinct banks.
  // Transfer j covers rows QR*j .. +QR-1; wavefront w issues j = w + 8n, so
  // j mod 4 = w mod 4 and each lane's source offset is one constant.
  constexpr int QR = 1024 / (2 * D);              // rows per transfer
  constexpr int QT = G::BM / QR;                  // transfers per Q block
  constexpr int QPW = QT / W;                     // per wavefront
  constexpr int CPQ = D / 8;                      // 16-byte chunks per row
  char* const q_lo = smem + G::K_BYTES;                     // rows 0 .. BM/2-1
  char* const q_hi = smem + 2 * G::K_BYTES + G::V_BYTES;    // rows BM/2 ..
  {
    const int rin = lane / CPQ, jc = lane % CPQ;
    const int swz = (QR * (wave & 3) + rin) & (CPQ - 1);
    const unsigned q_lane = (unsigned)(rin * D + 8 * (jc ^ swz)) * 2u;
    const i32x4 rsrc = buffer_rsrc(qg + (int64_t)q0 * D);
    if (q0 + G::BM <= Nq) {
      unsigned soff = __builtin_amdgcn_readfirstlane(1024u * wave);
      unsigned lds = __builtin_amdgcn_readfirstlane(lds_offset(q_lo) + 1024u * wave);
#pragma unroll
      for (int n = 0; n < QPW / 2; ++n) buf_lds16<8192, 8192>(rsrc, q_lane, soff, lds);
      lds = __builtin_amdgcn_readfirstlane(lds_offset(q_hi) + 1024u * wave);
#pragma unroll
      for (int n = 0; n < QPW / 2; ++n) buf_lds16<8192, 8192>(rsrc, q_lane, soff, lds);
    } else {  // last block of a slice: rows past Nq read the last row
      unsigned soff = 0;
#pragma unroll 1
      for (int n = 0; n < QPW; ++n) {
        const int j = wave + W * n;
        unsigned lds = __builtin_amdgcn_readfirstlane(lds_offset(n < QPW / 2 ? q_lo : q_hi) +
                                                      1024u * (j % (QT / 2)));
        const int row = min(q0 + QR * j + rin, Nq - 1) - q0;
        buf_lds16<0, 0>(rsrc, (unsigned)(row * D * 2) + (q_lane - (unsigned)(rin * D * 2)), soff, lds);
      }
    }
  }
  if (ntiles > 0) lstore_v(0);
  publish();
  // Q fragment (B operand of S^T = K Q^T): row my_q, d = kk*16 + g*8 .. +8,
  // i.e. chunk 2kk + g of block row r = 32 wave + r32, at slot (2kk + g) ^ (r32
  // mod d/8).  Rows past Nq are zeroed.
  {
    const bool ok = my_q < Nq;
    const char* qrow = (wave < W / 2 ? q_lo : q_hi) + (r32 + 32 * (wave % (W / 2))) * (2 * D);
    const int x = g ^ (r32 & (CPQ - 1));
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 v = *(const u32x4*)(qrow + 16 * ((2 * kk) ^ x));
      v = (v & p.q_and) ^ p.q_xor;
      if (!ok) v = (u32x4){0u, 0u, 0u, 0u};
      qf[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // the second stage is refilled by the first tile's transfers
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const bool more = t + 1 < ntiles;
    if (more) {
      load_k(t + 1);
      gload_v(t + 1);
    }
    if (t < wtiles) {
      f32x16 sc[G::KB];
      qk(kstage(t), sc);
      if (tile_needs_mask(t)) mask(sc, t * BN);
      rebase(rowmax(sc));
      softmax_pv(sc, vstage(t));
    }
    if (more) lstore_v(t + 1);
    publish();
  }

  // ---- epilogue: one division by the normaliser, one write of O.
  const float l_tot = halves_sum(l_lane);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (EPI == kEpiFinalBf16) {
    // O in bf16 through LDS (free after the loop's last barrier): each lane
    // writes its row's 4-column pieces, then every store to memory is 16
    // contiguous bytes of one row, 16 lanes per row.
    constexpr int OP = 2 * D + 16;  // LDS row pitch of the O block
    char* orow = smem + (wave * 32 + r32) * OP;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 v = {oacc[db][4 * r] * inv, oacc[db][4 * r + 1] * inv, oacc[db][4 * r + 2] * inv,
                   oacc[db][4 * r + 3] * inv};
        *(bf16x4*)(orow + 2 * (32 * db + 8 * r + 4 * g)) = __builtin_convertvector(v, bf16x4);
      }
    if (p.lse && g == 0 && my_q < Nq)
      p.lse[(int64_t)bh * Nq + my_q] =
          l_tot > 0.f ? m_run * p.scale_abs + __log2f(l_tot) * 0.69314718055994530942f : -INFINITY;
    __syncthreads();
    constexpr int CPO = D / 8;  // 16-byte chunks per O row
    uint16_t* ob = (uint16_t*)p.o + ((int64_t)bh * Nq + q0) * D;
#pragma unroll
    for (int n = 0; n < G::BM * CPO / G::THREADS; ++n) {
      const int idx = n * G::THREADS + tid;
      const int r = idx / CPO, ch = idx % CPO;
      const u32x4 v = *(const u32x4*)(smem + r * OP + 16 * ch);
      if (q0 + r < Nq) *(u32x4*)(ob + (int64_t)r * D + 8 * ch) = v;
    }
  } else if (my_q < Nq) {
    const int64_t row = (int64_t)bh * Nq + my_q;
    if (EPI == kEpiMerge) {
      // Online-softmax merge with the accumulated state of this row ("Sequence
      // parallelism and ring attention", "Technical insight"): M = max(m_acc,
      // m_blk), w_x = l_x e^(m_x - M), O = (w_acc O_acc + w_blk O_blk) / (w_acc +
      // w_blk).  The empty state (m = -inf, l = 0) is the identity.  Both lanes
      // of a row read m_acc / l_acc in the same instruction before lane g = 0
      // rewrites them.
      float* oa = (float*)p.o + row * D;
      const float mb = l_tot > 0.f ? m_run * p.scale_abs : -INFINITY;
      const float ma = p.m_out[row], la = p.l_out[row];
      const float M = fmaxf(ma, mb);
      float wa = 0.f, wb = 0.f;
      if (M != -INFINITY) {
        if (ma != -INFINITY) wa = la * expf(ma - M);
        if (mb != -INFINITY) wb = l_tot * expf(mb - M);
      }
      const float l = wa + wb;
      const float il = l > 0.f ? 1.f / l : 0.f;
      const float ca = wa * il, cb = wb * inv * il;  // the block's O is oacc / l_tot
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int col = 32 * db + 8 * r + 4 * g;
          const f32x4 a = wa > 0.f ? *(const f32x4*)(oa + col) : (f32x4){0.f, 0.f, 0.f, 0.f};
          const f32x4 b = {oacc[db][4 * r], oacc[db][4 * r + 1], oacc[db][4 * r + 2], oacc[db][4 * r + 3]};
          const f32x4 v = ca * a + cb * b;
          *(f32x4*)(oa + col) = v;
          if (p.o_final) *(bf16x4*)((uint16_t*)p.o_final + row * D + col) = __builtin_convertvector(v, bf16x4);
        }
      if (g == 0) {
        p.m_out[row] = l > 0.f ? M : -INFINITY;
        p.l_out[row] = l;
        if (p.lse) p.lse[row] = l > 0.f ? M + logf(l) : -INFINITY;
      }
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
          p.m_out[row] = l_tot > 0.f ? m_run * p.scale_abs : -INFINITY;
          p.l_out[row] = l_tot;
        } else if (p.lse) {
          p.lse[row] = l_tot > 0.f ? m_run * p.scale_abs + __log2f(l_tot) * 0.69314718055994530942f : -INFINITY;
        }
      }
    }
  }
}

template <int D, bool CAUSAL, int EPI>
static hipError_t launch_one(FwdParams p, hipStream_t s) {
  constexpr int W = kWavesBf16, BN = kTileBf16;
  p.nqb = (p.Nq + 32 * W - 1) / (32 * W);
  const dim3 grid((unsigned)(p.nqb * p.BH));
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, EPI, W, BN>), grid, dim3(64 * W), 0, s, p);
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
    if (epi == kEpiMerge) return launch_d<128, kEpiMerge>(p, causal, s);
  } else if (d == 64) {
    if (epi == kEpiFinalBf16) return launch_d<64, kEpiFinalBf16>(p, causal, s);
    if (epi == kEpiState) return launch_d<64, kEpiState>(p, causal, s);
    if (epi == kEpiMerge) return launch_d<64, kEpiMerge>(p, causal, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace eta
