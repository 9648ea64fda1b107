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
// operand without any data movement.  The V^T fragments come from the
// row-major V tile by two transposing LDS reads (ds_read_b64_tr_b16) each.
//
// Issue order.  The probabilities of each 32-key block are formed right
// before that block's P.V products, so the exponentials of the next block
// issue between the current block's MFMAs: on gfx950 vector and matrix
// instructions overlap when they are interleaved in one wavefront's
// instruction stream.
//
// Staging.  A workgroup of W wavefronts owns 32*W query rows (W = 8: one
// workgroup per compute unit, two wavefronts per SIMD), so every K/V tile read
// from memory serves 256 rows.  K and V tiles go straight from global memory
// into LDS (buffer loads with an LDS destination), with no registers and no
// vector work on the way.  Tile t+1 is in flight while tile t is computed; one
// barrier per tile.
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
  static constexpr int KS = D * 2;            // K / V tile row pitch (bytes): unpadded, permuted
  static constexpr int K_BYTES = BN * KS;
  static constexpr int V_BYTES = BN * KS;
  static constexpr int LDS = 2 * K_BYTES + 2 * V_BYTES;  // two K stages, two V stages
  static constexpr int CPR = D / 8;           // 16-byte chunks per row (K, Q and O blocks)
  static constexpr int RPT = 64 / CPR;        // rows per wave-wide 1 KiB transfer
  static constexpr int K_LOADS = BN / RPT;    // transfers per K tile
  static constexpr int KPW = K_LOADS / W;     // ... per wavefront
  static_assert(KPW * W == K_LOADS, "K tile must be whole transfers per wavefront");
  // Wavefront w issues transfers w + W n: the chunk permutation of a row
  // (row mod CPR) is then the same for all of one lane's transfers.
  static_assert((RPT * W) % CPR == 0 && 32 % CPR == 0, "row permutation constant per lane");
  // The bf16 O block of the epilogue (rows of 2D bytes, chunks permuted) goes
  // half into a stage's K tile and half into its V tile.
  static_assert((BM / 2) * 2 * D <= K_BYTES && (BM / 2) * 2 * D <= V_BYTES, "O and Q halves fit a stage");
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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r32 = lane & 31;
  const int g = lane >> 5;
  const int Nq = p.Nq, Nk = p.Nk;
  const int nblocks = p.nqb * p.BH;

  // The lane index as a value the compiler cannot see through: per-lane
  // offsets that are cheap to form are derived from it where they are used,
  // instead of being computed once before the block loop and held in
  // registers across every tile.
  auto fresh_lane = [&]() {
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  };

  // ---- the blocks of this workgroup.  A block is (b*h slice, 256-row query
  // block); the workgroup walks its blocks in sched_block_pairs order (causal,
  // when the grid allows it) or sched_block order.  Per block:
  // the key range of the workgroup (tiles at or beyond it are skipped
  // wholesale) and of this wavefront.
  struct Blk {
    int q0, bh, ntiles, wtiles, wmask_from;
  };
  auto describe = [&](int k, Blk& b) {
    const int gi = (CAUSAL && pair_sched_ok(gridDim.x, p.nqb, p.BH))
                       ? sched_block_pairs(k, blockIdx.x, gridDim.x, p.nqb, p.BH)
                       : sched_block(k, blockIdx.x, gridDim.x, nblocks);
    if (gi < 0) return false;
    int qb, bh;
    map_block(block_perm(p, gi, nblocks), p.nqb, p.BH, CAUSAL, qb, bh);
    b.q0 = qb * G::BM;
    b.bh = bh;
    const int qw0 = b.q0 + wave * 32;
    int kend = Nk, wkend = Nk, wmask_from = Nk;
    if (CAUSAL) {
      const int last_row = min(b.q0 + G::BM, Nq) - 1;
      kend = min(Nk, last_row + p.diag + 1);
      wkend = min(Nk, min(qw0 + 31, Nq - 1) + p.diag + 1);
      wmask_from = min(Nk, qw0 + p.diag + 1);  // first key hidden from row qw0
    }
    b.ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;
    b.wtiles = (qw0 < Nq && wkend > 0) ? min(b.ntiles, (wkend + BN - 1) / BN) : 0;
    b.wmask_from = wmask_from;
    return true;
  };
  auto qbase = [&](const Blk& b) { return (const uint16_t*)p.q + (int64_t)b.bh * Nq * D; };

  bf16x8 qf[D / 16];  // Q fragments of the current block

  // ---- staging.  Stage s (0 or 1) holds one K tile and one V^T tile.
  // K: direct global -> LDS transfers, unpadded rows with their 16-byte
  // chunks permuted (chunk c of key row r at slot c ^ (r mod CPR)), so the
  // fragment reads below, 32 rows at one column, hit distinct banks.  Each
  // wave-wide transfer moves RPT whole rows; lane l loads chunk (l mod CPR) ^
  // (row mod CPR) of row l / CPR into slot l mod CPR, which is one constant
  // offset per lane for all of its transfers.  The buffer's range ends at the
  // last key, so rows past Nk read as zero (or keep older data): such keys are
  // always masked.  V: the same transfers, rows kept whole but their 64-byte
  // segments (32 columns) permuted: segment c of key row r sits at c ^ f(r),
  // f(r) = r mod 4 (d = 128) or (r ^ r / 2) mod 2 (d = 64), so that the
  // transposing fragment reads of the P.V products below hit distinct banks.
  auto kstage = [&](int s) { return smem + s * G::K_BYTES; };
  auto vstage = [&](int s) { return smem + 2 * G::K_BYTES + s * G::V_BYTES; };
  // LDS byte addresses of the stages for the transfers, from the array itself
  // (not from a generic pointer, whose conversion would need a null check).
  const unsigned lds0 = lds_offset(smem);
  auto kstage_lds = [&](int s) { return lds0 + (unsigned)(s * G::K_BYTES); };
  auto vstage_lds = [&](int s) { return lds0 + (unsigned)(2 * G::K_BYTES + s * G::V_BYTES); };
  // Byte offset of lane l's chunk in a block of rows whose first transfer is
  // this wavefront's (rows RPT * wave + l / CPR).
  auto chunk_lane = [&](int l) {
    const int row = G::RPT * wave + l / G::CPR;
    return (unsigned)(row * 2 * D + 16 * ((l % G::CPR) ^ (row & (G::CPR - 1))));
  };
  const unsigned k_lane = chunk_lane(lane);
  // V: lane l loads row RPT * wave + l / CPR, the 16-byte chunk whose
  // segment lands in its slot l mod CPR after the permutation.
  auto vseg = [](int r) { return D == 128 ? (r & 3) : ((r ^ (r >> 1)) & 1); };
  const unsigned v_lane = [&]() {
    const int l = lane, row = G::RPT * wave + l / G::CPR, jc = l % G::CPR;
    return (unsigned)(row * 2 * D + 16 * (4 * ((jc >> 2) ^ vseg(row)) + (jc & 3)));
  }();
  auto load_k = [&](int bh, int t, int s) {
    const int k0 = t * BN;
    const i32x4 rsrc = buffer_rsrc_n((const uint16_t*)p.k + ((int64_t)bh * Nk + k0) * D,
                                     (unsigned)(min(BN, Nk - k0) * 2 * D));
    // Every offset is in the lane's address (the scalar offset stays 0), so
    // the range check sees all of it.
    unsigned soff = 0;
    unsigned lds = __builtin_amdgcn_readfirstlane(kstage_lds(s) + 1024u * wave);
#pragma unroll
    for (int n = 0; n < G::KPW; ++n)
      buf_lds16<0, 1024 * W>(rsrc, k_lane + (unsigned)(n * G::RPT * W * 2 * D), soff, lds);
  };
  // V rows past Nk read as zero (or keep older data) through the buffer's
  // range: their probabilities are exactly 0, and 0 times any finite value
  // adds nothing.
  auto load_v = [&](int bh, int t, int s) {
    const int k0 = t * BN;
    const i32x4 rsrc = buffer_rsrc_n((const uint16_t*)p.v + ((int64_t)bh * Nk + k0) * D,
                                     (unsigned)(min(BN, Nk - k0) * 2 * D));
    unsigned soff = 0;
    unsigned lds = __builtin_amdgcn_readfirstlane(vstage_lds(s) + 1024u * wave);
#pragma unroll
    for (int n = 0; n < G::KPW; ++n)
      buf_lds16<0, 1024 * W>(rsrc, v_lane + (unsigned)(n * G::RPT * W * 2 * D), soff, lds);
  };
  // Direct loads are counted by vmcnt only: drain them before the barrier that
  // publishes the stage.
  auto publish = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  // ---- Q.  Fragment kk (B operand of S^T = K Q^T) of lane (r32, g) is row
  // q0 + 32 wave + r32, d = 16 kk + 8 g .. +8.  Q element bits become (bits &
  // q_and) ^ q_xor, and rows past Nq are zeroed, once the fragments are in.
  auto fix_q = [&](const Blk& b) {
    const bool ok = b.q0 + wave * 32 + (fresh_lane() & 31) < Nq;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 v = __builtin_bit_cast(u32x4, qf[kk]);
      v = (v & p.q_and) ^ p.q_xor;
      if (!ok) v = (u32x4){0u, 0u, 0u, 0u};
      qf[kk] = __builtin_bit_cast(bf16x8, v);
    }
  };
  // Straight into the fragments (rows past Nq read the last row), while the
  // previous block's last tile is computed.
  auto load_q_regs = [&](const Blk& b) {
    const int l = fresh_lane();
    const int row = min(b.q0 + wave * 32 + (l & 31), Nq - 1);
    const uint16_t* src = qbase(b) + (int64_t)row * D + 8 * (l >> 5);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = __builtin_bit_cast(bf16x8, *(const u32x4*)(src + 16 * kk));
  };
  // Through LDS stage s when nothing else is in flight (a workgroup's first
  // block): contiguous 1 KiB transfers, rows 0..BM/2-1 into the stage's K
  // tile and the rest into its V tile, each row's 16-byte chunks permuted
  // (chunk c of block row r at slot c ^ (r mod d/8)) so the fragment reads, 32
  // rows at one column, hit distinct banks.  Transfer j covers rows QR*j ..
  // +QR-1; wavefront w issues j = w + 8n, so j mod 4 = w mod 4 and each lane's
  // source offset is one constant.
  constexpr int QR = 1024 / (2 * D);  // rows per transfer
  constexpr int QT = G::BM / QR;      // transfers per Q block
  constexpr int QPW = QT / W;         // per wavefront
  constexpr int CPQ = D / 8;          // 16-byte chunks per row
  static_assert((G::BM / 2) * 2 * D <= G::K_BYTES && (G::BM / 2) * 2 * D <= G::V_BYTES, "Q halves fit a stage");
  auto load_q_lds = [&](const Blk& b, int s) {
    const unsigned q_lo = kstage_lds(s);
    const unsigned q_hi = vstage_lds(s);
    const int l = fresh_lane();
    const int rin = l / CPQ, jc = l % CPQ;
    const int swz = (QR * (wave & 3) + rin) & (CPQ - 1);
    const unsigned q_lane = (unsigned)(rin * D + 8 * (jc ^ swz)) * 2u;
    const i32x4 rsrc = buffer_rsrc(qbase(b) + (int64_t)b.q0 * D);
    if (b.q0 + G::BM <= Nq) {
      unsigned soff = __builtin_amdgcn_readfirstlane(1024u * wave);
      unsigned lds = __builtin_amdgcn_readfirstlane(q_lo + 1024u * wave);
#pragma unroll
      for (int n = 0; n < QPW / 2; ++n) buf_lds16<8192, 8192>(rsrc, q_lane, soff, lds);
      lds = __builtin_amdgcn_readfirstlane(q_hi + 1024u * wave);
#pragma unroll
      for (int n = 0; n < QPW / 2; ++n) buf_lds16<8192, 8192>(rsrc, q_lane, soff, lds);
    } else {  // last block of a slice: rows past Nq read the last row
      unsigned soff = 0;
#pragma unroll 1
      for (int n = 0; n < QPW; ++n) {
        const int j = wave + W * n;
        unsigned lds = __builtin_amdgcn_readfirstlane((n < QPW / 2 ? q_lo : q_hi) + 1024u * (j % (QT / 2)));
        const int row = min(b.q0 + QR * j + rin, Nq - 1) - b.q0;
        buf_lds16<0, 0>(rsrc, (unsigned)(row * D * 2) + (q_lane - (unsigned)(rin * D * 2)), soff, lds);
      }
    }
  };
  // Fragment kk of block row r = 32 wave + r32 is chunk 2kk + g, at slot
  // (2kk + g) ^ (r32 mod d/8).
  auto read_q_lds = [&](int s) {
    const int l = fresh_lane(), lr = l & 31;
    const char* qrow = (wave < W / 2 ? kstage(s) : vstage(s)) + (lr + 32 * (wave % (W / 2))) * (2 * D);
    const int x = (l >> 5) ^ (lr & (CPQ - 1));
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 16 * ((2 * kk) ^ x)));
  };

  // ---- per-row state
  f32x16 oacc[D / 32];
  float m_run;   // running maximum of the raw dot product q.k
  float l_lane;  // this lane's share of sum exp2(c (s - m_run))
  auto reset = [&]() {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = (f32x16){};
    m_run = -INFINITY;
    l_lane = 0.f;
  };
  const float c = p.c;

  // K fragment kk of lane (r32, g): row r32 of a 32-key block, chunk 2kk + g,
  // at slot (2kk + g) ^ (r32 mod CPR) = 2kk ^ (g ^ (r32 mod CPR)).
  const int k_off = r32 * G::KS;
  const int k_x = 16 * (g ^ (r32 & (G::CPR - 1)));
  // V^T fragment of block h, half, column block db (A operand: row d = 32 db
  // + l % 32, k = keys 8g .. 8g+7 of the half in P's key order, which is
  // 4g .. 4g+3 and 8+4g .. 8+4g+3): two transposing reads of 8-byte row pieces.
  // Within each 16-lane group, lane i receives element i % 4 of the pieces
  // addressed by lanes i / 4 + 4j (j = 0..3), so lane (q = (l / 16) % 2, m =
  // (l % 16) / 4, e = l % 4) addresses key 4g + m, columns 16 q + 4 e of the
  // segment: lane l then holds column 32 db + l % 32 of keys 4g .. 4g+3; the
  // second read (8 keys on) the other four.
  const unsigned v_frag = [&]() {
    const int vq = (lane >> 4) & 1, vm = (lane & 15) >> 2, ve = lane & 3;
    return (unsigned)((4 * g + vm) * 2 * D + 64 * vseg(4 * g + vm) + 32 * vq + 8 * ve);
  }();

  // S^T = K Q^T for one tile: fragment i = (kk, h) = (i / KB, i % KB).  The
  // source order is already the schedule (LDS reads four fragments ahead of
  // the MFMAs); the scheduling groups below ask for the same order.
  auto qk = [&](const char* kb, f32x16 (&s)[G::KB]) {
    constexpr int NF = G::KB * (D / 16);
    auto frag = [&](int i) {
      const int kk = i / G::KB, h = i % G::KB;
      return *(const bf16x8*)(kb + k_off + h * 32 * G::KS + ((kk * 32) ^ k_x));
    };
    bf16x8 a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = frag(i);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int kk = i / G::KB, h = i % G::KB;
      s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % 4], qf[kk], kk == 0 ? (f32x16){} : s[h], 0, 0, 0);
      if (i + 4 < NF) a[i % 4] = frag(i + 4);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < NF - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };
  // Keys beyond the causal limit or the end of K; exp2(-inf * c) = 0 as c > 0.
  auto mask = [&](f32x16 (&s)[G::KB], int k0, int my_q) {
    const int lim = CAUSAL ? min(my_q + p.diag, Nk - 1) : Nk - 1;
#pragma unroll
    for (int h = 0; h < G::KB; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 32 * h + 8 * (i >> 2) + 4 * g + (i & 3);
        if (key > lim) s[h][i] = -INFINITY;
      }
  };
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
  // time: block h's MFMAs need only block h's probabilities, so the
  // exponentials of block h+1 issue between them, and the V^T fragments are
  // read four MFMAs ahead.  The source order is that schedule (the scheduling
  // groups below ask for the same).  The row sum runs in four partial sums.
  auto softmax_pv = [&](const f32x16 (&s)[G::KB], unsigned vb) {
    const float bias = (m_run == -INFINITY) ? 0.f : -m_run * c;
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
    constexpr int MPB = 2 * (D / 32);  // MFMAs per 32-key block
    constexpr int NM = G::KB * MPB;    // MFMAs per tile
    constexpr int EPM = 16 / MPB;      // next block's exponentials per MFMA
    auto vfrag = [&](int i) {
      const int h = i / MPB, db = (i % MPB) / 2, half = i % 2;
      const unsigned a = ((vb + v_frag) ^ (unsigned)(64 * db)) + (unsigned)((32 * h + 16 * half) * 2 * D);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(a + 16 * D));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto probs = [&](int h, int j0, float* pv) {
#pragma unroll
      for (int j = j0; j < j0 + EPM; ++j) {
        pv[j] = fast_exp2(fmaf(s[h][j], c, bias));
        rs[j & 3] += pv[j];
      }
    };
    float pv[16];
    bf16x8 pb[2];
#pragma unroll
    for (int j0 = 0; j0 < 16; j0 += EPM) probs(0, j0, pv);
    pb[0] = pack_bf16(pv);
    pb[1] = pack_bf16(pv + 8);
    bf16x8 a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = vfrag(i);
    bf16x8 pbn[2];
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int h = i / MPB, m = i % MPB, db = m / 2, half = m % 2;
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % 4], pb[half], oacc[db], 0, 0, 0);
      if (i + 4 < NM) a[i % 4] = vfrag(i + 4);
      if (h + 1 < G::KB) {
        probs(h + 1, m * EPM, pv);
        if ((m + 1) * EPM == 8) pbn[0] = pack_bf16(pv);
        if (m == MPB - 1) {
          pbn[1] = pack_bf16(pv + 8);
          pb[0] = pbn[0];
          pb[1] = pbn[1];
        }
      }
    }
    l_lane += (rs[0] + rs[1]) + (rs[2] + rs[3]);
    constexpr int VPB = 56;                   // vector instructions per block's probabilities
    constexpr int VPM = (VPB + MPB - 1) / MPB;  // per MFMA: one block's worth per block's MFMAs
    __builtin_amdgcn_sched_group_barrier(0x002, VPB, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // two transposing reads per fragment
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + 4 < NM) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
    }
  };

  // ---- epilogue of a block whose last tile sat in stage s (free now): one
  // division by the normaliser, one write of O.
  constexpr int OP = 2 * D;  // LDS row pitch of O (16-byte chunks permuted as in K)
  auto epilogue = [&](const Blk& b, int s) {
    const int el = fresh_lane();
    const int r32 = el & 31, g = el >> 5;
    const int tid = wave * 64 + el;
    const int my_q = b.q0 + wave * 32 + r32;
    const float l_tot = halves_sum(l_lane);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (EPI == kEpiFinalBf16) {
      // O in bf16 through the stage: each lane writes its row's 4-column
      // pieces, then every store to memory is 16 contiguous bytes of one row,
      // 16 lanes per row.  Rows 0..BM/2-1 sit in the stage's K tile, the rest
      // in its V tile; chunk c of row r at slot c ^ (r mod CPR).
      auto orow = [&](int r) { return (r < G::BM / 2 ? kstage(s) + r * OP : vstage(s) + (r - G::BM / 2) * OP); };
      char* const mine = orow(wave * 32 + r32);
      const int ox = r32 & (G::CPR - 1);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          f32x4 v = {oacc[db][4 * r] * inv, oacc[db][4 * r + 1] * inv, oacc[db][4 * r + 2] * inv,
                     oacc[db][4 * r + 3] * inv};
          // columns 32 db + 8 r + 4 g .. +3: chunk 4 db + r, half g
          *(bf16x4*)(mine + 16 * ((4 * db + r) ^ ox) + 8 * g) = __builtin_convertvector(v, bf16x4);
        }
      if (p.lse && g == 0 && my_q < Nq)
        p.lse[(int64_t)b.bh * Nq + my_q] =
            l_tot > 0.f ? m_run * p.scale_abs + __log2f(l_tot) * 0.69314718055994530942f : -INFINITY;
      __syncthreads();
      constexpr int CPO = D / 8;  // 16-byte chunks per O row
      constexpr int NO = G::BM * CPO / G::THREADS;
      constexpr int RPN = G::THREADS / CPO;  // rows per pass
      // Thread tid takes chunk tid % CPO of rows n * RPN + tid / CPO (RPN is a
      // multiple of CPO, so the slot permutation is the same for all n).
      static_assert(RPN % CPO == 0, "one permutation per thread");
      const int rr = tid / CPO, ch = tid % CPO;
      const int cs = 16 * (ch ^ (rr & (CPO - 1)));
      u32x4 ov[NO];
#pragma unroll
      for (int n = 0; n < NO; ++n) ov[n] = *(const u32x4*)(orow(n * RPN + rr) + cs);
      // The stage is refilled next (the next block's second tile, or its
      // first tile and Q).
      __syncthreads();
      // Non-temporal: this kernel never reads O back, and a block's O left in
      // L2 would push out K/V lines that other workgroups still stream.
      uint16_t* ob = (uint16_t*)p.o + ((int64_t)b.bh * Nq + b.q0) * D;
#pragma unroll
      for (int n = 0; n < NO; ++n) {
        const int r = n * RPN + rr;
        if (b.q0 + r < Nq) __builtin_nontemporal_store(ov[n], (u32x4*)(ob + (int64_t)r * D + 8 * ch));
      }
    } else if (my_q < Nq) {
      const int64_t row = (int64_t)b.bh * Nq + my_q;
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
            const f32x4 bb = {oacc[db][4 * r], oacc[db][4 * r + 1], oacc[db][4 * r + 2], oacc[db][4 * r + 3]};
            const f32x4 v = ca * a + cb * bb;
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
  };

  // ---- block loop.  The K/V stream does not stop between blocks: the last
  // tile of a block loads the next block's first tile into the other stage
  // and, once its own Q.K^T products are issued, the next block's Q rows
  // straight into the fragments.  Only a workgroup's first block (or one
  // after a block with no tiles) is started from idle, with its Q through LDS.
  Blk cur;
  if (!describe(0, cur)) return;  // the grid never exceeds the block count
  int st = 0;                     // stage of the next tile to compute
  bool have_t0 = false, have_q = false;
  for (int k = 0;; ++k) {
    reset();
    if (!have_t0 || !have_q) {
      if (!have_t0 && cur.ntiles > 0) {
        load_k(cur.bh, 0, st);
        load_v(cur.bh, 0, st);
      }
      if (!have_q) load_q_lds(cur, st ^ 1);
      publish();
      if (!have_q) {
        read_q_lds(st ^ 1);
        __syncthreads();  // stage st^1 is refilled by the first tile's transfers
      }
    }
    fix_q(cur);
    const int my_q = cur.q0 + wave * 32 + r32;
    Blk nxt = cur;  // (stays cur when there is no next block)
    const bool has_next = describe(k + 1, nxt);
    const bool pre_q = has_next && cur.ntiles > 0;
    const bool pre_t0 = pre_q && nxt.ntiles > 0;
    for (int t = 0; t < cur.ntiles; ++t) {
      // The tile loaded now: this block's next one, or on its last tile the
      // next block's first.
      const bool last = t + 1 == cur.ntiles;
      const bool fill = !last || pre_t0;
      const int lbh = last ? nxt.bh : cur.bh;
      const int lt = last ? 0 : t + 1;
      if (fill) {
        load_k(lbh, lt, st ^ 1);
        load_v(lbh, lt, st ^ 1);
      }
      f32x16 sc[G::KB];
      if (t < cur.wtiles) {
        qk(kstage(st), sc);
        if (t * BN + BN > cur.wmask_from) mask(sc, t * BN, my_q);
        rebase(rowmax(sc));
      }
      if (last && pre_q) {
        __builtin_amdgcn_sched_barrier(0);
        load_q_regs(nxt);  // the fragments are free once the products above are issued
        __builtin_amdgcn_sched_barrier(0);
      }
      if (t < cur.wtiles) softmax_pv(sc, vstage_lds(st));
      publish();
      st ^= 1;
    }
    epilogue(cur, st ^ 1);
    if (!has_next) break;
    cur = nxt;
    have_t0 = pre_t0;
    have_q = pre_q;
  }
}

template <int D, bool CAUSAL, int EPI>
static hipError_t launch_one(FwdParams p, hipStream_t s) {
  constexpr int W = kWavesBf16, BN = kTileBf16;
  p.nqb = (p.Nq + 32 * W - 1) / (32 * W);
  // Persistent: at most one workgroup per compute unit (one fits, by LDS).
  const int nblocks = p.nqb * p.BH;
  const dim3 grid((unsigned)(p.ncu > 0 && p.ncu < nblocks ? p.ncu : nblocks));
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
