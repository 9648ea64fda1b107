// Internal declarations shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

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
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;  // an LDS operand of the transposing reads
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// -------------------------------------------------------------- tile geometry
// Every wavefront owns 32 query rows; a workgroup of kWaves wavefronts owns
// kBM rows (the bf16 kernel uses its own, larger workgroups); each inner
// iteration consumes kBN keys.
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;
constexpr int kBN = 64;
// bf16 forward: 8 wavefronts = 256 query rows per workgroup, one workgroup per
// compute unit, 128-key tiles; every K/V tile staged into LDS serves 256 rows.
constexpr int kWavesBf16 = 8;
constexpr int kTileBf16 = 128;

// What the epilogue of the forward kernels writes.
enum Epilogue : int {
  kEpiFinalBf16 = 0,  // O normalised, bf16; LSE (optional)
  kEpiState = 1,      // O normalised fp32, m (natural units), l
  kEpiFinalF32 = 2,   // O normalised, fp32; LSE (optional)
  kEpiMerge = 3,      // block state merged in place into the fp32 accumulator
                      // (o, m_out, l_out); o_final (bf16) and lse optional
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
  float* m_out;  // state and merge epilogues
  float* l_out;  // state and merge epilogues
  void* o_final; // merge epilogue: bf16 copy of the merged O, may be null
  int Nq, Nk;
  int BH;        // B * H
  int nqb;       // query blocks per (b,h) slice: ceil(Nq / rows per workgroup), set by the launcher
  int diag;      // causal: key j allowed for row i iff j <= i + diag
  float c;       // |scale| * log2(e) (> 0): raw dot product -> base-2 exponent
  float scale_abs;
  // Q element bits are replaced by (bits & q_and) ^ q_xor (mask for 16-bit
  // lanes, repeated): flips Q's sign when scale < 0 so that c > 0, and zeroes Q
  // when scale == 0 (all scores 0, the same problem as Q = 0).
  uint32_t q_and;
  uint32_t q_xor;
  // Workgroup order: workgroup g computes the tile of index (g * perm_mul +
  // perm_add) mod grid (perm_mul coprime to the grid size, so a bijection);
  // perm_mul = 0 is the identity.  Only the diagnostic entry point sets it.
  uint32_t perm_mul;
  uint32_t perm_add;
  // Compute units of the device (0 if unknown): persistent kernels launch at
  // most this many workgroups.
  int ncu;
};

// Tile index of this workgroup under the FwdParams workgroup order.
__device__ inline int tile_index(const FwdParams& p) {
  if (p.perm_mul == 0) return blockIdx.x;
  return (int)(((uint64_t)blockIdx.x * p.perm_mul + p.perm_add) % gridDim.x);
}
// The same order applied to block g of n (persistent kernels, which walk
// several blocks per workgroup).
__device__ inline int block_perm(const FwdParams& p, int g, int n) {
  if (p.perm_mul == 0) return g;
  return (int)(((uint64_t)g * p.perm_mul + p.perm_add) % (uint64_t)n);
}

// Persistent schedule: the k-th block (in map_block's numbering) of workgroup
// w of a grid of G, or -1 when it has no k-th block.  Rounds alternate
// direction (snake order), so with blocks numbered heaviest first every
// workgroup gets a near-equal share of tiles.  When G and n are multiples of
// 8, workgroup w only takes blocks g with g % 8 == w % 8: the workgroups on
// one XCD share that XCD's slices, and their K/V stays in its L2.  Every block
// goes to exactly one workgroup.
__device__ inline int sched_block(int k, int w, int G, int n) {
  if ((G & 7) == 0 && (n & 7) == 0) {
    const int x = w & 7, i = w >> 3, gx = G >> 3;
    const int t = k * gx + ((k & 1) ? gx - 1 - i : i);
    return t < (n >> 3) ? 8 * t + x : -1;
  }
  const int r = k * G + ((k & 1) ? G - 1 - w : w);
  return r < n ? r : -1;
}

// Causal persistent schedule in pairs.  With a square causal mask, query
// block j of a slice sees the first (j + 1) * BM keys and block nqb-1-j the
// first (nqb - j) * BM, so the pair (nqb-1-j, j) always covers (nqb + 1) * BM
// keys: a workgroup that takes whole pairs gets an exact share of the tiles.  Workgroup w (XCD
// w % 8) takes units u = r * G/8 + w / 8, r = 0, 1, ..., of its XCD's
// (BH/8) * (nqb/2) units; unit u is pair u % (nqb/2) of the XCD's slice
// u / (nqb/2), heavier block first.  The workgroups of an XCD that run at the
// same time therefore cover few slices, and the ones on the same slice stream
// its K/V tiles in step, out of the XCD's L2.  Returns the k-th block of
// workgroup w in map_block's numbering, or -1 when there is none.  Used when
// every workgroup gets at least one pair (fewer pairs than workgroups would
// leave some idle that the per-block schedule keeps busy).
__device__ inline bool pair_sched_ok(int G, int nqb, int BH) {
  return (G & 7) == 0 && (BH & 7) == 0 && (nqb & 1) == 0 && (BH >> 3) * (nqb >> 1) >= (G >> 3);
}
__device__ inline int sched_block_pairs(int k, int w, int G, int nqb, int BH) {
  const int x = w & 7, i = w >> 3, gx = G >> 3;
  const int hp = BH >> 3, np = nqb >> 1;
  const int u = (k >> 1) * gx + i;
  if (u >= hp * np) return -1;
  const int s = u / np, j = u % np;
  const int qi = (k & 1) ? nqb - 1 - j : j;  // map_block turns qi into qb = nqb - 1 - qi
  return 8 * (qi * hp + s) + x;
}

// Launchers (host side). Each returns hipGetLastError() after the launch.
hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, int epi, hipStream_t s);
hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, hipStream_t s);
// fp8 forward modes: QK^T on fp8 or fp16 matrix cores (P.V on fp16), or both
// products on f8f6f4 matrix cores with P in e4m3, or P in e2m1 (rounded
// exponential, or Direct-P: score mapped straight to the code).
enum Fp8Mode : int { kFp8QkFp8 = 0, kFp8QkFp16 = 1, kFp8AllFp8 = 2, kFp8PvFp4 = 3, kFp8PvFp4Direct = 4 };
hipError_t launch_fwd_fp8(const FwdParams& p, int d, bool causal, int mode, hipStream_t s);

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

// Backward pass (gradients of sum(dO * O)).  All tensors [B,H,N,d] bf16 except
// lse (fp32 [B,H,Nq], natural log, as the forward writes it) and delta (fp32
// [B,H,Nq] workspace: D_i = dO_i . O_i).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* delta;
  void* dq;
  void* dk;
  void* dv;
  int Nq, Nk;
  int BH;
  int diag;      // causal: key j allowed for row i iff j <= i + diag
  float scale;   // any finite value
  float c;       // scale * log2(e)
};
hipError_t launch_bwd(const BwdParams& p, int d, bool causal, hipStream_t s);

// Matrix-core measurements (mfma_probe.hip): kind 0 bf16, 1 fp16, 2 fp8
// (f8f6f4 with unit scales), 3 fp32.
double mfma_flop_per_instruction(int kind);
hipError_t launch_mfma_peak(int kind, int workgroups, int iters, float* out, hipStream_t s);
hipError_t launch_mfma_dot(int kind, const void* a, const void* b, float* c, hipStream_t s);

// ------------------------------------------------------------ device helpers
// Workgroup -> (query block, b*h slice).  Workgroups are dealt to the 8 XCDs
// round-robin (XCD = blockIdx % 8); when the slices divide evenly, each XCD is
// given a contiguous range of (b,h) slices, so a slice's K/V is only ever
// cached in one XCD's L2.  Inside an XCD the order is query-block level by
// level, heaviest level first for causal masks (longest-processing-time-first
// list scheduling of blocks whose lengths differ by up to Nk/kBN tiles).
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

// f(integral_constant<int, I>) for I = B .. E-1, expanded at compile time.
template <int B, int E, typename F>
__device__ __attribute__((always_inline)) inline void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// One wave-wide direct load of 64 x 16 bytes from global memory into LDS at
// lds_base + 16 * lane.  Issued as assembly so the compiler does not treat
// every later LDS read as possibly aliasing an outstanding transfer (which
// makes it wait for all LDS reads before each use, defeating the read-ahead);
// the kernel orders these transfers itself: vmcnt(0) and a barrier before any
// wavefront reads the stage, and a barrier after the last read before the
// stage is reloaded.
__device__ inline void load_lds16(const void* src, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(src) : "memory", "m0");
}
// The same transfer from a wave-uniform base plus a 32-bit per-lane byte
// offset (scalar-base form: no 64-bit lane address, so no VGPR pair).
__device__ inline void load_lds16_s(const void* sbase, unsigned voff, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// Wave-wide global->LDS transfers through a buffer resource: 16 bytes per lane
// from rsrc.base + soff + voff into LDS at lds + 16 * lane; soff and lds then
// advance by SSTEP and LSTEP bytes inside the same statement, so a run of
// transfers needs no precomputed addresses.  As with load_lds16, the kernel
// orders the transfers itself (vmcnt(0) and a barrier before the data is read).
typedef int i32x4 __attribute__((ext_vector_type(4)));
template <int SSTEP, int LSTEP>
__device__ inline void buf_lds16(i32x4 rsrc, unsigned voff, unsigned& soff, unsigned& lds) {
  asm volatile(
      "s_mov_b32 m0, %[l]\n\tbuffer_load_dwordx4 %[v], %[r], %[s] offen lds\n\t"
      "s_add_u32 %[s], %[s], %[ss]\n\ts_add_u32 %[l], %[l], %[ls]"
      : [s] "+s"(soff), [l] "+s"(lds)
      : [v] "v"(voff), [r] "s"(rsrc), [ss] "i"(SSTEP), [ls] "i"(LSTEP)
      : "memory", "m0", "scc");
}
// Raw buffer resource starting at base (no range check is relied on: every
// offset the kernels use stays inside the tensor).
__device__ inline i32x4 buffer_rsrc(const void* base) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4 r = {(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), -1, 0x00020000};
  r[0] = __builtin_amdgcn_readfirstlane(r[0]);
  r[1] = __builtin_amdgcn_readfirstlane(r[1]);
  return r;
}
// The same with a range: accesses at byte offsets >= nbytes read as zero and
// never touch memory (raw buffer, no swizzle).
__device__ inline i32x4 buffer_rsrc_n(const void* base, unsigned nbytes) {
  i32x4 r = buffer_rsrc(base);
  r[2] = (int)__builtin_amdgcn_readfirstlane(nbytes);
  return r;
}
__device__ inline unsigned lds_offset(const void* x) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)x;
}

// ---------------------------------------------------------------- V^T tile
// The P.V product reads V with keys along the MFMA k dimension, i.e. 8 keys of
// one column d per lane.  V is therefore staged into LDS transposed: one LDS row
// per column d, holding the tile's keys as 16-bit values.  Inside every
// 16-key group the keys are stored in the order that makes the 8 keys one lane
// needs for one MFMA adjacent: key 16q + 8a + 4g + b sits in slot
// 16q + 8g + 4a + b (bits 2 and 3 of the key index swapped), matching the keys
// the S^T accumulator hands each lane (rows 8*(i/4) + 4*(l/32) + i%4).  So one
// ds_read_b128 fetches a whole A fragment.  The row pitch (tile keys + 16
// bytes) keeps both the 16-byte reads down 32 consecutive rows and the 8-byte
// writes of the staging free of bank conflicts.
__host__ __device__ constexpr int vt_pitch(int bn) { return bn * 2 + 16; }
constexpr int kVtPitch = vt_pitch(kBN);

// Slot of key group kg (keys 4kg .. 4kg+3) inside a V^T row.
__device__ inline int vt_slot(int kg) { return 16 * (kg >> 2) + 8 * (kg & 1) + 4 * ((kg >> 1) & 1); }

// Store four keys (w[r] = 8 consecutive 16-bit values of key 4kg + r, columns
// d0 .. d0+7) into V^T rows d0 .. d0+7 of row pitch `pitch` bytes.
__device__ inline void store_vt(char* vt, int pitch, int d0, int kg, const u32x4 (&w)[4]) {
  const int col = vt_slot(kg) * 2;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int i = e >> 1;
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;  // high / low halves
    const u32x2 v = {__builtin_amdgcn_perm(w[1][i], w[0][i], sel), __builtin_amdgcn_perm(w[3][i], w[2][i], sel)};
    *(u32x2*)(vt + (d0 + e) * pitch + col) = v;
  }
}


// ---------------------------------------------------------------- W4A16 layer
struct W4Params {
  const uint16_t* x;       // fp16 [M, K]
  const uint32_t* packed;  // [N, K/8]
  const uint16_t* scales;  // fp16 [N, K/128]
  const uint8_t* zeros;    // [N, K/128]
  uint16_t* y;             // fp16 [M, N]
  float* part;             // fp32 [S, M, N] when S > 1, else null
  int M, N, K, NG;         // NG = K / 128
  int S, gps, ntiles;      // set from the plan by the launcher
};
// How a call is cut: S splits of K of gps groups each, gw groups per
// wavefront, ntiles 16-row tiles; work_floats = S * M * N when S > 1.
struct W4Plan {
  int S, gps, gw, ntiles;
  int nw;  // wavefronts per workgroup
  size_t work_floats;
};
W4Plan w4a16_plan(int64_t M, int64_t N, int64_t K);
hipError_t launch_w4a16(const W4Params& p, const W4Plan& pl, int compute_units, hipStream_t s);
// Device address of the fixed split-partial array of w4a16_gemm_noalloc on
// the current device (W4A16_NOALLOC_MAX_WORK_FLOATS floats).
hipError_t w4a16_scratch(float** out);

}  // namespace eta
