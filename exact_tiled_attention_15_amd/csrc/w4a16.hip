// W4A16 linear layer on gfx950: y[m][n] = sum_k x[m][k] * (q[n][k] - z[n][g]) * s[n][g],
// g = k / 128, following the on-the-fly dequantization steps of "Scaling
// FlashAttention, multi-GPU training and weight quantization" (itimpress),
// section 3: packed 4-bit weights are read from HBM once, opened in registers
// with shifts and masks, and fed to the fp16 matrix cores together with the
// fp16 activations; no widened weight is ever written back.
//
// Format: weight k = 8j + e of row n is the 4-bit field at bit 4(e/2) + 16(e%2)
// of word packed[n][j]; zero points are bytes zeros[n][g], scales are fp16
// scales[n][g]; x is fp16 [M][K], y is fp16 [M][N].
//
// Work split.  A workgroup (8 wavefronts) walks 16-row tiles of W; for one
// tile, wavefront w covers a fixed run of up to 8 groups of K, so its share of
// the activations (16 tokens x its K range) stays in registers for the whole
// kernel and only W streams from HBM.  The 8 partial 16x16 results of a tile
// meet in LDS (double-buffered, one barrier per tile) and are summed in a fixed
// order.  Long K is cut into S splits (grid.y) whose fp32 partials a second
// kernel adds in split order, so every result is deterministic.
//
// Unpacking.  With the interleaved field order, one AND-OR puts two codes into
// the mantissas of two fp16 values: fields at bits 0-3 / 16-19 become 1024 + q
// (exponent of 0x6400), fields at bits 4-7 / 20-23 become 64 + q (exponent of
// 0x5400, whose mantissa step is 1/16).  A word costs one shift and four
// AND-ORs for eight weights.  The offsets and the zero point are removed in
// fp32: each group's MFMA chain starts from -(X'g + z Xg), where, per token,
// Xg is the sum of the group's activations and X'g the sum weighted by the
// 1024 / 64 offsets (both computed once per workgroup on the matrix cores).
// The scale multiplies the group's fp32 partial once.  Mathematically this is
// the page's (q - z) * s per weight; it rounds less, since the widened weights
// are exact in fp16.
#include <algorithm>

#include "common.h"

namespace eta {
namespace {

constexpr int kW4Waves = 8;
constexpr int kW4Threads = 64 * kW4Waves;
constexpr int kW4Group = 128;  // k per group: 16 words per row
constexpr int kW4Rows = 16;    // rows of W per tile (one MFMA column block)
constexpr int64_t kW4FillTarget = 256;  // workgroups wanted in flight (MI355X compute units)

__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

// The eight codes of one word as the B operand of a 16x16x32 MFMA (codes in
// k order 0..7): pairs (0,1) and (4,5) as 1024 + q, pairs (2,3) and (6,7) as
// 64 + q.
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic) {
  uint32_t r;
  // One VOP3 instruction; the compiler would split it in two, since gfx950's
  // VOP3 encoding takes no 32-bit literal.
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(magic));
  return r;
}

__device__ __forceinline__ u32x4 widen_word(uint32_t w, uint32_t m1024, uint32_t m64) {
  const uint32_t w8 = w >> 8;
  u32x4 b;
  b[0] = and_or(w, 0x000F000Fu, m1024);
  b[1] = and_or(w, 0x00F000F0u, m64);
  b[2] = and_or(w8, 0x000F000Fu, m1024);
  b[3] = and_or(w8, 0x00F000F0u, m64);
  return b;
}

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(a), as_f16x8(b), c, 0, 0, 0);
}

// MFMA 16x16x32 layout used throughout: lane l = 16 * quad + col.  A operand
// (activations): token col, k = 8 * quad .. + 8 of the 32-k chunk.  B operand
// (weights): row col of the tile, same k.  D: tokens 4 * quad + i (i < 4),
// row col.  Within a group, chunk t of lane quad is word 4 * quad + t of the
// row, so one 16-byte load per lane brings a lane's four words of a group.
template <int GW>
__global__ __launch_bounds__(kW4Threads) void w4a16_kernel(W4Params p) {
  __shared__ float xs[kW4Waves][GW][2][16];        // per token: X'g, Xg
  __shared__ float red[2][kW4Waves][16][kW4Rows];  // per-wave partial tiles

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, quad = lane >> 4;
  const int gs0 = blockIdx.y * p.gps;
  const int gs1 = min(p.NG, gs0 + p.gps);
  const int g0 = gs0 + wave * GW;
  // Groups of this wavefront: [g0, g0 + ng).  Every wavefront runs GW slots
  // over groups gb .. gb + GW - 1 with gb = min(g0, NG - GW) >= 0 (GW <= NG),
  // so every slot reads a valid group; a slot whose group is not one of this
  // wavefront's gets zero activations and adds exactly 0.  No branch depends
  // on ng.
  const int ng = max(0, min(GW, gs1 - g0));
  const int gb = min(g0, p.NG - GW);
  const int64_t kw = p.K >> 3;  // words per row
  const uint32_t m1024 = 0x64006400u, m64 = 0x54005400u;

  u32x4 wb[GW];
  uint32_t sb[GW], zb[GW];
  // Loads of one tile's slots: a uniform base per tile, one 32-bit lane
  // offset, an immediate per slot.  Rows past N re-read row N-1 and are never
  // stored.
  auto issue = [&](int tile, int gi) {
    const int64_t r0 = int64_t(tile) * kW4Rows;
    const uint32_t rr = uint32_t(min(int64_t(col), p.N - 1 - r0));
    const char* wbase = reinterpret_cast<const char*>(p.packed) + r0 * kw * 4 + int64_t(gb) * 64;
    const char* sbase = reinterpret_cast<const char*>(p.scales) + (r0 * p.NG + gb) * 2;
    const char* zbase = reinterpret_cast<const char*>(p.zeros) + r0 * p.NG + gb;
    const uint32_t woff = rr * uint32_t(kw) * 4u + uint32_t(quad) * 16u;
    const uint32_t soff = rr * uint32_t(p.NG);
    wb[gi] = *reinterpret_cast<const u32x4*>(wbase + woff + gi * 64);
    sb[gi] = *reinterpret_cast<const uint16_t*>(sbase + soff * 2u + gi * 2);
    zb[gi] = *reinterpret_cast<const uint8_t*>(zbase + soff + gi);
  };
  const int tile0 = min(int(blockIdx.x), p.ntiles - 1);
#pragma unroll
  for (int gi = 0; gi < GW; ++gi) issue(tile0, gi);

  // Activations of each slot's group, in A-operand layout (zero for tokens
  // >= M and for groups that are not this wavefront's).
  u32x4 xa[GW][4];
  const bool live_tok = col < p.M;
  const uint16_t* xrow = p.x + int64_t(live_tok ? col : 0) * p.K;
#pragma unroll
  for (int gi = 0; gi < GW; ++gi)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      xa[gi][t] = u32x4{0u, 0u, 0u, 0u};
      const int g = gb + gi;
      if (g >= g0 && g < g0 + ng && live_tok)
        xa[gi][t] = *reinterpret_cast<const u32x4*>(xrow + g * kW4Group + 8 * (4 * quad + t));
    }

  // X'g (column 0: the widening offsets) and Xg (column 1: ones) per token.
  {
    u32x4 bc = u32x4{0u, 0u, 0u, 0u};
    if (col == 0) bc = u32x4{m1024, m64, m1024, m64};
    if (col == 1) bc = u32x4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
#pragma unroll
    for (int gi = 0; gi < GW; ++gi) {
      f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t) d = mfma16(xa[gi][t], bc, d);
      if (col < 2) *reinterpret_cast<f32x4*>(&xs[wave][gi][col][4 * quad]) = d;
    }
  }
  __syncthreads();

  int par = 0;
  for (int tile = blockIdx.x; tile < p.ntiles; tile += gridDim.x) {
    // The last tile re-loads itself (cache hits) instead of branching.
    const int next = (tile + int(gridDim.x) < p.ntiles) ? tile + int(gridDim.x) : tile;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gi = 0; gi < GW; ++gi) {
      const f32x4 xp = *reinterpret_cast<const f32x4*>(&xs[wave][gi][0][4 * quad]);
      const f32x4 xq = *reinterpret_cast<const f32x4*>(&xs[wave][gi][1][4 * quad]);
      const float z = float(zb[gi] & 0xFFu);
      const float s = float(__builtin_bit_cast(_Float16, uint16_t(sb[gi])));
      u32x4 b[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) b[t] = widen_word(wb[gi][t], m1024, m64);
      f32x4 d;
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = fmaf(-z, xq[i], -xp[i]);
#pragma unroll
      for (int t = 0; t < 4; ++t) d = mfma16(xa[gi][t], b[t], d);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(s, d[i], acc[i]);
      // The slot's registers are free now: prefetch its group of the next tile.
      // Loads complete in issue order; keeping each slot's prefetch inside its
      // own group lets every wait name exactly the slot it needs.
      issue(next, gi);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) red[par][wave][4 * quad + i][col] = acc[i];
    __syncthreads();
    if (threadIdx.x < 16 * kW4Rows) {
      const int m = threadIdx.x / kW4Rows, c = threadIdx.x % kW4Rows;
      const int n = tile * kW4Rows + c;
      if (m < p.M && n < p.N) {
        float sum = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < kW4Waves; ++w2) sum += red[par][w2][m][c];
        if (p.part)
          p.part[(int64_t(blockIdx.y) * p.M + m) * p.N + n] = sum;
        else
          p.y[int64_t(m) * p.N + n] = __builtin_bit_cast(uint16_t, _Float16(sum));
      }
    }
    par ^= 1;
  }
}

// y = fp16(sum over splits of part), splits added in order 0..S-1.
__global__ __launch_bounds__(256) void w4a16_reduce_kernel(const float* __restrict__ part, uint16_t* __restrict__ y,
                                                           int S, int64_t MN) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= MN) return;
  float sum = 0.f;
  for (int s = 0; s < S; ++s) sum += part[int64_t(s) * MN + i];
  y[i] = __builtin_bit_cast(uint16_t, _Float16(sum));
}

template <int GW>
hipError_t launch_gw(const W4Params& p, int gx, hipStream_t s) {
  hipLaunchKernelGGL(w4a16_kernel<GW>, dim3(gx, p.S), dim3(kW4Threads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

W4Plan w4a16_plan(int64_t M, int64_t N, int64_t K) {
  W4Plan pl{};
  const int64_t NG = K / kW4Group;
  const int64_t ntiles = (N + kW4Rows - 1) / kW4Rows;
  int64_t S = (NG + 8 * kW4Waves - 1) / (8 * kW4Waves);  // at most 8 groups per wavefront
  // Too few tiles for one workgroup per compute unit of the chip: cut K
  // further.  The target is a constant, so the split (and with it the order of
  // the fp32 additions) depends on the sizes only.
  if (ntiles * S < kW4FillTarget)
    S = std::min<int64_t>(NG, std::max<int64_t>(S, (kW4FillTarget + ntiles - 1) / ntiles));
  const int64_t gps = (NG + S - 1) / S;
  S = (NG + gps - 1) / gps;  // drop splits left empty by the rounding
  pl.S = int(S);
  pl.gps = int(gps);
  pl.gw = int((gps + kW4Waves - 1) / kW4Waves);
  pl.ntiles = int(ntiles);
  pl.work_floats = S > 1 ? size_t(S) * size_t(M) * size_t(N) : 0;
  return pl;
}

hipError_t launch_w4a16(const W4Params& p0, const W4Plan& pl, int compute_units, hipStream_t s) {
  W4Params p = p0;
  const int gx = int(std::max<int64_t>(1, std::min<int64_t>(pl.ntiles, (compute_units + pl.S - 1) / pl.S)));
  p.S = pl.S;
  p.gps = pl.gps;
  p.ntiles = pl.ntiles;
  hipError_t e;
  switch (pl.gw) {
    case 1: e = launch_gw<1>(p, gx, s); break;
    case 2: e = launch_gw<2>(p, gx, s); break;
    case 3: e = launch_gw<3>(p, gx, s); break;
    case 4: e = launch_gw<4>(p, gx, s); break;
    case 5: e = launch_gw<5>(p, gx, s); break;
    case 6: e = launch_gw<6>(p, gx, s); break;
    case 7: e = launch_gw<7>(p, gx, s); break;
    case 8: e = launch_gw<8>(p, gx, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || pl.S == 1) return e;
  const int64_t MN = int64_t(p.M) * p.N;
  hipLaunchKernelGGL(w4a16_reduce_kernel, dim3(unsigned((MN + 255) / 256)), dim3(256), 0, s, p.part, p.y, pl.S, MN);
  return hipGetLastError();
}

}  // namespace eta
