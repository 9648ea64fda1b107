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
// Work split.  A workgroup (8 wavefronts, one per compute unit) walks 16-row
// tiles of W; wavefront w always covers the same run of up to 8 groups of K,
// so its share of the activations (16 tokens x its K range) stays in registers
// for the whole kernel and only W streams from HBM, through a ring of a few
// 1 KB slots per wavefront.  Each tile's scales and zero points are loaded once
// by the whole workgroup into an LDS table, a tile ahead.  The 8 partial 16x16
// results of a tile meet in LDS (double-buffered, one barrier per tile) and
// are summed in a fixed order.  Long K is cut into S splits (grid.y) whose
// fp32 partials a second kernel adds in split order, so every result is
// deterministic.
//
// Activations are loaded coalesced (4 tokens x 256 B per load) and turned into
// the MFMA operand layout through a small LDS tile by the first tile, group by
// group, while the weight stream is already running.
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
#include <type_traits>

#include <atomic>
#include <mutex>

#include "common.h"
#include "w4a16.h"

// Split partials of w4a16_gemm_noalloc: a fixed device array, one copy per
// GPU, held until the process ends.  Host code never passes this name to a
// kernel (on the host it is only a stand-in for the symbol): the device
// address comes from w4a16_scratch below.
static __device__ __align__(256) float scratch[W4A16_NOALLOC_MAX_WORK_FLOATS];

namespace eta {

// Device address of `scratch` on the current device, looked up once per device
// (hipGetSymbolAddress with that device current) and kept.
hipError_t w4a16_scratch(float** out) {
  constexpr int kDevices = 64;
  static std::atomic<float*> ptrs[kDevices];
  static std::mutex mu;
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
  float* p = ptrs[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(mu);
    p = ptrs[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* a = nullptr;
      if (hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch))) return e;
      if (!a) return hipErrorInvalidSymbol;
      p = static_cast<float*>(a);
      ptrs[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

namespace {

constexpr int kW4Waves = 8;
constexpr int kW4Threads = 64 * kW4Waves;
constexpr int kW4Group = 128;  // k per group: 16 words per row
constexpr int kW4Rows = 16;    // rows of W per tile (one MFMA column block)
constexpr int64_t kW4FillTarget = 256;  // workgroups wanted in flight (MI355X compute units)
constexpr int kW4MaxSplitGroups = 8 * kW4Waves;  // groups of one K split: 8 per wavefront
constexpr int kW4ReduceUnroll = 8;               // split partials requested together

__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

// (w & mask) | magic as one instruction.
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic) {
  uint32_t r;
  // One VOP3 instruction; the compiler would split it in two, since gfx950's
  // VOP3 encoding takes no 32-bit literal.
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(magic));
  return r;
}

// The eight codes of one word as the B operand of a 16x16x32 MFMA (codes in
// k order 0..7): pairs (0,1) and (4,5) as 1024 + q, pairs (2,3) and (6,7) as
// 64 + q.
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
//
// Weight words in flight per wavefront: a ring of D slots of one group each
// (16 rows x 64 B per slot).  Three or four 1 KB slots per wavefront (24-32 KB
// per compute unit) stream this access pattern fastest on MI355X; deeper
// queues are slower.  D divides GW, so a group keeps its slot across tiles.
template <int GW>
constexpr int ring_depth() { return GW == 8 ? 4 : GW == 6 ? 3 : GW; }

template <int GW, int NW>
__global__ __launch_bounds__(64 * NW) void w4a16_kernel(W4Params p) {
  constexpr int D = ring_depth<GW>();
  static_assert(GW % D == 0, "ring depth must divide the slots per wavefront");
  constexpr int kTab = kW4MaxSplitGroups + 1;  // last column: zero scale for dead slots
  __shared__ float xs[NW][GW][2][16];        // per token: X'g, Xg
  // Per-wave partial tiles, row c of W (column of y) by token, each row padded
  // to 20 floats: the 16-byte writes of a wavefront (4 tokens of one row per
  // lane) and the reducing reads (16 rows of one token) both fall on distinct
  // banks.
  constexpr int kRedPitch = 20;
  __shared__ float red[2][NW][kW4Rows][kRedPitch];
  __shared__ float2 sz[2][kW4Rows][kTab];          // per tile: (scale, zero point) of each group
  // Activation staging, one group per wavefront: 16 tokens x 16 chunks of
  // 16 B, rows padded by one chunk so the transposed reads are conflict-free.
  __shared__ u32x4 xst[NW][16][17];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, quad = lane >> 4;
  const int gs0 = blockIdx.y * p.gps;
  const int gs1 = min(p.NG, gs0 + p.gps);
  const int ngs = gs1 - gs0;  // groups of this split (<= kW4MaxSplitGroups)
  const int g0 = gs0 + wave * GW;
  // Groups of this wavefront: [g0, g0 + ng).  Every wavefront runs GW slots
  // over groups gb .. gb + GW - 1 with gb = min(g0, NG - GW) >= 0 (GW <= NG),
  // so every slot reads a valid group; a slot whose group is not one of this
  // wavefront's gets zero activations and a zero scale, and adds exactly 0.
  const int ng = max(0, min(GW, gs1 - g0));
  const int gb = min(g0, p.NG - GW);
  const int64_t kw = p.K >> 3;  // words per row
  const uint32_t m1024 = 0x64006400u, m64 = 0x54005400u;
  const int tstep = gridDim.x;
  auto grp = [&](int gi) { return gb + gi; };  // group held by slot gi

  // ---- weight ring: group gi of a tile lives in slot gi % D
  u32x4 ring[D];
  // Per-lane address parts are 32-bit (a 16-row tile of W is below 4 GiB);
  // 64-bit parts are wave-uniform.
  auto row_in_tile = [&](int tile, int r) {  // rows past N re-read row N-1, never stored
    const int rmax = int(min(int64_t(kW4Rows - 1), p.N - 1 - int64_t(tile) * kW4Rows));
    return uint32_t(min(r, rmax));
  };
  auto issue = [&](int tile, int gi) {
    const char* wbase = reinterpret_cast<const char*>(p.packed) + (int64_t(tile) * kW4Rows * kw + grp(gi) * 16) * 4;
    const uint32_t woff = row_in_tile(tile, col) * uint32_t(kw * 4) + uint32_t(quad) * 16u;
    ring[gi % D] = *reinterpret_cast<const u32x4*>(wbase + woff);
  };

  // ---- (scale, zero point) table of a tile: loaded by the whole workgroup,
  // two entries per thread, converted once, parked in registers until the
  // tile before it ends, then written to LDS.
  int e_row[2], e_col[2];
  bool e_live[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = threadIdx.x + j * (64 * NW);
    e_live[j] = e < kW4Rows * ngs;
    e_row[j] = e_live[j] ? e / ngs : 0;
    e_col[j] = e_live[j] ? e % ngs : 0;
  }
  uint32_t sreg[2], zreg[2];
  auto issue_sz = [&](int tile) {
    const int64_t base = int64_t(tile) * kW4Rows * p.NG + gs0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // unconditional (dead entries read entry 0): every wait stays exact
      const uint32_t i = row_in_tile(tile, e_row[j]) * uint32_t(p.NG) + uint32_t(e_col[j]);
      sreg[j] = (p.scales + base)[i];
      zreg[j] = (p.zeros + base)[i];
    }
  };
  auto park_sz = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (e_live[j])
        sz[buf][e_row[j]][e_col[j]] =
            float2{float(__builtin_bit_cast(_Float16, uint16_t(sreg[j]))), float(zreg[j] & 0xFFu)};
  };
  // Table column of each slot (dead slots read the zero column).
  int tcol[GW];
#pragma unroll
  for (int gi = 0; gi < GW; ++gi) {
    const int g = grp(gi);
    tcol[gi] = (g >= g0 && g < g0 + ng) ? g - gs0 : kTab - 1;
  }

  // Prologue: this workgroup's first (scale, zero) table, its first D weight
  // slots, then every activation load, all without waiting.  The first tile
  // consumes the activations group by group, so they arrive while the weight
  // stream is already running.
  const int tile0 = min(int(blockIdx.x), p.ntiles - 1);
  issue_sz(tile0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int gi = 0; gi < D; ++gi) issue(tile0, gi);
  __builtin_amdgcn_sched_barrier(0);

  // Activations.  A group's 16 tokens x 256 B are loaded coalesced (load j:
  // tokens 4j..4j+3, one 16-byte chunk per lane, 8 full cache lines) and
  // turned into the A-operand layout through LDS by the first tile.  Loading
  // them in that layout directly touches 32 half-used lines per load and costs
  // three times as much address-unit time.  Loads are unconditional (tokens >=
  // M read token 0) so that every wait names its group; they run two groups
  // ahead of the first tile, interleaved with the weight stream.
  constexpr int kXAhead = GW < 2 ? GW : 2;
  u32x4 xa[GW][4];
  auto issue_x = [&](int gi) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = 4 * j + (lane >> 4);
      const uint16_t* src = p.x + int64_t(m < p.M ? m : 0) * p.K + grp(gi) * kW4Group + 8 * (lane & 15);
      xa[gi][j] = *reinterpret_cast<const u32x4*>(src);
    }
  };
  const bool live_tok = col < p.M;
#pragma unroll
  for (int gi = 0; gi < kXAhead; ++gi) issue_x(gi);
  __builtin_amdgcn_sched_barrier(0);

  if (threadIdx.x < 2 * kW4Rows) sz[threadIdx.x / kW4Rows][threadIdx.x % kW4Rows][kTab - 1] = float2{0.f, 0.f};
  park_sz(0);
  issue_sz(min(int(blockIdx.x) + tstep, p.ntiles - 1));
  __syncthreads();

  // B operand that turns a group's activations into X'g (column 0: the
  // widening offsets) and Xg (column 1: ones) per token.
  u32x4 bc = u32x4{0u, 0u, 0u, 0u};
  if (col == 0) bc = u32x4{m1024, m64, m1024, m64};
  if (col == 1) bc = u32x4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};

  auto tile_body = [&](int tile, int par, auto first) {
    constexpr bool kFirst = decltype(first)::value;
    // Prefetches past the last tile re-load this tile (cache hits, no branch).
    const int next = (tile + tstep < p.ntiles) ? tile + tstep : tile;
    const int next2 = (tile + 2 * tstep < p.ntiles) ? tile + 2 * tstep : next;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gi = 0; gi < GW; ++gi) {
      if constexpr (kFirst) {
        // Coalesced chunks -> A-operand layout (token col, chunks 4 quad + t).
        // One staging tile per wavefront; LDS runs a wavefront's accesses in
        // order, so the next group's writes cannot pass these reads.
#pragma unroll
        for (int j = 0; j < 4; ++j) xst[wave][4 * j + (lane >> 4)][lane & 15] = xa[gi][j];
#pragma unroll
        for (int t = 0; t < 4; ++t) xa[gi][t] = xst[wave][col][4 * quad + t];
        const bool live = (grp(gi) >= g0) && (grp(gi) < g0 + ng) && live_tok;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int c = 0; c < 4; ++c) xa[gi][t][c] = live ? xa[gi][t][c] : 0u;
        // X'g and Xg of this group, on the matrix cores, into this wavefront's
        // LDS rows (read back below by the same wavefront, in order).
        f32x4 d0 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) d0 = mfma16(xa[gi][t], bc, d0);
        if (col < 2) *reinterpret_cast<f32x4*>(&xs[wave][gi][col][4 * quad]) = d0;
      }
      const f32x4 xp = *reinterpret_cast<const f32x4*>(&xs[wave][gi][0][4 * quad]);
      const f32x4 xq = *reinterpret_cast<const f32x4*>(&xs[wave][gi][1][4 * quad]);
      const float2 sc = sz[par][col][tcol[gi]];
      u32x4 b[4];
      const u32x4 w = ring[gi % D];
#pragma unroll
      for (int t = 0; t < 4; ++t) b[t] = widen_word(w[t], m1024, m64);
      f32x4 d;
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = fmaf(-sc.y, xq[i], -xp[i]);
#pragma unroll
      for (int t = 0; t < 4; ++t) d = mfma16(xa[gi][t], b[t], d);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(sc.x, d[i], acc[i]);
      // The slot is free: refill it with the group D ahead (this tile or the
      // next).  Loads complete in issue order; keeping each refill inside its
      // own group lets every wait name exactly the slot it needs.
      if (gi + D < GW)
        issue(tile, gi + D);
      else
        issue(next, gi + D - GW);
      if constexpr (kFirst) {
        if (gi + kXAhead < GW) issue_x(gi + kXAhead);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    *reinterpret_cast<f32x4*>(&red[par][wave][col][4 * quad]) = acc;
    park_sz(par ^ 1);  // the table of the next tile (its loads were issued a tile ago)
    issue_sz(next2);
    __syncthreads();
    if (threadIdx.x < 16 * kW4Rows) {
      const int m = threadIdx.x / kW4Rows, c = threadIdx.x % kW4Rows;
      const int n = tile * kW4Rows + c;
      if (m < p.M && n < p.N) {
        float sum = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) sum += red[par][w2][c][m];
        if (p.part)
          p.part[(int64_t(blockIdx.y) * p.M + m) * p.N + n] = sum;
        else
          p.y[int64_t(m) * p.N + n] = __builtin_bit_cast(uint16_t, _Float16(sum));
      }
    }
  };

  tile_body(int(blockIdx.x), 0, std::true_type{});  // the grid never exceeds the tile count
  int par = 1;
  for (int tile = blockIdx.x + tstep; tile < p.ntiles; tile += tstep) {
    tile_body(tile, par, std::false_type{});
    par ^= 1;
  }
}

// y = fp16(sum over splits of part), splits added in order 0..S-1; four
// outputs per thread, vectorised when the pointers allow it.
__global__ __launch_bounds__(256) void w4a16_reduce_kernel(const float* __restrict__ part, uint16_t* __restrict__ y,
                                                           int S, int64_t MN) {
  const int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  const bool vec = (MN & 3) == 0 && (reinterpret_cast<uintptr_t>(part) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(y) & 7) == 0;
  if (vec && i + 4 <= MN) {
    // Every partial is requested before the first is added (one memory
    // latency, not S), then they are added in split order.
    f32x4 v[kW4ReduceUnroll];
    f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += kW4ReduceUnroll) {
#pragma unroll
      for (int u = 0; u < kW4ReduceUnroll; ++u)
        if (s0 + u < S) v[u] = *reinterpret_cast<const f32x4*>(part + int64_t(s0 + u) * MN + i);
#pragma unroll
      for (int u = 0; u < kW4ReduceUnroll; ++u)
        if (s0 + u < S) sum = (s0 + u == 0) ? v[u] : sum + v[u];
    }
    uint16_t o[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = __builtin_bit_cast(uint16_t, _Float16(sum[c]));
    *reinterpret_cast<uint2*>(y + i) = uint2{o[0] | (uint32_t(o[1]) << 16), o[2] | (uint32_t(o[3]) << 16)};
    return;
  }
  for (int64_t j = i; j < i + 4 && j < MN; ++j) {
    float sum = part[j];
    for (int s = 1; s < S; ++s) sum += part[int64_t(s) * MN + j];
    y[j] = __builtin_bit_cast(uint16_t, _Float16(sum));
  }
}

template <int GW, int NW = kW4Waves>
hipError_t launch_gw(const W4Params& p, int gx, hipStream_t s) {
  hipLaunchKernelGGL((w4a16_kernel<GW, NW>), dim3(gx, p.S), dim3(64 * NW), 0, s, p);
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
  int gw = int((gps + kW4Waves - 1) / kW4Waves);
  if (gw == 5 || gw == 7) ++gw;  // slot rings of 3 or 4 need GW in {1, 2, 3, 4, 6, 8}
  pl.gw = gw;
  pl.nw = kW4Waves;
  // A split of 7 x 8 groups (K = 28672 in four splits): seven wavefronts of
  // eight groups each, rather than eight wavefronts of which the last would
  // hold no group of the split.
  if (gps == 7 * 8) {
    pl.gw = 8;
    pl.nw = 7;
  }
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
  if (pl.nw == 7) {
    if (pl.gw != 8) return hipErrorInvalidValue;
    e = launch_gw<8, 7>(p, gx, s);
  } else switch (pl.gw) {
    case 1: e = launch_gw<1>(p, gx, s); break;
    case 2: e = launch_gw<2>(p, gx, s); break;
    case 3: e = launch_gw<3>(p, gx, s); break;
    case 4: e = launch_gw<4>(p, gx, s); break;
    case 6: e = launch_gw<6>(p, gx, s); break;
    case 8: e = launch_gw<8>(p, gx, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || pl.S == 1) return e;
  const int64_t MN = int64_t(p.M) * p.N;
  hipLaunchKernelGGL(w4a16_reduce_kernel, dim3(unsigned((MN + 1023) / 1024)), dim3(256), 0, s, p.part, p.y, pl.S, MN);
  return hipGetLastError();
}

}  // namespace eta
