// C ABI of libattn.so: argument validation on the host, then kernel dispatch.
// Nothing here allocates device memory or synchronises the host; every check
// happens before the first HIP call, so a rejected call has no side effect.
// The one HIP object the library creates itself is attn_fwd_ring_host's copy
// stream (with its events), once per device.
#include "attn.h"
#include "attn_diag.h"
#include "mfma_probe.h"
#include "w4a16.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "common.h"

namespace {

using eta::FwdParams;

constexpr int64_t kMaxTokens = int64_t(1) << 30;  // keeps every in-kernel token index in int

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

attn_status check_shape(int B, int H, int Nq, int Nk, int d) {
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return ATTN_ERR_INVALID;
  if (Nq > kMaxTokens || Nk > kMaxTokens) return ATTN_ERR_INVALID;
  const int64_t BH = int64_t(B) * H;
  const int64_t nqb = (int64_t(Nq) + eta::kBM - 1) / eta::kBM;
  if (BH * nqb > INT32_MAX) return ATTN_ERR_INVALID;  // grid size
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

attn_status check_ptrs16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!p || !aligned(p, 16)) return ATTN_ERR_INVALID;
  return ATTN_OK;
}

attn_status check_ptrs4(std::initializer_list<const void*> ps, bool nullable) {
  for (const void* p : ps) {
    if (!p) {
      if (!nullable) return ATTN_ERR_INVALID;
      continue;
    }
    if (!aligned(p, 4)) return ATTN_ERR_INVALID;
  }
  return ATTN_OK;
}

int device_compute_units();

FwdParams base_params(int B, int H, int Nq, int Nk, float scale) {
  FwdParams p{};
  p.ncu = device_compute_units();
  p.Nq = Nq;
  p.Nk = Nk;
  p.BH = B * H;
  p.nqb = (Nq + eta::kBM - 1) / eta::kBM;
  p.diag = Nk - Nq;
  const double a = std::fabs(double(scale));
  p.scale_abs = float(a);
  if (scale == 0.f) {
    // Every score is 0: run as Q = 0 with a positive exponent factor, so masked
    // keys still get exp2(-inf) = 0.
    p.c = 1.f;
    p.q_and = 0u;
    p.q_xor = 0u;
  } else {
    p.c = float(a * 1.4426950408889634074);  // log2(e)
    p.q_and = 0xFFFFFFFFu;
    p.q_xor = scale < 0.f ? 0x80008000u : 0u;  // sign bit of each 16-bit element
  }
  return p;
}

attn_status from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// Partial (O, m, l) state of q against one K/V block at global positions
// (arguments already validated).
hipError_t launch_kvblock(const void* q, const void* k_blk, const void* v_blk, float* o_part, float* m_part,
                          float* l_part, int B, int H, int Nq, int Nk_blk, int d, bool causal, int64_t q_pos0,
                          int64_t k_pos0, float scale, hipStream_t stream) {
  FwdParams p = base_params(B, H, Nq, Nk_blk, scale);
  // Key j allowed for row i iff k_pos0 + j <= q_pos0 + i, i.e. j <= i + diag.
  // Clamping diag to [-Nq, Nk] keeps every allowed set unchanged.
  int64_t diag = q_pos0 - k_pos0;
  if (diag > Nk_blk) diag = Nk_blk;
  if (diag < -int64_t(Nq)) diag = -int64_t(Nq);
  p.diag = int(diag);
  p.q = q;
  p.k = k_blk;
  p.v = v_blk;
  p.o = o_part;
  p.m_out = m_part;
  p.l_out = l_part;
  return eta::launch_fwd_bf16(p, d, causal, eta::kEpiState, stream);
}

// Attention of q against one K/V block merged straight into the accumulator
// (o_acc, m_acc, l_acc) by the kernel's epilogue; with o_final / lse_final the
// merged result is also written as bf16 O and LSE (arguments already
// validated).  Same result as launch_kvblock followed by launch_merge_rows,
// without the block state's round trip through memory.
hipError_t launch_kvblock_merge(const void* q, const void* k_blk, const void* v_blk, float* o_acc, float* m_acc,
                                float* l_acc, void* o_final, float* lse_final, int B, int H, int Nq, int Nk_blk,
                                int d, bool causal, int64_t q_pos0, int64_t k_pos0, float scale,
                                hipStream_t stream) {
  FwdParams p = base_params(B, H, Nq, Nk_blk, scale);
  int64_t diag = q_pos0 - k_pos0;
  if (diag > Nk_blk) diag = Nk_blk;
  if (diag < -int64_t(Nq)) diag = -int64_t(Nq);
  p.diag = int(diag);
  p.q = q;
  p.k = k_blk;
  p.v = v_blk;
  p.o = o_acc;
  p.m_out = m_acc;
  p.l_out = l_acc;
  p.o_final = o_final;
  p.lse = lse_final;
  return eta::launch_fwd_bf16(p, d, causal, eta::kEpiMerge, stream);
}

// Merge (o_part, m_part, l_part) into the accumulator (arguments already
// validated).  Inside the library a null accumulator or part stands for the
// empty state.
hipError_t launch_merge_rows(float* o_acc, float* m_acc, float* l_acc, const float* o_part, const float* m_part,
                             const float* l_part, void* o_final, float* lse_final, int64_t rows, int d,
                             hipStream_t stream) {
  eta::MergeParams p{};
  p.o_acc = o_acc;
  p.m_acc = m_acc;
  p.l_acc = l_acc;
  p.o_part = o_part;
  p.m_part = m_part;
  p.l_part = l_part;
  p.o_final = o_final;
  p.lse_final = lse_final;
  p.rows = rows;
  p.d = d;
  return eta::launch_merge(p, stream);
}

bool merge_grid_ok(int64_t rows, int d) {
  const int vpr = d / 4;
  const int rpb = vpr >= 256 ? 1 : 256 / vpr;
  return (rows + rpb - 1) / rpb <= INT32_MAX;
}

// Compute units of the current device (queried once per device; 0 if unknown).
int device_compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cu = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev].store(cu, std::memory_order_relaxed);
  return cu;
}

attn_status check_w4a16(int64_t M, int64_t N, int64_t K, int64_t group) {
  if (M < 1 || N < 1 || K < 1 || group < 1) return ATTN_ERR_INVALID;
  if (group != W4A16_GROUP) return ATTN_ERR_UNSUPPORTED;
  if (K % group) return ATTN_ERR_INVALID;
  // Keeps every row index in int and a 16-row tile of W below 4 GiB (32-bit lane offsets).
  if (N > (int64_t(1) << 30) || K > (int64_t(1) << 24)) return ATTN_ERR_INVALID;
  if (M > W4A16_MAX_M) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// Arguments shared by attn_fwd_ring and attn_fwd_ring_host.
attn_status check_ring(const void* q, const void* const* k_blks, const void* const* v_blks, const int64_t* k_pos,
                       int n_blk, void* o, float* lse, float* work, int B, int H, int Nq, int Nk_blk, int d,
                       int causal, int64_t q_pos0, float scale) {
  if (n_blk < 0) return ATTN_ERR_INVALID;
  if (attn_status s = check_shape(B, H, Nq, Nk_blk, d)) return s;
  if (attn_status s = check_ptrs16({q, o, work})) return s;
  if (attn_status s = check_ptrs4({lse}, true)) return s;
  if (!std::isfinite(scale)) return ATTN_ERR_INVALID;
  if (n_blk > 0 && (!k_blks || !v_blks || !k_pos)) return ATTN_ERR_INVALID;
  if (causal && q_pos0 < 0) return ATTN_ERR_INVALID;
  for (int b = 0; b < n_blk; ++b)
    if (causal && k_pos[b] < 0) return ATTN_ERR_INVALID;
  if (!merge_grid_ok(int64_t(B) * H * Nq, d)) return ATTN_ERR_INVALID;
  return ATTN_OK;
}

// The hop loop of one GPU's ring share over the live blocks (with a causal
// mask, a block whose first key comes after the shard's last row holds no
// allowed key for any row and is skipped).  before(i, b) runs ahead of live
// block i's launches (it returns that block's device K and V), after(i) runs
// behind them; both return a HIP error or hipSuccess.
template <class Before, class After>
attn_status run_ring(const void* q, const int64_t* k_pos, int n_blk, void* o, float* lse, float* work, int B, int H,
                     int Nq, int Nk_blk, int d, int causal, int64_t q_pos0, float scale, hipStream_t s,
                     Before before, After after) {
  const int64_t rows = int64_t(B) * H * Nq;
  float* o_acc = work;
  float* m_acc = work + rows * d;
  float* l_acc = m_acc + rows;
  const int64_t last_row = q_pos0 + Nq - 1;
  auto live = [&](int b) { return !causal || k_pos[b] <= last_row; };
  int n_live = 0;
  for (int b = 0; b < n_blk; ++b) n_live += live(b) ? 1 : 0;
  if (n_live == 0)  // every row sees no key: O = 0, LSE = -inf
    return from_hip(launch_merge_rows(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, o, lse, rows, d, s));
  int i = 0;
  for (int b = 0; b < n_blk; ++b) {
    if (!live(b)) continue;
    const void* kb = nullptr;
    const void* vb = nullptr;
    if (hipError_t e = before(i, b, kb, vb)) return from_hip(e);
    if (i == 0) {  // the first live block's state becomes the accumulator
      if (hipError_t e = launch_kvblock(q, kb, vb, o_acc, m_acc, l_acc, B, H, Nq, Nk_blk, d, causal != 0, q_pos0,
                                        k_pos[b], scale, s))
        return from_hip(e);
    } else {  // later blocks merge into it in the attention kernel's epilogue
      const bool last = i == n_live - 1;
      if (hipError_t e = launch_kvblock_merge(q, kb, vb, o_acc, m_acc, l_acc, last ? o : nullptr,
                                              last ? lse : nullptr, B, H, Nq, Nk_blk, d, causal != 0, q_pos0,
                                              k_pos[b], scale, s))
        return from_hip(e);
    }
    if (hipError_t e = after(i)) return from_hip(e);
    ++i;
  }
  if (n_live == 1)  // finish the single block: merge it with the empty state
    return from_hip(launch_merge_rows(o_acc, m_acc, l_acc, nullptr, nullptr, nullptr, o, lse, rows, d, s));
  return ATTN_OK;
}

// Per-device copy stream and events of attn_fwd_ring_host, created on first
// use and kept until the process ends.  The mutex serialises whole calls, so
// the events' record/wait order is the order of the enqueued work.
struct RingCopier {
  std::mutex mu;
  bool ready = false;
  hipStream_t copy = nullptr;
  hipEvent_t start = nullptr;
  hipEvent_t copied[2] = {nullptr, nullptr};
  hipEvent_t freed[2] = {nullptr, nullptr};
};
constexpr int kMaxDevices = 64;
RingCopier g_copiers[kMaxDevices];

hipError_t copier_init(RingCopier& c) {
  if (c.ready) return hipSuccess;
  if (hipError_t e = hipStreamCreateWithFlags(&c.copy, hipStreamNonBlocking)) return e;
  hipEvent_t* evs[5] = {&c.start, &c.copied[0], &c.copied[1], &c.freed[0], &c.freed[1]};
  for (hipEvent_t* ev : evs)
    if (hipError_t e = hipEventCreateWithFlags(ev, hipEventDisableTiming)) return e;
  c.ready = true;
  return hipSuccess;
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char* attn_status_str(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID: return "ATTN_ERR_INVALID: invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED: unsupported configuration";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP: HIP runtime error at launch";
  }
  return "unknown attn_status";
}

attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                     int Nq, int Nk, int d, int causal, float scale, void* stream) {
  if (attn_status s = check_shape(B, H, Nq, Nk, d)) return s;
  if (attn_status s = check_ptrs16({q, k, v, o})) return s;
  if (attn_status s = check_ptrs4({lse}, true)) return s;
  if (!std::isfinite(scale)) return ATTN_ERR_INVALID;
  FwdParams p = base_params(B, H, Nq, Nk, scale);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  return from_hip(eta::launch_fwd_bf16(p, d, causal != 0, eta::kEpiFinalBf16, (hipStream_t)stream));
}

attn_status attn_fwd_block_order(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                 int Nq, int Nk, int d, int causal, float scale, uint32_t order, void* stream) {
  if (attn_status s = check_shape(B, H, Nq, Nk, d)) return s;
  if (attn_status s = check_ptrs16({q, k, v, o})) return s;
  if (attn_status s = check_ptrs4({lse}, true)) return s;
  if (!std::isfinite(scale)) return ATTN_ERR_INVALID;
  FwdParams p = base_params(B, H, Nq, Nk, scale);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  if (order != 0) {
    // grid size of the bf16 forward: one workgroup per (b, h, 256-row block)
    const uint64_t n = uint64_t(B) * H * ((uint64_t(Nq) + 255) / 256);
    uint64_t mul = (uint64_t(order) * 2654435761u) % n;
    if (mul == 0) mul = 1;
    auto gcd = [](uint64_t a, uint64_t b) { while (b) { const uint64_t t = a % b; a = b; b = t; } return a; };
    while (gcd(mul, n) != 1) mul = mul + 1 < n ? mul + 1 : 1;
    p.perm_mul = uint32_t(mul);
    p.perm_add = uint32_t((uint64_t(order) * 40503u) % n);
  }
  return from_hip(eta::launch_fwd_bf16(p, d, causal != 0, eta::kEpiFinalBf16, (hipStream_t)stream));
}

attn_status attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                         int H, int Nq, int Nk, int d, int causal, float scale, void* stream) {
  if (attn_status s = check_shape(B, H, Nq, Nk, d)) return s;
  if (attn_status s = check_ptrs16({q, k, v, o})) return s;
  if (attn_status s = check_ptrs4({lse}, true)) return s;
  if (!std::isfinite(scale)) return ATTN_ERR_INVALID;
  FwdParams p = base_params(B, H, Nq, Nk, scale);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  return from_hip(eta::launch_fwd_f32(p, d, causal != 0, (hipStream_t)stream));
}

attn_status attn_fwd_kvblock(const void* q, const void* k_blk, const void* v_blk, float* o_part,
                             float* m_part, float* l_part, int B, int H, int Nq, int Nk_blk, int d,
                             int causal, int64_t q_pos0, int64_t k_pos0, float scale, void* stream) {
  if (attn_status s = check_shape(B, H, Nq, Nk_blk, d)) return s;
  if (attn_status s = check_ptrs16({q, k_blk, v_blk, o_part})) return s;
  if (attn_status s = check_ptrs4({m_part, l_part}, false)) return s;
  if (!std::isfinite(scale)) return ATTN_ERR_INVALID;
  if (causal && (q_pos0 < 0 || k_pos0 < 0)) return ATTN_ERR_INVALID;
  return from_hip(launch_kvblock(q, k_blk, v_blk, o_part, m_part, l_part, B, H, Nq, Nk_blk, d, causal != 0,
                                 q_pos0, k_pos0, scale, (hipStream_t)stream));
}

attn_status attn_merge(float* o_acc, float* m_acc, float* l_acc, const float* o_part,
                       const float* m_part, const float* l_part, void* o_final, float* lse_final,
                       int B, int H, int Nq, int d, void* stream) {
  if (B <= 0 || H <= 0 || Nq <= 0 || d <= 0) return ATTN_ERR_INVALID;
  if (d % 4 != 0 || d > 1024) return ATTN_ERR_UNSUPPORTED;
  if (attn_status s = check_ptrs16({o_acc, o_part})) return s;
  if (attn_status s = check_ptrs4({m_acc, l_acc, m_part, l_part}, false)) return s;
  if (attn_status s = check_ptrs4({lse_final}, true)) return s;
  if (o_final && !aligned(o_final, 8)) return ATTN_ERR_INVALID;
  const int64_t rows = int64_t(B) * H * Nq;
  if (!merge_grid_ok(rows, d)) return ATTN_ERR_INVALID;
  if (o_acc == o_part || m_acc == m_part || l_acc == l_part) return ATTN_ERR_INVALID;
  return from_hip(launch_merge_rows(o_acc, m_acc, l_acc, o_part, m_part, l_part, o_final, lse_final, rows, d,
                                    (hipStream_t)stream));
}

size_t attn_ring_work_floats(int B, int H, int Nq, int d) {
  if (B <= 0 || H <= 0 || Nq <= 0 || d <= 0) return 0;
  const size_t rows = size_t(B) * size_t(H) * size_t(Nq);
  return rows * size_t(d) + 2 * rows;  // the accumulated O, m and l
}


attn_status attn_fwd_ring(const void* q, const void* const* k_blks, const void* const* v_blks,
                          const int64_t* k_pos, int n_blk, void* o, float* lse, float* work, int B, int H,
                          int Nq, int Nk_blk, int d, int causal, int64_t q_pos0, float scale, void* stream) {
  if (attn_status s = check_ring(q, k_blks, v_blks, k_pos, n_blk, o, lse, work, B, H, Nq, Nk_blk, d, causal,
                                 q_pos0, scale))
    return s;
  for (int b = 0; b < n_blk; ++b)
    if (attn_status s = check_ptrs16({k_blks[b], v_blks[b]})) return s;
  auto before = [&](int, int b, const void*& kb, const void*& vb) {
    kb = k_blks[b];
    vb = v_blks[b];
    return hipSuccess;
  };
  auto after = [](int) { return hipSuccess; };
  return run_ring(q, k_pos, n_blk, o, lse, work, B, H, Nq, Nk_blk, d, causal, q_pos0, scale, (hipStream_t)stream,
                  before, after);
}

size_t attn_ring_stage_bytes(int B, int H, int Nk_blk, int d) {
  if (B <= 0 || H <= 0 || Nk_blk <= 0 || d <= 0) return 0;
  return 4 * size_t(B) * size_t(H) * size_t(Nk_blk) * size_t(d) * 2;  // two slots of K and V, bf16
}

attn_status attn_fwd_ring_host(const void* q, const void* const* k_blks, const void* const* v_blks,
                               const int64_t* k_pos, int n_blk, void* o, float* lse, float* work, void* stage,
                               int B, int H, int Nq, int Nk_blk, int d, int causal, int64_t q_pos0, float scale,
                               void* stream) {
  if (attn_status s = check_ring(q, k_blks, v_blks, k_pos, n_blk, o, lse, work, B, H, Nq, Nk_blk, d, causal,
                                 q_pos0, scale))
    return s;
  for (int b = 0; b < n_blk; ++b)
    if (!k_blks[b] || !v_blks[b]) return ATTN_ERR_INVALID;
  if (attn_status s = check_ptrs16({stage})) return s;
  const size_t stage_bytes = attn_ring_stage_bytes(B, H, Nk_blk, d);
  const size_t work_bytes = attn_ring_work_floats(B, H, Nq, d) * sizeof(float);
  {
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(stage), w0 = reinterpret_cast<uintptr_t>(work);
    if (s0 < w0 + work_bytes && w0 < s0 + stage_bytes) return ATTN_ERR_INVALID;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  RingCopier& c = g_copiers[dev];
  std::lock_guard<std::mutex> lock(c.mu);
  if (copier_init(c) != hipSuccess) return ATTN_ERR_HIP;
  const hipStream_t s = (hipStream_t)stream;
  const size_t blk_bytes = stage_bytes / 4;
  char* slots = static_cast<char*>(stage);
  // The first copy waits for the caller's earlier work on `stream` (which may
  // still read the staging buffer).
  if (hipEventRecord(c.start, s) != hipSuccess || hipStreamWaitEvent(c.copy, c.start, 0) != hipSuccess)
    return ATTN_ERR_HIP;
  auto before = [&](int i, int b, const void*& kb, const void*& vb) -> hipError_t {
    const int slot = i & 1;
    char* kd = slots + size_t(slot) * 2 * blk_bytes;
    char* vd = kd + blk_bytes;
    // live block i - 2 read this slot: its attention must have finished
    if (i >= 2)
      if (hipError_t e = hipStreamWaitEvent(c.copy, c.freed[slot], 0)) return e;
    if (hipError_t e = hipMemcpyAsync(kd, k_blks[b], blk_bytes, hipMemcpyHostToDevice, c.copy)) return e;
    if (hipError_t e = hipMemcpyAsync(vd, v_blks[b], blk_bytes, hipMemcpyHostToDevice, c.copy)) return e;
    if (hipError_t e = hipEventRecord(c.copied[slot], c.copy)) return e;
    if (hipError_t e = hipStreamWaitEvent(s, c.copied[slot], 0)) return e;
    kb = kd;
    vb = vd;
    return hipSuccess;
  };
  auto after = [&](int i) { return hipEventRecord(c.freed[i & 1], s); };
  return run_ring(q, k_pos, n_blk, o, lse, work, B, H, Nq, Nk_blk, d, causal, q_pos0, scale, s, before, after);
}

size_t attn_bwd_work_floats(int B, int H, int Nq) {
  if (B <= 0 || H <= 0 || Nq <= 0) return 0;
  return size_t(B) * size_t(H) * size_t(Nq);
}

attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, float* work, int B, int H, int Nq, int Nk,
                     int d, int causal, float scale, void* stream) {
  if (attn_status s = check_shape(B, H, Nq, Nk, d)) return s;
  if (attn_status s = check_ptrs16({q, k, v, o, dout, dq, dk, dv})) return s;
  if (attn_status s = check_ptrs4({lse, work}, false)) return s;
  if (!std::isfinite(scale)) return ATTN_ERR_INVALID;
  eta::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.delta = work;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.Nq = Nq;
  p.Nk = Nk;
  p.BH = B * H;
  p.diag = Nk - Nq;
  p.scale = scale;
  p.c = float(double(scale) * 1.4426950408889634074);  // log2(e)
  return from_hip(eta::launch_bwd(p, d, causal != 0, (hipStream_t)stream));
}

static attn_status fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_scale,
                           const float* k_scale, const float* v_scale, float* o, float* lse, int B, int H,
                           int Nq, int Nk, int d, int causal, float scale, void* stream, int mode) {
  if (attn_status s = check_shape(B, H, Nq, Nk, d)) return s;
  if (attn_status s = check_ptrs16({q8, k8, v8, o})) return s;
  if (attn_status s = check_ptrs4({q_scale, k_scale, v_scale}, false)) return s;
  if (attn_status s = check_ptrs4({lse}, true)) return s;
  if (!std::isfinite(scale)) return ATTN_ERR_INVALID;
  FwdParams p = base_params(B, H, Nq, Nk, scale);
  p.q = q8;
  p.k = k8;
  p.v = v8;
  p.q_scale = q_scale;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.o = o;
  p.lse = lse;
  return from_hip(eta::launch_fwd_fp8(p, d, causal != 0, mode, (hipStream_t)stream));
}

attn_status attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_scale,
                         const float* k_scale, const float* v_scale, float* o, float* lse, int B, int H,
                         int Nq, int Nk, int d, int causal, float scale, void* stream) {
  return fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B, H, Nq, Nk, d, causal, scale, stream,
                 eta::kFp8QkFp8);
}

attn_status attn_fwd_fp8_qk16(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_scale,
                              const float* k_scale, const float* v_scale, float* o, float* lse, int B, int H,
                              int Nq, int Nk, int d, int causal, float scale, void* stream) {
  return fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B, H, Nq, Nk, d, causal, scale, stream,
                 eta::kFp8QkFp16);
}

attn_status attn_fwd_fp8_pv8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_scale,
                             const float* k_scale, const float* v_scale, float* o, float* lse, int B, int H,
                             int Nq, int Nk, int d, int causal, float scale, void* stream) {
  return fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B, H, Nq, Nk, d, causal, scale, stream,
                 eta::kFp8AllFp8);
}

attn_status attn_fwd_fp8_pv4(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_scale,
                             const float* k_scale, const float* v_scale, float* o, float* lse, int B, int H,
                             int Nq, int Nk, int d, int causal, float scale, int direct_p, void* stream) {
  if (direct_p != 0 && direct_p != 1) return ATTN_ERR_INVALID;
  return fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B, H, Nq, Nk, d, causal, scale, stream,
                 direct_p ? eta::kFp8PvFp4Direct : eta::kFp8PvFp4);
}

size_t w4a16_work_floats(int64_t M, int64_t N, int64_t K, int64_t group) {
  if (check_w4a16(M, N, K, group) != ATTN_OK) return 0;
  return eta::w4a16_plan(std::min<int64_t>(M, W4A16_TOKENS_PER_PASS), N, K).work_floats;
}

}  // extern "C"

namespace {

// The passes of one W4A16 call (arguments already validated; work holds
// pl.work_floats floats when pl.work_floats > 0).
attn_status run_w4a16(const void* x, const uint32_t* packed, const void* scales, const uint8_t* zeros, void* y,
                      float* work, const eta::W4Plan& pl, int64_t M, int64_t N, int64_t K, int64_t group,
                      void* stream) {
  const int cu = device_compute_units();
  // One pass per block of up to 16 tokens, in order on the caller's stream
  // (passes reuse the workspace one after another).
  for (int64_t m0 = 0; m0 < M; m0 += W4A16_TOKENS_PER_PASS) {
    eta::W4Params p{};
    p.x = static_cast<const uint16_t*>(x) + m0 * K;
    p.packed = packed;
    p.scales = static_cast<const uint16_t*>(scales);
    p.zeros = zeros;
    p.y = static_cast<uint16_t*>(y) + m0 * N;
    p.part = pl.work_floats ? work : nullptr;
    p.M = int(std::min<int64_t>(W4A16_TOKENS_PER_PASS, M - m0));
    p.N = int(N);
    p.K = int(K);
    p.NG = int(K / group);
    if (attn_status s = from_hip(eta::launch_w4a16(p, pl, cu > 0 ? cu : 256, (hipStream_t)stream))) return s;
  }
  return ATTN_OK;
}

attn_status check_w4a16_ptrs(const void* x, const uint32_t* packed, const void* scales, const uint8_t* zeros,
                             const void* y) {
  if (attn_status s = check_ptrs16({x, packed})) return s;
  if (!scales || !aligned(scales, 2) || !zeros || !y || !aligned(y, 2)) return ATTN_ERR_INVALID;
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status w4a16_gemm(const void* x, const uint32_t* packed, const void* scales, const uint8_t* zeros, void* y,
                       float* work, int64_t M, int64_t N, int64_t K, int64_t group, void* stream) {
  if (attn_status s = check_w4a16(M, N, K, group)) return s;
  if (attn_status s = check_w4a16_ptrs(x, packed, scales, zeros, y)) return s;
  const eta::W4Plan pl = eta::w4a16_plan(std::min<int64_t>(M, W4A16_TOKENS_PER_PASS), N, K);
  if (pl.work_floats && (!work || !aligned(work, 4))) return ATTN_ERR_INVALID;
  return run_w4a16(x, packed, scales, zeros, y, work, pl, M, N, K, group, stream);
}

attn_status w4a16_gemm_noalloc(const void* x, const uint32_t* packed, const void* scales, const uint8_t* zeros,
                               void* y, int64_t M, int64_t N, int64_t K, int64_t group, void* stream) {
  if (attn_status s = check_w4a16(M, N, K, group)) return s;
  if (attn_status s = check_w4a16_ptrs(x, packed, scales, zeros, y)) return s;
  const eta::W4Plan pl = eta::w4a16_plan(std::min<int64_t>(M, W4A16_TOKENS_PER_PASS), N, K);
  if (pl.work_floats > W4A16_NOALLOC_MAX_WORK_FLOATS) return ATTN_ERR_UNSUPPORTED;
  float* work = nullptr;
  if (pl.work_floats && eta::w4a16_scratch(&work) != hipSuccess) return ATTN_ERR_HIP;
  return run_w4a16(x, packed, scales, zeros, y, work, pl, M, N, K, group, stream);
}

double attn_mfma_peak_flop(int kind, int workgroups, int iters) {
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 24)) return 0.0;
  const double per = eta::mfma_flop_per_instruction(kind);
  return per * 4.0 * double(iters) * 8.0 * double(workgroups);
}

attn_status attn_mfma_peak(int kind, int workgroups, int iters, float* out, void* stream) {
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 24)) return ATTN_ERR_INVALID;
  if (attn_status s = check_ptrs4({out}, false)) return s;
  if (kind < ATTN_MFMA_BF16 || kind > ATTN_MFMA_F32) return ATTN_ERR_UNSUPPORTED;
  return from_hip(eta::launch_mfma_peak(kind, workgroups, iters, out, (hipStream_t)stream));
}

attn_status attn_mfma_dot(int kind, const void* a, const void* b, float* c, void* stream) {
  if (attn_status s = check_ptrs16({a, b})) return s;
  if (attn_status s = check_ptrs4({c}, false)) return s;
  if (kind < ATTN_MFMA_BF16 || kind > ATTN_MFMA_FP8) return ATTN_ERR_UNSUPPORTED;
  return from_hip(eta::launch_mfma_dot(kind, a, b, c, (hipStream_t)stream));
}

}  // extern "C"
