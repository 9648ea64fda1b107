// Online-softmax merge of two (O, m, l) states, the accumulation step of ring
// attention ("Sequence parallelism and ring attention", "Deep dive" and
// "Technical insight": the earlier partial result is rescaled when a larger
// running maximum appears, which keeps the block-wise result equal to full
// attention).  Element-wise and bound by HBM bandwidth: each thread owns 4
// consecutive columns of one row (16-byte loads/stores); whole rows stay inside
// one workgroup so that the row scalars m, l can be read by every thread of
// the row before one thread overwrites them.
#include "common.h"

namespace eta {

__global__ void __launch_bounds__(256) merge_kernel(MergeParams p, int vpr, int rows_per_block) {
  const int local_row = threadIdx.x / vpr;
  const int cv = threadIdx.x % vpr;
  const int64_t row = (int64_t)blockIdx.x * rows_per_block + local_row;
  const bool live = local_row < rows_per_block && row < p.rows;

  float M = -INFINITY, l = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  // A null accumulator or part stands for the empty state (m = -inf, l = 0),
  // the identity of the merge: the library's ring driver uses it to finish a
  // single block (null part) or an all-masked shard (both null).
  const bool has_acc = p.o_acc != nullptr, has_part = p.o_part != nullptr;
  if (live) {
    const float ma = has_acc ? p.m_acc[row] : -INFINITY, mb = has_part ? p.m_part[row] : -INFINITY;
    const float la = has_acc ? p.l_acc[row] : 0.f, lb = has_part ? p.l_part[row] : 0.f;
    M = fmaxf(ma, mb);
    float wa = 0.f, wb = 0.f;
    if (M != -INFINITY) {
      if (ma != -INFINITY) wa = la * expf(ma - M);
      if (mb != -INFINITY) wb = lb * expf(mb - M);
    }
    l = wa + wb;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t off = row * p.d + 4 * cv;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const f32x4 oa = wa > 0.f ? *(const f32x4*)(p.o_acc + off) : zero;
    const f32x4 ob = wb > 0.f ? *(const f32x4*)(p.o_part + off) : zero;
    o = (wa * oa + wb * ob) * inv;
  }
  __syncthreads();  // every read of m_acc / l_acc of this block's rows is done
  if (!live) return;
  const int64_t off = row * p.d + 4 * cv;
  if (has_acc) *(f32x4*)(p.o_acc + off) = o;
  if (p.o_final) *(bf16x4*)((uint16_t*)p.o_final + off) = __builtin_convertvector(o, bf16x4);
  if (cv == 0) {
    if (has_acc) {
      p.m_acc[row] = l > 0.f ? M : -INFINITY;
      p.l_acc[row] = l;
    }
    if (p.lse_final) p.lse_final[row] = l > 0.f ? M + logf(l) : -INFINITY;
  }
}

hipError_t launch_merge(const MergeParams& p, hipStream_t s) {
  const int vpr = p.d / 4;                       // 1 .. 256
  const int rows_per_block = vpr >= 256 ? 1 : 256 / vpr;
  const int threads = rows_per_block * vpr;
  const int64_t blocks = (p.rows + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(threads), 0, s, p, vpr, rows_per_block);
  return hipGetLastError();
}

}  // namespace eta
