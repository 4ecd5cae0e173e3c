// Log-sum-exp merge of split-KV partials ("GPT-OSS on Day 0", section "Attention
// sinks": attention split into blocks along the sequence length; each block's partial
// is its normalised output and log-sum-exp, the sink counted in the first block only).
//
// One wave per (row, head); lane = head-dim element. Partial weights are
// exp(lse_c - max lse); partials at -inf weigh 0.
#include "common.hpp"
#include "kernels.hpp"

namespace attn_sink {

__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int r = blockIdx.x;
  if (h >= p.hq) return;
  const int p0 = clampi(p.indptr[r], 0, p.num_partials);
  const int p1 = clampi(p.indptr[r + 1], p0, p.num_partials);

  float M = kNegInf;
  for (int i = p0; i < p1; ++i) M = fmaxf(M, p.lse_part[(size_t)i * p.hq + h]);
  float acc = 0.f, W = 0.f;
  if (M != kNegInf) {
    for (int i = p0; i < p1; ++i) {
      const float wgt = fast_exp2((p.lse_part[(size_t)i * p.hq + h] - M) * kLog2e);
      W += wgt;
      acc += wgt * p.o_part[((size_t)i * p.hq + h) * kHeadDim + lane];
    }
  }
  const float o = (W > 0.f) ? acc / W : 0.f;
  p.out[((size_t)r * p.hq + h) * kHeadDim + lane] = (uint16_t)f32_to_bf16_bits(o);
  if (p.lse != nullptr && lane == 0) {
    p.lse[(size_t)r * p.hq + h] = (W > 0.f) ? M + fast_log2(W) * kLn2 : kNegInf;
  }
}

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  if (p.rows == 0 || p.hq == 0) return hipSuccess;
  dim3 grid(p.rows, (p.hq + 3) / 4), block(256);
  hipLaunchKernelGGL(merge_kernel, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn_sink
