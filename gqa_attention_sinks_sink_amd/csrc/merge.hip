// Log-sum-exp merge of split-KV partials ("GPT-OSS on Day 0", section "Attention
// sinks": attention split into blocks along the sequence length; each block's partial
// is its normalised output and log-sum-exp, the sink counted in the first block only).
//
// 32 threads per (row, head): two groups of 16, 4 head-dim elements (16 B) per thread.
// Each group reads every other batch of 8 partials (group 0 partials 0-7, 16-23, ...,
// group 1 partials 8-15, 24-31, ...) with independent loads and folds them into a running
// (max, weight sum, sum) triple; the two triples are then folded through a lane exchange.
// A row of n partials costs ceil(n / 16) memory round trips. Partials at -inf weigh 0
// whatever their o holds; a row with no live partial yields out = 0, lse = -inf.
#include "common.hpp"
#include "kernels.hpp"

namespace attn_sink {

namespace {
constexpr int kThreads = 256;
constexpr int kPairsPerBlock = kThreads / 32;
constexpr int kBatch = 8;
}  // namespace

__global__ __launch_bounds__(kThreads) void merge_kernel(MergeParams p) {
  const long pair = (long)blockIdx.x * kPairsPerBlock + (threadIdx.x >> 5);
  if (pair >= (long)p.rows * p.hq) return;
  const int r = (int)(pair / p.hq);
  const int h = (int)(pair - (long)r * p.hq);
  const int d4 = (threadIdx.x & 15) * 4;
  const int grp = (threadIdx.x >> 4) & 1;  // the group: which batches of 8 this thread folds
  const int p0 = clampi(p.indptr[r], 0, p.num_partials);
  const int p1 = clampi(p.indptr[r + 1], p0, p.num_partials);

  float M = kNegInf, W = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int i0 = p0 + kBatch * grp; i0 < p1; i0 += 2 * kBatch) {
    float l[kBatch];
    f32x4 o[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = i0 + u;
      if (i < p1) {
        l[u] = p.lse_part[(size_t)i * p.hq + h] * kLog2e;
        o[u] = *reinterpret_cast<const f32x4*>(p.o_part + ((size_t)i * p.hq + h) * kHeadDim + d4);
        if (!(l[u] > kNegInf)) {  // an empty partial (or a NaN lse): weight 0, its o unused
          l[u] = kNegInf;
          o[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      } else {
        l[u] = kNegInf;
        o[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    float bm = kNegInf;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) bm = fmaxf(bm, l[u]);
    const float Mn = fmaxf(M, bm);
    if (Mn == kNegInf) continue;
    const float s = fast_exp2(M - Mn);  // 0 when M is still -inf
    W *= s;
    acc *= s;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float wu = fast_exp2(l[u] - Mn);
      W += wu;
      acc += o[u] * wu;
    }
    M = Mn;
  }
  // Fold in the other group's triple (lane ^ 16: the same head-dim elements); the group-0
  // threads write the row.
  {
    const float M2 = __shfl_xor(M, 16, 64), W2 = __shfl_xor(W, 16, 64);
    f32x4 a2;
#pragma unroll
    for (int e = 0; e < 4; ++e) a2[e] = __shfl_xor(acc[e], 16, 64);
    const float Mn = fmaxf(M, M2);
    if (Mn > kNegInf) {
      const float s1 = fast_exp2(M - Mn), s2 = fast_exp2(M2 - Mn);
      W = W * s1 + W2 * s2;
      acc = acc * s1 + a2 * s2;
      M = Mn;
    }
  }
  if (grp != 0) return;
  const float inv = (W > 0.f) ? 1.0f / W : 0.f;
  u32x2 pk;
  pk[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  pk[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<u32x2*>(p.out + ((size_t)r * p.hq + h) * kHeadDim + d4) = pk;
  if (p.lse != nullptr && d4 == 0) {
    p.lse[(size_t)r * p.hq + h] = (W > 0.f) ? (M + fast_log2(W)) * kLn2 : kNegInf;
  }
}

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  const long pairs = (long)p.rows * p.hq;
  if (pairs == 0) return hipSuccess;
  const long blocks = (pairs + kPairsPerBlock - 1) / kPairsPerBlock;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn_sink
