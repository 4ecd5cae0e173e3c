// YaRN rotary encoding of new tokens and their append into the paged KV cache (the page
// "GPT-OSS on Day 0", section "GPT-OSS on Hopper", names YaRN positional encoding for the
// model; the method is YaRN's published one: pair (i, i + 32) of a head vector turned by
// p * f_i, frequencies and temperature computed on the host).
//
// One workgroup per kTokens consecutive new tokens of one sequence. First every thread
// computes one (token, pair) angle (reduced modulo 2 pi in fp64, trigonometry in fp32) into
// LDS; then the (token, row, 8-pair chunk) items are dealt evenly over the threads (two
// 16-byte loads each): q rows are rotated into q_out, k rows rotated into the token's page
// slot, v rows copied there.
// Memory-bound: each byte is read once and written once.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace attn_sink {

namespace {
constexpr int kThreads = 256;
constexpr int kTokens = 8;  // new tokens per workgroup
}  // namespace

__global__ __launch_bounds__(kThreads) void rope_append_kernel(RopeParams p) {
  static_assert(kThreads == kTokens * 32, "one thread per (token, pair) angle");
  __shared__ float cs[kTokens][2][32];
  const int b = blockIdx.y;
  const int q0 = clampi(p.cu_q[b], 0, p.total_q);
  const int q1 = clampi(p.cu_q[b + 1], q0, p.total_q);
  const int Lq = min(q1 - q0, p.max_q);
  const int L = clampi(p.kv_lens[b], 0, min(p.max_kv, p.max_pages << p.page_shift));
  const int t_begin = blockIdx.x * kTokens;
  const int n_tok = min(kTokens, Lq - t_begin);
  if (n_tok <= 0) return;
  {
    const int j = threadIdx.x >> 5, i = threadIdx.x & 31;
    const double turn = 6.283185307179586;
    double a = (double)(L - Lq + t_begin + j) * p.freqs[i];
    a -= turn * floor(a / turn);
    float sn, cn;
    sincosf((float)a, &sn, &cn);
    cs[j][0][i] = cn * p.mscale;
    cs[j][1][i] = sn * p.mscale;
  }
  __syncthreads();
  const int rows = p.hq + 2 * p.hkv;
  // Items (token, row, chunk of 8 pairs) dealt evenly over the threads.
  const int items = n_tok * rows * 4;
  for (int it = threadIdx.x; it < items; it += kThreads) {
    const int i0 = 8 * (it & 3);
    const int row = (it >> 2) % rows;
    const int j = (it >> 2) / rows;
    const int t = t_begin + j;
    const int tok = q0 + t;
    const int pos = L - Lq + t;  // negative only for inconsistent metadata: then no cache write
    const bool is_q = row < p.hq;
    const bool is_k = !is_q && row < p.hq + p.hkv;
    const int h = is_q ? row : (is_k ? row - p.hq : row - p.hq - p.hkv);
    const uint16_t* src = (is_q ? p.q : (is_k ? p.k : p.v)) + ((size_t)tok * (is_q ? p.hq : p.hkv) + h) * kHeadDim;
    uint16_t* dst;
    if (is_q) {
      dst = p.q_out + ((size_t)tok * p.hq + h) * kHeadDim;
    } else {
      if (pos < 0) continue;
      const int page = clampi(p.page_table[(size_t)b * p.max_pages + (pos >> p.page_shift)], 0, p.num_pages - 1);
      dst = (is_k ? p.k_cache : p.v_cache) +
            (((size_t)page * p.hkv + h) * p.page_size + (pos & (p.page_size - 1))) * kHeadDim;
    }
    const u32x4 lo = *reinterpret_cast<const u32x4*>(src + i0);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(src + 32 + i0);
    if (!is_q && !is_k) {
      *reinterpret_cast<u32x4*>(dst + i0) = lo;
      *reinterpret_cast<u32x4*>(dst + 32 + i0) = hi;
      continue;
    }
    u32x4 ra, rcv;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a0 = bf16_lo(lo[w]), a1 = bf16_hi(lo[w]);
      const float c0 = bf16_lo(hi[w]), c1 = bf16_hi(hi[w]);
      const float cn0 = cs[j][0][i0 + 2 * w], sn0 = cs[j][1][i0 + 2 * w];
      const float cn1 = cs[j][0][i0 + 2 * w + 1], sn1 = cs[j][1][i0 + 2 * w + 1];
      ra[w] = pack_bf16x2(a0 * cn0 - c0 * sn0, a1 * cn1 - c1 * sn1);
      rcv[w] = pack_bf16x2(a0 * sn0 + c0 * cn0, a1 * sn1 + c1 * cn1);
    }
    *reinterpret_cast<u32x4*>(dst + i0) = ra;
    *reinterpret_cast<u32x4*>(dst + 32 + i0) = rcv;
  }
}

hipError_t launch_rope_append(const RopeParams& p, hipStream_t stream) {
  if (p.batch == 0 || p.total_q == 0 || p.max_q == 0) return hipSuccess;
  dim3 grid((unsigned)((p.max_q + kTokens - 1) / kTokens), (unsigned)p.batch), block(kThreads);
  hipLaunchKernelGGL(rope_append_kernel, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn_sink
