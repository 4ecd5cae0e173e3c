// YaRN rotary encoding of new tokens and their append into the paged KV cache (the page
// "GPT-OSS on Day 0", section "GPT-OSS on Hopper", names YaRN positional encoding for the
// model; the method is YaRN's published one: pair (i, i + 32) of a head vector turned by
// p * f_i, frequencies and temperature computed on the host).
//
// One workgroup per group of kTokens consecutive new tokens of one sequence. Per token,
// lanes 0..31 compute cos / sin of the 32 pair angles (the angle reduced modulo 2 pi in
// fp64, the trigonometry in fp32) into LDS; then every thread takes 4 pairs of one row:
// q rows are rotated into q_out, k rows rotated into the token's page slot, v rows copied
// there. Memory-bound: each byte is read once and written once.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace attn_sink {

namespace {
constexpr int kThreads = 256;
constexpr int kTokens = 8;  // new tokens per workgroup
}  // namespace

__global__ __launch_bounds__(kThreads) void rope_append_kernel(RopeParams p) {
  __shared__ float cs[2][32];
  const int b = blockIdx.y;
  const int q0 = clampi(p.cu_q[b], 0, p.total_q);
  const int q1 = clampi(p.cu_q[b + 1], q0, p.total_q);
  const int Lq = min(q1 - q0, p.max_q);
  const int L = clampi(p.kv_lens[b], 0, min(p.max_kv, p.max_pages << p.page_shift));
  const int t_begin = blockIdx.x * kTokens;
  const int t_end = min(t_begin + kTokens, Lq);
  const int rows = p.hq + 2 * p.hkv;

  for (int t = t_begin; t < t_end; ++t) {
    const int tok = q0 + t;
    const int pos = L - Lq + t;  // negative only for inconsistent metadata: then no cache write
    if (threadIdx.x < 32) {
      const double turn = 6.283185307179586;
      double a = (double)pos * p.freqs[threadIdx.x];
      a -= turn * floor(a / turn);
      float sn, cn;
      sincosf((float)a, &sn, &cn);
      cs[0][threadIdx.x] = cn * p.mscale;
      cs[1][threadIdx.x] = sn * p.mscale;
    }
    __syncthreads();
    uint16_t* kdst = nullptr;
    uint16_t* vdst = nullptr;
    if (pos >= 0) {
      const int slot = pos >> p.page_shift;
      const int page = clampi(p.page_table[(size_t)b * p.max_pages + slot], 0, p.num_pages - 1);
      const size_t base = ((size_t)page * p.hkv * p.page_size + (pos & (p.page_size - 1))) * kHeadDim;
      kdst = p.k_cache + base;
      vdst = p.v_cache + base;
    }
    for (int it = threadIdx.x; it < rows * 8; it += kThreads) {
      const int row = it >> 3;
      const int i0 = (it & 7) * 4;  // pairs i0 .. i0 + 3
      const uint16_t* src;
      uint16_t* dst;
      bool rot = true;
      if (row < p.hq) {
        src = p.q + ((size_t)tok * p.hq + row) * kHeadDim;
        dst = p.q_out + ((size_t)tok * p.hq + row) * kHeadDim;
      } else if (row < p.hq + p.hkv) {
        const int h = row - p.hq;
        src = p.k + ((size_t)tok * p.hkv + h) * kHeadDim;
        dst = kdst == nullptr ? nullptr : kdst + (size_t)h * p.page_size * kHeadDim;
      } else {
        const int h = row - p.hq - p.hkv;
        src = p.v + ((size_t)tok * p.hkv + h) * kHeadDim;
        dst = vdst == nullptr ? nullptr : vdst + (size_t)h * p.page_size * kHeadDim;
        rot = false;
      }
      if (dst == nullptr) continue;
      const u32x2 lo = *reinterpret_cast<const u32x2*>(src + i0);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(src + 32 + i0);
      if (!rot) {
        *reinterpret_cast<u32x2*>(dst + i0) = lo;
        *reinterpret_cast<u32x2*>(dst + 32 + i0) = hi;
        continue;
      }
      const float a[4] = {bf16_lo(lo[0]), bf16_hi(lo[0]), bf16_lo(lo[1]), bf16_hi(lo[1])};
      const float c[4] = {bf16_lo(hi[0]), bf16_hi(hi[0]), bf16_lo(hi[1]), bf16_hi(hi[1])};
      float ra[4], rc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float cn = cs[0][i0 + j], sn = cs[1][i0 + j];
        ra[j] = a[j] * cn - c[j] * sn;
        rc[j] = a[j] * sn + c[j] * cn;
      }
      *reinterpret_cast<u32x2*>(dst + i0) = u32x2{pack_bf16x2(ra[0], ra[1]), pack_bf16x2(ra[2], ra[3])};
      *reinterpret_cast<u32x2*>(dst + 32 + i0) = u32x2{pack_bf16x2(rc[0], rc[1]), pack_bf16x2(rc[2], rc[3])};
    }
    __syncthreads();  // cs is rewritten for the next token
  }
}

hipError_t launch_rope_append(const RopeParams& p, hipStream_t stream) {
  if (p.batch == 0 || p.total_q == 0 || p.max_q == 0) return hipSuccess;
  dim3 grid((unsigned)((p.max_q + kTokens - 1) / kTokens), (unsigned)p.batch), block(kThreads);
  hipLaunchKernelGGL(rope_append_kernel, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn_sink
