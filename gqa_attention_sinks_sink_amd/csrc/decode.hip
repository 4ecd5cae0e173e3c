// Split-KV paged decode / verify kernel for attention with per-head sink logits.
//
// Method ("GPT-OSS on Day 0", section "Attention sinks"): softmax over the scaled Q.K
// scores plus one sink logit per head; computed online with a running maximum m and a
// scale d; the running maximum of the first KV chunk is seeded with the head's sink
// (d = 1), later chunks start from m = -inf; chunk partials are merged by log-sum-exp
// (merge.hip).
//
// Work decomposition (one workgroup = one sequence x one KV head x one KV chunk):
//   * columns = the q_len query tokens x G query heads that share the KV head
//     (GQA: one K/V fetch serves all of them), padded to NT tiles of 16;
//   * 4 waves split the chunk's keys; each wave streams 32 keys (two 16-key groups)
//     per step straight from HBM into registers in the MFMA operand layout;
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (keys x columns), masks from indices,
//     online softmax in the exp2 domain, O^T += V^T P^T with V transposed on its way
//     out of LDS by ds_read_b64_tr_b16;
//   * the 4 wave states are combined in LDS and the chunk partial (o/d, m + ln d) is
//     written to the workspace at the plan's offset.
#include "common.hpp"
#include "kernels.hpp"

namespace attn_sink {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kVRowBytes = 160;               // padded LDS row of V (64 bf16 = 128 B + 32)
constexpr int kVWaveBytes = 32 * kVRowBytes;  // 32 keys per wave step

__device__ __forceinline__ int seq_len_clamped(const DecodeParams& p, int b) {
  int L = p.kv_lens[b];
  int cap = p.max_kv_len < p.max_pages * p.page_size ? p.max_kv_len : p.max_pages * p.page_size;
  return clampi(L, 0, cap);
}

__device__ __forceinline__ int chunks_for(int L, int chunk) {
  int n = (L + chunk - 1) / chunk;
  return n < 1 ? 1 : n;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Byte offset of the K/V row (page, kv head, slot) in the cache.
__device__ __forceinline__ size_t cache_row(const DecodeParams& p, int page, int kvh, int slot) {
  return (((size_t)page * p.hkv + kvh) * p.page_size + slot) * (size_t)kHeadDim;
}

}  // namespace

template <int NT>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kWaves * kVWaveBytes];
  __shared__ float red_m[kWaves][NT * 16];
  __shared__ float red_l[kWaves][NT * 16];

  const int max_chunks = gridDim.x / p.batch;
  const int b = blockIdx.x / max_chunks;
  const int c = blockIdx.x - b * max_chunks;
  const int kvh = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;

  const int L = seq_len_clamped(p, b);
  const int n_b = chunks_for(L, p.kv_chunk);
  if (c >= n_b) return;

  // ---- plan: partial offset of this sequence (exclusive prefix over earlier sequences)
  int acc = 0;
  for (int i = lane; i < b; i += 64) acc += chunks_for(seq_len_clamped(p, i), p.kv_chunk);
  const int base = wave_sum_int(acc) * p.q_len;  // indptr of row b*q_len
  if (c == 0 && kvh == 0 && w == 0) {
    if (lane < p.q_len) {
      p.counts[b * p.q_len + lane] = n_b;
      p.indptr[b * p.q_len + lane] = base + lane * n_b;
    }
    if (b == p.batch - 1 && lane == 0) p.indptr[p.batch * p.q_len] = base + p.q_len * n_b;
  }

  const int G = p.group;
  const int R = p.q_len * G;  // live columns
  const int col_lo = lane & 15;
  const int grp = lane >> 4;  // 16-lane group 0..3

  // ---- Q^T as the B operand (k = head dim), one 16-column tile per nt
  u32x4 qb[NT][2];
  int pos[NT];  // absolute position of each lane's column (for masks)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = nt * 16 + col_lo;
    const int t = col / G, gh = col - (col / G) * G;
    pos[nt] = L - p.q_len + t;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (col < R) {
        const size_t off = ((size_t)(b * p.q_len + t) * p.hq + kvh * G + gh) * kHeadDim + ks * 32 + grp * 8;
        qb[nt][ks] = *reinterpret_cast<const u32x4*>(p.q + off);
      } else {
        qb[nt][ks] = u32x4{0, 0, 0, 0};
      }
    }
  }

  // ---- online-softmax state per lane: m (exp2 domain, same across the 4 lane groups of a
  // column), a partial row sum, and O^T tiles (d = dt*16 + 4*grp + i, column nt*16 + col_lo).
  float m[NT], lsum[NT];
  f32x4 o[NT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = nt * 16 + col_lo;
    const int h = kvh * G + (col < R ? col % G : 0);
    // First chunk: the running max starts at the head's sink and d at 1 (held by lane group 0
    // so the column sum counts it once). Other chunks and waves: m = -inf (d = 1 is inert).
    const float sink2 = (p.sinks != nullptr) ? p.sinks[h] * kLog2e : kNegInf;
    m[nt] = (c == 0 && w == 0) ? sink2 : kNegInf;
    lsum[nt] = (grp == 0) ? 1.0f : 0.0f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[nt][dt] = f32x4{0, 0, 0, 0};
  }

  // ---- this wave's key range inside the chunk
  const int chunk_lo = c * p.kv_chunk;
  const int chunk_hi = min(chunk_lo + p.kv_chunk, L);
  const int per_wave = p.kv_chunk / kWaves;  // multiple of 16
  const int w_lo = chunk_lo + w * per_wave;
  const int w_hi = min(w_lo + per_wave, chunk_hi);
  unsigned char* vl = lds + w * kVWaveBytes;
  const int* ptab = p.page_table + (size_t)b * p.max_pages;

  // Address of 16-key group starting at key j (group lies inside one page: page_size % 16 == 0).
  auto group_row = [&](int j) -> size_t {
    int pg = ptab[j >> p.page_shift];
    pg = clampi(pg, 0, p.num_pages - 1);
    return cache_row(p, pg, kvh, j & (p.page_size - 1));
  };

  for (int j0 = w_lo; j0 < w_hi; j0 += 32) {
    const bool hasB = (j0 + 16) < w_hi;
    // K as the A operand: row = key (lane & 15), k = head dim slice.
    u32x4 ka[2][2], vrow[4];
    {
      const size_t rA = group_row(j0);
      const size_t rB = hasB ? group_row(j0 + 16) : rA;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        ka[0][ks] = *reinterpret_cast<const u32x4*>(p.k_cache + rA + (size_t)col_lo * kHeadDim + ks * 32 + grp * 8);
        ka[1][ks] = hasB ? *reinterpret_cast<const u32x4*>(p.k_cache + rB + (size_t)col_lo * kHeadDim + ks * 32 + grp * 8)
                         : u32x4{0, 0, 0, 0};
      }
      // V rows for LDS: lane covers key (lane>>3) + 8*ii of the 32, 16 B chunk (lane & 7).
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int kr = (lane >> 3) + 8 * ii;  // 0..31
        const int key = j0 + kr;
        const size_t rr = (kr < 16) ? rA : rB;
        if (key < w_hi) {
          vrow[ii] = *reinterpret_cast<const u32x4*>(p.v_cache + rr + (size_t)(kr & 15) * kHeadDim + (lane & 7) * 8);
        } else {
          vrow[ii] = u32x4{0, 0, 0, 0};  // keys past the range contribute exact zeros
        }
      }
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int kr = (lane >> 3) + 8 * ii;
      *reinterpret_cast<u32x4*>(vl + kr * kVRowBytes + (lane & 7) * 16) = vrow[ii];
    }

    // S^T tiles: 16 keys x 16 columns per (group, nt).
    f32x4 s[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        f32x4 a = f32x4{0, 0, 0, 0};
        a = mfma16(as_bf16x8(ka[g][0]), as_bf16x8(qb[nt][0]), a);
        a = mfma16(as_bf16x8(ka[g][1]), as_bf16x8(qb[nt][1]), a);
        s[nt][g] = a;
      }
    }

    // Masks + online softmax update per column tile.
    bf16x8 pb[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float mx = kNegInf;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = j0 + g * 16 + grp * 4 + i;
          bool ok = key < w_hi;
          if (p.causal) ok = ok && key <= pos[nt];
          if (p.window > 0) ok = ok && (pos[nt] - key) < p.window;
          const float v = ok ? s[nt][g][i] * p.scale_log2 : kNegInf;
          s[nt][g][i] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float m_new = fmaxf(m[nt], mx);
      const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
      const float alpha = fast_exp2(m[nt] - m_use);
      m[nt] = m_new;
      float ps = 0.f;
      uint32_t packed[4];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          e[i] = fast_exp2(s[nt][g][i] - m_use);
          ps += e[i];
        }
        packed[g * 2 + 0] = pack_bf16x2(e[0], e[1]);
        packed[g * 2 + 1] = pack_bf16x2(e[2], e[3]);
      }
      lsum[nt] = lsum[nt] * alpha + ps;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[nt][dt] *= alpha;
      pb[nt] = as_bf16x8(u32x4{packed[0], packed[1], packed[2], packed[3]});
    }

    // O^T += V^T P^T. A operand (V^T): lane = d (dt*16 + col_lo), k slots 0..3 = group A
    // keys 4*grp..+3, slots 4..7 = group B keys 4*grp..+3 (matches the P layout above).
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int rsel = grp * 4 + (col_lo >> 2);
      const int csel = dt * 16 + 4 * (col_lo & 3);
      const s16x4 lo = lds_read_tr16(vl + rsel * kVRowBytes + csel * 2);
      const s16x4 hi = lds_read_tr16(vl + (16 + rsel) * kVRowBytes + csel * 2);
      u32x4 av;
      av[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
      av[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
      av[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
      av[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[nt][dt] = mfma16(as_bf16x8(av), pb[nt], o[nt][dt]);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }

  // ---- combine the 4 wave states of this chunk
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float lt = lsum[nt];
    lt += shfl_xor(lt, 16);
    lt += shfl_xor(lt, 32);
    lsum[nt] = lt;
    if (grp == 0) {
      red_m[w][nt * 16 + col_lo] = m[nt];
      red_l[w][nt * 16 + col_lo] = lt;
    }
  }
  __syncthreads();  // also: every wave is done with its V staging area
  float* obuf = reinterpret_cast<float*>(lds);  // [NT*16 columns][64 d] fp32, reuses V staging
  float mtot[NT], ltot[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = nt * 16 + col_lo;
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, red_m[ww][col]);
    const float Mu = (M == kNegInf) ? 0.f : M;
    float Lt = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) Lt += red_l[ww][col] * fast_exp2(red_m[ww][col] - Mu);
    mtot[nt] = M;
    ltot[nt] = Lt;
  }
  // Waves add their rescaled O^T into the buffer one after another (fixed order, so the
  // result is bit-reproducible).
  float f[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float Mu = (mtot[nt] == kNegInf) ? 0.f : mtot[nt];
    f[nt] = (ltot[nt] > 0.f) ? fast_exp2(m[nt] - Mu) / ltot[nt] : 0.f;
  }
  for (int ww = 0; ww < kWaves; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int col = nt * 16 + col_lo;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          f32x4* dst = reinterpret_cast<f32x4*>(&obuf[col * kHeadDim + dt * 16 + grp * 4]);
          const f32x4 add = o[nt][dt] * f[nt];
          *dst = (ww == 0) ? add : (*dst + add);
        }
      }
    }
    __syncthreads();
  }

  // ---- write the partial: o_c (normalised), lse_c (natural log)
  for (int i = threadIdx.x; i < R * (kHeadDim / 4); i += kThreads) {
    const int col = i / (kHeadDim / 4);
    const int d4 = (i % (kHeadDim / 4)) * 4;
    const int t = col / G, gh = col % G;
    const int pidx = base + t * n_b + c;
    const int h = kvh * G + gh;
    f32x4 val = *reinterpret_cast<const f32x4*>(&obuf[col * kHeadDim + d4]);
    *reinterpret_cast<f32x4*>(p.o_part + ((size_t)pidx * p.hq + h) * kHeadDim + d4) = val;
  }
  if (w == 0 && lane < 16) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int col = nt * 16 + lane;
      if (col < R) {
        const int t = col / G, gh = col % G;
        const int pidx = base + t * n_b + c;
        const float M = mtot[nt], Lt = ltot[nt];
        const float lse = (M == kNegInf || !(Lt > 0.f)) ? kNegInf : (M + fast_log2(Lt)) * kLn2;
        p.lse_part[(size_t)pidx * p.hq + kvh * G + gh] = lse;
      }
    }
  }
}

hipError_t launch_decode_split(const DecodeParams& p, int max_chunks, hipStream_t stream) {
  const int R = p.q_len * p.group;
  const int nt = (R + 15) / 16;
  dim3 grid(max_chunks * p.batch, p.hkv), block(kThreads);
  switch (nt) {
    case 1: hipLaunchKernelGGL(decode_split_kernel<1>, grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL(decode_split_kernel<2>, grid, block, 0, stream, p); break;
    case 3: hipLaunchKernelGGL(decode_split_kernel<3>, grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL(decode_split_kernel<4>, grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace attn_sink
