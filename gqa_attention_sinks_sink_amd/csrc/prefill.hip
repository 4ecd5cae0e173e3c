// Varlen self-attention with per-head sink logits: causal / sliding-window prefill and
// bidirectional embedding batches, no KV cache.
//
// Method ("GPT-OSS on Day 0", section "Attention sinks"): softmax over the scaled Q.K
// scores plus the head's sink logit, computed online; the running maximum starts at
// the sink and the running scale at 1. A prefill workgroup owns the whole KV range of
// its rows, so it is the "first chunk" and always carries the sink. Ragged batches are
// addressed through cu_seqlens without padding ("Fast Embeddings on GPUs", section on
// ragged attention).
//
// Work decomposition: one workgroup = 128 rows = (128 / GP) consecutive query tokens x
// GP query heads of one KV head group (GQA heads packed into the row dimension so that
// one K/V tile in LDS serves all of them); 4 waves x 32 rows. Per 64-key tile:
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K from LDS, Q^T held in registers);
//   masks computed from indices only on tiles that need them; online softmax in the
//   exp2 domain with one FMA per score; O^T += V^T P^T where P^T is the score tile
//   converted to bf16 in place and V^T comes out of LDS through ds_read_b64_tr_b16.
#include "common.hpp"
#include "kernels.hpp"

namespace attn_sink {

namespace {
constexpr int kThreads = 256;
constexpr int kTileN = 64;        // keys per tile
constexpr int kKRowBytes = 144;   // K tile row stride (128 B + 16): conflict-free 16 B reads
constexpr int kVRowBytes = 192;   // V tile row stride (128 B + 64): conflict-free transposing reads
constexpr float kLazyMax = 8.0f;  // running-max slack (log2 units) before a rescale
}  // namespace

template <int GP>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillParams p) {
  constexpr int TOK = 128 / GP;
  // Double-buffered K/V tiles: the next tile is written while the current one is read.
  __shared__ __attribute__((aligned(16))) unsigned char k_lds[2][kTileN * kKRowBytes];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds[2][kTileN * kVRowBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int half = lane >> 5;   // which 32-lane half
  const int r32 = lane & 31;

  const int n_tiles = gridDim.x / p.batch;
  const int b = blockIdx.x / n_tiles;
  const int tile = n_tiles - 1 - (blockIdx.x - b * n_tiles);  // longest causal rows first
  const int nhb = p.group / GP;
  const int kvh = blockIdx.y / nhb;
  const int head0 = kvh * p.group + (blockIdx.y - kvh * nhb) * GP;

  // Sequence bounds, clamped into the declared buffer sizes.
  const int q0 = clampi(p.cu_q[b], 0, p.total_q);
  const int q1 = clampi(p.cu_q[b + 1], q0, p.total_q);
  const int k0 = clampi(p.cu_kv[b], 0, p.total_kv);
  const int k1 = clampi(p.cu_kv[b + 1], k0, p.total_kv);
  const int Lq = min(q1 - q0, p.max_q);
  const int Lk = min(k1 - k0, p.max_kv);
  const int ts = tile * TOK;
  if (ts >= Lq) return;
  const int te = min(ts + TOK, Lq);
  const int off = Lk - Lq;  // absolute position of query token t is off + t

  // This lane's row.
  const int r = w * 32 + r32;
  const int t = ts + r / GP;
  const int head = head0 + (r % GP);
  const bool row_ok = t < Lq;
  const int pos = off + t;

  // Q^T as the B operand: column = row, k = head dim (16 per step, 8 per lane half).
  u32x4 qb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    qb[ks] = row_ok ? *reinterpret_cast<const u32x4*>(p.q + ((size_t)(q0 + t) * p.hq + head) * kHeadDim + ks * 16 + half * 8)
                    : u32x4{0, 0, 0, 0};
  }

  // Online softmax state; the sink seeds the running max, d starts at 1 (held by lane half 0).
  float m = (p.sinks != nullptr) ? p.sinks[head] * kLog2e : kNegInf;
  float lsum = (half == 0) ? 1.0f : 0.0f;
  f32x16 o[2];
#pragma unroll
  for (int i = 0; i < 16; ++i) { o[0][i] = 0.f; o[1][i] = 0.f; }

  // Key range of the workgroup; keys visible to this lane's row: [vis_lo, vis_hi).
  const int p_lo = off + ts, p_hi = off + te - 1;
  int jb = (p.window > 0) ? max(0, p_lo - p.window + 1) : 0;
  jb &= ~(kTileN - 1);
  const int je = p.causal ? min(Lk, p_hi + 1) : Lk;
  int vis_hi = p.causal ? min(Lk, pos + 1) : Lk;
  const int vis_lo = (p.window > 0) ? max(0, pos - p.window + 1) : 0;
  if (vis_hi < vis_lo) vis_hi = vis_lo;
  const unsigned vis_span = (unsigned)(vis_hi - vis_lo);
  // Wave-wide bounds over the wave's valid rows: a tile inside [lo_max, hi_min) needs no mask.
  int hi_min = row_ok ? vis_hi : 0x7fffffff, lo_max = row_ok ? vis_lo : -0x7fffffff;
#pragma unroll
  for (int o2 = 32; o2 >= 1; o2 >>= 1) {
    hi_min = min(hi_min, __shfl_xor(hi_min, o2, 64));
    lo_max = max(lo_max, __shfl_xor(lo_max, o2, 64));
  }

  // K/V staging: thread covers rows (tid >> 3) and (tid >> 3) + 32, 16 B chunk (tid & 7).
  auto load_tile = [&](int jt, u32x4 (&kr)[2], u32x4 (&vr)[2]) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int j = jt + (tid >> 3) + 32 * ii;
      if (j < Lk) {
        const size_t g = ((size_t)(k0 + j) * p.hkv + kvh) * kHeadDim + (tid & 7) * 8;
        kr[ii] = *reinterpret_cast<const u32x4*>(p.k + g);
        vr[ii] = *reinterpret_cast<const u32x4*>(p.v + g);
      } else {
        kr[ii] = u32x4{0, 0, 0, 0};  // keys past the sequence: exact zeros
        vr[ii] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf, const u32x4 (&kr)[2], const u32x4 (&vr)[2]) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int row = (tid >> 3) + 32 * ii;
      *reinterpret_cast<u32x4*>(k_lds[buf] + row * kKRowBytes + (tid & 7) * 16) = kr[ii];
      *reinterpret_cast<u32x4*>(v_lds[buf] + row * kVRowBytes + (tid & 7) * 16) = vr[ii];
    }
  };

  if (jb < je) {
    u32x4 kr[2], vr[2];
    load_tile(jb, kr, vr);
    store_tile(0, kr, vr);
  }
  __syncthreads();

  int buf = 0;
  for (int jt = jb; jt < je; jt += kTileN, buf ^= 1) {
    // Next tile's K/V go to registers now and to the other LDS buffer after this tile's math.
    const bool has_next = jt + kTileN < je;
    u32x4 kn[2], vn[2];
    if (has_next) load_tile(jt + kTileN, kn, vn);
    const unsigned char* kt_lds = k_lds[buf];
    const unsigned char* vt_lds = v_lds[buf];

    // S^T: 2 x (32 keys x 32 rows), k = 64 in 4 steps.
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kt_lds + (kt * 32 + r32) * kKRowBytes + (ks * 16 + half * 8) * 2);
        s[kt] = mfma32(as_bf16x8(a), as_bf16x8(qb[ks]), s[kt]);
      }
    }

    // Masks only on tiles that straddle a row's visible range.
    if (!(jt >= lo_max && jt + kTileN <= hi_min)) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = jt + kt * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
          s[kt][i] = ((unsigned)(j - vis_lo) < vis_span) ? s[kt][i] : kNegInf;
        }
      }
    }

    // Lazy running max (log2 units): it moves only when a score exceeds it by more than
    // kLazyMax, so most tiles need neither the cross-lane max nor a rescale of O. Every term
    // of a row uses the row's current m, so the softmax is unchanged.
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
    }
    mx *= p.scale_log2;
    if (__any(mx > m + kLazyMax)) {
      const float m_new = fmaxf(m, fmaxf(mx, shfl_xor(mx, 32)));
      const float alpha = (m_new == kNegInf) ? 1.0f : fast_exp2(m - m_new);
      m = m_new;
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < 16; ++i) { o[0][i] *= alpha; o[1][i] *= alpha; }
    }
    const float neg_m = (m == kNegInf) ? 0.f : -m;

    float ps = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(__builtin_fmaf(s[kt][i], p.scale_log2, neg_m));
        s[kt][i] = e;
        ps += e;
      }
    }
    lsum += ps;

    // O^T += V^T P^T over 4 steps of 16 keys.
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int kt = kk >> 1, ib = (kk & 1) * 8;
      u32x4 pw;
      pw[0] = pack_bf16x2(s[kt][ib + 0], s[kt][ib + 1]);
      pw[1] = pack_bf16x2(s[kt][ib + 2], s[kt][ib + 3]);
      pw[2] = pack_bf16x2(s[kt][ib + 4], s[kt][ib + 5]);
      pw[3] = pack_bf16x2(s[kt][ib + 6], s[kt][ib + 7]);
      const int grp = lane >> 4;
      const int jl = lane & 15;
      const int krow = kk * 16 + 4 * (grp >> 1) + (jl >> 2);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const int c0 = dt * 32 + 16 * (grp & 1) + 4 * (jl & 3);
        const s16x4 lo = lds_read_tr16(vt_lds + krow * kVRowBytes + c0 * 2);
        const s16x4 hi = lds_read_tr16(vt_lds + (krow + 8) * kVRowBytes + c0 * 2);
        const u32x4 av = join_tr16(lo, hi);
        o[dt] = mfma32(as_bf16x8(av), as_bf16x8(pw), o[dt]);
      }
    }

    if (has_next) store_tile(buf ^ 1, kn, vn);
    __syncthreads();
  }

  // Epilogue: out = O / d, lse = m + log2(d) converted to natural log.
  const float lt = lsum + shfl_xor(lsum, 32);
  const float inv = (lt > 0.f) ? 1.0f / lt : 0.f;
  if (row_ok) {
    uint16_t* orow = p.out + ((size_t)(q0 + t) * p.hq + head) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = dt * 32 + 8 * q4 + 4 * half;
        u32x2 pk;
        pk[0] = pack_bf16x2(o[dt][q4 * 4 + 0] * inv, o[dt][q4 * 4 + 1] * inv);
        pk[1] = pack_bf16x2(o[dt][q4 * 4 + 2] * inv, o[dt][q4 * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d0) = pk;
      }
    }
    if (p.lse != nullptr && half == 0) {
      p.lse[(size_t)(q0 + t) * p.hq + head] = (m == kNegInf || !(lt > 0.f)) ? kNegInf : (m + fast_log2(lt)) * kLn2;
    }
  }
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  if (p.batch == 0 || p.total_q == 0 || p.max_q == 0) return hipSuccess;
  int gp = 1;
  while (gp < 16 && p.group % (gp * 2) == 0) gp *= 2;
  const int tok = 128 / gp;
  const int n_tiles = (p.max_q + tok - 1) / tok;
  dim3 grid(n_tiles * p.batch, p.hkv * (p.group / gp)), block(kThreads);
  switch (gp) {
    case 1: hipLaunchKernelGGL(prefill_kernel<1>, grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL(prefill_kernel<2>, grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL(prefill_kernel<4>, grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL(prefill_kernel<8>, grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL(prefill_kernel<16>, grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace attn_sink
