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
// Work decomposition: one workgroup = 4 waves; a wave owns RB blocks of 32 rows, a row
// being one (query token, query head) pair. GP query heads of one KV head group are
// packed into the row dimension so that one K/V tile in LDS serves all of them. Per
// 64-key tile every K or V fragment read from LDS feeds RB MFMAs (one per row block),
// which is what keeps LDS traffic below the MFMA time:
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K from LDS, Q^T held in registers);
//   masks computed from indices only on tiles that need them; online softmax in the
//   exp2 domain with one FMA and one exp per score; O^T += V^T P^T where P^T is the
//   score tile converted to bf16 and V^T comes out of LDS through ds_read_b64_tr_b16.
//
// Lazy running maximum: the max m of a row moves only when needed. The fast path computes
// p = exp2(s - m) for the tile and its sum without looking at the maximum; if some lane's
// sum exceeds 2^10 (or is not finite, which also covers m = -inf before any visible key),
// the wave redoes the tile with the exact maximum (S recomputed from the K tile still in
// LDS) and rescales O. Terms are at most 2^10 on the fast path, so nothing overflows, and
// every term of a row uses the row's current m: the softmax is unchanged.
#include "common.hpp"
#include "kernels.hpp"

namespace attn_sink {

namespace {
constexpr int kThreads = 256;
constexpr int kTileN = 64;          // keys per tile
constexpr int kStages = 3;          // K/V tiles in flight: the current one and two prefetched
constexpr int kTileBytes = kTileN * kHeadDim * 2;  // 8 KB of K (or V) per tile
constexpr int kStageBytes = 2 * kTileBytes;        // K then V
constexpr float kSumGuard = 1024.f; // fast-path bound on a lane's tile sum of exp2(s - m)
}  // namespace

template <int GP, int RB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(PrefillParams p) {
  constexpr int ROWS = 128 * RB;  // rows per workgroup
  constexpr int TOK = ROWS / GP;  // query tokens per workgroup
  // Ring of K/V tiles filled by buffer loads that write LDS directly. A tile row is one key
  // (128 B = 8 chunks of 16 B); chunk c of row r sits at chunk position c ^ f(r), with
  // f = (r >> 1) & 7 for K and ((r >> 1) & 1) * 4 for V. That makes both the 16 B K reads
  // (16 lanes, 16 rows, one chunk) and the 8 B transposing V reads (32 lanes, 4 rows,
  // 64 B each) hit 64 distinct banks.
  __shared__ __attribute__((aligned(1024))) unsigned char kv_lds[kStages][kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int half = lane >> 5;  // which 32-lane half
  const int r32 = lane & 31;

  // Work item -> (sequence, head group, unit). Items are numbered sequence-major, then head
  // group, then unit, and dealt to the 8 XCDs in contiguous ranges (workgroup L runs on XCD
  // L % 8), so the workgroups sharing one sequence's K/V share one L2.
  const int n_hg = p.hkv * (p.group / GP);
  const int per_xcd = gridDim.x / 8;
  const int item = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  const int unit = item % p.units;
  const int bh = item / p.units;
  if (bh >= p.batch * n_hg) return;
  const int b = bh / n_hg;
  const int hg = bh - b * n_hg;
  const int nhb = p.group / GP;
  const int kvh = hg / nhb;
  const int head0 = kvh * p.group + (hg - kvh * nhb) * GP;

  // Sequence bounds, clamped into the declared buffer sizes.
  const int q0 = clampi(p.cu_q[b], 0, p.total_q);
  const int q1 = clampi(p.cu_q[b + 1], q0, p.total_q);
  const int k0 = clampi(p.cu_kv[b], 0, p.total_kv);
  const int k1 = clampi(p.cu_kv[b + 1], k0, p.total_kv);
  const int Lq = min(q1 - q0, p.max_q);
  const int Lk = min(k1 - k0, p.max_kv);
  const int off = Lk - Lq;  // absolute position of query token t is off + t
  const float c = p.scale_log2;
  const int n_blk = (Lq + TOK - 1) / TOK;

  // A unit is one row block, or with causal pairing the blocks u and n_blk - 1 - u, whose
  // key ranges add up to about the same length for every unit.
  for (int pass = 0; pass < (p.pair_blocks ? 2 : 1); ++pass) {
  if (pass == 0 && unit >= (p.pair_blocks ? (n_blk + 1) / 2 : n_blk)) break;
  const int tile = (pass == 0) ? unit : n_blk - 1 - unit;
  if (pass == 1 && tile <= unit) break;
  const int ts = tile * TOK;
  const int te = min(ts + TOK, Lq);

  // This lane's rows: row block rb covers rows w*32*RB + rb*32 + [0, 32). Keys visible to a
  // row: [vl, vh).
  auto visible_keys = [&](int rb, int& vl, int& vh) {
    const int pos = off + ts + ((w * RB + rb) * 32 + r32) / GP;
    vh = p.causal ? min(Lk, pos + 1) : Lk;
    vl = (p.window > 0) ? max(0, pos - p.window + 1) : 0;
    if (vh < vl) vh = vl;
  };
  u32x4 qb[RB][4];  // Q^T as the B operand: column = row, k = head dim (16 per step)
  float m[RB], lsum[RB];
  f32x16 o[RB][2];
  int hi_min = 0x7fffffff, lo_max = -0x7fffffff, hi_max = -0x7fffffff, lo_min = 0x7fffffff;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = (w * RB + rb) * 32 + r32;
    const int t = ts + r / GP;
    const int head = head0 + (r % GP);
    const bool row_ok = t < te;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qb[rb][ks] = row_ok ? *reinterpret_cast<const u32x4*>(p.q + ((size_t)(q0 + t) * p.hq + head) * kHeadDim + ks * 16 + half * 8)
                          : u32x4{0, 0, 0, 0};
    }
    // Online softmax state; the sink seeds the running max, d starts at 1 (held by lane half 0).
    m[rb] = (p.sinks != nullptr) ? p.sinks[head] * kLog2e : kNegInf;
    lsum[rb] = (half == 0) ? 1.0f : 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) { o[rb][0][i] = 0.f; o[rb][1][i] = 0.f; }
    int vl, vh;
    visible_keys(rb, vl, vh);
    if (row_ok) {
      hi_min = min(hi_min, vh);
      lo_max = max(lo_max, vl);
      if (vh > vl) {
        hi_max = max(hi_max, vh);
        lo_min = min(lo_min, vl);
      }
    }
  }
  // Wave-wide bounds: a tile inside [lo_max, hi_min) needs no mask; a tile outside
  // [lo_min, hi_max) has no visible key for any row of the wave and is skipped.
#pragma unroll
  for (int o2 = 32; o2 >= 1; o2 >>= 1) {
    hi_min = min(hi_min, __shfl_xor(hi_min, o2, 64));
    lo_max = max(lo_max, __shfl_xor(lo_max, o2, 64));
    hi_max = max(hi_max, __shfl_xor(hi_max, o2, 64));
    lo_min = min(lo_min, __shfl_xor(lo_min, o2, 64));
  }
  // wave-uniform: keep them in scalar registers
  hi_min = __builtin_amdgcn_readfirstlane(hi_min);
  lo_max = __builtin_amdgcn_readfirstlane(lo_max);
  hi_max = __builtin_amdgcn_readfirstlane(hi_max);
  lo_min = __builtin_amdgcn_readfirstlane(lo_min);

  // Key range of the workgroup.
  const int p_lo = off + ts, p_hi = off + te - 1;
  int jb = (p.window > 0) ? max(0, p_lo - p.window + 1) : 0;
  jb &= ~(kTileN - 1);
  const int je = p.causal ? min(Lk, p_hi + 1) : Lk;

  // K/V tiles: buffer loads bounded by the sequence's last key return zeros past it (exact
  // zeros for keys that are masked anyway). Wave w fills rows [16w, 16w + 16) of a tile's K
  // and V with two 1 KB loads each; lane i writes chunk position i & 7 of row i >> 3.
  const uint32_t row_bytes = (uint32_t)p.hkv * (kHeadDim * 2);  // one token of K (or V), all heads
  const size_t seq_base = (size_t)k0 * p.hkv * kHeadDim;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + seq_base, (uint32_t)Lk * row_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + seq_base, (uint32_t)Lk * row_bytes);
  auto issue_tile = [&](int jt, int st) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int r = 16 * w + 8 * ii + (lane >> 3);
      const int pch = lane & 7;
      const uint32_t rowoff = (uint32_t)(jt + r) * row_bytes + (uint32_t)kvh * (kHeadDim * 2);
      unsigned char* dst = kv_lds[st] + (16 * w + 8 * ii) * 128;
      buffer_load16_lds(rk, dst, rowoff + (uint32_t)((pch ^ ((r >> 1) & 7)) * 16));
      buffer_load16_lds(rv, dst + kTileBytes, rowoff + (uint32_t)((pch ^ (((r >> 1) & 1) * 4)) * 16));
    }
  };

  // Up to two tiles in flight before the loop; every iteration issues at most one more.
  // (The first load is issued even for an empty range: it is retired after the loop.)
  issue_tile(jb, 0);
  if (jb + kTileN < je) issue_tile(jb + kTileN, 1);

  int st = 0;
  for (int jt = jb; jt < je; jt += kTileN) {
    // This wave's loads of the current tile are done once at most the 4 loads of the next
    // tile are outstanding; the barrier makes every wave's part visible and also means
    // every wave is done with the stage the new loads overwrite.
    if (jt + kTileN < je) {
      WAIT_VMCNT(4);
    } else {
      WAIT_VMCNT(0);
    }
    __builtin_amdgcn_s_barrier();
    if (jt + 2 * kTileN < je) issue_tile(jt + 2 * kTileN, st == 0 ? 2 : st - 1);
    const unsigned char* kt_lds = kv_lds[st];
    const unsigned char* vt_lds = kv_lds[st] + kTileBytes;
    st = (st == kStages - 1) ? 0 : st + 1;

    if (jt < hi_max && jt + kTileN > lo_min) {
      const bool need_mask = !(jt >= lo_max && jt + kTileN <= hi_min);
      f32x16 s[RB][2];  // S^T per row block and 32-key half
      // S^T for one 32-key half: k = 64 in 4 steps; each K fragment serves every row block.
      auto qk_half = [&](int kt) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i) s[rb][kt][i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int row = kt * 32 + r32;
          const u32x4 a = *reinterpret_cast<const u32x4*>(kt_lds + row * 128 + (((2 * ks + half) ^ ((row >> 1) & 7)) << 4));
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) s[rb][kt] = mfma32(as_bf16x8(a), as_bf16x8(qb[rb][ks]), s[rb][kt]);
        }
      };
      auto mask_half = [&](int kt) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          int vl, vh;
          visible_keys(rb, vl, vh);
          const unsigned span = (unsigned)(vh - vl);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int j = jt + kt * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
            s[rb][kt][i] = ((unsigned)(j - vl) < span) ? s[rb][kt][i] : kNegInf;
          }
        }
      };
      // P for one row block and 32-key half: p = exp2(c*s - m), packed to bf16 as the B
      // operands of the two PV steps of that half; returns the per-lane sum. S stays intact.
      u32x4 pk[RB][2][2];
      auto exp_half = [&](int kt, int rb, float nm) -> float {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float e0 = fast_exp2(__builtin_fmaf(s[rb][kt][i], c, nm));
          const float e1 = fast_exp2(__builtin_fmaf(s[rb][kt][i + 1], c, nm));
          a0 += e0;
          a1 += e1;
          pk[rb][kt][i >> 3][(i & 7) >> 1] = pack_bf16x2(e0, e1);
        }
        return a0 + a1;
      };
      // P and d for one half. The fast attempt uses the current m; if the guard trips for any
      // lane, m moves to the exact running maximum (from S, which is still intact), O and d
      // are rescaled, and P is redone; the second attempt always passes for finite scores.
      auto softmax_half = [&](int kt) {
        float ps[RB];
        for (int attempt = 0; attempt < 2; ++attempt) {
          bool ok = true;
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            ps[rb] = exp_half(kt, rb, (m[rb] == kNegInf && attempt > 0) ? 0.f : -m[rb]);
            ok = ok && (ps[rb] <= kSumGuard);  // false for inf / NaN
          }
          if (__builtin_expect(!__any(!ok), 1) || attempt > 0) break;
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            float mx = kNegInf;
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[rb][kt][i]);
            mx = fmaxf(mx, shfl_xor(mx, 32)) * c;
            const float m_new = fmaxf(m[rb], mx);
            const float alpha = (m_new == kNegInf) ? 1.0f : fast_exp2(m[rb] - m_new);
            m[rb] = m_new;
            lsum[rb] *= alpha;
#pragma unroll
            for (int i = 0; i < 16; ++i) { o[rb][0][i] *= alpha; o[rb][1][i] *= alpha; }
          }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) lsum[rb] += ps[rb];
      };
      // O^T += V^T P^T for the 16 keys of step kk; each V^T fragment serves every row block.
      auto pv_step = [&](int kk) {
        const int kt = kk >> 1;
        const int grp = lane >> 4;
        const int jl = lane & 15;
        const int krow = kk * 16 + 4 * (grp >> 1) + (jl >> 2);
        u32x4 av[2];
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const int c0 = dt * 32 + 16 * (grp & 1) + 4 * (jl & 3);
          // krow and krow + 8 have the same ((row >> 1) & 1), hence the same swizzle
          const int cb = (((c0 >> 3) ^ (((krow >> 1) & 1) * 4)) << 4) + ((c0 & 7) << 1);
          const s16x4 lo = lds_read_tr16(vt_lds + krow * 128 + cb);
          const s16x4 hi = lds_read_tr16(vt_lds + (krow + 8) * 128 + cb);
          av[dt] = join_tr16(lo, hi);
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) o[rb][dt] = mfma32(as_bf16x8(av[dt]), as_bf16x8(pk[rb][kt][kk & 1]), o[rb][dt]);
      };

      // Software pipeline inside the tile: the exps of one half run in the shadow of the
      // MFMAs of other work (S of the second half, then PV of the first half).
      qk_half(0);
      if (need_mask) mask_half(0);
      qk_half(1);
      softmax_half(0);
      if (need_mask) mask_half(1);
      pv_step(0);
      pv_step(1);
      softmax_half(1);
      pv_step(2);
      pv_step(3);
    }

  }
  // Retire the loads past the last tile and let every wave finish with the ring before it
  // is reused.
  WAIT_VMCNT(0);
  __syncthreads();

  // Epilogue: out = O / d, lse = m + log2(d) converted to natural log.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float lt = lsum[rb] + shfl_xor(lsum[rb], 32);
    const float inv = (lt > 0.f) ? 1.0f / lt : 0.f;
    const int r = (w * RB + rb) * 32 + r32;
    const int t = ts + r / GP;
    const int head = head0 + (r % GP);
    if (t < te) {
      uint16_t* orow = p.out + ((size_t)(q0 + t) * p.hq + head) * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = dt * 32 + 8 * q4 + 4 * half;
          u32x2 pk;
          pk[0] = pack_bf16x2(o[rb][dt][q4 * 4 + 0] * inv, o[rb][dt][q4 * 4 + 1] * inv);
          pk[1] = pack_bf16x2(o[rb][dt][q4 * 4 + 2] * inv, o[rb][dt][q4 * 4 + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + d0) = pk;
        }
      }
      if (p.lse != nullptr && half == 0) {
        p.lse[(size_t)(q0 + t) * p.hq + head] =
            (m[rb] == kNegInf || !(lt > 0.f)) ? kNegInf : (m[rb] + fast_log2(lt)) * kLn2;
      }
    }
  }
  }  // pass
}

namespace {
template <int RB>
hipError_t launch_rb(PrefillParams p, int gp, hipStream_t stream) {
  const int tok = 128 * RB / gp;
  const int n_blk = (p.max_q + tok - 1) / tok;
  p.pair_blocks = (p.causal && p.window == 0) ? 1 : 0;
  p.units = p.pair_blocks ? (n_blk + 1) / 2 : n_blk;
  const long items = (long)p.units * p.batch * p.hkv * (p.group / gp);
  dim3 grid((unsigned)(8 * ((items + 7) / 8))), block(kThreads);
  switch (gp) {
    case 1: hipLaunchKernelGGL((prefill_kernel<1, RB>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<2, RB>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<4, RB>), grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<8, RB>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((prefill_kernel<16, RB>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}
}  // namespace

int prefill_heads_per_tile(int group) {
  int gp = 1;
  while (gp < 16 && group % (gp * 2) == 0) gp *= 2;
  return gp;
}

int prefill_row_blocks(int max_q, int gp) {
  // 64 rows per wave halve the LDS traffic per MFMA; short sequences keep 32-row waves so
  // that a workgroup's rows are not mostly padding.
  return (max_q / gp >= 1024 / gp || max_q >= 512) ? 2 : 1;
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  if (p.batch == 0 || p.total_q == 0 || p.max_q == 0) return hipSuccess;
  const int gp = prefill_heads_per_tile(p.group);
  return prefill_row_blocks(p.max_q, gp) == 2 ? launch_rb<2>(p, gp, stream) : launch_rb<1>(p, gp, stream);
}

}  // namespace attn_sink
