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
// Work decomposition: a wave owns blocks of 32 rows, a row being one (query token, query
// head) pair. GP query heads of one KV head group are packed into the row dimension so that
// one K/V tile in LDS serves all of them. Every K or V fragment read from LDS feeds one MFMA
// per row block of the wave, which is what keeps LDS traffic below the MFMA time:
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K and the wave's Q rows from LDS);
//   masks computed from indices only on tiles that need them; online softmax in the
//   exp2 domain with one FMA and one exp per score; O^T += V^T P^T where P^T is the
//   score tile converted to bf16 and V^T comes out of LDS through ds_read_b64_tr_b16.
//
// Lazy running maximum: the max m of a row moves only when needed. The fast path computes
// p = exp2(s - m) for a tile and its sum without looking at the maximum; if some lane's
// sum exceeds 2^32 (or is not finite, which also covers m = -inf before any visible key),
// the wave redoes the tile with the exact maximum (S is still in registers) and rescales O.
// bf16 P and fp32 O / d keep their relative precision at any magnitude, so the bound only
// has to rule out overflow: terms stay below 2^32, and every term of a row uses the row's
// current m, so the softmax is unchanged.
//
// Two kernels share these steps: a 4-wave kernel for short items (windows, short sequences;
// 32-key tiles, three or four workgroups per CU) and an 8-wave "ping-pong" kernel for long
// sequences (64-key tiles, one workgroup per CU; described above prefill_pp_kernel).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace attn_sink {

namespace {
constexpr int kThreads = 256;
constexpr int kTileN = 64;          // keys per tile
constexpr int kTileBytes = kTileN * kHeadDim * 2;  // 8 KB of K (or V) per tile
constexpr int kStageBytes = 2 * kTileBytes;        // K then V
constexpr float kSumGuard = 4294967296.f;  // fast-path bound (2^32) on a lane's sum of exp2(s - m)
// The 4-wave kernel streams K/V in 32-key tiles through a ring of two.
constexpr int kShortTileN = 32;
constexpr int kShortTileBytes = kShortTileN * kHeadDim * 2;  // 4 KB of K (or V) per tile
constexpr int kShortStageBytes = 2 * kShortTileBytes;        // K then V
}  // namespace

template <int GP, int RB, bool PAGED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(RB == 2 ? 3 : 5, RB == 2 ? 3 : 5)))
void prefill_kernel(PrefillParams p) {
  constexpr int ROWS = 128 * RB;  // rows per workgroup
  constexpr int TOK = ROWS / GP;  // query tokens per workgroup
  constexpr int TN = kShortTileN;
  // Ring of two 32-key K/V tiles filled by buffer loads that write LDS directly. A tile row is
  // one key (128 B = 8 chunks of 16 B); chunk c of row r sits at chunk position c ^ f(r), with
  // f = (r >> 1) & 7 for K and ((r >> 1) & 1) * 4 for V. That makes both the 16 B K reads
  // (16 lanes, 16 rows, one chunk) and the 8 B transposing V reads (32 lanes, 4 rows, 64 B
  // each) hit 64 distinct banks.
  __shared__ __attribute__((aligned(1024))) unsigned char kv_lds[2][kShortStageBytes];
  // Per-wave slice of 32 RB rows x 128 bytes: the wave's Q rows during a pass (16-byte chunk c
  // of row i at chunk position c ^ ((i >> 1) & 7), as for K), its output rows at the end. Q is
  // read from here for every tile rather than held in registers: with 16 KB of ring and the
  // slices, three workgroups of 64-row waves (or five of 32-row waves) fit in one CU, and
  // their waves hide each other's load latency.
  __shared__ __attribute__((aligned(1024))) unsigned char q_lds[kThreads / 64][32 * RB * kHeadDim * 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  int k0 = 0, Lk;
  if constexpr (PAGED) {
    Lk = min(clampi(p.kv_lens[b], 0, p.max_kv), p.max_pages << p.page_shift);
  } else {
    k0 = clampi(p.cu_kv[b], 0, p.total_kv);
    const int k1 = clampi(p.cu_kv[b + 1], k0, p.total_kv);
    Lk = min(k1 - k0, p.max_kv);
  }
  const int Lq = min(q1 - q0, p.max_q);
  const int off = Lk - Lq;  // absolute position of query token t is off + t
  const float c = p.scale_log2;
  const int n_blk = (Lq + TOK - 1) / TOK;

  const uint32_t row_bytes = (uint32_t)p.hkv * (kHeadDim * 2);  // one token of K (or V), all heads
  const size_t seq_base = (size_t)k0 * p.hkv * kHeadDim;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc_uniform(p.k + seq_base, (uint32_t)Lk * row_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc_uniform(p.v + seq_base, (uint32_t)Lk * row_bytes);
  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc_uniform(p.q + (size_t)q0 * p.hq * kHeadDim, (uint32_t)Lq * p.hq * (kHeadDim * 2));

  // A lane's head is head0 + lane % GP in every row block and pass (GP divides 32). The GP
  // sink logits come in through scalar loads, once per workgroup.
  float sink_l2 = kNegInf;
  if (p.sinks != nullptr) {
    float sv[GP];
#pragma unroll
    for (int i = 0; i < GP; ++i) sv[i] = p.sinks[head0 + i];
    sink_l2 = sv[0];
#pragma unroll
    for (int i = 1; i < GP; ++i) sink_l2 = ((lane & (GP - 1)) == i) ? sv[i] : sink_l2;
    sink_l2 *= kLog2e;
  }
  unsigned char* const qw = q_lds[w];

  // A unit is one row block, or with causal pairing the blocks u and n_blk - 1 - u, whose
  // key ranges add up to about the same length for every unit.
  for (int pass = 0; pass < (p.pair_blocks ? 2 : 1); ++pass) {
  if (pass == 0 && unit >= (p.pair_blocks ? (n_blk + 1) / 2 : n_blk)) break;
  const int tile = (pass == 0) ? unit : n_blk - 1 - unit;
  if (pass == 1 && tile <= unit) break;
  const int ts = tile * TOK;
  const int te = min(ts + TOK, Lq);

  // Keys visible to query token t: [vis_lo(t), vis_hi(t)), both non-decreasing in t.
  auto vis_lo = [&](int t) { return (p.window > 0) ? max(0, off + t - p.window + 1) : 0; };
  auto vis_hi = [&](int t) { return max(p.causal ? min(Lk, off + t + 1) : Lk, vis_lo(t)); };
  // This lane's rows: row block rb covers rows w*32*RB + rb*32 + [0, 32), query token
  // ts + row / GP. The wave's tokens run from t_first to t_last; a tile inside
  // [lo_max, hi_min) needs no mask, a tile outside [lo_min, hi_max) has no visible key for any
  // row of the wave and is skipped. (Scalar: the bounds follow from the first and last token.)
  const int t_first = ts + (w * RB * 32) / GP;
  const int t_last = min(te - 1, ts + ((w + 1) * RB * 32 - 1) / GP);
  int hi_min = 0x7fffffff, lo_max = -0x7fffffff, hi_max = -0x7fffffff, lo_min = 0x7fffffff;
  if (t_first < te) {
    hi_min = vis_hi(t_first);
    lo_min = vis_lo(t_first);
    hi_max = vis_hi(t_last);
    lo_max = vis_lo(t_last);
  }

  // Q rows of the pass into the slice by DMA, issued before the first K/V tile (so they have
  // landed once it has). Rows past the end load the last valid row (their results are never
  // stored). Addresses come from a fresh lane id (the compiler would otherwise compute them
  // before the key loop and keep them in spill slots).
  // Row i = 8 k + x of the slice (x = lane / 8) is wave row w RB 32 + i: query token
  // t_w + (8 k + x) / GP, head head0 + (8 k + x) % GP. GP divides 32, so for GP <= 8 the token
  // steps by 8 / GP per k and the head stays; for GP = 16 the token steps every second k and
  // the head alternates between x and 8 + x.
  const int t_w = ts + (w * RB * 32) / GP;
  auto row_token = [](int k) { return GP <= 8 ? k * (8 / GP) : (k >> 1); };
  auto row_head = [](int k) { return GP <= 8 ? 0 : 8 * (k & 1); };
  {
    WAIT_LGKMCNT0();  // this wave's reads of the slice (previous pass's output) are done
    const int ln = opaque_lane_id();
    const int x = ln >> 3;
    const uint32_t S = (uint32_t)p.hq * (kHeadDim * 2);  // bytes per token of Q
    const uint32_t t_lane = (uint32_t)(t_w + (GP <= 8 ? x / GP : 0)) * S;
    const uint32_t h_lane = (uint32_t)(head0 + (GP <= 8 ? x % GP : x)) * (kHeadDim * 2);
    const uint32_t t_cap = (uint32_t)(te - 1) * S;
#pragma unroll
    for (int k = 0; k < 4 * RB; ++k) {
      const int i = 8 * k + x;
      const uint32_t voff = min(t_lane + (uint32_t)row_token(k) * S, t_cap) + h_lane +
                            (uint32_t)(row_head(k) * (kHeadDim * 2)) + (uint32_t)(((ln & 7) ^ ((i >> 1) & 7)) << 4);
      buffer_load16_lds_async(rq, qw + k * 1024, voff);
    }
  }
  float m[RB], lsum[RB];
  f32x16 o[RB][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    // Online softmax state; the sink seeds the running max, d starts at 1 (held by lane half 0).
    m[rb] = sink_l2;
    lsum[rb] = (half == 0) ? 1.0f : 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) { o[rb][0][i] = 0.f; o[rb][1][i] = 0.f; }
  }

  // Key range of the workgroup, in 32-key tiles.
  const int p_lo = off + ts, p_hi = off + te - 1;
  int jb = (p.window > 0) ? max(0, p_lo - p.window + 1) : 0;
  jb &= ~(TN - 1);
  const int je = p.causal ? min(Lk, p_hi + 1) : Lk;
  const int nt = (je > jb) ? (je - jb + TN - 1) / TN : 0;

  // K/V tiles: buffer loads bounded by the sequence's last key return zeros past it (exact
  // zeros for keys that are masked anyway). Wave w fills rows [8w, 8w + 8) of a tile's K and V
  // with one 1 KB load each; lane i writes chunk position i & 7 of row i >> 3. The loads are
  // hidden from the compiler (its own tracking would wait for all of them before any LDS read);
  // the waits below retire them explicitly.
  // Per-lane parts of a tile's load offsets, kept for the whole pass: lane i writes chunk
  // position i & 7 of row 8 w + (i >> 3), which holds global chunk (i & 7) ^ f(row).
  uint32_t k_lane, v_lane;
  {
    const int ln = opaque_lane_id();
    const int r = 8 * w + (ln >> 3);  // row inside the tile
    const uint32_t row = PAGED ? (uint32_t)(ln >> 3) * (kHeadDim * 2) : (uint32_t)r * row_bytes + (uint32_t)kvh * (kHeadDim * 2);
    k_lane = row + (uint32_t)(((ln & 7) ^ ((r >> 1) & 7)) << 4);
    v_lane = row + (uint32_t)(((ln & 7) ^ (((r >> 1) & 1) * 4)) << 4);
  }
  auto issue_tile = [&](int jt, int st) {
    unsigned char* dst = kv_lds[st] + 8 * w * 128;
    if constexpr (PAGED) {
      // Rows [8w, 8w + 8) of the tile are 8 consecutive keys inside one page (pages hold a
      // power of two >= 16 keys); the buffer range stops at the sequence's last key, so rows
      // past it read as zeros.
      const int kr = jt + 8 * w;
      const int slot = min(kr >> p.page_shift, p.max_pages - 1);
      const int pid = clampi(load_invariant(p.page_table, (size_t)b * p.max_pages + slot), 0, p.num_pages - 1);
      const uint32_t valid = (uint32_t)clampi(Lk - kr, 0, 8);
      const size_t blk = (((size_t)pid * p.hkv + kvh) * p.page_size + (kr & (p.page_size - 1))) * kHeadDim;
      buffer_load16_lds_async(make_rsrc_uniform(p.k + blk, valid * (kHeadDim * 2)), dst, k_lane);
      buffer_load16_lds_async(make_rsrc_uniform(p.v + blk, valid * (kHeadDim * 2)), dst + kShortTileBytes, v_lane);
      return;
    }
    buffer_load16_lds_async(rk, dst, k_lane + (uint32_t)jt * row_bytes);
    buffer_load16_lds_async(rv, dst + kShortTileBytes, v_lane + (uint32_t)jt * row_bytes);
  };

  // Per-lane LDS offsets. K and Q: row r32 of a 32-row block, 16-byte chunk (2 ks + half) ^ f(row)
  // (f depends only on the row inside the block). V: the transposing reads of 16-key step kk start
  // at row 16 kk + 4 (grp >> 1) + (jl >> 2) and row + 8; their swizzle does not depend on kk.
  auto k_off = [&](int ks) -> uint32_t { return r32 * 128 + (((2 * ks + half) ^ ((r32 >> 1) & 7)) << 4); };
  auto v_off = [&](int dt) -> uint32_t {
    const int grp = lane >> 4, jl = lane & 15;
    const int krow = 4 * (grp >> 1) + (jl >> 2);
    const int c0 = dt * 32 + 16 * (grp & 1) + 4 * (jl & 3);
    return krow * 128 + ((((c0 >> 3) ^ (((krow >> 1) & 1) * 4)) << 4) + ((c0 & 7) << 1));
  };

  if (nt > 0) issue_tile(jb, 0);
  for (int j = 0; j < nt; ++j) {
    const int jt = jb + j * TN;
    // This wave's loads of tile j (and of Q, issued earlier) are done; the barrier makes every
    // wave's part visible and means every wave is done with tile j - 1, whose stage the next
    // tile's loads overwrite.
    WAIT_VMCNT(0);
    lds_barrier();
    if (j + 1 < nt) issue_tile(jt + TN, (j + 1) & 1);
    const unsigned char* kt_lds = kv_lds[j & 1];
    const unsigned char* vt_lds = kv_lds[j & 1] + kShortTileBytes;
    if (!(jt < hi_max && jt + TN > lo_min)) continue;

    // Issue priority: the waves of a SIMD (three workgroups' worth) are raised while they issue
    // MFMAs, so the matrix unit is fed first and the softmax of the others fills the VALU.
    __builtin_amdgcn_s_setprio(3);
    // S^T = K Q^T for the 32 keys of the tile: k = 64 in 4 steps; each K fragment serves every
    // row block.
    f32x16 s[RB];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(kt_lds + k_off(ks));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const u32x4 qf = *reinterpret_cast<const u32x4*>(qw + rb * 4096 + k_off(ks));
        s[rb] = mfma32(as_bf16x8(a), as_bf16x8(qf), ks == 0 ? f32x16{} : s[rb]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // Masks from indices, unless every row of the wave sees the whole tile.
    if (!(jt >= lo_max && jt + TN <= hi_min)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int t = ts + ((w * RB + rb) * 32 + r32) / GP;
        const int vl = vis_lo(t), vh = vis_hi(t);
        const unsigned span = (unsigned)(vh - vl);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int jk = jt + 8 * (i >> 2) + 4 * half + (i & 3);
          s[rb][i] = ((unsigned)(jk - vl) < span) ? s[rb][i] : kNegInf;
        }
      }
    }
    // P = exp2(c*s - m), packed to bf16 as the B operands of the two PV steps; the per-lane
    // sums. The fast attempt uses the current m; if the guard trips for any lane, m moves to
    // the exact running maximum (from S, which is still intact), O and d are rescaled, and P is
    // redone; the second attempt always passes for finite scores.
    u32x4 pk[RB][2];
    float ps[RB];
    for (int attempt = 0; attempt < 2; ++attempt) {
      bool ok = true;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float nm = (m[rb] == kNegInf && attempt > 0) ? 0.f : -m[rb];
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float e0 = fast_exp2(__builtin_fmaf(s[rb][i], c, nm));
          const float e1 = fast_exp2(__builtin_fmaf(s[rb][i + 1], c, nm));
          a0 += e0;
          a1 += e1;
          pk[rb][i >> 3][(i & 7) >> 1] = pack_bf16x2(e0, e1);
        }
        ps[rb] = a0 + a1;
        ok = ok && (ps[rb] <= kSumGuard);  // false for inf / NaN
      }
      if (__builtin_expect(!__any(!ok), 1) || attempt > 0) break;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float mx = kNegInf;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[rb][i]);
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
    __builtin_amdgcn_s_setprio(3);
    // O^T += V^T P^T in two 16-key steps; each V^T fragment serves every row block.
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 av[2];
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        // rows krow and krow + 8 have the same ((row >> 1) & 1), hence the same swizzle
        const unsigned char* vp = vt_lds + kk * 2048 + v_off(dt);
        av[dt] = join_tr16(lds_read_tr16(vp), lds_read_tr16(vp + 1024));
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) o[rb][dt] = mfma32(as_bf16x8(av[dt]), as_bf16x8(pk[rb][kk]), o[rb][dt]);
    }
  }
  __builtin_amdgcn_s_setprio(0);
  // No key is visible (nt = 0): Q is not needed, but its DMA must land before the slice is
  // reused for the output. Every wave is done with the ring before the next pass reuses it.
  WAIT_VMCNT(0);
  __syncthreads();

  // Epilogue: out = O / d, lse = m + log2(d) converted to natural log. O goes through this
  // wave's LDS slice: the accumulator layout gives a lane 8-byte pieces of one row, the
  // stores then write whole 128-byte rows (8 lanes per row). 16-byte chunk c of row i sits
  // at chunk position c ^ (i & 7).
  {
    // (Addresses from a fresh lane id: the compiler would otherwise compute them before the
    // key loop and keep them in spill slots.)
    const int ln = opaque_lane_id();
    const int hf = ln >> 5;
    unsigned char* ow = qw;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float lt = lsum[rb] + shfl_xor(lsum[rb], 32);
      const float inv = (lt > 0.f) ? 1.0f / lt : 0.f;
      const int i = rb * 32 + (ln & 31);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          u32x2 pkd;
          pkd[0] = pack_bf16x2(o[rb][dt][q4 * 4 + 0] * inv, o[rb][dt][q4 * 4 + 1] * inv);
          pkd[1] = pack_bf16x2(o[rb][dt][q4 * 4 + 2] * inv, o[rb][dt][q4 * 4 + 3] * inv);
          const int cc = dt * 4 + q4;
          *reinterpret_cast<u32x2*>(ow + i * 128 + ((cc ^ (i & 7)) << 4) + hf * 8) = pkd;
        }
      }
      const int r = (w * RB + rb) * 32 + (ln & 31);
      const int t = ts + r / GP;
      if (p.lse != nullptr && hf == 0 && t < te) {
        p.lse[(size_t)(q0 + t) * p.hq + head0 + (r % GP)] =
            (m[rb] == kNegInf || !(lt > 0.f)) ? kNegInf : (m[rb] + fast_log2(lt)) * kLn2;
      }
    }
    const int cc = ln & 7;
    const int x = ln >> 3;
    const int t_lane = t_w + (GP <= 8 ? x / GP : 0);
    uint16_t* const ob = p.out + ((size_t)(q0 + t_lane) * p.hq + head0 + (GP <= 8 ? x % GP : x)) * kHeadDim + cc * 8;
#pragma unroll
    for (int k = 0; k < 4 * RB; ++k) {
      const int i = 8 * k + x;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ow + i * 128 + ((cc ^ (i & 7)) << 4));
      if (t_lane + row_token(k) < te)
        *reinterpret_cast<u32x4*>(ob + ((size_t)row_token(k) * p.hq + row_head(k)) * kHeadDim) = v;
    }
  }
  }  // pass
}

// Ping-pong variant for long sequences (no window): 8 waves per workgroup, each owning 64 rows
// (two 32-row blocks). Waves w and w + 4 run on the same SIMD; group A (waves 0-3) and group B
// (waves 4-7) walk the same sequence of phases one phase apart, separated by workgroup
// barriers, so in every slot one wave of each SIMD is in a matrix phase and the other in a
// softmax phase:
//   matrix phase t:  O^T += V_{t-1}^T P_{t-1}^T, then S_t^T = K_t Q^T   (MFMA, LDS reads)
//   softmax phase t: P_t = exp2(c S_t - m) with the lazy-max guard       (VALU only)
// The softmax of one wave then runs while the other wave's MFMAs occupy the matrix unit,
// instead of both waves alternating between the two kinds of work on their own.
// K/V tiles (64 keys) go through a 4-stage LDS ring: tile t is read in slots 2t .. 2t + 3 and
// is loaded (buffer loads straight into LDS) during slots 2t - 4 .. 2t - 1.
template <int GP, bool PAGED>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_pp_kernel(PrefillParams p) {
  constexpr int RB = 2;
  constexpr int NW = 8;
  constexpr int ROWS = 64 * NW;
  constexpr int TOK = ROWS / GP;
  constexpr int kRing = 4;
  __shared__ __attribute__((aligned(1024))) unsigned char kv_lds[kRing][kStageBytes];
  // Per-wave slice (64 rows x 128 bytes): the wave's Q rows during a pass, then its output rows.
  __shared__ __attribute__((aligned(16))) unsigned char q_lds[NW][64 * kHeadDim * 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lag = w >> 2;  // group B runs one phase behind group A
  const int half = lane >> 5;
  const int r32 = lane & 31;

  // Work item -> (sequence, head group, unit). Workgroup L runs on XCD L % 8. When the
  // (sequence, head group) pairs come in multiples of 8, they are dealt to the XCDs round-robin,
  // all units of a pair to the same XCD: the workgroups sharing one head's K/V share one L2, and
  // every XCD gets an equal share of pairs from every sequence, so sequences of unequal length
  // (chunks on different context lengths) do not load the XCDs unequally. Otherwise (few pairs)
  // the items, numbered pair-major, are dealt in contiguous ranges, which splits a pair's units
  // over several XCDs rather than leaving XCDs idle.
  const int n_hg = p.hkv * (p.group / GP);
  int unit, bh;
  if (p.xcd_round_robin) {
    const int j_xcd = blockIdx.x / 8;
    unit = j_xcd % p.units;
    bh = (int)(blockIdx.x % 8) + 8 * (j_xcd / p.units);
  } else {
    const int item = (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
    unit = item % p.units;
    bh = item / p.units;
  }
  if (bh >= p.batch * n_hg) return;
  const int b = bh / n_hg;
  const int hg = bh - b * n_hg;
  const int nhb = p.group / GP;
  const int kvh = hg / nhb;
  const int head0 = kvh * p.group + (hg - kvh * nhb) * GP;

  const int q0 = clampi(p.cu_q[b], 0, p.total_q);
  const int q1 = clampi(p.cu_q[b + 1], q0, p.total_q);
  int k0 = 0, Lk;
  if constexpr (PAGED) {
    Lk = min(clampi(p.kv_lens[b], 0, p.max_kv), p.max_pages << p.page_shift);
  } else {
    k0 = clampi(p.cu_kv[b], 0, p.total_kv);
    const int k1 = clampi(p.cu_kv[b + 1], k0, p.total_kv);
    Lk = min(k1 - k0, p.max_kv);
  }
  const int Lq = min(q1 - q0, p.max_q);
  const int off = Lk - Lq;
  const float c = p.scale_log2;
  const int n_blk = (Lq + TOK - 1) / TOK;

  const uint32_t row_bytes = (uint32_t)p.hkv * (kHeadDim * 2);
  const size_t seq_base = (size_t)k0 * p.hkv * kHeadDim;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + seq_base, (uint32_t)Lk * row_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + seq_base, (uint32_t)Lk * row_bytes);
  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc_uniform(p.q + (size_t)q0 * p.hq * kHeadDim, (uint32_t)Lq * p.hq * (kHeadDim * 2));

  // A lane's head is head0 + lane % GP in every row block and pass (GP divides 32). The GP
  // sink logits come in through scalar loads, once per workgroup.
  float sink_l2 = kNegInf;
  if (p.sinks != nullptr) {
    float sv[GP];
#pragma unroll
    for (int i = 0; i < GP; ++i) sv[i] = p.sinks[head0 + i];
    sink_l2 = sv[0];
#pragma unroll
    for (int i = 1; i < GP; ++i) sink_l2 = ((lane & (GP - 1)) == i) ? sv[i] : sink_l2;
    sink_l2 *= kLog2e;
  }

  for (int pass = 0; pass < (p.pair_blocks ? 2 : 1); ++pass) {
  if (pass == 0 && unit >= (p.pair_blocks ? (n_blk + 1) / 2 : n_blk)) break;
  const int tile = (pass == 0) ? unit : n_blk - 1 - unit;
  if (pass == 1 && tile <= unit) break;
  const int ts = tile * TOK;
  const int te = min(ts + TOK, Lq);

  auto visible_keys = [&](int rb, int& vl, int& vh) {
    const int pos = off + ts + ((w * RB + rb) * 32 + r32) / GP;
    vh = p.causal ? min(Lk, pos + 1) : Lk;
    vl = 0;
    if (vh < vl) vh = vl;
  };
  // The wave's 64 Q rows of the pass go to its LDS slice by DMA, issued before the first
  // K/V tiles (so they have landed once tile 0 has); 16-byte chunk c of row i sits at chunk
  // position c ^ ((i >> 1) & 7), as for K. Rows past the end load the last valid row (their
  // results are never stored). Q lives in LDS, not in registers, for the whole pass.
  unsigned char* qw = q_lds[w];
  {
    const int ln = opaque_lane_id();
    const int pos = ln & 7;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = 8 * k + (ln >> 3);
      const int r = 64 * w + i;
      const int t = min(ts + r / GP, te - 1);
      const int c = pos ^ ((i >> 1) & 7);
      buffer_load16_lds_async(rq, qw + 8 * k * 128,
                              ((uint32_t)t * p.hq + head0 + (r % GP)) * (kHeadDim * 2) + (uint32_t)(c * 16));
    }
  }
  float m[RB], lsum[RB];
  f32x16 o[RB][2];
  int hi_min = 0x7fffffff, lo_max = -0x7fffffff;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = (w * RB + rb) * 32 + r32;
    const int t = ts + r / GP;
    const bool row_ok = t < te;
    m[rb] = sink_l2;
    lsum[rb] = (half == 0) ? 1.0f : 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) { o[rb][0][i] = 0.f; o[rb][1][i] = 0.f; }
    int vl, vh;
    visible_keys(rb, vl, vh);
    if (row_ok) {
      hi_min = min(hi_min, vh);
      lo_max = max(lo_max, vl);
    }
  }
#pragma unroll
  for (int o2 = 32; o2 >= 1; o2 >>= 1) {
    hi_min = min(hi_min, __shfl_xor(hi_min, o2, 64));
    lo_max = max(lo_max, __shfl_xor(lo_max, o2, 64));
  }
  hi_min = __builtin_amdgcn_readfirstlane(hi_min);
  lo_max = __builtin_amdgcn_readfirstlane(lo_max);

  const int p_hi = off + te - 1;
  const int jb = 0;
  const int je = p.causal ? min(Lk, p_hi + 1) : Lk;
  const int nt = (je > jb) ? (je - jb + kTileN - 1) / kTileN : 0;

  if (nt > 0) {
    // Wave w loads rows [8w, 8w + 8) of a tile's K and V (one 1 KB load each); lane i writes
    // chunk position i & 7 of row 8 w + (i >> 3), which holds global chunk (i & 7) ^ f(row), with
    // f(r) = (r >> 1) & 7 for K and ((r >> 1) & 1) * 4 for V, the swizzles of the 4-wave kernel.
    // Contiguous layout: the per-lane parts of the offsets are computed once and kept for the
    // pass. Paged layout: they are rebuilt from the lane id at every issue, beside the page's
    // buffer descriptor; kept in registers across the pass they would be spilled, and each
    // reload would wait for every tile in flight.
    uint32_t k_lane = 0, v_lane = 0;
    if constexpr (!PAGED) {
      const int ln = opaque_lane_id();
      const int r8 = ln >> 3;
      const int pch = ln & 7;
      const int swz_k = (r8 >> 1) | ((w & 1) << 2);
      const int swz_v = (r8 & 2) << 1;
      k_lane = (uint32_t)r8 * row_bytes + (uint32_t)((pch ^ swz_k) << 4);
      v_lane = (uint32_t)r8 * row_bytes + (uint32_t)((pch ^ swz_v) << 4);
    }
    auto issue_tile = [&](int t) {
      if constexpr (PAGED) {
        // Rows [8w, 8w + 8) of the tile are 8 consecutive keys inside one page (pages hold a
        // power of two >= 16 keys); the buffer range ends at the sequence's last key.
        const int kr = jb + t * kTileN + 8 * w;
        const int slot = min(kr >> p.page_shift, p.max_pages - 1);
        const int pid = clampi(load_invariant(p.page_table, (size_t)b * p.max_pages + slot), 0, p.num_pages - 1);
        const uint32_t valid = (uint32_t)clampi(Lk - kr, 0, 8);
        const size_t blk = (((size_t)pid * p.hkv + kvh) * p.page_size + (kr & (p.page_size - 1))) * kHeadDim;
        const int ln = opaque_lane_id();
        const int r8 = ln >> 3;
        const int pch = ln & 7;
        const int swz_k = (r8 >> 1) | ((w & 1) << 2);
        const int swz_v = (r8 & 2) << 1;
        unsigned char* dst = kv_lds[t & (kRing - 1)] + 8 * w * 128;
        buffer_load16_lds_async(make_rsrc_uniform(p.k + blk, valid * (kHeadDim * 2)), dst,
                                (uint32_t)(r8 * 128 + ((pch ^ swz_k) << 4)));
        buffer_load16_lds_async(make_rsrc_uniform(p.v + blk, valid * (kHeadDim * 2)), dst + kTileBytes,
                                (uint32_t)(r8 * 128 + ((pch ^ swz_v) << 4)));
        return;
      }
      const uint32_t row0 = (uint32_t)(jb + t * kTileN + 8 * w) * row_bytes + (uint32_t)kvh * (kHeadDim * 2);
      unsigned char* dst = kv_lds[t & (kRing - 1)] + 8 * w * 128;
      buffer_load16_lds_async(rk, dst, k_lane + row0);
      buffer_load16_lds_async(rv, dst + kTileBytes, v_lane + row0);
    };
    issue_tile(0);
    if (nt > 1) issue_tile(1);

    f32x16 s[RB][2];      // S^T of the current tile, per row block and 32-key half
    u32x4 pk[RB][2][2];   // P^T as bf16 B operands, per row block, half and 16-key step

    // Per-lane LDS offsets. K: row r32 of a half, 16-byte chunk (2 ks + half) ^ f(row) (f only
    // depends on the row inside the half). V: the transposing reads of 16-key step kk start at
    // row 16 kk + 4 (grp >> 1) + (jl >> 2); their swizzle does not depend on kk.
    uint32_t k_off[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) k_off[ks] = r32 * 128 + (((2 * ks + half) ^ ((r32 >> 1) & 7)) << 4);
    uint32_t v_off[2];
    {
      const int grp = lane >> 4;
      const int jl = lane & 15;
      const int krow = 4 * (grp >> 1) + (jl >> 2);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const int c0 = dt * 32 + 16 * (grp & 1) + 4 * (jl & 3);
        v_off[dt] = krow * 128 + ((((c0 >> 3) ^ (((krow >> 1) & 1) * 4)) << 4) + ((c0 & 7) << 1));
      }
    }

    // Matrix phase t: O^T += V_{t-1}^T P_{t-1}^T (if t >= 1), then S_t^T = K_t Q^T (if t < nt).
    // Every LDS fragment of the phase is requested before the first MFMA.
    auto matrix_phase = [&](int t, auto pv_tag, auto qk_tag) {
      constexpr bool do_pv = decltype(pv_tag)::value, do_qk = decltype(qk_tag)::value;
      // The phases of one wave stay apart: letting the scheduler hoist this phase's LDS reads
      // into the softmax phase would keep S, P and all fragments live at once.
      __builtin_amdgcn_sched_barrier(0);
      u32x4 av[4][2], ka[2][4], qa[RB][4];
      if constexpr (do_pv) {
        const unsigned char* vt = kv_lds[(t - 1) & (kRing - 1)] + kTileBytes;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int dt = 0; dt < 2; ++dt)
            av[kk][dt] = join_tr16(lds_read_tr16(vt + kk * 2048 + v_off[dt]), lds_read_tr16(vt + kk * 2048 + 1024 + v_off[dt]));
      }
      if constexpr (do_qk) {
        const unsigned char* kt_lds = kv_lds[t & (kRing - 1)];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) ka[kt][ks] = *reinterpret_cast<const u32x4*>(kt_lds + kt * 4096 + k_off[ks]);
        // Q^T fragments: the same lane layout as K (row r32 of a 32-row block).
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) qa[rb][ks] = *reinterpret_cast<const u32x4*>(qw + rb * 4096 + k_off[ks]);
      }
      // Keep the PV products ahead of the QK products: interleaving them would keep P, S and
      // both sets of fragments live at once.
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (do_pv) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int dt = 0; dt < 2; ++dt)
              o[rb][dt] = mfma32(as_bf16x8(av[kk][dt]), as_bf16x8(pk[rb][kk >> 1][kk & 1]), o[rb][dt]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (do_qk) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              s[rb][kt] = mfma32(as_bf16x8(ka[kt][ks]), as_bf16x8(qa[rb][ks]), ks == 0 ? f32x16{} : s[rb][kt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    auto mask_half = [&](int hs, int kt) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        int vl, vh;
        visible_keys(rb, vl, vh);
        const unsigned span = (unsigned)(vh - vl);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = hs + 8 * (i >> 2) + 4 * half + (i & 3);
          s[rb][kt][i] = ((unsigned)(j - vl) < span) ? s[rb][kt][i] : kNegInf;
        }
      }
    };
    auto exp_half = [&](int kt, int rb, float nm) -> float {
      float a0, a1;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float e0 = fast_exp2(__builtin_fmaf(s[rb][kt][i], c, nm));
        const float e1 = fast_exp2(__builtin_fmaf(s[rb][kt][i + 1], c, nm));
        a0 = (i == 0) ? e0 : a0 + e0;
        a1 = (i == 0) ? e1 : a1 + e1;
        pk[rb][kt][i >> 3][(i & 7) >> 1] = pack_bf16x2(e0, e1);
      }
      return a0 + a1;
    };
    // Softmax phase t: P_t from S_t with the lazy-max guard, taken over the whole 64-key tile:
    // both halves are converted before the PV product of the next matrix phase, so a move of m
    // must redo both of them (a P computed with the old m would be added to the rescaled O).
    auto softmax_phase = [&](int t) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int hs = jb + t * kTileN + kt * 32;
        if (!(hs >= lo_max && hs + 32 <= hi_min)) mask_half(hs, kt);
      }
      float ps[RB][2];
      for (int attempt = 0; attempt < 2; ++attempt) {
        bool ok = true;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            ps[rb][kt] = exp_half(kt, rb, (m[rb] == kNegInf && attempt > 0) ? 0.f : -m[rb]);
            ok = ok && (ps[rb][kt] <= kSumGuard);
          }
        if (__builtin_expect(!__any(!ok), 1) || attempt > 0) break;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          float mx = kNegInf;
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fmaxf(s[rb][0][i], s[rb][1][i]));
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
      for (int rb = 0; rb < RB; ++rb) lsum[rb] += ps[rb][0] + ps[rb][1];
    };
    // Slots: group A runs M_t in slot 2t and V_t in slot 2t + 1; group B runs one slot later.
    // There is one workgroup barrier per tile, at the start of every even slot 2u: before it,
    // tile u must be in LDS (tile u + 1 may still be in flight); after it, tile u + 2 goes into
    // the stage of tile u - 2. Between two barriers (the period of tile u) group A runs
    // M_u, V_u and group B runs V_{u-1}, M_u, so the reads of tile u - 2 all happened in
    // earlier periods, and the two waves of a SIMD stay in opposite phases.
    auto sync_slot = [&](int slot) {
      if (slot & 1) return;
      const int u = slot >> 1;
      if (u < nt) {
        if (u + 1 < nt) {
          WAIT_VMCNT(2);
        } else {
          WAIT_VMCNT(0);
        }
      }
      lds_barrier();
      if (u + 2 < nt) issue_tile(u + 2);
    };

    // 2 nt + 3 slots for every wave (group A idles in the last one, group B in the first).
    // The first and last matrix phases are peeled so that S is always written before it is
    // read inside the loop (and so is dead across its back edge).
    // Issue priorities keep the two groups in opposite phases between barriers: matrix phases
    // first (their MFMAs then issue as soon as the matrix unit frees up), then the softmax
    // phase that opened the period (group B's), then the one that started mid-period (group
    // A's), which would otherwise win the VALU and push group B's softmax into the next slot.
    auto prio_matrix = [&]() { __builtin_amdgcn_s_setprio(3); };
    auto prio_softmax = [&]() {
      if (lag) {
        __builtin_amdgcn_s_setprio(2);
      } else {
        __builtin_amdgcn_s_setprio(1);
      }
    };
    const std::true_type yes{};
    const std::false_type no{};
    if (lag) sync_slot(0);
    sync_slot(lag);
    prio_matrix();
    matrix_phase(0, no, yes);
    sync_slot(1 + lag);
    prio_softmax();
    softmax_phase(0);
    for (int t = 1; t < nt; ++t) {
      sync_slot(2 * t + lag);
      prio_matrix();
      matrix_phase(t, yes, yes);
      sync_slot(2 * t + 1 + lag);
      prio_softmax();
      softmax_phase(t);
    }
    sync_slot(2 * nt + lag);
    prio_matrix();
    matrix_phase(nt, yes, no);
    __builtin_amdgcn_s_setprio(0);
    sync_slot(2 * nt + 1 + lag);
    if (!lag) sync_slot(2 * nt + 2);
    // The last loads were retired in the loop; every wave is done with the ring before the
    // next pass reuses it.
    __syncthreads();
  } else {
    // No key is visible: Q is not needed, but its DMA must land before the slice is reused
    // for the output.
    WAIT_VMCNT(0);
  }

  // O goes through this wave's LDS slice: the accumulator layout gives a lane 8-byte pieces
  // of one row, the stores then write whole 128-byte rows (8 lanes per row, 8 rows per
  // instruction). 16-byte chunk c of row i sits at chunk position c ^ (i & 7).
  {
    const int ln = opaque_lane_id();
    const int hf = ln >> 5;
    unsigned char* ow = qw;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float lt = lsum[rb] + shfl_xor(lsum[rb], 32);
      const float inv = (lt > 0.f) ? 1.0f / lt : 0.f;
      const int i = rb * 32 + (ln & 31);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          u32x2 pkd;
          pkd[0] = pack_bf16x2(o[rb][dt][q4 * 4 + 0] * inv, o[rb][dt][q4 * 4 + 1] * inv);
          pkd[1] = pack_bf16x2(o[rb][dt][q4 * 4 + 2] * inv, o[rb][dt][q4 * 4 + 3] * inv);
          const int c = dt * 4 + q4;
          *reinterpret_cast<u32x2*>(ow + i * 128 + ((c ^ (i & 7)) << 4) + hf * 8) = pkd;
        }
      }
      const int r = (w * RB + rb) * 32 + (ln & 31);
      const int t = ts + r / GP;
      if (p.lse != nullptr && hf == 0 && t < te) {
        p.lse[(size_t)(q0 + t) * p.hq + head0 + (r % GP)] =
            (m[rb] == kNegInf || !(lt > 0.f)) ? kNegInf : (m[rb] + fast_log2(lt)) * kLn2;
      }
    }
    const int c = ln & 7;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = 8 * k + (ln >> 3);
      const u32x4 v = *reinterpret_cast<const u32x4*>(ow + i * 128 + ((c ^ (i & 7)) << 4));
      const int r = (w * RB + (i >> 5)) * 32 + (i & 31);
      const int t = ts + r / GP;
      if (t < te)
        *reinterpret_cast<u32x4*>(p.out + ((size_t)(q0 + t) * p.hq + head0 + (r % GP)) * kHeadDim + c * 8) = v;
    }
  }
  }  // pass
}

namespace {
template <int RB, bool PAGED>
hipError_t launch_rb(PrefillParams p, int gp, hipStream_t stream) {
  const int tok = 128 * RB / gp;
  const int n_blk = (p.max_q + tok - 1) / tok;
  p.pair_blocks = (p.causal && p.window == 0) ? 1 : 0;
  p.units = p.pair_blocks ? (n_blk + 1) / 2 : n_blk;
  const long items = (long)p.units * p.batch * p.hkv * (p.group / gp);
  if (items > 0x7ffffff0L) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)(8 * ((items + 7) / 8))), block(kThreads);
  switch (gp) {
    case 1: hipLaunchKernelGGL((prefill_kernel<1, RB, PAGED>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<2, RB, PAGED>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<4, RB, PAGED>), grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<8, RB, PAGED>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((prefill_kernel<16, RB, PAGED>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

template <bool PAGED>
hipError_t launch_pp(PrefillParams p, int gp, hipStream_t stream) {
  const int tok = 512 / gp;
  const int n_blk = (p.max_q + tok - 1) / tok;
  p.pair_blocks = p.causal ? 1 : 0;
  p.units = p.pair_blocks ? (n_blk + 1) / 2 : n_blk;
  const long pairs = (long)p.batch * p.hkv * (p.group / gp);  // (sequence, head group)
  p.xcd_round_robin = (pairs % 8 == 0) ? 1 : 0;
  const long items = pairs * (long)p.units;  // a multiple of 8 when dealing pairs round-robin
  if (items > 0x7ffffff0L) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)(8 * ((items + 7) / 8))), block(512);
  switch (gp) {
    case 1: hipLaunchKernelGGL((prefill_pp_kernel<1, PAGED>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((prefill_pp_kernel<2, PAGED>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((prefill_pp_kernel<4, PAGED>), grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL((prefill_pp_kernel<8, PAGED>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((prefill_pp_kernel<16, PAGED>), grid, block, 0, stream, p); break;
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
  const bool rb2 = prefill_row_blocks(p.max_q, gp) == 2;
  const bool paged = p.page_table != nullptr;  // chunked prefill on a paged cache
  // Long query ranges without a window: the 8-wave ping-pong kernel.
  if (p.window == 0 && p.max_q >= 2048) return paged ? launch_pp<true>(p, gp, stream) : launch_pp<false>(p, gp, stream);
  if (paged) return rb2 ? launch_rb<2, true>(p, gp, stream) : launch_rb<1, true>(p, gp, stream);
  return rb2 ? launch_rb<2, false>(p, gp, stream) : launch_rb<1, false>(p, gp, stream);
}

}  // namespace attn_sink
