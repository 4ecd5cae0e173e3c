// Split-KV paged decode / verify kernel for attention with per-head sink logits.
//
// Method ("GPT-OSS on Day 0", section "Attention sinks"): softmax over the scaled Q.K
// scores plus one sink logit per head; computed online with a running maximum m and a
// scale d; the running maximum of the first KV chunk is seeded with the head's sink
// (d = 1), later chunks start from m = -inf; chunk partials are merged by log-sum-exp
// (merge.hip). Heads and the KV length are processed in parallel (same section).
//
// Work decomposition
//   * A work item is (sequence b, KV chunk c, KV head g). Items are enumerated densely
//     over the chunks that exist (n_b = max(1, ceil(L_b / chunk)) per sequence), with the
//     KV head varying fastest so that the workgroups running side by side read all heads'
//     blocks of the same pages (one page of all heads is contiguous in HBM).
//   * The kernel is persistent: a grid sized to fill the chip walks the item list with a
//     stride of gridDim.x. Each workgroup finds the sequence of an item with a running
//     prefix-sum cursor over kv_lens (64 sequences per wave-wide step), so no host-side
//     plan and no per-item search table are needed, and the grid depends only on host
//     scalars.
//   * Inside an item, columns = the q_len query tokens x G query heads that share the KV
//     head (one K/V fetch serves all of them), padded to NT tiles of 16. The chunk's keys
//     are cut into 16-key groups (each inside one page: a contiguous 2 KB block of K and
//     one of V); wave w owns groups w, w + 4, w + 8, ...
//   * Streaming: every wave moves its own groups HBM -> LDS with non-temporal buffer loads
//     that write LDS directly, through a private ring of S stages, so S groups are in
//     flight per wave without holding registers, and the next item's first groups are
//     already requested before the current item is combined. A wave only reads the LDS it
//     filled, so the streaming needs no workgroup barrier; the compiler does not see these
//     loads (it would otherwise wait for all of them before every LDS read) and the waits
//     are explicit s_waitcnt vmcnt counts.
//   * Per group: S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (K fragments from LDS, Q^T in
//     registers); masks from indices; online softmax in the exp2 domain with a lazy
//     running max; P^T (which already has the B-operand layout of the 16x16x16 product)
//     times V^T read from LDS transposed (ds_read_b64_tr_b16): O^T += V^T P^T with
//     v_mfma_f32_16x16x16_bf16.
//   * The 4 wave states are combined in a fixed order ((w0 + w1) + (w2 + w3),
//     bit-reproducible) through LDS and the chunk partial (o/d, m + ln d) goes to the
//     workspace at the plan's offset.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace attn_sink {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kGroupKeys = 16;
constexpr int kGroupBytes = kGroupKeys * kHeadDim * 2;  // 2 KB of K (or V) per group
constexpr int kStageBytes = 2 * kGroupBytes;            // K then V
constexpr int kSegGroups = 64;                          // page ids held by one lane vector
constexpr float kLazyMax = 16.0f;                       // running-max slack (log2 units)

// Ring stages per wave, by column-tile count: as deep as the LDS budget of two
// workgroups per CU allows next to the combine buffers.
template <int NT> struct DecodeRing { static constexpr int value = 3; };
template <> struct DecodeRing<1> { static constexpr int value = 3; };
template <> struct DecodeRing<4> { static constexpr int value = 2; };

__device__ __forceinline__ int chunks_for(int L, int chunk) {
  int n = (L + chunk - 1) / chunk;
  return n < 1 ? 1 : n;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  return v;
}

// LDS layout of a group: row r (key) holds 8 chunks of 16 B; chunk c sits at position
// c ^ swz(r). K: swz = (r >> 1) & 7, so that the 16 rows read by one 16-lane group at the
// same chunk (A operand of the 16x16x32 product) hit 64 distinct banks. V: swz flips bit 2
// with (r >> 1) & 1 and bit 1 with (r >> 2) & 1, so that the transposing reads (4 rows x
// 32 B per 16 lanes) of two neighbouring lane groups do not share banks.
__device__ __forceinline__ int k_swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int v_swz(int r) { return (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1); }

// s_waitcnt vmcnt(N) (N < 64) that also orders memory accesses for the compiler.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}
// vmcnt(4 k) for a runtime k in [0, 15].
__device__ __forceinline__ void wait_groups(int k) {
  switch (k) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<4>(); break;
    case 2: wait_vmcnt<8>(); break;
    case 3: wait_vmcnt<12>(); break;
    case 4: wait_vmcnt<16>(); break;
    case 5: wait_vmcnt<20>(); break;
    case 6: wait_vmcnt<24>(); break;
    default: wait_vmcnt<28>(); break;
  }
}

__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0 << 8) | (3 << 14));
  asm volatile("" ::: "memory");
}

}  // namespace

template <int NT, bool TREE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_split_kernel(DecodeParams p) {
  constexpr int S = DecodeRing<NT>::value;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kWaves][S][kStageBytes];
  // Combine exchange: two slots of per-lane wave states (O^T tiles, then m and d per tile).
  __shared__ __attribute__((aligned(16))) f32x4 xo[2][NT][4][64];
  __shared__ __attribute__((aligned(8))) float xm[2][NT][64], xl[2][NT][64];

  // LDS byte address of the ring (a constant of the kernel's LDS layout)
  const uint32_t ring_lds = (uint32_t)(uintptr_t)LDS_PTR(unsigned char, &ring[0][0][0]);

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = p.group;
  const int R = p.q_len * G;  // live columns
  const int col_lo = lane & 15;
  const int grp = lane >> 4;  // 16-lane group 0..3
  const float c2 = p.scale_log2;

  // Sinks of heads 0..255 in four lane vectors (one load at the start, none per item).
  float sink_vec[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 64 * i + lane;
    sink_vec[i] = (p.sinks != nullptr && h < p.hq) ? p.sinks[h] * kLog2e : kNegInf;
  }
  auto sink_of = [&](int h) -> float {
    if (p.sinks == nullptr) return kNegInf;
    if (h >= 256) return p.sinks[h] * kLog2e;  // more heads than the vectors hold
    const float v0 = __shfl(sink_vec[0], h & 63, 64), v1 = __shfl(sink_vec[1], h & 63, 64);
    const float v2 = __shfl(sink_vec[2], h & 63, 64), v3 = __shfl(sink_vec[3], h & 63, 64);
    const int i = h >> 6;
    return i == 0 ? v0 : (i == 1 ? v1 : (i == 2 ? v2 : v3));
  };

  // ---- total number of (sequence, chunk) pairs, and a cursor over sequences
  const int cap = p.max_kv_len < p.max_pages * p.page_size ? p.max_kv_len : p.max_pages * p.page_size;
  int tot = 0;
  for (int i = lane; i < p.batch; i += 64) tot += chunks_for(clampi(p.kv_lens[i], 0, cap), p.kv_chunk);
  const int total_items = wave_sum_int(tot) * p.hkv;

  int cur_base = 0;    // first sequence of the cursor window
  int cur_before = 0;  // pairs before cur_base
  int win_incl = 0;    // inclusive prefix of chunk counts inside the window (this lane's sequence)
  int win_len = 0;     // clamped length of this lane's sequence
  int win_total = 0;
  auto load_window = [&]() {
    const int i = cur_base + lane;
    win_len = (i < p.batch) ? clampi(p.kv_lens[i], 0, cap) : 0;
    const int n = (i < p.batch) ? chunks_for(win_len, p.kv_chunk) : 0;
    win_incl = wave_inclusive_scan(n, lane);
    win_total = __builtin_amdgcn_readlane(win_incl, 63);
  };
  load_window();

  struct Loc {
    int b, c, kvh, L, n_b, base, chunk_lo, chunk_hi, n_groups;
  };
  // Location of an item (the cursor only moves forward: items are visited in order).
  auto locate = [&](int item) -> Loc {
    Loc r;
    const int P = item / p.hkv;
    r.kvh = item - P * p.hkv;
    // (P < the pair count, so a later window holds it; the batch bound keeps the walk finite even
    // if kv_lens changed since the count was taken.)
    while (P >= cur_before + win_total && cur_base + 64 < p.batch) {
      cur_before += win_total;
      cur_base += 64;
      load_window();
    }
    const unsigned long long before_mask = __ballot(cur_before + win_incl <= P);
    const int idx = __popcll(before_mask);
    r.b = cur_base + idx;
    const int pairs_before = cur_before + (idx > 0 ? __builtin_amdgcn_readlane(win_incl, idx - 1) : 0);
    r.c = P - pairs_before;
    r.L = __builtin_amdgcn_readlane(win_len, idx);
    r.n_b = chunks_for(r.L, p.kv_chunk);
    r.base = pairs_before * p.q_len;  // indptr of row b*q_len
    r.chunk_lo = r.c * p.kv_chunk;
    r.chunk_hi = min(r.chunk_lo + p.kv_chunk, r.L);
    r.n_groups = (r.chunk_hi > r.chunk_lo) ? (r.chunk_hi - r.chunk_lo + kGroupKeys - 1) / kGroupKeys : 0;
    r.b = __builtin_amdgcn_readfirstlane(r.b);
    r.c = __builtin_amdgcn_readfirstlane(r.c);
    r.kvh = __builtin_amdgcn_readfirstlane(r.kvh);
    r.L = __builtin_amdgcn_readfirstlane(r.L);
    r.n_b = __builtin_amdgcn_readfirstlane(r.n_b);
    r.base = __builtin_amdgcn_readfirstlane(r.base);
    r.chunk_lo = __builtin_amdgcn_readfirstlane(r.chunk_lo);
    r.chunk_hi = __builtin_amdgcn_readfirstlane(r.chunk_hi);
    r.n_groups = __builtin_amdgcn_readfirstlane(r.n_groups);
    return r;
  };
  // Raw page ids of groups [64 seg, 64 seg + 64) of an item, one per lane (lanes past the last
  // group repeat it). The load is unconditional and its value is only touched where a group
  // is issued (clamped there), so the wait for it does not come right after the load, when
  // the item's first groups are still in flight.
  auto load_page_ids = [&](const Loc& l, int seg) -> int {
    const int g = min(64 * seg + lane, max(l.n_groups - 1, 0));
    const int j = l.chunk_lo + kGroupKeys * g;
    return p.page_table[(size_t)l.b * p.max_pages + (j >> p.page_shift)];
  };
  // Q^T as the B operand (k = head dim), one 16-column tile per nt. Plain loads, issued at the
  // end of the previous item: the compiler's wait for them at this item's first product also
  // retires the groups requested after them (loads return in order), which have landed during
  // the combine by then (measured: no slower than keeping the wait on the Q loads alone).
  auto load_q = [&](const Loc& l, u32x4 (&qb)[NT][2]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int col = nt * 16 + col_lo;
      const int cc = col < R ? col : 0;
      const int t = cc / G, gh = cc - (cc / G) * G;
      const uint16_t* src = p.q + ((size_t)(l.b * p.q_len + t) * p.hq + l.kvh * G + gh) * kHeadDim + grp * 8;
      qb[nt][0] = *reinterpret_cast<const u32x4*>(src);
      qb[nt][1] = *reinterpret_cast<const u32x4*>(src + 32);
    }
  };
  // DMA of this wave's group g of item l (page id taken from pid, the vector of the group's
  // 64-group segment) into ring stage st. Rows past the chunk's last key read as zeros (the
  // buffer range stops there), so masked keys multiply exact zeros.
  auto issue_group = [&](const Loc& l, int pid, int g, int st) {
    const int key0 = l.chunk_lo + kGroupKeys * g;
    const int page = clampi(__builtin_amdgcn_readlane(pid, g & (kSegGroups - 1)), 0, p.num_pages - 1);
    const size_t row0 = (((size_t)page * p.hkv + l.kvh) * p.page_size + (key0 & (p.page_size - 1))) * kHeadDim;
    const int valid = min(kGroupKeys, l.chunk_hi - key0);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc_uniform(p.k_cache + row0, (uint32_t)valid * (kHeadDim * 2));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc_uniform(p.v_cache + row0, (uint32_t)valid * (kHeadDim * 2));
    const uint32_t dst = ring_lds + (uint32_t)((w * S + st) * kStageBytes);
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int r = 8 * ii + (lane >> 3);
      const int pch = lane & 7;
      buffer_load16_lds_async_nt(rk, dst + ii * 1024, (uint32_t)(r * 128 + ((pch ^ k_swz(r)) << 4)));
      buffer_load16_lds_async_nt(rv, dst + kGroupBytes + ii * 1024, (uint32_t)(r * 128 + ((pch ^ v_swz(r)) << 4)));
    }
  };

  // Per-lane LDS offsets of a group's fragments.
  const uint32_t k_off0 = col_lo * 128 + (((0 + grp) ^ k_swz(col_lo)) << 4);
  const uint32_t k_off1 = col_lo * 128 + (((4 + grp) ^ k_swz(col_lo)) << 4);
  uint32_t v_off[4];
  {
    const int vr = 4 * grp + (col_lo >> 2);  // row this lane points at
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int byte = dt * 32 + 8 * (col_lo & 3);
      v_off[dt] = kGroupBytes + vr * 128 + ((((byte >> 4) ^ v_swz(vr))) << 4) + (byte & 15);
    }
  }

  int ring_ctr = 0;  // ring position of this wave's next group
  int pid_next;      // raw page ids of the next item's first segment (loaded during an item)
  if ((int)blockIdx.x >= total_items) return;
  Loc cur = locate(blockIdx.x);
  int pid = load_page_ids(cur, 0);
  asm volatile("" ::"v"(pid));  // wait for it before any group is requested
  int pid_seg = 0;  // segment of the item whose page ids pid holds
  u32x4 qb[NT][2];
  load_q(cur, qb);
  auto my_groups = [&](const Loc& l) -> int { return (l.n_groups > w) ? (l.n_groups - w + kWaves - 1) / kWaves : 0; };
  int n_mine = my_groups(cur);
  int n_pref = min(S, n_mine);
  for (int k = 0; k < n_pref; ++k) issue_group(cur, pid, w + kWaves * k, (ring_ctr + k) % S);

  for (int item = blockIdx.x; item < total_items; item += gridDim.x) {
    // The next item is located and its page ids loaded on every iteration (the last one
    // re-reads its own): the compiler's wait analysis does not follow branch conditions, and
    // a conditional load would make it wait again after the next item's loads are issued.
    const bool has_next = item + (int)gridDim.x < total_items;
    const Loc nxt = locate(has_next ? item + (int)gridDim.x : item);
    pid_next = load_page_ids(nxt, 0);

    const int b = cur.b, c = cur.c, kvh = cur.kvh, L = cur.L;
    // Position of the first query token in this range's key numbering, and whether this range
    // holds key 0 of its sequence (only that range counts the sink).
    int q0_pos = L - p.q_len;
    bool seeds_sink = true;
    if (p.kv_start != nullptr) {
      const int start = load_invariant(p.kv_start, (size_t)b);
      q0_pos = load_invariant(p.kv_total, (size_t)b) - p.q_len - start;
      seeds_sink = start == 0;
    }
    // ---- keys visible to each column inside this chunk: [vis_lo, vis_hi); wave-wide bounds
    // decide whether a group needs masking at all.
    int vis_lo[NT], vis_hi[NT];
    int hi_min = 0x7fffffff, lo_max = -0x7fffffff;
    float m[NT], lsum[NT];
    f32x4 o[NT][4];
    // Draft tree: each column's bitmap of visible draft tokens (the last q_len keys); the q_len
    // bitmaps of the sequence come in through scalar loads.
    const int blk0 = L - p.q_len;
    int tbits[NT];
    if constexpr (TREE) {
      const int32_t* tb = p.tree_mask + (size_t)b * p.q_len;
      int sv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) sv[i] = tb[min(i, p.q_len - 1)];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int col = nt * 16 + col_lo;
        const int t = col < R ? col / G : 0;
        int v = sv[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) v = (t == i) ? sv[i] : v;
        tbits[nt] = v;
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int col = nt * 16 + col_lo;
      const int pos = q0_pos + col / G;
      vis_hi[nt] = (p.causal && !TREE) ? min(cur.chunk_hi, pos + 1) : cur.chunk_hi;
      vis_lo[nt] = (p.window > 0) ? max(cur.chunk_lo, pos - p.window + 1) : cur.chunk_lo;
      if (vis_hi[nt] < vis_lo[nt]) vis_hi[nt] = vis_lo[nt];
      if (col < R) {
        hi_min = min(hi_min, vis_hi[nt]);
        lo_max = max(lo_max, vis_lo[nt]);
      }
      // First chunk: the running max starts at the head's sink and d at 1 (held by lane group
      // 0 so the column sum counts it once). Other chunks and waves: m = -inf (d = 1 is inert).
      const int h = kvh * G + (col < R ? col % G : 0);
      const float sink2 = sink_of(h);
      m[nt] = (c == 0 && w == 0 && seeds_sink) ? sink2 : kNegInf;
      lsum[nt] = (grp == 0) ? 1.0f : 0.0f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[nt][dt] = f32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      hi_min = min(hi_min, __shfl_xor(hi_min, off, 64));
      lo_max = max(lo_max, __shfl_xor(lo_max, off, 64));
    }
    hi_min = __builtin_amdgcn_readfirstlane(hi_min);
    lo_max = __builtin_amdgcn_readfirstlane(lo_max);

    for (int k = 0; k < n_mine; ++k) {
      const int g = w + kWaves * k;
      wait_groups(min(S - 1, n_mine - 1 - k));
      const unsigned char* st = ring[w][(ring_ctr + k) % S];
      const int key0 = cur.chunk_lo + kGroupKeys * g;

      // S^T: 16 keys x 16 columns per nt
      const u32x4 ka0 = *reinterpret_cast<const u32x4*>(st + k_off0);
      const u32x4 ka1 = *reinterpret_cast<const u32x4*>(st + k_off1);
      s16x4 av[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) av[dt] = lds_read_tr16(st + v_off[dt]);
      f32x4 sc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4 a = f32x4{0, 0, 0, 0};
        a = mfma16(as_bf16x8(ka0), as_bf16x8(qb[nt][0]), a);
        a = mfma16(as_bf16x8(ka1), as_bf16x8(qb[nt][1]), a);
        sc[nt] = a;
      }
      // the ring stage is free again once its LDS reads have returned: request the group S
      // places ahead
      if (k + S < n_mine) {
        wait_lgkm0();
        const int g2 = g + kWaves * S;
        if ((g2 >> 6) != pid_seg) {
          // items longer than 64 groups: next segment's page ids, loaded and waited for right
          // here (it drains this wave's loads, once per 64 groups). The load is kept out of
          // the compiler's sight, which would otherwise wait before every group.
          pid_seg = __builtin_amdgcn_readfirstlane(g2 >> 6);
          const int gi = min(64 * pid_seg + lane, max(cur.n_groups - 1, 0));
          const int32_t* src = p.page_table + (size_t)cur.b * p.max_pages + ((cur.chunk_lo + kGroupKeys * gi) >> p.page_shift);
          asm volatile("global_load_dword %0, %1, off\n\ts_waitcnt vmcnt(0)" : "=v"(pid) : "v"(src) : "memory");
        }
        issue_group(cur, pid, g2, (ring_ctr + k + S) % S);
      }

      // ---- masks (only on groups that straddle a bound) + online softmax with a lazy max:
      // m moves only when some score exceeds it by more than kLazyMax (log2 units); every term
      // of a column always uses that column's current m, so the softmax is unchanged.
      if (!(key0 + kGroupKeys <= hi_min && key0 >= lo_max) || (TREE && key0 + kGroupKeys > blk0)) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const unsigned span = (unsigned)(vis_hi[nt] - vis_lo[nt]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = key0 + 4 * grp + i;
            bool vis = (unsigned)(key - vis_lo[nt]) < span;
            if constexpr (TREE) {
              // Draft keys follow the column's bitmap; prefix keys (dk wraps past 31) are kept.
              // Branch-free, with the shift amount kept in range.
              const unsigned dk = (unsigned)(key - blk0);
              const unsigned bit = ((unsigned)tbits[nt] >> (dk & 31u)) & 1u;
              vis = vis && (dk > 31u || bit != 0u);
            }
            sc[nt][i] = vis ? sc[nt][i] : kNegInf;
          }
        }
      }
      bool bump = false;
      float mx[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        mx[nt] = fmaxf(fmaxf(sc[nt][0], sc[nt][1]), fmaxf(sc[nt][2], sc[nt][3])) * c2;
        bump = bump || (mx[nt] > m[nt] + kLazyMax);
      }
      if (__any(bump)) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float v = mx[nt];
          v = fmaxf(v, shfl_xor(v, 16));
          v = fmaxf(v, shfl_xor(v, 32));
          const float m_new = fmaxf(m[nt], v);
          const float alpha = (m_new == kNegInf) ? 1.0f : fast_exp2(m[nt] - m_new);
          m[nt] = m_new;
          lsum[nt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) o[nt][dt] *= alpha;
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float neg_m = (m[nt] == kNegInf) ? 0.0f : -m[nt];
        const float e0 = fast_exp2(__builtin_fmaf(sc[nt][0], c2, neg_m));
        const float e1 = fast_exp2(__builtin_fmaf(sc[nt][1], c2, neg_m));
        const float e2 = fast_exp2(__builtin_fmaf(sc[nt][2], c2, neg_m));
        const float e3 = fast_exp2(__builtin_fmaf(sc[nt][3], c2, neg_m));
        lsum[nt] += (e0 + e1) + (e2 + e3);
        const u32x2 pw = u32x2{pack_bf16x2(e0, e1), pack_bf16x2(e2, e3)};
        const s16x4 pb = __builtin_bit_cast(s16x4, pw);
        // O^T += V^T P^T: A = V^T (row = head dim, k = the 4 keys of this lane group)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[nt][dt] = mfma16k16(av[dt], pb, o[nt][dt]);
      }
    }
    ring_ctr += n_mine;

    // ---- the next item's Q and first groups go out before this item is combined
    int n_mine_next = 0, n_pref_next = 0;
    if (has_next) {
      n_mine_next = my_groups(nxt);
      n_pref_next = min(S, n_mine_next);
    }

    // ---- plan: chunk counts and partial offsets (one writer per sequence)
    if (c == 0 && kvh == 0 && w == 0) {
      if (lane < p.q_len) {
        p.counts[b * p.q_len + lane] = cur.n_b;
        p.indptr[b * p.q_len + lane] = cur.base + lane * cur.n_b;
      }
      if (b == p.batch - 1 && lane == 0) p.indptr[p.batch * p.q_len] = cur.base + p.q_len * cur.n_b;
    }

    // ---- combine the 4 wave states in the order (w0 + w1) + (w2 + w3); each lane holds the
    // same (column, head-dim) slots in every wave. Column sums first.
    float lt[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      lt[nt] = lsum[nt];
      lt[nt] += shfl_xor(lt[nt], 16);
      lt[nt] += shfl_xor(lt[nt], 32);
    }
    auto put = [&](int slot) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) xo[slot][nt][dt][lane] = o[nt][dt];
        xm[slot][nt][lane] = m[nt];
        xl[slot][nt][lane] = lt[nt];
      }
    };
    auto fold = [&](int slot) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float m2 = xm[slot][nt][lane], l2 = xl[slot][nt][lane];
        const float M = fmaxf(m[nt], m2);
        const float Mu = (M == kNegInf) ? 0.f : M;
        const float a1 = fast_exp2(m[nt] - Mu), a2 = fast_exp2(m2 - Mu);
        lt[nt] = lt[nt] * a1 + l2 * a2;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[nt][dt] = o[nt][dt] * a1 + xo[slot][nt][dt][lane] * a2;
        m[nt] = M;
      }
    };
    // The next item's DMAs are issued first (their ring stages are free: every group of this
    // item has been consumed).
    // The page-id load is compiler-visible: make its wait (a vmcnt(0), free here since every
    // group of this item has arrived) happen before the next Q loads are issued.
    asm volatile("" ::"v"(pid_next));
    if (has_next) {
      load_q(nxt, qb);
      for (int k = 0; k < n_pref_next; ++k) issue_group(nxt, pid_next, w + kWaves * k, (ring_ctr + k) % S);
    }
    if (w == 1 || w == 3) put(w >> 1);
    wait_lgkm0();
    lds_barrier();
    if (w == 0 || w == 2) fold(w >> 1);
    if (w == 2) put(1);
    wait_lgkm0();
    lds_barrier();
    if (w == 0) fold(1);
    // Slot 1 is written again by wave 3 before the next item's first barrier (at once, when it
    // has no group of that item): every wave waits here until wave 0 has read it.
    wait_lgkm0();
    lds_barrier();
    if (w == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int col = nt * 16 + col_lo;
        if (col < R) {
          const float inv = (lt[nt] > 0.f) ? 1.0f / lt[nt] : 0.f;
          const int t = col / G, gh = col % G;
          const int pidx = cur.base + t * cur.n_b + c;
          const int h = kvh * G + gh;
          float* dst = p.o_part + ((size_t)pidx * p.hq + h) * kHeadDim + 4 * grp;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) *reinterpret_cast<f32x4*>(dst + dt * 16) = o[nt][dt] * inv;
          if (grp == 0)
            p.lse_part[(size_t)pidx * p.hq + h] =
                (m[nt] == kNegInf || !(lt[nt] > 0.f)) ? kNegInf : (m[nt] + fast_log2(lt[nt])) * kLn2;
        }
      }
    }
    // Slot 0 is read by wave 0 before the second barrier and written next by wave 1 before the
    // next item's first barrier, which wave 1 reaches only after that second barrier; slot 1 is
    // free once the third barrier is passed.
    cur = nxt;
    pid = pid_next;
    pid_seg = 0;
    n_mine = n_mine_next;
    n_pref = n_pref_next;
  }
}

namespace {
template <int NT, bool TREE>
int resident_blocks_per_cu() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_split_kernel<NT, TREE>, kThreads, 0) != hipSuccess || n < 1)
    n = 1;
  return n;
}

struct DeviceShape {
  int cus = 0;
  int blocks_per_cu[2][5] = {{0, 0, 0, 0, 0}, {0, 0, 0, 0, 0}};  // [tree][column tiles]
};

// Per-device launch shape, computed once per device from host-side queries (call_once: the
// library may be called from several host threads).
const DeviceShape& device_shape() {
  static DeviceShape shapes[64];
  static std::once_flag once[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  DeviceShape& s = shapes[dev];
  std::call_once(once[dev], [&]() {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    s.blocks_per_cu[0][1] = resident_blocks_per_cu<1, false>();
    s.blocks_per_cu[0][2] = resident_blocks_per_cu<2, false>();
    s.blocks_per_cu[0][3] = resident_blocks_per_cu<3, false>();
    s.blocks_per_cu[0][4] = resident_blocks_per_cu<4, false>();
    s.blocks_per_cu[1][1] = resident_blocks_per_cu<1, true>();
    s.blocks_per_cu[1][2] = resident_blocks_per_cu<2, true>();
    s.blocks_per_cu[1][3] = resident_blocks_per_cu<3, true>();
    s.blocks_per_cu[1][4] = resident_blocks_per_cu<4, true>();
    s.cus = cus;
  });
  return s;
}
}  // namespace

int decode_resident_workgroups(int column_tiles, bool tree) {
  if (column_tiles < 1 || column_tiles > 4) return 0;
  const DeviceShape& ds = device_shape();
  return ds.cus * ds.blocks_per_cu[tree ? 1 : 0][column_tiles];
}

hipError_t launch_decode_split(const DecodeParams& p, int max_chunks, hipStream_t stream) {
  const int R = p.q_len * p.group;
  const int nt = (R + 15) / 16;
  if (nt < 1 || nt > 4) return hipErrorInvalidValue;
  const DeviceShape& ds = device_shape();
  const bool tree = p.tree_mask != nullptr;
  // Persistent grid: enough workgroups to fill every CU, never more than the item bound.
  const long item_bound = (long)max_chunks * p.batch * p.hkv;
  long blocks = (long)ds.cus * ds.blocks_per_cu[tree ? 1 : 0][nt];
  if (blocks > item_bound) blocks = item_bound;
  if (blocks < 1) blocks = 1;
  dim3 grid((unsigned)blocks), block(kThreads);
  if (tree) {
    switch (nt) {
      case 1: hipLaunchKernelGGL((decode_split_kernel<1, true>), grid, block, 0, stream, p); break;
      case 2: hipLaunchKernelGGL((decode_split_kernel<2, true>), grid, block, 0, stream, p); break;
      case 3: hipLaunchKernelGGL((decode_split_kernel<3, true>), grid, block, 0, stream, p); break;
      default: hipLaunchKernelGGL((decode_split_kernel<4, true>), grid, block, 0, stream, p); break;
    }
  } else {
    switch (nt) {
      case 1: hipLaunchKernelGGL((decode_split_kernel<1, false>), grid, block, 0, stream, p); break;
      case 2: hipLaunchKernelGGL((decode_split_kernel<2, false>), grid, block, 0, stream, p); break;
      case 3: hipLaunchKernelGGL((decode_split_kernel<3, false>), grid, block, 0, stream, p); break;
      default: hipLaunchKernelGGL((decode_split_kernel<4, false>), grid, block, 0, stream, p); break;
    }
  }
  return hipGetLastError();
}

}  // namespace attn_sink
