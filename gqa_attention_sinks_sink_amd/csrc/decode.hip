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
//     are cut into 32-key steps dealt round-robin to the 4 waves; a step is two 16-key
//     groups, each inside one page.
//   * Per step: K goes from HBM straight into registers in the MFMA A layout; S^T = K Q^T
//     with v_mfma_f32_16x16x32_bf16; masks from indices; online softmax in the exp2
//     domain; V rows pass through LDS and come back transposed (ds_read_b64_tr_b16) as
//     the A operand of O^T += V^T P^T.
//   * The 4 wave states are combined in LDS in a fixed order (bit-reproducible) and the
//     chunk partial (o/d, m + ln d) goes to the workspace at the plan's offset.
#include "common.hpp"
#include "kernels.hpp"

namespace attn_sink {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kVRowBytes = 160;               // padded LDS row of V (64 bf16 = 128 B + 32)
constexpr int kVWaveBytes = 32 * kVRowBytes;  // 32 keys per wave step
constexpr int kSegKeys = 1024;                // keys whose page ids one wave holds (64 lanes x 16)
constexpr float kLazyMax = 8.0f;              // running-max slack (log2 units) before a rescale

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

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  return v;
}

// Element offset of the K/V row (page, kv head, slot) in the cache.
__device__ __forceinline__ size_t cache_row(const DecodeParams& p, int page, int kvh, int slot) {
  return (((size_t)page * p.hkv + kvh) * p.page_size + slot) * (size_t)kHeadDim;
}

}  // namespace

// Resident waves per SIMD and steps of loads in flight per wave, per column-tile count
// (measured on MI355X). With one tile (single-token decode) the step math is short and 4
// waves per SIMD with one step each stream best; with more tiles the step math is longer,
// so each wave keeps two steps in flight and the register budget sets the occupancy.
template <int NT>
struct DecodeOccupancy { static constexpr int value = 1; };
template <> struct DecodeOccupancy<1> { static constexpr int value = 4; };
template <> struct DecodeOccupancy<2> { static constexpr int value = 2; };
template <> struct DecodeOccupancy<3> { static constexpr int value = 2; };
template <> struct DecodeOccupancy<4> { static constexpr int value = 1; };
template <int NT>
constexpr int kStepsInFlight = (NT == 1) ? 1 : 2;

template <int NT>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(DecodeOccupancy<NT>::value, DecodeOccupancy<NT>::value)))
void decode_split_kernel(DecodeParams p) {
  // Per-wave LDS region: V staging of a step, then the wave's O^T for the combine.
  constexpr int kWaveRegion = (kVWaveBytes > NT * 16 * kHeadDim * 4) ? kVWaveBytes : NT * 16 * kHeadDim * 4;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kWaves * kWaveRegion];
  __shared__ float red_m[kWaves][NT * 16];
  __shared__ float red_l[kWaves][NT * 16];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int G = p.group;
  const int R = p.q_len * G;  // live columns
  const int col_lo = lane & 15;
  const int grp = lane >> 4;  // 16-lane group 0..3
  unsigned char* vl = lds + w * kWaveRegion;

  // ---- total number of (sequence, chunk) pairs, and a cursor over sequences
  int tot = 0;
  for (int i = lane; i < p.batch; i += 64) tot += chunks_for(seq_len_clamped(p, i), p.kv_chunk);
  const int total_items = wave_sum_int(tot) * p.hkv;

  int cur_base = 0;    // first sequence of the cursor window
  int cur_before = 0;  // pairs before cur_base
  int win_incl = 0;    // inclusive prefix of chunk counts inside the window (this lane's sequence)
  int win_total = 0;
  auto load_window = [&]() {
    const int i = cur_base + lane;
    const int n = (i < p.batch) ? chunks_for(seq_len_clamped(p, i), p.kv_chunk) : 0;
    win_incl = wave_inclusive_scan(n, lane);
    win_total = __builtin_amdgcn_readlane(win_incl, 63);
  };
  load_window();

  for (int item = blockIdx.x; item < total_items; item += gridDim.x) {
    const int P = item / p.hkv;
    const int kvh = item - P * p.hkv;
    while (P >= cur_before + win_total) {
      cur_before += win_total;
      cur_base += 64;
      load_window();
    }
    const unsigned long long before_mask = __ballot(cur_before + win_incl <= P);
    const int idx = __popcll(before_mask);
    const int b = cur_base + idx;
    const int pairs_before = cur_before + (idx > 0 ? __builtin_amdgcn_readlane(win_incl, idx - 1) : 0);
    const int c = P - pairs_before;

    const int L = seq_len_clamped(p, b);
    const int n_b = chunks_for(L, p.kv_chunk);
    const int base = pairs_before * p.q_len;  // indptr of row b*q_len
    const int chunk_lo = c * p.kv_chunk;
    const int chunk_hi = min(chunk_lo + p.kv_chunk, L);
    const int* ptab = p.page_table + (size_t)b * p.max_pages;

    // Page ids of up to 64 16-key groups (one per lane) for a segment of <= 1024 keys.
    auto load_page_ids = [&](int seg_lo, int seg_hi) -> int {
      const int j = seg_lo + 16 * lane;
      int pg = 0;
      if (j < seg_hi) pg = clampi(ptab[j >> p.page_shift], 0, p.num_pages - 1);
      return pg;
    };
    int pid = load_page_ids(chunk_lo, min(chunk_lo + kSegKeys, chunk_hi));

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

    // ---- keys visible to each column inside this chunk: [vis_lo, vis_hi); wave-wide bounds
    // decide whether a step needs masking at all.
    int vis_lo[NT], vis_hi[NT];
    int hi_min = 0x7fffffff, lo_max = -0x7fffffff;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      vis_hi[nt] = p.causal ? min(chunk_hi, pos[nt] + 1) : chunk_hi;
      vis_lo[nt] = (p.window > 0) ? max(chunk_lo, pos[nt] - p.window + 1) : chunk_lo;
      if (vis_hi[nt] < vis_lo[nt]) vis_hi[nt] = vis_lo[nt];
      if (nt * 16 + col_lo < R) {
        hi_min = min(hi_min, vis_hi[nt]);
        lo_max = max(lo_max, vis_lo[nt]);
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      hi_min = min(hi_min, __shfl_xor(hi_min, off, 64));
      lo_max = max(lo_max, __shfl_xor(lo_max, off, 64));
    }
    const int vis_hi_min = hi_min, vis_lo_max = lo_max;

    // ---- online-softmax state per lane: m (exp2 domain, same across the 4 lane groups of a
    // column), a partial row sum, and O^T tiles (d = dt*16 + 4*grp + i, column nt*16 + col_lo).
    float m[NT], lsum[NT];
    f32x4 o[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int col = nt * 16 + col_lo;
      const int h = kvh * G + (col < R ? col % G : 0);
      // First chunk: the running max starts at the head's sink and d at 1 (held by lane group
      // 0 so the column sum counts it once). Other chunks and waves: m = -inf (d = 1 is inert).
      const float sink2 = (p.sinks != nullptr) ? p.sinks[h] * kLog2e : kNegInf;
      m[nt] = (c == 0 && w == 0) ? sink2 : kNegInf;
      lsum[nt] = (grp == 0) ? 1.0f : 0.0f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[nt][dt] = f32x4{0, 0, 0, 0};
    }

    for (int seg_lo = chunk_lo; seg_lo < chunk_hi; seg_lo += kSegKeys) {
      const int seg_hi = min(seg_lo + kSegKeys, chunk_hi);
      if (seg_lo != chunk_lo) pid = load_page_ids(seg_lo, seg_hi);
      const int n_steps = (seg_hi - seg_lo + 31) / 32;
        // ---- load: K straight to registers (row = key, k = head-dim slice), V rows for LDS.
        // Loads are unconditional: a missing second group re-reads the first group's page and
        // tail keys read slots of an allocated page; their scores are masked and their V rows
        // zeroed before use.
        auto issue_loads = [&](int s, u32x4 (&kr)[4], u32x4 (&vr)[4]) {
          const int j0 = seg_lo + 32 * s;
          const bool hasB = (j0 + 16) < seg_hi;
          const int pa = __builtin_amdgcn_readlane(pid, 2 * s);
          const int pb = __builtin_amdgcn_readlane(pid, 2 * s + 1);
          const size_t rA = cache_row(p, pa, kvh, j0 & (p.page_size - 1));
          const size_t rB = hasB ? cache_row(p, pb, kvh, (j0 + 16) & (p.page_size - 1)) : rA;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            kr[ks] = *reinterpret_cast<const u32x4*>(p.k_cache + rA + (size_t)col_lo * kHeadDim + ks * 32 + grp * 8);
            kr[2 + ks] = *reinterpret_cast<const u32x4*>(p.k_cache + rB + (size_t)col_lo * kHeadDim + ks * 32 + grp * 8);
          }
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int krow = (lane >> 3) + 8 * ii;  // 0..31
            const size_t rr = (krow < 16) ? rA : rB;
            vr[ii] = *reinterpret_cast<const u32x4*>(p.v_cache + rr + (size_t)(krow & 15) * kHeadDim + (lane & 7) * 8);
          }
        };
        auto run_step = [&](int s, const u32x4 (&kr)[4], u32x4 (&vr)[4]) {
        const int j0 = seg_lo + 32 * s;
        if (j0 + 32 > seg_hi) {
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int krow = (lane >> 3) + 8 * ii;
            if (j0 + krow >= seg_hi) vr[ii] = u32x4{0, 0, 0, 0};  // keys past the range: exact zeros
          }
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int krow = (lane >> 3) + 8 * ii;
          *reinterpret_cast<u32x4*>(vl + krow * kVRowBytes + (lane & 7) * 16) = vr[ii];
        }

        // ---- S^T tiles: 16 keys x 16 columns per (group, nt)
        f32x4 sc[NT][2];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            f32x4 a = f32x4{0, 0, 0, 0};
            a = mfma16(as_bf16x8(kr[2 * g]), as_bf16x8(qb[nt][0]), a);
            a = mfma16(as_bf16x8(kr[2 * g + 1]), as_bf16x8(qb[nt][1]), a);
            sc[nt][g] = a;
          }
        }

        // ---- masks (only on steps that straddle a bound) + online softmax update.
        // The running max m is lazy: it moves only when some score exceeds it by more than
        // kLazyMax (log2 units), so most steps need neither a cross-lane reduction nor a rescale
        // of O; every term of a column always uses that column's current m, so the result is
        // the same softmax (terms are at most 2^kLazyMax before the final division).
        const bool full_step = (j0 + 32 <= vis_hi_min) && (j0 >= vis_lo_max);
        if (!full_step) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const unsigned span = (unsigned)(vis_hi[nt] - vis_lo[nt]);
#pragma unroll
            for (int g = 0; g < 2; ++g) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int key = j0 + g * 16 + grp * 4 + i;
                sc[nt][g][i] = ((unsigned)(key - vis_lo[nt]) < span) ? sc[nt][g][i] : kNegInf;
              }
            }
          }
        }
        bool bump = false;
        float mx[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float v = fmaxf(fmaxf(sc[nt][0][0], sc[nt][0][1]), fmaxf(sc[nt][0][2], sc[nt][0][3]));
          v = fmaxf(v, fmaxf(fmaxf(sc[nt][1][0], sc[nt][1][1]), fmaxf(sc[nt][1][2], sc[nt][1][3])));
          mx[nt] = v * p.scale_log2;
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
        bf16x8 pbf[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float neg_m = (m[nt] == kNegInf) ? 0.0f : -m[nt];
          float ps = 0.f;
          uint32_t packed[4];
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            float e[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              e[i] = fast_exp2(__builtin_fmaf(sc[nt][g][i], p.scale_log2, neg_m));
              ps += e[i];
            }
            packed[g * 2 + 0] = pack_bf16x2(e[0], e[1]);
            packed[g * 2 + 1] = pack_bf16x2(e[2], e[3]);
          }
          lsum[nt] += ps;
          pbf[nt] = as_bf16x8(u32x4{packed[0], packed[1], packed[2], packed[3]});
        }

        // ---- O^T += V^T P^T. A operand (V^T): lane = d (dt*16 + col_lo), k slots 0..3 =
        // group A keys 4*grp..+3, slots 4..7 = group B keys 4*grp..+3 (the P layout above).
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int rsel = grp * 4 + (col_lo >> 2);
          const int csel = dt * 16 + 4 * (col_lo & 3);
          const s16x4 lo = lds_read_tr16(vl + rsel * kVRowBytes + csel * 2);
          const s16x4 hi = lds_read_tr16(vl + (16 + rsel) * kVRowBytes + csel * 2);
          const u32x4 av = join_tr16(lo, hi);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) o[nt][dt] = mfma16(as_bf16x8(av), pbf[nt], o[nt][dt]);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        };

        // This wave owns steps w, w + 4, w + 8, ... of the segment, with two steps in
        // flight (ping-pong register buffers): the loads of step k + 1 are issued before
        // step k is computed.
        const int n_mine = (w < n_steps) ? (n_steps - w + kWaves - 1) / kWaves : 0;
        if constexpr (kStepsInFlight<NT> == 1) {
          for (int k = 0; k < n_mine; ++k) {
            u32x4 kA[4], vA[4];
            issue_loads(w + kWaves * k, kA, vA);
            run_step(w + kWaves * k, kA, vA);
          }
        } else {
          // The steady-state loop issues its loads unconditionally, so the compiler waits for
          // exactly the older step's loads (a conditional load makes it wait for all of them).
          u32x4 kA[4], vA[4], kB[4], vB[4];
          int k = 0;
          if (n_mine > 0) issue_loads(w, kA, vA);
          for (; k + 2 < n_mine; k += 2) {
            issue_loads(w + kWaves * (k + 1), kB, vB);
            run_step(w + kWaves * k, kA, vA);
            issue_loads(w + kWaves * (k + 2), kA, vA);
            run_step(w + kWaves * (k + 1), kB, vB);
          }
          if (k + 1 < n_mine) {
            issue_loads(w + kWaves * (k + 1), kB, vB);
            run_step(w + kWaves * k, kA, vA);
            run_step(w + kWaves * (k + 1), kB, vB);
          } else if (k < n_mine) {
            run_step(w + kWaves * k, kA, vA);
          }
        }
    }

    // ---- plan: chunk counts and partial offsets (one writer per sequence)
    if (c == 0 && kvh == 0 && w == 0) {
      if (lane < p.q_len) {
        p.counts[b * p.q_len + lane] = n_b;
        p.indptr[b * p.q_len + lane] = base + lane * n_b;
      }
      if (b == p.batch - 1 && lane == 0) p.indptr[p.batch * p.q_len] = base + p.q_len * n_b;
    }

    // ---- combine the 4 wave states of this chunk. Each wave leaves its (m, d) per column and
    // its unnormalised O^T in its own LDS region (which held its V staging); after one
    // barrier every thread merges 4 columns x 4 head-dim values over the waves in a fixed
    // order (bit-reproducible) and writes the chunk partial: o_c = O / d, lse_c = m + ln d.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float lt = lsum[nt];
      lt += shfl_xor(lt, 16);
      lt += shfl_xor(lt, 32);
      if (grp == 0) {
        red_m[w][nt * 16 + col_lo] = m[nt];
        red_l[w][nt * 16 + col_lo] = lt;
      }
      float* slot = reinterpret_cast<float*>(vl);  // [NT*16 columns][64 d]
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        *reinterpret_cast<f32x4*>(&slot[(nt * 16 + col_lo) * kHeadDim + dt * 16 + grp * 4]) = o[nt][dt];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < R * (kHeadDim / 4); i += kThreads) {
      const int col = i / (kHeadDim / 4);
      const int d4 = (i % (kHeadDim / 4)) * 4;
      float M = kNegInf;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, red_m[ww][col]);
      const float Mu = (M == kNegInf) ? 0.f : M;
      float Lt = 0.f;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float sc = fast_exp2(red_m[ww][col] - Mu);
        Lt += red_l[ww][col] * sc;
        const float* slot = reinterpret_cast<const float*>(lds + ww * kWaveRegion);
        acc += *reinterpret_cast<const f32x4*>(&slot[col * kHeadDim + d4]) * sc;
      }
      const float inv = (Lt > 0.f) ? 1.0f / Lt : 0.f;
      const int t = col / G, gh = col % G;
      const int pidx = base + t * n_b + c;
      const int h = kvh * G + gh;
      *reinterpret_cast<f32x4*>(p.o_part + ((size_t)pidx * p.hq + h) * kHeadDim + d4) = acc * inv;
      if (d4 == 0) p.lse_part[(size_t)pidx * p.hq + h] = (M == kNegInf || !(Lt > 0.f)) ? kNegInf : (M + fast_log2(Lt)) * kLn2;
    }
    __syncthreads();  // the LDS regions and red_* are reused by the next item
  }
}

namespace {
template <int NT>
int resident_blocks_per_cu() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_split_kernel<NT>, kThreads, 0) != hipSuccess || n < 1)
    n = 1;
  return n;
}

struct DeviceShape {
  int cus = 0;
  int blocks_per_cu[5] = {0, 0, 0, 0, 0};
};

// Per-device launch shape, computed once per device from host-side queries.
const DeviceShape& device_shape() {
  static DeviceShape shapes[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  DeviceShape& s = shapes[dev];
  if (s.cus == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    s.blocks_per_cu[1] = resident_blocks_per_cu<1>();
    s.blocks_per_cu[2] = resident_blocks_per_cu<2>();
    s.blocks_per_cu[3] = resident_blocks_per_cu<3>();
    s.blocks_per_cu[4] = resident_blocks_per_cu<4>();
    s.cus = cus;
  }
  return s;
}
}  // namespace

hipError_t launch_decode_split(const DecodeParams& p, int max_chunks, hipStream_t stream) {
  const int R = p.q_len * p.group;
  const int nt = (R + 15) / 16;
  if (nt < 1 || nt > 4) return hipErrorInvalidValue;
  const DeviceShape& ds = device_shape();
  // Persistent grid: enough workgroups to fill every CU, never more than the item bound.
  const long item_bound = (long)max_chunks * p.batch * p.hkv;
  long blocks = (long)ds.cus * ds.blocks_per_cu[nt];
  if (blocks > item_bound) blocks = item_bound;
  if (blocks < 1) blocks = 1;
  dim3 grid((unsigned)blocks), block(kThreads);
  switch (nt) {
    case 1: hipLaunchKernelGGL(decode_split_kernel<1>, grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL(decode_split_kernel<2>, grid, block, 0, stream, p); break;
    case 3: hipLaunchKernelGGL(decode_split_kernel<3>, grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL(decode_split_kernel<4>, grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace attn_sink
