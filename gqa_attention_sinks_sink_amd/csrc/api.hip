// C ABI of libattnsink.so: argument validation, workspace layout and kernel launches.
// Every check runs on the host before anything is enqueued; nothing here allocates,
// frees or synchronises.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <mutex>
#include <vector>

#include "../../include/attn_sink.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace attn_sink;

namespace {

constexpr int32_t kSupportedHeadDim = 64;
constexpr int32_t kMaxQLen = 8;
constexpr int32_t kMaxColumns = 64;   // q_len * (num_q_heads / num_kv_heads) per decode workgroup
// Fixed cost of one split-KV work item (plan, combine, partial, its share of the merge), in
// keys: fitted to whole-call times of the verify-shaped workloads over chunk lengths 1024-4096.
constexpr int64_t kPlanItemKeys = 1024;
// Cost of one merge round trip (16 partials of a row), in keys: the merge lasts as long as its
// row with the most partials. Fitted to whole-call times over batch 1-64, lengths 2048-32768.
constexpr int64_t kPlanMergeKeys = 384;
constexpr int64_t kMaxGridY = 65535;

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
// The kernels move bf16 rows and fp32 partials in 16-byte pieces.
inline bool misaligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) != 0; }

inline bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

// A sequence's capacity in tokens (its page-table row times the page size) is an int32 in the
// kernels, which bound every sequence length by it.
inline bool capacity_fits(int32_t max_pages_per_seq, int32_t page_size) {
  return (int64_t)max_pages_per_seq * page_size <= INT32_MAX;
}

inline int32_t ilog2(int32_t x) {
  int32_t s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

// Effective chunk length: kv_chunk if positive, else one chunk covering max_kv_len (rounded
// up to the kernel's 64-key granularity and to whole pages).
inline int64_t effective_chunk(int32_t kv_chunk, int32_t max_kv_len, int32_t page_size) {
  if (kv_chunk > 0) return kv_chunk;
  int64_t g = page_size > 64 ? page_size : 64;
  int64_t L = max_kv_len > 0 ? max_kv_len : 1;
  return ((L + g - 1) / g) * g;
}

struct DecodeLayout {
  int64_t rows, chunks, partials;
  size_t off_indptr, off_counts, off_o, off_lse, total;
};

inline bool decode_layout(int32_t batch, int32_t q_len, int32_t max_kv_len, int32_t num_q_heads,
                          int64_t chunk, DecodeLayout* out) {
  if (batch < 0 || q_len < 1 || max_kv_len < 0 || num_q_heads <= 0 || chunk <= 0) return false;
  DecodeLayout l;
  l.rows = (int64_t)batch * q_len;
  l.chunks = (max_kv_len + chunk - 1) / chunk;
  if (l.chunks < 1) l.chunks = 1;
  l.partials = l.rows * l.chunks;
  if (l.partials > INT32_MAX / 2) return false;
  l.off_indptr = 0;
  l.off_counts = align256(sizeof(int32_t) * (size_t)(l.rows + 1));
  l.off_o = l.off_counts + align256(sizeof(int32_t) * (size_t)l.rows);
  l.off_lse = l.off_o + align256(sizeof(float) * (size_t)l.partials * num_q_heads * kSupportedHeadDim);
  l.total = l.off_lse + align256(sizeof(float) * (size_t)l.partials * num_q_heads);
  *out = l;
  return true;
}

// Scratch of attn_sink_decode_paged_noalloc (the plan and the chunk partials of one call), in
// device memory the library owns: each GPU the library runs on holds its own copy until the
// process ends. Host code never uses the array's name as an address: the device address comes
// from hipGetSymbolAddress, once per device with that device current.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of the current device's scratch (looked up on the first call on that device).
hipError_t current_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&]() {
    void* ptr = nullptr;
    slot.err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (slot.err == hipSuccess && ptr == nullptr) slot.err = hipErrorInvalidSymbol;
    slot.ptr = ptr;
  });
  if (slot.err != hipSuccess) return slot.err;
  *out = slot.ptr;
  return hipSuccess;
}

// Launchers return hipErrorInvalidConfiguration for a grid beyond the launch limits.
inline attn_sink_status hip_status(hipError_t e) {
  if (e == hipSuccess) return ATTN_SINK_OK;
  return e == hipErrorInvalidConfiguration ? ATTN_SINK_ERR_UNSUPPORTED : ATTN_SINK_ERR_HIP;
}

}  // namespace

extern "C" {

const char* attn_sink_status_string(attn_sink_status status) {
  switch (status) {
    case ATTN_SINK_OK: return "ok";
    case ATTN_SINK_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_SINK_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_SINK_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case ATTN_SINK_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

const char* attn_sink_version(void) { return "attn_sink 0.1.0 gfx950"; }

attn_sink_status attn_sink_prefill(const void* q, const void* k, const void* v, const float* sinks,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int32_t batch,
                                   int32_t total_q, int32_t total_kv, int32_t max_seqlen_q, int32_t max_seqlen_kv,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
                                   int32_t causal, int32_t window, void* out, float* lse, void* stream) {
  if (batch < 0 || total_q < 0 || total_kv < 0 || max_seqlen_q < 0 || max_seqlen_kv < 0) return ATTN_SINK_ERR_INVALID_ARG;
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return ATTN_SINK_ERR_INVALID_ARG;
  if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f)) return ATTN_SINK_ERR_INVALID_ARG;
  if (head_dim != kSupportedHeadDim) return ATTN_SINK_ERR_UNSUPPORTED;
  if (batch == 0 || total_q == 0 || max_seqlen_q == 0) return ATTN_SINK_OK;
  if (q == nullptr || out == nullptr || cu_seqlens_q == nullptr || cu_seqlens_kv == nullptr) return ATTN_SINK_ERR_INVALID_ARG;
  if (total_kv > 0 && (k == nullptr || v == nullptr)) return ATTN_SINK_ERR_INVALID_ARG;
  if (misaligned16(q) || misaligned16(k) || misaligned16(v) || misaligned16(out)) return ATTN_SINK_ERR_INVALID_ARG;
  // Q, K and V of one sequence are addressed with 32-bit byte offsets.
  if ((int64_t)max_seqlen_kv * num_kv_heads * kSupportedHeadDim * 2 + 64ll * num_kv_heads * kSupportedHeadDim * 2 > INT32_MAX)
    return ATTN_SINK_ERR_UNSUPPORTED;
  if ((int64_t)max_seqlen_q * num_q_heads * kSupportedHeadDim * 2 > INT32_MAX) return ATTN_SINK_ERR_UNSUPPORTED;
  const int32_t group = num_q_heads / num_kv_heads;
  const int32_t gp = prefill_heads_per_tile(group);
  const int64_t tok = 128 * prefill_row_blocks(max_seqlen_q, gp) / gp;  // query tokens per workgroup
  const int64_t tiles = ((int64_t)max_seqlen_q + tok - 1) / tok;
  if (tiles * batch * num_kv_heads * (group / gp) + 8 > INT32_MAX) return ATTN_SINK_ERR_UNSUPPORTED;

  PrefillParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.sinks = sinks;
  p.cu_q = cu_seqlens_q;
  p.cu_kv = cu_seqlens_kv;
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.batch = batch;
  p.total_q = total_q;
  p.total_kv = total_kv;
  p.max_q = max_seqlen_q;
  p.max_kv = max_seqlen_kv;
  p.hq = num_q_heads;
  p.hkv = num_kv_heads;
  p.group = group;
  p.causal = causal != 0;
  p.window = window > 0 ? window : 0;
  p.scale_log2 = softmax_scale * kLog2e;
  return hip_status(launch_prefill(p, reinterpret_cast<hipStream_t>(stream)));
}

attn_sink_status attn_sink_prefill_paged(const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* page_table, int32_t max_pages_per_seq, int32_t num_pages,
                                         const int32_t* cu_seqlens_q, const int32_t* kv_lens, const float* sinks,
                                         int32_t batch, int32_t total_q, int32_t max_seqlen_q, int32_t max_kv_len,
                                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                         int32_t page_size, float softmax_scale, int32_t causal, int32_t window,
                                         void* out, float* lse, void* stream) {
  if (batch < 0 || total_q < 0 || max_seqlen_q < 0 || max_kv_len < 0 || max_pages_per_seq < 1 || num_pages < 1)
    return ATTN_SINK_ERR_INVALID_ARG;
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return ATTN_SINK_ERR_INVALID_ARG;
  if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f)) return ATTN_SINK_ERR_INVALID_ARG;
  if (head_dim != kSupportedHeadDim) return ATTN_SINK_ERR_UNSUPPORTED;
  if (!is_pow2(page_size) || page_size < 16 || page_size > 256) return ATTN_SINK_ERR_UNSUPPORTED;
  if (!capacity_fits(max_pages_per_seq, page_size)) return ATTN_SINK_ERR_UNSUPPORTED;
  if (batch == 0 || total_q == 0 || max_seqlen_q == 0) return ATTN_SINK_OK;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || page_table == nullptr || kv_lens == nullptr ||
      cu_seqlens_q == nullptr || out == nullptr)
    return ATTN_SINK_ERR_INVALID_ARG;
  if (misaligned16(q) || misaligned16(k_cache) || misaligned16(v_cache) || misaligned16(out))
    return ATTN_SINK_ERR_INVALID_ARG;
  // One sequence's Q rows are addressed with 32-bit byte offsets.
  if ((int64_t)max_seqlen_q * num_q_heads * kSupportedHeadDim * 2 > INT32_MAX) return ATTN_SINK_ERR_UNSUPPORTED;
  const int32_t group = num_q_heads / num_kv_heads;
  const int32_t gp = prefill_heads_per_tile(group);
  const int64_t tok = 128 * prefill_row_blocks(max_seqlen_q, gp) / gp;
  const int64_t tiles = ((int64_t)max_seqlen_q + tok - 1) / tok;
  if (tiles * batch * num_kv_heads * (group / gp) + 8 > INT32_MAX) return ATTN_SINK_ERR_UNSUPPORTED;

  PrefillParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k_cache);
  p.v = static_cast<const uint16_t*>(v_cache);
  p.sinks = sinks;
  p.cu_q = cu_seqlens_q;
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.batch = batch;
  p.total_q = total_q;
  p.max_q = max_seqlen_q;
  p.max_kv = max_kv_len;
  p.hq = num_q_heads;
  p.hkv = num_kv_heads;
  p.group = group;
  p.causal = causal != 0;
  p.window = window > 0 ? window : 0;
  p.scale_log2 = softmax_scale * kLog2e;
  p.page_table = page_table;
  p.kv_lens = kv_lens;
  p.max_pages = max_pages_per_seq;
  p.num_pages = num_pages;
  p.page_size = page_size;
  p.page_shift = ilog2(page_size);
  return hip_status(launch_prefill(p, reinterpret_cast<hipStream_t>(stream)));
}

attn_sink_status attn_sink_rope_append(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                                       const int32_t* kv_lens, const int32_t* page_table, int32_t max_pages_per_seq,
                                       int32_t num_pages, void* k_cache, void* v_cache, int32_t batch, int32_t total_q,
                                       int32_t max_seqlen_q, int32_t max_kv_len, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t page_size, float rope_theta,
                                       float yarn_factor, int32_t yarn_original_len, float yarn_alpha,
                                       float yarn_beta, int32_t yarn_ramp, void* q_out, void* stream) {
  if (batch < 0 || total_q < 0 || max_seqlen_q < 0 || max_kv_len < 0 || max_pages_per_seq < 1 || num_pages < 1)
    return ATTN_SINK_ERR_INVALID_ARG;
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return ATTN_SINK_ERR_INVALID_ARG;
  if (!(std::isfinite(rope_theta) && rope_theta > 1.f) || !(std::isfinite(yarn_factor) && yarn_factor > 0.f))
    return ATTN_SINK_ERR_INVALID_ARG;
  if (yarn_factor > 1.f && !(yarn_original_len > 0 && std::isfinite(yarn_alpha) && std::isfinite(yarn_beta) &&
                             yarn_alpha < yarn_beta))
    return ATTN_SINK_ERR_INVALID_ARG;
  if (yarn_ramp != ATTN_SINK_YARN_RAMP_TURNS && yarn_ramp != ATTN_SINK_YARN_RAMP_INDEX) return ATTN_SINK_ERR_INVALID_ARG;
  if (yarn_factor > 1.f && yarn_ramp == ATTN_SINK_YARN_RAMP_INDEX && !(yarn_alpha > 0.f)) return ATTN_SINK_ERR_INVALID_ARG;
  if (head_dim != kSupportedHeadDim) return ATTN_SINK_ERR_UNSUPPORTED;
  if (!is_pow2(page_size) || page_size < 16 || page_size > 256) return ATTN_SINK_ERR_UNSUPPORTED;
  if (!capacity_fits(max_pages_per_seq, page_size)) return ATTN_SINK_ERR_UNSUPPORTED;
  if (batch > kMaxGridY) return ATTN_SINK_ERR_UNSUPPORTED;
  if (batch == 0 || total_q == 0 || max_seqlen_q == 0) return ATTN_SINK_OK;
  if (q == nullptr || k == nullptr || v == nullptr || cu_seqlens_q == nullptr || kv_lens == nullptr ||
      page_table == nullptr || k_cache == nullptr || v_cache == nullptr || q_out == nullptr)
    return ATTN_SINK_ERR_INVALID_ARG;
  if (misaligned16(q) || misaligned16(k) || misaligned16(v) || misaligned16(k_cache) || misaligned16(v_cache) ||
      misaligned16(q_out))
    return ATTN_SINK_ERR_INVALID_ARG;

  RopeParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.cu_q = cu_seqlens_q;
  p.kv_lens = kv_lens;
  p.page_table = page_table;
  p.k_cache = static_cast<uint16_t*>(k_cache);
  p.v_cache = static_cast<uint16_t*>(v_cache);
  p.q_out = static_cast<uint16_t*>(q_out);
  p.batch = batch;
  p.total_q = total_q;
  p.max_q = max_seqlen_q;
  p.max_kv = max_kv_len;
  p.hq = num_q_heads;
  p.hkv = num_kv_heads;
  p.max_pages = max_pages_per_seq;
  p.num_pages = num_pages;
  p.page_size = page_size;
  p.page_shift = ilog2(page_size);
  // YaRN: base frequencies theta^(-2i/d); with factor s > 1, a ramp over the turns r_i each
  // pair makes in the original context keeps fast pairs (r >= beta), divides slow ones
  // (r <= alpha) by s and blends in between, linearly in r or in ln r (the pair index); the
  // temperature 0.1 ln s + 1 scales cos and sin.
  const double pi2 = 6.283185307179586;
  for (int i = 0; i < kSupportedHeadDim / 2; ++i) {
    const double f = std::pow((double)rope_theta, -2.0 * i / kSupportedHeadDim);
    double fi = f;
    if (yarn_factor > 1.f) {
      const double r = (double)yarn_original_len * f / pi2;
      const double t = (yarn_ramp == ATTN_SINK_YARN_RAMP_TURNS)
                           ? (r - yarn_alpha) / ((double)yarn_beta - yarn_alpha)
                           : std::log(r / yarn_alpha) / std::log((double)yarn_beta / yarn_alpha);
      const double g = std::min(1.0, std::max(0.0, t));
      fi = g * f + (1.0 - g) * f / yarn_factor;
    }
    p.freqs[i] = fi;
  }
  p.mscale = yarn_factor > 1.f ? (float)(0.1 * std::log((double)yarn_factor) + 1.0) : 1.f;
  return hip_status(launch_rope_append(p, reinterpret_cast<hipStream_t>(stream)));
}

size_t attn_sink_decode_workspace_size(int32_t batch, int32_t q_len, int32_t max_kv_len, int32_t num_q_heads,
                                       int32_t head_dim, int32_t kv_chunk) {
  if (head_dim != kSupportedHeadDim) return 0;
  DecodeLayout l;
  // The page size only rounds the single-chunk length up; it never changes the chunk count.
  if (!decode_layout(batch, q_len, max_kv_len, num_q_heads, effective_chunk(kv_chunk, max_kv_len, 16), &l)) return 0;
  return l.total;
}

attn_sink_status attn_sink_decode_plan_chunk(const int32_t* kv_lens, int32_t batch, int32_t q_len,
                                             int32_t num_q_heads, int32_t num_kv_heads, int32_t page_size,
                                             int32_t workgroups, int32_t* kv_chunk) {
  if (kv_chunk == nullptr || batch < 0 || q_len < 1) return ATTN_SINK_ERR_INVALID_ARG;
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return ATTN_SINK_ERR_INVALID_ARG;
  const int32_t group = num_q_heads / num_kv_heads;
  if (q_len > kMaxQLen || (int64_t)q_len * group > kMaxColumns) return ATTN_SINK_ERR_UNSUPPORTED;
  if (!is_pow2(page_size) || page_size < 16 || page_size > 256) return ATTN_SINK_ERR_UNSUPPORTED;
  if (batch > 0 && kv_lens == nullptr) return ATTN_SINK_ERR_INVALID_ARG;
  int64_t grid = workgroups;
  if (grid <= 0) {
    grid = decode_resident_workgroups((q_len * group + 15) / 16, false);
    if (grid <= 0) return ATTN_SINK_ERR_HIP;
  }
  int64_t max_len = 0;
  for (int32_t b = 0; b < batch; ++b) max_len = std::max<int64_t>(max_len, kv_lens[b]);
  // Candidates: multiples of 256 (and of the page size) up to one chunk per sequence.
  const int64_t step = std::max<int64_t>(256, page_size);
  const int64_t top = std::max<int64_t>(step, (max_len + step - 1) / step * step);
  int64_t best = top, best_load = INT64_MAX;
  std::vector<int64_t> load((size_t)grid);
  for (int64_t c = step; c <= top; c += step) {
    int64_t items = 0, most = 1;
    for (int32_t b = 0; b < batch; ++b) {
      const int64_t n = std::max<int64_t>(1, (std::max(0, kv_lens[b]) + c - 1) / c);
      items += n;
      most = std::max(most, n);
    }
    items *= num_kv_heads;
    if (items > 64 * grid && c != top) continue;  // much finer than the grid: never the cheapest
    std::fill(load.begin(), load.end(), 0);
    int64_t i = 0;
    for (int32_t b = 0; b < batch; ++b) {
      const int64_t L = std::max(0, kv_lens[b]);
      const int64_t n = std::max<int64_t>(1, (L + c - 1) / c);
      for (int64_t ch = 0; ch < n; ++ch) {
        const int64_t keys = std::max<int64_t>(0, std::min(c, L - ch * c));
        for (int32_t h = 0; h < num_kv_heads; ++h, ++i) load[(size_t)(i % grid)] += keys + kPlanItemKeys;
      }
    }
    const int64_t worst = *std::max_element(load.begin(), load.end()) + kPlanMergeKeys * ((most + 15) / 16);
    if (worst <= best_load) {  // ties go to the longer chunk (fewer partials to merge)
      best_load = worst;
      best = c;
    }
  }
  *kv_chunk = (int32_t)std::min<int64_t>(best, INT32_MAX / 2 / step * step);
  return ATTN_SINK_OK;
}

attn_sink_status attn_sink_decode_workspace_layout(int32_t batch, int32_t q_len, int32_t max_kv_len,
                                                   int32_t num_q_heads, int32_t head_dim, int32_t kv_chunk,
                                                   attn_sink_decode_layout* layout) {
  if (layout == nullptr || head_dim != kSupportedHeadDim) return ATTN_SINK_ERR_INVALID_ARG;
  DecodeLayout l;
  if (!decode_layout(batch, q_len, max_kv_len, num_q_heads, effective_chunk(kv_chunk, max_kv_len, 16), &l))
    return ATTN_SINK_ERR_INVALID_ARG;
  layout->rows = l.rows;
  layout->chunks = l.chunks;
  layout->partials = l.partials;
  layout->off_indptr = (int64_t)l.off_indptr;
  layout->off_counts = (int64_t)l.off_counts;
  layout->off_o = (int64_t)l.off_o;
  layout->off_lse = (int64_t)l.off_lse;
  layout->total = (int64_t)l.total;
  return ATTN_SINK_OK;
}

}  // extern "C"

namespace {
// Points the plan and partial arrays of p into a workspace laid out as lay.
void bind_workspace(DecodeParams* pp, const DecodeLayout& lay, void* workspace) {
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  pp->indptr = reinterpret_cast<int32_t*>(ws + lay.off_indptr);
  pp->counts = reinterpret_cast<int32_t*>(ws + lay.off_counts);
  pp->o_part = reinterpret_cast<float*>(ws + lay.off_o);
  pp->lse_part = reinterpret_cast<float*>(ws + lay.off_lse);
}

// Validation and parameters shared by the decode entry points. out_required: the call also
// merges (out must be given). caller_workspace: the workspace pointer comes from the caller
// (checked for NULL and alignment here, and bound into *pp); otherwise the caller of this
// function binds the library's own scratch after validation, and workspace is unused.
attn_sink_status decode_prepare(const void* q, const void* k_cache, const void* v_cache, const int32_t* page_table,
                                int32_t max_pages_per_seq, int32_t num_pages, const int32_t* kv_lens,
                                const float* sinks, int32_t batch, int32_t q_len, int32_t max_kv_len,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                float softmax_scale, int32_t causal, int32_t window, int32_t kv_chunk,
                                void* workspace, size_t workspace_bytes, bool caller_workspace, const void* out,
                                bool out_required, DecodeParams* pp, DecodeLayout* lp) {
  if (batch < 0 || max_kv_len < 0 || max_pages_per_seq < 1 || num_pages < 1 || q_len < 1) return ATTN_SINK_ERR_INVALID_ARG;
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return ATTN_SINK_ERR_INVALID_ARG;
  if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f)) return ATTN_SINK_ERR_INVALID_ARG;
  if (head_dim != kSupportedHeadDim || q_len > kMaxQLen) return ATTN_SINK_ERR_UNSUPPORTED;
  const int32_t group = num_q_heads / num_kv_heads;
  if ((int64_t)q_len * group > kMaxColumns) return ATTN_SINK_ERR_UNSUPPORTED;
  if (!is_pow2(page_size) || page_size < 16 || page_size > 256) return ATTN_SINK_ERR_UNSUPPORTED;
  if (!capacity_fits(max_pages_per_seq, page_size)) return ATTN_SINK_ERR_UNSUPPORTED;
  if (kv_chunk > 0 && (kv_chunk % 64 != 0 || kv_chunk % page_size != 0)) return ATTN_SINK_ERR_UNSUPPORTED;
  if (num_kv_heads > kMaxGridY) return ATTN_SINK_ERR_UNSUPPORTED;
  const int64_t chunk = effective_chunk(kv_chunk, max_kv_len, page_size);
  if (chunk > INT32_MAX / 2) return ATTN_SINK_ERR_UNSUPPORTED;
  DecodeLayout lay;
  if (!decode_layout(batch, q_len, max_kv_len, num_q_heads, chunk, &lay)) return ATTN_SINK_ERR_UNSUPPORTED;
  if (lay.chunks * batch * num_kv_heads > INT32_MAX) return ATTN_SINK_ERR_UNSUPPORTED;
  *lp = lay;
  if (batch == 0) return ATTN_SINK_OK;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || page_table == nullptr || kv_lens == nullptr ||
      (out_required && out == nullptr) || (caller_workspace && workspace == nullptr))
    return ATTN_SINK_ERR_INVALID_ARG;
  if (misaligned16(q) || misaligned16(k_cache) || misaligned16(v_cache) || (out != nullptr && misaligned16(out)))
    return ATTN_SINK_ERR_INVALID_ARG;
  if (caller_workspace && (reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return ATTN_SINK_ERR_INVALID_ARG;
  if (workspace_bytes < attn_sink_decode_workspace_size(batch, q_len, max_kv_len, num_q_heads, head_dim, kv_chunk) ||
      workspace_bytes < lay.total)
    return ATTN_SINK_ERR_WORKSPACE_TOO_SMALL;

  DecodeParams& p = *pp;
  p.q = static_cast<const uint16_t*>(q);
  p.k_cache = static_cast<const uint16_t*>(k_cache);
  p.v_cache = static_cast<const uint16_t*>(v_cache);
  p.page_table = page_table;
  p.kv_lens = kv_lens;
  p.sinks = sinks;
  if (caller_workspace) bind_workspace(&p, lay, workspace);
  p.batch = batch;
  p.q_len = q_len;
  p.max_kv_len = max_kv_len;
  p.hq = num_q_heads;
  p.hkv = num_kv_heads;
  p.group = group;
  p.page_size = page_size;
  p.page_shift = ilog2(page_size);
  p.max_pages = max_pages_per_seq;
  p.num_pages = num_pages;
  p.kv_chunk = (int)chunk;
  p.causal = causal != 0;
  p.window = window > 0 ? window : 0;
  p.scale_log2 = softmax_scale * kLog2e;
  p.tree_mask = nullptr;
  return ATTN_SINK_OK;
}

// The split-KV kernel, then the merge of its partials into out / lse.
attn_sink_status decode_split_and_merge(const DecodeParams& p, const DecodeLayout& lay, void* out, float* lse,
                                        hipStream_t s) {
  if (launch_decode_split(p, (int)lay.chunks, s) != hipSuccess) return ATTN_SINK_ERR_HIP;
  MergeParams mp;
  mp.o_part = p.o_part;
  mp.lse_part = p.lse_part;
  mp.indptr = p.indptr;
  mp.out = static_cast<uint16_t*>(out);
  mp.lse = lse;
  mp.num_partials = (int)lay.partials;
  mp.rows = (int)lay.rows;
  mp.hq = p.hq;
  return hip_status(launch_merge(mp, s));
}
}  // namespace

extern "C" {

attn_sink_status attn_sink_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* page_table, int32_t max_pages_per_seq, int32_t num_pages,
                                        const int32_t* kv_lens, const float* sinks, int32_t batch, int32_t q_len,
                                        int32_t max_kv_len, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t page_size, float softmax_scale, int32_t causal,
                                        int32_t window, int32_t kv_chunk, void* workspace, size_t workspace_bytes,
                                        void* out, float* lse, void* stream) {
  DecodeParams p{};
  DecodeLayout lay;
  const attn_sink_status st = decode_prepare(q, k_cache, v_cache, page_table, max_pages_per_seq, num_pages, kv_lens,
                                             sinks, batch, q_len, max_kv_len, num_q_heads, num_kv_heads, head_dim,
                                             page_size, softmax_scale, causal, window, kv_chunk, workspace,
                                             workspace_bytes, true, out, true, &p, &lay);
  if (st != ATTN_SINK_OK || batch == 0) return st;
  return decode_split_and_merge(p, lay, out, lse, reinterpret_cast<hipStream_t>(stream));
}

attn_sink_status attn_sink_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                                const int32_t* page_table, int32_t max_pages_per_seq,
                                                int32_t num_pages, const int32_t* kv_lens, const float* sinks,
                                                int32_t batch, int32_t q_len, int32_t max_kv_len,
                                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                                int32_t page_size, float softmax_scale, int32_t causal,
                                                int32_t window, int32_t kv_chunk, void* out, float* lse,
                                                void* stream) {
  DecodeParams p{};
  DecodeLayout lay;
  // Everything is validated (the layout against the scratch's size included) before the first
  // HIP call.
  const attn_sink_status st = decode_prepare(q, k_cache, v_cache, page_table, max_pages_per_seq, num_pages, kv_lens,
                                             sinks, batch, q_len, max_kv_len, num_q_heads, num_kv_heads, head_dim,
                                             page_size, softmax_scale, causal, window, kv_chunk, nullptr,
                                             kNoAllocScratchBytes, false, out, true, &p, &lay);
  if (st != ATTN_SINK_OK || batch == 0) return st;
  void* ws = nullptr;
  if (current_scratch(&ws) != hipSuccess) return ATTN_SINK_ERR_HIP;
  bind_workspace(&p, lay, ws);
  return decode_split_and_merge(p, lay, out, lse, reinterpret_cast<hipStream_t>(stream));
}

size_t attn_sink_decode_noalloc_capacity(void) { return kNoAllocScratchBytes; }

attn_sink_status attn_sink_decode_paged_tree(const void* q, const void* k_cache, const void* v_cache,
                                             const int32_t* page_table, int32_t max_pages_per_seq, int32_t num_pages,
                                             const int32_t* kv_lens, const int32_t* tree_mask, const float* sinks,
                                             int32_t batch, int32_t q_len, int32_t max_kv_len, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                             float softmax_scale, int32_t window, int32_t kv_chunk, void* workspace,
                                             size_t workspace_bytes, void* out, float* lse, void* stream) {
  DecodeParams p{};
  DecodeLayout lay;
  const attn_sink_status st = decode_prepare(q, k_cache, v_cache, page_table, max_pages_per_seq, num_pages, kv_lens,
                                             sinks, batch, q_len, max_kv_len, num_q_heads, num_kv_heads, head_dim,
                                             page_size, softmax_scale, 1, window, kv_chunk, workspace,
                                             workspace_bytes, true, out, true, &p, &lay);
  if (st != ATTN_SINK_OK || batch == 0) return st;
  if (tree_mask == nullptr) return ATTN_SINK_ERR_INVALID_ARG;
  p.tree_mask = tree_mask;
  return decode_split_and_merge(p, lay, out, lse, reinterpret_cast<hipStream_t>(stream));
}

attn_sink_status attn_sink_decode_paged_partials(const void* q, const void* k_cache, const void* v_cache,
                                                 const int32_t* page_table, int32_t max_pages_per_seq,
                                                 int32_t num_pages, const int32_t* kv_lens, const float* sinks,
                                                 int32_t batch, int32_t q_len, int32_t max_kv_len,
                                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                                 int32_t page_size, float softmax_scale, int32_t causal,
                                                 int32_t window, int32_t kv_chunk, void* workspace,
                                                 size_t workspace_bytes, void* stream) {
  DecodeParams p{};
  DecodeLayout lay;
  const attn_sink_status st = decode_prepare(q, k_cache, v_cache, page_table, max_pages_per_seq, num_pages, kv_lens,
                                             sinks, batch, q_len, max_kv_len, num_q_heads, num_kv_heads, head_dim,
                                             page_size, softmax_scale, causal, window, kv_chunk, workspace,
                                             workspace_bytes, true, nullptr, false, &p, &lay);
  if (st != ATTN_SINK_OK || batch == 0) return st;
  return hip_status(launch_decode_split(p, (int)lay.chunks, reinterpret_cast<hipStream_t>(stream)));
}

attn_sink_status attn_sink_decode_paged_range_partials(const void* q, const void* k_cache, const void* v_cache,
                                                       const int32_t* page_table, int32_t max_pages_per_seq,
                                                       int32_t num_pages, const int32_t* kv_lens,
                                                       const int32_t* kv_start, const int32_t* kv_total,
                                                       const float* sinks, int32_t batch, int32_t q_len,
                                                       int32_t max_kv_len, int32_t num_q_heads, int32_t num_kv_heads,
                                                       int32_t head_dim, int32_t page_size, float softmax_scale,
                                                       int32_t causal, int32_t window, int32_t kv_chunk,
                                                       void* workspace, size_t workspace_bytes, void* stream) {
  DecodeParams p{};
  DecodeLayout lay;
  const attn_sink_status st = decode_prepare(q, k_cache, v_cache, page_table, max_pages_per_seq, num_pages, kv_lens,
                                             sinks, batch, q_len, max_kv_len, num_q_heads, num_kv_heads, head_dim,
                                             page_size, softmax_scale, causal, window, kv_chunk, workspace,
                                             workspace_bytes, true, nullptr, false, &p, &lay);
  if (st != ATTN_SINK_OK || batch == 0) return st;
  if (kv_start == nullptr || kv_total == nullptr) return ATTN_SINK_ERR_INVALID_ARG;
  p.kv_start = kv_start;
  p.kv_total = kv_total;
  return hip_status(launch_decode_split(p, (int)lay.chunks, reinterpret_cast<hipStream_t>(stream)));
}

attn_sink_status attn_sink_decode_paged_tree_partials(const void* q, const void* k_cache, const void* v_cache,
                                                      const int32_t* page_table, int32_t max_pages_per_seq,
                                                      int32_t num_pages, const int32_t* kv_lens,
                                                      const int32_t* tree_mask, const float* sinks, int32_t batch,
                                                      int32_t q_len, int32_t max_kv_len, int32_t num_q_heads,
                                                      int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                                      float softmax_scale, int32_t window, int32_t kv_chunk,
                                                      void* workspace, size_t workspace_bytes, void* stream) {
  DecodeParams p{};
  DecodeLayout lay;
  const attn_sink_status st = decode_prepare(q, k_cache, v_cache, page_table, max_pages_per_seq, num_pages, kv_lens,
                                             sinks, batch, q_len, max_kv_len, num_q_heads, num_kv_heads, head_dim,
                                             page_size, softmax_scale, 1, window, kv_chunk, workspace,
                                             workspace_bytes, true, nullptr, false, &p, &lay);
  if (st != ATTN_SINK_OK || batch == 0) return st;
  if (tree_mask == nullptr) return ATTN_SINK_ERR_INVALID_ARG;
  p.tree_mask = tree_mask;
  return hip_status(launch_decode_split(p, (int)lay.chunks, reinterpret_cast<hipStream_t>(stream)));
}

attn_sink_status attn_sink_merge_partials(const float* o_partial, const float* lse_partial, int32_t num_partials,
                                          const int32_t* partial_indptr, int32_t num_rows, int32_t num_q_heads,
                                          int32_t head_dim, void* out, float* lse, void* stream) {
  if (num_partials < 0 || num_rows < 0 || num_q_heads <= 0) return ATTN_SINK_ERR_INVALID_ARG;
  if (head_dim != kSupportedHeadDim) return ATTN_SINK_ERR_UNSUPPORTED;
  if (num_rows == 0) return ATTN_SINK_OK;
  if (partial_indptr == nullptr || out == nullptr) return ATTN_SINK_ERR_INVALID_ARG;
  if (num_partials > 0 && (o_partial == nullptr || lse_partial == nullptr)) return ATTN_SINK_ERR_INVALID_ARG;
  if (misaligned16(o_partial) || misaligned16(out)) return ATTN_SINK_ERR_INVALID_ARG;
  MergeParams mp;
  mp.o_part = o_partial;
  mp.lse_part = lse_partial;
  mp.indptr = partial_indptr;
  mp.out = static_cast<uint16_t*>(out);
  mp.lse = lse;
  mp.num_partials = num_partials;
  mp.rows = num_rows;
  mp.hq = num_q_heads;
  return hip_status(launch_merge(mp, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
