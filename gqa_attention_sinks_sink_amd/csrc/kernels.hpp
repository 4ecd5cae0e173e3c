// Kernel parameter blocks and launchers (internal to libattnsink.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn_sink {

struct DecodeParams {
  const uint16_t* q;        // bf16 [batch*q_len, hq, 64]
  const uint16_t* k_cache;  // bf16 [num_pages, hkv, page_size, 64]
  const uint16_t* v_cache;
  const int32_t* page_table;  // [batch, max_pages]
  const int32_t* kv_lens;     // [batch]
  const float* sinks;         // [hq] or nullptr
  int32_t* indptr;            // workspace: [batch*q_len + 1]
  int32_t* counts;            // workspace: [batch*q_len]
  float* o_part;              // workspace: [n_partials, hq, 64]
  float* lse_part;            // workspace: [n_partials, hq]
  int batch, q_len, max_kv_len, hq, hkv, group;
  int page_size, page_shift, max_pages, num_pages;
  int kv_chunk, causal, window;
  float scale_log2;  // softmax_scale * log2(e)
  // Draft-tree verification when non-null: [batch * q_len] bitmaps, bit i of row b * q_len + t
  // = draft token i visible to token t (the prefix is always visible; causal is not used).
  const int32_t* tree_mask;
  // One range of each sequence's keys (context parallelism) when non-null: sequence b's
  // kv_lens[b] keys sit at absolute positions kv_start[b] .. of a sequence of kv_total[b] keys
  // (queries = its last q_len); masks use absolute positions and only the range starting at
  // key 0 carries the sink. Null: the range is the whole sequence.
  const int32_t* kv_start;
  const int32_t* kv_total;
};

struct MergeParams {
  const float* o_part;
  const float* lse_part;
  const int32_t* indptr;
  uint16_t* out;  // bf16 [rows, hq, 64]
  float* lse;     // [rows, hq] or nullptr
  int num_partials, rows, hq;
};

struct PrefillParams {
  const uint16_t* q;  // bf16 [total_q, hq, 64]
  const uint16_t* k;  // bf16 [total_kv, hkv, 64]
  const uint16_t* v;
  const float* sinks;
  const int32_t* cu_q;
  const int32_t* cu_kv;
  uint16_t* out;  // bf16 [total_q, hq, 64]
  float* lse;     // [total_q, hq] or nullptr
  int batch, total_q, total_kv, max_q, max_kv;
  int hq, hkv, group, causal, window;
  float scale_log2;
  int units;        // work units per (sequence, head group); set by the launcher
  int pair_blocks;  // causal pairing of row blocks u and n-1-u; set by the launcher
  int xcd_round_robin;  // 8-wave kernel: deal (sequence, head group) pairs to XCDs round-robin
  // Paged K/V (chunked prefill) when page_table != nullptr: k and v are caches
  // [num_pages, hkv, page_size, 64], sequence b holds kv_lens[b] tokens (its queries are the
  // newest ones) and cu_kv / total_kv are unused.
  const int32_t* page_table;  // [batch, max_pages]
  const int32_t* kv_lens;     // [batch]
  int max_pages, num_pages, page_size, page_shift;
};

// YaRN rotary encoding of new tokens and their append into the paged cache.
struct RopeParams {
  const uint16_t* q;  // bf16 [total_q, hq, 64]: the new tokens
  const uint16_t* k;  // bf16 [total_q, hkv, 64]
  const uint16_t* v;
  const int32_t* cu_q;        // [batch + 1]
  const int32_t* kv_lens;     // [batch], the new tokens included
  const int32_t* page_table;  // [batch, max_pages]
  uint16_t* k_cache;          // bf16 [num_pages, hkv, page_size, 64]
  uint16_t* v_cache;
  uint16_t* q_out;            // bf16 [total_q, hq, 64] (may be q)
  int batch, total_q, max_q, max_kv, hq, hkv;
  int max_pages, num_pages, page_size, page_shift;
  float mscale;       // attention temperature factor applied to cos and sin
  double freqs[32];   // angular frequency of pair (i, i + 32)
};

hipError_t launch_decode_split(const DecodeParams& p, int max_chunks, hipStream_t stream);
// Workgroups of the split-KV kernel resident at once on the current device (its persistent grid).
int decode_resident_workgroups(int column_tiles, bool tree);
hipError_t launch_rope_append(const RopeParams& p, hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);
// Prefill launch shape: query heads packed per tile row block, and 32-row blocks per wave.
int prefill_heads_per_tile(int group);
int prefill_row_blocks(int max_q, int heads_per_tile);

}  // namespace attn_sink
