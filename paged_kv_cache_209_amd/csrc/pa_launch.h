// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum class Dtype { kF32 = 0, kBF16 = 1 };

hipError_t launch_kv_store(void* k_cache, void* v_cache, const void* k, const void* v, const int32_t* slot_mapping,
                           int32_t num_tokens, int32_t row_bytes, hipStream_t stream);

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;
  int32_t num_workgroups;  // the context work is split evenly over this many (0: one resident round)
  int64_t max_units;       // upper bound of the work units (the grid never exceeds it)
  int32_t max_parts;       // row stride of the partial-result arrays
  float scale_log2;   // scale * log2(e): scores are kept in base-2 units
  int32_t* counters;  // [num_seqs * num_q_heads], zero between calls
  float* part_lse;    // [num_seqs * num_q_heads * max_parts]
  float* part_out;    // [num_seqs * num_q_heads * max_parts * head_dim]
};

hipError_t launch_decode(const DecodeArgs& args, Dtype dtype, int32_t head_dim, hipStream_t stream);

// Grid the decode launcher uses when the caller does not fix one.
int decode_default_workgroups(Dtype dtype, int32_t head_dim, int32_t group, int64_t max_units);

// Workgroups of `kernel` (with `threads` per workgroup) that are resident on
// the current device at once: occupancy per compute unit times compute units,
// capped by `max_units` (queried once per kernel and device, then cached).
int resident_workgroups(const void* kernel, int threads, int64_t max_units);

// Query heads handled together by one decode workgroup (they share one KV
// head's rows): the largest of 4, 2, 1 that divides the GQA group size.
inline int decode_head_group(int group) { return group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1); }

struct PrefillArgs {
  void* out;
  const void* q;
  const void* k;
  const void* v;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* cu_seqlens;
  int32_t num_seqs;
  int32_t total_q;
  int32_t max_q_len;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;
  float scale_log2;        // |scale * log2(e)|, at least 1e-30 (so that it is positive)
  int32_t negate_q;        // 1 when the scale is negative: q is negated on load
  int32_t rows_per_tile;   // query rows per item: 128 (4 waves) or 32 (1 wave)
  int32_t num_workgroups;  // the key tiles of all items are split evenly over these
  int32_t* counters;       // [num_seqs * num_q_heads * (max_q_len + 1)], zero between calls
  float* part_lse;         // [2 * num_workgroups * rows_per_tile]
  float* part_out;         // [2 * num_workgroups * rows_per_tile * head_dim]
};

// Largest grids the prefill launcher uses for each tile height, and the
// partial-result rows their workspace holds (two pieces per workgroup).
constexpr int kPrefillMaxWorkgroups128 = 512;
constexpr int kPrefillMaxWorkgroups32 = 1024;
constexpr int64_t kPrefillSlotRows = 2 * 512 * 128;

hipError_t launch_prefill(const PrefillArgs& args, int32_t head_dim, hipStream_t stream);

// Workspace layout shared by the split-context paths: an int32 counter array,
// padded to 256 bytes, then fp32 log-sum-exp values, then fp32 partial outputs.
struct WorkspaceLayout {
  size_t counters_bytes;
  size_t lse_bytes;
  size_t out_bytes;
  size_t total() const { return counters_bytes + lse_bytes + out_bytes; }
};

inline WorkspaceLayout workspace_layout(int64_t num_seqs, int64_t num_q_heads, int64_t head_dim, int64_t rows_per_seq,
                                        int64_t max_parts) {
  WorkspaceLayout w;
  const int64_t units = num_seqs * num_q_heads * rows_per_seq;
  w.counters_bytes = static_cast<size_t>(((num_seqs * num_q_heads * 4) + 255) / 256 * 256);
  w.lse_bytes = static_cast<size_t>((units * max_parts * 4 + 255) / 256 * 256);
  w.out_bytes = static_cast<size_t>(units * max_parts * head_dim * 4);
  return w;
}

}  // namespace pa
