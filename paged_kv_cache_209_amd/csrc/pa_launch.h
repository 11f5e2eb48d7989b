// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "paged_attn.h"

namespace pa {

enum class Dtype { kF32 = 0, kBF16 = 1 };

hipError_t launch_kv_store(void* k_cache, void* v_cache, const void* k, const void* v, const int32_t* slot_mapping,
                           int32_t num_tokens, int32_t row_bytes, hipStream_t stream);

struct RopeStoreArgs {
  void* q_out;
  void* k_cache;
  void* v_cache;
  const void* q;
  const void* k;
  const void* v;
  const int32_t* positions;
  const int32_t* slot_mapping;
  int32_t num_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  float base;  // rope theta
  const void* q_weight;  // QK-Norm weights [head_dim] (both null: no normalisation)
  const void* k_weight;
  float eps;
};

hipError_t launch_rope_kv_store(const RopeStoreArgs& args, Dtype dtype, int32_t head_dim, hipStream_t stream);

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
  int32_t num_workgroups;  // the context work is split evenly over this many (0: the library's grid)
  int64_t max_units;       // upper bound of the work units (the grid never exceeds it)
  float scale_log2;   // scale * log2(e) (times the K pool's scale for fp8 pools): scores in base-2 units
  float v_scale;      // fp8 pools: the V pool's scale, applied to the output; 1 otherwise
  uint64_t* counters;  // [num_seqs * num_q_heads]: tagged piece counts of each split item
  uint32_t* ws_flags;  // workspace error word (bit 0: a counter held another call's tag)
  // Tag of this call's piece counts (epoch << 16): taken from *epoch_word when
  // that is not null (graph replays, whose kernel arguments are fixed at
  // capture), else from epoch_tag.
  uint64_t epoch_tag;
  const uint64_t* epoch_word;
  float* part_lse;    // [2 * kDecodeMaxWorkgroups][group]: log2-sum-exp of each stored piece
  float* part_out;    // [2 * kDecodeMaxWorkgroups][group][head_dim]: normalised output of each piece
  // Fused store (all null otherwise): sequence t's new token, [num_seqs,
  // num_kv_heads, head_dim] each, is stored at slot_mapping[t] (if >= 0) and
  // read in flight at position context_lens[t] - 1.
  const void* k_new;
  const void* v_new;
  const int32_t* slot_mapping;
};

// Decode work unit: 64 tokens of one (sequence, query-head group). Each item
// also costs kDecodeItemCost units that hold no tokens (the fixed work of a
// segment), so the split over workgroups balances time rather than tokens.
constexpr int32_t kDecodeUnitTokens = 64;
constexpr int32_t kDecodeItemCost = 2;
// Largest decode grid; a workgroup stores at most two split pieces (its
// first and its last segment), in slots 2w and 2w + 1.
constexpr int32_t kDecodeMaxWorkgroups = 2048;
constexpr int32_t kDecodeMaxGroup = 4;  // query heads per decode workgroup

hipError_t launch_decode(const DecodeArgs& args, Dtype dtype, int32_t head_dim, hipStream_t stream);

// fp8 (E4M3) KV cache: the quantising store.
hipError_t launch_kv_store_fp8(void* k_cache, void* v_cache, const void* k, const void* v,
                               const int32_t* slot_mapping, int32_t num_tokens, int32_t row_elems, float inv_k,
                               float inv_v, hipStream_t stream);

// Decode over fp8 (E4M3) pools, head_dim 128, with the bf16/fp32 decode
// kernel's work split and in-kernel merge: q and out bf16.
hipError_t launch_decode_fp8_pools(const DecodeArgs& a, hipStream_t stream);


// Grid the decode launcher uses when the caller does not fix one (`items` =
// sequences x query-head groups).
int decode_default_workgroups(Dtype dtype, int32_t head_dim, int32_t group, int64_t max_units, int64_t items);

// Workgroups of `kernel` (with `threads` per workgroup) that are resident on
// the current device at once: occupancy per compute unit (at most
// `max_per_cu` when that is positive) times compute units, capped by
// `max_units` (queried once per kernel and device, then cached). The number
// of compute units is stored in `*compute_units` when that is not null.
int resident_workgroups(const void* kernel, int threads, int64_t max_units, int max_per_cu = 0,
                        int* compute_units = nullptr);

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
  int32_t rows_per_tile;   // query rows per item: 256 (8 waves), 128 (4 waves) or 32 (1 wave)
  int32_t num_workgroups;  // the key tiles of all items are split evenly over these
  uint64_t* counters;      // [num_seqs * num_q_heads * (max_q_len + 1)]: tagged piece counts
  uint32_t* ws_flags;      // workspace error word (bit 0: a counter held another call's tag)
  uint64_t epoch_tag;      // this call's tag (epoch << 16)
  float* part_lse;         // [2 * num_workgroups * rows_per_tile]
  uint16_t* part_out;      // [2 * num_workgroups * rows_per_tile * head_dim]: bf16 (half of the
                           // space the workspace layout reserves)
};

// Largest grids the prefill launcher uses for each tile height (one 8-wave
// workgroup per CU, two 4-wave ones, four 1-wave ones), and the
// partial-result rows their workspace holds (two pieces per workgroup).
constexpr int kPrefillMaxWorkgroups256 = 256;
constexpr int kPrefillMaxWorkgroups128 = 512;
constexpr int kPrefillMaxWorkgroups32 = 1024;
constexpr int64_t kPrefillSlotRows = 2 * 512 * 128;
static_assert(2 * kPrefillMaxWorkgroups256 * 256 <= kPrefillSlotRows, "slot rows");
static_assert(2 * kPrefillMaxWorkgroups32 * 32 <= kPrefillSlotRows, "slot rows");

hipError_t launch_prefill(const PrefillArgs& args, int32_t head_dim, hipStream_t stream);

// Workspace layout of the split-context paths: a 256-byte header (error
// word, graph-replay epoch), fp32 log-sum-exp values and fp32 partial outputs
// in regions of a fixed size (sized for the largest head dimension), then the
// 64-bit piece counters. The counters start at the same offset for every
// call, whatever its sizes.
//
// Piece counters carry the tag of the call that counts on them: a counter
// word is (epoch << 16) | count, the epoch being unique to the call (a
// process-wide sequence from a random 47-bit start). An arrival first raises
// the word to at least (epoch << 16) (atomic max) and then adds one, so a
// word left by any earlier call of this process, or zero, restarts at this
// call's tag without anybody clearing it; a word that holds a larger foreign
// value (memory that was never zero-filled) is reported: the arrival sees a
// tag that is not its own, sets bit 0 of the error word and writes NaN to the
// item's output rows instead of merging pieces that may not be there.
constexpr int64_t kMaxHeadDim = 128;
constexpr size_t kWorkspaceHeaderBytes = 256;
constexpr size_t kWorkspaceFlagsOff = 0;   // uint32 error word
constexpr size_t kWorkspaceEpochOff = 8;   // uint64 epoch tag of a graph replay
constexpr uint32_t kWorkspaceErrStaleCounter = 1u;

struct WorkspaceLayout {
  size_t lse_off, out_off, counters_off, total;
};

inline WorkspaceLayout make_workspace_layout(int64_t slot_rows, int64_t counters) {
  WorkspaceLayout w;
  w.lse_off = kWorkspaceHeaderBytes;
  w.out_off = w.lse_off + static_cast<size_t>((slot_rows * 4 + 255) / 256 * 256);
  w.counters_off = w.out_off + static_cast<size_t>(slot_rows * kMaxHeadDim * 4);
  w.total = w.counters_off + static_cast<size_t>(counters * 8);
  return w;
}

// The next call's counter tag, (epoch << 16) with a fresh epoch (never 0).
uint64_t next_epoch_tag();

// Decode: two piece slots per workgroup of the largest grid, each for up to
// kDecodeMaxGroup query heads; one counter per (sequence, query head).
inline WorkspaceLayout decode_workspace_layout(int64_t num_seqs, int64_t num_q_heads) {
  return make_workspace_layout(int64_t{2} * kDecodeMaxWorkgroups * kDecodeMaxGroup, num_seqs * num_q_heads);
}

// pa_paged_attn_decode_store for graph capture: the kernel reads its counter
// tag at run time from the workspace header's epoch word, which the replay's
// set-up kernel writes before every replay (a captured launch keeps the
// arguments it was captured with).
pa_status decode_store_for_graph(void* out, const void* q, void* k_cache, void* v_cache, const void* k_new,
                                 const void* v_new, const int32_t* slot_mapping, const int32_t* block_tables,
                                 const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 int32_t max_blocks_per_seq, int32_t max_context_len, float scale, pa_dtype dtype,
                                 void* workspace, size_t workspace_bytes, pa_stream_t stream);

}  // namespace pa
