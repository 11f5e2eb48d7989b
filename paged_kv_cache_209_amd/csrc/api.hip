// C ABI of libpagedattn.so: host-side argument validation, workspace sizing
// and kernel launches on the caller's stream. Validation runs entirely on the
// host and touches no HIP API, so every error path can be exercised without a
// GPU.
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <unistd.h>

#include <atomic>
#include <chrono>

#include "paged_attn.h"
#include "pa_launch.h"

namespace pa {

// Epochs of the piece-counter tags: one process-wide sequence, started at a
// random point below 2^47 (so that memory left by another process that used
// this library is unlikely to hold a tag of ours, and 2^47 calls fit before
// the 48-bit field would wrap).
uint64_t next_epoch_tag() {
  static std::atomic<uint64_t> next{[] {
    uint64_t x = static_cast<uint64_t>(std::chrono::high_resolution_clock::now().time_since_epoch().count());
    x ^= static_cast<uint64_t>(getpid()) << 32;
    x ^= reinterpret_cast<uintptr_t>(&x);
    // splitmix64 finaliser (mixes every input bit into every output bit)
    x += 0x9E3779B97F4A7C15ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    x ^= x >> 31;
    return (x & ((uint64_t{1} << 46) - 1)) + 1;
  }()};
  const uint64_t epoch = next.fetch_add(1, std::memory_order_relaxed) & ((uint64_t{1} << 48) - 1);
  return (epoch == 0 ? 1 : epoch) << 16;
}

}  // namespace pa

namespace {

constexpr int32_t kBlockSize = 256;
constexpr float kLog2e = 1.4426950408889634f;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

pa_status check_common(int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                       pa_dtype dtype) {
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0) return PA_ERR_INVALID_ARG;
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_INVALID_ARG;
  if (block_size != kBlockSize) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(num_blocks) * block_size >= (int64_t{1} << 31)) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

pa_status to_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// Upper bound of the decode work units that hold tokens (one per 64 tokens
// of the longest context, for every (sequence, query-head group)): the
// library's grid never exceeds it.
int64_t decode_max_units(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t max_context_len) {
  const int64_t head_groups = num_q_heads / pa::decode_head_group(num_q_heads / num_kv_heads);
  return static_cast<int64_t>(num_seqs) * head_groups * ceil_div(max_context_len, pa::kDecodeUnitTokens);
}

// An item is split over workgroups only if its context has more than one unit.
size_t decode_workspace(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t max_context_len) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len <= pa::kDecodeUnitTokens) return 0;
  return pa::decode_workspace_layout(num_seqs, num_q_heads).total;
}

// Prefill workspace: one counter per (sequence, query head, query tile) bound
// and two partial-result pieces per workgroup of the largest grid.
pa::WorkspaceLayout prefill_layout(int32_t num_seqs, int32_t num_q_heads, int32_t max_q_len) {
  const int64_t counters = static_cast<int64_t>(num_seqs) * num_q_heads * (static_cast<int64_t>(max_q_len) + 1);
  return pa::make_workspace_layout(pa::kPrefillSlotRows, counters);
}

}  // namespace

extern "C" {

const char* pa_version(void) { return "pagedattn 0.1.0 gfx950"; }

const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK:
      return "PA_OK";
    case PA_ERR_INVALID_ARG:
      return "PA_ERR_INVALID_ARG: invalid argument";
    case PA_ERR_UNSUPPORTED:
      return "PA_ERR_UNSUPPORTED: unsupported dtype, head_dim or block_size";
    case PA_ERR_WORKSPACE:
      return "PA_ERR_WORKSPACE: workspace missing, too small, or not zero-filled before its first use";
    case PA_ERR_HIP:
      return "PA_ERR_HIP: HIP runtime error";
    case PA_ERR_NO_BLOCKS:
      return "PA_ERR_NO_BLOCKS: too few free KV-cache blocks";
  }
  return "unknown pa_status";
}

pa_status pa_kv_store(void* k_cache, void* v_cache, const void* k, const void* v, const int32_t* slot_mapping,
                      int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t num_blocks, pa_dtype dtype, pa_stream_t stream) {
  if (num_tokens < 0) return PA_ERR_INVALID_ARG;
  const pa_status st = check_common(num_kv_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (k_cache == nullptr || v_cache == nullptr) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (k == nullptr || v == nullptr || slot_mapping == nullptr) return PA_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k) || !aligned16(v)) return PA_ERR_INVALID_ARG;
  const int32_t elt = dtype == PA_BF16 ? 2 : 4;
  const int32_t row_bytes = num_kv_heads * head_dim * elt;
  (void)hipGetLastError();
  return to_status(pa::launch_kv_store(k_cache, v_cache, k, v, slot_mapping, num_tokens, row_bytes,
                                       static_cast<hipStream_t>(stream)));
}

int32_t pa_decode_num_workgroups(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_context_len, pa_dtype dtype) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len <= 0 ||
      num_q_heads % num_kv_heads != 0 || (head_dim != 64 && head_dim != 128) || (dtype != PA_F32 && dtype != PA_BF16))
    return 0;
  const int32_t group = num_q_heads / num_kv_heads;
  const int64_t items = static_cast<int64_t>(num_seqs) * (num_q_heads / pa::decode_head_group(group));
  return pa::decode_default_workgroups(dtype == PA_BF16 ? pa::Dtype::kBF16 : pa::Dtype::kF32, head_dim, group,
                                       decode_max_units(num_seqs, num_q_heads, num_kv_heads, max_context_len), items);
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t max_q_len,
                                 int32_t max_context_len) {
  (void)max_q_len;
  return decode_workspace(num_seqs, num_q_heads, head_dim, max_context_len);
}

}  // extern "C"

namespace {

pa_status rope_store_common(void* q_out, void* k_cache, void* v_cache, const void* q, const void* k, const void* v,
                            const void* q_weight, const void* k_weight, float eps, const int32_t* positions,
                            const int32_t* slot_mapping, int32_t num_tokens, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            float rope_theta, pa_dtype dtype, pa_stream_t stream) {
  if (num_tokens < 0 || num_q_heads <= 0) return PA_ERR_INVALID_ARG;
  const pa_status st = check_common(num_kv_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (!isfinite(rope_theta) || !(rope_theta > 0.0f)) return PA_ERR_INVALID_ARG;
  if (k_cache == nullptr || v_cache == nullptr) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (q_out == nullptr || q == nullptr || k == nullptr || v == nullptr || positions == nullptr ||
      slot_mapping == nullptr)
    return PA_ERR_INVALID_ARG;
  if (!aligned16(q_out) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(q) || !aligned16(k) ||
      !aligned16(v))
    return PA_ERR_INVALID_ARG;
  pa::RopeStoreArgs a;
  a.q_out = q_out;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.q = q;
  a.k = k;
  a.v = v;
  a.positions = positions;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.base = rope_theta;
  a.q_weight = q_weight;
  a.k_weight = k_weight;
  a.eps = eps;
  (void)hipGetLastError();
  return to_status(pa::launch_rope_kv_store(a, dtype == PA_BF16 ? pa::Dtype::kBF16 : pa::Dtype::kF32, head_dim,
                                            static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

pa_status pa_rope_kv_store(void* q_out, void* k_cache, void* v_cache, const void* q, const void* k, const void* v,
                           const int32_t* positions, const int32_t* slot_mapping, int32_t num_tokens,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, float rope_theta, pa_dtype dtype, pa_stream_t stream) {
  return rope_store_common(q_out, k_cache, v_cache, q, k, v, nullptr, nullptr, 0.0f, positions, slot_mapping,
                           num_tokens, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, rope_theta, dtype,
                           stream);
}

pa_status pa_qknorm_rope_kv_store(void* q_out, void* k_cache, void* v_cache, const void* q, const void* k,
                                  const void* v, const void* q_norm_weight, const void* k_norm_weight, float eps,
                                  const int32_t* positions, const int32_t* slot_mapping, int32_t num_tokens,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t num_blocks, float rope_theta, pa_dtype dtype, pa_stream_t stream) {
  if (q_norm_weight == nullptr || k_norm_weight == nullptr) return PA_ERR_INVALID_ARG;
  if (!aligned16(q_norm_weight) || !aligned16(k_norm_weight)) return PA_ERR_INVALID_ARG;
  if (!isfinite(eps) || eps < 0.0f) return PA_ERR_INVALID_ARG;
  return rope_store_common(q_out, k_cache, v_cache, q, k, v, q_norm_weight, k_norm_weight, eps, positions,
                           slot_mapping, num_tokens, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                           rope_theta, dtype, stream);
}

}  // extern "C"

namespace {

// Points the decode arguments at the workspace's regions (all null when the
// call splits nothing) and gives the call its counter tag: a fresh one, or,
// for graph replays, the tag the replay's set-up kernel writes into the
// workspace header (`epoch_word`).
void set_decode_workspace(pa::DecodeArgs& a, void* workspace, const pa::WorkspaceLayout& lay,
                          const uint64_t* epoch_word) {
  char* ws = static_cast<char*>(workspace);
  a.counters = ws ? reinterpret_cast<uint64_t*>(ws + lay.counters_off) : nullptr;
  a.ws_flags = ws ? reinterpret_cast<uint32_t*>(ws + pa::kWorkspaceFlagsOff) : nullptr;
  a.part_lse = ws ? reinterpret_cast<float*>(ws + lay.lse_off) : nullptr;
  a.part_out = ws ? reinterpret_cast<float*>(ws + lay.out_off) : nullptr;
  a.epoch_tag = pa::next_epoch_tag();
  a.epoch_word = ws ? epoch_word : nullptr;
}

// Decode, optionally fused with the store of the step's new K/V rows
// (k_new non-null: k_new, v_new [num_seqs, num_kv_heads, head_dim] and
// slot_mapping [num_seqs]).
pa_status decode_common(void* out, const void* q, const void* k_cache, const void* v_cache, const void* k_new,
                        const void* v_new, const int32_t* slot_mapping, const int32_t* block_tables,
                        const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                        int32_t max_context_len, float scale, pa_dtype dtype, int32_t num_workgroups,
                        void* workspace, size_t workspace_bytes, pa_stream_t stream,
                        const uint64_t* epoch_word = nullptr) {
  if (num_seqs < 0 || num_q_heads <= 0) return PA_ERR_INVALID_ARG;
  const pa_status st = check_common(num_kv_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (max_blocks_per_seq <= 0 || max_context_len <= 0) return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return PA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (num_workgroups < 0 || num_workgroups > pa::kDecodeMaxWorkgroups) return PA_ERR_INVALID_ARG;
  if (k_cache == nullptr || v_cache == nullptr) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (out == nullptr || q == nullptr || block_tables == nullptr || context_lens == nullptr) return PA_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_INVALID_ARG;

  const pa::WorkspaceLayout lay = pa::decode_workspace_layout(num_seqs, num_q_heads);
  // An item is split over workgroups only if some workgroup gets less than a
  // whole item; with one unit per context nothing is ever split.
  const bool split = max_context_len > pa::kDecodeUnitTokens && num_workgroups != 1;
  if (split) {
    if (workspace == nullptr || workspace_bytes < lay.total) return PA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PA_ERR_INVALID_ARG;
  }

  pa::DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.num_workgroups = num_workgroups;  // 0: one resident round, chosen by the launcher
  a.max_units = decode_max_units(num_seqs, num_q_heads, num_kv_heads, max_context_len);
  a.scale_log2 = scale * kLog2e;
  a.v_scale = 1.0f;
  set_decode_workspace(a, split ? workspace : nullptr, lay, epoch_word);
  a.k_new = k_new;
  a.v_new = v_new;
  a.slot_mapping = slot_mapping;
  (void)hipGetLastError();
  return to_status(pa::launch_decode(a, dtype == PA_BF16 ? pa::Dtype::kBF16 : pa::Dtype::kF32, head_dim,
                                     static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

pa_status pa_paged_attn_decode_ex(void* out, const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                                  float scale, pa_dtype dtype, int32_t num_workgroups, void* workspace,
                                  size_t workspace_bytes, pa_stream_t stream) {
  return decode_common(out, q, k_cache, v_cache, nullptr, nullptr, nullptr, block_tables, context_lens, num_seqs,
                       num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                       max_context_len, scale, dtype, num_workgroups, workspace, workspace_bytes, stream);
}

pa_status pa_paged_attn_decode_store(void* out, const void* q, void* k_cache, void* v_cache, const void* k_new,
                                     const void* v_new, const int32_t* slot_mapping, const int32_t* block_tables,
                                     const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                     int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                                     pa_dtype dtype, void* workspace, size_t workspace_bytes, pa_stream_t stream) {
  if (num_seqs > 0 && (k_new == nullptr || v_new == nullptr || slot_mapping == nullptr)) return PA_ERR_INVALID_ARG;
  if (num_seqs > 0 && (!aligned16(k_new) || !aligned16(v_new))) return PA_ERR_INVALID_ARG;
  return decode_common(out, q, k_cache, v_cache, num_seqs > 0 ? k_new : nullptr, v_new, slot_mapping, block_tables,
                       context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, max_context_len, scale, dtype, 0, workspace, workspace_bytes, stream);
}

pa_status pa_workspace_status(void* workspace, size_t workspace_bytes, pa_stream_t stream) {
  if (workspace == nullptr || workspace_bytes < pa::kWorkspaceHeaderBytes) return PA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* word = static_cast<char*>(workspace) + pa::kWorkspaceFlagsOff;
  uint32_t flags = 0;
  (void)hipGetLastError();
  if (hipMemcpyAsync(&flags, word, sizeof(flags), hipMemcpyDeviceToHost, s) != hipSuccess) return PA_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return PA_ERR_HIP;
  if (flags == 0) return PA_OK;
  static const uint32_t kZero = 0;
  if (hipMemcpyAsync(word, &kZero, sizeof(kZero), hipMemcpyHostToDevice, s) != hipSuccess) return PA_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return PA_ERR_HIP;
  return PA_ERR_WORKSPACE;
}

pa_status pa_paged_attn_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                               pa_dtype dtype, void* workspace, size_t workspace_bytes, pa_stream_t stream) {
  return pa_paged_attn_decode_ex(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                                          num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                          max_blocks_per_seq, max_context_len, scale, dtype, 0, workspace,
                                          workspace_bytes, stream);
}

pa_status pa_kv_store_fp8(void* k_cache, void* v_cache, const void* k, const void* v, const int32_t* slot_mapping,
                          int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          int32_t num_blocks, float k_scale, float v_scale, pa_stream_t stream) {
  if (num_tokens < 0) return PA_ERR_INVALID_ARG;
  const pa_status st = check_common(num_kv_heads, head_dim, block_size, num_blocks, PA_BF16);
  if (st != PA_OK) return st;
  if (head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (!isfinite(k_scale) || !isfinite(v_scale) || !(k_scale > 0.0f) || !(v_scale > 0.0f)) return PA_ERR_INVALID_ARG;
  if (k_cache == nullptr || v_cache == nullptr) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (k == nullptr || v == nullptr || slot_mapping == nullptr) return PA_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k) || !aligned16(v)) return PA_ERR_INVALID_ARG;
  (void)hipGetLastError();
  return to_status(pa::launch_kv_store_fp8(k_cache, v_cache, k, v, slot_mapping, num_tokens, num_kv_heads * head_dim,
                                           1.0f / k_scale, 1.0f / v_scale, static_cast<hipStream_t>(stream)));
}

size_t pa_decode_fp8_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                     int32_t max_context_len) {
  if (head_dim != 128) return 0;
  return decode_workspace(num_seqs, num_q_heads, head_dim, max_context_len);
}

pa_status pa_paged_attn_decode_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                   int32_t max_context_len, float scale, float k_scale, float v_scale,
                                   void* workspace, size_t workspace_bytes, pa_stream_t stream) {
  if (num_seqs < 0 || num_q_heads <= 0) return PA_ERR_INVALID_ARG;
  const pa_status st = check_common(num_kv_heads, head_dim, block_size, num_blocks, PA_BF16);
  if (st != PA_OK) return st;
  if (head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (max_blocks_per_seq <= 0 || max_context_len <= 0) return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return PA_ERR_INVALID_ARG;
  if (!isfinite(scale) || !isfinite(k_scale) || !isfinite(v_scale) || !(k_scale > 0.0f) || !(v_scale > 0.0f))
    return PA_ERR_INVALID_ARG;
  if (k_cache == nullptr || v_cache == nullptr) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (out == nullptr || q == nullptr || block_tables == nullptr || context_lens == nullptr) return PA_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_INVALID_ARG;
  // the decode kernel's work split and workspace rule (counters zero between calls)
  const pa::WorkspaceLayout lay = pa::decode_workspace_layout(num_seqs, num_q_heads);
  const bool split = max_context_len > pa::kDecodeUnitTokens;
  if (split) {
    if (workspace == nullptr || workspace_bytes < lay.total) return PA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PA_ERR_INVALID_ARG;
  }
  pa::DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.num_workgroups = 0;
  a.max_units = decode_max_units(num_seqs, num_q_heads, num_kv_heads, max_context_len);
  a.scale_log2 = scale * k_scale * kLog2e;
  a.v_scale = v_scale;
  set_decode_workspace(a, split ? workspace : nullptr, lay, nullptr);
  a.k_new = nullptr;
  a.v_new = nullptr;
  a.slot_mapping = nullptr;
  (void)hipGetLastError();
  return to_status(pa::launch_decode_fp8_pools(a, static_cast<hipStream_t>(stream)));
}

size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t max_q_len,
                                  int32_t max_context_len) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_q_len <= 0 || max_context_len <= 0) return 0;
  return prefill_layout(num_seqs, num_q_heads, max_q_len).total;
}

pa_status pa_paged_attn_prefill(void* out, const void* q, const void* k, const void* v, const void* k_cache,
                                const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                                const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                                float scale, pa_dtype dtype, void* workspace, size_t workspace_bytes,
                                pa_stream_t stream) {
  return pa_paged_attn_prefill_ex(out, q, k, v, k_cache, v_cache, block_tables, context_lens, cu_seqlens, num_seqs,
                                  total_q, max_q_len, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                  max_blocks_per_seq, max_context_len, scale, dtype, 0, workspace, workspace_bytes,
                                  stream);
}

pa_status pa_paged_attn_prefill_ex(void* out, const void* q, const void* k, const void* v, const void* k_cache,
                                   const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                                   const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                                   float scale, pa_dtype dtype, int32_t num_workgroups, void* workspace,
                                   size_t workspace_bytes, pa_stream_t stream) {
  if (num_seqs < 0 || total_q < 0 || max_q_len < 0 || num_q_heads <= 0 || num_workgroups < 0)
    return PA_ERR_INVALID_ARG;
  const pa_status st = check_common(num_kv_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (max_blocks_per_seq <= 0 || max_context_len <= 0) return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return PA_ERR_INVALID_ARG;
  if (max_q_len > max_context_len) return PA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (k_cache == nullptr || v_cache == nullptr) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0 || total_q == 0 || max_q_len == 0) return PA_OK;
  if (out == nullptr || q == nullptr || k == nullptr || v == nullptr || block_tables == nullptr ||
      context_lens == nullptr || cu_seqlens == nullptr)
    return PA_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return PA_ERR_INVALID_ARG;
  const pa::WorkspaceLayout lay = prefill_layout(num_seqs, num_q_heads, max_q_len);
  if (workspace == nullptr || workspace_bytes < lay.total) return PA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PA_ERR_INVALID_ARG;

  const int32_t group = num_q_heads / num_kv_heads;
  // Query rows per work item: a sequence's (token, head) rows of one KV head
  // in tiles of 32 (one wave), 128 or 256 (4 or 8 waves sharing each K/V tile).
  const int64_t seq_rows = static_cast<int64_t>(max_q_len) * group;
  const int32_t rows = seq_rows <= 32 ? 32 : (seq_rows <= 128 ? 128 : 256);
  const int64_t qtiles = ceil_div(seq_rows, rows);
  const int64_t key_tile = rows == 32 ? 32 : 64;  // keys per work unit (the kernels' tile width)
  const int64_t max_units = static_cast<int64_t>(num_seqs) * num_kv_heads * qtiles * ceil_div(max_context_len, key_tile);
  const int64_t cap = rows == 256 ? pa::kPrefillMaxWorkgroups256
                                  : (rows == 128 ? pa::kPrefillMaxWorkgroups128 : pa::kPrefillMaxWorkgroups32);

  pa::PrefillArgs a;
  a.out = out;
  a.q = q;
  a.k = k;
  a.v = v;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.cu_seqlens = cu_seqlens;
  a.num_seqs = num_seqs;
  a.total_q = total_q;
  a.max_q_len = max_q_len;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  // The kernel keeps scores in log2 units with a positive factor; a negative
  // scale is applied by negating q, and a zero scale by a vanishing factor
  // (every weight then rounds to exactly 1, the plain mean).
  const float sl = scale * kLog2e;
  a.scale_log2 = fabsf(sl) > 1e-30f ? fabsf(sl) : 1e-30f;
  a.negate_q = sl < 0.0f ? 1 : 0;
  a.rows_per_tile = rows;
  const int64_t grid = num_workgroups > 0 && num_workgroups < cap ? num_workgroups : cap;
  a.num_workgroups = static_cast<int32_t>(max_units < grid ? max_units : grid);
  char* ws = static_cast<char*>(workspace);
  a.counters = reinterpret_cast<uint64_t*>(ws + lay.counters_off);
  a.ws_flags = reinterpret_cast<uint32_t*>(ws + pa::kWorkspaceFlagsOff);
  a.epoch_tag = pa::next_epoch_tag();
  a.part_lse = reinterpret_cast<float*>(ws + lay.lse_off);
  a.part_out = reinterpret_cast<uint16_t*>(ws + lay.out_off);
  (void)hipGetLastError();
  return to_status(pa::launch_prefill(a, head_dim, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace pa {

pa_status decode_store_for_graph(void* out, const void* q, void* k_cache, void* v_cache, const void* k_new,
                                 const void* v_new, const int32_t* slot_mapping, const int32_t* block_tables,
                                 const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 int32_t max_blocks_per_seq, int32_t max_context_len, float scale, pa_dtype dtype,
                                 void* workspace, size_t workspace_bytes, pa_stream_t stream) {
  if (num_seqs > 0 && (k_new == nullptr || v_new == nullptr || slot_mapping == nullptr)) return PA_ERR_INVALID_ARG;
  if (num_seqs > 0 && (!aligned16(k_new) || !aligned16(v_new))) return PA_ERR_INVALID_ARG;
  if (workspace == nullptr || workspace_bytes < kWorkspaceHeaderBytes) return PA_ERR_WORKSPACE;
  const uint64_t* epoch_word =
      reinterpret_cast<const uint64_t*>(static_cast<const char*>(workspace) + kWorkspaceEpochOff);
  return decode_common(out, q, k_cache, v_cache, num_seqs > 0 ? k_new : nullptr, v_new, slot_mapping, block_tables,
                       context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, max_context_len, scale, dtype, 0, workspace, workspace_bytes, stream,
                       epoch_word);
}

}  // namespace pa
