// pa_paged_attn_decode_noalloc: pa_paged_attn_decode for callers that cannot
// allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid allocation). The split-context scratch the decode
// kernel needs (partial results and piece counters) lives in a file-scope
// device array of a fixed size instead of a caller workspace; each GPU the
// library runs on holds its own copy of the array until the process ends.
//
// The array is zero when the code object loads, and the piece counters carry
// a fresh tag per call, so nothing in it needs clearing between calls. Every
// call on one GPU shares that GPU's array: calls that overlap in time on one
// GPU (different streams, or different threads) race on it and must not be
// issued.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "paged_attn.h"
#include "pa_launch.h"

namespace {

// Scratch size: the decode workspace's fixed regions (header, two partial
// slots per workgroup of the largest grid) plus 8 bytes per (sequence, query
// head) for up to kNoAllocMaxPairs pairs.
constexpr int64_t kNoAllocMaxPairs = 65536;
constexpr size_t kScratchBytes = 256 + 64 * 1024 + 8 * 1024 * 1024 + 8 * kNoAllocMaxPairs;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The array's device address on each GPU, from hipGetSymbolAddress with that
// GPU current (the name `scratch` is only a host-side stand-in in host code).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

pa_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return PA_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

size_t pa_decode_noalloc_scratch_bytes(void) { return kScratchBytes; }

pa_status pa_paged_attn_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                       int32_t max_context_len, float scale, pa_dtype dtype, pa_stream_t stream) {
  if (num_seqs < 0 || num_q_heads <= 0) return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(num_seqs) * num_q_heads > kNoAllocMaxPairs) return PA_ERR_WORKSPACE;
  if (pa_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, 1, max_context_len) > kScratchBytes)
    return PA_ERR_WORKSPACE;
  // Argument checks that need no device run first (a zero-sequence call
  // validates without launching), so a bad call never touches the device.
  const pa_status st = pa_paged_attn_decode(out, q, k_cache, v_cache, block_tables, context_lens, 0, num_q_heads,
                                            num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                            max_context_len, scale, dtype, nullptr, 0, stream);
  if (st != PA_OK || num_seqs == 0) return st;
  void* ws = nullptr;
  const pa_status sp = scratch_for_current_device(&ws);
  if (sp != PA_OK) return sp;
  return pa_paged_attn_decode(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                              num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                              scale, dtype, ws, kScratchBytes, stream);
}

}  // extern "C"
