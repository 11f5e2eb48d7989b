// KV store: copy each new token's K and V rows into the pools at the slot the
// caller's slot mapping names ("Nano-vLLM System Architecture Analysis",
// section 2, "Attention with Paged Cache": computed K/V entries are stored into
// the paged cache via slot_mapping). Pure data movement: every thread moves
// one 16-byte piece of one token's [Hkv, D] row of K and the same piece of V,
// so a wavefront reads and writes whole contiguous rows (fully coalesced).
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

__global__ __launch_bounds__(256) void kv_store_kernel(u32x4_t* __restrict__ k_cache, u32x4_t* __restrict__ v_cache,
                                                       const u32x4_t* __restrict__ k,
                                                       const u32x4_t* __restrict__ v,
                                                       const int32_t* __restrict__ slot_mapping,
                                                       int64_t total_pieces, int32_t pieces_per_row) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total_pieces) return;
  const int64_t token = i / pieces_per_row;
  const int32_t piece = static_cast<int32_t>(i - token * pieces_per_row);
  const int32_t slot = slot_mapping[token];
  if (slot < 0) return;
  const int64_t dst = static_cast<int64_t>(slot) * pieces_per_row + piece;
  const u32x4_t kk = __builtin_nontemporal_load(k + i);
  const u32x4_t vv = __builtin_nontemporal_load(v + i);
  k_cache[dst] = kk;
  v_cache[dst] = vv;
}

hipError_t launch_kv_store(void* k_cache, void* v_cache, const void* k, const void* v, const int32_t* slot_mapping,
                           int32_t num_tokens, int32_t row_bytes, hipStream_t stream) {
  const int32_t pieces_per_row = row_bytes / 16;
  const int64_t total = static_cast<int64_t>(num_tokens) * pieces_per_row;
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  kv_store_kernel<<<dim3(static_cast<uint32_t>(blocks)), dim3(threads), 0, stream>>>(
      static_cast<u32x4_t*>(k_cache), static_cast<u32x4_t*>(v_cache), static_cast<const u32x4_t*>(k),
      static_cast<const u32x4_t*>(v), slot_mapping, total, pieces_per_row);
  return hipGetLastError();
}

}  // namespace pa
