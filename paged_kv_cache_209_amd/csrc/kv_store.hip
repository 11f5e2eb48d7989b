// KV store: copy each new token's K and V rows into the pools at the slot the
// caller's slot mapping names ("Nano-vLLM System Architecture Analysis",
// section 2, "Attention with Paged Cache": computed K/V entries are stored into
// the paged cache via slot_mapping). Pure data movement. The new tokens' K (and
// V) rows form one flat array of 16-byte pieces; a workgroup moves 1 or 4
// sweeps of 256 consecutive pieces (each sweep fully coalesced), issuing every
// load of its sweeps -- the slots and the K and V pieces -- before the first
// store, so no K/V load waits behind its slot and a thread of a large store
// keeps 8 16-byte loads in flight. Pieces of a token whose slot is negative
// are read but not stored.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kStoreThreads = 256;

// kStorePieces sweeps per workgroup: 4 for large stores, 1 for small ones,
// where spreading the few pieces over more compute units matters more than
// loads in flight per thread.
template <int kStorePieces>
__global__ __launch_bounds__(kStoreThreads) void kv_store_kernel(u32x4_t* __restrict__ k_cache,
                                                                u32x4_t* __restrict__ v_cache,
                                                                const u32x4_t* __restrict__ k,
                                                                const u32x4_t* __restrict__ v,
                                                                const int32_t* __restrict__ slot_mapping,
                                                                int64_t total_pieces, int32_t pieces_per_row) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kStoreThreads * kStorePieces + threadIdx.x;
  u32x4_t kk[kStorePieces], vv[kStorePieces];
  int32_t slot[kStorePieces], piece[kStorePieces];
#pragma unroll
  for (int m = 0; m < kStorePieces; ++m) {
    const int64_t i = base + static_cast<int64_t>(m) * kStoreThreads;
    slot[m] = -1;
    if (i < total_pieces) {
      const int64_t token = i / pieces_per_row;
      piece[m] = static_cast<int32_t>(i - token * pieces_per_row);
      slot[m] = slot_mapping[token];
      // Streaming loads: each byte is read once.
      kk[m] = __builtin_nontemporal_load(k + i);
      vv[m] = __builtin_nontemporal_load(v + i);
    }
  }
#pragma unroll
  for (int m = 0; m < kStorePieces; ++m) {
    if (slot[m] >= 0) {
      const int64_t dst = static_cast<int64_t>(slot[m]) * pieces_per_row + piece[m];
      k_cache[dst] = kk[m];
      v_cache[dst] = vv[m];
    }
  }
}

}  // namespace

hipError_t launch_kv_store(void* k_cache, void* v_cache, const void* k, const void* v, const int32_t* slot_mapping,
                           int32_t num_tokens, int32_t row_bytes, hipStream_t stream) {
  const int32_t pieces_per_row = row_bytes / 16;
  const int64_t total = static_cast<int64_t>(num_tokens) * pieces_per_row;
  if (total == 0) return hipSuccess;
  // Four sweeps per workgroup once that still gives at least 256 workgroups.
  constexpr int64_t kLarge = int64_t{256} * kStoreThreads * 4;
  u32x4_t* kc = static_cast<u32x4_t*>(k_cache);
  u32x4_t* vc = static_cast<u32x4_t*>(v_cache);
  const u32x4_t* kk = static_cast<const u32x4_t*>(k);
  const u32x4_t* vv = static_cast<const u32x4_t*>(v);
  if (total >= kLarge) {
    const int64_t blocks = (total + kStoreThreads * 4 - 1) / (kStoreThreads * 4);
    kv_store_kernel<4><<<dim3(static_cast<uint32_t>(blocks)), dim3(kStoreThreads), 0, stream>>>(
        kc, vc, kk, vv, slot_mapping, total, pieces_per_row);
  } else {
    const int64_t blocks = (total + kStoreThreads - 1) / kStoreThreads;
    kv_store_kernel<1><<<dim3(static_cast<uint32_t>(blocks)), dim3(kStoreThreads), 0, stream>>>(
        kc, vc, kk, vv, slot_mapping, total, pieces_per_row);
  }
  return hipGetLastError();
}

}  // namespace pa
