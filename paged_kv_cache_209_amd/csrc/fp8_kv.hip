// fp8 KV cache: a quantising store and decode attention that reads the fp8
// pools (half the bytes of bf16) and dequantises on the fly. The pages name
// quantised KV-cache transfers ("Why Understand Inference Engine
// Architecture?", Tensor Parallelism Optimization, item 3) without a format;
// the format here is OCP FP8 E4M3 with one fp32 scale per pool: a value x is
// stored as the code nearest to clamp(x * (1/s), -448, 448) (ties to even, the
// hardware converter's rounding) and read back as code * s.
//
// Decode over fp8 pools is the bf16/fp32 decode kernel instantiated for fp8
// pool elements (decode.hip): its cost-balanced work split and in-kernel
// merge, with each lane's 16 codes of a row turned into bf16 pairs (exact)
// before the same v_dot2 arithmetic; the K pool's scale folds into the
// softmax scale and the V pool's into the output.
#include <math.h>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

// Saturation to the largest finite E4M3 magnitude (infinities included).
// fminf/fmaxf return the non-NaN operand, so a NaN would come out as -448:
// NaNs are given their code separately (nan_fixup).
__device__ __forceinline__ float clamp_fp8(float x) { return fminf(fmaxf(x, -448.0f), 448.0f); }

// Replaces the code of every NaN among the four values packed into w (value
// b in byte b) by the E4M3 NaN pattern with the value's sign, S.1111.111.
__device__ __forceinline__ uint32_t nan_fixup(uint32_t w, float x0, float x1, float x2, float x3) {
  const float xs[4] = {x0, x1, x2, x3};
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (xs[b] != xs[b]) {
      const uint32_t code = 0x7Fu | ((__float_as_uint(xs[b]) >> 31) << 7);
      w = (w & ~(0xFFu << (8 * b))) | (code << (8 * b));
    }
  }
  return w;
}

// Quantising store: one thread per 8 elements of a token's [Hkv, D] row of K
// and the same of V.
__global__ __launch_bounds__(256) void kv_store_fp8_kernel(uint8_t* __restrict__ k_cache,
                                                          uint8_t* __restrict__ v_cache,
                                                          const u32x4_t* __restrict__ k,
                                                          const u32x4_t* __restrict__ v,
                                                          const int32_t* __restrict__ slot_mapping,
                                                          int64_t total_pieces, int32_t pieces_per_row, float inv_k,
                                                          float inv_v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total_pieces) return;
  const int64_t token = i / pieces_per_row;
  const int32_t piece = static_cast<int32_t>(i - token * pieces_per_row);
  const int32_t slot = slot_mapping[token];
  const u32x4_t kk = __builtin_nontemporal_load(k + i);
  const u32x4_t vv = __builtin_nontemporal_load(v + i);
  if (slot < 0) return;
  uint32_t kw[2], vw[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // bf16 words 2h and 2h+1 hold elements 4h .. 4h+3
    const float k0 = bf16_lo(kk[2 * h]) * inv_k, k1 = bf16_hi(kk[2 * h]) * inv_k;
    const float k2 = bf16_lo(kk[2 * h + 1]) * inv_k, k3 = bf16_hi(kk[2 * h + 1]) * inv_k;
    const float v0 = bf16_lo(vv[2 * h]) * inv_v, v1 = bf16_hi(vv[2 * h]) * inv_v;
    const float v2 = bf16_lo(vv[2 * h + 1]) * inv_v, v3 = bf16_hi(vv[2 * h + 1]) * inv_v;
    int wk = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_fp8(k0), clamp_fp8(k1), 0, false);
    wk = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_fp8(k2), clamp_fp8(k3), wk, true);
    int wv = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_fp8(v0), clamp_fp8(v1), 0, false);
    wv = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_fp8(v2), clamp_fp8(v3), wv, true);
    kw[h] = nan_fixup(static_cast<uint32_t>(wk), k0, k1, k2, k3);
    vw[h] = nan_fixup(static_cast<uint32_t>(wv), v0, v1, v2, v3);
  }
  const int64_t dst = (static_cast<int64_t>(slot) * pieces_per_row + piece) * 8;
  uint2 ko, vo;
  ko.x = kw[0];
  ko.y = kw[1];
  vo.x = vw[0];
  vo.y = vw[1];
  *reinterpret_cast<uint2*>(k_cache + dst) = ko;
  *reinterpret_cast<uint2*>(v_cache + dst) = vo;
}

}  // namespace

hipError_t launch_kv_store_fp8(void* k_cache, void* v_cache, const void* k, const void* v,
                               const int32_t* slot_mapping, int32_t num_tokens, int32_t row_elems, float inv_k,
                               float inv_v, hipStream_t stream) {
  const int32_t pieces_per_row = row_elems / 8;
  const int64_t total = static_cast<int64_t>(num_tokens) * pieces_per_row;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  kv_store_fp8_kernel<<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream>>>(
      static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), static_cast<const u32x4_t*>(k),
      static_cast<const u32x4_t*>(v), slot_mapping, total, pieces_per_row, inv_k, inv_v);
  return hipGetLastError();
}

}  // namespace pa
