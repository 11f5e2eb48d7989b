// Rotary position embedding of the new tokens' q and k, fused with the KV
// store (optionally after QK-Norm: RMSNorm of every q and k head row with a
// per-dimension weight; the pages name QK-Norm among the served model's
// features in the same list as RoPE). The pages name RoPE among the features of the model Nano-vLLM serves
// ("Nano-vLLM System Architecture Analysis", section "Differences from Normal
// nanoGPT Inference", item 6) and store each step's computed K/V into the
// paged cache via slot_mapping (section 2, "Attention with Paged Cache"), so
// rotating k on its way into the pool saves one read and one write of every
// new K row against a separate rotation pass.
//
// Reading of the rotation (the pages give no formula): head dimension D is
// split in halves, element i and element i + D/2 form pair i, and pair i of a
// token at position p turns by p * base^(-2i/D) radians:
//   (a, b) -> (a cos t - b sin t, b cos t + a sin t).
//
// Layout of the work: one wave per token, looping over its heads four at a
// time (16 lanes per head); lane j of a head handles pairs [jP, jP + P) with
// P = D / 32, i.e. P consecutive elements of each half of the row, loaded and
// stored as one vector each. The angle is formed in fp64 (p * theta_i with
// theta_i = base^(-2i/D), reduced modulo 2 pi), so that positions in the tens
// of thousands keep full fp32 accuracy; the rotation itself is fp32.
#include <math.h>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kRopeWaves = 4;  // tokens per workgroup (one wave each)
constexpr int kLanesPerHead = 16;
constexpr int kHeadsPerPass = kWave / kLanesPerHead;

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) {
  return x;
}
template <>
__device__ __forceinline__ float to_f32<bf16_t>(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) {
  return x;
}
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  bf16_t r;
  r.bits = to_bf16_bits(x);
  return r;
}

// P consecutive elements of T, moved as one vector.
template <typename T, int P>
struct alignas(sizeof(T) * P) Pack {
  T e[P];
};

template <typename T, int D, bool NORM>
__global__ __launch_bounds__(kRopeWaves * kWave) void rope_kv_store_kernel(RopeStoreArgs a) {
  constexpr int P = D / 2 / kLanesPerHead;  // pairs per lane
  using V = Pack<T, P>;
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kRopeWaves + __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
  if (t >= a.num_tokens) return;
  const int hs = lane / kLanesPerHead;  // head within a pass of four
  const int j = lane % kLanesPerHead;
  const int pos = load_uniform(a.positions, t);
  const int slot = load_uniform(a.slot_mapping, t);

  // cos and sin of the lane's P angles
  float cs[P], sn[P];
  constexpr double kTwoPi = 6.283185307179586476925;
#pragma unroll
  for (int e = 0; e < P; ++e) {
    const int i = j * P + e;
    const double theta = pow(static_cast<double>(a.base), -2.0 * i / D);
    const double ang = static_cast<double>(pos) * theta;
    const double r = ang - kTwoPi * rint(ang * (1.0 / kTwoPi));  // |r| <= pi
    sincosf(static_cast<float>(r), &sn[e], &cs[e]);
  }

  const int64_t qrow = static_cast<int64_t>(t) * a.num_q_heads * D;
  const int64_t krow = static_cast<int64_t>(t) * a.num_kv_heads * D;
  const int64_t prow = static_cast<int64_t>(slot) * a.num_kv_heads * D;
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  T* q_out = static_cast<T*>(a.q_out);
  T* k_cache = static_cast<T*>(a.k_cache);
  T* v_cache = static_cast<T*>(a.v_cache);

  // Rotates the two P-element pieces of one head row and writes them to dst
  // (src and dst may be the same row). With NORM the row is first divided by
  // its root mean square (the 16 lanes of the head sum their squares by lane
  // shuffles) and multiplied by the per-dimension weight w.
  auto rotate = [&](const T* src, T* dst, const T* w) {
    const V lo = *reinterpret_cast<const V*>(src + j * P);
    const V hi = *reinterpret_cast<const V*>(src + D / 2 + j * P);
    float x[P], y[P];
#pragma unroll
    for (int e = 0; e < P; ++e) {
      x[e] = to_f32<T>(lo.e[e]);
      y[e] = to_f32<T>(hi.e[e]);
    }
    if constexpr (NORM) {
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < P; ++e) ss = fmaf(x[e], x[e], fmaf(y[e], y[e], ss));
#pragma unroll
      for (int off = 1; off < kLanesPerHead; off <<= 1) ss += __shfl_xor(ss, off, kWave);
      const float inv = 1.0f / sqrtf(ss * (1.0f / D) + a.eps);
      const V wlo = *reinterpret_cast<const V*>(w + j * P);
      const V whi = *reinterpret_cast<const V*>(w + D / 2 + j * P);
#pragma unroll
      for (int e = 0; e < P; ++e) {
        x[e] = x[e] * inv * to_f32<T>(wlo.e[e]);
        y[e] = y[e] * inv * to_f32<T>(whi.e[e]);
      }
    }
    V olo, ohi;
#pragma unroll
    for (int e = 0; e < P; ++e) {
      olo.e[e] = from_f32<T>(x[e] * cs[e] - y[e] * sn[e]);
      ohi.e[e] = from_f32<T>(y[e] * cs[e] + x[e] * sn[e]);
    }
    *reinterpret_cast<V*>(dst + j * P) = olo;
    *reinterpret_cast<V*>(dst + D / 2 + j * P) = ohi;
  };
  const T* q_w = static_cast<const T*>(a.q_weight);
  const T* k_w = static_cast<const T*>(a.k_weight);

  for (int h0 = 0; h0 < a.num_q_heads; h0 += kHeadsPerPass) {
    const int h = h0 + hs;
    if (h < a.num_q_heads) rotate(q + qrow + h * D, q_out + qrow + h * D, q_w);
  }
  if (slot < 0) return;  // the token's K/V are not stored (its query still is rotated)
  for (int h0 = 0; h0 < a.num_kv_heads; h0 += kHeadsPerPass) {
    const int h = h0 + hs;
    if (h < a.num_kv_heads) {
      rotate(k + krow + h * D, k_cache + prow + h * D, k_w);
      const V lo = *reinterpret_cast<const V*>(v + krow + h * D + j * P);
      const V hi = *reinterpret_cast<const V*>(v + krow + h * D + D / 2 + j * P);
      *reinterpret_cast<V*>(v_cache + prow + h * D + j * P) = lo;
      *reinterpret_cast<V*>(v_cache + prow + h * D + D / 2 + j * P) = hi;
    }
  }
}

template <typename T, int D>
hipError_t launch_typed(const RopeStoreArgs& a, hipStream_t stream) {
  const int blocks = (a.num_tokens + kRopeWaves - 1) / kRopeWaves;
  if (a.q_weight != nullptr)
    rope_kv_store_kernel<T, D, true><<<dim3(static_cast<uint32_t>(blocks)), dim3(kRopeWaves * kWave), 0, stream>>>(a);
  else
    rope_kv_store_kernel<T, D, false><<<dim3(static_cast<uint32_t>(blocks)), dim3(kRopeWaves * kWave), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_kv_store(const RopeStoreArgs& a, Dtype dtype, int32_t head_dim, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  if (dtype == Dtype::kBF16)
    return head_dim == 128 ? launch_typed<bf16_t, 128>(a, stream) : launch_typed<bf16_t, 64>(a, stream);
  return head_dim == 128 ? launch_typed<float, 128>(a, stream) : launch_typed<float, 64>(a, stream);
}

}  // namespace pa
