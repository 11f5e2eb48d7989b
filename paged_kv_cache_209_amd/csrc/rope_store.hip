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
// Layout of the work: one wave per token, its heads four at a time (16 lanes
// per head); lane j of a head handles pairs [jP, jP + P) with P = D / 32,
// i.e. P consecutive elements of each half of the row, loaded and stored as
// one vector each. The loads of up to four such passes of q, k and v are
// issued together before any arithmetic.
//
// The angle is formed in fp64 (p * theta_i, reduced modulo 2 pi), so that
// positions in the tens of thousands keep full fp32 accuracy; the rotation
// itself is fp32. theta_i = base^(-2i/D) is taken as exp2(-2i/D * log2(base)):
// its relative error (~1e-15) moves an angle by far less than fp32 resolves,
// and a general fp64 pow cost a third of the kernel's time (16.0 against
// 11.5 us for the Qwen3-0.6B-shaped chunked prefill's 4096 tokens).
#include <math.h>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kRopeWaves = 4;  // tokens per workgroup (one wave each)
constexpr int kLanesPerHead = 16;
constexpr int kHeadsPerPass = kWave / kLanesPerHead;
constexpr int kBatchPasses = 4;  // passes (of kHeadsPerPass heads) whose loads are issued together

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

  // cos and sin of the lane's P angles (formed after the batch's loads are
  // issued, so that the fp64 angle arithmetic overlaps them)
  float cs[P], sn[P];
  auto angles = [&]() {
    constexpr double kTwoPi = 6.283185307179586476925;
    const double log2b = log2(static_cast<double>(a.base));
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const int i = j * P + e;
      const double theta = exp2(-2.0 * i / D * log2b);
      const double ang = static_cast<double>(pos) * theta;
      const double r = ang - kTwoPi * rint(ang * (1.0 / kTwoPi));  // |r| <= pi
      sincosf(static_cast<float>(r), &sn[e], &cs[e]);
    }
  };

  const int64_t qrow = static_cast<int64_t>(t) * a.num_q_heads * D;
  const int64_t krow = static_cast<int64_t>(t) * a.num_kv_heads * D;
  const int64_t prow = static_cast<int64_t>(slot) * a.num_kv_heads * D;
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  T* q_out = static_cast<T*>(a.q_out);
  T* k_cache = static_cast<T*>(a.k_cache);
  T* v_cache = static_cast<T*>(a.v_cache);

  // Rotates the two P-element pieces (lo, hi) of one head row and writes them
  // to dst. With NORM the row is first divided by its root mean square (the
  // 16 lanes of the head, one DPP row, sum their squares) and multiplied
  // by the per-dimension weight (wlo, whi).
  auto rotate = [&](const V& lo, const V& hi, const V& wlo, const V& whi, T* dst) {
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
      static_assert(kLanesPerHead == 16, "a head's lanes are one 16-lane row");
      ss = sum16(ss);  // DPP within the head's row of 16 lanes
      const float inv = 1.0f / sqrtf(ss * (1.0f / D) + a.eps);
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
  auto piece = [&](const T* row) { return *reinterpret_cast<const V*>(row); };

  V wq_lo{}, wq_hi{}, wk_lo{}, wk_hi{};
  if constexpr (NORM) {
    const T* q_w = static_cast<const T*>(a.q_weight);
    const T* k_w = static_cast<const T*>(a.k_weight);
    wq_lo = piece(q_w + j * P);
    wq_hi = piece(q_w + D / 2 + j * P);
    wk_lo = piece(k_w + j * P);
    wk_hi = piece(k_w + D / 2 + j * P);
  }

  // The token's q, k and v pieces of up to kBatchPasses passes per tensor are
  // all loaded before any of them is rotated or stored, so a wave waits for
  // memory once per batch rather than once per pass. (q_out may be q itself:
  // every lane reads its own pieces before it writes them.) A token with a
  // negative slot rotates its q only.
  const int nq = a.num_q_heads;
  const int nkv = slot >= 0 ? a.num_kv_heads : 0;
  const int passes = (max(nq, nkv) + kHeadsPerPass - 1) / kHeadsPerPass;
  auto batch = [&](int p0) {
    V qlo[kBatchPasses], qhi[kBatchPasses], klo[kBatchPasses], khi[kBatchPasses], vlo[kBatchPasses],
        vhi[kBatchPasses];
#pragma unroll
    for (int p = 0; p < kBatchPasses; ++p) {
      const int h = (p0 + p) * kHeadsPerPass + hs;
      if (h < nq) {
        qlo[p] = piece(q + qrow + h * D + j * P);
        qhi[p] = piece(q + qrow + h * D + D / 2 + j * P);
      }
      if (h < nkv) {
        klo[p] = piece(k + krow + h * D + j * P);
        khi[p] = piece(k + krow + h * D + D / 2 + j * P);
        vlo[p] = piece(v + krow + h * D + j * P);
        vhi[p] = piece(v + krow + h * D + D / 2 + j * P);
      }
    }
    if (p0 == 0) angles();
#pragma unroll
    for (int p = 0; p < kBatchPasses; ++p) {
      const int h = (p0 + p) * kHeadsPerPass + hs;
      if (h < nq) rotate(qlo[p], qhi[p], wq_lo, wq_hi, q_out + qrow + h * D);
      if (h < nkv) {
        rotate(klo[p], khi[p], wk_lo, wk_hi, k_cache + prow + h * D);
        *reinterpret_cast<V*>(v_cache + prow + h * D + j * P) = vlo[p];
        *reinterpret_cast<V*>(v_cache + prow + h * D + D / 2 + j * P) = vhi[p];
      }
    }
  };
  // One batch (the usual case, up to 16 heads) runs outside any loop, so the
  // compiler sees no back edge carrying loads in flight and waits only once.
  if (passes <= kBatchPasses) {
    batch(0);
  } else {
    for (int p0 = 0; p0 < passes; p0 += kBatchPasses) batch(p0);
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
