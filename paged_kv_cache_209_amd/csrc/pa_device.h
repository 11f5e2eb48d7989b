// Device-side helpers shared by the paged-attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kWave = 64;
constexpr int kTokensPerBlock = 256;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

// Storage types: bf16 is carried as raw 16-bit patterns, fp32 as float.
struct bf16_t {
  uint16_t bits;
};

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kBytes = 4;
};
template <>
struct Elem<bf16_t> {
  static constexpr int kBytes = 2;
};

// fp8 KV-cache element: one OCP E4M3 code (the pool's scale is applied by
// the kernels that read it).
struct fp8_t {
  uint8_t bits;
};
template <>
struct Elem<fp8_t> {
  static constexpr int kBytes = 1;
};

// Element type of the tensors a pool element type is read with (q, out and
// the in-flight K/V rows): the pool's own, bf16 for fp8 pools.
template <typename T>
struct IoElem {
  using type = T;
};
template <>
struct IoElem<fp8_t> {
  using type = bf16_t;
};

// bf16 <-> fp32. Widening is exact (the bf16 pattern is the top half of the
// fp32 pattern); narrowing rounds to nearest-even through the hardware
// converter (v_cvt_pk_bf16_f32).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Two E4M3 codes (the low or the high 16 bits of w, the first code in the
// lower byte) as a bf16 pair, the first code in the low half: gfx950's
// scaled converter with scale 1, which is exact (every E4M3 value is a bf16
// value).
template <bool kHigh>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHigh));
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  return static_cast<uint16_t>(pack_bf16x2(x, 0.0f) & 0xffffu);
}

// fp32 dot of two bf16 pairs plus an fp32 addend (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// Pairs of bf16 taken from two words: lo halves (a.lo, b.lo) and hi halves
// (a.hi, b.hi), each as one packed word with a's half in the low 16 bits.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// 2^x on the hardware unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane moves within a 16-lane row. Control codes: quad_perm(1,0,3,2),
// quad_perm(2,3,0,1), row_half_mirror, row_ror:8, row_mirror.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xf, 0xf, true));
}
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowMirror = 0x140;

// Sum over each aligned group of 8 lanes; every lane of the group gets it.
__device__ __forceinline__ float sum8(float x) {
  x += dpp_f32<kDppXor1>(x);
  x += dpp_f32<kDppXor2>(x);
  x += dpp_f32<kDppHalfMirror>(x);
  return x;
}

// Sum over each 16-lane row; every lane of the row gets it (the same
// additions, in the same order, as a butterfly over lane bits 0 to 3).
__device__ __forceinline__ float sum16(float x) {
  x = sum8(x);
  x += dpp_f32<kDppRowMirror>(x);
  return x;
}

__device__ __forceinline__ float shfl_xor_f32(float x, int mask) {
  return __shfl_xor(x, mask, kWave);
}

// The two values of x at lane positions that differ only in lane bit 5
// (halves) or bit 4 (16-lane rows), handed to every lane by one VALU swap
// (v_permlane32_swap / v_permlane16_swap, new in gfx950) instead of an LDS
// crossbar permute: `lo` is x at the position with the bit clear, `hi` with
// it set.
struct LanePair {
  float lo, hi;
};
__device__ __forceinline__ LanePair pair_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ LanePair pair_across_rows(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// A read-only int32 read at a wave-uniform index, through the constant
// address space, so that it is a scalar load: it waits on the scalar-memory
// counter, never on the queue of vector loads in flight. Only for arrays that
// no kernel of this library writes (sequence lengths, offsets).
__device__ __forceinline__ int load_uniform(const int32_t* p, int64_t i) {
  using ConstPtr = const __attribute__((address_space(4))) int32_t*;
  return ((ConstPtr)p)[i];
}

// Split-context partial results cross workgroups (and XCDs, whose L2 caches
// are not coherent with each other). They are written and read with
// agent-scope atomic stores/loads, which are coherent by themselves, so no
// cache-wide write-back or invalidate (a full fence) is ever needed: a writer
// only waits until its stores are acknowledged before bumping the counter.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int add_agent(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent_int(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One arrival on a tagged piece counter (the workspace layout describes the
// tags): raise the word to the call's tag, then add one. Both atomics go to
// the same word from the same lane, so they take effect in program order.
// Returns the count after this arrival, or -1 when the word holds a foreign
// tag above the call's own (never-cleared memory).
__device__ __forceinline__ int count_arrival(uint64_t* ctr, uint64_t tag) {
  __hip_atomic_fetch_max(ctr, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t old = __hip_atomic_fetch_add(ctr, uint64_t{1}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((old >> 16) != (tag >> 16)) return -1;
  return static_cast<int>(old & 0xFFFFu) + 1;
}

// Sets error bits in the workspace's error word.
__device__ __forceinline__ void flag_workspace(uint32_t* flags, uint32_t bits) {
  __hip_atomic_fetch_or(flags, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte agent-coherent accesses through a raw buffer descriptor (cache
// policy sc1): the descriptor covers `bytes` bytes from `base` (out-of-range
// offsets read 0 and drop writes).
typedef int i32x4_t __attribute__((ext_vector_type(4)));
constexpr int kBufferFlags = 0x00020000;  // raw, untyped dword access
constexpr int kPolicyAgent = 16;         // sc1: coherent at agent scope
constexpr int kPolicyStream = 2;         // nt: streaming, read once
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kBufferFlags);
}
__device__ __forceinline__ void store4_agent(__amdgpu_buffer_rsrc_t r, int byte_off, f32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, v), r, byte_off, 0, kPolicyAgent);
}
__device__ __forceinline__ f32x4_t load4_agent(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kPolicyAgent));
}

// Wait until every vector-memory operation this wave issued (stores included)
// has completed: s_waitcnt vmcnt(0), leaving the other counters unconstrained.
__device__ __forceinline__ void wait_vector_memory() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

}  // namespace pa
