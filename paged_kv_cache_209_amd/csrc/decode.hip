// Paged decode attention: one query token per sequence attends over the K/V
// rows its block table names ("Nano-vLLM System Architecture Analysis",
// section 2, "Attention with Paged Cache": decode attends over all cached K/V
// of the sequence's blocks). Unlike a gather-then-attend implementation, the
// rows are streamed from the pool in place and never copied. The pool element
// type is fp32, bf16 or fp8 (E4M3 codes, read with bf16 q and out; each
// lane's codes become exact bf16 pairs at consume time, the K pool's scale is
// in the softmax scale and the V pool's is applied to the output).
//
// Work split. An item is (sequence, group of GT query heads sharing one KV
// head); it costs one unit per 64 tokens of its context plus a fixed cost for
// finishing it. The units of all items, ordered sequence-major, are cut into
// equal contiguous ranges, one per workgroup, so every workgroup has about
// the same time of work however ragged the contexts are. A range may hold the
// tail of one item, whole items and the head of another; each such piece is a
// segment.
//
// Data flow inside a workgroup (256 threads = 4 wave64, gfx950):
//   * the 4 waves take 16-token chunks of a segment round-robin, each wave
//     keeping the next chunk's loads in flight while it computes;
//   * in a chunk, lane l handles tokens (l / 8) and 8 + (l / 8); its 8-lane
//     group reads each token's head row as 16-byte pieces, so one load
//     instruction covers whole 128-byte lines of 8 tokens (coalesced), straight
//     into registers: every lane consumes exactly the bytes it loads, so no
//     LDS round trip is needed;
//   * q.k partial dot products (v_dot2_f32_bf16 for bf16) are summed over the
//     8 lanes with three DPP adds; every lane of the group then holds the score;
//   * each 8-lane group keeps its own online-softmax state (running max m, sum
//     l, fp32 accumulator for its 16 dims) per query head; the max is only
//     refreshed when a score exceeds it by more than 2^8, which keeps the
//     rescale off the common path without risking overflow;
//   * p.V pairs two tokens per v_dot2_f32_bf16 (p rounded to bf16, and l
//     accumulated from the same rounded p so the weights stay normalised);
//   * at the end of a segment the 8 groups of a wave merge by VALU lane
//     swaps and a row rotate (no LDS traffic), the 4 waves through LDS; a
//     whole item is written as the final output, a piece as a (normalised
//     output, log2-sum-exp) partial.
//   * consecutive segments overlap: the next segment's block-table window,
//     query rows and first chunk load while the current one finishes;
//   * the pieces of a split item are counted on a device-scope counter per
//     item, one count per wave and piece, when the workgroup ends; the wave
//     whose count completes the item merges all its pieces, in piece order,
//     so results are bit-identical from run to run and no floating-point
//     atomics are used.
#include <math.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kDecodeWaves = 4;
constexpr int kDecodeThreads = kDecodeWaves * kWave;
constexpr int kChunk = 16;           // tokens per wave iteration
constexpr float kStaleMaxSlack = 8.0f;  // log2 units the running max may lag by
constexpr float kEmptyMax = -1.0e30f;   // running max of a stream with no token yet

template <typename T, int D>
struct DecodeShape {
  static constexpr int kRowBytes = D * Elem<T>::kBytes;
  static constexpr int kVecs = kRowBytes / 128;  // 16-byte pieces per lane per row
  static constexpr int kElemsPerVec = 16 / Elem<T>::kBytes;
  static constexpr int kWords = kVecs * 4;  // 32-bit words per lane per row
  static constexpr int kLaneElems = kVecs * kElemsPerVec;
  static constexpr int kVecStride = 128 / Elem<T>::kBytes;  // elements between a lane's pieces
  // 32-bit words of the lane's query elements (q has the pool's element type,
  // bf16 for fp8 pools)
  static constexpr int kQWords = kLaneElems * Elem<typename IoElem<T>::type>::kBytes / 4;
  static_assert(kRowBytes % 128 == 0, "head row must be a multiple of 128 bytes");
};

// Element index (within a head row) of lane element j for sub-lane sl.
template <typename T, int D>
__device__ __forceinline__ int lane_dim(int sl, int j) {
  using S = DecodeShape<T, D>;
  return (j / S::kElemsPerVec) * S::kVecStride + sl * S::kElemsPerVec + (j % S::kElemsPerVec);
}

template <typename T>
__device__ __forceinline__ void store_out(T* p, float x);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float x) {
  *p = x;
}
template <>
__device__ __forceinline__ void store_out<bf16_t>(bf16_t* p, float x) {
  p->bits = to_bf16_bits(x);
}

// Leading tokens of every context read with cache-allocating loads. A
// prefix cache shares blocks only at the start of contexts (a shared system
// prompt), so those rows may be read again by other sequences of the same
// launch and are worth keeping in the caches; every later row is read once
// and streams past them.
constexpr int kCachedLeadTokens = 4 * kTokensPerBlock;

// Loads the lane's words of one head row: kVecs 16-byte pieces.
template <typename T, int D, bool kStream>
__device__ __forceinline__ void load_row(const T* row, int sl, uint32_t (&w)[DecodeShape<T, D>::kWords]) {
  using S = DecodeShape<T, D>;
#pragma unroll
  for (int v = 0; v < S::kVecs; ++v) {
    // Streaming (non-temporal) loads where every K/V byte is used once: on
    // MI355X they sustain about 10% more bandwidth than cached loads.
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(row + v * S::kVecStride + sl * S::kElemsPerVec);
    const u32x4_t x = kStream ? __builtin_nontemporal_load(p) : *p;
    w[4 * v + 0] = x[0];
    w[4 * v + 1] = x[1];
    w[4 * v + 2] = x[2];
    w[4 * v + 3] = x[3];
  }
}

// Partial q.k over the lane's elements.
// sum8 of every element of a and b, the same adds in the same order, taken
// one butterfly step at a time across all of them.
template <int N>
__device__ __forceinline__ void sum8_steps(float (&a)[N], float (&b)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    a[i] += dpp_f32<kDppXor1>(a[i]);
    b[i] += dpp_f32<kDppXor1>(b[i]);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    a[i] += dpp_f32<kDppXor2>(a[i]);
    b[i] += dpp_f32<kDppXor2>(b[i]);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    a[i] += dpp_f32<kDppHalfMirror>(a[i]);
    b[i] += dpp_f32<kDppHalfMirror>(b[i]);
  }
}

// fp32 dot of two bf16 pairs with a zero addend: v_dot2_f32_bf16 with an
// inline 0 (one ALU instruction, no memory access).
__device__ __forceinline__ float dot2_bf16_zero(uint32_t a, uint32_t b) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

template <typename T, int D>
__device__ __forceinline__ float partial_dot(const uint32_t (&qw)[DecodeShape<T, D>::kQWords],
                                             const uint32_t (&kw)[DecodeShape<T, D>::kWords]) {
  using S = DecodeShape<T, D>;
  float s0 = 0.0f, s1 = 0.0f;
  if constexpr (Elem<T>::kBytes == 1) {
    // fp8 codes, four per word, become bf16 pairs (exact) for the bf16 q. The
    // chain starts with the three-operand form and an inline 0 addend: left
    // to itself the compiler zeroes a register for the two-operand form, one
    // more VALU instruction per chain in a VALU-bound loop (8 per chunk).
    s0 = dot2_bf16_zero(qw[0], fp8x2_to_bf16x2<false>(kw[0]));
    s0 = dot2_bf16(qw[1], fp8x2_to_bf16x2<true>(kw[0]), s0);
#pragma unroll
    for (int w = 1; w < S::kWords; ++w) {
      s0 = dot2_bf16(qw[2 * w], fp8x2_to_bf16x2<false>(kw[w]), s0);
      s0 = dot2_bf16(qw[2 * w + 1], fp8x2_to_bf16x2<true>(kw[w]), s0);
    }
    return s0;  // one chain: the 8 (row, head) chains of a chunk give the overlap
  } else if constexpr (Elem<T>::kBytes == 2) {
#pragma unroll
    for (int w = 0; w < S::kWords; w += 2) {
      s0 = dot2_bf16(qw[w], kw[w], s0);
      s1 = dot2_bf16(qw[w + 1], kw[w + 1], s1);
    }
  } else {
#pragma unroll
    for (int w = 0; w < S::kWords; w += 2) {
      s0 = fmaf(__uint_as_float(qw[w]), __uint_as_float(kw[w]), s0);
      s1 = fmaf(__uint_as_float(qw[w + 1]), __uint_as_float(kw[w + 1]), s1);
    }
  }
  return s0 + s1;
}

// Online-softmax state of one lane: per query head, running max m (log2
// units), running sum l and the accumulator of the lane's head dims.
template <int GT, int E>
struct LaneState {
  float m[GT];
  float l[GT];
  float acc[GT][E];
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      m[g] = kEmptyMax;
      l[g] = 0.0f;
#pragma unroll
      for (int j = 0; j < E; ++j) acc[g][j] = 0.0f;
    }
  }
};

// K/V words of one 16-token chunk for this lane: tokens a = c0 + ts and
// b = c0 + 8 + ts, and whether they lie inside the range.
template <int W>
struct Chunk {
  uint32_t ka[W], kb[W], va[W], vb[W];
};

template <typename T, int D, bool FUSED, bool kStream = true>
__device__ __forceinline__ void load_chunk(Chunk<DecodeShape<T, D>::kWords>& c, const T* kpool, const T* vpool,
                                           int block, int64_t row_stride, int c0, int t_end, int ts, int sl,
                                           const T* knew, const T* vnew, int new_pos) {
  // Wave-uniform base of the chunk's first row plus a small per-lane offset.
  // Rows past the range are never read: their lanes re-read the last valid
  // row (always in the same block as the chunk start) and get zero weight.
  // With FUSED, the row at position new_pos (the step's new token) comes from
  // the call's in-flight knew/vnew rows instead of the pool.
  const int64_t r0 = static_cast<int64_t>(block) * kTokensPerBlock + (c0 % kTokensPerBlock);
  const T* kb = kpool + r0 * row_stride;
  const T* vb = vpool + r0 * row_stride;
  const int last = t_end - 1 - c0;
  const int rs = static_cast<int>(row_stride);
  const int ra = min(ts, last), rb = min(ts + 8, last);
  const T* ka = kb + ra * rs;
  const T* va = vb + ra * rs;
  const T* kbb = kb + rb * rs;
  const T* vbb = vb + rb * rs;
  if constexpr (FUSED) {
    const int nr = new_pos - c0;
    if (ra == nr) {
      ka = knew;
      va = vnew;
    }
    if (rb == nr) {
      kbb = knew;
      vbb = vnew;
    }
  }
  load_row<T, D, kStream>(ka, sl, c.ka);
  load_row<T, D, kStream>(kbb, sl, c.kb);
  load_row<T, D, kStream>(va, sl, c.va);
  load_row<T, D, kStream>(vbb, sl, c.vb);
}

// Loads a chunk whose 16 rows all lie inside the range and none of which is
// the call's new token (every chunk of a wave that has a later chunk in the
// same segment): no row clamp and no new-token check, and the lane's rows sit
// at fixed byte offsets (off_a, off_b) from the chunk's first row, so the
// loads go through a raw buffer descriptor of the chunk's 16 rows (a scalar
// base) with the offset as the only per-lane operand: no per-chunk vector
// address arithmetic.
template <typename T, int D, bool kStream>
__device__ __forceinline__ void load_full_chunk(Chunk<DecodeShape<T, D>::kWords>& c, const T* kpool, const T* vpool,
                                                int block, int64_t row_stride, int c0, uint32_t off_a,
                                                uint32_t off_b) {
  using S = DecodeShape<T, D>;
  const int64_t r0 = static_cast<int64_t>(block) * kTokensPerBlock + (c0 % kTokensPerBlock);
  const uint32_t bytes = static_cast<uint32_t>(kChunk * row_stride * sizeof(T));
  const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(kpool + r0 * row_stride, bytes);
  const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(vpool + r0 * row_stride, bytes);
  // cache policy: nt (streaming) where every byte is read once
  constexpr int kPolicy = kStream ? kPolicyStream : 0;
  const auto row = [&](__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t (&w)[S::kWords]) {
#pragma unroll
    for (int v = 0; v < S::kVecs; ++v) {
      const i32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, off, v * 128, kPolicy);
#pragma unroll
      for (int k = 0; k < 4; ++k) w[4 * v + k] = static_cast<uint32_t>(x[k]);
    }
  };
  row(kr, off_a, c.ka);
  row(kr, off_b, c.kb);
  row(vr, off_a, c.va);
  row(vr, off_b, c.vb);
}

// Block ids of a segment, one per lane, 64 at a time. Each chunk takes its id
// with a lane read (no memory wait), so block-table reads never sit in the
// in-order queue of vector loads behind the K/V stream.
struct BlockWindow {
  const int32_t* table;
  int base;   // first block index held
  int limit;  // one past the segment's last block index
  int id;     // this lane's block id: table[base + lane]
  __device__ __forceinline__ void fill(int b, int lane) {
    base = b;
    id = b + lane < limit ? table[b + lane] : 0;
    // Complete the load here, on this (rare) path, so that no later
    // instruction inherits a pending table read and waits for the whole
    // queue of K/V loads in front of it.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }
  // Starts loading the window at b without waiting: for a segment that
  // follows the current one, whose ids are first needed a whole segment later.
  __device__ __forceinline__ void fill_async(int b, int lane) {
    base = b;
    id = b + lane < limit ? table[b + lane] : 0;
  }
  __device__ __forceinline__ int get(int b, int lane) {
    if (b - base >= kWave) fill(b - (b - base) % kWave, lane);  // wave-uniform, rare
    return __builtin_amdgcn_readlane(id, b - base);
  }
};

// The lane's words of query head g, read from the wave's copy of the group's
// query rows in LDS (the same pieces of the row that the lane loads of K).
template <typename T, int D>
__device__ __forceinline__ void q_words(const u32x4_t* sq, int g, int sl, uint32_t (&w)[DecodeShape<T, D>::kQWords]) {
  using S = DecodeShape<T, D>;
  if constexpr (Elem<T>::kBytes == 1) {
    // fp8 pools: the lane's 16 consecutive dims of the bf16 query row
    const u32x4_t x0 = sq[(g * D + sl * 16) / 8];
    const u32x4_t x1 = sq[(g * D + sl * 16) / 8 + 1];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      w[k] = x0[k];
      w[4 + k] = x1[k];
    }
    return;
  }
#pragma unroll
  for (int v = 0; v < S::kVecs; ++v) {
    const u32x4_t x = sq[(g * D + v * S::kVecStride + sl * S::kElemsPerVec) * Elem<T>::kBytes / 16];
    w[4 * v + 0] = x[0];
    w[4 * v + 1] = x[1];
    w[4 * v + 2] = x[2];
    w[4 * v + 3] = x[3];
  }
}

// fp8 pools: the lane's query words of every head of the group, held in
// registers for a whole segment (32 VGPRs at 4 heads); the wider bf16 and
// fp32 rows would not fit, so those kernels read them from LDS per chunk.
template <typename T, int D, int GT>
using QRegs = uint32_t[Elem<T>::kBytes == 1 ? GT : 1][DecodeShape<T, D>::kQWords];

// One chunk: scores, the lazy max update and the p.V accumulation. kFull: all
// 16 rows lie inside the range (va and vb are not consulted).
template <typename T, int D, int GT, bool kFull = false>
__device__ __forceinline__ void consume_chunk(LaneState<GT, DecodeShape<T, D>::kLaneElems>& st,
                                              const Chunk<DecodeShape<T, D>::kWords>& c, const u32x4_t* sq, int sl,
                                              bool va, bool vb, float sc, const QRegs<T, D, GT>& qr) {
  constexpr int W = DecodeShape<T, D>::kWords;
  constexpr int E = DecodeShape<T, D>::kLaneElems;
  // Per query head: the two rows' raw dots, and their exponents
  // e = s - m = dot * sc - m (log2 units) against the running max, each one
  // fused multiply-add; the lazy-max test looks at the same exponents.
  float xa[GT], xb[GT], ea[GT], eb[GT];
  bool need = false;
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    uint32_t qw[DecodeShape<T, D>::kQWords];
    if constexpr (Elem<T>::kBytes == 1) {
#pragma unroll
      for (int k = 0; k < DecodeShape<T, D>::kQWords; ++k) qw[k] = qr[g][k];
    } else {
      q_words<T, D>(sq, g, sl, qw);
    }
    xa[g] = partial_dot<T, D>(qw, c.ka);
    xb[g] = partial_dot<T, D>(qw, c.kb);
  }
  // The lane-group sums, one DPP step at a time over all 2 GT dots, so that
  // each step's adds are independent of one another (a dependent DPP read
  // right after its VALU write costs wait states).
  sum8_steps(xa, xb);
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    ea[g] = kFull || va ? fmaf(xa[g], sc, -st.m[g]) : -INFINITY;
    eb[g] = kFull || vb ? fmaf(xb[g], sc, -st.m[g]) : -INFINITY;
    need |= fmaxf(ea[g], eb[g]) > kStaleMaxSlack;
  }
  if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float sa = kFull || va ? xa[g] * sc : -INFINITY;
      const float sb = kFull || vb ? xb[g] * sc : -INFINITY;
      const float mn = fmaxf(st.m[g], fmaxf(sa, sb));
      const float alpha = exp2_fast(st.m[g] - mn);
      st.l[g] *= alpha;
#pragma unroll
      for (int j = 0; j < E; ++j) st.acc[g][j] *= alpha;
      st.m[g] = mn;
      ea[g] = kFull || va ? fmaf(xa[g], sc, -mn) : -INFINITY;
      eb[g] = kFull || vb ? fmaf(xb[g], sc, -mn) : -INFINITY;
    }
  }
  if constexpr (Elem<T>::kBytes <= 2) {
    uint32_t vp[E];
    if constexpr (Elem<T>::kBytes == 1) {
      // fp8: word w holds elements 4w .. 4w+3 of each row. The two rows'
      // codes are interleaved first (a0 b0 a1 b1 and a2 b2 a3 b3), so that each
      // conversion yields the (row a, row b) pair of one element directly.
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const uint32_t x = __builtin_amdgcn_perm(c.vb[w], c.va[w], 0x05010400u);
        const uint32_t y = __builtin_amdgcn_perm(c.vb[w], c.va[w], 0x07030602u);
        vp[4 * w] = fp8x2_to_bf16x2<false>(x);
        vp[4 * w + 1] = fp8x2_to_bf16x2<true>(x);
        vp[4 * w + 2] = fp8x2_to_bf16x2<false>(y);
        vp[4 * w + 3] = fp8x2_to_bf16x2<true>(y);
      }
    } else {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        vp[2 * w] = pair_lo(c.va[w], c.vb[w]);
        vp[2 * w + 1] = pair_hi(c.va[w], c.vb[w]);
      }
    }
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const uint32_t pp = pack_bf16x2(exp2_fast(ea[g]), exp2_fast(eb[g]));
      st.l[g] = dot2_bf16(pp, 0x3F803F80u, st.l[g]);  // + p_a + p_b as rounded
#pragma unroll
      for (int j = 0; j < E; ++j) st.acc[g][j] = dot2_bf16(pp, vp[j], st.acc[g][j]);
    }
  } else {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float pa = exp2_fast(ea[g]);
      const float pb = exp2_fast(eb[g]);
      st.l[g] += pa + pb;
#pragma unroll
      for (int j = 0; j < E; ++j)
        st.acc[g][j] = fmaf(pa, __uint_as_float(c.va[j]), fmaf(pb, __uint_as_float(c.vb[j]), st.acc[g][j]));
    }
  }
}

// Work units (64 tokens each) of a context, with the length clamped to
// [0, max_context_len] (lengths outside [1, max_context_len] are a caller
// error; clamping keeps every read inside the block table and every loop
// finite).
__device__ __forceinline__ int context_units(int ctx, int max_ctx) {
  ctx = min(max(ctx, 0), max_ctx);
  return (ctx + kDecodeUnitTokens - 1) / kDecodeUnitTokens;
}

// The U cost units are split into G equal contiguous ranges, one per
// workgroup: workgroup w owns [start(w), start(w + 1)). An item costs one
// unit per 64 tokens of context plus kItemCost units ahead of them that hold
// no tokens: they stand for the fixed work of finishing a segment (the
// cross-wave merge and its barriers), so ranges of many short items carry
// fewer tokens and all ranges take about the same time. The owners of an
// item's real units are consecutive workgroups.
constexpr int kItemCost = kDecodeItemCost;

// Cost units of one item of a sequence (none for an empty context).
__device__ __forceinline__ int item_cost(int ctx, int max_ctx) {
  const int nu = context_units(ctx, max_ctx);
  return nu > 0 ? nu + kItemCost : 0;
}

struct EvenSplit {
  int64_t U, G;
  __device__ __forceinline__ int64_t start(int64_t w) const { return U * w / G; }
  __device__ __forceinline__ int64_t owner(int64_t u) const { return ((u + 1) * G - 1) / U; }
};

// The piece of one item (sequence, head group) that lies in a workgroup's
// unit range: the tokens it covers and the blocks that hold them.
struct Segment {
  int seq, hg;
  int t_lo, t_hi;        // tokens [t_lo, t_hi)
  int b_lo, b_hi;        // blocks [b_lo, b_hi) holding them
  int last_pos;          // position of the sequence's last token (the step's new one)
  int n_parts;           // pieces of the item over all workgroups
  int64_t first_owner;   // workgroup holding the item's first piece
  int64_t item_first;    // the item's first cost unit (a virtual one)
};

// Walks the segments of the unit range [u, u_end) in order, item by item:
// after the first item the walk only steps forward, so it divides only for
// the owners of items that cross the range's ends. All its state is
// wave-uniform (kept in scalar registers).
struct SegmentWalk {
  EvenSplit split;
  int64_t u, u_end;    // units still to walk
  int64_t range_lo;    // first unit of the workgroup's range
  int64_t item_first;  // first cost unit of the current item (a virtual one)
  int w;               // the workgroup (owner of the range)
  int seq, hg;         // the current item
  int ctx;             // its sequence's length as given
  int B, HG, max_ctx;
  const int32_t* context_lens;

  // Places the walk at unit u0 of sequence seq0, whose units start at
  // seq_base and whose length is ctx0.
  __device__ __forceinline__ void start(int64_t u0, int64_t u1, int seq0, int64_t seq_base, int ctx0) {
    u = u0;
    u_end = u1;
    range_lo = u0;
    seq = seq0;
    ctx = ctx0;
    const int64_t span = context_units(ctx0, max_ctx) + kItemCost;
    hg = static_cast<int>((u0 - seq_base) / span);
    item_first = seq_base + hg * span;
  }

  // The next segment with tokens, if any is left in the range.
  __device__ __forceinline__ bool next(Segment& s) {
    while (u < u_end) {
      const int64_t span = context_units(ctx, max_ctx) + kItemCost;  // cost units of the item
      const int64_t real_first = item_first + kItemCost;
      const int64_t item_end = item_first + span;
      const int64_t seg_end = u_end < item_end ? u_end : item_end;
      const int64_t lo = u > real_first ? u : real_first;
      const bool has_tokens = lo < seg_end;
      if (has_tokens) {
        s.seq = seq;
        s.hg = hg;
        s.t_lo = static_cast<int>(lo - real_first) * kDecodeUnitTokens;
        s.t_hi = min(min(ctx, max_ctx), static_cast<int>(seg_end - real_first) * kDecodeUnitTokens);
        s.last_pos = min(ctx, max_ctx) - 1;
        s.b_lo = s.t_lo / kTokensPerBlock;
        s.b_hi = (s.t_hi + kTokensPerBlock - 1) / kTokensPerBlock;
        // lo < seg_end <= u_end: the item's real units start before the
        // range ends, and in it unless they start before it
        s.first_owner = real_first >= range_lo ? w : split.owner(real_first);
        const int64_t last_owner = item_end <= u_end ? w : split.owner(item_end - 1);
        s.n_parts = static_cast<int>(last_owner - s.first_owner + 1);
        s.item_first = item_first;
      }
      u = seg_end;
      if (u == item_end) {  // on to the next item
        item_first = item_end;
        if (++hg == HG) {  // ... of the next sequence with work (an empty one has no units)
          hg = 0;
          ++seq;
          if (u < u_end) {
            int c = load_uniform(context_lens, seq);
            while (context_units(c, max_ctx) == 0 && seq < B - 1) c = load_uniform(context_lens, ++seq);
            ctx = c;
          }
        }
      }
      if (has_tokens) return true;
    }
    return false;
  }
};

// Combines the pieces of one split item into its final output, run by one
// wave: o = sum_j 2^(lse_j - M) o_j / sum_j 2^(lse_j - M), M = max_j lse_j,
// folded in piece order with a running maximum (so the result does not depend
// on which workgroup computed which piece). Pieces are read a batch at a time,
// all loads of a batch in flight together, so a merge costs one memory round
// trip per batch rather than one per piece.
// The slot of piece p of an item: a workgroup stores its first segment in
// slot 2w and a later one (only its last can be a piece of a split item) in
// slot 2w + 1. Every piece but the first is its holder's first segment; the
// first piece is too when its holder's range starts inside the item's
// virtual units (real units of earlier items would come first otherwise).
__device__ __forceinline__ int64_t piece_slot(const EvenSplit& split, int64_t first_owner, int p,
                                              int64_t item_first) {
  const int64_t w = first_owner + p;
  return p > 0 || split.start(w) >= item_first ? 2 * w : 2 * w + 1;
}

template <typename T, int D, int GT, bool kOutScale>
__device__ __forceinline__ void merge_item(const DecodeArgs& a, T* out, int64_t unit0, const EvenSplit& split,
                                           int64_t first_owner, int n_parts, int64_t item_first, int lane) {
  constexpr int DL = D / kWave;                             // dims per lane
  constexpr int NB = GT >= 4 ? 4 : (GT == 2 ? 8 : 16);      // pieces per batch
  float m[GT], den[GT], num[GT][DL];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    m[g] = -INFINITY;
    den[g] = 0.0f;
#pragma unroll
    for (int k = 0; k < DL; ++k) num[g][k] = 0.0f;
  }
  for (int p0 = 0; p0 < n_parts; p0 += NB) {
    float lv[GT][NB], ov[GT][NB][DL];
#pragma unroll
    for (int g = 0; g < GT; ++g) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int64_t row = piece_slot(split, first_owner, min(p0 + j, n_parts - 1), item_first) * GT + g;
        lv[g][j] = load_agent(a.part_lse + row);
#pragma unroll
        for (int k = 0; k < DL; ++k) ov[g][j][k] = load_agent(a.part_out + row * D + k * kWave + lane);
      }
    }
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      float mn = m[g];
#pragma unroll
      for (int j = 0; j < NB; ++j)
        if (p0 + j < n_parts) mn = fmaxf(mn, lv[g][j]);
      const float r = exp2_fast(m[g] - mn);
      den[g] *= r;
#pragma unroll
      for (int k = 0; k < DL; ++k) num[g][k] *= r;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (p0 + j < n_parts) {
          const float f = exp2_fast(lv[g][j] - mn);
          den[g] += f;
#pragma unroll
          for (int k = 0; k < DL; ++k) num[g][k] += f * ov[g][j][k];
        }
      }
      m[g] = mn;
    }
  }
#pragma unroll
  for (int g = 0; g < GT; ++g)
#pragma unroll
    for (int k = 0; k < DL; ++k) {
      const float o = num[g][k] / den[g];
      store_out<T>(out + (unit0 + g) * D + k * kWave + lane, kOutScale ? o * a.v_scale : o);
    }
}

template <typename T, int D, int GT, bool FUSED>
__global__ __launch_bounds__(kDecodeThreads, 2) void paged_decode_kernel(DecodeArgs a) {
  using S = DecodeShape<T, D>;
  using IoT = typename IoElem<T>::type;  // q and out (bf16 for fp8 pools)
  constexpr bool kOutScale = Elem<T>::kBytes == 1;  // fp8 pools: out *= the V pool's scale
  constexpr int W = S::kWords;
  constexpr int E = S::kLaneElems;
  constexpr int kStride = kDecodeWaves * kChunk;  // tokens between a wave's chunks
  constexpr int kQVecs = GT * D * Elem<IoT>::kBytes / 16;  // 16-byte pieces of a group's query rows
  constexpr int kQPerLane = (kQVecs + kWave - 1) / kWave;
  __shared__ int s_wsum[kDecodeWaves];
  __shared__ int s_loc[3];
  __shared__ float s_acc[kDecodeWaves][GT][D];
  __shared__ float s_m[kDecodeWaves][GT];
  __shared__ float s_l[kDecodeWaves][GT];
  __shared__ u32x4_t s_q[kDecodeWaves][kQVecs];  // each wave's copy of the segment's query rows

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // wave index made provably wave-uniform, so per-wave addresses (block-table
  // entries) are scalar loads that do not queue behind the vector loads
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const u32x4_t* sq = s_q[wave];
  const int ts = lane >> 3;  // token slot within a chunk (and ts + 8)
  const int sl = lane & 7;   // sub-lane: which 16-byte pieces of the row
  const int B = a.num_seqs;
  const int HG = a.num_q_heads / GT;  // head groups per sequence
  const int group = a.num_q_heads / a.num_kv_heads;
  const int groups_per_kv = group / GT;

  // ---- 0. (FUSED) Store the step's new K/V rows, one token per sequence,
  // token t by workgroup t mod grid. Nothing in this launch reads those pool
  // rows: each sequence's new position is read from the in-flight rows.
  if constexpr (FUSED) {
    const int pieces = a.num_kv_heads * D * Elem<T>::kBytes / 16;  // 16-byte pieces per token row
    for (int t = blockIdx.x; t < B; t += gridDim.x) {
      const int slot = load_uniform(a.slot_mapping, t);
      if (slot < 0) continue;
      for (int p = tid; p < 2 * pieces; p += kDecodeThreads) {
        const bool is_v = p >= pieces;
        const int pp = is_v ? p - pieces : p;
        const u32x4_t* src = static_cast<const u32x4_t*>(is_v ? a.v_new : a.k_new) + static_cast<int64_t>(t) * pieces;
        u32x4_t* dst = static_cast<u32x4_t*>(const_cast<void*>(is_v ? a.v_cache : a.k_cache)) +
                       static_cast<int64_t>(slot) * pieces;
        dst[pp] = __builtin_nontemporal_load(src + pp);
      }
    }
  }

  // ---- 1. Cost units: item (seq i, head group hg) costs one unit per 64
  // context tokens plus kItemCost units of fixed work, ordered seq-major.
  // Count them with a workgroup-wide scan over the sequences.
  const int per = (B + kDecodeThreads - 1) / kDecodeThreads;
  int mine = 0;
  for (int k = 0; k < per; ++k) {
    const int i = tid * per + k;
    if (i < B) mine += item_cost(a.context_lens[i], a.max_context_len);
  }
  // Inclusive prefix sum of `mine` over the workgroup: within each wave by
  // lane shuffles, then across the waves through LDS (one barrier).
  int incl = mine;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int t = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += t;
  }
  if (lane == kWave - 1) s_wsum[wave] = incl;
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int k = 0; k < kDecodeWaves; ++k) {
    const int v = s_wsum[k];
    if (k < wave) incl += v;
    total += v;
  }
  const int64_t U = static_cast<int64_t>(HG) * total;
  // With no more workgroups than units every workgroup owns at least one
  // unit, so the owners of an item's units are consecutive workgroups, and
  // only the first and the last segment of a range can be pieces of items
  // that other workgroups share.
  const int64_t G = min(static_cast<int64_t>(gridDim.x), U);
  const int w = blockIdx.x;
  if (w >= G) return;
  const EvenSplit split{U, G};
  const int64_t u_begin = split.start(w);
  const int64_t u_end = split.start(w + 1);

  // ---- 2. The sequence holding u_begin: the thread whose sequences span it
  // walks them.
  {
    const int64_t lo = static_cast<int64_t>(HG) * (incl - mine);
    const int64_t hi = static_cast<int64_t>(HG) * incl;
    if (u_begin >= lo && u_begin < hi) {
      int64_t base = lo;
      for (int k = 0; k < per && tid * per + k < B; ++k) {
        const int i = tid * per + k;
        const int64_t span = static_cast<int64_t>(HG) * item_cost(a.context_lens[i], a.max_context_len);
        if (u_begin < base + span) {
          s_loc[0] = i;
          s_loc[1] = static_cast<int>(base / HG);  // cost units of all earlier sequences
          s_loc[2] = a.context_lens[i];            // its length, so the walk need not read it again
          break;
        }
        base += span;
      }
    }
  }
  __syncthreads();
  SegmentWalk walk;
  walk.split = split;
  walk.w = w;
  walk.B = B;
  walk.HG = HG;
  walk.max_ctx = a.max_context_len;
  walk.context_lens = a.context_lens;
  // values read back from LDS are uniform; say so, so that the walk stays in
  // scalar registers
  walk.start(u_begin, u_end, __builtin_amdgcn_readfirstlane(s_loc[0]),
             static_cast<int64_t>(HG) * __builtin_amdgcn_readfirstlane(s_loc[1]),
             __builtin_amdgcn_readfirstlane(s_loc[2]));

  const int64_t row_stride = static_cast<int64_t>(a.num_kv_heads) * D;
  const float sc = a.scale_log2;
  IoT* out = static_cast<IoT*>(a.out);
  const IoT* q = static_cast<const IoT*>(a.q);
  const T* k_cache = static_cast<const T*>(a.k_cache);
  const T* v_cache = static_cast<const T*>(a.v_cache);
  // (FUSED) the in-flight K/V rows: token t = sequence t, [num_seqs, Hkv, D]
  const T* knew_base = static_cast<const T*>(a.k_new);
  const T* vnew_base = static_cast<const T*>(a.v_new);
  const int nkv = a.num_kv_heads;
  auto new_row = [nkv](const T* base, int seq, int kvh) -> const T* {
    return FUSED ? base + (static_cast<int64_t>(seq) * nkv + kvh) * D : nullptr;
  };
  LaneState<GT, E> st;

  // ---- 3. Stream the segments. While a segment streams, the next one's
  // block-table window and query rows are already loading, and the tail of
  // the segment issues the next segment's first chunk, so no wave drains its
  // loads between segments. A wave with no token in a (short) segment takes
  // one chunk at the segment's first row with every token masked, so every
  // wave runs the same steps.
  Segment cs;
  // A range that holds only virtual units has nothing to do.
  if (!walk.next(cs)) return;
  BlockWindow bw;
  bw.table = a.block_tables + static_cast<int64_t>(cs.seq) * a.max_blocks_per_seq;
  bw.limit = cs.b_hi;
  u32x4_t qv[kQPerLane];
  {
    const int hq0 = (cs.hg / groups_per_kv) * group + (cs.hg % groups_per_kv) * GT;
    const u32x4_t* qsrc = reinterpret_cast<const u32x4_t*>(q + (static_cast<int64_t>(cs.seq) * a.num_q_heads + hq0) * D);
#pragma unroll
    for (int k = 0; k < kQPerLane; ++k)
      if (k * kWave + lane < kQVecs) qv[k] = qsrc[k * kWave + lane];
  }
  bw.fill(cs.b_lo, lane);  // waits for the query rows too
#pragma unroll
  for (int k = 0; k < kQPerLane; ++k)
    if (k * kWave + lane < kQVecs) s_q[wave][k * kWave + lane] = qv[k];

  Chunk<W> cur, nxt;
  int c0;     // this wave's current chunk position
  int t_end;  // tokens before t_end are unmasked for this wave (t_lo for a dummy chunk)
  int left;   // chunks of this wave in the segment, at least one
  {
    const int c = cs.t_lo + wave * kChunk;
    const bool real = c < cs.t_hi;
    c0 = real ? c : cs.t_lo;
    t_end = real ? cs.t_hi : cs.t_lo;
    left = real ? (cs.t_hi - c + kStride - 1) / kStride : 1;
    const int kvh = cs.hg / groups_per_kv;
    load_chunk<T, D, FUSED>(cur, k_cache + kvh * D, v_cache + kvh * D, bw.get(c0 / kTokensPerBlock, lane), row_stride,
                            c0, cs.t_hi, ts, sl, new_row(knew_base, cs.seq, kvh), new_row(vnew_base, cs.seq, kvh),
                            cs.last_pos);
  }

  // Split-item pieces this workgroup stores (at most the first and the last
  // segment), counted at the end: item index, piece count, first output row.
  int pend_item[2] = {-1, -1};
  int pend_n[2] = {0, 0};
  int64_t pend_unit0[2] = {0, 0};
  int64_t pend_first[2] = {0, 0};
  int64_t pend_item_first[2] = {0, 0};
  bool first_seg = true;

  while (true) {
    const int kvh = cs.hg / groups_per_kv;
    const int hq0 = kvh * group + (cs.hg % groups_per_kv) * GT;
    const T* kpool = k_cache + static_cast<int64_t>(kvh) * D;
    const T* vpool = v_cache + static_cast<int64_t>(kvh) * D;
    const T* knew = new_row(knew_base, cs.seq, kvh);
    const T* vnew = new_row(vnew_base, cs.seq, kvh);

    // The next segment (or, after the last one, this segment again, so that
    // the loads below are issued on every path): its block-table window and
    // query rows start loading now.
    Segment ns;
    const bool has_next = walk.next(ns);
    if (!has_next) ns = cs;
    BlockWindow bwn;
    bwn.table = a.block_tables + static_cast<int64_t>(ns.seq) * a.max_blocks_per_seq;
    bwn.limit = ns.b_hi;
    bwn.fill_async(ns.b_lo, lane);
    const int n_kvh = ns.hg / groups_per_kv;
    const int n_hq0 = n_kvh * group + (ns.hg % groups_per_kv) * GT;
    {
      const u32x4_t* qsrc =
          reinterpret_cast<const u32x4_t*>(q + (static_cast<int64_t>(ns.seq) * a.num_q_heads + n_hq0) * D);
#pragma unroll
      for (int k = 0; k < kQPerLane; ++k)
        if (k * kWave + lane < kQVecs) qv[k] = qsrc[k * kWave + lane];
    }
    const int nc = ns.t_lo + wave * kChunk;
    const bool n_real = has_next && nc < ns.t_hi;
    const int n_c0 = n_real ? nc : ns.t_lo;

    // This segment's chunks: whole pairs while at least three remain, then
    // the last one or two, overlapping the next segment's first chunk. The
    // loop has a single exit at its head, so every path into a consume has
    // the same loads in flight and the compiler's wait before it covers that
    // chunk only.
    st.reset();
    // byte offsets of the lane's rows (ts and ts + 8) and piece in a full chunk
    const uint32_t off_a = static_cast<uint32_t>((ts * row_stride + sl * S::kElemsPerVec) * sizeof(T));
    const uint32_t off_b = off_a + static_cast<uint32_t>(8 * row_stride * sizeof(T));
    QRegs<T, D, GT> qr;
    if constexpr (Elem<T>::kBytes == 1) {
#pragma unroll
      for (int g = 0; g < GT; ++g) q_words<T, D>(sq, g, sl, qr[g]);
    }
    int cn = c0;
    // Pairs whose loads lie in the context's leading rows (the ones a prefix
    // cache may share) use cache-allocating loads, later pairs streaming ones;
    // two loops, so that each keeps its own kind of load.
    // Passes of two chunks while more than three remain: every chunk a pass
    // consumes or loads then has a later chunk of the wave in the segment,
    // so all its rows are in range and none is the new token's (full
    // chunks). With exactly three left, one more pass whose second load is
    // the wave's last chunk, which takes the general load (row clamp, new-
    // token row); kept out of the loops so that they carry no branch.
    const auto full_pass = [&](auto stream) {
      constexpr bool kStream = decltype(stream)::value;
      cn += kStride;
      load_full_chunk<T, D, kStream>(nxt, kpool, vpool, bw.get(cn / kTokensPerBlock, lane), row_stride, cn, off_a,
                                     off_b);
      consume_chunk<T, D, GT, true>(st, cur, sq, sl, true, true, sc, qr);
      c0 += kStride;
      cn += kStride;
      load_full_chunk<T, D, kStream>(cur, kpool, vpool, bw.get(cn / kTokensPerBlock, lane), row_stride, cn, off_a,
                                     off_b);
      consume_chunk<T, D, GT, true>(st, nxt, sq, sl, true, true, sc, qr);
      c0 += kStride;
      left -= 2;
    };
    while (left > 3 && cn + 2 * kStride < kCachedLeadTokens) full_pass(std::false_type{});
    while (left > 3) full_pass(std::true_type{});
    if (left == 3) {
      cn += kStride;
      load_full_chunk<T, D, true>(nxt, kpool, vpool, bw.get(cn / kTokensPerBlock, lane), row_stride, cn, off_a,
                                  off_b);
      consume_chunk<T, D, GT, true>(st, cur, sq, sl, true, true, sc, qr);
      c0 += kStride;
      cn += kStride;
      load_chunk<T, D, FUSED>(cur, kpool, vpool, bw.get(cn / kTokensPerBlock, lane), row_stride, cn, cs.t_hi, ts, sl,
                              knew, vnew, cs.last_pos);
      consume_chunk<T, D, GT, true>(st, nxt, sq, sl, true, true, sc, qr);
      c0 += kStride;
      left -= 2;
    }
    // The last two chunk slots. With one chunk left, the second slot re-reads
    // the first one's rows (a recent read) with every token masked: the tail
    // then has one shape, with every load issued on every path, so the
    // next segment's first chunk lands straight in `cur` and nothing waits
    // for it before the next segment.
    const T* n_kpool = k_cache + static_cast<int64_t>(n_kvh) * D;
    const T* n_vpool = v_cache + static_cast<int64_t>(n_kvh) * D;
    const bool two = left == 2;
    cn = two ? cn + kStride : cn;
    load_chunk<T, D, FUSED>(nxt, kpool, vpool, bw.get(cn / kTokensPerBlock, lane), row_stride, cn, cs.t_hi, ts, sl,
                            knew, vnew, cs.last_pos);
    consume_chunk<T, D, GT>(st, cur, sq, sl, c0 + ts < t_end, c0 + 8 + ts < t_end, sc, qr);
    c0 += kStride;
    load_chunk<T, D, FUSED>(cur, n_kpool, n_vpool, bwn.get(n_c0 / kTokensPerBlock, lane), row_stride, n_c0, ns.t_hi,
                            ts, sl, new_row(knew_base, ns.seq, n_kvh), new_row(vnew_base, ns.seq, n_kvh),
                            ns.last_pos);
    consume_chunk<T, D, GT>(st, nxt, sq, sl, two && c0 + ts < t_end, two && c0 + 8 + ts < t_end, sc, qr);

    // Merge the 8 lane groups of each wave into lanes 0-7: the upper half
    // into the lower, odd rows into even ones (VALU lane swaps that hand
    // every lane both values), then lanes 8-15 into 0-7 (row rotate by 8) ...
#pragma unroll
    for (int g = 0; g < GT; ++g) {
#pragma unroll
      for (int step = 0; step < 2; ++step) {
        const auto pair = [step](float x) { return step == 0 ? pair_across_halves(x) : pair_across_rows(x); };
        const LanePair pm = pair(st.m[g]);
        const LanePair pl = pair(st.l[g]);
        const float mx = fmaxf(pm.lo, pm.hi);
        const float fa = exp2_fast(pm.lo - mx);
        const float fb = exp2_fast(pm.hi - mx);
        st.l[g] = pl.lo * fa + pl.hi * fb;
#pragma unroll
        for (int j = 0; j < E; ++j) {
          const LanePair pa = pair(st.acc[g][j]);
          st.acc[g][j] = pa.lo * fa + pa.hi * fb;
        }
        st.m[g] = mx;
      }
      const float mo = dpp_f32<kDppRowRor8>(st.m[g]);
      const float lo = dpp_f32<kDppRowRor8>(st.l[g]);
      const float mx = fmaxf(st.m[g], mo);
      const float fa = exp2_fast(st.m[g] - mx);
      const float fb = exp2_fast(mo - mx);
      st.l[g] = st.l[g] * fa + lo * fb;
#pragma unroll
      for (int j = 0; j < E; ++j) st.acc[g][j] = st.acc[g][j] * fa + dpp_f32<kDppRowRor8>(st.acc[g][j]) * fb;
      st.m[g] = mx;
    }
    // ... then the 4 waves through LDS.
    if (ts == 0) {
#pragma unroll
      for (int g = 0; g < GT; ++g) {
#pragma unroll
        for (int j = 0; j < E; ++j) s_acc[wave][g][lane_dim<T, D>(sl, j)] = st.acc[g][j];
        if (sl == 0) {
          s_m[wave][g] = st.m[g];
          s_l[wave][g] = st.l[g];
        }
      }
    }
    __syncthreads();

    const int64_t unit0 = static_cast<int64_t>(cs.seq) * a.num_q_heads + hq0;
    for (int o = tid; o < GT * D; o += kDecodeThreads) {
      const int g = o / D;
      const int d = o % D;
      float mx = s_m[0][g];
#pragma unroll
      for (int k = 1; k < kDecodeWaves; ++k) mx = fmaxf(mx, s_m[k][g]);
      float num = 0.0f, den = 0.0f;
#pragma unroll
      for (int k = 0; k < kDecodeWaves; ++k) {
        const float f = exp2_fast(s_m[k][g] - mx);
        num += f * s_acc[k][g][d];
        den += f * s_l[k][g];
      }
      const float val = num / den;
      if (cs.n_parts == 1) {
        store_out<IoT>(out + (unit0 + g) * D + d, kOutScale ? val * a.v_scale : val);
      } else {
        // A piece of a split item: its normalised output and log2-sum-exp go
        // to the piece's slot, written through to the device-coherent level
        // (the merging wave may run on another XCD).
        const int64_t row = (2 * static_cast<int64_t>(w) + (first_seg ? 0 : 1)) * GT + g;
        store_agent(a.part_out + row * D + d, val);
        if (d == 0) store_agent(a.part_lse + row, mx + __log2f(den));
      }
    }
    if (cs.n_parts > 1) {
      const int k = pend_item[0] < 0 ? 0 : 1;
      pend_item[k] = cs.seq * HG + cs.hg;
      pend_n[k] = cs.n_parts;
      pend_unit0[k] = unit0;
      pend_first[k] = cs.first_owner;
      pend_item_first[k] = cs.item_first;
    }
    __syncthreads();  // LDS is reused by the next segment

    if (!has_next) break;
    first_seg = false;
    cs = ns;
    bw = bwn;
    // the wave's own LDS copy of the query rows: its last read of the old
    // rows came before this point in the wave's program order
#pragma unroll
    for (int k = 0; k < kQPerLane; ++k)
      if (k * kWave + lane < kQVecs) s_q[wave][k * kWave + lane] = qv[k];
    c0 = n_c0;
    t_end = n_real ? ns.t_hi : ns.t_lo;
    left = n_real ? (ns.t_hi - nc + kStride - 1) / kStride : 1;
  }

  // ---- 4. Count the stored pieces once this wave's stores are complete:
  // each wave counts its own share, and an item is complete at kDecodeWaves
  // counts per piece. The wave whose count completes an item merges its
  // pieces in piece order, so the result does not depend on timing.
  //
  // Ordering this relies on (gfx950): the pieces' partials are agent-scope
  // stores, which write through to the device-coherent level, and a wave's
  // vector-memory counter covers stores until that level has acknowledged
  // them, so after the wait each stored partial is visible to every XCD
  // before the count that announces it is issued. The merging wave issues its
  // agent-scope loads (which bypass the non-coherent caches) only after its
  // count has returned. The write-back and invalidate a release/acquire pair
  // would add cover plain cached accesses, which the partials never use.
  if (pend_item[0] >= 0) {
    wait_vector_memory();
    // lanes 0 and 1 count the two pieces together
    const int mine_item = lane == 0 ? pend_item[0] : pend_item[1];
    const uint64_t tag = a.epoch_word != nullptr ? __hip_atomic_load(const_cast<uint64_t*>(a.epoch_word),
                                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                                 : a.epoch_tag;
    int t = 0;
    if (lane < 2 && mine_item >= 0) t = count_arrival(a.counters + mine_item, tag);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int tk = __builtin_amdgcn_readlane(t, k);
      if (pend_item[k] < 0) continue;
      const int expected = kDecodeWaves * pend_n[k];
      if (tk == expected) {
        merge_item<IoT, D, GT, kOutScale>(a, out, pend_unit0[k], split, pend_first[k], pend_n[k],
                                          pend_item_first[k], lane);
      } else if (tk < 0 || tk > expected) {
        // A counter that was not this call's (never-cleared workspace): the
        // pieces cannot be trusted, so the item's rows are set to NaN and the
        // error word tells the caller.
        if (lane == 0) flag_workspace(a.ws_flags, kWorkspaceErrStaleCounter);
        for (int o = lane; o < GT * D; o += kWave)
          store_out<IoT>(out + pend_unit0[k] * D + o, __builtin_nanf(""));
      }
    }
  }
}

// The library's grid: one workgroup per compute unit. Measured on MI355X, one
// resident workgroup (one wave per SIMD) streams faster than two: the second
// workgroup on a CU only adds contention for the same memory path. With few
// items (small batches) the grid is also capped at kDecodePiecesPerItem
// workgroups per item: splitting an item further costs more in partial
// stores and merge latency than it gains (batch 1, Qwen3-0.6B shape: 26 us
// at 256 workgroups, 13 us at 64).
constexpr int kDecodePerCu = 1;
// fp8 pools: a lane loads half the bytes of a bf16 row per token, so one
// workgroup per CU keeps too few bytes in flight; two per CU measured 64 us
// against 66-69 us (one) and 67 us (three) on the Qwen3-0.6B-shaped decode.
constexpr int kDecodePerCuFp8 = 2;
constexpr int64_t kDecodePiecesPerItem = 8;

template <typename T, int D, int GT, bool FUSED>
hipError_t launch_fused_or_not(const DecodeArgs& a, hipStream_t stream) {
  int wgs = a.num_workgroups;
  if (wgs <= 0) {
    const int64_t items = static_cast<int64_t>(a.num_seqs) * (a.num_q_heads / GT);
    wgs = min(kDecodeMaxWorkgroups,
              resident_workgroups(reinterpret_cast<const void*>(&paged_decode_kernel<T, D, GT, FUSED>),
                                  kDecodeThreads, a.max_units, Elem<T>::kBytes == 1 ? kDecodePerCuFp8 : kDecodePerCu));
    wgs = static_cast<int>(min(static_cast<int64_t>(wgs), max(int64_t{1}, items * kDecodePiecesPerItem)));
  }
  paged_decode_kernel<T, D, GT, FUSED><<<dim3(static_cast<uint32_t>(wgs)), dim3(kDecodeThreads), 0, stream>>>(a);
  return hipGetLastError();
}

template <typename T, int D, int GT>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  return a.k_new != nullptr ? launch_fused_or_not<T, D, GT, true>(a, stream)
                            : launch_fused_or_not<T, D, GT, false>(a, stream);
}

template <typename T, int D>
int default_grid(int group, int64_t max_units) {
  switch (decode_head_group(group)) {
    case 4:
      return resident_workgroups(reinterpret_cast<const void*>(&paged_decode_kernel<T, D, 4, false>), kDecodeThreads,
                                 max_units, kDecodePerCu);
    case 2:
      return resident_workgroups(reinterpret_cast<const void*>(&paged_decode_kernel<T, D, 2, false>), kDecodeThreads,
                                 max_units, kDecodePerCu);
    default:
      return resident_workgroups(reinterpret_cast<const void*>(&paged_decode_kernel<T, D, 1, false>), kDecodeThreads,
                                 max_units, kDecodePerCu);
  }
}

template <typename T, int D>
hipError_t launch_group(const DecodeArgs& a, hipStream_t stream) {
  switch (decode_head_group(a.num_q_heads / a.num_kv_heads)) {
    case 4:
      return launch_typed<T, D, 4>(a, stream);
    case 2:
      return launch_typed<T, D, 2>(a, stream);
    default:
      return launch_typed<T, D, 1>(a, stream);
  }
}

}  // namespace

hipError_t launch_decode_fp8_pools(const DecodeArgs& a, hipStream_t stream) {
  switch (decode_head_group(a.num_q_heads / a.num_kv_heads)) {
    case 4:
      return launch_fused_or_not<fp8_t, 128, 4, false>(a, stream);
    case 2:
      return launch_fused_or_not<fp8_t, 128, 2, false>(a, stream);
    default:
      return launch_fused_or_not<fp8_t, 128, 1, false>(a, stream);
  }
}

hipError_t launch_decode(const DecodeArgs& a, Dtype dtype, int32_t head_dim, hipStream_t stream) {
  if (dtype == Dtype::kBF16) {
    if (head_dim == 128) return launch_group<bf16_t, 128>(a, stream);
    return launch_group<bf16_t, 64>(a, stream);
  }
  if (head_dim == 128) return launch_group<float, 128>(a, stream);
  return launch_group<float, 64>(a, stream);
}

int decode_default_workgroups(Dtype dtype, int32_t head_dim, int32_t group, int64_t max_units, int64_t items) {
  int n;
  if (dtype == Dtype::kBF16)
    n = head_dim == 128 ? default_grid<bf16_t, 128>(group, max_units) : default_grid<bf16_t, 64>(group, max_units);
  else
    n = head_dim == 128 ? default_grid<float, 128>(group, max_units) : default_grid<float, 64>(group, max_units);
  n = min(n, kDecodeMaxWorkgroups);
  return static_cast<int>(min(static_cast<int64_t>(n), max(int64_t{1}, items * kDecodePiecesPerItem)));
}

}  // namespace pa
