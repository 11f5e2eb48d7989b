// Paged decode attention: one query token per sequence attends over the K/V
// rows its block table names ("Nano-vLLM System Architecture Analysis",
// section 2, "Attention with Paged Cache": decode attends over all cached K/V
// of the sequence's blocks). Unlike a gather-then-attend implementation, the
// rows are streamed from the pool in place and never copied.
//
// Work split. An item is (sequence, group of GT query heads sharing one KV
// head); it has one work unit per 256-token block of its context. The units of
// all items, ordered sequence-major, are cut into equal contiguous ranges, one
// per workgroup, so every workgroup streams the same number of blocks however
// ragged the contexts are. A range may hold the tail of one item, whole items
// and the head of another; each such piece is a segment.
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
//   * at the end of a segment the 8 groups of a wave merge by lane shuffles,
//     the 4 waves through LDS; a whole item is written as the final output,
//     a piece as a (normalised output, log2-sum-exp) partial.
//   * The last workgroup to finish a piece of a split item -- found with a
//     device-scope counter -- merges all its pieces in order. The merge order
//     is fixed, so results are bit-identical from run to run; no floating-
//     point atomics are used. Partials move through agent-coherent atomic
//     stores/loads, never through cache-wide fences.
#include <math.h>

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

// Loads the lane's words of one head row: kVecs 16-byte pieces.
template <typename T, int D>
__device__ __forceinline__ void load_row(const T* row, int sl, uint32_t (&w)[DecodeShape<T, D>::kWords]) {
  using S = DecodeShape<T, D>;
#pragma unroll
  for (int v = 0; v < S::kVecs; ++v) {
    // Streaming (non-temporal) loads: every K/V byte is used once, and on
    // MI355X they sustain about 10% more bandwidth than cached loads.
    const u32x4_t x =
        __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(row + v * S::kVecStride + sl * S::kElemsPerVec));
    w[4 * v + 0] = x[0];
    w[4 * v + 1] = x[1];
    w[4 * v + 2] = x[2];
    w[4 * v + 3] = x[3];
  }
}

// Partial q.k over the lane's elements.
template <typename T, int D>
__device__ __forceinline__ float partial_dot(const uint32_t (&qw)[DecodeShape<T, D>::kWords],
                                             const uint32_t (&kw)[DecodeShape<T, D>::kWords]) {
  using S = DecodeShape<T, D>;
  float s0 = 0.0f, s1 = 0.0f;
  if constexpr (Elem<T>::kBytes == 2) {
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

template <typename T, int D>
__device__ __forceinline__ void load_chunk(Chunk<DecodeShape<T, D>::kWords>& c, const T* kpool, const T* vpool,
                                           int block, int64_t row_stride, int c0, int t_end, int ts, int sl) {
  // Wave-uniform base of the chunk's first row plus a small per-lane offset.
  // Rows past the range are never read: their lanes re-read the last valid
  // row (always in the same block as the chunk start) and get zero weight.
  const int64_t r0 = static_cast<int64_t>(block) * kTokensPerBlock + (c0 % kTokensPerBlock);
  const T* kb = kpool + r0 * row_stride;
  const T* vb = vpool + r0 * row_stride;
  const int last = t_end - 1 - c0;
  const int rs = static_cast<int>(row_stride);
  const int oa = min(ts, last) * rs;
  const int ob = min(ts + 8, last) * rs;
  load_row<T, D>(kb + oa, sl, c.ka);
  load_row<T, D>(kb + ob, sl, c.kb);
  load_row<T, D>(vb + oa, sl, c.va);
  load_row<T, D>(vb + ob, sl, c.vb);
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
  __device__ __forceinline__ int get(int b, int lane) {
    if (b - base >= kWave) fill(b - (b - base) % kWave, lane);  // wave-uniform, rare
    return __builtin_amdgcn_readlane(id, b - base);
  }
};

template <typename T, int D, int GT>
__device__ __forceinline__ void consume_chunk(LaneState<GT, DecodeShape<T, D>::kLaneElems>& st,
                                              const Chunk<DecodeShape<T, D>::kWords>& c,
                                              const uint32_t (&qw)[GT][DecodeShape<T, D>::kWords], bool va, bool vb,
                                              float sc) {
  constexpr int W = DecodeShape<T, D>::kWords;
  constexpr int E = DecodeShape<T, D>::kLaneElems;
  float sa[GT], sb[GT];
  bool need = false;
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    const float da = sum8(partial_dot<T, D>(qw[g], c.ka));
    const float db = sum8(partial_dot<T, D>(qw[g], c.kb));
    sa[g] = va ? da * sc : -INFINITY;
    sb[g] = vb ? db * sc : -INFINITY;
    need |= fmaxf(sa[g], sb[g]) > st.m[g] + kStaleMaxSlack;
  }
  if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float mn = fmaxf(st.m[g], fmaxf(sa[g], sb[g]));
      const float alpha = exp2_fast(st.m[g] - mn);
      st.l[g] *= alpha;
#pragma unroll
      for (int j = 0; j < E; ++j) st.acc[g][j] *= alpha;
      st.m[g] = mn;
    }
  }
  if constexpr (Elem<T>::kBytes == 2) {
    uint32_t vp[E];
#pragma unroll
    for (int w = 0; w < W; ++w) {
      vp[2 * w] = pair_lo(c.va[w], c.vb[w]);
      vp[2 * w + 1] = pair_hi(c.va[w], c.vb[w]);
    }
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const uint32_t pp = pack_bf16x2(exp2_fast(sa[g] - st.m[g]), exp2_fast(sb[g] - st.m[g]));
      st.l[g] = dot2_bf16(pp, 0x3F803F80u, st.l[g]);  // + p_a + p_b as rounded
#pragma unroll
      for (int j = 0; j < E; ++j) st.acc[g][j] = dot2_bf16(pp, vp[j], st.acc[g][j]);
    }
  } else {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float pa = exp2_fast(sa[g] - st.m[g]);
      const float pb = exp2_fast(sb[g] - st.m[g]);
      st.l[g] += pa + pb;
#pragma unroll
      for (int j = 0; j < E; ++j)
        st.acc[g][j] = fmaf(pa, __uint_as_float(c.va[j]), fmaf(pb, __uint_as_float(c.vb[j]), st.acc[g][j]));
    }
  }
}

// Blocks of a context, with the length clamped to [0, max_context_len]
// (lengths outside [1, max_context_len] are a caller error; clamping keeps
// every read inside the block table and the workspace, and every loop finite).
__device__ __forceinline__ int context_blocks(int ctx, int max_ctx) {
  ctx = min(max(ctx, 0), max_ctx);
  return (ctx + kTokensPerBlock - 1) / kTokensPerBlock;
}

// Which workgroup owns work unit u when U units are split evenly over G
// workgroups (workgroup w owns [w*U/G, (w+1)*U/G)).
__device__ __forceinline__ int owner_of(int64_t u, int64_t U, int64_t G) {
  return static_cast<int>(((u + 1) * G - 1) / U);
}

template <typename T, int D, int GT>
__global__ __launch_bounds__(kDecodeThreads) void paged_decode_kernel(DecodeArgs a) {
  using S = DecodeShape<T, D>;
  constexpr int W = S::kWords;
  constexpr int E = S::kLaneElems;
  __shared__ int s_scan[kDecodeThreads];
  __shared__ int s_loc[2];
  __shared__ float s_acc[kDecodeWaves][GT][D];
  __shared__ float s_m[kDecodeWaves][GT];
  __shared__ float s_l[kDecodeWaves][GT];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // wave index made provably wave-uniform, so per-wave addresses (block-table
  // entries) are scalar loads that do not queue behind the vector loads
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int ts = lane >> 3;  // token slot within a chunk (and ts + 8)
  const int sl = lane & 7;   // sub-lane: which 16-byte pieces of the row
  const int B = a.num_seqs;
  const int HG = a.num_q_heads / GT;  // head groups per sequence
  const int group = a.num_q_heads / a.num_kv_heads;
  const int groups_per_kv = group / GT;

  // ---- 1. Work units: item (seq i, head group hg) has ceil(ctx_i / 256)
  // units of one 256-token block each, ordered seq-major. Count them with a
  // block-wide scan over the sequences.
  const int per = (B + kDecodeThreads - 1) / kDecodeThreads;
  int mine = 0;
  for (int k = 0; k < per; ++k) {
    const int i = tid * per + k;
    if (i < B) mine += context_blocks(a.context_lens[i], a.max_context_len);
  }
  s_scan[tid] = mine;
  __syncthreads();
  for (int off = 1; off < kDecodeThreads; off <<= 1) {
    const int v = tid >= off ? s_scan[tid - off] : 0;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  const int64_t U = static_cast<int64_t>(HG) * __builtin_amdgcn_readfirstlane(s_scan[kDecodeThreads - 1]);
  // With no more workgroups than units every workgroup owns at least one
  // unit, so the owners of an item's units are consecutive workgroups.
  const int64_t G = min(static_cast<int64_t>(gridDim.x), U);
  const int w = blockIdx.x;
  if (w >= G) return;
  const int64_t u_begin = static_cast<int64_t>(w) * U / G;
  const int64_t u_end = static_cast<int64_t>(w + 1) * U / G;

  // ---- 2. The sequence holding u_begin: the thread whose sequences span it
  // walks them.
  {
    const int64_t lo = static_cast<int64_t>(HG) * (s_scan[tid] - mine);
    const int64_t hi = static_cast<int64_t>(HG) * s_scan[tid];
    if (u_begin >= lo && u_begin < hi) {
      int64_t base = lo;
      for (int k = 0; k < per && tid * per + k < B; ++k) {
        const int i = tid * per + k;
        const int64_t span = static_cast<int64_t>(HG) * context_blocks(a.context_lens[i], a.max_context_len);
        if (u_begin < base + span) {
          s_loc[0] = i;
          s_loc[1] = static_cast<int>(base / HG);  // blocks of all earlier sequences
          break;
        }
        base += span;
      }
    }
  }
  __syncthreads();
  // Values read back from LDS are uniform; say so, so that the whole walk
  // (and every block-table lookup) stays in scalar registers.
  int seq = __builtin_amdgcn_readfirstlane(s_loc[0]);
  int64_t seq_base = static_cast<int64_t>(HG) * __builtin_amdgcn_readfirstlane(s_loc[1]);  // first unit of seq

  const int64_t row_stride = static_cast<int64_t>(a.num_kv_heads) * D;
  const float sc = a.scale_log2;
  T* out = static_cast<T*>(a.out);
  LaneState<GT, E> st;

  // ---- 3. Walk the segments (pieces of items) in [u_begin, u_end).
  int64_t u = u_begin;
  while (u < u_end) {
    const int ctx_raw = __builtin_amdgcn_readfirstlane(a.context_lens[seq]);
    const int nb = context_blocks(ctx_raw, a.max_context_len);
    const int ctx = min(ctx_raw, a.max_context_len);
    const int64_t r = u - seq_base;
    const int hg = static_cast<int>(r / nb);
    const int b_lo = static_cast<int>(r % nb);
    const int64_t item_first = seq_base + static_cast<int64_t>(hg) * nb;
    const int64_t item_end = item_first + nb;
    const int64_t seg_end = u_end < item_end ? u_end : item_end;
    const int b_hi = b_lo + static_cast<int>(seg_end - u);
    const int t_lo = b_lo * kTokensPerBlock;
    const int t_hi = min(ctx, b_hi * kTokensPerBlock);

    const int kvh = hg / groups_per_kv;
    const int hq0 = kvh * group + (hg % groups_per_kv) * GT;
    uint32_t qw[GT][W];
    const T* qbase = static_cast<const T*>(a.q) + (static_cast<int64_t>(seq) * a.num_q_heads + hq0) * D;
#pragma unroll
    for (int g = 0; g < GT; ++g) load_row<T, D>(qbase + g * D, sl, qw[g]);
    const T* kpool = static_cast<const T*>(a.k_cache) + static_cast<int64_t>(kvh) * D;
    const T* vpool = static_cast<const T*>(a.v_cache) + static_cast<int64_t>(kvh) * D;
    BlockWindow bw;
    bw.table = a.block_tables + static_cast<int64_t>(seq) * a.max_blocks_per_seq;
    bw.limit = b_hi;
    bw.fill(b_lo, lane);

    // The 4 waves take 16-token chunks round-robin; each wave keeps the next
    // chunk's loads in flight while it works on the current one.
    st.reset();
    {
      // The next chunk's loads are always issued (past the end they re-read
      // the wave's last chunk, which the L2 still holds), so the number of
      // loads in flight at each consume is the same on every path and the
      // wait before it covers only the chunk being consumed.
      constexpr int kStride = kDecodeWaves * kChunk;
      int c0 = t_lo + wave * kChunk;
      if (c0 < t_hi) {
        const int c_last = c0 + (t_hi - 1 - c0) / kStride * kStride;
        Chunk<W> cur, nxt;
        load_chunk<T, D>(cur, kpool, vpool, bw.get(c0 / kTokensPerBlock, lane), row_stride, c0, t_hi, ts, sl);
        while (true) {
          int cn = min(c0 + kStride, c_last);
          load_chunk<T, D>(nxt, kpool, vpool, bw.get(cn / kTokensPerBlock, lane), row_stride, cn, t_hi, ts, sl);
          consume_chunk<T, D, GT>(st, cur, qw, c0 + ts < t_hi, c0 + 8 + ts < t_hi, sc);
          c0 += kStride;
          if (c0 >= t_hi) break;
          cn = min(c0 + kStride, c_last);
          load_chunk<T, D>(cur, kpool, vpool, bw.get(cn / kTokensPerBlock, lane), row_stride, cn, t_hi, ts, sl);
          consume_chunk<T, D, GT>(st, nxt, qw, c0 + ts < t_hi, c0 + 8 + ts < t_hi, sc);
          c0 += kStride;
          if (c0 >= t_hi) break;
        }
      }
    }

    // Merge the 8 lane groups of each wave (lane distance 8, 16, 32) ...
#pragma unroll
    for (int step = 0; step < 3; ++step) {
      const int mask = 8 << step;
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        const float mo = shfl_xor_f32(st.m[g], mask);
        const float lo = shfl_xor_f32(st.l[g], mask);
        const float mx = fmaxf(st.m[g], mo);
        const float fa = exp2_fast(st.m[g] - mx);
        const float fb = exp2_fast(mo - mx);
        st.l[g] = st.l[g] * fa + lo * fb;
#pragma unroll
        for (int j = 0; j < E; ++j) st.acc[g][j] = st.acc[g][j] * fa + shfl_xor_f32(st.acc[g][j], mask) * fb;
        st.m[g] = mx;
      }
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

    const int64_t unit0 = static_cast<int64_t>(seq) * a.num_q_heads + hq0;
    const int first_owner = owner_of(item_first, U, G);
    const int n_parts = owner_of(item_end - 1, U, G) - first_owner + 1;
    const int part = w - first_owner;
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
      if (n_parts == 1) {
        store_out<T>(out + (unit0 + g) * D + d, val);
      } else {
        const int64_t slot = (unit0 + g) * a.max_parts + part;
        store_agent(a.part_out + slot * D + d, val);
        if (d == 0) store_agent(a.part_lse + slot, mx + __log2f(den));
      }
    }

    if (n_parts > 1) {
      // Split item: the last workgroup to finish its piece merges all the
      // pieces' partial results, in piece order.
      wait_vector_memory();
      __syncthreads();
      if (tid == 0) {
        int* ctr = a.counters + static_cast<int64_t>(seq) * HG + hg;
        const int prev = add_agent(ctr, 1);
        const int last = prev == n_parts - 1;
        if (last) store_agent_int(ctr, 0);
        s_last = last;
      }
      __syncthreads();
      if (s_last) {
        for (int o = tid; o < GT * D; o += kDecodeThreads) {
          const int g = o / D;
          const int d = o % D;
          const int64_t base = (unit0 + g) * a.max_parts;
          float mx = -INFINITY;
          for (int p = 0; p < n_parts; ++p) mx = fmaxf(mx, load_agent(a.part_lse + base + p));
          float num = 0.0f, den = 0.0f;
          for (int p = 0; p < n_parts; ++p) {
            const float f = exp2_fast(load_agent(a.part_lse + base + p) - mx);
            num += f * load_agent(a.part_out + (base + p) * D + d);
            den += f;
          }
          store_out<T>(out + (unit0 + g) * D + d, num / den);
        }
      }
    }
    __syncthreads();  // LDS is reused by the next segment

    u = seg_end;
    if (u == item_end && hg == HG - 1) {  // next sequence with work
      seq_base = item_end;
      ++seq;
      while (u < u_end && seq < B - 1 &&
             context_blocks(__builtin_amdgcn_readfirstlane(a.context_lens[seq]), a.max_context_len) == 0)
        ++seq;
    }
  }
}

template <typename T, int D, int GT>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  int wgs = a.num_workgroups;
  if (wgs <= 0) wgs = resident_workgroups(reinterpret_cast<const void*>(&paged_decode_kernel<T, D, GT>),
                                          kDecodeThreads, a.max_units);
  paged_decode_kernel<T, D, GT><<<dim3(static_cast<uint32_t>(wgs)), dim3(kDecodeThreads), 0, stream>>>(a);
  return hipGetLastError();
}

template <typename T, int D>
int default_grid(int group, int64_t max_units) {
  switch (decode_head_group(group)) {
    case 4:
      return resident_workgroups(reinterpret_cast<const void*>(&paged_decode_kernel<T, D, 4>), kDecodeThreads, max_units);
    case 2:
      return resident_workgroups(reinterpret_cast<const void*>(&paged_decode_kernel<T, D, 2>), kDecodeThreads, max_units);
    default:
      return resident_workgroups(reinterpret_cast<const void*>(&paged_decode_kernel<T, D, 1>), kDecodeThreads, max_units);
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

hipError_t launch_decode(const DecodeArgs& a, Dtype dtype, int32_t head_dim, hipStream_t stream) {
  if (dtype == Dtype::kBF16) {
    if (head_dim == 128) return launch_group<bf16_t, 128>(a, stream);
    return launch_group<bf16_t, 64>(a, stream);
  }
  if (head_dim == 128) return launch_group<float, 128>(a, stream);
  return launch_group<float, 64>(a, stream);
}

int decode_default_workgroups(Dtype dtype, int32_t head_dim, int32_t group, int64_t max_units) {
  if (dtype == Dtype::kBF16) return head_dim == 128 ? default_grid<bf16_t, 128>(group, max_units)
                                                    : default_grid<bf16_t, 64>(group, max_units);
  return head_dim == 128 ? default_grid<float, 128>(group, max_units) : default_grid<float, 64>(group, max_units);
}

}  // namespace pa
