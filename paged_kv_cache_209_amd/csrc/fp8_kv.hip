// fp8 KV cache: a quantising store and decode attention that reads the fp8
// pools (half the bytes of bf16) and dequantises on the fly. The pages name
// quantised KV-cache transfers ("Why Understand Inference Engine
// Architecture?", Tensor Parallelism Optimization, item 3) without a format;
// the format here is OCP FP8 E4M3 with one fp32 scale per pool: a value x is
// stored as the code nearest to clamp(x * (1/s), -448, 448) (ties to even, the
// hardware converter's rounding) and read back as code * s.
//
// Decode works per (sequence, chunk of 256-token blocks -- 1, 2, 4, or a
// whole context of up to 32 -- group of GT query heads of one KV head): one
// workgroup streams the chunk's K and V rows (128 bytes per row and head at
// D = 128) block by block and leaves an online-softmax partial (reference
// max, sum, unnormalised output) in the workspace; a second kernel merges a
// sequence's chunk partials in order (deterministic, no atomics) and writes
// the bf16 output. Inside a workgroup each wave takes 64 rows of each block:
// 8 lane groups of 8 lanes, a lane holding 16 consecutive dims of a row. A
// block's rows are loaded in two halves of 4 rows per lane; while one half is
// consumed the other is in flight, and the consumed half's registers take the
// same half of the next block. q.k sums over the
// 8 lanes of a group by DPP; the 8 groups of a wave merge their softmax states
// by a DPP row rotate and the gfx950 permlane swaps, the 4 waves through LDS.
#include <math.h>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kF8Threads = 256;
constexpr int kF8Waves = kF8Threads / kWave;
constexpr int kF8D = 128;                       // head dim supported
constexpr int kF8RowsPerWave = kTokensPerBlock / kF8Waves;  // 64
constexpr int kF8Iters = kF8RowsPerWave / 8;    // rows per lane group
constexpr int kF8Half = kF8Iters / 2;          // rows per lane group in one load half
constexpr float kF8Empty = -1.0e30f;            // running max before any row
constexpr float kF8Slack = 8.0f;                // log2 units the reference max may lag by

// Two fp8 codes (the low or the high half of a word) to a bf16 pair (exact:
// every E4M3 value is a bf16 value), the first code in the low half.
template <bool kHigh>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHigh));
}

__device__ __forceinline__ float clamp_fp8(float x) { return fminf(fmaxf(x, -448.0f), 448.0f); }

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
    int wk = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_fp8(bf16_lo(kk[2 * h]) * inv_k),
                                             clamp_fp8(bf16_hi(kk[2 * h]) * inv_k), 0, false);
    wk = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_fp8(bf16_lo(kk[2 * h + 1]) * inv_k),
                                         clamp_fp8(bf16_hi(kk[2 * h + 1]) * inv_k), wk, true);
    int wv = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_fp8(bf16_lo(vv[2 * h]) * inv_v),
                                             clamp_fp8(bf16_hi(vv[2 * h]) * inv_v), 0, false);
    wv = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_fp8(bf16_lo(vv[2 * h + 1]) * inv_v),
                                         clamp_fp8(bf16_hi(vv[2 * h + 1]) * inv_v), wv, true);
    kw[h] = static_cast<uint32_t>(wk);
    vw[h] = static_cast<uint32_t>(wv);
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

template <int GT>
__global__ __launch_bounds__(kF8Threads) void decode_fp8_block_kernel(DecodeFp8Args a) {
  __shared__ float s_m[kF8Waves][GT];
  __shared__ float s_l[kF8Waves][GT];
  __shared__ float s_acc[kF8Waves][GT][kF8D];
  const int HG = a.num_q_heads / GT;
  int item = blockIdx.x;
  const int hg = item % HG;
  item /= HG;
  const int chunk = item % a.max_chunks;
  const int seq = item / a.max_chunks;
  const int ctx = min(max(a.context_lens[seq], 0), a.max_context_len);
  const int nb_ctx = (ctx + kTokensPerBlock - 1) / kTokensPerBlock;
  const int b_begin = chunk * a.blocks_per_chunk;
  if (b_begin >= nb_ctx) return;  // the whole workgroup: past this sequence's context
  const int b_end = min(b_begin + a.blocks_per_chunk, nb_ctx);
  const int group = a.num_q_heads / a.num_kv_heads;
  const int hq0 = hg * GT;
  const int kvh = hq0 / group;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int grp = lane >> 3;  // lane group: one row at a time
  const int sl = lane & 7;    // dims [16 sl, 16 sl + 16)
  const int64_t row_stride = static_cast<int64_t>(a.num_kv_heads) * kF8D;

  // the lane's 16 query dims of each head, as 8 bf16 pairs
  uint32_t qp[GT][8];
  const uint32_t* qw = static_cast<const uint32_t*>(a.q);
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    const int64_t base = ((static_cast<int64_t>(seq) * a.num_q_heads + hq0 + g) * kF8D + sl * 16) / 2;
#pragma unroll
    for (int j = 0; j < 8; ++j) qp[g][j] = qw[base + j];
  }

  float m[GT], l[GT], acc[GT][16];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    m[g] = kF8Empty;
    l[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[g][e] = 0.0f;
  }
  const float sc = a.scale_log2;
  // The block's rows are loaded in two halves (rows it * 8 + grp of the
  // wave's 64 for it < 4, then it >= 4). While one half is consumed, the other
  // is in flight; each consumed half's registers take the same half of the
  // next block, so loads stay in flight across the whole chunk without extra
  // registers. After the chunk's last block the refills read the current
  // block's first row again (a cached line that is never used), which keeps
  // the loop free of branches around loads.
  const int64_t table_row = static_cast<int64_t>(seq) * a.max_blocks_per_seq;
  auto block_base = [&](const void* pool, int blk) {
    return static_cast<const uint8_t*>(pool) + (static_cast<int64_t>(blk) * kTokensPerBlock) * row_stride +
           kvh * kF8D + sl * 16;
  };
  auto load_half = [&](const uint8_t* kbase, const uint8_t* vbase, int nrows, int it0, bool real,
                       u32x4_t (&kr)[kF8Half], u32x4_t (&vr)[kF8Half]) {
#pragma unroll
    for (int i = 0; i < kF8Half; ++i) {
      // past the context: re-read a row; not real: the block's first row
      const int r = real ? min(wave * kF8RowsPerWave + (it0 + i) * 8 + grp, nrows - 1) : 0;
      kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kbase + r * row_stride));
      vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vbase + r * row_stride));
    }
  };
  auto consume = [&](const u32x4_t (&kr)[kF8Half], const u32x4_t (&vr)[kF8Half], int it0, int nrows) {
    // Two rows (a, b) per step: codes become bf16 pairs (exact), q.k is 8
    // v_dot2_f32_bf16 per row, and p.V pairs the two rows in one v_dot2 per dim
    // (p rounded to bf16, the sum l taken from the same rounded p). m is a
    // reference, not necessarily the running max: l and acc are relative to it,
    // which every later merge respects.
#pragma unroll
    for (int i = 0; i < kF8Half; i += 2) {
      const int it = it0 + i;
      const int ra = wave * kF8RowsPerWave + it * 8 + grp;
      const bool a_ok = ra < nrows, b_ok = ra + 8 < nrows;
      uint32_t ka[8], kb[8], vl[8], vh[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        ka[2 * w] = fp8x2_to_bf16x2<false>(kr[i][w]);
        ka[2 * w + 1] = fp8x2_to_bf16x2<true>(kr[i][w]);
        kb[2 * w] = fp8x2_to_bf16x2<false>(kr[i + 1][w]);
        kb[2 * w + 1] = fp8x2_to_bf16x2<true>(kr[i + 1][w]);
        const uint32_t va0 = fp8x2_to_bf16x2<false>(vr[i][w]), va1 = fp8x2_to_bf16x2<true>(vr[i][w]);
        const uint32_t vb0 = fp8x2_to_bf16x2<false>(vr[i + 1][w]), vb1 = fp8x2_to_bf16x2<true>(vr[i + 1][w]);
        // (v_a[e], v_b[e]) for dims e = 4w .. 4w+3
        vl[2 * w] = pair_lo(va0, vb0);
        vh[2 * w] = pair_hi(va0, vb0);
        vl[2 * w + 1] = pair_lo(va1, vb1);
        vh[2 * w + 1] = pair_hi(va1, vb1);
      }
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float sa0 = 0.0f, sa1 = 0.0f, sb0 = 0.0f, sb1 = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          sa0 = dot2_bf16(qp[g][j], ka[j], sa0);
          sa1 = dot2_bf16(qp[g][j + 1], ka[j + 1], sa1);
          sb0 = dot2_bf16(qp[g][j], kb[j], sb0);
          sb1 = dot2_bf16(qp[g][j + 1], kb[j + 1], sb1);
        }
        // rows past the context (finite re-reads) get -inf without a branch
        const float sa = fmaf(sum8(sa0 + sa1), sc, a_ok ? 0.0f : -INFINITY);
        const float sb = fmaf(sum8(sb0 + sb1), sc, b_ok ? 0.0f : -INFINITY);
        // The reference max moves only when a score passes it by more than
        // 2^8 (weights stay <= 256), so the rescale of l and acc is rare.
        const float smax = fmaxf(sa, sb);
        if (smax > m[g] + kF8Slack) {
          const float corr = exp2_fast(m[g] - smax);
          l[g] *= corr;
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[g][e] *= corr;
          m[g] = smax;
        }
        const uint32_t pp = pack_bf16x2(exp2_fast(sa - m[g]), exp2_fast(sb - m[g]));
        l[g] += bf16_lo(pp) + bf16_hi(pp);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          acc[g][2 * j] = dot2_bf16(pp, vl[j], acc[g][2 * j]);
          acc[g][2 * j + 1] = dot2_bf16(pp, vh[j], acc[g][2 * j + 1]);
        }
      }
    }
  };
  // Both halves of the first block are issued behind the query loads; the
  // query rows are then waited for (an empty asm that reads them), so that the
  // loop is entered, like its back edge, with exactly the two halves in
  // flight, the older one first (scheduling barriers keep that order).
  u32x4_t kA[kF8Half], vA[kF8Half], kB[kF8Half], vB[kF8Half];
  int nrows = min(kTokensPerBlock, ctx - b_begin * kTokensPerBlock);
  {
    const int blk = load_uniform(a.block_tables, table_row + b_begin);
    load_half(block_base(a.k_cache, blk), block_base(a.v_cache, blk), nrows, 0, true, kA, vA);
    __builtin_amdgcn_sched_barrier(0);
    load_half(block_base(a.k_cache, blk), block_base(a.v_cache, blk), nrows, kF8Half, true, kB, vB);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) asm volatile("" ::"v"(qp[g][j]));
  }
  for (int b = b_begin; b < b_end; ++b) {
    const bool more = b + 1 < b_end;
    const int blk_n = load_uniform(a.block_tables, table_row + (more ? b + 1 : b));
    const int nrows_n = more ? min(kTokensPerBlock, ctx - (b + 1) * kTokensPerBlock) : nrows;
    const uint8_t* kbn = block_base(a.k_cache, blk_n);
    const uint8_t* vbn = block_base(a.v_cache, blk_n);
    consume(kA, vA, 0, nrows);
    __builtin_amdgcn_sched_barrier(0);
    load_half(kbn, vbn, nrows_n, 0, more, kA, vA);
    __builtin_amdgcn_sched_barrier(0);
    consume(kB, vB, kF8Half, nrows);
    __builtin_amdgcn_sched_barrier(0);
    load_half(kbn, vbn, nrows_n, kF8Half, more, kB, vB);
    __builtin_amdgcn_sched_barrier(0);
    nrows = nrows_n;
  }
  // merge the 8 lane groups of the wave (lanes with the same dims differ in
  // bits 3..5): the bit-3 partner by a DPP row rotate, bits 4 and 5 by the
  // gfx950 permlane swaps (no LDS traffic). Both lanes of a pair form the same
  // merged state from the same two inputs.
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    {
      const float mo = dpp_f32<kDppRowRor8>(m[g]);
      const float lo = dpp_f32<kDppRowRor8>(l[g]);
      const bool upper = (lane & 8) != 0;
      const float m_lo = upper ? mo : m[g], m_hi = upper ? m[g] : mo;
      const float l_lo = upper ? lo : l[g], l_hi = upper ? l[g] : lo;
      const float mn = fmaxf(m_lo, m_hi);
      const float ca = exp2_fast(m_lo - mn), cb = exp2_fast(m_hi - mn);
      l[g] = l_lo * ca + l_hi * cb;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float ao = dpp_f32<kDppRowRor8>(acc[g][e]);
        const float a_lo = upper ? ao : acc[g][e], a_hi = upper ? acc[g][e] : ao;
        acc[g][e] = a_lo * ca + a_hi * cb;
      }
      m[g] = mn;
    }
#pragma unroll
    for (int step = 0; step < 2; ++step) {
      const LanePair mp = step == 0 ? pair_across_rows(m[g]) : pair_across_halves(m[g]);
      const LanePair lp = step == 0 ? pair_across_rows(l[g]) : pair_across_halves(l[g]);
      const float mn = fmaxf(mp.lo, mp.hi);
      const float ca = exp2_fast(mp.lo - mn), cb = exp2_fast(mp.hi - mn);
      l[g] = lp.lo * ca + lp.hi * cb;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const LanePair ap = step == 0 ? pair_across_rows(acc[g][e]) : pair_across_halves(acc[g][e]);
        acc[g][e] = ap.lo * ca + ap.hi * cb;
      }
      m[g] = mn;
    }
  }
  if (lane < 8) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      if (lane == 0) {
        s_m[wave][g] = m[g];
        s_l[wave][g] = l[g];
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) s_acc[wave][g][sl * 16 + e] = acc[g][e];
    }
  }
  __syncthreads();
  // the block's partial for each head: threads 0..127 take one dim each
  if (tid < kF8D) {
    const int64_t prow = (static_cast<int64_t>(seq) * a.max_chunks + chunk) * a.num_q_heads + hq0;
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      float mm = kF8Empty;
#pragma unroll
      for (int w = 0; w < kF8Waves; ++w) mm = fmaxf(mm, s_m[w][g]);
      float ll = 0.0f, aa = 0.0f;
#pragma unroll
      for (int w = 0; w < kF8Waves; ++w) {
        const float c = exp2_fast(s_m[w][g] - mm);
        ll = fmaf(s_l[w][g], c, ll);
        aa = fmaf(s_acc[w][g][tid], c, aa);
      }
      a.part_acc[(prow + g) * kF8D + tid] = aa;
      if (tid == 0) {
        a.part_ml[2 * (prow + g)] = mm;
        a.part_ml[2 * (prow + g) + 1] = ll;
      }
    }
  }
}

// Merges a sequence's block partials (in block order) into the bf16 output.
__global__ __launch_bounds__(kF8D) void decode_fp8_merge_kernel(DecodeFp8Args a) {
  const int seq = blockIdx.x / a.num_q_heads;
  const int hq = blockIdx.x % a.num_q_heads;
  const int d = threadIdx.x;
  const int ctx = min(max(a.context_lens[seq], 0), a.max_context_len);
  const int nb = (ctx + kTokensPerBlock - 1) / kTokensPerBlock;
  const int nc = (nb + a.blocks_per_chunk - 1) / a.blocks_per_chunk;
  if (nc == 0) return;  // empty context: the row stays unwritten
  float mm = kF8Empty, ll = 0.0f, aa = 0.0f;
  for (int c = 0; c < nc; ++c) {
    const int64_t prow = (static_cast<int64_t>(seq) * a.max_chunks + c) * a.num_q_heads + hq;
    const float mb = a.part_ml[2 * prow];
    const float lb = a.part_ml[2 * prow + 1];
    const float ab = a.part_acc[prow * kF8D + d];
    const float mn = fmaxf(mm, mb);
    const float ca = exp2_fast(mm - mn);
    const float cb = exp2_fast(mb - mn);
    ll = ll * ca + lb * cb;
    aa = aa * ca + ab * cb;
    mm = mn;
  }
  bf16_t* out = static_cast<bf16_t*>(a.out);
  out[(static_cast<int64_t>(seq) * a.num_q_heads + hq) * kF8D + d].bits = to_bf16_bits(aa / ll * a.v_scale);
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

hipError_t launch_decode_fp8(const DecodeFp8Args& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const int gt = decode_head_group(group);
  const int64_t items = static_cast<int64_t>(a.num_seqs) * a.max_chunks * (a.num_q_heads / gt);
  if (items == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>(items)), block(kF8Threads);
  if (gt == 4)
    decode_fp8_block_kernel<4><<<grid, block, 0, stream>>>(a);
  else if (gt == 2)
    decode_fp8_block_kernel<2><<<grid, block, 0, stream>>>(a);
  else
    decode_fp8_block_kernel<1><<<grid, block, 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_fp8_merge_kernel<<<dim3(static_cast<uint32_t>(static_cast<int64_t>(a.num_seqs) * a.num_q_heads)),
                            dim3(kF8D), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace pa
