// Paged prefill / speculative-verify attention on the matrix cores.
//
// New tokens of a sequence attend causally to its cached tokens (read from
// the pool through the block table) followed by the new tokens themselves
// (read from the call's k/v): "Nano-vLLM System Architecture Analysis",
// section 2, "Attention with Paged Cache" (prefill with a prefix cache gathers
// the cached K/V and concatenates the newly computed ones) and "Scheduler"
// (chunked prefill). Speculative verification is the same computation with a
// few new tokens ("What Is an Inference Engine, Anyway?", Technical details:
// the target model checks the proposed tokens in one mini-prefill).
//
// Items and work split. Query rows are (new token j, query head g) pairs of
// one KV head, token-major, so all GQA heads sharing the KV head ride in one
// tile. An item is (sequence, KV head, tile of ROWS query rows); its work
// units are the key tiles (64 keys; 32 for 1-wave tiles) its rows can see
// (causal: up to the tile's last token). As in decode, the units of all items are cut into equal contiguous
// shares, one per workgroup; a piece of an item is finished by the last
// workgroup to reach it, which merges the pieces' partial results in order.
//
// Per key tile, each wave (32 query rows = two 16-column MFMA tiles):
//   S^T = K Q^T   with v_mfma_f32_16x16x32_bf16: A = K rows from LDS
//                 (16 keys x 32 dims per lane group), B = the wave's query
//                 fragments held in registers. Each lane ends with 4 keys of
//                 one query column, so the softmax max is an in-lane max plus
//                 two cross-group shuffles.
//   P = 2^(S*scale*log2e - m), rounded to bf16 in registers: the S^T result
//                 layout already is the B-operand layout of the next product
//                 once the 32 keys of a step are taken in the order
//                 {4q..4q+3, 16+4q..16+4q+3} for lane group q. The row sums
//                 add the same rounded weights with v_dot2 (two per
//                 instruction) and are summed over the column's lane groups
//                 once per segment.
//   O^T += V^T P^T: A = V^T fragments read with ds_read_b64_tr_b16 from the
//                 row-major V tile (the LDS transpose read hands each lane 4
//                 consecutive keys of one head dim), B = P^T.
// The LDS operand reads of each 16-key (QK) or 32-key (PV) step are issued
// together ahead of its MFMAs.
// K/V tiles are staged in LDS by direct-to-LDS loads (no register round
// trip), in a swizzled layout, double-buffered so the next tile streams in
// while the current one is used; all waves of the workgroup share them. Rows
// beyond the context re-read a valid row and get weight 0.
#include <math.h>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr float kEmptyMaxP = -1.0e30f;
constexpr float kSlack = 8.0f;
// Cache-policy operands of the direct-to-LDS tile loads.
constexpr int kCacheAllocate = 0;  // default: the rows stay in L2 for re-reads
constexpr int kNonTemporal = 2;    // streaming: read once

typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// Shapes for head dim D and key tiles of KT keys (64 for the 8- and 4-wave
// tiles, 32 for the 1-wave verify tiles).
template <int D, int KT>
struct PShape {
  static constexpr int kDChunks = D / 32;  // k-steps of the Q.K product
  static constexpr int kDTiles = D / 16;   // 16-row tiles of O^T
  static constexpr int kRowBytes = D * 2;  // one key's head row in LDS (no padding)
  static constexpr int kPieces = D * 2 / 16;  // 16-byte pieces per row
  static constexpr int kTileBytes = KT * kRowBytes;
  static constexpr int kMt = KT / 16;   // 16-key tiles of S^T
  static constexpr int kKc2 = KT / 32;  // 32-key steps of O^T += V^T P^T
  static_assert(KT == 32 || KT == 64, "key tile");
};

// Swizzled LDS tiles: 16-byte piece c of key row r is stored at slot
// c ^ f(r) of that row (no padding bytes, which direct-to-LDS loads could not
// skip). The K pattern spreads the 16 rows an MFMA operand read touches over
// 16 bank groups; the V pattern spreads the 4 rows x 2 pieces of one
// transpose-read lane group, and neighbouring lane groups, over distinct
// bank groups.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int r) {
  return D == 128 ? (((r & 3) << 1) | (((r >> 2) & 1) << 3)) : ((r & 3) << 1);
}

// s_waitcnt vmcnt(N): wait until at most N vector-memory operations of this
// wave are outstanding (other counters unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Geometry of one sequence: n new tokens after c cached ones. Lengths are
// clamped to what the call declared (max_q_len, max_context_len), so a bad
// length can never drive a read outside the block table or a loop forever.
struct SeqGeom {
  int start;  // first row of the sequence in q/k/v/out
  int n;
  int c;
};

__device__ __forceinline__ SeqGeom seq_geom(const PrefillArgs& a, int i) {
  SeqGeom s;
  s.start = min(max(a.cu_seqlens[i], 0), a.total_q);
  s.n = min(min(max(a.cu_seqlens[i + 1] - s.start, 0), a.max_q_len), a.total_q - s.start);
  s.c = min(max(a.context_lens[i] - s.n, 0), max(a.max_context_len - s.n, 0));
  return s;
}

// KT-key tiles visible to query tile qt (rows qt*ROWS .. qt*ROWS+ROWS-1).
template <int ROWS, int KT>
__device__ __forceinline__ int tiles_of(const SeqGeom& s, int group, int qt) {
  const int jmax = min(s.n - 1, ((qt + 1) * ROWS - 1) / group);
  return (s.c + jmax + 1 + KT - 1) / KT;
}

template <int ROWS>
__device__ __forceinline__ int qtiles_of(const SeqGeom& s, int group) {
  return (s.n * group + ROWS - 1) / ROWS;
}

// An item (sequence, KV head, query tile) costs its key tiles plus
// kItemCost units ahead of them that hold no tiles: they stand for the fixed
// work of a segment (loading its query rows, the first tile's latency, the
// output and the barriers), about three tiles' time on MI355X, so ranges of
// many items carry fewer tiles and all ranges take about the same time.
constexpr int kItemCost = 3;

template <int ROWS, int KT>
__device__ int units_per_head(const SeqGeom& s, int group) {
  if (s.n <= 0) return 0;
  const int qts = qtiles_of<ROWS>(s, group);
  int u = 0;
  for (int qt = 0; qt < qts; ++qt) u += tiles_of<ROWS, KT>(s, group, qt) + kItemCost;
  return u;
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2), so workgroup ids w, w+8, w+16, ... share an L2. Give those workgroups
// consecutive work ranges: the query tiles of one (sequence, KV head), which
// stream the same K/V tiles, then run under one L2. A bijection on [0, G).
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_local_range(int wg, int G) {
  const int per = G / kXcds;
  if (wg >= per * kXcds) return wg;  // the remainder keeps its own id
  return (wg % kXcds) * per + wg / kXcds;
}

__device__ __forceinline__ int owner_of_unit(int64_t u, int64_t U, int64_t G) {
  return static_cast<int>(((u + 1) * G - 1) / U);
}

// Where the rows of a key tile come from: the pool (through the block table)
// for positions below c, the call's k/v for the new tokens.
template <int D_, int NT_, int KT_>
struct TileSrc {
  static constexpr int D = D_;
  static constexpr int NT = NT_;
  static constexpr int KT = KT_;
  // The 8-wave tiles serve items of more than 128 query rows, i.e. long runs
  // of new tokens whose query tiles each read the same keys (and whose
  // sequences often share a prefix): their loads allocate in the caches, so
  // those re-reads are served by the 256 MB memory-side cache rather than
  // HBM (chunked prefill with a shared prefix on MI355X: 82 -> 71 us, while
  // the L2 hit rate moved only from 38% to 41%). The verify tiles read each
  // row once and stream (allocating there slowed a 5 GB verify by 13%); the
  // 4-wave tiles, one query tile per item, stream as well.
  static constexpr int kPolicy = NT >= 512 ? kCacheAllocate : kNonTemporal;
  const bf16_t* kpool;
  const bf16_t* vpool;
  const bf16_t* kg;
  const bf16_t* vg;
  const int32_t* table;
  int64_t tok_stride;
  int64_t head_off;
  int start;  // first row of the sequence's new tokens in k/v
  int c;      // cached positions
  int total;  // cached + new positions
  // Block ids of the cached part, one per lane, 64 at a time: a tile takes
  // its id with a lane read, so no tile issue waits on a block-table load
  // (which, in the in-order queue of vector loads, would wait for every tile
  // load in flight).
  int win_base;   // first block index held
  int win_limit;  // blocks of the cached part
  int win;        // this lane's id: table[win_base + lane]

  // Loads the window at block b and completes it (a rare path: once per
  // segment and once per 64 blocks).
  __device__ __forceinline__ void fill(int b, int lane) {
    win_base = b;
    win = b + lane < win_limit ? table[b + lane] : 0;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }
  __device__ __forceinline__ int block(int b, int lane) {
    if (b - win_base >= kWave) fill(b, lane);  // wave-uniform, rare
    return __builtin_amdgcn_readlane(win, b - win_base);
  }
};

// Issue the direct-to-LDS loads of key tile kt into one stage ([K tile | V
// tile]). Each wave instruction fills 1 KB of LDS in lane order. A tile that
// lies wholly in the pool or wholly in the new tokens uses one wave-uniform
// base plus the precomputed lane offsets; a tile that straddles the two, or
// runs past the last key (its rows re-read the last key), resolves each
// lane's row on its own.
template <class Src>
__device__ __forceinline__ void issue_tile(Src& t, int kt, char* stage, const int* krow, const int* kgo,
                                           const int* vgo, int tid, int wave) {
  constexpr int D = Src::D;
  constexpr int NT = Src::NT;
  constexpr int KT = Src::KT;
  constexpr int kIters = KT * PShape<D, KT>::kPieces / NT;  // one 16-byte piece per thread and iteration
  constexpr int TB = PShape<D, KT>::kTileBytes;
  const int k0 = kt * KT;
  char* kdst = stage;
  char* vdst = stage + TB;
  const bool in_pool = k0 + KT <= t.c;
  const bool in_new = k0 >= t.c && k0 + KT <= t.total;
  if (in_pool || in_new) {
    int64_t row0;
    const bf16_t* kb;
    const bf16_t* vb;
    if (in_pool) {
      const int block = t.block(k0 / kTokensPerBlock, tid & (kWave - 1));
      row0 = static_cast<int64_t>(block) * kTokensPerBlock + k0 % kTokensPerBlock;
      kb = t.kpool;
      vb = t.vpool;
    } else {
      row0 = static_cast<int64_t>(t.start) + (k0 - t.c);
      kb = t.kg;
      vb = t.vg;
    }
    kb += row0 * t.tok_stride + t.head_off;
    vb += row0 * t.tok_stride + t.head_off;
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int lds_off = (it * NT + wave * kWave) * 16;
      __builtin_amdgcn_global_load_lds(kb + kgo[it], (lds_void_t*)(kdst + lds_off), 16, 0, Src::kPolicy);
      __builtin_amdgcn_global_load_lds(vb + vgo[it], (lds_void_t*)(vdst + lds_off), 16, 0, Src::kPolicy);
    }
  } else {
    const int block = k0 < t.c ? t.block(k0 / kTokensPerBlock, tid & (kWave - 1)) : 0;
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int kr = krow[it];
      const int lds_off = (it * NT + wave * kWave) * 16;
      const int pos = min(k0 + kr, t.total - 1);
      const bool cached = pos < t.c;
      const int64_t row = cached ? static_cast<int64_t>(block) * kTokensPerBlock + pos % kTokensPerBlock
                                 : static_cast<int64_t>(t.start) + (pos - t.c);
      // kgo/vgo hold kr * tok_stride + piece; re-base them on the lane's own row
      const int64_t base = (row - kr) * t.tok_stride + t.head_off;
      const bf16_t* ksrc = (cached ? t.kpool : t.kg) + base + kgo[it];
      const bf16_t* vsrc = (cached ? t.vpool : t.vg) + base + vgo[it];
      __builtin_amdgcn_global_load_lds(ksrc, (lds_void_t*)(kdst + lds_off), 16, 0, Src::kPolicy);
      __builtin_amdgcn_global_load_lds(vsrc, (lds_void_t*)(vdst + lds_off), 16, 0, Src::kPolicy);
    }
  }
}

// Log-sum-exp merge of the pieces of one split item, for the query rows and
// dims one lane holds in the MFMA output layout (rows wave*RPW + 16nt + col,
// dims 16dt + 4grp .. +3). Row r of the result is
// sum_p 2^(lse_p - M) o_p / sum_p 2^(lse_p - M): the pieces are folded one by
// one in piece order with a running maximum M, each fold step written with
// explicit fused multiply-adds, so that the result does not depend on which
// workgroup merges or where the pieces come from (a piece whose keys are all
// causally hidden from a row has lse = -inf and weight 0). A piece's partial
// o_p is four bf16 values per dt, packed in a uint2.
template <int DT>
__device__ __forceinline__ void fold_piece(float& m, float& den, f32x4_t (&num)[DT], float lse,
                                           const uint2 (&o)[DT]) {
  if (lse == -INFINITY) return;
  const float mn = fmaxf(m, lse);
  const float r = m == -INFINITY ? 0.0f : exp2_fast(m - mn);
  const float f = exp2_fast(lse - mn);
  den = __builtin_fmaf(den, r, f);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const float v[4] = {bf16_lo(o[dt].x), bf16_hi(o[dt].x), bf16_lo(o[dt].y), bf16_hi(o[dt].y)};
#pragma unroll
    for (int e = 0; e < 4; ++e) num[dt][e] = __builtin_fmaf(f, v[e], num[dt][e] * r);
  }
  m = mn;
}

// Tagged piece counter of item (sequence seq, KV head h, query tile qt):
// one word per query tile the longest query could have.
__device__ __forceinline__ uint64_t* piece_counter(const PrefillArgs& a, int seq, int h, int qt, int group, int Hkv,
                                                   int rows) {
  const int64_t qtiles_max = (static_cast<int64_t>(a.max_q_len) * group + rows - 1) / rows;
  return a.counters + (static_cast<int64_t>(seq) * Hkv + h) * qtiles_max + qt;
}

// A value the caller knows to be the same on every lane of the wave, moved to
// scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint64_t u = static_cast<uint64_t>(v);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Byte offset, in a piece slot, of the 16 bytes that lane `lane` of wave
// `wave` holds for its MFMA column tile nt and dims 32c .. 32c + 31 (its
// dt = 2c and 2c + 1 quadruples), as bf16. The slot is laid out in the
// lanes' own order, so that each store or load instruction of a wave covers
// 1 KB of contiguous memory.
template <int DT, int NTW>
__device__ __forceinline__ int piece_chunk_offset(int wave, int nt, int c, int lane) {
  return (((wave * NTW + nt) * (DT / 2) + c) * 64 + lane) * 16;
}

// Where a split item's pieces live: piece p in slot 2(first_owner + p), or
// 2 first_owner + 1 for the first piece when its owner's range starts inside
// an earlier item (that owner's first segment took slot 2 first_owner).
struct PieceSlots {
  int64_t first_owner;
  int n_parts;
  bool first_late;
  __device__ int64_t slot(int p) const { return 2 * (first_owner + p) + (p == 0 && first_late ? 1 : 0); }
};

// Merges a split item's pieces into the output rows this lane holds. Piece
// `own` (or none, -1) is taken from the caller's registers (own_o, own_lse:
// its bf16 partial and log-sum-exp, as they would have been stored); the
// other pieces are read from the workspace, kBatch of them in flight at a
// time. With `poison` (the item's counter held another call's tag, so its
// pieces cannot be trusted) the rows are written as NaN instead.
template <int D, int ROWS, int NTW, int kBatch>
__device__ __forceinline__ void merge_item_rows(const PrefillArgs& a, bf16_t* outp, const PieceSlots& ps, int own,
                                                const uint2 (&own_o)[NTW][D / 16], const float (&own_lse)[NTW],
                                                const SeqGeom& sg, int qt, int h, int group, int wave, int col,
                                                int grp, bool poison) {
  constexpr int DT = D / 16;
  constexpr int RPW = 16 * NTW;
  const int lane = grp * 16 + col;
  int tok[NTW], head[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int R = qt * ROWS + wave * RPW + nt * 16 + col;
    tok[nt] = R / group;
    head[nt] = h * group + R % group;
  }
  if (poison) {
    const uint32_t nan2 = pack_bf16x2(__builtin_nanf(""), __builtin_nanf(""));
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      if (tok[nt] >= sg.n) continue;
      bf16_t* orow = outp + (static_cast<int64_t>(sg.start + tok[nt]) * a.num_q_heads + head[nt]) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<uint2*>(orow + dt * 16 + grp * 4) = make_uint2(nan2, nan2);
    }
    return;
  }
  float m[NTW], den[NTW];
  f32x4_t num[NTW][DT];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    m[nt] = -INFINITY;
    den[nt] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) num[nt][dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
  // pieces [p_begin, p_end) from the workspace
  auto fold_stored = [&](int p_begin, int p_end) {
    for (int p0 = p_begin; p0 < p_end; p0 += kBatch) {
      float lv[kBatch][NTW];
      uint2 ov[kBatch][NTW][DT];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (p0 + j >= p_end) continue;
        // the slot is the same on every lane: keep it (and the descriptor) scalar
        const int64_t slot = uniform64(ps.slot(p0 + j));
        const __amdgpu_buffer_rsrc_t pr = buffer_rsrc(a.part_out + slot * ROWS * D, ROWS * D * 2);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          const int row = wave * RPW + nt * 16 + col;
          lv[j][nt] = load_agent(a.part_lse + slot * ROWS + row);
#pragma unroll
          for (int c = 0; c < DT / 2; ++c) {
            const f32x4_t v = load4_agent(pr, piece_chunk_offset<DT, NTW>(wave, nt, c, lane));
            const uint4 u = __builtin_bit_cast(uint4, v);
            ov[j][nt][2 * c] = make_uint2(u.x, u.y);
            ov[j][nt][2 * c + 1] = make_uint2(u.z, u.w);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (p0 + j >= p_end) break;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) fold_piece<DT>(m[nt], den[nt], num[nt], lv[j][nt], ov[j][nt]);
      }
    }
  };
  if (own < 0) {
    fold_stored(0, ps.n_parts);
  } else {
    fold_stored(0, own);
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) fold_piece<DT>(m[nt], den[nt], num[nt], own_lse[nt], own_o[nt]);
    fold_stored(own + 1, ps.n_parts);
  }
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    if (tok[nt] >= sg.n) continue;
    const float inv = 1.0f / den[nt];
    bf16_t* orow = outp + (static_cast<int64_t>(sg.start + tok[nt]) * a.num_q_heads + head[nt]) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint32_t lo = pack_bf16x2(num[nt][dt][0] * inv, num[nt][dt][1] * inv);
      const uint32_t hi = pack_bf16x2(num[nt][dt][2] * inv, num[nt][dt][3] * inv);
      *reinterpret_cast<uint2*>(orow + dt * 16 + grp * 4) = make_uint2(lo, hi);
    }
  }
}

// A workgroup barrier without the memory fence of __syncthreads(). With
// direct-to-LDS loads in flight that fence makes the compiler wait for all
// of them (vmcnt 0), the next tile's included; the two-stage tile loop
// instead waits for its own tile explicitly before the barrier, and every
// LDS read is consumed (waited for) before its wave reaches the next one.
__device__ __forceinline__ void tile_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// LDS stages of [K tile | V tile] per workgroup: the 8-wave workgroup (one
// per CU) works its 64-key tiles in pairs, four stages (128 KB): one barrier
// per pair, after which the next pair loads while this one is used, so the
// waves drift apart within a pair instead of meeting at every tile (measured
// 4% faster than three stages with a barrier per tile); the 4-wave ones (two
// per CU) keep one tile in flight while they work on another. The 1-wave
// verify workgroup takes 32-key tiles, two stages (32 KB), so that four fit
// in a CU's LDS: measured on MI355X, four such workgroups per CU stream 8%
// faster than two with 64-key tiles (more waves, and more loads in flight
// per CU), while one or two workgroups with deeper pipelines are slower.
template <int ROWS>
constexpr int prefill_stages() {
  return ROWS >= 256 ? 4 : 2;
}
template <int WM, int ROWS>
constexpr int prefill_workgroups_per_cu() {
  return ROWS >= 256 ? 1 : (WM == 1 ? 4 : 2);
}

// WM waves per workgroup, each owning NTW 16-column MFMA tiles of query
// rows (16 * NTW rows), so ROWS = 16 * NTW * WM rows per item.
template <int D, int WM, int KT, int NTW>
__global__ __launch_bounds__(64 * WM, (prefill_workgroups_per_cu<WM, 16 * NTW * WM>())) void paged_prefill_kernel(
    PrefillArgs a) {
  using S = PShape<D, KT>;
  constexpr int RPW = 16 * NTW;  // query rows per wave
  constexpr int ROWS = RPW * WM;
  constexpr int NT = kWave * WM;
  constexpr int TB = S::kTileBytes;
  constexpr int kStages = prefill_stages<ROWS>();
  constexpr bool kPaired = kStages == 4;  // tiles in pairs, one barrier per pair
  constexpr int kAhead = kPaired ? 2 : 1;  // tiles issued before the loop
  static_assert(kStages == (kPaired ? 4 : 2), "two stages, or four in pairs");
  // One LDS object per stage ([K tile | V tile]), each named where it is
  // used: the compiler's waits for direct-to-LDS loads then tell the stages
  // apart (one alias scope per object), so the reads of one stage do not wait
  // for the loads still filling another. With one array indexed by stage it
  // waited for every load in flight before a tile's first LDS read, and the
  // next tiles' loads never overlapped the work on this one. Stages 2 and 3
  // are used by the paired 8-wave tiles only.
  __shared__ __attribute__((aligned(16))) char s_kv0[2 * TB];
  __shared__ __attribute__((aligned(16))) char s_kv1[2 * TB];
  __shared__ __attribute__((aligned(16))) char s_kv2[kPaired ? 2 * TB : 16];
  __shared__ __attribute__((aligned(16))) char s_kv3[kPaired ? 2 * TB : 16];
  __shared__ int s_wsum[WM];
  __shared__ int s_loc[2];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // wave index made provably wave-uniform, so per-wave addresses (block-table
  // entries) are scalar loads that do not queue behind the vector loads
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int col = lane & 15;  // MFMA column (query) / row-in-tile index
  const int grp = lane >> 4;  // MFMA lane group (k sub-block)
  const int B = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  const int group = a.num_q_heads / Hkv;

  // ---- 1. Units per sequence (all KV heads), and their inclusive prefix sum
  // over the threads: within each wave by lane shuffles, then across the
  // waves through LDS (one barrier).
  const int per = (B + NT - 1) / NT;
  int mine = 0;
  for (int k = 0; k < per; ++k) {
    const int i = tid * per + k;
    if (i < B) mine += Hkv * units_per_head<ROWS, KT>(seq_geom(a, i), group);
  }
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
  for (int k = 0; k < WM; ++k) {
    const int v = s_wsum[k];
    if (k < wave) incl += v;
    total += v;
  }
  const int64_t U = __builtin_amdgcn_readfirstlane(total);
  if (U == 0) return;
  const int64_t G = min(static_cast<int64_t>(gridDim.x), U);
  const int w = xcd_local_range(static_cast<int>(blockIdx.x), static_cast<int>(G));
  if (w >= G) return;
  const int64_t u_begin = static_cast<int64_t>(w) * U / G;
  const int64_t u_end = static_cast<int64_t>(w + 1) * U / G;

  // ---- 2. Sequence holding u_begin.
  {
    const int64_t lo = incl - mine;
    if (u_begin >= lo && u_begin < incl) {
      int64_t base = lo;
      for (int k = 0; k < per && tid * per + k < B; ++k) {
        const int i = tid * per + k;
        const int64_t span = static_cast<int64_t>(Hkv) * units_per_head<ROWS, KT>(seq_geom(a, i), group);
        if (u_begin < base + span) {
          s_loc[0] = i;
          s_loc[1] = static_cast<int>(base);
          break;
        }
        base += span;
      }
    }
  }
  __syncthreads();
  // Values read back from LDS are uniform; say so, so that the walk and the
  // block-table lookups stay in scalar registers.
  int seq = __builtin_amdgcn_readfirstlane(s_loc[0]);
  int64_t seq_base = __builtin_amdgcn_readfirstlane(s_loc[1]);

  // Per-lane LDS offsets of the MFMA operands, fixed for the whole kernel:
  // K rows 16mt + col, piece 4kc + grp (the mt step is an immediate);
  // V transpose reads rows 32kc2 + 4grp + col/4 (+16), 4 dims at
  // 16dt + 4(col%4) (the kc2 and +16 steps are immediates).
  constexpr int RB = S::kRowBytes;
  int koff[S::kDChunks];
#pragma unroll
  for (int kc = 0; kc < S::kDChunks; ++kc) koff[kc] = col * RB + (((kc * 4 + grp) ^ k_swz<D>(col)) << 4);
  int voff[S::kDTiles];
  {
    const int vr = grp * 4 + (col >> 2);
#pragma unroll
    for (int dt = 0; dt < S::kDTiles; ++dt)
      voff[dt] = vr * RB + (((dt * 2 + ((col & 3) >> 1)) ^ v_swz<D>(vr)) << 4) + (col & 1) * 8;
  }
  // Per-lane global element offsets of the tile loads (row kr of the tile,
  // the 16-byte piece that lands in this lane's LDS slot), for K and V.
  constexpr int kIters = KT * S::kPieces / NT;
  const int64_t tok_stride = static_cast<int64_t>(Hkv) * D;  // elements between token rows
  int krow[kIters], kgo[kIters], vgo[kIters];
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int idx = it * NT + tid;
    const int kr = idx / S::kPieces;
    const int slot = idx % S::kPieces;
    krow[it] = kr;
    kgo[it] = kr * static_cast<int>(tok_stride) + ((slot ^ k_swz<D>(kr)) << 3);
    vgo[it] = kr * static_cast<int>(tok_stride) + ((slot ^ v_swz<D>(kr)) << 3);
  }

  const bf16_t* qg = static_cast<const bf16_t*>(a.q);
  const bf16_t* kg = static_cast<const bf16_t*>(a.k);
  const bf16_t* vg = static_cast<const bf16_t*>(a.v);
  const bf16_t* kpool = static_cast<const bf16_t*>(a.k_cache);
  const bf16_t* vpool = static_cast<const bf16_t*>(a.v_cache);
  bf16_t* outp = static_cast<bf16_t*>(a.out);
  // Scores are kept in log2 units: p = 2^(s*sc - m). The host passes
  // sc = |scale * log2(e)| (never 0) and asks for q to be negated when the
  // scale is negative, so that max(s) * sc is the scaled maximum.
  const float sc = a.scale_log2;
  const uint32_t qflip = a.negate_q ? 0x80008000u : 0u;

  // Split-item pieces this workgroup stores (at most its first and its last
  // segment), counted at the end.
  int pend_n[2] = {0, 0};
  int pend_seq[2] = {0, 0};
  int pend_h[2] = {0, 0};
  int pend_qt[2] = {0, 0};
  int64_t pend_first[2] = {0, 0};
  int64_t pend_item_first[2] = {0, 0};
  bool first_counted = false;  // the first pending piece was counted when it was stored
  int first_state = 0;         // (thread 0) that count: 1 completes the item, -1 foreign counter
  __shared__ int s_cnt[2];

  // ---- 3. Segments.
  bool first_seg = true;  // no segment with tiles done yet (its piece goes to slot 2w)
  // A last piece merged at once (see the end of a segment): its item; the
  // piece itself, as it would have been stored, waits in LDS (the K/V stages,
  // free by then; each wave its own words, lane-major), so that it does not
  // occupy registers through the tile loops of every earlier segment.
  bool merge_last = false;
  PieceSlots last_ps{0, 0, false};
  int last_seq = 0, last_h = 0, last_qt = 0;
  constexpr int kLastWords = NTW * S::kDTiles * 2 + NTW;  // bf16 words of the piece, then its lse
  constexpr int kLastBytes = kLastWords * kWave * 4;  // one wave's words
  constexpr int kLastPerStage = 2 * TB / kLastBytes;  // waves whose words fit in one stage
  static_assert(kLastPerStage >= 1 && WM <= kLastPerStage * kStages, "last piece in LDS");
  char* const last_stage = wave < kLastPerStage       ? s_kv0
                           : wave < 2 * kLastPerStage ? s_kv1
                           : wave < 3 * kLastPerStage ? s_kv2
                                                      : s_kv3;
  uint32_t* const s_last = reinterpret_cast<uint32_t*>(last_stage + (wave % kLastPerStage) * kLastBytes) + lane;
  int64_t u = u_begin;
  while (u < u_end) {
    const SeqGeom sg = seq_geom(a, seq);
    const int uph = units_per_head<ROWS, KT>(sg, group);
    const int64_t r = u - seq_base;
    const int h = static_cast<int>(r / uph);
    int r2 = static_cast<int>(r % uph);
    int qt = 0;
    int acc_units = 0;
    int nkt = tiles_of<ROWS, KT>(sg, group, 0);
    while (r2 >= acc_units + nkt + kItemCost) {
      acc_units += nkt + kItemCost;
      ++qt;
      nkt = tiles_of<ROWS, KT>(sg, group, qt);
    }
    // cost units of the item: kItemCost virtual ones, then one per key tile
    const int64_t item_first = seq_base + static_cast<int64_t>(h) * uph + acc_units;
    const int64_t real_first = item_first + kItemCost;
    const int64_t item_end = real_first + nkt;
    const int64_t seg_end = u_end < item_end ? u_end : item_end;
    const int64_t lo = u > real_first ? u : real_first;
    if (lo >= seg_end) {  // only virtual units of this item lie in the range
      u = seg_end;
      if (u == item_end && u < u_end && u - seq_base >= static_cast<int64_t>(Hkv) * uph) {
        seq_base = u;
        ++seq;
        while (seq < B - 1 && units_per_head<ROWS, KT>(seq_geom(a, seq), group) == 0) ++seq;
      }
      continue;
    }
    const int t_lo = static_cast<int>(lo - real_first);
    const int t_hi = static_cast<int>(seg_end - real_first);
    const int total_keys = sg.c + sg.n;

    // The segment's first K/V tile starts loading before the query rows, so
    // the two latencies overlap.
    const int32_t* table = a.block_tables + static_cast<int64_t>(seq) * a.max_blocks_per_seq;
    const int64_t head_off = static_cast<int64_t>(h) * D;
    TileSrc<D, NT, KT> src;
    src.kpool = kpool;
    src.vpool = vpool;
    src.kg = kg;
    src.vg = vg;
    src.table = table;
    src.tok_stride = tok_stride;
    src.head_off = head_off;
    src.start = sg.start;
    src.c = sg.c;
    src.total = total_keys;
    src.win_limit = (sg.c + kTokensPerBlock - 1) / kTokensPerBlock;
    src.fill(t_lo * KT / kTokensPerBlock, lane);
    if (t_lo < t_hi) issue_tile(src, t_lo, s_kv0, krow, kgo, vgo, tid, wave);
    // This wave's query columns: nt in {0,1}, column col.
    int qrow_tok[NTW];   // token index j of the lane's query column (may be >= n: padding)
    int qrow_head[NTW];  // query head
    bf16x8_t qf[NTW][S::kDChunks];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const int R = qt * ROWS + wave * RPW + nt * 16 + col;
      const int j = R / group;
      const int g = R % group;
      qrow_tok[nt] = j;
      qrow_head[nt] = h * group + g;
      const int jj = min(j, sg.n - 1);
      const bf16_t* qrow = qg + (static_cast<int64_t>(sg.start + jj) * a.num_q_heads + h * group + g) * D;
#pragma unroll
      for (int kc = 0; kc < S::kDChunks; ++kc) {
        u32x4_t w4 = *reinterpret_cast<const u32x4_t*>(qrow + kc * 32 + grp * 8);
        w4 ^= qflip;
        qf[nt][kc] = __builtin_bit_cast(bf16x8_t, w4);
      }
    }
    // Later prologue tiles are issued after the query rows, so the wait for
    // those rows (in-order completion) does not wait for them.
    if constexpr (kAhead > 1)
      if (t_lo + 1 < t_hi) issue_tile(src, t_lo + 1, s_kv1, krow, kgo, vgo, tid, wave);
    // Keys a query column may see: positions <= c + j, clamped to the last key.
    int vis[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) vis[nt] = min(sg.c + qrow_tok[nt], total_keys - 1);
    // Smallest visible-key bound over the wave's real rows (its first row):
    // a tile entirely below it needs no mask.
    const int wave_min_vis = min(sg.c + (qt * ROWS + wave * RPW) / group, total_keys - 1);

    f32x4_t acc_o[NTW][S::kDTiles];
    // Row sums of the bf16-rounded weights over the lane's own keys (each
    // lane holds 4 keys of every 16-key tile of its column), summed across
    // the column's 4 lane groups when the segment ends.
    float lsum[NTW];
    float m[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      m[nt] = kEmptyMaxP;
      lsum[nt] = 0.0f;
#pragma unroll
      for (int dt = 0; dt < S::kDTiles; ++dt) acc_o[nt][dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // The three phases of a key tile, for one wave's rows.
    // S^T = K Q^T: st[mt][nt] holds keys 16mt + 4grp + e of query column col.
    // The operand reads of a 16-key step are all issued before its MFMAs,
    // so the LDS latency is exposed once per step rather than once per read.
    auto qk = [&](const char* s_k, f32x4_t (&st)[S::kMt][NTW]) __attribute__((always_inline)) {
#pragma unroll
      for (int mt = 0; mt < S::kMt; ++mt) {
        bf16x8_t kfrag[S::kDChunks];
#pragma unroll
        for (int kc = 0; kc < S::kDChunks; ++kc)
          kfrag[kc] = *reinterpret_cast<const bf16x8_t*>(s_k + koff[kc] + mt * 16 * RB);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) st[mt][nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kc = 0; kc < S::kDChunks; ++kc)
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) st[mt][nt] = mfma16(kfrag[kc], qf[nt][kc], st[mt][nt]);
        __builtin_amdgcn_sched_group_barrier(0x100, S::kDChunks, 0);  // the step's LDS reads first
        __builtin_amdgcn_sched_group_barrier(0x008, S::kDChunks * NTW, 0);  // then its MFMAs
      }
    };
    // Online softmax of a tile starting at key k0 (raw scores; sc > 0): the
    // causal mask, the running max (refreshed only when a score passes it by
    // 2^kSlack), and the bf16 weights as P^T operands: for key step kc2 the
    // lane's 8 keys are {4grp..4grp+3} of S^T tile 2kc2 and the same of tile
    // 2kc2+1. The row sums take the same bf16-rounded weights.
    auto softmax = [&](f32x4_t (&st)[S::kMt][NTW], int k0, bf16x8_t (&pb)[NTW][S::kKc2]) __attribute__((always_inline)) {
      const bool full_tile = k0 + KT - 1 <= wave_min_vis;
      if (!full_tile) {
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
          for (int mt = 0; mt < S::kMt; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (k0 + mt * 16 + grp * 4 + e > vis[nt]) st[mt][nt][e] = -INFINITY;
      }
      bool need = false;
      float mx[NTW];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        float t = fmaxf(fmaxf(st[0][nt][0], st[0][nt][1]), fmaxf(st[0][nt][2], st[0][nt][3]));
#pragma unroll
        for (int mt = 1; mt < S::kMt; ++mt)
          t = fmaxf(t, fmaxf(fmaxf(st[mt][nt][0], st[mt][nt][1]), fmaxf(st[mt][nt][2], st[mt][nt][3])));
        {
          const LanePair r = pair_across_rows(t);
          t = fmaxf(r.lo, r.hi);
          const LanePair h = pair_across_halves(t);
          t = fmaxf(h.lo, h.hi);
        }
        mx[nt] = fmaxf(m[nt], t * sc);
        need |= mx[nt] > m[nt] + kSlack;
      }
      if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          const float alpha = exp2_fast(m[nt] - mx[nt]);
          lsum[nt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < S::kDTiles; ++dt) acc_o[nt][dt] *= alpha;
          m[nt] = mx[nt];
        }
      }
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const float nm = -m[nt];
#pragma unroll
        for (int kc2 = 0; kc2 < S::kKc2; ++kc2) {
          const f32x4_t& s0 = st[2 * kc2][nt];
          const f32x4_t& s1 = st[2 * kc2 + 1][nt];
          const u32x4_t w = {pack_bf16x2(exp2_fast(fmaf(s0[0], sc, nm)), exp2_fast(fmaf(s0[1], sc, nm))),
                             pack_bf16x2(exp2_fast(fmaf(s0[2], sc, nm)), exp2_fast(fmaf(s0[3], sc, nm))),
                             pack_bf16x2(exp2_fast(fmaf(s1[0], sc, nm)), exp2_fast(fmaf(s1[1], sc, nm))),
                             pack_bf16x2(exp2_fast(fmaf(s1[2], sc, nm)), exp2_fast(fmaf(s1[3], sc, nm)))};
          pb[nt][kc2] = __builtin_bit_cast(bf16x8_t, w);
#pragma unroll
          for (int e = 0; e < 4; ++e) lsum[nt] = dot2_bf16(w[e], 0x3F803F80u, lsum[nt]);
        }
      }
    };
    // O^T += V^T P^T: V^T operands by LDS transpose reads of the row-major V tile.
    auto pv = [&](const char* s_v, const bf16x8_t (&pb)[NTW][S::kKc2]) __attribute__((always_inline)) {
      typedef short i16x8_t __attribute__((ext_vector_type(8)));
#pragma unroll
      for (int kc2 = 0; kc2 < S::kKc2; ++kc2) {
        bf16x8_t vfrag[S::kDTiles];
#pragma unroll
        for (int dt = 0; dt < S::kDTiles; ++dt) {
          const char* pvp = s_v + voff[dt] + kc2 * 32 * RB;
          const i16x4_t ta = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(pvp));
          const i16x4_t tb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(pvp + 16 * RB));
          const i16x8_t t8 = {ta[0], ta[1], ta[2], ta[3], tb[0], tb[1], tb[2], tb[3]};
          vfrag[dt] = __builtin_bit_cast(bf16x8_t, t8);
        }
#pragma unroll
        for (int dt = 0; dt < S::kDTiles; ++dt)
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) acc_o[nt][dt] = mfma16(vfrag[dt], pb[nt][kc2], acc_o[nt][dt]);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * S::kDTiles, 0);  // the step's LDS reads first
        __builtin_amdgcn_sched_group_barrier(0x008, S::kDTiles * NTW, 0);  // then its MFMAs
      }
    };
    constexpr int L = 2 * kIters;  // loads per tile per thread

    // One key tile of this wave's rows from stage `stg`.
    auto tile = [&](int kt, const char* stg) __attribute__((always_inline)) {
      f32x4_t st[S::kMt][NTW];
      qk(stg, st);
      bf16x8_t pb[NTW][S::kKc2];
      softmax(st, kt * KT, pb);
      pv(stg + TB, pb);
    };
    if constexpr (kPaired) {
      // At a pair's start its two tiles are the only loads in flight: wait
      // for both, then one barrier makes them complete for every wave and
      // shows every wave is done with the previous pair, whose stages then
      // take the next two tiles. Stages 0/1 and 2/3 alternate.
      auto pair = [&](int kt, const char* use0, const char* use1, char* next0, char* next1) __attribute__((always_inline)) {
        wait_vmcnt<0>();
        __syncthreads();
        if (kt + 2 < t_hi) issue_tile(src, kt + 2, next0, krow, kgo, vgo, tid, wave);
        if (kt + 3 < t_hi) issue_tile(src, kt + 3, next1, krow, kgo, vgo, tid, wave);
        tile(kt, use0);
        if (kt + 1 < t_hi) tile(kt + 1, use1);
      };
      for (int kt = t_lo; kt < t_hi; kt += 4) {
        pair(kt, s_kv0, s_kv1, s_kv2, s_kv3);
        if (kt + 2 < t_hi) pair(kt + 2, s_kv2, s_kv3, s_kv0, s_kv1);
      }
    } else {
      // Issue the next tile into the other stage (every wave finished with
      // it at the barrier ending the previous tile), then wait for this one.
      // The 4-wave tiles meet at fence-free barriers, so the next tile's
      // loads stay in flight (an 8 x 512-token chunked prefill forced onto
      // 128-row tiles: 90 -> 72-77 us on MI355X); the 1-wave verify tile
      // keeps __syncthreads(), whose wait for every load in flight measured
      // 2% faster on a 5 GB verify.
      auto barrier = [&]() __attribute__((always_inline)) {
        if constexpr (WM > 1) tile_barrier();
        else __syncthreads();
      };
      auto step = [&](int kt, const char* use, char* next) __attribute__((always_inline)) {
        if (kt + 1 < t_hi) {
          issue_tile(src, kt + 1, next, krow, kgo, vgo, tid, wave);
          wait_vmcnt<L>();
        } else {
          wait_vmcnt<0>();
        }
        barrier();
        tile(kt, use);
        barrier();  // the next tile overwrites this stage
      };
      for (int kt = t_lo; kt < t_hi; kt += 2) {
        step(kt, s_kv0, s_kv1);
        if (kt + 1 < t_hi) step(kt + 1, s_kv1, s_kv0);
      }
    }

    // ---- finish the segment: output or partial
    float lt[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      // the column's 4 lane groups: rows 16-apart, then halves (same order on
      // every lane, so every lane of the column gets the same sum)
      const LanePair r = pair_across_rows(lsum[nt]);
      const float t = r.lo + r.hi;
      const LanePair h = pair_across_halves(t);
      lt[nt] = h.lo + h.hi;
    }
    const int first_owner = owner_of_unit(real_first, U, G);
    const int n_parts = owner_of_unit(item_end - 1, U, G) - first_owner + 1;
    if (n_parts == 1) {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        if (qrow_tok[nt] >= sg.n) continue;
        const float inv = 1.0f / lt[nt];
        bf16_t* orow = outp + (static_cast<int64_t>(sg.start + qrow_tok[nt]) * a.num_q_heads + qrow_head[nt]) * D;
#pragma unroll
        for (int dt = 0; dt < S::kDTiles; ++dt) {
          const uint32_t lo = pack_bf16x2(acc_o[nt][dt][0] * inv, acc_o[nt][dt][1] * inv);
          const uint32_t hi = pack_bf16x2(acc_o[nt][dt][2] * inv, acc_o[nt][dt][3] * inv);
          *reinterpret_cast<uint2*>(orow + dt * 16 + grp * 4) = make_uint2(lo, hi);
        }
      }
    } else {
      // This piece's normalised partial, rounded to bf16 (the form in which
      // pieces are stored: it halves their traffic, and the merge adds no
      // more than the final bf16 rounding of the output), and its fp32
      // log-sum-exp. A piece may hold only keys that are causally hidden
      // from some of its rows (sum 0): such a row's partial is 0 with
      // log-sum-exp -inf, so the merge gives it weight 0.
      uint2 pw[NTW][S::kDTiles];
      float plse[NTW];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const bool seen = lt[nt] > 0.0f;
        const float inv = seen ? 1.0f / lt[nt] : 0.0f;
#pragma unroll
        for (int dt = 0; dt < S::kDTiles; ++dt)
          pw[nt][dt] = make_uint2(pack_bf16x2(acc_o[nt][dt][0] * inv, acc_o[nt][dt][1] * inv),
                                  pack_bf16x2(acc_o[nt][dt][2] * inv, acc_o[nt][dt][3] * inv));
        plse[nt] = seen ? m[nt] + __log2f(lt[nt]) : -INFINITY;
      }
      const PieceSlots ps{first_owner, n_parts, first_owner * U / G < item_first};
      // On the workgroup's last segment: if every other piece of the item is
      // counted already (typically the item's later pieces, which were the
      // first segments of later workgroups), no other workgroup can complete
      // the item, and this one merges it at once with its own piece taken
      // from registers, never storing it. Otherwise the piece is stored and
      // counted when the workgroup ends.
      bool merged = false;
      if (seg_end == u_end) {
        if (tid == 0) {
          const uint64_t v = __hip_atomic_load(piece_counter(a, seq, h, qt, group, Hkv, ROWS), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
          s_cnt[0] = (v >> 16) == (a.epoch_tag >> 16) && static_cast<int>(v & 0xFFFFu) == n_parts - 1;
        }
        __syncthreads();
        merged = s_cnt[0] != 0;
      }
      if (merged) {  // merged after the segment loop, which ends here
        merge_last = true;
        last_ps = ps;
        last_seq = seq;
        last_h = h;
        last_qt = qt;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
          for (int dt = 0; dt < S::kDTiles; ++dt) {
            s_last[((nt * S::kDTiles + dt) * 2) * kWave] = pw[nt][dt].x;
            s_last[((nt * S::kDTiles + dt) * 2 + 1) * kWave] = pw[nt][dt].y;
          }
          s_last[(NTW * S::kDTiles * 2 + nt) * kWave] = __float_as_uint(plse[nt]);
        }
        break;
      } else {
        // Slot of this piece: a workgroup's first segment with tiles uses
        // slot 2w, its last (when it has more than one) uses slot 2w + 1.
        const int which = first_seg ? 0 : 1;
        const int64_t slot = 2 * static_cast<int64_t>(w) + which;
        const __amdgpu_buffer_rsrc_t pr = buffer_rsrc(a.part_out + slot * ROWS * D, ROWS * D * 2);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          const int row = wave * RPW + nt * 16 + col;
#pragma unroll
          for (int c = 0; c < S::kDTiles / 2; ++c) {
            const uint4 u = make_uint4(pw[nt][2 * c].x, pw[nt][2 * c].y, pw[nt][2 * c + 1].x, pw[nt][2 * c + 1].y);
            store4_agent(pr, piece_chunk_offset<S::kDTiles, NTW>(wave, nt, c, lane), __builtin_bit_cast(f32x4_t, u));
          }
          if (grp == 0) store_agent(a.part_lse + slot * ROWS + row, plse[nt]);
        }
        // Only a range's first and last segment can be pieces. A first
        // segment that is not the last is the end of an item that an earlier
        // workgroup started and finishes late: its piece is counted now
        // (after every thread's stores are complete), so that the owner of
        // the item's first piece can find the item complete when it gets
        // there. The count's result is only looked at when this workgroup
        // ends. Other pieces are counted when the workgroup ends.
        const int k = pend_n[0] == 0 ? 0 : 1;
        pend_n[k] = n_parts;
        pend_first[k] = first_owner;
        pend_item_first[k] = item_first;
        pend_seq[k] = seq;
        pend_h[k] = h;
        pend_qt[k] = qt;
        if (k == 0 && seg_end < u_end) {
          wait_vector_memory();
          __syncthreads();
          if (tid == 0) {
            const int cnt = count_arrival(piece_counter(a, seq, h, qt, group, Hkv, ROWS), a.epoch_tag);
            first_state = cnt == n_parts ? 1 : (cnt < 0 || cnt > n_parts ? -1 : 0);
          }
          first_counted = true;
        }
      }
    }
    __syncthreads();
    first_seg = false;

    u = seg_end;
    if (u == item_end && u < u_end) {
      // next item: same sequence unless this was its last unit
      if (u - seq_base >= static_cast<int64_t>(Hkv) * uph) {
        seq_base = u;
        ++seq;
        while (seq < B - 1 && units_per_head<ROWS, KT>(seq_geom(a, seq), group) == 0) ++seq;
      }
    }
  }

  if (merge_last) {
    // (written by this wave before it left the loop: no barrier needed)
    uint2 last_o[NTW][S::kDTiles];
    float last_lse[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
      for (int dt = 0; dt < S::kDTiles; ++dt)
        last_o[nt][dt] = make_uint2(s_last[((nt * S::kDTiles + dt) * 2) * kWave],
                                    s_last[((nt * S::kDTiles + dt) * 2 + 1) * kWave]);
      last_lse[nt] = __uint_as_float(s_last[(NTW * S::kDTiles * 2 + nt) * kWave]);
    }
    merge_item_rows<D, ROWS, NTW, 2>(a, outp, last_ps, static_cast<int>(w - last_ps.first_owner), last_o, last_lse,
                                     seq_geom(a, last_seq), last_qt, last_h, group, wave, col, grp, false);
  }

  // ---- 4. Count the stored pieces once every thread's stores are complete;
  // the workgroup whose count completes an item merges its pieces.
  if (pend_n[0] > 0) {
    wait_vector_memory();
    __syncthreads();
    if (tid < 2) {  // threads 0 and 1 count the two pieces (tagged counters, see pa_launch.h)
      const int n = tid == 0 ? pend_n[0] : pend_n[1];
      int state = 0;  // 1: this arrival completes the item; -1: foreign counter
      if (tid == 0 && first_counted) {
        state = first_state;
        if (state < 0) flag_workspace(a.ws_flags, kWorkspaceErrStaleCounter);
      } else if (n > 0) {
        const int cnt = count_arrival(piece_counter(a, tid == 0 ? pend_seq[0] : pend_seq[1],
                                                    tid == 0 ? pend_h[0] : pend_h[1],
                                                    tid == 0 ? pend_qt[0] : pend_qt[1], group, Hkv, ROWS),
                                      a.epoch_tag);
        state = cnt == n ? 1 : (cnt < 0 || cnt > n ? -1 : 0);
        if (state < 0) flag_workspace(a.ws_flags, kWorkspaceErrStaleCounter);
      }
      s_cnt[tid] = state;
    }
    __syncthreads();
    const uint2 none_o[NTW][S::kDTiles] = {};
    const float none_lse[NTW] = {};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (pend_n[k] > 0 && s_cnt[k] != 0) {
        const PieceSlots ps{pend_first[k], pend_n[k], pend_first[k] * U / G < pend_item_first[k]};
        merge_item_rows<D, ROWS, NTW, 2>(a, outp, ps, -1, none_o, none_lse, seq_geom(a, pend_seq[k]), pend_qt[k],
                                         pend_h[k], group, wave, col, grp, s_cnt[k] < 0);
      }
    }
  }
}

template <int D, int WM, int KT, int NTW>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream) {
  paged_prefill_kernel<D, WM, KT, NTW><<<dim3(static_cast<uint32_t>(a.num_workgroups)), dim3(64 * WM), 0, stream>>>(
      a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int32_t head_dim, hipStream_t stream) {
  // 256-row items: 8 waves of 32 rows, one workgroup per CU; 128-row items:
  // 4 waves of 32 rows, two per CU; 32-row items (verify): 1 wave, four per
  // CU.
  if (a.rows_per_tile == 256) {
    return head_dim == 128 ? launch_typed<128, 8, 64, 2>(a, stream) : launch_typed<64, 8, 64, 2>(a, stream);
  }
  if (a.rows_per_tile == 128) {
    return head_dim == 128 ? launch_typed<128, 4, 64, 2>(a, stream) : launch_typed<64, 4, 64, 2>(a, stream);
  }
  return head_dim == 128 ? launch_typed<128, 1, 32, 2>(a, stream) : launch_typed<64, 1, 32, 2>(a, stream);
}

}  // namespace pa
