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
// units are the 64-key tiles its rows can see (causal: up to the tile's last
// token). As in decode, the units of all items are cut into equal contiguous
// shares, one per workgroup; a piece of an item is finished by the last
// workgroup to reach it, which merges the pieces' partial results in order.
//
// Per 64-key tile, each wave (32 query rows = two 16-column MFMA tiles):
//   S^T = K Q^T   with v_mfma_f32_16x16x32_bf16: A = K rows from LDS
//                 (16 keys x 32 dims per lane group), B = the wave's query
//                 fragments held in registers. Each lane ends with 4 keys of
//                 one query column, so the softmax max is an in-lane max plus
//                 two cross-group shuffles.
//   P = 2^(S*scale*log2e - m), rounded to bf16 in registers: the S^T result
//                 layout already is the B-operand layout of the next product
//                 once the 32 keys of a step are taken in the order
//                 {4q..4q+3, 16+4q..16+4q+3} for lane group q.
//   O^T += V^T P^T: A = V^T fragments read with ds_read_b64_tr_b16 from the
//                 row-major V tile (the LDS transpose read hands each lane 4
//                 consecutive keys of one head dim), B = P^T.
// K/V tiles are staged in LDS by direct-to-LDS loads (no register round
// trip), in a swizzled layout, double-buffered so the next tile streams in
// while the current one is used; all waves of the workgroup share them. Rows
// beyond the context re-read a valid row and get weight 0.
#include <math.h>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kKeysPerTile = 64;
constexpr int kRowsPerWave = 32;
constexpr float kEmptyMaxP = -1.0e30f;
constexpr float kSlack = 8.0f;

typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

template <int D>
struct PShape {
  static constexpr int kDChunks = D / 32;  // k-steps of the Q.K product
  static constexpr int kDTiles = D / 16;   // 16-row tiles of O^T
  static constexpr int kRowBytes = D * 2;  // one key's head row in LDS (no padding)
  static constexpr int kPieces = D * 2 / 16;  // 16-byte pieces per row
  static constexpr int kTileBytes = kKeysPerTile * kRowBytes;
};

// LDS byte offset of 16-byte piece c of row r in a swizzled tile: piece c is
// stored at slot c ^ (r mod pieces), so the 16 rows an MFMA operand read
// touches fall on 16 different bank groups, with no padding bytes (which
// direct-to-LDS loads could not skip).
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  constexpr int P = PShape<D>::kPieces;
  return r * PShape<D>::kRowBytes + ((c ^ (r & (P - 1))) << 4);
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

// 64-key tiles visible to query tile qt (rows qt*ROWS .. qt*ROWS+ROWS-1).
template <int ROWS>
__device__ __forceinline__ int tiles_of(const SeqGeom& s, int group, int qt) {
  const int jmax = min(s.n - 1, ((qt + 1) * ROWS - 1) / group);
  return (s.c + jmax + 1 + kKeysPerTile - 1) / kKeysPerTile;
}

template <int ROWS>
__device__ __forceinline__ int qtiles_of(const SeqGeom& s, int group) {
  return (s.n * group + ROWS - 1) / ROWS;
}

template <int ROWS>
__device__ int units_per_head(const SeqGeom& s, int group) {
  if (s.n <= 0) return 0;
  const int qts = qtiles_of<ROWS>(s, group);
  int u = 0;
  for (int qt = 0; qt < qts; ++qt) u += tiles_of<ROWS>(s, group, qt);
  return u;
}

__device__ __forceinline__ int owner_of_unit(int64_t u, int64_t U, int64_t G) {
  return static_cast<int>(((u + 1) * G - 1) / U);
}

template <int D, int WM>
__global__ __launch_bounds__(64 * WM) void paged_prefill_kernel(PrefillArgs a) {
  using S = PShape<D>;
  constexpr int ROWS = kRowsPerWave * WM;
  constexpr int NT = kWave * WM;
  constexpr int TB = S::kTileBytes;
  constexpr int kLoadsPerTile = 2 * kKeysPerTile * S::kPieces / NT;  // per thread, K and V
  // Two stages of [K tile | V tile]: tile t+1 streams in while t is used.
  __shared__ __attribute__((aligned(16))) char s_kv[2][2 * TB];
  __shared__ int s_scan[NT];
  __shared__ int s_loc[2];
  __shared__ int s_last;

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

  // ---- 1. Units per sequence (all KV heads), block-wide scan.
  const int per = (B + NT - 1) / NT;
  int mine = 0;
  for (int k = 0; k < per; ++k) {
    const int i = tid * per + k;
    if (i < B) mine += Hkv * units_per_head<ROWS>(seq_geom(a, i), group);
  }
  s_scan[tid] = mine;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {
    const int v = tid >= off ? s_scan[tid - off] : 0;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  const int64_t U = __builtin_amdgcn_readfirstlane(s_scan[NT - 1]);
  if (U == 0) return;
  const int64_t G = min(static_cast<int64_t>(gridDim.x), U);
  const int w = blockIdx.x;
  if (w >= G) return;
  const int64_t u_begin = static_cast<int64_t>(w) * U / G;
  const int64_t u_end = static_cast<int64_t>(w + 1) * U / G;

  // ---- 2. Sequence holding u_begin.
  {
    const int64_t lo = s_scan[tid] - mine;
    if (u_begin >= lo && u_begin < s_scan[tid]) {
      int64_t base = lo;
      for (int k = 0; k < per && tid * per + k < B; ++k) {
        const int i = tid * per + k;
        const int64_t span = static_cast<int64_t>(Hkv) * units_per_head<ROWS>(seq_geom(a, i), group);
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

  const bf16_t* qg = static_cast<const bf16_t*>(a.q);
  const bf16_t* kg = static_cast<const bf16_t*>(a.k);
  const bf16_t* vg = static_cast<const bf16_t*>(a.v);
  const bf16_t* kpool = static_cast<const bf16_t*>(a.k_cache);
  const bf16_t* vpool = static_cast<const bf16_t*>(a.v_cache);
  bf16_t* outp = static_cast<bf16_t*>(a.out);
  const int64_t tok_stride = static_cast<int64_t>(Hkv) * D;  // elements between token rows (k, v, pools)
  const float sc = a.scale_log2;

  // ---- 3. Segments.
  int64_t u = u_begin;
  while (u < u_end) {
    const SeqGeom sg = seq_geom(a, seq);
    const int uph = units_per_head<ROWS>(sg, group);
    const int64_t r = u - seq_base;
    const int h = static_cast<int>(r / uph);
    int r2 = static_cast<int>(r % uph);
    int qt = 0;
    int acc_units = 0;
    int nkt = tiles_of<ROWS>(sg, group, 0);
    while (r2 >= acc_units + nkt) {
      acc_units += nkt;
      ++qt;
      nkt = tiles_of<ROWS>(sg, group, qt);
    }
    const int t_lo = r2 - acc_units;
    const int64_t item_first = seq_base + static_cast<int64_t>(h) * uph + acc_units;
    const int64_t item_end = item_first + nkt;
    const int64_t seg_end = u_end < item_end ? u_end : item_end;
    const int t_hi = t_lo + static_cast<int>(seg_end - u);
    const int total_keys = sg.c + sg.n;

    // This wave's query columns: nt in {0,1}, column col.
    int qrow_tok[2];   // token index j of the lane's query column (may be >= n: padding)
    int qrow_head[2];  // query head
    bf16x8_t qf[2][S::kDChunks];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int R = qt * ROWS + wave * kRowsPerWave + nt * 16 + col;
      const int j = R / group;
      const int g = R % group;
      qrow_tok[nt] = j;
      qrow_head[nt] = h * group + g;
      const int jj = min(j, sg.n - 1);
      const bf16_t* qrow = qg + (static_cast<int64_t>(sg.start + jj) * a.num_q_heads + h * group + g) * D;
#pragma unroll
      for (int kc = 0; kc < S::kDChunks; ++kc) {
        qf[nt][kc] = *reinterpret_cast<const bf16x8_t*>(qrow + kc * 32 + grp * 8);
      }
    }
    // Keys a query column may see: positions <= c + j, clamped to the last key.
    int vis[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) vis[nt] = min(sg.c + qrow_tok[nt], total_keys - 1);
    // Smallest visible-key bound over the wave's real rows (its first row):
    // a tile entirely below it needs no mask.
    const int wave_min_vis = min(sg.c + (qt * ROWS + wave * kRowsPerWave) / group, total_keys - 1);

    f32x4_t acc_o[2][S::kDTiles];
    float m[2], l[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      m[nt] = kEmptyMaxP;
      l[nt] = 0.0f;
#pragma unroll
      for (int dt = 0; dt < S::kDTiles; ++dt) acc_o[nt][dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }

    const int32_t* table = a.block_tables + static_cast<int64_t>(seq) * a.max_blocks_per_seq;
    // Issue the direct-to-LDS loads of key tile kt into stage `stage`. Each
    // wave instruction fills 1 KB of LDS in lane order; lane slot (row, slot)
    // fetches global piece slot ^ (row mod pieces) of that row, which is
    // exactly the swizzled layout. Rows past the last key re-read it.
    auto issue_tile = [&](int kt, int stage) {
      const int k0 = kt * kKeysPerTile;
      const int block = k0 < sg.c ? table[k0 / kTokensPerBlock] : 0;
      char* kdst = s_kv[stage];
      char* vdst = s_kv[stage] + TB;
#pragma unroll
      for (int it = 0; it < kKeysPerTile * S::kPieces / NT; ++it) {
        const int idx = it * NT + tid;
        const int kr = idx / S::kPieces;
        const int slot = idx % S::kPieces;
        const int pc = slot ^ (kr & (S::kPieces - 1));
        const int pos = min(k0 + kr, total_keys - 1);
        const bool cached = pos < sg.c;
        const int64_t row = cached ? static_cast<int64_t>(block) * kTokensPerBlock + pos % kTokensPerBlock
                                   : static_cast<int64_t>(sg.start) + (pos - sg.c);
        const int64_t off = row * tok_stride + h * D + pc * 8;
        const bf16_t* ksrc = (cached ? kpool : kg) + off;
        const bf16_t* vsrc = (cached ? vpool : vg) + off;
        const int lds_off = (it * NT + wave * kWave) * 16;  // this wave instruction's 1 KB
        __builtin_amdgcn_global_load_lds(ksrc, (lds_void_t*)(kdst + lds_off), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vsrc, (lds_void_t*)(vdst + lds_off), 16, 0, 0);
      }
    };

    if (t_lo < t_hi) issue_tile(t_lo, 0);
    for (int kt = t_lo; kt < t_hi; ++kt) {
      const int k0 = kt * kKeysPerTile;
      const int stage = (kt - t_lo) & 1;
      if (kt + 1 < t_hi) {
        issue_tile(kt + 1, stage ^ 1);
        wait_vmcnt<kLoadsPerTile>();  // this tile's loads are done, the next one's may fly
      } else {
        wait_vmcnt<0>();
      }
      __syncthreads();
      const char* s_k = s_kv[stage];
      const char* s_v = s_kv[stage] + TB;

      // -- S^T = K Q^T: st[mt][nt] holds keys 16mt + 4grp + e of query column col
      f32x4_t st[4][2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        st[mt][0] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        st[mt][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kc = 0; kc < S::kDChunks; ++kc) {
          const bf16x8_t kfrag = *reinterpret_cast<const bf16x8_t*>(s_k + swz<D>(mt * 16 + col, kc * 4 + grp));
          st[mt][0] = mfma16(kfrag, qf[0][kc], st[mt][0]);
          st[mt][1] = mfma16(kfrag, qf[1][kc], st[mt][1]);
        }
      }

      // -- online softmax per query column
      const bool full_tile = k0 + kKeysPerTile - 1 <= wave_min_vis;
      uint32_t pw[2][2][4];  // [nt][kc2][word]: P^T operand, bf16 pairs
      bool need = false;
      float mx[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float tmax = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float s = st[mt][nt][e] * sc;
            if (!full_tile) {
              const int kp = k0 + mt * 16 + grp * 4 + e;
              s = kp <= vis[nt] ? s : -INFINITY;
            }
            st[mt][nt][e] = s;
            tmax = fmaxf(tmax, s);
          }
        }
        tmax = fmaxf(tmax, shfl_xor_f32(tmax, 16));
        tmax = fmaxf(tmax, shfl_xor_f32(tmax, 32));
        mx[nt] = fmaxf(m[nt], tmax);
        need |= mx[nt] > m[nt] + kSlack;
      }
      if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const float alpha = exp2_fast(m[nt] - mx[nt]);
          l[nt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < S::kDTiles; ++dt) acc_o[nt][dt] *= alpha;
          m[nt] = mx[nt];
        }
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
        for (int kc2 = 0; kc2 < 2; ++kc2) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const f32x4_t& sv = st[2 * kc2 + half][nt];
            const uint32_t w0 = pack_bf16x2(exp2_fast(sv[0] - m[nt]), exp2_fast(sv[1] - m[nt]));
            const uint32_t w1 = pack_bf16x2(exp2_fast(sv[2] - m[nt]), exp2_fast(sv[3] - m[nt]));
            pw[nt][kc2][2 * half + 0] = w0;
            pw[nt][kc2][2 * half + 1] = w1;
            l[nt] += (bf16_lo(w0) + bf16_hi(w0)) + (bf16_lo(w1) + bf16_hi(w1));
          }
        }
      }

      // -- O^T += V^T P^T
#pragma unroll
      for (int kc2 = 0; kc2 < 2; ++kc2) {
        const bf16x8_t pb0 = __builtin_bit_cast(bf16x8_t, u32x4_t{pw[0][kc2][0], pw[0][kc2][1], pw[0][kc2][2], pw[0][kc2][3]});
        const bf16x8_t pb1 = __builtin_bit_cast(bf16x8_t, u32x4_t{pw[1][kc2][0], pw[1][kc2][1], pw[1][kc2][2], pw[1][kc2][3]});
        const int key_a = kc2 * 32 + grp * 4 + (col >> 2);
        const int key_b = key_a + 16;
        const int half = (col & 1) * 8;  // byte offset of the lane's 4 dims inside a 16-byte piece
#pragma unroll
        for (int dt = 0; dt < S::kDTiles; ++dt) {
          const int pc = dt * 2 + ((col & 3) >> 1);
          const i16x4_t ta =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(s_v + swz<D>(key_a, pc) + half));
          const i16x4_t tb =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(s_v + swz<D>(key_b, pc) + half));
          typedef short i16x8_t __attribute__((ext_vector_type(8)));
          const i16x8_t t8 = {ta[0], ta[1], ta[2], ta[3], tb[0], tb[1], tb[2], tb[3]};
          const bf16x8_t vfrag = __builtin_bit_cast(bf16x8_t, t8);
          acc_o[0][dt] = mfma16(vfrag, pb0, acc_o[0][dt]);
          acc_o[1][dt] = mfma16(vfrag, pb1, acc_o[1][dt]);
        }
      }
      __syncthreads();  // the next tile overwrites the LDS tiles
    }

    // ---- finish the segment: lane group sums of l, then output or partial
    float lt[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float x = l[nt];
      x += shfl_xor_f32(x, 16);
      x += shfl_xor_f32(x, 32);
      lt[nt] = x;
    }
    const int first_owner = owner_of_unit(item_first, U, G);
    const int n_parts = owner_of_unit(item_end - 1, U, G) - first_owner + 1;
    if (n_parts == 1) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
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
      // Partial slot of this piece: a workgroup's first segment uses slot
      // 2w, its last (when it has more than one) uses slot 2w + 1.
      // A piece may hold only keys that are causally hidden from some of its
      // rows (sum 0): such a row's partial is 0 with log-sum-exp -inf, so the
      // merge gives it weight 0.
      const int which = u > u_begin ? 1 : 0;
      const int64_t slot = 2 * static_cast<int64_t>(w) + which;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int row = wave * kRowsPerWave + nt * 16 + col;
        const bool seen = lt[nt] > 0.0f;
        const float inv = seen ? 1.0f / lt[nt] : 0.0f;
        float* po = a.part_out + (slot * ROWS + row) * D;
#pragma unroll
        for (int dt = 0; dt < S::kDTiles; ++dt) {
#pragma unroll
          for (int e = 0; e < 4; ++e) store_agent(po + dt * 16 + grp * 4 + e, acc_o[nt][dt][e] * inv);
        }
        if (grp == 0) store_agent(a.part_lse + slot * ROWS + row, seen ? m[nt] + __log2f(lt[nt]) : -INFINITY);
      }
      wait_vector_memory();
      __syncthreads();
      if (tid == 0) {
        const int64_t qtiles_max = (static_cast<int64_t>(a.max_q_len) * group + ROWS - 1) / ROWS;
        int* ctr = a.counters + (static_cast<int64_t>(seq) * Hkv + h) * qtiles_max + qt;
        const int prev = add_agent(ctr, 1);
        const int last = prev == n_parts - 1;
        if (last) store_agent_int(ctr, 0);
        s_last = last;
      }
      __syncthreads();
      if (s_last) {
        // Merge the pieces in order. Piece p is owned by workgroup
        // first_owner + p; it is that workgroup's first segment except for
        // the first piece when its owner started inside an earlier item.
        // Each thread owns 4 consecutive dims of kMergeRows rows at a time
        // and issues all of a piece's loads together.
        const int64_t first_start = static_cast<int64_t>(first_owner) * U / G;
        constexpr int D4 = D / 4;
        constexpr int kRowStep = NT / D4;
        constexpr int kMergeRows = 8;
        const int d4 = tid % D4;
        for (int rb = tid / D4; rb < ROWS; rb += kRowStep * kMergeRows) {
          float mxr[kMergeRows];
#pragma unroll
          for (int k = 0; k < kMergeRows; ++k) mxr[k] = -INFINITY;
          for (int p = 0; p < n_parts; ++p) {
            const int64_t sl = 2 * static_cast<int64_t>(first_owner + p) + ((p == 0 && first_start < item_first) ? 1 : 0);
#pragma unroll
            for (int k = 0; k < kMergeRows; ++k) {
              const int row = rb + k * kRowStep;
              if (row < ROWS) mxr[k] = fmaxf(mxr[k], load_agent(a.part_lse + sl * ROWS + row));
            }
          }
          f32x4_t num[kMergeRows];
          float den[kMergeRows];
#pragma unroll
          for (int k = 0; k < kMergeRows; ++k) {
            num[k] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            den[k] = 0.0f;
          }
          for (int p = 0; p < n_parts; ++p) {
            const int64_t sl = 2 * static_cast<int64_t>(first_owner + p) + ((p == 0 && first_start < item_first) ? 1 : 0);
#pragma unroll
            for (int k = 0; k < kMergeRows; ++k) {
              const int row = rb + k * kRowStep;
              if (row >= ROWS) continue;
              const float f = exp2_fast(load_agent(a.part_lse + sl * ROWS + row) - mxr[k]);
              const float* po = a.part_out + (sl * ROWS + row) * D + 4 * d4;
              const f32x4_t o4 = {load_agent(po), load_agent(po + 1), load_agent(po + 2), load_agent(po + 3)};
              num[k] += f * o4;
              den[k] += f;
            }
          }
#pragma unroll
          for (int k = 0; k < kMergeRows; ++k) {
            const int row = rb + k * kRowStep;
            if (row >= ROWS) continue;
            const int R = qt * ROWS + row;
            const int j = R / group;
            if (j >= sg.n) continue;
            const float inv = 1.0f / den[k];
            const uint32_t lo = pack_bf16x2(num[k][0] * inv, num[k][1] * inv);
            const uint32_t hi = pack_bf16x2(num[k][2] * inv, num[k][3] * inv);
            bf16_t* orow = outp + (static_cast<int64_t>(sg.start + j) * a.num_q_heads + h * group + R % group) * D;
            *reinterpret_cast<uint2*>(orow + 4 * d4) = make_uint2(lo, hi);
          }
        }
      }
    }
    __syncthreads();

    u = seg_end;
    if (u == item_end && u < u_end) {
      // next item: same sequence unless this was its last unit
      if (u - seq_base >= static_cast<int64_t>(Hkv) * uph) {
        seq_base = u;
        ++seq;
        while (seq < B - 1 && units_per_head<ROWS>(seq_geom(a, seq), group) == 0) ++seq;
      }
    }
  }
}

template <int D, int WM>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream) {
  paged_prefill_kernel<D, WM><<<dim3(static_cast<uint32_t>(a.num_workgroups)), dim3(64 * WM), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int32_t head_dim, hipStream_t stream) {
  if (a.rows_per_tile == 128) {
    return head_dim == 128 ? launch_typed<128, 4>(a, stream) : launch_typed<64, 4>(a, stream);
  }
  return head_dim == 128 ? launch_typed<128, 1>(a, stream) : launch_typed<64, 1>(a, stream);
}

}  // namespace pa
