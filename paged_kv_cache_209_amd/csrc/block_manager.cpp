// Host-side block manager of the paged KV cache ("Nano-vLLM System
// Architecture Analysis", section 2 "Paged KV Cache" and "Scheduler", section 3
// "Lifecycle of a Request"): a first-in first-out free list, reference counts,
// a content-hash table for prefix sharing, and the per-step metadata
// (positions, slot mappings, block tables, context lengths, cumulative query
// lengths) that the attention kernels read. The rules are stated in
// include/block_manager.h.
//
// Data structures: the free list is an intrusive doubly linked list over block
// ids (prev/next arrays), so taking back a released block that a prefix hit
// names is O(1); each block keeps its content hash and, while it is
// registered, its token ids (to tell a hash collision from a hit); sequences
// live in a hash map keyed by the caller's id.
#include <stdint.h>
#include <string.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "block_manager.h"

namespace {

// ---------------------------------------------------------------------------
// XXH64, written from the published xxHash specification (64-bit variant).
// ---------------------------------------------------------------------------
constexpr uint64_t kP1 = 0x9E3779B185EBCA87ULL;
constexpr uint64_t kP2 = 0xC2B2AE3D27D4EB4FULL;
constexpr uint64_t kP3 = 0x165667B19E3779F9ULL;
constexpr uint64_t kP4 = 0x85EBCA77C2B2AE63ULL;
constexpr uint64_t kP5 = 0x27D4EB2F165667C5ULL;

inline uint64_t rotl(uint64_t x, int r) { return (x << r) | (x >> (64 - r)); }

inline uint64_t load64(const uint8_t* p) {
  uint64_t v;
  memcpy(&v, p, 8);  // x86-64 and the GPU hosts are little-endian, as the spec reads
  return v;
}

inline uint32_t load32(const uint8_t* p) {
  uint32_t v;
  memcpy(&v, p, 4);
  return v;
}

inline uint64_t xxh_round(uint64_t acc, uint64_t lane) {
  acc += lane * kP2;
  acc = rotl(acc, 31);
  return acc * kP1;
}

inline uint64_t xxh_merge(uint64_t acc, uint64_t v) {
  acc ^= xxh_round(0, v);
  return acc * kP1 + kP4;
}

uint64_t xxh64(const void* data, size_t len, uint64_t seed) {
  const uint8_t* p = static_cast<const uint8_t*>(data);
  const uint8_t* const end = p + len;
  uint64_t acc;
  if (len >= 32) {
    uint64_t v1 = seed + kP1 + kP2, v2 = seed + kP2, v3 = seed, v4 = seed - kP1;
    const uint8_t* const limit = end - 32;
    do {
      v1 = xxh_round(v1, load64(p));
      v2 = xxh_round(v2, load64(p + 8));
      v3 = xxh_round(v3, load64(p + 16));
      v4 = xxh_round(v4, load64(p + 24));
      p += 32;
    } while (p <= limit);
    acc = rotl(v1, 1) + rotl(v2, 7) + rotl(v3, 12) + rotl(v4, 18);
    acc = xxh_merge(acc, v1);
    acc = xxh_merge(acc, v2);
    acc = xxh_merge(acc, v3);
    acc = xxh_merge(acc, v4);
  } else {
    acc = seed + kP5;
  }
  acc += static_cast<uint64_t>(len);
  while (end - p >= 8) {
    acc ^= xxh_round(0, load64(p));
    acc = rotl(acc, 27) * kP1 + kP4;
    p += 8;
  }
  if (end - p >= 4) {
    acc ^= static_cast<uint64_t>(load32(p)) * kP1;
    acc = rotl(acc, 23) * kP2 + kP3;
    p += 4;
  }
  while (p < end) {
    acc ^= static_cast<uint64_t>(*p) * kP5;
    acc = rotl(acc, 11) * kP1;
    ++p;
  }
  acc ^= acc >> 33;
  acc *= kP2;
  acc ^= acc >> 29;
  acc *= kP3;
  acc ^= acc >> 32;
  return acc;
}

}  // namespace

struct pa_block_manager {
  struct Block {
    int32_t ref = 0;
    bool registered = false;  // holds the hash-table entry of `hash`
    uint64_t hash = 0;
    std::vector<int32_t> tokens;  // the block's token ids while registered
  };
  struct Seq {
    std::vector<int32_t> tokens;
    std::vector<int32_t> blocks;
    std::vector<uint64_t> hashes;  // chain hashes of full blocks 0 .. hashes.size()-1
    int32_t computed = 0;          // tokens emitted by prepare calls
    uint64_t mark = 0;             // the last batch call that named this sequence
  };

  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<Block> blocks;
  // free list: intrusive, -1 terminated; in_free marks membership
  std::vector<int32_t> prev, next;
  std::vector<uint8_t> in_free;
  int32_t head = -1, tail = -1, free_count = 0;
  std::unordered_map<uint64_t, int32_t> table;  // content hash -> block id
  std::unordered_map<int64_t, Seq> seqs;
  uint64_t batch = 0;  // numbers batch calls, to find a sequence named twice in one call

  // Looks up the sequences of a batch call; nullptr entries or a repeat fail.
  bool gather(const int64_t* ids, int32_t n, std::vector<Seq*>* out) {
    ++batch;
    out->resize(n);
    for (int32_t i = 0; i < n; ++i) {
      auto it = seqs.find(ids[i]);
      if (it == seqs.end() || it->second.mark == batch) return false;
      it->second.mark = batch;
      (*out)[i] = &it->second;
    }
    return true;
  }

  void push_tail(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    in_free[b] = 1;
    ++free_count;
  }

  void unlink(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    prev[b] = next[b] = -1;
    in_free[b] = 0;
    --free_count;
  }

  // Takes the head of the free list for new content: its old entry leaves the table.
  int32_t take_fresh() {
    const int32_t b = head;
    unlink(b);
    Block& blk = blocks[b];
    if (blk.registered) {
      auto it = table.find(blk.hash);
      if (it != table.end() && it->second == b) table.erase(it);
      blk.registered = false;
      blk.tokens.clear();
      blk.tokens.shrink_to_fit();
    }
    blk.ref = 1;
    return b;
  }

  // Hash of full block `b` of `tokens`, chained on `seed`.
  uint64_t block_hash(const int32_t* tokens, int32_t b, uint64_t seed) const {
    return xxh64(tokens + static_cast<int64_t>(b) * block_size, sizeof(int32_t) * block_size, seed);
  }

  // The registered block holding full block `b` of `tokens` under hash h, or -1.
  int32_t lookup(const int32_t* tokens, int32_t b, uint64_t h) const {
    auto it = table.find(h);
    if (it == table.end()) return -1;
    const Block& blk = blocks[it->second];
    if (memcmp(blk.tokens.data(), tokens + static_cast<int64_t>(b) * block_size, sizeof(int32_t) * block_size) != 0)
      return -1;  // a collision: same hash, other tokens
    return it->second;
  }

  // Prefix hits of a prompt: block ids and chain hashes of the leading full
  // blocks found in the table (never all of a prompt's tokens).
  void find_hits(const int32_t* tokens, int32_t n, std::vector<int32_t>* ids, std::vector<uint64_t>* hashes) const {
    int32_t full = n / block_size;
    if (full * block_size == n) --full;  // leave the last block to compute
    uint64_t h = 0;
    for (int32_t b = 0; b < full; ++b) {
      h = block_hash(tokens, b, h);
      const int32_t id = lookup(tokens, b, h);
      if (id < 0) break;
      ids->push_back(id);
      hashes->push_back(h);
    }
  }

  // Free-list blocks an allocation of this prompt consumes.
  int64_t blocks_needed(const int32_t* tokens, int32_t n, std::vector<int32_t>* ids,
                        std::vector<uint64_t>* hashes) const {
    find_hits(tokens, n, ids, hashes);
    int64_t hits_in_use = 0;
    for (int32_t id : *ids) hits_in_use += blocks[id].ref > 0 ? 1 : 0;
    const int64_t total = (static_cast<int64_t>(n) + block_size - 1) / block_size;
    return total - hits_in_use;
  }

  // Registers full block b of s (its last row was just emitted).
  void register_block(Seq& s, int32_t b) {
    const uint64_t seed = b == 0 ? 0 : s.hashes[b - 1];
    const uint64_t h = block_hash(s.tokens.data(), b, seed);
    s.hashes.push_back(h);
    Block& blk = blocks[s.blocks[b]];
    if (blk.registered || table.count(h)) return;  // the first block under a hash keeps the entry
    table.emplace(h, s.blocks[b]);
    blk.registered = true;
    blk.hash = h;
    blk.tokens.assign(s.tokens.begin() + static_cast<int64_t>(b) * block_size,
                      s.tokens.begin() + static_cast<int64_t>(b + 1) * block_size);
  }

  // Marks tokens [s.computed, upto) as emitted, registering blocks they complete.
  void advance(Seq& s, int32_t upto) {
    for (int32_t b = s.computed / block_size; (b + 1) * block_size <= upto; ++b)
      if (static_cast<int32_t>(s.hashes.size()) == b) register_block(s, b);
    s.computed = upto;
  }

  void write_table(const Seq& s, int32_t* row, int32_t width) const {
    const int32_t nb = static_cast<int32_t>(s.blocks.size());
    for (int32_t j = 0; j < width; ++j) row[j] = j < nb ? s.blocks[j] : -1;
  }

  int32_t slot(const Seq& s, int32_t pos) const { return s.blocks[pos / block_size] * block_size + pos % block_size; }
};

namespace {

bool valid(const pa_block_manager* bm) { return bm != nullptr && bm->num_blocks > 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

extern "C" {

uint64_t pa_xxh64(const void* data, size_t len, uint64_t seed) {
  if (data == nullptr && len != 0) return 0;
  return xxh64(data, len, seed);
}

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, pa_block_manager** out) {
  if (out == nullptr) return PA_ERR_INVALID_ARG;
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0) return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(num_blocks) * block_size >= (int64_t{1} << 31)) return PA_ERR_INVALID_ARG;
  pa_block_manager* bm = new (std::nothrow) pa_block_manager();
  if (bm == nullptr) return PA_ERR_INVALID_ARG;
  try {
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->blocks.resize(num_blocks);
    bm->prev.assign(num_blocks, -1);
    bm->next.assign(num_blocks, -1);
    bm->in_free.assign(num_blocks, 0);
    for (int32_t b = 0; b < num_blocks; ++b) bm->push_tail(b);
  } catch (...) {
    delete bm;
    return PA_ERR_INVALID_ARG;
  }
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int32_t pa_bm_num_free_blocks(const pa_block_manager* bm) { return valid(bm) ? bm->free_count : -1; }

int32_t pa_bm_ref_count(const pa_block_manager* bm, int32_t block_id) {
  if (!valid(bm) || block_id < 0 || block_id >= bm->num_blocks) return -1;
  return bm->blocks[block_id].ref;
}

pa_status pa_bm_can_allocate(const pa_block_manager* bm, const int32_t* token_ids, int32_t num_tokens, int32_t* ok) {
  if (!valid(bm) || token_ids == nullptr || num_tokens <= 0 || ok == nullptr) return PA_ERR_INVALID_ARG;
  std::vector<int32_t> ids;
  std::vector<uint64_t> hashes;
  *ok = bm->blocks_needed(token_ids, num_tokens, &ids, &hashes) <= bm->free_count ? 1 : 0;
  return PA_OK;
}

pa_status pa_bm_allocate(pa_block_manager* bm, int64_t seq_id, const int32_t* token_ids, int32_t num_tokens,
                         int32_t* num_cached_tokens) {
  if (!valid(bm) || token_ids == nullptr || num_tokens <= 0) return PA_ERR_INVALID_ARG;
  if (bm->seqs.count(seq_id)) return PA_ERR_INVALID_ARG;
  std::vector<int32_t> ids;
  std::vector<uint64_t> hashes;
  if (bm->blocks_needed(token_ids, num_tokens, &ids, &hashes) > bm->free_count) return PA_ERR_NO_BLOCKS;
  pa_block_manager::Seq s;
  s.tokens.assign(token_ids, token_ids + num_tokens);
  const int32_t total = static_cast<int32_t>(ceil_div(num_tokens, bm->block_size));
  s.blocks.reserve(total);
  // hits first: a released block named by a hit must not be taken as a fresh one
  for (int32_t id : ids) {
    if (bm->blocks[id].ref == 0) bm->unlink(id);
    ++bm->blocks[id].ref;
    s.blocks.push_back(id);
  }
  while (static_cast<int32_t>(s.blocks.size()) < total) s.blocks.push_back(bm->take_fresh());
  s.hashes = hashes;
  s.computed = static_cast<int32_t>(ids.size()) * bm->block_size;
  if (num_cached_tokens) *num_cached_tokens = s.computed;
  bm->seqs.emplace(seq_id, std::move(s));
  return PA_OK;
}

pa_status pa_bm_append_token(pa_block_manager* bm, int64_t seq_id, int32_t token_id) {
  if (!valid(bm)) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
  pa_block_manager::Seq& s = it->second;
  const int32_t n = static_cast<int32_t>(s.tokens.size());
  if (s.computed != n) return PA_ERR_INVALID_ARG;  // the previous tokens were not all emitted
  if (static_cast<int64_t>(n) + 1 >= (int64_t{1} << 31)) return PA_ERR_INVALID_ARG;
  if (n % bm->block_size == 0) {
    if (bm->free_count == 0) return PA_ERR_NO_BLOCKS;
    s.blocks.push_back(bm->take_fresh());
  }
  s.tokens.push_back(token_id);
  return PA_OK;
}

pa_status pa_bm_append_tokens(pa_block_manager* bm, const int64_t* seq_ids, const int32_t* token_ids,
                              int32_t num_seqs) {
  if (!valid(bm) || num_seqs < 0) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (seq_ids == nullptr || token_ids == nullptr) return PA_ERR_INVALID_ARG;
  std::vector<pa_block_manager::Seq*> seqs;
  if (!bm->gather(seq_ids, num_seqs, &seqs)) return PA_ERR_INVALID_ARG;
  int64_t opening = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const pa_block_manager::Seq& s = *seqs[i];
    const int32_t n = static_cast<int32_t>(s.tokens.size());
    if (s.computed != n || static_cast<int64_t>(n) + 1 >= (int64_t{1} << 31)) return PA_ERR_INVALID_ARG;
    opening += n % bm->block_size == 0 ? 1 : 0;
  }
  if (opening > bm->free_count) return PA_ERR_NO_BLOCKS;
  for (int32_t i = 0; i < num_seqs; ++i) {
    pa_block_manager::Seq& s = *seqs[i];
    if (s.tokens.size() % bm->block_size == 0) s.blocks.push_back(bm->take_fresh());
    s.tokens.push_back(token_ids[i]);
  }
  return PA_OK;
}

pa_status pa_bm_free(pa_block_manager* bm, int64_t seq_id) {
  if (!valid(bm)) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
  const std::vector<int32_t>& blocks = it->second.blocks;
  for (auto b = blocks.rbegin(); b != blocks.rend(); ++b)
    if (--bm->blocks[*b].ref == 0) bm->push_tail(*b);
  bm->seqs.erase(it);
  return PA_OK;
}

pa_status pa_bm_seq_info(const pa_block_manager* bm, int64_t seq_id, int32_t* num_tokens, int32_t* num_computed,
                         int32_t* num_blocks) {
  if (!valid(bm)) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
  if (num_tokens) *num_tokens = static_cast<int32_t>(it->second.tokens.size());
  if (num_computed) *num_computed = it->second.computed;
  if (num_blocks) *num_blocks = static_cast<int32_t>(it->second.blocks.size());
  return PA_OK;
}

pa_status pa_bm_block_table(const pa_block_manager* bm, int64_t seq_id, int32_t* out, int32_t capacity) {
  if (!valid(bm) || out == nullptr) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
  const std::vector<int32_t>& blocks = it->second.blocks;
  if (capacity < static_cast<int32_t>(blocks.size())) return PA_ERR_INVALID_ARG;
  for (size_t j = 0; j < blocks.size(); ++j) out[j] = blocks[j];
  return PA_OK;
}

pa_status pa_bm_prepare_prefill(pa_block_manager* bm, const int64_t* seq_ids, int32_t num_seqs,
                                const int32_t* max_new_tokens, int32_t max_blocks_per_seq, int32_t max_total_q,
                                int32_t* positions, int32_t* slot_mapping, int32_t* block_tables,
                                int32_t* context_lens, int32_t* cu_seqlens, int32_t* total_q) {
  if (!valid(bm) || num_seqs < 0 || max_blocks_per_seq <= 0 || max_total_q < 0) return PA_ERR_INVALID_ARG;
  if (num_seqs > 0 && (seq_ids == nullptr || block_tables == nullptr || context_lens == nullptr))
    return PA_ERR_INVALID_ARG;
  if (cu_seqlens == nullptr || total_q == nullptr) return PA_ERR_INVALID_ARG;
  // validation pass: nothing changes unless every sequence is fine
  std::vector<pa_block_manager::Seq*> seqs;
  if (!bm->gather(seq_ids, num_seqs, &seqs)) return PA_ERR_INVALID_ARG;  // unknown, or twice in one step
  std::vector<int32_t> counts(num_seqs);
  int64_t tq = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const pa_block_manager::Seq& s = *seqs[i];
    int32_t n = static_cast<int32_t>(s.tokens.size()) - s.computed;
    if (max_new_tokens && max_new_tokens[i] < n) n = max_new_tokens[i];
    if (n <= 0) return PA_ERR_INVALID_ARG;
    if (static_cast<int32_t>(s.blocks.size()) > max_blocks_per_seq) return PA_ERR_INVALID_ARG;
    counts[i] = n;
    tq += n;
  }
  if (tq > max_total_q) return PA_ERR_INVALID_ARG;
  if (tq > 0 && (positions == nullptr || slot_mapping == nullptr)) return PA_ERR_INVALID_ARG;
  int32_t off = 0;
  cu_seqlens[0] = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    pa_block_manager::Seq& s = *seqs[i];
    const int32_t c = s.computed, n = counts[i];
    for (int32_t j = 0; j < n; ++j) {
      positions[off + j] = c + j;
      slot_mapping[off + j] = bm->slot(s, c + j);
    }
    bm->write_table(s, block_tables + static_cast<int64_t>(i) * max_blocks_per_seq, max_blocks_per_seq);
    context_lens[i] = c + n;
    off += n;
    cu_seqlens[i + 1] = off;
    bm->advance(s, c + n);
  }
  *total_q = off;
  return PA_OK;
}

pa_status pa_bm_prepare_decode(pa_block_manager* bm, const int64_t* seq_ids, int32_t num_seqs,
                               int32_t max_blocks_per_seq, int32_t* positions, int32_t* slot_mapping,
                               int32_t* block_tables, int32_t* context_lens) {
  if (!valid(bm) || num_seqs < 0 || max_blocks_per_seq <= 0) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (seq_ids == nullptr || positions == nullptr || slot_mapping == nullptr || block_tables == nullptr ||
      context_lens == nullptr)
    return PA_ERR_INVALID_ARG;
  std::vector<pa_block_manager::Seq*> seqs;
  if (!bm->gather(seq_ids, num_seqs, &seqs)) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const pa_block_manager::Seq& s = *seqs[i];
    if (s.computed != static_cast<int32_t>(s.tokens.size()) - 1) return PA_ERR_INVALID_ARG;
    if (static_cast<int32_t>(s.blocks.size()) > max_blocks_per_seq) return PA_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    pa_block_manager::Seq& s = *seqs[i];
    const int32_t pos = s.computed;
    positions[i] = pos;
    slot_mapping[i] = bm->slot(s, pos);
    context_lens[i] = pos + 1;
    bm->write_table(s, block_tables + static_cast<int64_t>(i) * max_blocks_per_seq, max_blocks_per_seq);
    bm->advance(s, pos + 1);
  }
  return PA_OK;
}

}  // extern "C"
