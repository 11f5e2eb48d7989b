// Randomised driver of the native block manager for sanitizer builds (host
// code only): admissions with shared prefixes, chunked prefill, decode steps
// with batched appends, preemption on exhaustion, releases, and invalid calls,
// checking after every step that reference counts equal the number of live
// tables holding each block and that free + held blocks cover the pool. Built
// and run by tests/test_block_manager_sanitize.py with AddressSanitizer and
// UndefinedBehaviorSanitizer; exits non-zero on the first violated check.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <map>
#include <random>
#include <vector>

#include "block_manager.h"

#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      exit(1);                                                \
    }                                                         \
  } while (0)

int main(int argc, char** argv) {
  const int seed = argc > 1 ? atoi(argv[1]) : 1;
  const int nb = 48, bs = 8, width = 48;
  std::mt19937 rng(seed);
  auto rnd = [&](int n) { return static_cast<int>(rng() % static_cast<uint32_t>(n)); };
  pa_block_manager* bm = nullptr;
  CHECK(pa_bm_create(nb, bs, &bm) == PA_OK && bm != nullptr);
  std::vector<std::vector<int32_t>> systems(3);
  for (auto& s : systems)
    for (int i = 0, n = bs + rnd(3 * bs); i < n; ++i) s.push_back(rnd(50));
  std::map<int64_t, std::vector<int32_t>> live;  // admitted sequences and their tokens
  int64_t next_id = 0;
  std::vector<int32_t> pos(4096), slot(4096), tables(64 * width), ctx(64), cu(65);
  for (int step = 0; step < 3000; ++step) {
    const int op = rnd(10);
    if (op < 3 || live.empty()) {  // admit a prompt
      std::vector<int32_t> p = rnd(10) < 7 ? systems[rnd(3)] : std::vector<int32_t>();
      for (int i = 0, n = 1 + rnd(3 * bs); i < n; ++i) p.push_back(rnd(50));
      int32_t ok = 0, cached = -1;
      CHECK(pa_bm_can_allocate(bm, p.data(), static_cast<int32_t>(p.size()), &ok) == PA_OK);
      const pa_status st = pa_bm_allocate(bm, next_id, p.data(), static_cast<int32_t>(p.size()), &cached);
      CHECK((st == PA_OK) == (ok == 1));
      if (st == PA_OK) {
        CHECK(cached >= 0 && cached % bs == 0 && cached < static_cast<int32_t>(p.size()));
        live[next_id] = p;
      }
      ++next_id;
    } else if (op < 6) {  // prefill or decode step over every live sequence
      std::vector<int64_t> pre, dec;
      for (auto& kv : live) {
        int32_t n = 0, c = 0, b = 0;
        CHECK(pa_bm_seq_info(bm, kv.first, &n, &c, &b) == PA_OK);
        (c < n ? pre : dec).push_back(kv.first);
      }
      if (!pre.empty() && pre.size() <= 64) {
        std::vector<int32_t> cap(pre.size(), 1 + rnd(2 * bs));
        int32_t tq = 0;
        CHECK(pa_bm_prepare_prefill(bm, pre.data(), static_cast<int32_t>(pre.size()), cap.data(), width, 4096,
                                    pos.data(), slot.data(), tables.data(), ctx.data(), cu.data(), &tq) == PA_OK);
        CHECK(tq == cu[pre.size()]);
        for (int32_t t = 0; t < tq; ++t) CHECK(slot[t] >= 0 && slot[t] < nb * bs);
      } else if (!dec.empty() && dec.size() <= 64) {
        std::vector<int32_t> toks(dec.size());
        for (auto& t : toks) t = rnd(50);
        pa_status st = pa_bm_append_tokens(bm, dec.data(), toks.data(), static_cast<int32_t>(dec.size()));
        while (st == PA_ERR_NO_BLOCKS && !dec.empty()) {  // preempt the newest and retry
          const int64_t victim = dec.back();
          CHECK(pa_bm_free(bm, victim) == PA_OK);
          live.erase(victim);
          dec.pop_back();
          toks.pop_back();
          st = dec.empty() ? PA_OK : pa_bm_append_tokens(bm, dec.data(), toks.data(), static_cast<int32_t>(dec.size()));
        }
        CHECK(st == PA_OK);
        for (size_t i = 0; i < dec.size(); ++i) live[dec[i]].push_back(toks[i]);
        if (!dec.empty())
          CHECK(pa_bm_prepare_decode(bm, dec.data(), static_cast<int32_t>(dec.size()), width, pos.data(), slot.data(),
                                     tables.data(), ctx.data()) == PA_OK);
      }
    } else if (op < 8) {  // release one
      auto it = live.begin();
      std::advance(it, rnd(static_cast<int>(live.size())));
      CHECK(pa_bm_free(bm, it->first) == PA_OK);
      live.erase(it);
    } else {  // invalid calls change nothing
      int32_t before = pa_bm_num_free_blocks(bm);
      CHECK(pa_bm_free(bm, -12345) == PA_ERR_INVALID_ARG);
      CHECK(pa_bm_append_token(bm, -12345, 1) == PA_ERR_INVALID_ARG);
      int64_t dup[2] = {live.begin()->first, live.begin()->first};
      CHECK(pa_bm_prepare_decode(bm, dup, 2, width, pos.data(), slot.data(), tables.data(), ctx.data()) ==
            PA_ERR_INVALID_ARG);
      CHECK(pa_bm_num_free_blocks(bm) == before);
    }
    // invariants: reference counts equal holders; free + held cover the pool
    std::vector<int> holders(nb, 0);
    for (auto& kv : live) {
      int32_t n = 0, c = 0, b = 0;
      CHECK(pa_bm_seq_info(bm, kv.first, &n, &c, &b) == PA_OK);
      CHECK(n == static_cast<int32_t>(kv.second.size()) && b == (n + bs - 1) / bs && c <= n);
      std::vector<int32_t> row(b > 0 ? b : 1);
      CHECK(pa_bm_block_table(bm, kv.first, row.data(), b) == PA_OK);
      for (int j = 0; j < b; ++j) {
        CHECK(row[j] >= 0 && row[j] < nb);
        ++holders[row[j]];
      }
    }
    int free_blocks = 0;
    for (int blk = 0; blk < nb; ++blk) {
      CHECK(pa_bm_ref_count(bm, blk) == holders[blk]);
      free_blocks += holders[blk] == 0;
    }
    CHECK(pa_bm_num_free_blocks(bm) == free_blocks);
  }
  pa_bm_destroy(bm);
  printf("ok seed %d\n", seed);
  return 0;
}
