// Host-only fuzz driver for the step scheduler (built with g++ and the
// address and undefined-behaviour sanitizers by tests/test_sched_sanitize.py).
// Random configurations, random submit/step interleavings; checks the step
// arrays' structure and that every accepted request finishes with its limit.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <memory>
#include <random>
#include <vector>

#include "mab.h"

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      return 1;                                                    \
    }                                                              \
  } while (0)

static int run(uint64_t seed) {
  std::mt19937_64 rng(seed);
  auto uni = [&](int lo, int hi) { return (int)(lo + rng() % (uint64_t)(hi - lo + 1)); };
  mab_sched_config cfg;
  cfg.sessions = uni(1, 12);
  cfg.prefill_chunk = uni(1, 70);
  cfg.max_pending_per_client = uni(1, 4);
  cfg.near_done_gate = uni(0, 10);
  cfg.max_decode_rows = uni(0, cfg.sessions);
  cfg.page_size = uni(1, 40);
  cfg.num_pages = uni(1, 300);
  cfg.max_pages_per_seq = uni(1, 64);
  mab_sched* raw = nullptr;
  CHECK(mab_sched_create(&cfg, &raw) == MAB_OK && raw);
  std::unique_ptr<mab_sched, void (*)(mab_sched*)> owner(raw, mab_sched_destroy);
  mab_sched* s = raw;
  const int cap = (cfg.max_decode_rows ? cfg.max_decode_rows : cfg.sessions) + 1;
  const int w = cfg.max_pages_per_seq;
  std::vector<int64_t> ids(cap);
  std::vector<int32_t> qs(cap + 1), pl(cap), bt((size_t)cap * w), emit(cap), fin(cap);
  std::vector<int> limit, got;
  int ticks = 0, idle_after = 0;
  for (int t = 0; t < 2000000; ++t) {
    const int k = t < 100 ? uni(0, 1) : 0;
    for (int i = 0; i < k; ++i) {
      int64_t id = -2;
      const int lim = uni(1, 30);
      const int32_t st = mab_sched_submit(s, uni(0, 5), uni(1, 200), lim, &id);
      CHECK(st == MAB_OK || st == MAB_ERR_SHAPE || st == MAB_ERR_QUOTA);
      CHECK((st == MAB_OK) == (id >= 0));
      if (st == MAB_OK) {
        CHECK(id == (int64_t)limit.size());
        limit.push_back(lim);
        got.push_back(0);
      }
    }
    mab_step_info info;
    CHECK(mab_sched_step(s, &info, ids.data(), qs.data(), pl.data(), bt.data(), emit.data(), fin.data(), cap) ==
          MAB_OK);
    if (info.kind == 0) {
      if (t >= 100 && ++idle_after > 2) break;
      continue;
    }
    ++ticks;
    CHECK(info.num_seqs >= 1 && info.num_seqs <= cap && qs[0] == 0 && qs[info.num_seqs] == info.num_rows);
    for (int i = 0; i < info.num_seqs; ++i) {
      const int q = qs[i + 1] - qs[i];
      CHECK(q >= 1 && q <= (q == 1 ? 1 : cfg.prefill_chunk));
      CHECK(ids[i] >= 0 && ids[i] < (int64_t)limit.size());
      const int used = (pl[i] + q + cfg.page_size - 1) / cfg.page_size;
      CHECK(used <= w);
      for (int j = 0; j < used; ++j) CHECK(bt[(size_t)i * w + j] >= 0 && bt[(size_t)i * w + j] < cfg.num_pages);
      if (emit[i]) ++got[ids[i]];
      if (fin[i]) CHECK(got[ids[i]] == limit[ids[i]]);
    }
  }
  for (size_t i = 0; i < limit.size(); ++i) CHECK(got[i] == limit[i]);
  return ticks > 0 || limit.empty() ? 0 : 1;
}

int main(int argc, char** argv) {
  const int n = argc > 1 ? atoi(argv[1]) : 200;
  for (int i = 0; i < n; ++i)
    if (run(1000 + i)) {
      fprintf(stderr, "seed %d failed\n", 1000 + i);
      return 1;
    }
  printf("ok %d\n", n);
  return 0;
}
