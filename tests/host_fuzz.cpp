// Seeded random driver of the host control plane (include/pagedkv_host.h),
// built by tests/test_host_sanitized.py with AddressSanitizer and
// UndefinedBehaviorSanitizer.  It calls only the public C functions, mixes
// valid calls with calls that must fail (stale handles, too few pages, bad
// sizes), and after every operation checks the invariants the header states:
//  - free + used pages = the pool's pages, and the pages in use are exactly
//    those with a positive reference count;
//  - a live sequence of L tokens holds ceil(L / page_size) pages, each in use;
//  - a failing call changes nothing (lengths, free pages);
//  - the step builder's table rows are the sequences' pages, padded.
// At the end every sequence, page handle and index entry is released and the
// whole pool must be free again.  Usage: host_fuzz SEED STEPS; prints "ok".
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <random>
#include <vector>

#include "pagedkv.h"
#include "pagedkv_host.h"

namespace {

int g_failures = 0;

void check(bool ok, const char* what, long step) {
  if (!ok) {
    fprintf(stderr, "step %ld: %s\n", step, what);
    ++g_failures;
  }
}

struct Seq {
  int64_t handle;
  std::vector<int32_t> tokens;  // the token ids the harness assigned, one per position
};

}  // namespace

int main(int argc, char** argv) {
  if (argc < 3) return 2;
  const uint64_t seed = strtoull(argv[1], nullptr, 10);
  const long steps = strtol(argv[2], nullptr, 10);
  std::mt19937_64 rng(seed);
  auto uni = [&](int64_t lo, int64_t hi) { return std::uniform_int_distribution<int64_t>(lo, hi)(rng); };

  const int32_t ps = (int32_t)(int64_t[]){4, 8, 16}[uni(0, 2)];
  const int64_t num_pages = uni(16, 160);
  pkv_page_pool* pool = pkv_pool_create(num_pages, ps);
  if (!pool) return 3;
  check(pkv_pool_create(0, ps) == nullptr && pkv_pool_create(8, 0) == nullptr, "create accepted a bad size", -1);

  std::vector<Seq> seqs;
  std::vector<int64_t> dead;     // handles of released sequences (stale)
  std::vector<int64_t> raw;      // page handles the harness holds itself
  std::vector<int64_t> raw_dead; // released page handles (stale)
  const uint64_t ns = 0x9E3779B97F4A7C15ull ^ seed;
  // tokens come from a small vocabulary in long runs, so prompts share prefixes
  auto token_at = [&](int64_t family, int64_t pos) { return (int32_t)((family * 31 + pos / 3) % 7); };

  auto invariants = [&](long step) {
    const int64_t fr = pkv_pool_free_pages(pool), us = pkv_pool_used_pages(pool);
    check(fr >= 0 && us >= 0 && fr + us == num_pages, "free + used != pages", step);
    int64_t in_use = 0;
    for (int64_t p = 0; p < num_pages; ++p) {
      const int32_t rc = pkv_page_refcount(pool, p);
      check(rc >= 0, "negative refcount", step);
      in_use += rc > 0;
      check(pkv_page_dirty(pool, p) == 0 || pkv_page_dirty(pool, p) == 1, "dirty flag not 0/1", step);
    }
    check(in_use == us, "pages in use != used count", step);
    check(pkv_page_refcount(pool, num_pages) == -1 && pkv_page_refcount(pool, -1) == -1, "out-of-range refcount", step);
    check(pkv_prefix_pages(pool) >= 0 && pkv_prefix_pages(pool) <= us, "index holds more pages than are used", step);
    for (const Seq& s : seqs) {
      const int64_t L = pkv_seq_length(pool, s.handle);
      check(L == (int64_t)s.tokens.size(), "sequence length differs from the harness's", step);
      std::vector<int64_t> pages((size_t)(L / ps + 2));
      const int64_t n = pkv_seq_pages(pool, s.handle, pages.data(), (int64_t)pages.size());
      check(n == (L + ps - 1) / ps, "page count != ceil(L / page_size)", step);
      for (int64_t i = 0; i < std::min<int64_t>(n, (int64_t)pages.size()); ++i)
        check(pkv_page_refcount(pool, pages[(size_t)i]) >= 1, "a sequence holds a free page", step);
      // a short output array is written only up to its capacity
      int64_t one[2] = {-7, -7};
      if (n > 1) {
        pkv_seq_pages(pool, s.handle, one, 1);
        check(one[1] == -7, "pkv_seq_pages wrote past its capacity", step);
      }
    }
    for (int64_t h : dead) check(pkv_seq_length(pool, h) == PKV_ERR_BAD_HANDLE, "a released sequence answers", step);
  };

  for (long step = 0; step < steps; ++step) {
    const int op = (int)uni(0, 13);
    const int64_t free_before = pkv_pool_free_pages(pool);
    if (op == 0 || seqs.empty()) {  // create
      int64_t h = -1;
      check(pkv_seq_create(pool, &h) == PKV_OK && h >= 0, "create failed", step);
      seqs.push_back({h, {}});
    } else if (op == 1) {  // append
      Seq& s = seqs[(size_t)uni(0, (int64_t)seqs.size() - 1)];
      const int64_t n = uni(0, 3 * ps);
      std::vector<int64_t> slots((size_t)n + 1, -5);
      const int st = pkv_seq_append(pool, s.handle, n, slots.data());
      if (st == PKV_OK) {
        const int64_t fam = s.tokens.empty() ? uni(0, 3) : s.tokens[0];
        for (int64_t i = 0; i < n; ++i) {
          const int64_t pos = (int64_t)s.tokens.size();
          check(slots[(size_t)i] >= 0 && slots[(size_t)i] < num_pages * ps, "slot out of range", step);
          check(slots[(size_t)i] % ps == pos % ps, "slot row != position mod page_size", step);
          s.tokens.push_back(token_at(fam, pos));
        }
        check(slots[(size_t)n] == -5, "append wrote past n slots", step);
      } else {
        check(st == PKV_ERR_NO_PAGES, "append failed with an unexpected status", step);
        check(pkv_pool_free_pages(pool) == free_before, "a failed append changed the pool", step);
      }
    } else if (op == 2) {  // batched append over distinct sequences
      std::vector<size_t> idx(seqs.size());
      for (size_t i = 0; i < idx.size(); ++i) idx[i] = i;
      std::shuffle(idx.begin(), idx.end(), rng);
      idx.resize((size_t)uni(1, (int64_t)idx.size()));
      std::vector<int64_t> hs, ns_;
      int64_t total = 0;
      for (size_t i : idx) {
        hs.push_back(seqs[i].handle);
        ns_.push_back(uni(0, ps + 1));
        total += ns_.back();
      }
      const bool repeat = uni(0, 9) == 0 && hs.size() > 1;
      if (repeat) hs.back() = hs.front();
      std::vector<int64_t> slots((size_t)total + 1, -5);
      const int st = pkv_seq_append_batch(pool, hs.data(), (int64_t)hs.size(), ns_.data(), slots.data());
      if (repeat) {
        check(st != PKV_OK && pkv_pool_free_pages(pool) == free_before, "a repeated sequence was accepted", step);
      } else if (st == PKV_OK) {
        size_t k = 0;
        for (size_t j = 0; j < idx.size(); ++j) {
          Seq& s = seqs[idx[j]];
          const int64_t fam = s.tokens.empty() ? uni(0, 3) : s.tokens[0];
          for (int64_t i = 0; i < ns_[j]; ++i, ++k) {
            check(slots[k] >= 0 && slots[k] % ps == (int64_t)s.tokens.size() % ps, "batch slot", step);
            s.tokens.push_back(token_at(fam, (int64_t)s.tokens.size()));
          }
        }
        check(slots[(size_t)total] == -5, "batch wrote past its slots", step);
      } else {
        check(st == PKV_ERR_NO_PAGES && pkv_pool_free_pages(pool) == free_before, "a failed batch changed the pool",
              step);
      }
    } else if (op == 3) {  // fork
      const Seq& parent = seqs[(size_t)uni(0, (int64_t)seqs.size() - 1)];
      const int64_t L = (int64_t)parent.tokens.size();
      const int64_t n = uni(0, L + 1);  // L + 1 must be refused
      int64_t child = -1, copy[3] = {-1, -1, -1};
      const int st = pkv_seq_fork(pool, parent.handle, n, &child, copy);
      if (n > L) {
        check(st != PKV_OK && pkv_pool_free_pages(pool) == free_before, "fork past the parent's length", step);
      } else if (st == PKV_OK) {
        check(copy[2] == n % ps, "fork copy count != n mod page_size", step);
        Seq c{child, std::vector<int32_t>(parent.tokens.begin(), parent.tokens.begin() + n)};
        seqs.push_back(c);
      } else {
        check(st == PKV_ERR_NO_PAGES && pkv_pool_free_pages(pool) == free_before, "a failed fork changed the pool",
              step);
      }
    } else if (op == 4) {  // release a sequence
      const size_t i = (size_t)uni(0, (int64_t)seqs.size() - 1);
      check(pkv_seq_release(pool, seqs[i].handle) == PKV_OK, "release failed", step);
      dead.push_back(seqs[i].handle);
      seqs.erase(seqs.begin() + (long)i);
      if (!dead.empty() && uni(0, 3) == 0)
        check(pkv_seq_release(pool, dead.back()) == PKV_ERR_BAD_HANDLE, "a stale sequence was released", step);
    } else if (op == 5) {  // raw page handles
      const int64_t n = uni(0, 4);
      std::vector<int64_t> h((size_t)n + 1, -5);
      const int st = pkv_page_alloc(pool, n, h.data());
      if (st == PKV_OK) {
        for (int64_t i = 0; i < n; ++i) raw.push_back(h[(size_t)i]);
        check(h[(size_t)n] == -5, "alloc wrote past n handles", step);
      } else {
        check(st == PKV_ERR_NO_PAGES && pkv_pool_free_pages(pool) == free_before, "a failed alloc changed the pool",
              step);
      }
    } else if (op == 6 && !raw.empty()) {  // release raw pages (and a stale one)
      const size_t i = (size_t)uni(0, (int64_t)raw.size() - 1);
      check(pkv_page_release(pool, &raw[i], 1) == PKV_OK, "page release failed", step);
      raw_dead.push_back(raw[i]);
      raw.erase(raw.begin() + (long)i);
      const int64_t stale = raw_dead[(size_t)uni(0, (int64_t)raw_dead.size() - 1)];
      const int st = pkv_page_release(pool, &stale, 1);
      check(st == PKV_ERR_BAD_HANDLE, "a stale page handle was released", step);
    } else if (op == 7) {  // index a sequence's whole pages
      const Seq& s = seqs[(size_t)uni(0, (int64_t)seqs.size() - 1)];
      const int64_t n = uni(0, (int64_t)s.tokens.size());
      check(pkv_prefix_insert(pool, ns, s.handle, s.tokens.data(), n) == PKV_OK, "insert failed", step);
      check(pkv_prefix_insert(pool, ns, s.handle, s.tokens.data(), (int64_t)s.tokens.size() + 1) != PKV_OK,
            "insert past the sequence's length", step);
    } else if (op == 8) {  // match a prompt drawn like the sequences' tokens
      const int64_t fam = uni(0, 3), n = uni(1, 4 * ps);
      std::vector<int32_t> prompt((size_t)n);
      for (int64_t i = 0; i < n; ++i) prompt[(size_t)i] = token_at(fam, i);
      int64_t h = -1, matched = -1;
      const int st = pkv_prefix_match(pool, ns ^ (uint64_t)uni(0, 1), prompt.data(), n, &h, &matched);
      if (st == PKV_OK) {
        check(matched >= 0 && matched % ps == 0 && matched <= n - 1, "matched count", step);
        seqs.push_back({h, std::vector<int32_t>(prompt.begin(), prompt.begin() + matched)});
      } else {
        check(pkv_pool_free_pages(pool) == free_before, "a failed match changed the pool", step);
      }
    } else if (op == 9) {  // evict
      int64_t freed = -1;
      check(pkv_prefix_evict(pool, uni(0, 6), &freed) == PKV_OK && freed >= 0, "evict failed", step);
      check(pkv_pool_free_pages(pool) == free_before + freed, "evict freed a different count", step);
    } else if (op == 10) {  // step metadata over distinct sequences
      std::vector<size_t> idx(seqs.size());
      for (size_t i = 0; i < idx.size(); ++i) idx[i] = i;
      std::shuffle(idx.begin(), idx.end(), rng);
      idx.resize((size_t)uni(1, (int64_t)idx.size()));
      const int64_t B = (int64_t)idx.size(), max_blocks = uni(1, 12), pad = num_pages - 1;
      std::vector<int64_t> hs, nn;
      for (size_t i : idx) {
        hs.push_back(seqs[i].handle);
        nn.push_back(std::min<int64_t>((int64_t)seqs[i].tokens.size(), uni(0, 2)));
      }
      std::vector<int64_t> bt((size_t)(B * max_blocks) + 1, -5), lens((size_t)B + 1, -5), qsl((size_t)B + 2, -5);
      const int st = pkv_build_step(pool, hs.data(), B, nn.data(), max_blocks, pad, bt.data(), lens.data(), qsl.data());
      check(bt[(size_t)(B * max_blocks)] == -5 && lens[(size_t)B] == -5 && qsl[(size_t)B + 1] == -5,
            "build_step wrote past its outputs", step);
      if (st == PKV_OK) {
        int64_t run = 0;
        check(qsl[0] == 0, "query_start_loc[0] != 0", step);
        for (int64_t b = 0; b < B; ++b) {
          const Seq& s = seqs[idx[(size_t)b]];
          check(lens[(size_t)b] == (int64_t)s.tokens.size(), "seq_lens", step);
          run += nn[(size_t)b];
          check(qsl[(size_t)b + 1] == run, "query_start_loc", step);
          std::vector<int64_t> pages((size_t)max_blocks + 1);
          const int64_t n = pkv_seq_pages(pool, s.handle, pages.data(), max_blocks + 1);
          for (int64_t j = 0; j < max_blocks; ++j)
            check(bt[(size_t)(b * max_blocks + j)] == (j < n ? pages[(size_t)j] : pad), "block_table row", step);
        }
      } else {
        check(st == PKV_ERR_SHAPE || st == PKV_ERR_DIRTY, "build_step failed with an unexpected status", step);
        check(lens[0] == -5, "a failed build_step wrote", step);
      }
    } else if (op == 11) {  // mark a sequence's pages overwritten
      const Seq& s = seqs[(size_t)uni(0, (int64_t)seqs.size() - 1)];
      std::vector<int64_t> pages(s.tokens.size() / (size_t)ps + 2);
      const int64_t n = pkv_seq_pages(pool, s.handle, pages.data(), (int64_t)pages.size());
      check(pkv_page_confirm(pool, pages.data(), n) == PKV_OK, "confirm failed", step);
      for (int64_t i = 0; i < n; ++i) check(pkv_page_dirty(pool, pages[(size_t)i]) == 0, "confirmed page dirty", step);
    } else if (op == 12) {  // bad arguments change nothing
      check(pkv_seq_append(pool, seqs[0].handle, -1, nullptr) != PKV_OK, "negative append accepted", step);
      check(pkv_page_alloc(pool, num_pages + 1, nullptr) != PKV_OK, "alloc of too many pages accepted", step);
      check(pkv_page_release(pool, nullptr, 1) != PKV_OK, "release of NULL accepted", step);
      check(pkv_pool_free_pages(pool) == free_before, "a refused call changed the pool", step);
    }
    invariants(step);
    if (g_failures > 20) break;
  }

  // tear down: everything goes back to the free list
  for (const Seq& s : seqs) check(pkv_seq_release(pool, s.handle) == PKV_OK, "final release", steps);
  seqs.clear();
  if (!raw.empty()) check(pkv_page_release(pool, raw.data(), (int64_t)raw.size()) == PKV_OK, "final page release", steps);
  int64_t freed = 0;
  check(pkv_prefix_evict(pool, num_pages, &freed) == PKV_OK, "final evict", steps);
  check(pkv_prefix_pages(pool) == 0, "the index still holds pages", steps);
  check(pkv_pool_free_pages(pool) == num_pages && pkv_pool_used_pages(pool) == 0, "pages leaked", steps);
  pkv_pool_destroy(pool);
  if (g_failures) {
    fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
