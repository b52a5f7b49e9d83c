// Randomised check of the host block allocator through its C ABI, built with
// the address and undefined-behaviour sanitizers by tests/test_alloc_sanitize.py.
//
// Usage: alloc_check <seed> <num_ops> <num_blocks> <block_size>
// Runs a seeded sequence of add / append / append_tokens / fork / free /
// trim / swap operations and checks after every one of them the invariants
// the pages fix for the block tables:
//  - a block's reference count equals the number of tables that hold it
//    ("08. PagedAttention": shared blocks carry a reference count);
//  - the free list holds each block at most once, only blocks with count 0,
//    and free + used blocks = the pool;
//  - a sequence of length L has ceil(L / B) table entries and wastes fewer
//    than B slots (cnblogs section 4);
//  - slots follow slot = table[pos / B] * B + pos % B ("08. PagedAttention",
//    section "why the name");
//  - a failed append (not enough blocks) changes nothing.
// Exit status 0 when every check holds, 1 with a message otherwise.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <map>
#include <set>
#include <vector>

#include "pagedkv.h"

namespace {

uint64_t g_state = 1;

// splitmix64: a published counter-based generator (input generation only)
uint64_t next_u64() {
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int rnd(int lo, int hi) {  // inclusive
  return lo + (int)(next_u64() % (uint64_t)(hi - lo + 1));
}

int g_failures = 0;

#define CHECK(cond, ...)                              \
  do {                                                \
    if (!(cond)) {                                    \
      fprintf(stderr, "check failed: %s: ", #cond);   \
      fprintf(stderr, __VA_ARGS__);                   \
      fprintf(stderr, "\n");                          \
      ++g_failures;                                   \
      return false;                                   \
    }                                                 \
  } while (0)

struct Seq {
  bool swapped = false;
  bool tokened = true;  // every append so far carried token ids
};

struct World {
  pkv_alloc* a = nullptr;
  int N = 0, B = 0;
  std::map<int64_t, Seq> seqs;
  int64_t next_id = 0;
};

std::vector<int32_t> table_of(const World& w, int64_t s) {
  std::vector<int32_t> t(w.N + 8);
  int len = 0;
  if (pkv_get_block_table(w.a, s, t.data(), (int)t.size(), &len) != PKV_OK) return {};
  t.resize(len);
  return t;
}

bool check_invariants(const World& w) {
  std::vector<int> holders(w.N, 0);
  int64_t logical = 0, slots = 0;
  for (const auto& kv : w.seqs) {
    int64_t len = 0;
    CHECK(pkv_seq_len(w.a, kv.first, &len) == PKV_OK, "seq %lld has no length", (long long)kv.first);
    logical += len;
    if (kv.second.swapped) continue;
    const std::vector<int32_t> t = table_of(w, kv.first);
    CHECK((int64_t)t.size() == (len + w.B - 1) / w.B, "seq %lld: %zu entries for length %lld",
          (long long)kv.first, t.size(), (long long)len);
    CHECK((int64_t)t.size() * w.B - len < w.B, "seq %lld wastes a whole block", (long long)kv.first);
    slots += (int64_t)t.size() * w.B;
    std::set<int32_t> mine;
    for (int32_t b : t) {
      if (b < 0) continue;  // hole left by a trim
      CHECK(b < w.N, "block %d out of range", b);
      CHECK(mine.insert(b).second, "seq %lld holds block %d twice", (long long)kv.first, b);
      ++holders[b];
    }
  }
  std::vector<int32_t> fl(w.N + 8);
  int nfree = 0;
  CHECK(pkv_free_list(w.a, fl.data(), (int)fl.size(), &nfree) == PKV_OK, "free list");
  std::set<int32_t> fset;
  for (int i = 0; i < nfree; ++i) {
    CHECK(fl[i] >= 0 && fl[i] < w.N, "free entry %d out of range", fl[i]);
    CHECK(fset.insert(fl[i]).second, "block %d twice on the free list", fl[i]);
  }
  int used = 0;
  for (int b = 0; b < w.N; ++b) {
    int ref = -1;
    CHECK(pkv_block_ref(w.a, b, &ref) == PKV_OK, "ref of %d", b);
    CHECK(ref == holders[b], "block %d: ref %d, held by %d tables", b, ref, holders[b]);
    if (ref > 0) {
      ++used;
      CHECK(!fset.count(b), "block %d is used and free", b);
    }
  }
  CHECK(used + nfree == w.N, "used %d + free %d != %d", used, nfree, w.N);
  pkv_stats st;
  CHECK(pkv_alloc_stats(w.a, &st) == PKV_OK, "stats");
  CHECK(st.num_free == nfree && st.num_used == used, "stats disagree with the free list");
  CHECK(st.logical_tokens == logical, "stats: %lld logical tokens, counted %lld", (long long)st.logical_tokens,
        (long long)logical);
  (void)slots;
  return true;
}

bool same_stats(const pkv_stats& x, const pkv_stats& y) {
  return x.num_free == y.num_free && x.num_used == y.num_used && x.num_seqs == y.num_seqs &&
         x.num_shared == y.num_shared && x.logical_tokens == y.logical_tokens && x.table_slots == y.table_slots;
}

// Append n tokens (with token ids from a small vocabulary when `tokens`);
// checks the slot formula against the table afterwards.
bool do_append(World& w, int64_t s, int n, bool tokens) {
  int64_t len0 = 0;
  pkv_seq_len(w.a, s, &len0);
  std::vector<int32_t> sl(n), cp(2 * 4), ids(n);
  for (int i = 0; i < n; ++i) ids[i] = rnd(0, 2);  // few distinct ids: prefix-cache hits happen
  int ncp = 0, ncached = 0;
  pkv_stats before, after;
  pkv_alloc_stats(w.a, &before);
  const int rc = tokens ? pkv_seq_append_tokens(w.a, s, ids.data(), n, sl.data(), &ncached, cp.data(), 4, &ncp)
                        : pkv_seq_append(w.a, s, n, sl.data(), cp.data(), 4, &ncp);
  if (rc == PKV_ERR_NO_BLOCKS) {
    pkv_alloc_stats(w.a, &after);
    CHECK(same_stats(before, after), "a failed append changed the allocator");
    return true;
  }
  CHECK(rc == PKV_OK, "append returned %d", rc);
  if (!tokens) w.seqs[s].tokened = false;
  const std::vector<int32_t> t = table_of(w, s);
  for (int i = 0; i < n; ++i) {
    if (sl[i] < 0) {
      CHECK(tokens, "slot -1 from a plain append");
      continue;
    }
    const int64_t p = len0 + i;
    CHECK(p / w.B < (int64_t)t.size(), "position past the table");
    CHECK(sl[i] == t[p / w.B] * w.B + (int32_t)(p % w.B), "slot %d for position %lld, table entry %d", sl[i],
          (long long)p, t[p / w.B]);
  }
  for (int c = 0; c < ncp; ++c) {
    CHECK(cp[2 * c] >= 0 && cp[2 * c] < w.N && cp[2 * c + 1] >= 0 && cp[2 * c + 1] < w.N &&
              cp[2 * c] != cp[2 * c + 1],
          "bad copy pair (%d, %d)", cp[2 * c], cp[2 * c + 1]);
  }
  return true;
}

int64_t pick(const World& w, bool want_swapped, bool any = false) {
  std::vector<int64_t> c;
  for (const auto& kv : w.seqs)
    if (any || kv.second.swapped == want_swapped) c.push_back(kv.first);
  if (c.empty()) return -1;
  return c[rnd(0, (int)c.size() - 1)];
}

bool step(World& w) {
  const int op = rnd(0, 99);
  if (op < 15 || w.seqs.empty()) {  // new sequence with a first append
    const int64_t s = w.next_id++;
    CHECK(pkv_seq_add(w.a, s) == PKV_OK, "add");
    w.seqs[s] = Seq();
    return do_append(w, s, rnd(1, 3 * w.B + 2), rnd(0, 1) == 0);
  }
  if (op < 50) {  // append to a live sequence
    const int64_t s = pick(w, false);
    if (s < 0) return true;
    const bool tok = w.seqs[s].tokened && rnd(0, 1) == 0;
    return do_append(w, s, rnd(1, 2 * w.B + 1), tok);
  }
  if (op < 62) {  // fork
    const int64_t p = pick(w, false);
    if (p < 0) return true;
    int64_t len = 0;
    pkv_seq_len(w.a, p, &len);
    const int64_t c = w.next_id++;
    CHECK(pkv_seq_fork(w.a, p, c, rnd(0, (int)len)) == PKV_OK, "fork");
    w.seqs[c] = Seq();
    w.seqs[c].tokened = false;
    return true;
  }
  if (op < 77) {  // free
    const int64_t s = pick(w, false, true);
    CHECK(pkv_seq_free(w.a, s) == PKV_OK, "free");
    w.seqs.erase(s);
    return true;
  }
  if (op < 85) {  // trim (sliding window)
    const int64_t s = pick(w, false);
    if (s < 0) return true;
    int64_t len = 0;
    pkv_seq_len(w.a, s, &len);
    int freed = 0;
    CHECK(pkv_seq_trim(w.a, s, rnd(0, (int)len), &freed) == PKV_OK, "trim");
    return true;
  }
  if (op < 93) {  // swap out
    const int64_t s = pick(w, false);
    if (s < 0) return true;
    std::vector<int32_t> blocks(w.N + 8);
    int n = 0;
    CHECK(pkv_seq_swap_out(w.a, s, blocks.data(), (int)blocks.size(), &n) == PKV_OK, "swap out");
    w.seqs[s].swapped = true;
    return true;
  }
  // swap in
  const int64_t s = pick(w, true);
  if (s < 0) return true;
  std::vector<int32_t> blocks(w.N + 8);
  int n = 0;
  const int rc = pkv_seq_swap_in(w.a, s, blocks.data(), (int)blocks.size(), &n);
  CHECK(rc == PKV_OK || rc == PKV_ERR_NO_BLOCKS, "swap in returned %d", rc);
  if (rc == PKV_OK) w.seqs[s].swapped = false;
  return true;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 5) {
    fprintf(stderr, "usage: %s seed num_ops num_blocks block_size\n", argv[0]);
    return 2;
  }
  g_state = strtoull(argv[1], nullptr, 10) * 0x2545F4914F6CDD1Dull + 1;
  const int ops = atoi(argv[2]);
  World w;
  w.N = atoi(argv[3]);
  w.B = atoi(argv[4]);
  std::vector<int32_t> order(w.N);
  for (int i = 0; i < w.N; ++i) order[i] = i;
  for (int i = w.N - 1; i > 0; --i) {
    const int j = rnd(0, i);
    const int32_t t = order[i];
    order[i] = order[j];
    order[j] = t;
  }
  w.a = pkv_alloc_create(w.N, w.B, order.data());
  if (!w.a) {
    fprintf(stderr, "pkv_alloc_create failed\n");
    return 1;
  }
  for (int i = 0; i < ops && g_failures == 0; ++i) {
    if (!step(w) || !check_invariants(w)) fprintf(stderr, "after operation %d\n", i);
  }
  // release everything: the whole pool must come back
  while (!w.seqs.empty()) {
    pkv_seq_free(w.a, w.seqs.begin()->first);
    w.seqs.erase(w.seqs.begin());
  }
  pkv_stats st;
  pkv_alloc_stats(w.a, &st);
  if (st.num_free != w.N) {
    fprintf(stderr, "%d of %d blocks free after releasing every sequence\n", st.num_free, w.N);
    ++g_failures;
  }
  pkv_alloc_destroy(w.a);
  printf("%s: %d operations, %d blocks of %d\n", g_failures ? "FAILED" : "ok", ops, w.N, w.B);
  return g_failures ? 1 : 0;
}
