// Host block allocator: free list, reference counts, block tables, slot
// mappings and copy-on-write copy lists.  Pure C++; never touches the GPU.
//
// Semantics from the pages: equal fixed-size physical blocks and per-sequence
// block tables (cnblogs "paged attention", sections 2-3); blocks taken on
// demand, a new one only when the last is full, and returned to the free
// list at request end for immediate reuse (cnblogs sections 7-8;
// "08. PagedAttention", section "borrowing OS paging"); shared blocks carry a
// reference count and a sequence about to modify a shared block first gets
// a private copy (intelliparadigm.com article, section 2.3;
// "08. PagedAttention", section "what else paging solves"); slot =
// table[logical block] * block_size + offset ("08. PagedAttention", section
// "why the name").
//
// Orders the pages leave open, fixed here so results are reproducible: LIFO
// free stack seeded with init_order[0] on top; release pushes a sequence's
// blocks last-to-first; copy only when ref > 1 at the first write into the
// block (the last holder writes in place); appends are all-or-nothing.
//
// Swapping (preemption by swap, intelliparadigm.com article, sections 3.1
// and 6.1; "08. PagedAttention", section "what it does not solve"): a
// swapped-out sequence gives its blocks back exactly as a release would,
// keeps its length, and holds no blocks until it is swapped in, which takes
// fresh blocks off the free list in logical order (all-or-nothing).
//
// Prefix caching (cnblogs section 9: a shared system prompt is stored once;
// "08. PagedAttention", section "what else paging solves": only full blocks
// are shared, by reference count): appends that carry token ids name each
// full block by a chained FNV-1a hash of (previous block's hash, the block's
// token ids).  A block the append covers whole whose hash, and tokens, match
// a cached block reuses it (ref + 1, taken back off the free list if its
// count was 0) and its tokens get slot -1 (nothing to write).  Hits are
// decided for the whole append before anything is popped; a block that
// becomes full is registered unless its hash is already cached; a block
// popped off the free list loses its cache entry (its contents are about to
// be overwritten).
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pagedkv.h"

struct pkv_alloc {
  struct Seq {
    std::vector<int32_t> table;
    int64_t len = 0;
    bool swapped = false;
    std::vector<char> swapped_holes;  // table shape when it was swapped out: 1 = hole
    // prefix caching: every append so far carried token ids
    bool tok_ok = true;
    std::vector<uint64_t> hashes;  // chained hash of each full block
    std::vector<int32_t> pending;  // token ids of the partial last block
  };
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_stack;  // back() is the top
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;
  std::unordered_map<uint64_t, int32_t> cache;        // block hash -> block
  std::vector<uint64_t> block_hash;                   // hash a cached block is filed under
  std::vector<char> block_cached;                     // block has a cache entry
  std::vector<std::vector<int32_t>> block_tokens;     // token ids of a cached block
};

namespace {

// FNV-1a, 64 bit: offset basis 14695981039346656037, prime 1099511628211.
uint64_t fnv1a(uint64_t h, const unsigned char* p, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 1099511628211ull;
  }
  return h;
}

// Hash of a full block: FNV-1a over the previous block's hash (8 bytes,
// little endian) followed by the block's token ids (4 bytes each, little
// endian); the first block's previous hash is 0.
uint64_t block_hash_of(uint64_t prev, const int32_t* tokens, int B) {
  unsigned char buf[8];
  for (int i = 0; i < 8; ++i) buf[i] = (unsigned char)(prev >> (8 * i));
  uint64_t h = fnv1a(14695981039346656037ull, buf, 8);
  for (int j = 0; j < B; ++j) {
    const uint32_t t = (uint32_t)tokens[j];
    unsigned char b4[4] = {(unsigned char)t, (unsigned char)(t >> 8), (unsigned char)(t >> 16),
                           (unsigned char)(t >> 24)};
    h = fnv1a(h, b4, 4);
  }
  return h;
}

// Pop the top of the free stack; the block's cache entry, if any, goes.
int32_t pop_block(pkv_alloc* a) {
  const int32_t b = a->free_stack.back();
  a->free_stack.pop_back();
  if (a->block_cached[(size_t)b]) {
    a->cache.erase(a->block_hash[(size_t)b]);
    a->block_cached[(size_t)b] = 0;
    a->block_tokens[(size_t)b].clear();
  }
  return b;
}

}  // namespace

extern "C" {

pkv_alloc* pkv_alloc_create(int num_blocks, int block_size, const int32_t* init_order) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  pkv_alloc* a = new (std::nothrow) pkv_alloc;
  if (!a) return nullptr;
  try {
    a->num_blocks = num_blocks;
    a->block_size = block_size;
    a->ref.assign((size_t)num_blocks, 0);
    a->block_hash.assign((size_t)num_blocks, 0);
    a->block_cached.assign((size_t)num_blocks, 0);
    a->block_tokens.resize((size_t)num_blocks);
    a->free_stack.resize((size_t)num_blocks);
    std::vector<char> seen((size_t)num_blocks, 0);
    for (int i = 0; i < num_blocks; ++i) {
      const int32_t b = init_order ? init_order[i] : i;
      if (b < 0 || b >= num_blocks || seen[(size_t)b]) {
        delete a;
        return nullptr;
      }
      seen[(size_t)b] = 1;
      a->free_stack[(size_t)(num_blocks - 1 - i)] = b;
    }
  } catch (...) {
    delete a;
    return nullptr;
  }
  return a;
}

void pkv_alloc_destroy(pkv_alloc* a) { delete a; }

int pkv_seq_add(pkv_alloc* a, int64_t seq) {
  if (!a) return PKV_ERR_INVALID;
  if (a->seqs.count(seq)) return PKV_ERR_INVALID;
  try {
    a->seqs.emplace(seq, pkv_alloc::Seq{});
  } catch (...) {
    return PKV_ERR_STATE;
  }
  return PKV_OK;
}

int pkv_seq_append(pkv_alloc* a, int64_t seq, int n, int32_t* slots_out, int32_t* copy_pairs_out, int copy_cap,
                   int* num_copies_out) {
  if (!a || n < 0 || (n > 0 && !slots_out)) return PKV_ERR_INVALID;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PKV_ERR_INVALID;
  pkv_alloc::Seq& s = it->second;
  if (s.swapped) return PKV_ERR_STATE;
  const int64_t B = a->block_size;
  const int64_t start = s.len;
  const int64_t end = start + n;
  // Blocks needed: new logical blocks past the table, plus a copy of the
  // partially filled last block if this append writes into it while shared,
  // or a fresh block if that entry is a hole (-1: released by a trim of the
  // sequence this one was forked from; a write into a missing block takes a
  // new one, as a write past the table does).
  const int64_t have = (int64_t)s.table.size();
  const int64_t want = (end + B - 1) / B;
  int64_t need = want > have ? want - have : 0;
  int copies = 0;
  if (n > 0 && start / B < have) {
    const int32_t b0 = s.table[(size_t)(start / B)];
    if (b0 < 0) {
      ++need;
    } else if (a->ref[(size_t)b0] > 1) {
      ++need;
      copies = 1;
    }
  }
  if (copies > 0 && (copy_cap < copies || !copy_pairs_out)) return PKV_ERR_INVALID;
  if (need > (int64_t)a->free_stack.size()) return PKV_ERR_NO_BLOCKS;
  try {
    s.table.reserve((size_t)want);
  } catch (...) {
    return PKV_ERR_STATE;
  }
  int nc = 0;
  if (n > 0) {
    s.tok_ok = false;
    s.pending.clear();
  }
  for (int64_t p = start; p < end; ++p) {
    const int64_t lb = p / B;
    if (lb == (int64_t)s.table.size()) {
      const int32_t b = pop_block(a);
      a->ref[(size_t)b] = 1;
      s.table.push_back(b);
    } else if (s.table[(size_t)lb] < 0) {
      const int32_t b = pop_block(a);
      a->ref[(size_t)b] = 1;
      s.table[(size_t)lb] = b;
    } else if (a->ref[(size_t)s.table[(size_t)lb]] > 1) {
      const int32_t old = s.table[(size_t)lb];
      const int32_t b = pop_block(a);
      copy_pairs_out[2 * nc] = old;
      copy_pairs_out[2 * nc + 1] = b;
      ++nc;
      a->ref[(size_t)old] -= 1;
      a->ref[(size_t)b] = 1;
      s.table[(size_t)lb] = b;
    }
    slots_out[p - start] = (int32_t)(s.table[(size_t)lb] * B + p % B);
  }
  s.len = end;
  if (num_copies_out) *num_copies_out = nc;
  return PKV_OK;
}

int pkv_seq_append_tokens(pkv_alloc* a, int64_t seq, const int32_t* tokens, int n, int32_t* slots_out,
                          int* num_cached_out, int32_t* copy_pairs_out, int copy_cap, int* num_copies_out) {
  if (!a || n < 0 || (n > 0 && (!slots_out || !tokens))) return PKV_ERR_INVALID;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PKV_ERR_INVALID;
  pkv_alloc::Seq& s = it->second;
  if (s.swapped) return PKV_ERR_STATE;
  // no hash chain (an earlier append carried no tokens), or a hole where the
  // append starts: no caching
  if (!s.tok_ok || (s.len % a->block_size != 0 && (int64_t)s.table.size() > s.len / a->block_size &&
                    s.table[(size_t)(s.len / a->block_size)] < 0)) {
    const int st = pkv_seq_append(a, seq, n, slots_out, copy_pairs_out, copy_cap, num_copies_out);
    if (st == PKV_OK && num_cached_out) *num_cached_out = 0;
    return st;
  }
  const int64_t B = a->block_size;
  const int64_t start = s.len;
  const int64_t end = start + n;
  const int64_t have = (int64_t)s.table.size();
  const int64_t first = start / B;
  const int64_t want = (end + B - 1) / B;
  const int64_t nb = want > first ? want - first : 0;
  // 1. hashes of the blocks that become full, and hits, decided on the
  //    cache as it is before this append: a block past the table (so
  //    covered whole by the append) hits if a cached block carries its hash
  //    and tokens, as long as every earlier new block of the append hit
  std::vector<uint64_t> hsh;
  std::vector<int32_t> hit;
  std::vector<char> full;
  std::vector<int32_t> cur;
  try {
    hsh.assign((size_t)nb, 0);
    hit.assign((size_t)nb, -1);
    full.assign((size_t)nb, 0);
    cur = s.pending;
    uint64_t prev = s.hashes.empty() ? 0 : s.hashes.back();
    bool chain = true;
    for (int64_t p = start; p < end; ++p) {
      cur.push_back(tokens[p - start]);
      if ((int64_t)cur.size() == B) {
        const int64_t lb = p / B;
        const size_t i = (size_t)(lb - first);
        const uint64_t h = block_hash_of(prev, cur.data(), (int)B);
        hsh[i] = h;
        full[i] = 1;
        if (lb >= have) {
          if (chain) {
            auto c = a->cache.find(h);
            if (c != a->cache.end() &&
                memcmp(a->block_tokens[(size_t)c->second].data(), cur.data(), (size_t)B * sizeof(int32_t)) == 0)
              hit[i] = c->second;
          }
          if (hit[i] < 0) chain = false;
        }
        prev = h;
        cur.clear();
      }
    }
  } catch (...) {
    return PKV_ERR_STATE;
  }
  // 2. blocks taken off the free list: the copy of a shared partial block,
  //    every new block that misses, and hits whose count is 0
  int64_t need = 0;
  const bool cow = n > 0 && first < have && a->ref[(size_t)s.table[(size_t)first]] > 1;
  if (cow) ++need;
  for (int64_t lb = std::max(first, have); lb < want; ++lb) {
    const int32_t hb = hit[(size_t)(lb - first)];
    if (hb < 0 || a->ref[(size_t)hb] == 0) ++need;
  }
  if (cow && (copy_cap < 1 || !copy_pairs_out)) return PKV_ERR_INVALID;
  if (need > (int64_t)a->free_stack.size()) return PKV_ERR_NO_BLOCKS;
  try {
    s.table.reserve((size_t)want);
    s.hashes.reserve(s.hashes.size() + (size_t)nb);
  } catch (...) {
    return PKV_ERR_STATE;
  }
  // 3. hits with count 0 leave the free list before anything is popped
  for (int64_t lb = std::max(first, have); lb < want; ++lb) {
    const int32_t hb = hit[(size_t)(lb - first)];
    if (hb >= 0 && a->ref[(size_t)hb] == 0)
      a->free_stack.erase(std::find(a->free_stack.begin(), a->free_stack.end(), hb));
  }
  // 4. as a plain append: the copy first, then new blocks in logical order
  int nc = 0;
  if (cow) {
    const int32_t old = s.table[(size_t)first];
    const int32_t b = pop_block(a);
    copy_pairs_out[0] = old;
    copy_pairs_out[1] = b;
    nc = 1;
    a->ref[(size_t)old] -= 1;
    a->ref[(size_t)b] = 1;
    s.table[(size_t)first] = b;
  }
  for (int64_t lb = std::max(first, have); lb < want; ++lb) {
    const int32_t hb = hit[(size_t)(lb - first)];
    if (hb >= 0) {
      a->ref[(size_t)hb] += 1;
      s.table.push_back(hb);
    } else {
      const int32_t b = pop_block(a);
      a->ref[(size_t)b] = 1;
      s.table.push_back(b);
    }
  }
  // 5. slots (-1 for tokens already in a cached block), hash chain, and
  //    registration of the blocks this append filled
  int ncached = 0;
  for (int64_t p = start; p < end; ++p) {
    const int64_t lb = p / B;
    if (hit[(size_t)(lb - first)] >= 0) {
      slots_out[p - start] = -1;
      ++ncached;
    } else {
      slots_out[p - start] = (int32_t)(s.table[(size_t)lb] * B + p % B);
    }
  }
  std::vector<int32_t> blk_tokens;
  blk_tokens = s.pending;
  for (int64_t p = start; p < end; ++p) {
    blk_tokens.push_back(tokens[p - start]);
    if ((int64_t)blk_tokens.size() == B) {
      const int64_t lb = p / B;
      const size_t i = (size_t)(lb - first);
      const int32_t blk = s.table[(size_t)lb];
      s.hashes.push_back(hsh[i]);
      if (hit[i] < 0 && !a->cache.count(hsh[i])) {
        a->cache.emplace(hsh[i], blk);
        a->block_hash[(size_t)blk] = hsh[i];
        a->block_cached[(size_t)blk] = 1;
        a->block_tokens[(size_t)blk] = blk_tokens;
      }
      blk_tokens.clear();
    }
  }
  s.pending = blk_tokens;
  s.len = end;
  if (num_copies_out) *num_copies_out = nc;
  if (num_cached_out) *num_cached_out = ncached;
  return PKV_OK;
}

int pkv_seq_trim(pkv_alloc* a, int64_t seq, int64_t keep_from, int* freed_out) {
  if (!a || !freed_out) return PKV_ERR_INVALID;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PKV_ERR_INVALID;
  pkv_alloc::Seq& s = it->second;
  if (s.swapped) return PKV_ERR_STATE;
  if (keep_from < 0 || keep_from > s.len) return PKV_ERR_INVALID;
  const int64_t upto = std::min<int64_t>(keep_from / a->block_size, (int64_t)s.table.size());
  for (int64_t lb = upto - 1; lb >= 0; --lb) {
    const int32_t b = s.table[(size_t)lb];
    if (b >= 0 && a->ref[(size_t)b] <= 0) return PKV_ERR_STATE;
  }
  int freed = 0;
  for (int64_t lb = upto - 1; lb >= 0; --lb) {
    const int32_t b = s.table[(size_t)lb];
    if (b < 0) continue;
    if (--a->ref[(size_t)b] == 0) a->free_stack.push_back(b);
    s.table[(size_t)lb] = -1;
    ++freed;
  }
  *freed_out = freed;
  return PKV_OK;
}

int pkv_prefix_cache_size(const pkv_alloc* a, int* entries_out) {
  if (!a || !entries_out) return PKV_ERR_INVALID;
  *entries_out = (int)a->cache.size();
  return PKV_OK;
}

int pkv_seq_fork(pkv_alloc* a, int64_t parent, int64_t child, int fork_pos) {
  if (!a) return PKV_ERR_INVALID;
  auto it = a->seqs.find(parent);
  if (it == a->seqs.end() || a->seqs.count(child)) return PKV_ERR_INVALID;
  if (it->second.swapped) return PKV_ERR_STATE;
  if (fork_pos < 0 || fork_pos > it->second.len) return PKV_ERR_INVALID;
  const int64_t nb = ((int64_t)fork_pos + a->block_size - 1) / a->block_size;
  pkv_alloc::Seq c;
  try {
    c.table.assign(it->second.table.begin(), it->second.table.begin() + nb);
    c.len = fork_pos;
    // a child forked on a block boundary inherits the hash chain; one forked
    // inside a block does not take part in prefix caching
    const pkv_alloc::Seq& par = it->second;
    c.tok_ok = par.tok_ok && fork_pos % a->block_size == 0 &&
               (int64_t)par.hashes.size() >= fork_pos / a->block_size;
    if (c.tok_ok) c.hashes.assign(par.hashes.begin(), par.hashes.begin() + fork_pos / a->block_size);
    for (int32_t b : c.table)
      if (b >= 0) a->ref[(size_t)b] += 1;  // holes (released by a trim) stay holes
    a->seqs.emplace(child, std::move(c));
  } catch (...) {
    return PKV_ERR_STATE;
  }
  return PKV_OK;
}

int pkv_seq_free(pkv_alloc* a, int64_t seq) {
  if (!a) return PKV_ERR_INVALID;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PKV_ERR_INVALID;
  const std::vector<int32_t>& t = it->second.table;
  for (auto b = t.rbegin(); b != t.rend(); ++b)
    if (*b >= 0 && a->ref[(size_t)*b] <= 0) return PKV_ERR_STATE;
  for (auto b = t.rbegin(); b != t.rend(); ++b) {
    if (*b >= 0 && --a->ref[(size_t)*b] == 0) a->free_stack.push_back(*b);
  }
  a->seqs.erase(it);
  return PKV_OK;
}

int pkv_seq_swap_out(pkv_alloc* a, int64_t seq, int32_t* blocks_out, int cap, int* num_out) {
  if (!a || !num_out) return PKV_ERR_INVALID;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PKV_ERR_INVALID;
  pkv_alloc::Seq& s = it->second;
  if (s.swapped) return PKV_ERR_STATE;
  const std::vector<int32_t>& t = s.table;
  *num_out = (int)t.size();
  if ((int64_t)t.size() > cap || (!t.empty() && !blocks_out)) return PKV_ERR_INVALID;
  for (auto b = t.rbegin(); b != t.rend(); ++b)
    if (*b >= 0 && a->ref[(size_t)*b] <= 0) return PKV_ERR_STATE;
  try {
    s.swapped_holes.assign(t.size(), 0);
  } catch (...) {
    return PKV_ERR_STATE;
  }
  for (size_t i = 0; i < t.size(); ++i) {
    blocks_out[i] = t[i];
    s.swapped_holes[i] = t[i] < 0;
  }
  for (auto b = t.rbegin(); b != t.rend(); ++b) {
    if (*b >= 0 && --a->ref[(size_t)*b] == 0) a->free_stack.push_back(*b);
  }
  s.table.clear();
  s.swapped = true;
  return PKV_OK;
}

int pkv_seq_swap_in(pkv_alloc* a, int64_t seq, int32_t* blocks_out, int cap, int* num_out) {
  if (!a || !num_out) return PKV_ERR_INVALID;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PKV_ERR_INVALID;
  pkv_alloc::Seq& s = it->second;
  if (!s.swapped) return PKV_ERR_STATE;
  const int64_t n = (int64_t)s.swapped_holes.size();
  *num_out = (int)n;
  if (n > cap || (n > 0 && !blocks_out)) return PKV_ERR_INVALID;
  int64_t live = 0;
  for (char h : s.swapped_holes) live += !h;
  if (live > (int64_t)a->free_stack.size()) return PKV_ERR_NO_BLOCKS;
  try {
    s.table.reserve((size_t)n);
  } catch (...) {
    return PKV_ERR_STATE;
  }
  for (int64_t i = 0; i < n; ++i) {
    int32_t b = -1;
    if (!s.swapped_holes[(size_t)i]) {
      b = pop_block(a);
      a->ref[(size_t)b] = 1;
    }
    s.table.push_back(b);
    blocks_out[i] = b;
  }
  s.swapped = false;
  s.swapped_holes.clear();
  return PKV_OK;
}

int pkv_seq_len(const pkv_alloc* a, int64_t seq, int64_t* len_out) {
  if (!a || !len_out) return PKV_ERR_INVALID;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PKV_ERR_INVALID;
  *len_out = it->second.len;
  return PKV_OK;
}

int pkv_get_block_table(const pkv_alloc* a, int64_t seq, int32_t* out, int cap, int* len_out) {
  if (!a || !len_out) return PKV_ERR_INVALID;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PKV_ERR_INVALID;
  const std::vector<int32_t>& t = it->second.table;
  *len_out = (int)t.size();
  if ((int64_t)t.size() > cap || (!t.empty() && !out)) return PKV_ERR_INVALID;
  for (size_t i = 0; i < t.size(); ++i) out[i] = t[i];
  return PKV_OK;
}

int pkv_build_block_tables(const pkv_alloc* a, const int64_t* seqs, int num_seqs, int max_blocks_per_seq,
                           int32_t* tables_out, int32_t* context_lens_out) {
  if (!a || num_seqs < 0 || max_blocks_per_seq <= 0) return PKV_ERR_INVALID;
  if (num_seqs > 0 && (!seqs || !tables_out || !context_lens_out)) return PKV_ERR_INVALID;
  for (int i = 0; i < num_seqs; ++i) {
    auto it = a->seqs.find(seqs[i]);
    if (it == a->seqs.end()) return PKV_ERR_INVALID;
    if (it->second.swapped) return PKV_ERR_STATE;
    if ((int64_t)it->second.table.size() > max_blocks_per_seq || it->second.len > INT32_MAX)
      return PKV_ERR_INVALID;
  }
  for (int i = 0; i < num_seqs; ++i) {
    const pkv_alloc::Seq& s = a->seqs.find(seqs[i])->second;
    int32_t* row = tables_out + (size_t)i * max_blocks_per_seq;
    size_t j = 0;
    for (; j < s.table.size(); ++j) row[j] = s.table[j];
    for (; j < (size_t)max_blocks_per_seq; ++j) row[j] = -1;
    context_lens_out[i] = (int32_t)s.len;
  }
  return PKV_OK;
}

int pkv_shared_prefix_groups(const pkv_alloc* a, const int64_t* seqs, int num_seqs, int max_members,
                             int32_t* group_start_out, int32_t* shared_blocks_out, int* num_groups_out) {
  if (!a || num_seqs < 0 || max_members < 1 || !num_groups_out) return PKV_ERR_INVALID;
  if (num_seqs > 0 && (!seqs || !group_start_out || !shared_blocks_out)) return PKV_ERR_INVALID;
  std::vector<const pkv_alloc::Seq*> ss((size_t)num_seqs);
  for (int i = 0; i < num_seqs; ++i) {
    auto it = a->seqs.find(seqs[i]);
    if (it == a->seqs.end()) return PKV_ERR_INVALID;
    if (it->second.swapped) return PKV_ERR_STATE;
    ss[(size_t)i] = &it->second;
  }
  const int64_t B = a->block_size;
  int ng = 0;
  int i = 0;
  while (i < num_seqs) {
    // a group: this sequence and the ones right after it that hold the same
    // physical block as their first block (forks of one prompt), up to
    // max_members
    const std::vector<int32_t>& t0 = ss[(size_t)i]->table;
    int j = i + 1;
    while (j < num_seqs && j - i < max_members && !t0.empty() && t0[0] >= 0 && !ss[(size_t)j]->table.empty() &&
           ss[(size_t)j]->table[0] == t0[0])
      ++j;
    // shared: the longest common prefix of the members' tables, of live
    // blocks wholly inside every member's context
    int64_t k = 0;
    if (j - i > 1) {
      for (;; ++k) {
        if (k >= (int64_t)t0.size() || t0[(size_t)k] < 0) break;
        bool same = true;
        for (int m = i; m < j && same; ++m) {
          const pkv_alloc::Seq& s = *ss[(size_t)m];
          same = k < (int64_t)s.table.size() && s.table[(size_t)k] == t0[(size_t)k] && (k + 1) * B <= s.len;
        }
        if (!same) break;
      }
    }
    group_start_out[ng] = i;
    shared_blocks_out[ng] = (int32_t)k;
    ++ng;
    i = j;
  }
  if (num_seqs > 0) group_start_out[ng] = num_seqs;
  else group_start_out[0] = 0;
  *num_groups_out = ng;
  return PKV_OK;
}

int pkv_alloc_stats(const pkv_alloc* a, pkv_stats* out) {
  if (!a || !out) return PKV_ERR_INVALID;
  out->num_blocks = a->num_blocks;
  out->block_size = a->block_size;
  out->num_free = (int32_t)a->free_stack.size();
  int32_t used = 0, shared = 0;
  for (int32_t r : a->ref) {
    used += r > 0;
    shared += r > 1;
  }
  out->num_used = used;
  out->num_shared = shared;
  out->num_seqs = (int32_t)a->seqs.size();
  int64_t toks = 0, slots = 0;
  for (const auto& kv : a->seqs) {
    toks += kv.second.len;
    for (int32_t b : kv.second.table) slots += b >= 0 ? a->block_size : 0;
  }
  out->logical_tokens = toks;
  out->table_slots = slots;
  return PKV_OK;
}

int pkv_block_ref(const pkv_alloc* a, int block, int* ref_out) {
  if (!a || !ref_out || block < 0 || block >= a->num_blocks) return PKV_ERR_INVALID;
  *ref_out = a->ref[(size_t)block];
  return PKV_OK;
}

int pkv_free_list(const pkv_alloc* a, int32_t* out, int cap, int* len_out) {
  if (!a || !len_out) return PKV_ERR_INVALID;
  const size_t n = a->free_stack.size();
  *len_out = (int)n;
  if ((int64_t)n > cap || (n && !out)) return PKV_ERR_INVALID;
  for (size_t i = 0; i < n; ++i) out[i] = a->free_stack[n - 1 - i];
  return PKV_OK;
}

}  // extern "C"
