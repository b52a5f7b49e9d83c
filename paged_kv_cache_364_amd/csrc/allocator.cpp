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
#include <stdint.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pagedkv.h"

struct pkv_alloc {
  struct Seq {
    std::vector<int32_t> table;
    int64_t len = 0;
    bool swapped = false;
    int64_t swapped_blocks = 0;  // table length when it was swapped out
  };
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_stack;  // back() is the top
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;
};

extern "C" {

pkv_alloc* pkv_alloc_create(int num_blocks, int block_size, const int32_t* init_order) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  pkv_alloc* a = new (std::nothrow) pkv_alloc;
  if (!a) return nullptr;
  try {
    a->num_blocks = num_blocks;
    a->block_size = block_size;
    a->ref.assign((size_t)num_blocks, 0);
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
  // partially filled last block if this append writes into it while shared.
  const int64_t have = (int64_t)s.table.size();
  const int64_t want = (end + B - 1) / B;
  int64_t need = want > have ? want - have : 0;
  int copies = 0;
  if (n > 0 && start / B < have && a->ref[(size_t)s.table[(size_t)(start / B)]] > 1) {
    ++need;
    copies = 1;
  }
  if (copies > 0 && (copy_cap < copies || !copy_pairs_out)) return PKV_ERR_INVALID;
  if (need > (int64_t)a->free_stack.size()) return PKV_ERR_NO_BLOCKS;
  try {
    s.table.reserve((size_t)want);
  } catch (...) {
    return PKV_ERR_STATE;
  }
  int nc = 0;
  for (int64_t p = start; p < end; ++p) {
    const int64_t lb = p / B;
    if (lb == (int64_t)s.table.size()) {
      const int32_t b = a->free_stack.back();
      a->free_stack.pop_back();
      a->ref[(size_t)b] = 1;
      s.table.push_back(b);
    } else if (a->ref[(size_t)s.table[(size_t)lb]] > 1) {
      const int32_t old = s.table[(size_t)lb];
      const int32_t b = a->free_stack.back();
      a->free_stack.pop_back();
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
    for (int32_t b : c.table) a->ref[(size_t)b] += 1;
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
    if (a->ref[(size_t)*b] <= 0) return PKV_ERR_STATE;
  for (auto b = t.rbegin(); b != t.rend(); ++b) {
    if (--a->ref[(size_t)*b] == 0) a->free_stack.push_back(*b);
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
    if (a->ref[(size_t)*b] <= 0) return PKV_ERR_STATE;
  for (size_t i = 0; i < t.size(); ++i) blocks_out[i] = t[i];
  for (auto b = t.rbegin(); b != t.rend(); ++b) {
    if (--a->ref[(size_t)*b] == 0) a->free_stack.push_back(*b);
  }
  s.swapped_blocks = (int64_t)t.size();
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
  const int64_t n = s.swapped_blocks;
  *num_out = (int)n;
  if (n > cap || (n > 0 && !blocks_out)) return PKV_ERR_INVALID;
  if (n > (int64_t)a->free_stack.size()) return PKV_ERR_NO_BLOCKS;
  try {
    s.table.reserve((size_t)n);
  } catch (...) {
    return PKV_ERR_STATE;
  }
  for (int64_t i = 0; i < n; ++i) {
    const int32_t b = a->free_stack.back();
    a->free_stack.pop_back();
    a->ref[(size_t)b] = 1;
    s.table.push_back(b);
    blocks_out[i] = b;
  }
  s.swapped = false;
  s.swapped_blocks = 0;
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
    slots += (int64_t)kv.second.table.size() * a->block_size;
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
