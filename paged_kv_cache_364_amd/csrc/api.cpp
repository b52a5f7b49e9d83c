// The C ABI: argument checks on the host, then a launch on the caller's
// stream.  Declarations and their contracts are in include/pagedkv.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>
#include <vector>

#include "../../include/pagedkv.h"
#include "kernels.h"

static_assert(PKV_DECODE_SCRATCH_BYTES == pkv::kDecodeScratchBytes, "header and library disagree on the scratch size");

namespace pkv {

const DeviceInfo& device_info() {
  static DeviceInfo infos[64];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    static DeviceInfo none;
    return none;
  }
  std::lock_guard<std::mutex> lock(mu);
  DeviceInfo& d = infos[dev];
  if (!d.ok) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0) {
      d.device = dev;
      d.num_cus = cus;
      d.ok = true;
    }
  }
  return d;
}

int occupancy(const void* kernel, int threads) {
  struct Entry {
    int dev;
    const void* kernel;
    int threads;
    int blocks;
  };
  static std::vector<Entry> known;
  static std::mutex mu;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  std::lock_guard<std::mutex> lock(mu);
  for (const Entry& e : known)
    if (e.dev == dev && e.kernel == kernel && e.threads == threads) return e.blocks;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n < 1) return 1;
  known.push_back({dev, kernel, threads, n});
  return n;
}

int tuning_int(const char* name, int dflt) {
  const char* v = getenv(name);
  if (!v || !*v) return dflt;
  char* end = nullptr;
  const long x = strtol(v, &end, 10);
  return (end && *end == 0) ? (int)x : dflt;
}

}  // namespace pkv

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int elem_bytes(int dtype) { return dtype == PKV_DTYPE_F32 ? 4 : dtype == PKV_DTYPE_BF16 ? 2 : 0; }

bool head_dim_ok(int D) { return D == 16 || D == 32 || D == 64 || D == 128; }
bool block_ok(int B) { return pow2(B) && B <= 256; }

// Common checks of the cache geometry.
int check_cache(int num_blocks, int Hkv, int B, int D, int dtype) {
  if (num_blocks <= 0 || Hkv <= 0 || B <= 0 || D <= 0) return PKV_ERR_INVALID;
  if (!elem_bytes(dtype) || !head_dim_ok(D) || !block_ok(B)) return PKV_ERR_UNSUPPORTED;
  if ((long long)num_blocks * B > INT32_MAX) return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PKV_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case PKV_ERR_NO_BLOCKS: return "not enough free blocks";
    case PKV_ERR_STATE: return "allocator state error";
    case PKV_ERR_HIP: return "HIP runtime error";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

int pkv_kv_write(const void* k_new, const void* v_new, const int32_t* slot_mapping, int num_tokens, void* k_cache,
                 void* v_cache, int num_blocks, int num_kv_heads, int block_size, int head_dim, int dtype,
                 void* stream) {
  int st = check_cache(num_blocks, num_kv_heads, block_size, head_dim, dtype);
  if (st) return st;
  if (num_tokens < 0) return PKV_ERR_INVALID;
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PKV_ERR_INVALID;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned4(slot_mapping))
    return PKV_ERR_ALIGN;
  return pkv::launch_kv_write(k_new, v_new, slot_mapping, num_tokens, k_cache, v_cache, num_blocks, num_kv_heads,
                              block_size, head_dim, elem_bytes(dtype), (hipStream_t)stream);
}

int pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int num_pairs, int num_blocks,
                    int num_kv_heads, int block_size, int head_dim, int dtype, void* stream) {
  int st = check_cache(num_blocks, num_kv_heads, block_size, head_dim, dtype);
  if (st) return st;
  if (num_pairs < 0) return PKV_ERR_INVALID;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !pairs) return PKV_ERR_INVALID;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned4(pairs)) return PKV_ERR_ALIGN;
  return pkv::launch_copy_blocks(k_cache, v_cache, pairs, num_pairs, num_blocks, num_kv_heads, block_size, head_dim,
                                 elem_bytes(dtype), (hipStream_t)stream);
}

static int swap_blocks(bool out, void* k_cache, void* v_cache, const int32_t* block_ids, int num, int num_blocks,
                       int num_kv_heads, int block_size, int head_dim, int dtype, void* host_k, void* host_v,
                       void* stream) {
  int st = check_cache(num_blocks, num_kv_heads, block_size, head_dim, dtype);
  if (st) return st;
  if (num < 0) return PKV_ERR_INVALID;
  if (num == 0) return PKV_OK;
  if (!k_cache || !v_cache || !block_ids || !host_k || !host_v) return PKV_ERR_INVALID;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(host_k) || !aligned16(host_v) ||
      !aligned4(block_ids))
    return PKV_ERR_ALIGN;
  return pkv::launch_swap_blocks(out, k_cache, v_cache, block_ids, num, num_blocks, num_kv_heads, block_size,
                                 head_dim, elem_bytes(dtype), host_k, host_v, (hipStream_t)stream);
}

int pkv_swap_out(const void* k_cache, const void* v_cache, const int32_t* block_ids, int num, int num_blocks,
                 int num_kv_heads, int block_size, int head_dim, int dtype, void* host_k, void* host_v,
                 void* stream) {
  return swap_blocks(true, const_cast<void*>(k_cache), const_cast<void*>(v_cache), block_ids, num, num_blocks,
                     num_kv_heads, block_size, head_dim, dtype, host_k, host_v, stream);
}

int pkv_swap_in(void* k_cache, void* v_cache, const int32_t* block_ids, int num, int num_blocks, int num_kv_heads,
                int block_size, int head_dim, int dtype, const void* host_k, const void* host_v, void* stream) {
  return swap_blocks(false, k_cache, v_cache, block_ids, num, num_blocks, num_kv_heads, block_size, head_dim, dtype,
                     const_cast<void*>(host_k), const_cast<void*>(host_v), stream);
}

static int check_attention(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                           int num_blocks, int max_blocks, int dtype) {
  int st = check_cache(num_blocks, num_kv_heads, block_size, head_dim, dtype);
  if (st) return st;
  if (num_seqs < 0 || num_heads <= 0 || max_blocks <= 0) return PKV_ERR_INVALID;
  if (num_heads % num_kv_heads) return PKV_ERR_INVALID;
  if ((long long)max_blocks * block_size > INT32_MAX) return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

size_t pkv_decode_workspace_size(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                                 int max_blocks_per_seq, int dtype) {
  if (num_kv_heads <= 0) return 0;
  if (check_attention(num_seqs, num_heads, num_kv_heads, head_dim, block_size, 1, max_blocks_per_seq, dtype))
    return 0;
  const int G = num_heads / num_kv_heads;
  if (!pkv::decode_supported(dtype, head_dim, G)) return 0;
  if (num_seqs == 0) return 256;
  return pkv::decode_workspace_bytes(dtype, head_dim, G, num_seqs, num_kv_heads, max_blocks_per_seq, block_size);
}

static int decode_call(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                       int num_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks, int window,
                       float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream,
                       const void* k_new = nullptr, const void* v_new = nullptr) {
  if (num_kv_heads <= 0) return PKV_ERR_INVALID;
  int st = check_attention(num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                           dtype);
  if (st) return st;
  const int G = num_heads / num_kv_heads;
  if (!pkv::decode_supported(dtype, head_dim, G)) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PKV_ERR_INVALID;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned4(block_tables) ||
      !aligned4(context_lens) || (workspace && !aligned16(workspace)))
    return PKV_ERR_ALIGN;
  if ((k_new != nullptr) != (v_new != nullptr)) return PKV_ERR_INVALID;
  if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return PKV_ERR_ALIGN;
  return pkv::launch_decode(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                            num_heads, num_kv_heads, head_dim, block_size, num_blocks, window, scale, dtype,
                            workspace, workspace_bytes, (hipStream_t)stream, k_new, v_new);
}

int pkv_paged_attention_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                               int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                               int num_blocks, float scale, int dtype, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return decode_call(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, 0, scale, dtype, workspace, workspace_bytes,
                     stream);
}

int pkv_paged_attention_decode_append(void* out, const void* q, const void* k_new, const void* v_new,
                                      void* k_cache, void* v_cache, const int32_t* block_tables,
                                      int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                                      int num_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                      float scale, int dtype, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new)) return PKV_ERR_INVALID;
  return decode_call(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, 0, scale, dtype, workspace, workspace_bytes,
                     stream, k_new, v_new);
}

int pkv_paged_attention_decode_window(void* out, const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, int max_blocks_per_seq,
                                      const int32_t* context_lens, int num_seqs, int num_heads, int num_kv_heads,
                                      int head_dim, int block_size, int num_blocks, int window, float scale,
                                      int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (window <= 0) return PKV_ERR_INVALID;
  return decode_call(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, window, scale, dtype, workspace,
                     workspace_bytes, stream);
}

int pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, int max_blocks_per_seq,
                                       const int32_t* context_lens, int num_seqs, int num_heads, int num_kv_heads,
                                       int head_dim, int block_size, int num_blocks, float scale, int dtype,
                                       void* stream) {
  if (num_kv_heads <= 0) return PKV_ERR_INVALID;
  int st = check_attention(num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                           dtype);
  if (st) return st;
  if (!pkv::decode_supported(dtype, head_dim, num_heads / num_kv_heads)) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PKV_ERR_INVALID;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned4(block_tables) ||
      !aligned4(context_lens))
    return PKV_ERR_ALIGN;
  return pkv::launch_decode_scratch(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                                    num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                                    (hipStream_t)stream);
}

int pkv_decode_shared_max_members(int num_heads, int num_kv_heads) {
  if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads) return 0;
  return pkv::max_shared_members(num_heads / num_kv_heads);
}

int pkv_paged_attention_decode_shared(void* out, const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, int max_blocks_per_seq,
                                      const int32_t* context_lens, int num_seqs, const int32_t* group_start,
                                      const int32_t* shared_blocks, int num_groups, int num_heads, int num_kv_heads,
                                      int head_dim, int block_size, int num_blocks, float scale, int dtype,
                                      void* stream) {
  if (num_kv_heads <= 0) return PKV_ERR_INVALID;
  int st = check_attention(num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                           dtype);
  if (st) return st;
  if (num_groups < 0 || num_groups > num_seqs) return PKV_ERR_INVALID;
  if (!pkv::decode_shared_supported(dtype, head_dim, num_heads / num_kv_heads, block_size))
    return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (num_groups == 0) return PKV_ERR_INVALID;  // groups must cover the batch
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !group_start || !shared_blocks)
    return PKV_ERR_INVALID;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned4(block_tables) ||
      !aligned4(context_lens) || !aligned4(group_start) || !aligned4(shared_blocks))
    return PKV_ERR_ALIGN;
  return pkv::launch_decode_shared(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                                   group_start, shared_blocks, num_groups, num_heads, num_kv_heads, head_dim,
                                   block_size, num_blocks, scale, (hipStream_t)stream);
}

int pkv_gather_units(const void* pool_a, const void* pool_b, const int32_t* unit_ids, int num_units, int unit_kib,
                     int64_t pool_units, void* sink, int sink_words, void* stream) {
  if (num_units < 0 || pool_units <= 0 || sink_words < 4) return PKV_ERR_INVALID;
  if (!pow2(unit_kib) || unit_kib > 4096) return PKV_ERR_UNSUPPORTED;
  if (num_units == 0) return PKV_OK;
  if (!pool_a || !unit_ids || !sink) return PKV_ERR_INVALID;
  if (!aligned16(pool_a) || (pool_b && !aligned16(pool_b)) || !aligned4(unit_ids) || !aligned4(sink))
    return PKV_ERR_ALIGN;
  return pkv::launch_gather_units(pool_a, pool_b, unit_ids, num_units, unit_kib, (long long)pool_units, sink,
                                  sink_words, (hipStream_t)stream);
}

int pkv_paged_attention_prefill(void* out, const void* q, const int32_t* cu_q_lens, int total_q, int max_q_len,
                                const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                int max_blocks_per_seq, const int32_t* context_lens, int num_seqs, int num_heads,
                                int num_kv_heads, int head_dim, int block_size, int num_blocks, float scale,
                                int dtype, void* stream) {
  if (num_kv_heads <= 0) return PKV_ERR_INVALID;
  int st = check_attention(num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                           dtype);
  if (st) return st;
  if (total_q < 0 || max_q_len < 0) return PKV_ERR_INVALID;
  const int G = num_heads / num_kv_heads;
  if (!pkv::prefill_supported(dtype, head_dim, G, block_size)) return PKV_ERR_UNSUPPORTED;
  // the prefill loads index pool rows (block, head, slot) in 32 bits
  if ((uint64_t)num_blocks * (uint64_t)num_kv_heads * (uint64_t)block_size > 0xffffffffull)
    return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0 || total_q == 0) return PKV_OK;
  if (max_q_len == 0) return PKV_ERR_INVALID;  // total_q > 0: some chunk has a row
  if (!out || !q || !cu_q_lens || !k_cache || !v_cache || !block_tables || !context_lens) return PKV_ERR_INVALID;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned4(block_tables) ||
      !aligned4(context_lens) || !aligned4(cu_q_lens))
    return PKV_ERR_ALIGN;
  return pkv::launch_prefill(out, q, cu_q_lens, total_q, max_q_len, k_cache, v_cache, block_tables,
                             max_blocks_per_seq, context_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                             block_size, num_blocks, scale, (hipStream_t)stream);
}

}  // extern "C"
