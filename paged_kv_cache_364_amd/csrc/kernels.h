// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Every launcher validates nothing beyond what its kernel needs; the C ABI
// checks arguments first.  Launchers return 0 or a PKV_ERR_* code.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace pkv {

struct DeviceInfo {
  int device = -1;
  int num_cus = 0;
  bool ok = false;
};

// Properties of the current device (queried once per device).
const DeviceInfo& device_info();

// Integer tuning knob from the environment (read at each call), or dflt.
int tuning_int(const char* name, int dflt);

// Workgroups of `threads` threads of `kernel` that fit on one compute unit of
// the current device (at least 1), queried once per device and kernel.
int occupancy(const void* kernel, int threads);

int launch_kv_write(const void* k_new, const void* v_new, const int32_t* slots, int num_tokens, void* k_cache,
                    void* v_cache, int num_blocks, int Hkv, int B, int D, int elem_bytes, hipStream_t stream);

int launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int num_pairs, int num_blocks, int Hkv,
                       int B, int D, int elem_bytes, hipStream_t stream);

int launch_swap_blocks(bool out, void* k_cache, void* v_cache, const int32_t* ids, int n, int num_blocks, int Hkv,
                       int B, int D, int elem_bytes, void* host_k, void* host_v, hipStream_t stream);

int launch_gather_units(const void* pool_a, const void* pool_b, const int32_t* ids, int n_units, int unit_kib,
                        long long pool_units, void* sink, int sink_words, hipStream_t stream);

bool decode_supported(int dtype, int head_dim, int group);
size_t decode_workspace_bytes(int dtype, int D, int G, int S, int Hkv, int max_blocks, int B);
// k_new / v_new non-null: the append variant (window must be 0).
int launch_decode(void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* tables,
                  int max_blocks, const int32_t* ctx, int S, int Hq, int Hkv, int D, int B, int num_blocks,
                  int window, float scale, int dtype, void* ws, size_t ws_bytes, hipStream_t stream,
                  const void* k_new = nullptr, const void* v_new = nullptr);

// Size of the library's own decode scratch array (per GPU).
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
int launch_decode_scratch(void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* tables,
                          int max_blocks, const int32_t* ctx, int S, int Hq, int Hkv, int D, int B, int num_blocks,
                          float scale, int dtype, hipStream_t stream);

bool decode_shared_supported(int dtype, int head_dim, int group, int block_size);
int max_shared_members(int group);
int launch_decode_shared(void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* tables,
                         int max_blocks, const int32_t* ctx, int S, const int32_t* group_start,
                         const int32_t* shared_blocks, int num_groups, int Hq, int Hkv, int D, int B, int num_blocks,
                         float scale, hipStream_t stream);

bool prefill_supported(int dtype, int head_dim, int group, int block_size);
int launch_prefill(void* out, const void* q, const int32_t* cu_q_lens, int total_q, int max_q_len,
                   const void* k_cache, const void* v_cache, const int32_t* tables, int max_blocks,
                   const int32_t* ctx, int S, int Hq, int Hkv, int D, int B, int num_blocks, float scale,
                   hipStream_t stream);

}  // namespace pkv
