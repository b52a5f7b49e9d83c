// Slot writes and copy-on-write block copies for the paged K/V pools.
//
// kv_write: every new token's K and V row goes to its slot, slot =
// block_table[logical block] * block_size + offset ("08. PagedAttention",
// section "why the name").  copy_blocks: a destination block becomes a copy
// of a shared source block before a sequence modifies it (intelliparadigm.com
// article, section 2.3).  Both are pure data movement; they are bound by HBM
// bandwidth and move 16 bytes per lane per access, consecutive lanes on
// consecutive bytes.
#include "common.h"
#include "kernels.h"

namespace pkv {

// One lane per 16-byte piece of a (token, kv head) row, pieces of a row on
// consecutive lanes: reads of k_new/v_new and writes into the block are both
// contiguous per row.
__global__ __launch_bounds__(256) void kv_write_kernel(const char* __restrict__ kn, const char* __restrict__ vn,
                                                       const int32_t* __restrict__ slots, int num_tokens,
                                                       char* __restrict__ kc, char* __restrict__ vc, int Hkv,
                                                       int log2B, int pieces_per_row, long long total_slots) {
  const int per_tok = Hkv * pieces_per_row;
  const long long total = (long long)num_tokens * per_tok;
  const size_t rowb = (size_t)pieces_per_row * 16;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int t = (int)(i / per_tok);
    const int rem = (int)(i - (long long)t * per_tok);
    const int h = rem / pieces_per_row;
    const int pc = rem - h * pieces_per_row;
    // the row loads do not depend on the slot: issue all three together
    const size_t src = ((size_t)t * Hkv + h) * rowb + (size_t)pc * 16;
    const uint4 kx = *(const uint4*)(kn + src);
    const uint4 vx = *(const uint4*)(vn + src);
    const int slot = slots[t];
    if (slot < 0 || slot >= total_slots) continue;
    const int blk = slot >> log2B;
    const int off = slot & ((1 << log2B) - 1);
    const size_t dst = ((((size_t)blk * Hkv + h) << log2B) + off) * rowb + (size_t)pc * 16;
    *(uint4*)(kc + dst) = kx;
    *(uint4*)(vc + dst) = vx;
  }
}

int launch_kv_write(const void* k_new, const void* v_new, const int32_t* slots, int num_tokens, void* k_cache,
                    void* v_cache, int num_blocks, int Hkv, int B, int D, int elem_bytes, hipStream_t stream) {
  if (num_tokens == 0) return 0;
  int log2B = 0;
  while ((1 << log2B) < B) ++log2B;
  const int ppr = D * elem_bytes / 16;
  const long long total = (long long)num_tokens * Hkv * ppr;
  const DeviceInfo& dev = device_info();
  long long grid = (total + 255) / 256;
  const long long cap = (long long)std::max(dev.num_cus, 1) * 16;
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (const char*)k_new,
                     (const char*)v_new, slots, num_tokens, (char*)k_cache, (char*)v_cache, Hkv, log2B, ppr,
                     (long long)num_blocks * B);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// grid.y walks the pairs; grid.x lanes stride over the block's bytes.  A
// block of one tensor is contiguous: [Hkv][B][D] elements.
__global__ __launch_bounds__(256) void copy_blocks_kernel(char* __restrict__ kc, char* __restrict__ vc,
                                                          const int32_t* __restrict__ pairs, int num_pairs,
                                                          int num_blocks, size_t block_bytes) {
  for (int p = blockIdx.y; p < num_pairs; p += gridDim.y) {
    const int src = pairs[2 * p];
    const int dst = pairs[2 * p + 1];
    if ((unsigned)src >= (unsigned)num_blocks || (unsigned)dst >= (unsigned)num_blocks) continue;
    const char* ks = kc + (size_t)src * block_bytes;
    const char* vs = vc + (size_t)src * block_bytes;
    char* kd = kc + (size_t)dst * block_bytes;
    char* vd = vc + (size_t)dst * block_bytes;
    for (size_t off = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 16; off < block_bytes;
         off += (size_t)gridDim.x * blockDim.x * 16) {
      const uint4 a = *(const uint4*)(ks + off);
      const uint4 b = *(const uint4*)(vs + off);
      *(uint4*)(kd + off) = a;
      *(uint4*)(vd + off) = b;
    }
  }
}

int launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int num_pairs, int num_blocks, int Hkv,
                       int B, int D, int elem_bytes, hipStream_t stream) {
  if (num_pairs == 0) return 0;
  const size_t block_bytes = (size_t)Hkv * B * D * elem_bytes;
  unsigned gx = (unsigned)std::min<size_t>((block_bytes / 16 + 255) / 256, 64);
  if (gx == 0) gx = 1;
  const unsigned gy = (unsigned)std::min(num_pairs, 65535);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(gx, gy), dim3(256), 0, stream, (char*)k_cache, (char*)v_cache, pairs,
                     num_pairs, num_blocks, block_bytes);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Swap of whole blocks between the device pools and caller-provided host
// memory (pinned, so the GPU reads and writes it directly over the bus):
// out: host[i] = cache[ids[i]]; in: cache[ids[i]] = host[i], for K and V.
// grid.y walks the blocks, grid.x lanes stride over a block's bytes.
template <bool OUT>
__global__ __launch_bounds__(256) void swap_blocks_kernel(char* __restrict__ kc, char* __restrict__ vc,
                                                          const int32_t* __restrict__ ids, int n, int num_blocks,
                                                          size_t block_bytes, char* __restrict__ hk,
                                                          char* __restrict__ hv) {
  for (int i = blockIdx.y; i < n; i += gridDim.y) {
    const int b = ids[i];
    if ((unsigned)b >= (unsigned)num_blocks) continue;
    char* dk = kc + (size_t)b * block_bytes;
    char* dv = vc + (size_t)b * block_bytes;
    char* pk = hk + (size_t)i * block_bytes;
    char* pv = hv + (size_t)i * block_bytes;
    for (size_t off = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 16; off < block_bytes;
         off += (size_t)gridDim.x * blockDim.x * 16) {
      if (OUT) {
        const uint4 x = *(const uint4*)(dk + off);
        const uint4 y = *(const uint4*)(dv + off);
        *(uint4*)(pk + off) = x;
        *(uint4*)(pv + off) = y;
      } else {
        const uint4 x = *(const uint4*)(pk + off);
        const uint4 y = *(const uint4*)(pv + off);
        *(uint4*)(dk + off) = x;
        *(uint4*)(dv + off) = y;
      }
    }
  }
}

int launch_swap_blocks(bool out, void* k_cache, void* v_cache, const int32_t* ids, int n, int num_blocks, int Hkv,
                       int B, int D, int elem_bytes, void* host_k, void* host_v, hipStream_t stream) {
  if (n == 0) return 0;
  const size_t block_bytes = (size_t)Hkv * B * D * elem_bytes;
  unsigned gx = (unsigned)std::min<size_t>((block_bytes / 16 + 255) / 256, 64);
  if (gx == 0) gx = 1;
  const unsigned gy = (unsigned)std::min(n, 65535);
  if (out)
    hipLaunchKernelGGL(swap_blocks_kernel<true>, dim3(gx, gy), dim3(256), 0, stream, (char*)k_cache,
                       (char*)v_cache, ids, n, num_blocks, block_bytes, (char*)host_k, (char*)host_v);
  else
    hipLaunchKernelGGL(swap_blocks_kernel<false>, dim3(gx, gy), dim3(256), 0, stream, (char*)k_cache,
                       (char*)v_cache, ids, n, num_blocks, block_bytes, (char*)host_k, (char*)host_v);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Read-only gather of whole units: every listed unit of `unit_bytes` of pool
// a (and of pool b, when given) is read once with 16-byte non-temporal
// loads and folded into one word per wavefront, with no other arithmetic.
// This is the access pattern of the decode (block-table lookups, then
// contiguous runs of K and V) without its computation, so its rate is the
// bandwidth ceiling that pattern can reach on the device.
//
// The units are cut into items of P KiB (P = min(4, unit KiB)); wavefront w
// takes an equal contiguous share of the items.  Unit ids come through the
// scalar cache, so waiting for an id never waits for the data loads (vector
// loads complete in order), and the loads of an item are issued
// unconditionally (an id outside the pool reads unit 0), so the compiler
// keeps them in the registers they are folded from instead of copying them
// there, which would wait for every load in flight.  One item per wavefront
// is in flight while the previous one is folded; eight wavefronts per
// compute unit (two workgroups) was the fastest shape of a sweep over 4..32
// wavefronts and 1..4 items in flight.
__device__ __forceinline__ uint4 gather_load(const void* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(t.x, t.y, t.z, t.w);
}

typedef __attribute__((address_space(4))) const int32_t sconst_i32_gather;

template <int P, bool TWO>
__global__ __launch_bounds__(256) void gather_units_kernel(const char* __restrict__ pa, const char* __restrict__ pb,
                                                           const int32_t* __restrict__ ids, long long n_items,
                                                           int log2_ipu, long long unit_bytes, long long pool_units,
                                                           uint32_t* __restrict__ sink) {
  constexpr int NL = TWO ? 2 * P : P;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const long long nw = (long long)gridDim.x * 4;
  const long long per = (n_items + nw - 1) / nw;
  const long long i0 = (long long)w * per;
  const long long i1 = i0 + per < n_items ? i0 + per : n_items;
  uint32_t acc = 0;
  if (i0 < i1) {
    uint4 r[NL];
    auto issue = [&](long long i) {
      const int id = ((sconst_i32_gather*)ids)[i >> log2_ipu];
      const long long uid = (unsigned long long)id < (unsigned long long)pool_units ? id : 0;
      const size_t off = (size_t)uid * (size_t)unit_bytes + (size_t)(i & ((1 << log2_ipu) - 1)) * (P * 1024) +
                         (size_t)lane * 16;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        r[p] = gather_load(pa + off + p * 1024);
        if constexpr (TWO) r[P + p] = gather_load(pb + off + p * 1024);
      }
    };
    auto fold = [&]() {
#pragma unroll
      for (int p = 0; p < NL; ++p) acc ^= r[p].x ^ r[p].y ^ r[p].z ^ r[p].w;
    };
    issue(i0);
    for (long long i = i0 + 1; i < i1; ++i) {
      fold();
      __builtin_amdgcn_sched_barrier(0);  // fold, then issue: the order that keeps one item in flight
      issue(i);
      __builtin_amdgcn_sched_barrier(0);
    }
    fold();
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) acc ^= __shfl_xor(acc, m);
  if (lane == 0) sink[w] = acc;
}

int launch_gather_units(const void* pool_a, const void* pool_b, const int32_t* ids, int n_units, int unit_kib,
                        long long pool_units, void* sink, int sink_words, hipStream_t stream) {
  int l = 0;
  while ((1 << l) < unit_kib) ++l;
  const int P = unit_kib < 4 ? unit_kib : 4;
  const int log2_ipu = unit_kib < 4 ? 0 : l - 2;
  const long long n_items = (long long)n_units << log2_ipu;
  const long long unit_bytes = (long long)unit_kib * 1024;
  const DeviceInfo& dev = device_info();
  const long long waves = std::min<long long>((long long)std::max(dev.num_cus, 1) * 8, sink_words);
  const int grid = (int)std::max<long long>(waves / 4, 1);
  const char* a = (const char*)pool_a;
  const char* b = (const char*)pool_b;
  uint32_t* sk = (uint32_t*)sink;
#define PKV_GATHER(PP)                                                                                        \
  if (P == PP) {                                                                                              \
    if (b)                                                                                                    \
      hipLaunchKernelGGL((gather_units_kernel<PP, true>), dim3(grid), dim3(256), 0, stream, a, b, ids, n_items, \
                         log2_ipu, unit_bytes, pool_units, sk);                                              \
    else                                                                                                      \
      hipLaunchKernelGGL((gather_units_kernel<PP, false>), dim3(grid), dim3(256), 0, stream, a, b, ids,        \
                         n_items, log2_ipu, unit_bytes, pool_units, sk);                                     \
  }
  PKV_GATHER(1)
  PKV_GATHER(2)
  PKV_GATHER(4)
#undef PKV_GATHER
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace pkv
