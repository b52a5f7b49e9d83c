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
// bandwidth ceiling that pattern can reach on the device.  Persistent grid
// of six 4-wavefront workgroups per compute unit (the fastest shape of a
// sweep over 2..12): wavefront w takes an equal contiguous share of the
// 1 KiB pieces of all units; a window of 64 unit ids is held in a register,
// and the loads of the next four pieces (of each pool) are in flight while
// the current four are folded.
__device__ __forceinline__ uint4 gather_load(const void* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(t.x, t.y, t.z, t.w);
}

__global__ __launch_bounds__(256) void gather_units_kernel(const char* __restrict__ pa, const char* __restrict__ pb,
                                                           const int32_t* __restrict__ ids, int n_units,
                                                           int log2_ppu, long long pool_units,
                                                           uint32_t* __restrict__ sink) {
  constexpr int DEPTH = 4;
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nw = gridDim.x * 4;
  const long long total = (long long)n_units << log2_ppu;
  const long long per = (total + nw - 1) / nw;
  const long long k0 = (long long)w * per;
  const long long k1 = k0 + per < total ? k0 + per : total;
  uint32_t acc = 0;
  if (k0 < k1) {
    const size_t ub = (size_t)1024 << log2_ppu;
    long long wu = k0 >> log2_ppu;  // first unit of the id window
    int win = wu + lane < n_units ? ids[wu + lane] : -1;
    auto addr = [&](const char* base, long long k, int id) -> const char* {
      return base + (size_t)id * ub + (size_t)(k & ((1 << log2_ppu) - 1)) * 1024 + lane * 16;
    };
    auto issue = [&](long long k, uint4 (&ra)[DEPTH], uint4 (&rb)[DEPTH]) {
#pragma unroll
      for (int j = 0; j < DEPTH; ++j) {
        const long long kk = k + j;
        ra[j] = make_uint4(0, 0, 0, 0);
        rb[j] = make_uint4(0, 0, 0, 0);
        if (kk < k1) {
          const long long u = kk >> log2_ppu;
          if (u - wu >= 64) {  // slide the window (wave-uniform)
            wu = u;
            win = wu + lane < n_units ? ids[wu + lane] : -1;
          }
          const int id = __builtin_amdgcn_readlane(win, (int)(u - wu));
          if ((unsigned long long)id < (unsigned long long)pool_units) {
            ra[j] = gather_load(addr(pa, kk, id));
            if (pb) rb[j] = gather_load(addr(pb, kk, id));
          }
        }
      }
    };
    uint4 xa[DEPTH], xb[DEPTH], ya[DEPTH], yb[DEPTH];
    issue(k0, xa, xb);
    for (long long k = k0; k < k1; k += 2 * DEPTH) {
      issue(k + DEPTH, ya, yb);
#pragma unroll
      for (int j = 0; j < DEPTH; ++j) acc ^= xa[j].x ^ xa[j].y ^ xa[j].z ^ xa[j].w ^ xb[j].x ^ xb[j].y ^ xb[j].z ^ xb[j].w;
      if (k + DEPTH >= k1) break;
      issue(k + 2 * DEPTH, xa, xb);
#pragma unroll
      for (int j = 0; j < DEPTH; ++j) acc ^= ya[j].x ^ ya[j].y ^ ya[j].z ^ ya[j].w ^ yb[j].x ^ yb[j].y ^ yb[j].z ^ yb[j].w;
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) acc ^= __shfl_xor(acc, m);
  if (lane == 0) sink[w] = acc;
}

int launch_gather_units(const void* pool_a, const void* pool_b, const int32_t* ids, int n_units, int unit_kib,
                        long long pool_units, void* sink, int sink_words, hipStream_t stream) {
  int l = 0;
  while ((1 << l) < unit_kib) ++l;
  const DeviceInfo& dev = device_info();
  const long long waves = std::min<long long>((long long)std::max(dev.num_cus, 1) * 6 * 4, sink_words);
  const int grid = (int)std::max<long long>(waves / 4, 1);
  hipLaunchKernelGGL(gather_units_kernel, dim3(grid), dim3(256), 0, stream, (const char*)pool_a,
                     (const char*)pool_b, ids, n_units, l, pool_units, (uint32_t*)sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace pkv
