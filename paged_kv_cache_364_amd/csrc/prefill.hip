// Paged prefill attention for gfx950 on the matrix cores.
//
// A chunk of C new query tokens per sequence attends, causally, to the
// sequence's cached prefix plus the chunk itself, all read through the
// block table (cnblogs "paged attention", section 5: position -> logical
// block -> physical block).  Scores are computed block-wise and partial
// results are merged as they go (intelliparadigm.com article, section 2.2),
// here with the running-max online softmax, so the result is the plain
// softmax(scale * Q K^T) V of the pages (cnblogs section 6).
//
// Tiling.  A workgroup of eight wavefronts computes BM = 256 query rows of
// one (sequence, head) at a time; wavefront w owns rows 32w .. 32w + 31.
// Keys and values are walked in tiles of KT = 64 tokens (several physical
// blocks gathered through the table), moved from global memory straight
// into LDS (global_load_lds) and triple-buffered there: the transfers of
// tile j + 2 are in flight while tile j is computed.  The query rows sit in
// LDS too, laid out like a K tile.
//
// Schedule.  The grid is persistent, one workgroup per compute unit.  A
// workgroup walks its share of the (sequence, head, q tile) items as one
// stream of key tiles, so the transfers run on across the end of an item
// and the next item's query rows load while the current item's last tile
// is computed: no workgroup start-up or drain between items.
//
// Per tile and wavefront:
//
//   S^T = K Q^T   on v_mfma_f32_32x32x16_bf16, A = K rows from LDS, B = the
//                 wavefront's query rows from LDS.  The accumulator layout
//                 puts query l % 32 on lane l
//                 and 16 keys in its registers, so the online-softmax state
//                 (running max, running sum) of a query lives in one lane
//                 pair (l, l ^ 32).
//   O^T += V^T P^T  A = V^T, B = P^T taken straight from the S^T
//                 accumulators (converted to bf16): the keys a lane holds
//                 in registers are the contraction index the B operand
//                 wants, so the A operand must hold the same keys of one
//                 column d of V, in that order.  V stays row-major in LDS
//                 and the transposing LDS read (ds_read_b64_tr_b16) builds
//                 those fragments.
//
// A matrix-core contraction sums over its k index in any order, so the
// assignment of keys (for O^T) or head dimensions (for S^T) to registers
// only has to agree between the two operands; rows and columns follow the
// documented 32x32 accumulator layout (lane l holds column l % 32 and rows
// 8 * (r / 4) + 4 * (l / 32) + r % 4 of register r).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace pkv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

struct PrefillArgs {
  uint16_t* out;
  const uint16_t* q;
  const int32_t* cu_q_lens;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* tables;
  const int32_t* ctx_lens;
  int S, Hq, Hkv, G, max_blocks, num_blocks, log2B, q_tiles;
  float scale_log2;
};

constexpr int kPWaves = 8;                 // wavefronts per workgroup, 32 query rows each
constexpr int kPBM = 32 * kPWaves;         // query rows per workgroup
constexpr int kPKT = 64;                   // keys per tile
constexpr int kPThreads = 64 * kPWaves;

template <int D>
struct PShape {
  static constexpr int KS = D / 16;                   // contraction steps of S^T
  static constexpr int DT = D / 32;                   // 32-row tiles of O^T
  static constexpr int PIECES = D / 8;                // 16-byte pieces per row
  static constexpr int ROWB = D * 2;                  // bytes per K or V row
  static constexpr int TILEB = kPKT * ROWB;           // bytes per tile and tensor
  static constexpr int DMA_PER_WAVE = TILEB / 1024 / kPWaves;  // 1 KiB transfers per wavefront and tensor
  static_assert(DMA_PER_WAVE >= 1 && DMA_PER_WAVE * 1024 * kPWaves == TILEB, "tile split");
};

// LDS layout of a K or V tile: row-major, 16-byte piece p of key `key` in
// slot key * PIECES + (p ^ swz(key)).  The XOR spreads over all banks both
// the K fragment reads (one piece of 16 consecutive keys per 16 lanes) and
// the transposed V reads (4 pieces of 4 consecutive keys per 32 lanes).
template <int D>
__device__ __forceinline__ int swz(int key) {
  if constexpr (D == 128)
    return ((key & 3) << 2) | ((key >> 2) & 3);
  else
    return (((key >> 1) & 1) << 2) | ((key >> 2) & 3);
}

// Rows for keys with no data: zeros past the context; for a block id outside
// the pool, a NaN key row and a zero value row, so exactly the query rows
// that attend such a key come out NaN (a masked key's weight is 0, and
// 0 times a zero value row stays 0).
__device__ __attribute__((aligned(16))) uint16_t g_pf_zero_row[128];
__device__ __attribute__((aligned(16))) uint16_t g_pf_nan_row[128] = {0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0, 0x7fc0};

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2v_t;

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  bf16x2v_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Workgroup barrier for the tile pipeline: this wavefront first waits until
// at most N of its vector-memory operations are outstanding (the transfers
// of the tile after next) and all its LDS operations are done, then meets
// the others.  In the loop LDS is written only by the transfers and every
// LDS read is consumed before the barrier, so no memory fence is needed:
// a fence would also wait for the transfers still in flight.  The signal
// fences only keep the compiler from moving memory accesses across.
template <int N>
__device__ __forceinline__ void tile_barrier() {
  static_assert(N < 64, "vmcnt range");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));  // vmcnt(N) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One 16-byte global -> LDS transfer per lane (global_load_lds_dwordx4):
// lane l's bytes land at dst + 16 l, dst the same for the whole wavefront.
// Written as assembly so that the compiler's wait-count pass, which cannot
// tell which LDS buffer such a transfer writes, adds no wait for it before
// every LDS read; tile_barrier waits for the transfers explicitly.
// The LDS destination is an LDS byte address (lds_addr of an LDS array),
// which stays a 32-bit constant: a generic pointer would be carried in a
// register pair and converted at every transfer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_void_t*)p; }

__device__ __forceinline__ void lds_dma16(const void* src, uint32_t dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(dst);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off"
      :
      : "s"(m0), "v"(src)
      : "memory", "m0");
}

// The same transfer with a wavefront-uniform 64-bit base in SGPRs and a
// 32-bit per-lane byte offset (the instruction's saddr form).
__device__ __forceinline__ void lds_dma16_s(const void* sbase, uint32_t voff, uint32_t dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(dst);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(m0), "v"(voff), "s"(sbase)
      : "memory", "m0");
}

typedef __attribute__((address_space(4))) const int32_t const_i32_t;

// Table entry i of a row, read through the scalar cache when i is the same
// for the whole wavefront (the table does not change during the kernel).
__device__ __forceinline__ int table_entry(const int32_t* trow, int i) { return ((const_i32_t*)trow)[i]; }

// Transfer g of tile t0 .. t0 + 63 in the general form: every lane finds
// its own key, block and source.  Used only when a block holds fewer keys
// than one transfer covers.  The entry is read with its index clamped into
// the row, and a key past the context reads the zero row whatever the entry
// holds.
template <int D>
__device__ __forceinline__ void dma_lanes(const PrefillArgs& a, const int32_t* trow, int kvh, int t0, int ctx, int g,
                                          int lane, uint32_t kdst, uint32_t vdst) {
  using PS = PShape<D>;
  const int sl = g * 64 + lane;  // 16-byte slot
  const int key = sl / PS::PIECES;
  const int p = (sl % PS::PIECES) ^ swz<D>(key);
  const int t = t0 + key;
  const bool in_ctx = t < ctx;
  const int blk = trow[min(t >> a.log2B, a.max_blocks - 1)];
  const bool outside = (unsigned)blk >= (unsigned)a.num_blocks;
  const uint32_t row =
      (((uint32_t)blk * (uint32_t)a.Hkv + (uint32_t)kvh) << a.log2B) + (uint32_t)(t & ((1 << a.log2B) - 1));
  const size_t off = (size_t)row * D + p * 8;
  const bool real = in_ctx && !outside;
  // used when !real: a key of a block outside the pool scores NaN (its V is
  // zero, so a row whose causal mask drops that key is unaffected)
  const uint16_t* kfill = in_ctx ? g_pf_nan_row + p * 8 : g_pf_zero_row + p * 8;
  const uint16_t* ksrc = real ? a.k_cache + off : kfill;
  const uint16_t* vsrc = real ? a.v_cache + off : g_pf_zero_row + p * 8;
  lds_dma16(ksrc, kdst + g * 1024);
  lds_dma16(vsrc, vdst + g * 1024);
}

// Per-lane byte offset of transfer g inside its block, from the block's row
// (t0 mod B): the same for every tile, so it is computed once.  A transfer
// covers 64 / PIECES consecutive keys, which lie in one block when the
// block holds at least that many.
template <int D>
__device__ __forceinline__ uint32_t dma_lane_offset(int g, int lane, int log2B) {
  using PS = PShape<D>;
  const int sl = g * 64 + lane;
  const int key = sl / PS::PIECES;
  const int p = (sl % PS::PIECES) ^ swz<D>(key);
  return (uint32_t)(((key & ((1 << log2B) - 1)) * D + p * 8) * 2);
}

// Block ids of this wavefront's transfers of tile t0 (one per transfer;
// index clamped into the row, so an entry past the table is never read).
template <int D>
struct TileEntries {
  int e[PShape<D>::DMA_PER_WAVE];
};
template <int D>
__device__ __forceinline__ TileEntries<D> tile_entries(const PrefillArgs& a, const int32_t* trow, int t0, int wave) {
  using PS = PShape<D>;
  constexpr int KPX = 64 / PS::PIECES;
  TileEntries<D> r;
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // uniform: a scalar load
#pragma unroll
  for (int i = 0; i < PS::DMA_PER_WAVE; ++i) {
    const int g = wv * PS::DMA_PER_WAVE + i;
    r.e[i] = table_entry(trow, min((t0 + g * KPX) >> a.log2B, a.max_blocks - 1));
  }
  return r;
}

// Issue the transfers of tile t0 .. t0 + 63 straight into LDS (K to kdst,
// V to vdst): each 1 KiB transfer of a wavefront fills 64 consecutive
// slots, lane l slot l, from the global piece that the swizzle puts there.
// When a block holds at least the 64 / PIECES keys of a transfer, the
// transfer's block id (ent, read ahead through the scalar cache) gives the
// block's address in SGPRs and the lanes add their fixed offsets (voff).
// Keys past the context read the zero row; a block id outside the pool
// reads the NaN row for K and the zero row for V.  Those cases pick a source
// per lane.
template <int D>
__device__ __forceinline__ void dma_tile(const PrefillArgs& a, const int32_t* trow, const TileEntries<D>& ent,
                                         int kvh, int t0, int ctx, int wave, int lane, const uint32_t* voff,
                                         uint32_t kdst, uint32_t vdst) {
  using PS = PShape<D>;
  constexpr int KPX = 64 / PS::PIECES;  // keys per transfer
  const bool whole = t0 + kPKT <= ctx;
#pragma unroll
  for (int i = 0; i < PS::DMA_PER_WAVE; ++i) {
    const int g = wave * PS::DMA_PER_WAVE + i;  // 1 KiB chunk of the tile
    if ((1 << a.log2B) < KPX) {
      dma_lanes<D>(a, trow, kvh, t0, ctx, g, lane, kdst, vdst);
      continue;
    }
    const int blk = ent.e[i];
    const bool valid = (unsigned)blk < (unsigned)a.num_blocks;
    const uint32_t row0 =
        (((uint32_t)blk * (uint32_t)a.Hkv + (uint32_t)kvh) << a.log2B) + (uint32_t)(t0 & ((1 << a.log2B) - 1));
    const size_t boff = (size_t)row0 * PS::ROWB;
    if (whole && valid) {
      lds_dma16_s((const uint8_t*)a.k_cache + boff, voff[i], kdst + g * 1024);
      lds_dma16_s((const uint8_t*)a.v_cache + boff, voff[i], vdst + g * 1024);
    } else {
      // an opaque copy of the lane index keeps the compiler from hoisting
      // this rarely taken path's per-lane values out of the loop
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int sl = g * 64 + ln;
      const int key = sl / PS::PIECES;
      const int p = (sl % PS::PIECES) ^ swz<D>(key);
      const bool in_ctx = t0 + key < ctx;
      const uint8_t* kfill = (const uint8_t*)(in_ctx ? g_pf_nan_row : g_pf_zero_row) + p * 16;
      const uint8_t* vfill = (const uint8_t*)g_pf_zero_row + p * 16;
      const bool real = in_ctx && valid;
      lds_dma16(real ? (const uint8_t*)a.k_cache + boff + voff[i] : kfill, kdst + g * 1024);
      lds_dma16(real ? (const uint8_t*)a.v_cache + boff + voff[i] : vfill, vdst + g * 1024);
    }
  }
}

// One (sequence, head, q tile) of a workgroup's share, as the two cursors
// of the tile stream see it.  k < 0: the share is exhausted.
struct PItem {
  int k;                // position in the workgroup's share
  int h, kvh, qbeg, C, P, ctx, q0, n_tiles;
  const int32_t* trow;  // the sequence's block-table row
};

// Key tiles that all q tiles of sequence s walk: the work it brings.
__device__ __forceinline__ int seq_tiles(const PrefillArgs& a, int s) {
  const int C = a.cu_q_lens[s + 1] - a.cu_q_lens[s];
  const int P = min(a.ctx_lens[s], a.max_blocks << a.log2B) - C;
  int n = 0;
  for (int q0 = 0; q0 < C; q0 += kPBM) n += max((P + min(C, q0 + kPBM) - 1) / kPKT + 1, 1);
  return n;
}

// Persistent grid.  Every workgroup walks a share of the work items
// (sequence, head, q tile) as one stream of key tiles: the transfers run two
// tiles ahead of the computation, across the end of an item, and the next
// item's query rows move into LDS while the last tile of the current one is
// computed.  Sequences are ranked by their number of key tiles, heaviest
// first (batches of at most 64 sequences; larger ones keep batch order), and
// the items of a round of gridDim.x go out in snake order (reversed every
// other round) so that the heavy ones spread evenly; consecutive items (the
// q tiles and heads of one sequence) go to workgroups on one XCD, which then
// share its L2 for the keys and values.
template <int D>
__global__ __launch_bounds__(kPThreads) void prefill_kernel(PrefillArgs a) {
  using PS = PShape<D>;
  constexpr int QX = 32 * PS::ROWB / 1024;  // 1 KiB query transfers per wavefront
  __shared__ __attribute__((aligned(1024))) uint8_t kb0[PS::TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t kb1[PS::TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t kb2[PS::TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t vb0[PS::TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t vb1[PS::TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t vb2[PS::TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t qb[kPBM * PS::ROWB];  // query rows, laid out like K
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;  // lane half
  const int lq = lane & 31;

  // Lane r of ordv holds the sequence of rank r.
  const bool ranked = a.S <= 64;
  int ordv = lane;
  if (ranked) {
    const int cs = lane < a.S ? seq_tiles(a, lane) : -1;
    int rank = 0;
    for (int t = 0; t < a.S; ++t) {
      const int ct = __shfl(cs, t);
      rank += (ct > cs) | ((ct == cs) & (t < lane));
    }
    ordv = __builtin_amdgcn_ds_permute(min(rank, 63) * 4, lane);
  }
  const int G = gridDim.x;
  const int per_seq = a.Hq * a.q_tiles;
  const int n_items = a.S * per_seq;
  const int slot = (G & 7) == 0 ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  const int maxctx = a.max_blocks << a.log2B;

  // The first item with work at or after position k of the share.
  auto item_at = [&](int k) __attribute__((always_inline)) {
    PItem it;
    for (;; ++k) {
      const int i = k * G + ((k & 1) ? G - 1 - slot : slot);
      if (i >= n_items) {
        it.k = -1;
        return it;
      }
      const int c = i / per_seq;
      const int rem = i - c * per_seq;
      const int h = rem / a.q_tiles;
      const int qt = a.q_tiles - 1 - (rem - h * a.q_tiles);  // heavier q tile first
      const int s = ranked ? __builtin_amdgcn_readlane(ordv, c) : c;
      const int qbeg = a.cu_q_lens[s];
      const int C = a.cu_q_lens[s + 1] - qbeg;
      const int q0 = qt * kPBM;
      if (q0 >= C) continue;
      it.k = k;
      it.h = h;
      it.kvh = h / a.G;
      it.qbeg = qbeg;
      it.C = C;
      it.ctx = min(a.ctx_lens[s], maxctx);  // never past the table
      it.P = it.ctx - C;                     // cached prefix length
      it.q0 = q0;
      it.n_tiles = max((it.P + min(C, q0 + kPBM) - 1) / kPKT + 1, 1);  // keys 0 .. P + last row
      it.trow = a.tables + (size_t)s * a.max_blocks;
      return it;
    }
  };

  PItem ci = item_at(0);  // item being computed
  if (ci.k < 0) return;
  PItem nci = item_at(ci.k + 1);  // the one after it
  PItem di = ci;                  // item of the next tile to transfer
  int tc = 0, td = 0;             // tile of ci being computed, of di to transfer next

  // this wavefront's query rows of item ci
  int wr0, my_row, my_pos, wave_last_pos, P;
  bool wave_live, row_ok;
  auto set_rows = [&]() __attribute__((always_inline)) {
    P = ci.P;
    wr0 = ci.q0 + wave * 32;
    wave_live = wr0 < ci.C;
    my_row = wr0 + lq;
    row_ok = my_row < ci.C;
    my_pos = P + my_row;
    wave_last_pos = P + min(wr0 + 31, ci.C - 1);
  };
  set_rows();

  f32x16_t acc_o[PS::DT];
#pragma unroll
  for (int dt = 0; dt < PS::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t sacc[2];
  bf16x8_t pb[4];

  // fixed per-lane offsets of the short-form transfers
  uint32_t voff[PS::DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < PS::DMA_PER_WAVE; ++i) voff[i] = dma_lane_offset<D>(wave * PS::DMA_PER_WAVE + i, lane, a.log2B);

  // three LDS buffers per tensor, picked at compile time (the loop below is
  // unrolled by three) so that reads of one are told apart from transfers
  // into another
  auto kbuf = [&](auto r) __attribute__((always_inline)) -> uint8_t* {
    constexpr int R = decltype(r)::value;
    if constexpr (R == 0) return kb0;
    else if constexpr (R == 1) return kb1;
    else return kb2;
  };
  auto vbuf = [&](auto r) __attribute__((always_inline)) -> uint8_t* {
    constexpr int R = decltype(r)::value;
    if constexpr (R == 0) return vb0;
    else if constexpr (R == 1) return vb1;
    else return vb2;
  };
  // transfer tile td of item di, then move that cursor on
  TileEntries<D> ent;  // block ids of tile td of di
  auto entries = [&]() __attribute__((always_inline)) { return tile_entries<D>(a, di.trow, td * kPKT, wave); };
  auto dma_next = [&](auto r) __attribute__((always_inline)) {
    dma_tile<D>(a, di.trow, ent, di.kvh, td * kPKT, di.ctx, wave, lane, voff, lds_addr(kbuf(r)), lds_addr(vbuf(r)));
    if (++td == di.n_tiles) {
      di = item_at(di.k + 1);
      td = 0;
    }
    if (di.k >= 0) ent = entries();  // arrives while a tile is computed
  };
  // this wavefront's 32 query rows of item it into LDS (rows past the
  // chunk repeat its last row; their outputs are not stored)
  auto q_dma = [&](const PItem& it) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < QX; ++x) {
      const int sl = x * 64 + lane;
      const int r = sl / PS::PIECES;
      const int p = (sl % PS::PIECES) ^ swz<D>(r);
      const int row = min(it.q0 + wave * 32 + r, it.C - 1);
      lds_dma16((const uint8_t*)a.q + ((size_t)(it.qbeg + row) * a.Hq + it.h) * PS::ROWB + p * 16,
                lds_addr(qb) + (uint32_t)(wave * 32 * PS::ROWB + x * 1024));
    }
  };
  auto live = [&](int j) __attribute__((always_inline)) { return wave_live && j * kPKT <= wave_last_pos; };

  // S^T for keys 64j .. 64j + 63 (two 32-key tiles) x this wave's 32
  // queries.  The two accumulators alternate; the K fragments are read two
  // contraction steps ahead, in an order the scheduler may not sink.
  const int ksw = swz<D>(lq);  // rows lq and lq + 32 share it
  const uint8_t* qrow = qb + (wave * 32 + lq) * PS::ROWB;  // this lane's query row
  auto s_phase = [&](auto r) __attribute__((always_inline)) {
    const uint8_t* k0 = kbuf(r) + lq * PS::ROWB;
    const uint8_t* k1 = k0 + 32 * PS::ROWB;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sacc[mt][rr] = 0.f;
    uint4 f0[PS::KS], f1[PS::KS], fq[PS::KS];
    auto kofs = [&](int ks) __attribute__((always_inline)) { return ((2 * ks + hh) ^ ksw) << 4; };
    f0[0] = *(const uint4*)(k0 + kofs(0));
    f1[0] = *(const uint4*)(k1 + kofs(0));
    fq[0] = *(const uint4*)(qrow + kofs(0));
    f0[1] = *(const uint4*)(k0 + kofs(1));
    f1[1] = *(const uint4*)(k1 + kofs(1));
    fq[1] = *(const uint4*)(qrow + kofs(1));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < PS::KS; ++ks) {
      if (ks + 2 < PS::KS) {
        f0[ks + 2] = *(const uint4*)(k0 + kofs(ks + 2));
        f1[ks + 2] = *(const uint4*)(k1 + kofs(ks + 2));
        fq[ks + 2] = *(const uint4*)(qrow + kofs(ks + 2));
      }
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8_t qf = __builtin_bit_cast(bf16x8_t, fq[ks]);
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, f0[ks]), qf, sacc[0], 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, f1[ks]), qf, sacc[1], 0, 0, 0);
    }
  };

  // Online softmax of tile j: weights P^T = exp2(c * s - m) in bf16 (c =
  // scale * log2 e), grouped by 16-key contraction steps, and the row sum
  // of those bf16 weights (v_dot2 with ones, so it adds what the matrix
  // cores see).  The reference m of a row is not moved every tile: weights
  // are formed against the current m, and only when a lane's weights sum
  // past 2^8 (a score above m by more than 8 in the log2 domain), or the
  // row has no reference yet, is the tile's true maximum taken, m raised
  // to it, the accumulators rescaled and the weights formed again.  So
  // weights stay below 2^8, far inside the bf16 and fp32 range, and the
  // final division by the row sum, taken against the same references,
  // cancels m exactly.  Masked keys (causal limit) occur only
  // in the tiles on the wave's diagonal, which take the masked variant.
  const float c = a.scale_log2;
  auto softmax = [&](auto masked, int t0) __attribute__((always_inline)) {
    constexpr bool M = decltype(masked)::value;
    if constexpr (M) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = t0 + mt * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          sacc[mt][r] = t > my_pos ? -INFINITY : sacc[mt][r] * c;
        }
    }
    const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
    auto weights = [&](float msub) __attribute__((always_inline)) {
      float psum = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        uint32_t w4[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float x0 = sacc[kk >> 1][8 * (kk & 1) + e];
          const float x1 = sacc[kk >> 1][8 * (kk & 1) + e + 1];
          const float p0 = __builtin_amdgcn_exp2f(M ? x0 - msub : __builtin_fmaf(x0, c, -msub));
          const float p1 = __builtin_amdgcn_exp2f(M ? x1 - msub : __builtin_fmaf(x1, c, -msub));
          w4[e >> 1] = pack2_bf16(p0, p1);
          psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w4[e >> 1]), ones, psum, false);
        }
        pb[kk] = __builtin_bit_cast(bf16x8_t, make_uint4(w4[0], w4[1], w4[2], w4[3]));
      }
      return psum;
    };
    bool slow = m_run == -INFINITY;
    float psum = 0.f;
    if (!__builtin_amdgcn_ballot_w64(slow)) {
      psum = weights(m_run);
      slow = psum > 256.f;  // false for NaN: such rows stay NaN
    }
    if (__builtin_amdgcn_ballot_w64(slow)) {
      float tmax;
      if constexpr (M) {
        tmax = sacc[0][0];
#pragma unroll
        for (int i = 1; i < 32; ++i) tmax = fmaxf(tmax, sacc[i >> 4][i & 15]);
      } else {
        float hi = sacc[0][0], lo = sacc[0][0];
#pragma unroll
        for (int i = 1; i < 32; ++i) {
          hi = fmaxf(hi, sacc[i >> 4][i & 15]);
          lo = fminf(lo, sacc[i >> 4][i & 15]);
        }
        tmax = c * (c >= 0.f ? hi : lo);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);  // stays -inf while the row is all masked
      const float alpha = m_new > m_run ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;  // exp2(-inf) = 0
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < PS::DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[dt][r] *= alpha;
      m_run = m_new;
      psum = weights(m_run == -INFINITY ? 0.f : m_run);
    }
    l_run += psum;
  };
  auto sm_phase = [&](int j) __attribute__((always_inline)) {
    const int t0 = j * kPKT;
    if (t0 + kPKT - 1 > P + wr0)
      softmax(std::true_type{}, t0);
    else
      softmax(std::false_type{}, t0);
  };

  // O^T += V^T P^T.  The A operand (row d, 8 keys in the order the S^T
  // accumulator holds them) comes from the row-major V tile through two
  // transposed reads (ds_read_b64_tr_b16): in each group of 16 lanes, lane
  // i names 4 columns d0 + 4 (i % 4) .. + 3 of key k0 + i / 4, and lane j
  // receives column d0 + j of keys k0 .. k0 + 3.  Byte offsets per lane for
  // each 32-row tile dt and key half h2 of a 16-key step:
  int vofs[PS::DT][2];
  {
    const int i16 = lane & 15, g16 = (lane >> 4) & 1;
#pragma unroll
    for (int dt = 0; dt < PS::DT; ++dt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int key = 8 * h2 + 4 * hh + (i16 >> 2);  // + 16 and 32 multiples: same swizzle
        const int p = 4 * dt + 2 * g16 + ((i16 & 3) >> 1);
        vofs[dt][h2] = key * PS::ROWB + ((p ^ swz<D>(key)) << 4) + ((i16 & 1) << 3);
      }
  }
  auto o_phase = [&](auto r) __attribute__((always_inline)) {
    const uint8_t* vb = vbuf(r);
    auto vfrag = [&](int dt, int kk) __attribute__((always_inline)) {
      const int ko = (32 * (kk >> 1) + 16 * (kk & 1)) * PS::ROWB;
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vb + vofs[dt][0] + ko));
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vb + vofs[dt][1] + ko));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8_t;
    s16x8_t fa[PS::DT], fb[PS::DT];
#pragma unroll
    for (int dt = 0; dt < PS::DT; ++dt) fa[dt] = vfrag(dt, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk + 1 < 4) {
#pragma unroll
        for (int dt = 0; dt < PS::DT; ++dt) fb[dt] = vfrag(dt, kk + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dt = 0; dt < PS::DT; ++dt)
        acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fa[dt]), pb[kk], acc_o[dt], 0, 0, 0);
      if (kk + 1 < 4) {
#pragma unroll
        for (int dt = 0; dt < PS::DT; ++dt) fa[dt] = fb[dt];
      }
    }
  };

  // Tiles go from global memory straight into LDS, three buffers deep:
  // step j computes tile j, issuing the transfers of tile j + 2 between its
  // softmax and its V products, then waits for its own share of tile j + 1
  // (issued one step earlier) and meets the other wavefronts at the
  // barrier, after which tile j + 1 is whole.
  // Tile j + 2 goes over tile j - 1, which every wavefront finished before
  // the previous barrier.
  // Output of item ci: the accumulated rows over their sums.
  auto finish_item = [&]() __attribute__((always_inline)) {
    // Rows that no q tile of the launch covers (a chunk longer than the
    // caller's bound on chunk lengths) come out NaN, never unwritten; the
    // last q tile of the sequence writes them.
    const int covered = a.q_tiles * kPBM;
    if (ci.q0 + kPBM == covered && ci.C > covered) {
      const uint4 nan8 = make_uint4(0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u);
      const int n = (ci.C - covered) * PS::PIECES;
      for (int i = tid; i < n; i += kPThreads) {
        const int r = covered + i / PS::PIECES;
        *(uint4*)(a.out + ((size_t)(ci.qbeg + r) * a.Hq + ci.h) * D + (i % PS::PIECES) * 8) = nan8;
      }
    }
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (row_ok) {
      const float inv = 1.f / l_tot;
      uint16_t* op = a.out + ((size_t)(ci.qbeg + my_row) * a.Hq + ci.h) * D;
#pragma unroll
      for (int dt = 0; dt < PS::DT; ++dt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int d0 = dt * 32 + 8 * rq + 4 * hh;
          const uint2 v = make_uint2(pack2_bf16(acc_o[dt][4 * rq] * inv, acc_o[dt][4 * rq + 1] * inv),
                                     pack2_bf16(acc_o[dt][4 * rq + 2] * inv, acc_o[dt][4 * rq + 3] * inv));
          *(uint2*)(op + d0) = v;
        }
    }
#pragma unroll
    for (int dt = 0; dt < PS::DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[dt][r] = 0.f;
    m_run = -INFINITY;
    l_run = 0.f;
  };

  // One step of the stream: compute tile tc of ci from buffer r, transfer
  // the tile two ahead (kept in buffer r + 2 mod 3, which held the tile
  // computed two steps ago), then wait for this wavefront's share of the
  // next tile and meet the others at the barrier.  On the last tile of an
  // item the next item's query rows go into LDS once this wavefront has
  // read its own (after its S^T products), ahead of the tile transfers; the
  // next step waits for them before its S^T products.  Returns false after
  // the last item.
  bool q_wait = false;   // the query rows of ci may still be on their way
  bool q_newer = false;  // and the previous step's tile transfers went out after them
  auto step = [&](auto r) __attribute__((always_inline)) {
    constexpr int R = decltype(r)::value;
    constexpr int NT = 2 * PS::DMA_PER_WAVE;  // transfers of one tile per wavefront
    const bool more = di.k >= 0;
    if (q_wait) {
      if (q_newer)
        __builtin_amdgcn_s_waitcnt((NT & 15) | ((NT >> 4) << 14) | (7 << 4) | (15 << 8));
      else
        __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
      q_wait = false;
    }
    const bool last = tc == ci.n_tiles - 1;
    const bool q_next = last && nci.k >= 0;
    const bool lv = live(tc);
    if (lv) s_phase(r);
    if (q_next) {
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wavefront's query reads are done
      q_dma(nci);
    }
    if (lv) sm_phase(tc);
    // The tile two ahead goes out after the softmax, while the matrix cores
    // still work on S^T and before the V products: issued at the start of
    // the step, the transfers held up the products (measured 4% slower).
    if (more) dma_next(std::integral_constant<int, (R + 2) % 3>{});
    if (lv) o_phase(r);
    q_newer = more;
    if (q_next) {
      if (more)
        tile_barrier<NT + QX>();
      else
        tile_barrier<QX>();
    } else if (more) {
      tile_barrier<NT>();
    } else {
      tile_barrier<0>();
    }
    if (!last) {
      ++tc;
      return true;
    }
    finish_item();
    ci = nci;
    tc = 0;
    if (ci.k < 0) return false;
    nci = item_at(ci.k + 1);
    set_rows();
    q_wait = true;
    return true;
  };

  // The first item's query rows, block ids and first two tiles are all in
  // flight at once; the barrier waits for every one of them, so the
  // compiler places no wait inside the loop.
  q_dma(ci);
  ent = entries();
  dma_next(std::integral_constant<int, 0>{});
  if (di.k >= 0) dma_next(std::integral_constant<int, 1>{});
  tile_barrier<0>();
  for (;;) {
    if (!step(std::integral_constant<int, 0>{})) break;
    if (!step(std::integral_constant<int, 1>{})) break;
    if (!step(std::integral_constant<int, 2>{})) break;
  }
}

bool prefill_supported(int dtype, int head_dim, int group, int block_size) {
  (void)group;
  return dtype == 1 && (head_dim == 64 || head_dim == 128) && block_size >= 1 && block_size <= 256 &&
         (block_size & (block_size - 1)) == 0;
}

int launch_prefill(void* out, const void* q, const int32_t* cu_q_lens, int total_q, int max_q_len,
                   const void* k_cache, const void* v_cache, const int32_t* tables, int max_blocks,
                   const int32_t* ctx, int S, int Hq, int Hkv, int D, int B, int num_blocks, float scale,
                   hipStream_t stream) {
  (void)total_q;
  PrefillArgs a;
  a.out = (uint16_t*)out;
  a.q = (const uint16_t*)q;
  a.cu_q_lens = cu_q_lens;
  a.k_cache = (const uint16_t*)k_cache;
  a.v_cache = (const uint16_t*)v_cache;
  a.tables = tables;
  a.ctx_lens = ctx;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.max_blocks = max_blocks;
  a.num_blocks = num_blocks;
  a.log2B = 0;
  while ((1 << a.log2B) < B) ++a.log2B;
  a.q_tiles = (max_q_len + kPBM - 1) / kPBM;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  const long long items = (long long)S * Hq * a.q_tiles;
  if (items <= 0) return 0;
  if (items > 0x7fffffffLL) return -2;
  const void* kfn = D == 128 ? (const void*)prefill_kernel<128> : (const void*)prefill_kernel<64>;
  const int per_cu = occupancy(kfn, kPThreads);
  const long long grid = std::min(items, (long long)per_cu * std::max(device_info().num_cus, 1));
  const dim3 g((unsigned)grid), b(kPThreads);
  if (D == 128)
    hipLaunchKernelGGL(prefill_kernel<128>, g, b, 0, stream, a);
  else if (D == 64)
    hipLaunchKernelGGL(prefill_kernel<64>, g, b, 0, stream, a);
  else
    return -2;
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace pkv
