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
// Tiling.  A workgroup of eight wavefronts owns BM = 256 query rows of one
// (sequence, head); wavefront w owns rows 32w .. 32w + 31.  Keys and values
// are walked in tiles of KT = 64 tokens (several physical blocks gathered
// through the table), moved from global memory straight into LDS
// (global_load_lds) and triple-buffered there: the transfers of tile j + 2
// are in flight while tile j is computed.  The block-table entries the
// tiles need sit in an LDS window.
// Per tile and wavefront:
//
//   S^T = K Q^T   on v_mfma_f32_32x32x16_bf16, A = K rows from LDS, B = the
//                 wavefront's query rows, held in registers for the whole
//                 loop.  The accumulator layout puts query l % 32 on lane l
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
constexpr int kPTableLds = 1024;  // block-table entries staged in LDS per workgroup

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

// Rows for keys with no data: zeros past the context, NaN for a block id
// outside the pool (so the rows that attend it come out NaN).
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
__device__ __forceinline__ void lds_dma16(const void* src, uint8_t* dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)dst);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off"
      :
      : "s"(m0), "v"(src)
      : "memory", "m0");
}

// Issue the transfers of tile t0 .. t0 + 63 straight into LDS (K to kdst,
// V to vdst): each 1 KiB transfer of a wavefront fills 64 consecutive
// slots, lane l slot l, from the global piece that the swizzle puts there.
// Block ids come from the workgroup's LDS window of the table (tbl[i] =
// entry tbase + i); the entry is read unconditionally, index clamped into
// the window, and a key past the context reads the zero row whatever the
// entry holds.
template <int D>
__device__ __forceinline__ void dma_tile(const PrefillArgs& a, const int* tbl, int tbase, int kvh, int t0, int ctx,
                                         int wave, int lane, uint8_t* kdst, uint8_t* vdst) {
  using PS = PShape<D>;
#pragma unroll
  for (int i = 0; i < PS::DMA_PER_WAVE; ++i) {
    const int g = wave * PS::DMA_PER_WAVE + i;  // 1 KiB chunk of the tile
    const int sl = g * 64 + lane;               // 16-byte slot
    const int key = sl / PS::PIECES;
    const int p = (sl % PS::PIECES) ^ swz<D>(key);
    const int t = t0 + key;
    const bool in_ctx = t < ctx;
    const int blk = tbl[min((t >> a.log2B) - tbase, kPTableLds - 1)];
    const bool outside = (unsigned)blk >= (unsigned)a.num_blocks;
    const uint32_t row =
        (((uint32_t)blk * (uint32_t)a.Hkv + (uint32_t)kvh) << a.log2B) + (uint32_t)(t & ((1 << a.log2B) - 1));
    const size_t off = (size_t)row * D + p * 8;
    const bool real = in_ctx && !outside;
    const uint16_t* fill = in_ctx ? g_pf_nan_row + p * 8 : g_pf_zero_row + p * 8;  // used when !real
    const uint16_t* ksrc = real ? a.k_cache + off : fill;
    const uint16_t* vsrc = real ? a.v_cache + off : fill;
    lds_dma16(ksrc, kdst + g * 1024);
    lds_dma16(vsrc, vdst + g * 1024);
  }
}

template <int D>
__global__ __launch_bounds__(kPThreads) void prefill_kernel(PrefillArgs a) {
  using PS = PShape<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t kb0[PS::TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t kb1[PS::TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t kb2[PS::TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t vb0[PS::TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t vb1[PS::TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t vb2[PS::TILEB];
  __shared__ int tbl[kPTableLds];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;  // lane half
  const int lq = lane & 31;

  // Workgroup -> (unit, q tile).  Workgroups are dealt to the 8 XCDs round
  // robin; all q tiles of one (sequence, head) go to one XCD, one after the
  // other and heaviest (last) first, so they share its L2 for the keys and
  // values, and consecutive units spread over the XCDs.
  const int f = blockIdx.x;
  const int xcd = f & 7;
  const int k = f >> 3;
  const int unit = (k / a.q_tiles) * 8 + xcd;
  const int qt = a.q_tiles - 1 - (k % a.q_tiles);
  if (unit >= a.S * a.Hq) return;
  const int s = unit / a.Hq;
  const int h = unit - s * a.Hq;
  const int kvh = h / a.G;
  const int qbeg = a.cu_q_lens[s];
  const int C = a.cu_q_lens[s + 1] - qbeg;
  const int q0 = qt * kPBM;
  if (q0 >= C) return;
  const int ctx = min(a.ctx_lens[s], a.max_blocks << a.log2B);  // never past the table
  const int P = ctx - C;  // cached prefix length
  const int rows_end = min(C, q0 + kPBM);
  const int n_tiles = (P + rows_end - 1) / kPKT + 1;  // keys 0 .. P + rows_end - 1
  const int32_t* trow = a.tables + (size_t)s * a.max_blocks;

  // this wavefront's query rows and their B operands (query l % 32)
  const int wr0 = q0 + wave * 32;
  const bool wave_live = wr0 < C;
  const int my_row = wr0 + lq;
  const bool row_ok = my_row < C;
  const int my_pos = P + my_row;
  const int wave_last_pos = P + min(wr0 + 31, C - 1);
  bf16x8_t qreg[PS::KS];
  {
    const uint16_t* qp = a.q + ((size_t)(qbeg + min(my_row, C - 1)) * a.Hq + h) * D + hh * 8;
#pragma unroll
    for (int ks = 0; ks < PS::KS; ++ks) {
      const uint4 v = row_ok ? *(const uint4*)(qp + ks * 16) : make_uint4(0, 0, 0, 0);
      qreg[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
    // all query rows in registers before the first tile transfer: the
    // compiler then never waits for them (and for the transfers behind
    // them) inside the loop
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
  }

  f32x16_t acc_o[PS::DT];
#pragma unroll
  for (int dt = 0; dt < PS::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t sacc[2];
  bf16x8_t pb[4];

  // Block-table window in LDS: entries tbase .. tbase + kPTableLds - 1 of
  // the sequence's row (those the tiles need; keys past the causal limit
  // are loaded too, then masked, so whole tiles must map to real blocks).
  const int nblk_all = (min(ctx, n_tiles * kPKT) + (1 << a.log2B) - 1) >> a.log2B;
  int tbase = 0;
  auto fill_window = [&](int base) __attribute__((always_inline)) {
    const int n = min(nblk_all - base, kPTableLds);
    for (int i = tid; i < n; i += kPThreads) tbl[i] = trow[base + i];
  };
  fill_window(0);
  __syncthreads();

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
  auto dma = [&](int jt, auto r) __attribute__((always_inline)) {
    // slide the window when tile jt leaves it (uniform over the workgroup)
    const int last_blk = (min((jt + 1) * kPKT, ctx) - 1) >> a.log2B;
    if (last_blk >= tbase + kPTableLds) {
      __syncthreads();
      tbase = (jt * kPKT) >> a.log2B;
      fill_window(tbase);
      __syncthreads();
    }
    dma_tile<D>(a, tbl, tbase, kvh, jt * kPKT, ctx, wave, lane, kbuf(r), vbuf(r));
  };
  auto live = [&](int j) __attribute__((always_inline)) { return wave_live && j * kPKT <= wave_last_pos; };

  // S^T for keys 64j .. 64j + 63 (two 32-key tiles) x this wave's 32
  // queries.  The two accumulators alternate; the K fragments are read two
  // contraction steps ahead, in an order the scheduler may not sink.
  const int ksw = swz<D>(lq);  // rows lq and lq + 32 share it
  auto s_phase = [&](auto r) __attribute__((always_inline)) {
    const uint8_t* k0 = kbuf(r) + lq * PS::ROWB;
    const uint8_t* k1 = k0 + 32 * PS::ROWB;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sacc[mt][rr] = 0.f;
    uint4 f0[PS::KS], f1[PS::KS];
    auto kofs = [&](int ks) __attribute__((always_inline)) { return ((2 * ks + hh) ^ ksw) << 4; };
    f0[0] = *(const uint4*)(k0 + kofs(0));
    f1[0] = *(const uint4*)(k1 + kofs(0));
    f0[1] = *(const uint4*)(k0 + kofs(1));
    f1[1] = *(const uint4*)(k1 + kofs(1));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < PS::KS; ++ks) {
      if (ks + 2 < PS::KS) {
        f0[ks + 2] = *(const uint4*)(k0 + kofs(ks + 2));
        f1[ks + 2] = *(const uint4*)(k1 + kofs(ks + 2));
      }
      __builtin_amdgcn_sched_barrier(0);
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, f0[ks]), qreg[ks], sacc[0], 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, f1[ks]), qreg[ks], sacc[1], 0, 0, 0);
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
  // step j issues the transfers of tile j + 2, computes tile j, then waits
  // for its own share of tile j + 1 (issued one step earlier) and meets the
  // other wavefronts at the barrier, after which tile j + 1 is whole.
  // Tile j + 2 goes over tile j - 1, which every wavefront finished before
  // the previous barrier.
  auto step = [&](int j, auto r) __attribute__((always_inline)) {
    constexpr int R = decltype(r)::value;
    const bool more = j + 2 < n_tiles;
    if (more) dma(j + 2, std::integral_constant<int, (R + 2) % 3>{});
    if (live(j)) {
      s_phase(r);
      sm_phase(j);
      o_phase(r);
    }
    if (more)
      tile_barrier<2 * PS::DMA_PER_WAVE>();
    else
      tile_barrier<0>();
  };

  dma(0, std::integral_constant<int, 0>{});
  if (n_tiles > 1) {
    dma(1, std::integral_constant<int, 1>{});
    tile_barrier<2 * PS::DMA_PER_WAVE>();
  } else {
    tile_barrier<0>();
  }
  for (int j = 0; j < n_tiles; j += 3) {
    step(j, std::integral_constant<int, 0>{});
    if (j + 1 < n_tiles) step(j + 1, std::integral_constant<int, 1>{});
    if (j + 2 < n_tiles) step(j + 2, std::integral_constant<int, 2>{});
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!row_ok) return;
  const float inv = 1.f / l_tot;
  uint16_t* op = a.out + ((size_t)(qbeg + my_row) * a.Hq + h) * D;
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
  const long long units = (long long)S * Hq;
  const long long grid = (units + 7) / 8 * 8 * a.q_tiles;
  if (grid <= 0) return 0;
  if (grid > 0x7fffffffLL) return -2;
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
