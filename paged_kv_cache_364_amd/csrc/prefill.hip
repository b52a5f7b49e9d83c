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
// through the table), double-buffered in LDS and staged through one set of
// registers: the global loads of tile j + 2 are in flight while tile j is
// computed.  The block-table entries the tiles need sit in an LDS window.
// Per tile and wavefront:
//
//   S^T = K Q^T   on v_mfma_f32_32x32x16_bf16, A = K rows from LDS, B = the
//                 wavefront's query rows, held in registers for the whole
//                 loop.  The accumulator layout puts query l % 32 on lane l
//                 and 16 keys in its registers, so the online-softmax state
//                 (running max, running sum) of a query lives in one lane
//                 pair (l, l ^ 32).
//   O^T += V^T P^T  A = V^T from LDS, B = P^T taken straight from the S^T
//                 accumulators (converted to bf16): the keys a lane holds
//                 in registers are exactly the contraction index the B
//                 operand wants, provided V^T stores each 16-key group in
//                 the order of that register layout.  V is written to LDS
//                 transposed, in that order.
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
  static constexpr int KS = D / 16;          // contraction steps of S^T
  static constexpr int DT = D / 32;          // 32-row tiles of O^T
  static constexpr int PIECES = D / 8;       // 16-byte pieces per row
  static constexpr int KROW = D + 8;         // K row in LDS (bf16), padded
  static constexpr int VROW = kPKT + 8;      // V^T row in LDS (bf16), padded
  static constexpr int K_ELEMS = kPKT * KROW;
  static constexpr int V_ELEMS = D * VROW;
  static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
  static constexpr int K_TOTAL = kPKT * PIECES;                    // 16-byte K pieces per tile
  static constexpr int V_TOTAL = (kPKT / 2) * PIECES;              // (2 keys x 16 bytes) V pieces per tile
  static constexpr int K_LOADS = (K_TOTAL + kPThreads - 1) / kPThreads;  // per thread
  static constexpr int V_PAIRS = (V_TOTAL + kPThreads - 1) / kPThreads;
};

// Position of key u (0..63) inside its 16-key group of a V^T row: the order
// in which the S^T accumulator registers of a lane pair hold those keys.
__device__ __forceinline__ int vt_pos(int u) {
  const int v = u & 15;
  return (u & ~15) + 8 * ((v >> 2) & 1) + 4 * (v >> 3) + (v & 3);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2v_t;

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  bf16x2v_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

template <int D>
struct TileRegs {
  uint4 k[PShape<D>::K_LOADS];
  uint4 v0[PShape<D>::V_PAIRS];
  uint4 v1[PShape<D>::V_PAIRS];
  uint32_t zero;  // bit per load: replace by zeros (key past the context)
  uint32_t nan;   // bit per load: replace by NaN (block id outside the pool)
};

// Element offset of 16-byte piece `piece` of absolute key t of the sequence.
// Every load is issued unconditionally from a valid address (block 0 when
// the key has none) and flagged (code 1: key past the context, read as
// zeros; code 2: block id outside the pool, read as NaN), so no branch sits
// between a load and its use; the flags are applied when the tile is written
// to LDS.  Block ids come from the workgroup's LDS window of the table:
// tbl[i] = entry tbase + i.
struct KeyPiece {
  size_t off;
  uint32_t code;
};

__device__ __forceinline__ KeyPiece key_piece(const PrefillArgs& a, const int* tbl, int tbase, int kvh, int t,
                                              int ctx, int D, int piece) {
  const bool in_ctx = t < ctx;
  // The entry is read unconditionally (index clamped into the window) so
  // that a tile's lookups issue together.  Past the context it may hold
  // any value: any id inside the pool gives a valid address (the data is
  // replaced by zeros), anything else falls back to block 0.
  int blk = tbl[min((t >> a.log2B) - tbase, kPTableLds - 1)];
  const bool outside = (unsigned)blk >= (unsigned)a.num_blocks;
  blk = outside ? 0 : blk;
  const uint32_t row = (((uint32_t)blk * (uint32_t)a.Hkv + (uint32_t)kvh) << a.log2B) + (uint32_t)(t & ((1 << a.log2B) - 1));
  return {(size_t)row * D + piece * 8, (in_ctx ? 0u : 1u) | (in_ctx && outside ? 2u : 0u)};
}

__device__ __forceinline__ uint4 apply_fill(uint4 v, uint32_t zero, uint32_t nan, int bit) {
  if ((zero >> bit) & 1) v = make_uint4(0, 0, 0, 0);
  if ((nan >> bit) & 1) v = make_uint4(0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u);
  return v;
}

template <int D, bool PAIRED>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, const PrefillArgs& a, const int* tbl, int tbase, int kvh,
                                          int t0, int ctx, int tid) {
  using PS = PShape<D>;
  r.zero = 0;
  r.nan = 0;
#pragma unroll
  for (int n = 0; n < PS::K_LOADS; ++n) {
    const int idx = tid + n * kPThreads;
    if (PS::K_TOTAL % kPThreads != 0 && idx >= PS::K_TOTAL) break;
    const int key = idx / PS::PIECES;
    const int pc = idx % PS::PIECES;
    const KeyPiece kp = key_piece(a, tbl, tbase, kvh, t0 + key, ctx, D, pc);
    r.k[n] = *(const uint4*)(a.k_cache + kp.off);
    r.zero |= (kp.code & 1u) << n;
    r.nan |= (kp.code >> 1) << n;
  }
#pragma unroll
  for (int n = 0; n < PS::V_PAIRS; ++n) {
    const int idx = tid + n * kPThreads;
    if (PS::V_TOTAL % kPThreads != 0 && idx >= PS::V_TOTAL) break;
    const int pair = idx % (kPKT / 2);
    const int pc = idx / (kPKT / 2);
    const int b0 = PS::K_LOADS + 2 * n;
    const KeyPiece p0 = key_piece(a, tbl, tbase, kvh, t0 + 2 * pair, ctx, D, pc);
    KeyPiece p1;
    if constexpr (PAIRED) {
      // blocks of two or more tokens: keys 2 * pair and 2 * pair + 1 share
      // a block, so the second row follows the first
      const bool in1 = t0 + 2 * pair + 1 < ctx;
      p1 = {p0.off + D, (in1 ? 0u : 1u) | (in1 && (p0.code & 3u) == 2u ? 2u : 0u)};
    } else {
      p1 = key_piece(a, tbl, tbase, kvh, t0 + 2 * pair + 1, ctx, D, pc);
    }
    r.v0[n] = *(const uint4*)(a.v_cache + p0.off);
    r.v1[n] = *(const uint4*)(a.v_cache + p1.off);
    r.zero |= ((p0.code & 1u) << b0) | ((p1.code & 1u) << (b0 + 1));
    r.nan |= ((p0.code >> 1) << b0) | ((p1.code >> 1) << (b0 + 1));
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& r, uint16_t* kl, uint16_t* vl, int tid) {
  using PS = PShape<D>;
  uint4 kx[PS::K_LOADS], v0x[PS::V_PAIRS], v1x[PS::V_PAIRS];
#pragma unroll
  for (int n = 0; n < PS::K_LOADS; ++n) kx[n] = r.k[n];
#pragma unroll
  for (int n = 0; n < PS::V_PAIRS; ++n) {
    v0x[n] = r.v0[n];
    v1x[n] = r.v1[n];
  }
  // zero / NaN fills are needed only past the context end or for bad block
  // ids: skipped (one scalar branch) unless some lane of the wave has one
  if (__builtin_amdgcn_ballot_w64((r.zero | r.nan) != 0u)) {
#pragma unroll
    for (int n = 0; n < PS::K_LOADS; ++n) kx[n] = apply_fill(kx[n], r.zero, r.nan, n);
#pragma unroll
    for (int n = 0; n < PS::V_PAIRS; ++n) {
      v0x[n] = apply_fill(v0x[n], r.zero, r.nan, PS::K_LOADS + 2 * n);
      v1x[n] = apply_fill(v1x[n], r.zero, r.nan, PS::K_LOADS + 2 * n + 1);
    }
  }
#pragma unroll
  for (int n = 0; n < PS::K_LOADS; ++n) {
    const int idx = tid + n * kPThreads;
    if (PS::K_TOTAL % kPThreads != 0 && idx >= PS::K_TOTAL) break;
    const int key = idx / PS::PIECES;
    const int pc = idx % PS::PIECES;
    *(uint4*)(kl + key * PS::KROW + pc * 8) = kx[n];
  }
#pragma unroll
  for (int n = 0; n < PS::V_PAIRS; ++n) {
    const int idx = tid + n * kPThreads;
    if (PS::V_TOTAL % kPThreads != 0 && idx >= PS::V_TOTAL) break;
    const int pair = idx % (kPKT / 2);
    const int pc = idx / (kPKT / 2);
    const int pos = vt_pos(2 * pair);  // even; key 2 * pair + 1 sits next to it
    const uint32_t a0[4] = {v0x[n].x, v0x[n].y, v0x[n].z, v0x[n].w};
    const uint32_t a1[4] = {v1x[n].x, v1x[n].y, v1x[n].z, v1x[n].w};
    // element e of key 2 * pair (low half) and of key 2 * pair + 1 (high
    // half) in one v_perm_b32: byte selectors 0-3 pick from a0, 4-7 from a1
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *(uint32_t*)(vl + (pc * 8 + e) * PS::VROW + pos) =
          __builtin_amdgcn_perm(a1[e >> 1], a0[e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
  }
}

template <int D, bool PAIRED>
__global__ __launch_bounds__(kPThreads) void prefill_kernel(PrefillArgs a) {
  using PS = PShape<D>;
  __shared__ __attribute__((aligned(16))) uint16_t klds[2 * PS::K_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t vlds[2 * PS::V_ELEMS];
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

  auto load = [&](TileRegs<D>& r, int jt) __attribute__((always_inline)) {
    // slide the window when tile jt leaves it (uniform over the workgroup)
    const int last_blk = (min((jt + 1) * kPKT, ctx) - 1) >> a.log2B;
    if (last_blk >= tbase + kPTableLds) {
      __syncthreads();
      tbase = (jt * kPKT) >> a.log2B;
      fill_window(tbase);
      __syncthreads();
    }
    load_tile<D, PAIRED>(r, a, tbl, tbase, kvh, jt * kPKT, ctx, tid);
  };
  auto live = [&](int j) __attribute__((always_inline)) { return wave_live && j * kPKT <= wave_last_pos; };

  // S^T for keys 64j .. 64j + 63 (two 32-key tiles) x this wave's 32
  // queries.  The two accumulators alternate; the K fragments are read two
  // contraction steps ahead, in an order the scheduler may not sink.
  auto s_phase = [&](int j) __attribute__((always_inline)) {
    const uint16_t* k0 = klds + (j & 1) * PS::K_ELEMS + lq * PS::KROW + hh * 8;
    const uint16_t* k1 = k0 + 32 * PS::KROW;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[mt][r] = 0.f;
    uint4 f0[PS::KS], f1[PS::KS];
    f0[0] = *(const uint4*)k0;
    f1[0] = *(const uint4*)k1;
    f0[1] = *(const uint4*)(k0 + 16);
    f1[1] = *(const uint4*)(k1 + 16);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < PS::KS; ++ks) {
      if (ks + 2 < PS::KS) {
        f0[ks + 2] = *(const uint4*)(k0 + (ks + 2) * 16);
        f1[ks + 2] = *(const uint4*)(k1 + (ks + 2) * 16);
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

  // O^T += V^T P^T: the DT accumulators alternate; the V^T fragments of the
  // next contraction step are read while this step's products run
  auto o_phase = [&](int j) __attribute__((always_inline)) {
    const uint16_t* v0 = vlds + (j & 1) * PS::V_ELEMS + lq * PS::VROW + hh * 8;
    uint4 fa[PS::DT], fb[PS::DT];
#pragma unroll
    for (int dt = 0; dt < PS::DT; ++dt) fa[dt] = *(const uint4*)(v0 + dt * 32 * PS::VROW);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk + 1 < 4) {
#pragma unroll
        for (int dt = 0; dt < PS::DT; ++dt) fb[dt] = *(const uint4*)(v0 + dt * 32 * PS::VROW + (kk + 1) * 16);
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

  // Key tiles flow global -> registers -> LDS through one register stage,
  // double buffered in LDS: step j first writes tile j + 1 (loaded during
  // step j - 1) over tile j - 1, then issues the loads of tile j + 2 into the
  // same registers, then computes tile j, so a tile's loads have a whole
  // step of compute to arrive.
  TileRegs<D> rg;
  auto step = [&](int j) __attribute__((always_inline)) {
    if (j + 1 < n_tiles) {
      store_tile<D>(rg, klds + ((j + 1) & 1) * PS::K_ELEMS, vlds + ((j + 1) & 1) * PS::V_ELEMS, tid);
      if (j + 2 < n_tiles) load(rg, j + 2);
    }
    if (live(j)) {
      s_phase(j);
      sm_phase(j);
      o_phase(j);
    }
    __syncthreads();
  };

  load(rg, 0);
  store_tile<D>(rg, klds, vlds, tid);
  if (n_tiles > 1) load(rg, 1);
  __syncthreads();
  for (int j = 0; j < n_tiles; ++j) step(j);

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
  if (D == 128 && B >= 2)
    hipLaunchKernelGGL((prefill_kernel<128, true>), g, b, 0, stream, a);
  else if (D == 128)
    hipLaunchKernelGGL((prefill_kernel<128, false>), g, b, 0, stream, a);
  else if (D == 64 && B >= 2)
    hipLaunchKernelGGL((prefill_kernel<64, true>), g, b, 0, stream, a);
  else if (D == 64)
    hipLaunchKernelGGL((prefill_kernel<64, false>), g, b, 0, stream, a);
  else
    return -2;
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace pkv
