// Paged decode for batches whose sequences share a prompt: parallel
// sampling and beam search, where the branches of one prompt hold its
// blocks together (reference counts, copy-on-write: intelliparadigm.com
// article, section 2.3; "08. PagedAttention", section "what else paging
// solves").  The pages store such a prompt once (cnblogs "paged attention",
// section 9); this kernel also reads it once per step.
//
// One workgroup per (group, kv head).  A group is a run of sequences of the
// batch whose block tables agree on their first `shared` entries.  The
// G query heads of every member that read this kv head are stacked into one
// set of up to 16 query rows, and the workgroup walks a list of 16-token
// tiles: the shared tiles, which every row attends, then each member's
// private tiles (the rest of its context), which only that member's rows
// attend (the other rows' scores are masked).  The result is the plain
// softmax(scale * q K^T) V of every (sequence, head) (cnblogs section 6).
//
// Per pair of tiles and wavefront (16 rows x 32 keys):
//   S^T = K Q^T   v_mfma_f32_16x16x32_bf16: A = 16 keys x 32 head dims of
//                 K (lane l: key l % 16, dims 8 (l / 16) .. + 7 of each
//                 32-wide step), B = the stacked query rows.  The accumulator gives lane l row l % 16 and
//                 keys 4 (l / 16) .. + 3, so a row's softmax state lives in
//                 the four lanes l % 16 + 16 j.
//   O^T += V^T P^T  the same instruction, A = V^T (16 head dims x the 32
//                 keys of the pair), read from LDS with the transposing
//                 ds_read_b64_tr_b16; B = P^T, the weights straight from the
//                 S^T accumulators.  A contraction sums over its k index in
//                 any order, so the pair's keys are assigned to k as the
//                 accumulators hold them: k = 8 (l / 16) + e is key
//                 4 (l / 16) + e % 4 of tile e / 4.
// K and V are read from global memory 1 KiB of a tile per instruction
// (lane l: the 16 bytes at 16 l), whole cache lines at a time, and pass
// through swizzled LDS into the operand layouts above: loading the operand
// layout directly reads half a cache line of each of 16 keys per
// instruction, and streams about a fifth slower.
// Online softmax with the lazy reference max of the plain decode (weights
// below 2^8), fp32 accumulation; the eight wavefronts' partials are merged
// in LDS with their log-sum-exp weights at the end.
#include "common.h"
#include "kernels.h"

namespace pkv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 sbf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float sf32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short ss16x4_t;
typedef __attribute__((address_space(3))) ss16x4_t lds_ss16x4_t;
typedef __attribute__((address_space(4))) const int32_t sconst_i32_t;

struct SharedArgs {
  uint16_t* out;
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* tables;
  const int32_t* ctx_lens;
  const int32_t* group_start;
  const int32_t* shared_blocks;
  int S, Hq, Hkv, G, max_blocks, num_blocks, log2B, num_groups;
  float scale_log2;
};

constexpr int kSW = 8;      // wavefronts per workgroup
constexpr int kRows = 16;   // stacked query rows
constexpr int kMaxMembers = 8;

// 16-byte load that does not keep the line in the caches.
__device__ __forceinline__ uint4 sload_stream(const void* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(t.x, t.y, t.z, t.w);
}

// Swizzled LDS slot of 16-byte piece p of key k in a 16 x 256-byte tile:
// the XOR spreads both the row-wise writes and the transposing reads over
// all banks.
__device__ __forceinline__ int vslot(int k, int p) { return k * 16 + (p ^ (((k & 3) << 2) | ((k >> 2) & 3))); }

__device__ __forceinline__ uint32_t pack2_bf16_rne(float a, float b) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 v2;
  v2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// A tile of the list: 16 keys of one block, the member whose rows attend it
// (-1: every member), and how many of its keys exist.
struct Tile {
  long long row0;  // first key's row in the pool ([block][kv head][slot]); 0 when nothing is read
  int owner;       // member index, or -1 for a shared tile
  int valid;       // keys 0 .. valid - 1 exist (0: no tile, or its block is outside the pool)
  int bad;         // the block lies outside the pool: the attending rows' results are NaN
};

template <int D>
__global__ __launch_bounds__(64 * kSW) void decode_shared_kernel(SharedArgs a) {
  static_assert(D == 128, "stacked decode: head_dim 128");
  constexpr int ROWB = D * 2;
  constexpr int TB = 16 * ROWB;  // bytes of one tile
  // Per wavefront: K0, K1, V0, V1 of the pair being computed (swizzled
  // rows); at the end the same bytes hold the wavefront's partial for the
  // merge (kRows x (D + 2) floats).
  __shared__ __attribute__((aligned(16))) uint8_t wb[kSW][4 * TB];
  static_assert(kRows * (D + 2) * 4 <= 4 * TB, "the partial fits the tile buffers");
  auto partw = [&](int w8) { return (float(*)[D + 2])(void*)wb[w8]; };
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar table reads
  const int gi = blockIdx.x / a.Hkv;
  const int h = blockIdx.x - gi * a.Hkv;
  const int B = 1 << a.log2B;
  const int maxctx = a.max_blocks << a.log2B;
  const int tiles_per_block = B / 16;

  // the group: members g0 .. g0 + nm - 1, their first `sb` table entries shared
  // (group bounds are trusted, but clamped into the batch so that no access
  // leaves it: a bad group only gives wrong rows)
  const int g0 = min(max(__builtin_amdgcn_readfirstlane(((sconst_i32_t*)a.group_start)[gi]), 0), a.S);
  const int g1 = __builtin_amdgcn_readfirstlane(((sconst_i32_t*)a.group_start)[gi + 1]);
  const int nm = min(min(max(g1 - g0, 0), a.S - g0), min(kMaxMembers, kRows / a.G));
  int sb = __builtin_amdgcn_readfirstlane(((sconst_i32_t*)a.shared_blocks)[gi]);
  sb = min(max(sb, 0), a.max_blocks);
  // lane m < nm: member m's context and private tiles
  const int my_ctx = lane < nm ? min(a.ctx_lens[g0 + lane], maxctx) : 0;
  const int sbt = nm > 0 ? sb * tiles_per_block : 0;  // shared tiles (none for a group with no member)
  const int my_priv = lane < nm ? max(0, (my_ctx - sb * B + 15) >> 4) : 0;
  int incl = my_priv;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  const int ntiles = sbt + __builtin_amdgcn_readlane(incl, 63);
  const int32_t* trow0 = a.tables + (size_t)g0 * a.max_blocks;

  // tile t of the list
  auto tile_at = [&](int t) -> Tile {
    Tile r;
    r.row0 = 0;
    r.owner = -1;
    r.valid = 0;
    r.bad = 0;
    if (t >= ntiles) return r;
    int blk, key0;
    if (t < sbt) {
      blk = ((sconst_i32_t*)trow0)[t / tiles_per_block];
      key0 = (t % tiles_per_block) * 16;
      r.valid = 16;
    } else {
      const int tp = t - sbt;
      const unsigned long long hit = __ballot(incl > tp);
      const int m = __ffsll((long long)hit) - 1;
      const int before = __builtin_amdgcn_readlane(incl - my_priv, m);
      const int ctx = __builtin_amdgcn_readlane(my_ctx, m);
      const int tok = sb * B + (tp - before) * 16;  // first key of the tile
      r.owner = m;
      blk = ((sconst_i32_t*)(a.tables + (size_t)(g0 + m) * a.max_blocks))[tok >> a.log2B];
      key0 = tok & (B - 1);
      r.valid = min(16, ctx - tok);
    }
    if ((unsigned)blk < (unsigned)a.num_blocks) {
      r.row0 = (((long long)blk * a.Hkv + h) << a.log2B) + key0;
    } else {
      r.bad = 1;
      r.valid = 0;  // nothing of it is read
    }
    return r;
  };

  // The stacked query rows (B operand of S^T): lane l holds row l % 16, dims
  // 32 s + 8 (l / 16) .. + 7 for s = 0..3.  Rows past the members are zero.
  const int row = lane & 15;
  const int grp = lane >> 4;
  const int row_member = row / a.G;
  const bool row_live = row_member < nm;
  uint4 qf[D / 32];
  {
    const uint16_t* qp = a.q + ((size_t)(g0 + (row_live ? row_member : 0)) * a.Hq + (size_t)h * a.G + row % a.G) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      qf[s] = row_live ? *(const uint4*)(qp + 32 * s + 8 * grp) : make_uint4(0, 0, 0, 0);
  }

  // K/V loads of a tile: instruction s reads 1 KiB, lane l the 16 bytes at
  // 1 KiB s + 16 l (key 4 s + l / 16, dims 8 (l % 16) .. + 7).  The loads
  // are unconditional (a missing tile reads row0 = 0 and is never used), so
  // that no load result is merged with a zero before use: keys past a
  // tile's end are masked in the scores and zeroed where V is staged.
  struct TileData {
    uint4 k[D / 32];
    uint4 v[D / 32];
  };
  auto load_tile = [&](const Tile& t, TileData& d) {
    const size_t off = (size_t)t.row0 * D + 8 * lane;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      d.k[s] = sload_stream(a.k_cache + off + 512 * s);
      d.v[s] = sload_stream(a.v_cache + off + 512 * s);
    }
  };

  sf32x4_t acc[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) acc[t] = sf32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.scale_log2;

  // S^T of one tile, masked: -inf for keys past the tile's end and for rows
  // of other members; lane keeps keys 4 grp .. 4 grp + 3 of row `row`.
  auto scores = [&](const Tile& t, int which, float (&sc)[4]) {
    const uint8_t* kb = wb[wid] + which * TB;
    uint4 kf[D / 32];
#pragma unroll
    for (int s = 0; s < D / 32; ++s) kf[s] = *(const uint4*)(kb + vslot(row, 4 * s + grp) * 16);
    sf32x4_t s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(sbf16x8_t, kf[s]),
                                                   __builtin_bit_cast(sbf16x8_t, qf[s]), s4, 0, 0, 0);
    const bool row_on = row_live && (t.owner < 0 || t.owner == row_member);
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = (row_on && 4 * grp + r < t.valid) ? s4[r] * c : -INFINITY;
  };

  // O^T += V^T P^T over the pair's V in LDS: for each 16-dim tile, two
  // transposing reads (keys 4 grp .. + 3 of each tile, dim 16 dt + l % 16).
  auto pv = [&](const sbf16x8_t& pb) {
    const uint8_t* base = wb[wid] + 2 * TB;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const int key = 4 * grp + (row >> 2);   // lane i of the 16-lane group names key 4 grp + i / 4
      const int col = 16 * dt + 4 * (row & 3);  // and 4 columns from here
      const int p = col >> 3;
      const int byte = vslot(key, p) * 16 + ((col & 7) ? 8 : 0);
      const ss16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ss16x4_t*)(base + byte));
      const ss16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ss16x4_t*)(base + 16 * ROWB + byte));
      typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
      const s16x8 vv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(sbf16x8_t, vv), pb, acc[dt], 0, 0, 0);
    }
  };

  // K and V of a tile into the wavefront's LDS buffers (row-major,
  // swizzled).  V rows past the tile's end become zeros: their weights are
  // zero, and 0 x NaN would not be.
  auto stage = [&](const Tile& t, const TileData& d, int which) {
    uint8_t* kb = wb[wid] + which * TB;
    uint8_t* vb = wb[wid] + (2 + which) * TB;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const int key = 4 * s + grp;
      const int slot = vslot(key, row) * 16;
      *(uint4*)(kb + slot) = d.k[s];
      *(uint4*)(vb + slot) = key < t.valid ? d.v[s] : make_uint4(0, 0, 0, 0);
    }
  };

  // One pair of tiles, staged in LDS: scores, online softmax, weighted V sum.
  auto step = [&](const Tile& t0, const Tile& t1) {
    float s0[4], s1[4];
    scores(t0, 0, s0);
    scores(t1, 1, s1);
    float cmax = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])), fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
    cmax = fmaxf(cmax, xor_lane<16>(cmax));
    cmax = fmaxf(cmax, xor_lane<32>(cmax));
    // lazy reference max (see the plain decode): move only past 2^8
    const bool move = cmax > m_run + 8.f;
    const float m_new = move ? cmax : m_run;
    if (__ballot(move)) {
      const float alpha = move ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;  // exp2(-inf) = 0
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[dt][r] *= alpha;
    }
    m_run = m_new;
    float w[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      w[r] = s0[r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s0[r] - m_run);
      w[4 + r] = s1[r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s1[r] - m_run);
    }
    const uint4 pw = make_uint4(pack2_bf16_rne(w[0], w[1]), pack2_bf16_rne(w[2], w[3]), pack2_bf16_rne(w[4], w[5]),
                                pack2_bf16_rne(w[6], w[7]));
    // the row sum adds the same bf16 weights the matrix cores see
    float ps = 0.f;
    ps = dot2_bf16(pw.x, 0x3f803f80u, ps);
    ps = dot2_bf16(pw.y, 0x3f803f80u, ps);
    ps = dot2_bf16(pw.z, 0x3f803f80u, ps);
    ps = dot2_bf16(pw.w, 0x3f803f80u, ps);
    const bool row_on0 = row_live && (t0.owner < 0 || t0.owner == row_member);
    const bool row_on1 = row_live && (t1.owner < 0 || t1.owner == row_member);
    l_run += ps + (((t0.bad && row_on0) || (t1.bad && row_on1)) ? __builtin_nanf("") : 0.f);
    wave_lds_sync();
    pv(__builtin_bit_cast(sbf16x8_t, pw));
    wave_lds_sync();  // the next pair's V overwrites the buffers
  };

  // Wavefront wid takes pairs wid, wid + kSW, ...: tiles 2 p and 2 p + 1.
  // A step stages pair c (the one computed) in LDS, which frees its
  // registers, issues the loads of pair x (the next one) and computes pair
  // c while they are in flight; the table entries of the pair after x are
  // read (through the scalar cache) in the same step.  The two register
  // sets swap roles every step, so no load result is ever copied.  The
  // loads of x are issued past the end too (a missing tile reads row0 = 0):
  // a load issued on one path only would make the compiler's wait counts
  // assume the worst for every load.
  const int npairs = (ntiles + 1) / 2;
  if (wid < npairs) {
    int pi = wid;
    Tile c0 = tile_at(2 * pi), c1 = tile_at(2 * pi + 1);
    Tile x0 = tile_at(2 * (pi + kSW)), x1 = tile_at(2 * (pi + kSW) + 1);
    TileData bufA[2], bufB[2];
    load_tile(c0, bufA[0]);
    load_tile(c1, bufA[1]);
    auto pair_step = [&](TileData (&cb)[2], TileData (&nb)[2]) -> bool {
      stage(c0, cb[0], 0);
      stage(c1, cb[1], 1);
      wave_lds_sync();
      load_tile(x0, nb[0]);
      load_tile(x1, nb[1]);
      const Tile y0 = tile_at(2 * (pi + 2 * kSW)), y1 = tile_at(2 * (pi + 2 * kSW) + 1);
      step(c0, c1);
      pi += kSW;
      c0 = x0;
      c1 = x1;
      x0 = y0;
      x1 = y1;
      return pi < npairs;
    };
    for (;;) {
      if (!pair_step(bufA, bufB)) break;
      if (!pair_step(bufB, bufA)) break;
    }
  }

  // this wavefront's partial (over its own tile buffers): lane l writes row
  // l % 16, dims 16 dt + 4 grp .. + 3
  float lsum = l_run + xor_lane<16>(l_run);
  lsum += xor_lane<32>(lsum);
  float(*pw)[D + 2] = partw(wid);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    *(float4*)&pw[row][16 * dt + 4 * grp] = make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
  if (grp == 0) {
    pw[row][D] = m_run;
    pw[row][D + 1] = lsum;
  }
  __syncthreads();

  // merge the wavefronts' partials: thread t takes row t / 32, dims 4 (t % 32) .. + 3
  {
    const int t = threadIdx.x;
    const int r = t >> 5;
    const int d0 = (t & 31) * 4;
    const int mb = r / a.G;
    if (r < kRows && mb < nm) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kSW; ++w) M = fmaxf(M, partw(w)[r][D]);
      float L = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kSW; ++w) {
        const float mw = partw(w)[r][D];
        const float ww = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        L = fmaf(ww, partw(w)[r][D + 1], L);
        const float4 x = *(const float4*)&partw(w)[r][d0];
        o[0] = fmaf(ww, x.x, o[0]);
        o[1] = fmaf(ww, x.y, o[1]);
        o[2] = fmaf(ww, x.z, o[2]);
        o[3] = fmaf(ww, x.w, o[3]);
      }
      const float inv = 1.f / L;  // a member with no key at all (context 0) gives NaN here; written as zeros below
      const int ctx = min(a.ctx_lens[g0 + mb], maxctx);
      uint16_t* op = a.out + ((size_t)(g0 + mb) * a.Hq + (size_t)h * a.G + r % a.G) * D + d0;
      const uint2 v = ctx > 0 ? make_uint2(pack2_bf16_rne(o[0] * inv, o[1] * inv), pack2_bf16_rne(o[2] * inv, o[3] * inv))
                              : make_uint2(0u, 0u);
      *(uint2*)op = v;
    }
    // members past the largest group this kernel stacks come out NaN
    const int extra = min(g1, a.S) - (g0 + nm);
    for (int i = threadIdx.x; i < extra * a.G * (D / 4); i += 64 * kSW) {
      const int mb = nm + i / (a.G * (D / 4));
      const int rem = i % (a.G * (D / 4));
      uint16_t* op = a.out + ((size_t)(g0 + mb) * a.Hq + (size_t)h * a.G + rem / (D / 4)) * D + (rem % (D / 4)) * 4;
      *(uint2*)op = make_uint2(0x7fc07fc0u, 0x7fc07fc0u);
    }
  }
}

bool decode_shared_supported(int dtype, int head_dim, int group, int block_size) {
  return dtype == 1 && head_dim == 128 && group >= 1 && group <= kRows && block_size >= 16 && block_size <= 256 &&
         (block_size & (block_size - 1)) == 0;
}

int max_shared_members(int group) { return std::min(kMaxMembers, kRows / std::max(group, 1)); }

int launch_decode_shared(void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* tables,
                         int max_blocks, const int32_t* ctx, int S, const int32_t* group_start,
                         const int32_t* shared_blocks, int num_groups, int Hq, int Hkv, int D, int B, int num_blocks,
                         float scale, hipStream_t stream) {
  SharedArgs a;
  a.out = (uint16_t*)out;
  a.q = (const uint16_t*)q;
  a.k_cache = (const uint16_t*)k_cache;
  a.v_cache = (const uint16_t*)v_cache;
  a.tables = tables;
  a.ctx_lens = ctx;
  a.group_start = group_start;
  a.shared_blocks = shared_blocks;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.max_blocks = max_blocks;
  a.num_blocks = num_blocks;
  a.log2B = 0;
  while ((1 << a.log2B) < B) ++a.log2B;
  a.num_groups = num_groups;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  if (D != 128) return -2;
  const long long grid = (long long)num_groups * Hkv;
  if (grid <= 0) return 0;
  if (grid > 0x7fffffffLL) return -2;
  hipLaunchKernelGGL(decode_shared_kernel<128>, dim3((unsigned)grid), dim3(64 * kSW), 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace pkv
