// Paged decode attention for gfx950.
//
// Computes out[s][h] = softmax(scale * q[s][h] . K_s^T) V_s where the keys and
// values of sequence s are found through its block table: position ->
// logical block -> physical block (cnblogs "paged attention", section 5; the
// formula itself is unchanged, section 6).  Decode reads the sequence's whole
// history every step ("08. PagedAttention", section "what it does not
// solve"), so this kernel is bound by HBM bandwidth.
//
// Work split.  The unit of work is a chunk of NT tokens of one (kv head,
// sequence): NT = 64 / G when a row of K fits in at most 16 lanes, fewer
// for wider rows so that a chunk never holds more than four 16-byte loads
// of K and of V per lane.  All chunks of the batch are laid end to end, kv head
// major, and every wavefront of a persistent grid takes an equal contiguous
// share (stream-K style), so ragged context lengths do not unbalance the
// chip.  A (kv head, sequence) whose chunks fall to one wavefront is finished
// there; one that spans several wavefronts leaves fp32 partials (unnormalised
// output, running max, running sum) in the workspace, and a second kernel
// combines them with their log-sum-exp weights.  This is the block-wise
// evaluation with a merge of partial results of the intelliparadigm.com
// article, section 2.2.
//
// Each wavefront walks its share as one pipelined stream of chunks: the
// loads of chunk i + 1 are in flight while chunk i is computed, also across
// the boundary between two (kv head, sequence) units, whose block-table
// window and query rows are fetched as soon as the previous unit starts.
//
// Inside a chunk.  Lanes load the K and V rows with coalesced 16-byte
// non-temporal loads straight into registers: lane l holds 16 bytes (piece l % LR) of row
// (l / LR) + j * RW for j < J.  All G query heads of the KV head share those
// registers (grouped-query attention, cnblogs section 6).  QK^T partial sums
// are finished by a DPP transpose-reduce inside each row group, leaving each
// (token, head) score in one lane (or a few identical lanes).  Online softmax state is kept per row group
// and head; softmax weights reach the P.V lanes through 256 bytes of LDS.
// P.V accumulates in fp32 registers; row groups are combined once per
// segment.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace pkv {

// 16-byte load that does not keep the line in the caches: each K/V byte of
// a decode step is read once, so there is nothing to gain by caching it,
// and streaming past the caches reads faster on this chip.
__device__ __forceinline__ uint4 load_stream(const void* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(t.x, t.y, t.z, t.w);
}

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* tables;
  const int32_t* ctx_lens;
  float* part;  // two partial slots of PSZ floats per wavefront
  int2* jobs;   // per wavefront: (unit, last wavefront) of the unit it starts, or (-1, 0)
  // Append variant: K/V rows [S][Hkv][D] of the token at position ctx - 1 of
  // each sequence, attended from here and stored into the cache.
  const void* k_new;
  const void* v_new;
  int S, Hq, Hkv, max_blocks, num_blocks, log2B, nW;
  int window;   // > 0: attend only the last `window` tokens of each context
  float scale_log2;
};

template <typename T, int D, int G>
struct DShape {
  static constexpr int ES = (int)sizeof(T);
  static constexpr int E = 16 / ES;       // elements per 16-byte piece
  static constexpr int LR = D * ES / 16;  // lanes per row
  static constexpr int RW = 64 / LR;      // rows per wavefront load
  static constexpr int JMAX = 4;          // loads per chunk and tensor, at most
  static constexpr int J = (LR / G < JMAX) ? LR / G : JMAX;
  static constexpr int NT = RW * J;       // tokens per chunk
  static constexpr int NS = J * G;        // scores per row group and chunk
  static constexpr int SH = ilog2(LR / NS);  // lanes sharing one score: 1 << SH
  static constexpr bool FULL_ROWS = LR >= 16;
  static constexpr int PSZ = G * (D + 2);
  static constexpr int OPL = (G * D >= 64) ? G * D / 64 : 1;
  static constexpr int OUT_LANES = G * D / OPL;
  // LDS (floats): p[RW*NS] | alpha[RW*G] | m[RW*G] | l[RW*G] | acc[RW*G*D]
  static constexpr int OFF_ALPHA = RW * NS;
  static constexpr int OFF_M = OFF_ALPHA + RW * G;
  static constexpr int OFF_L = OFF_M + RW * G;
  static constexpr int OFF_ACC = OFF_L + RW * G;
  static constexpr int LDS_FLOATS = OFF_ACC + RW * G * D;
  static_assert(LR >= G && LR <= 32 && J >= 1 && NS <= LR, "unsupported (dtype, head_dim, group) combination");
};

constexpr int kWavesPerWG = 4;

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ int wave_incl_scan_i(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

template <typename T>
__device__ __forceinline__ void store_out(void* out, size_t idx, const float* v, int n);

template <>
__device__ __forceinline__ void store_out<float>(void* out, size_t idx, const float* v, int n) {
  float* o = (float*)out + idx;
  if (n % 4 == 0) {
    for (int i = 0; i < n; i += 4) *(float4*)(o + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
  } else {
    for (int i = 0; i < n; ++i) o[i] = v[i];
  }
}

template <>
__device__ __forceinline__ void store_out<bf16_t>(void* out, size_t idx, const float* v, int n) {
  uint16_t* o = (uint16_t*)out + idx;
  if (n % 8 == 0) {
    for (int i = 0; i < n; i += 8)
      *(uint4*)(o + i) = make_uint4(pack_bf16x2(v[i], v[i + 1]), pack_bf16x2(v[i + 2], v[i + 3]),
                                    pack_bf16x2(v[i + 4], v[i + 5]), pack_bf16x2(v[i + 6], v[i + 7]));
  } else {
    for (int i = 0; i < n; ++i) o[i] = (uint16_t)f32_to_bf16(v[i]);
  }
}

// Dot product of a 16-byte piece of q and of k.
template <typename T>
__device__ __forceinline__ float dot16(const uint4& q, const uint4& k);

template <>
__device__ __forceinline__ float dot16<bf16_t>(const uint4& q, const uint4& k) {
  float d = dot2_bf16(q.x, k.x, 0.f);
  d = dot2_bf16(q.y, k.y, d);
  d = dot2_bf16(q.z, k.z, d);
  return dot2_bf16(q.w, k.w, d);
}

template <>
__device__ __forceinline__ float dot16<float>(const uint4& q, const uint4& k) {
  float d = __uint_as_float(q.x) * __uint_as_float(k.x);
  d = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), d);
  d = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), d);
  return fmaf(__uint_as_float(q.w), __uint_as_float(k.w), d);
}

template <typename T>
__device__ __forceinline__ void unpack16(const uint4& v, float* f);

template <>
__device__ __forceinline__ void unpack16<bf16_t>(const uint4& v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

template <>
__device__ __forceinline__ void unpack16<float>(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}

template <typename T, int D, int G>
struct Chunk {
  uint4 k[DShape<T, D, G>::J];
  uint4 v[DShape<T, D, G>::J];
  int ok;   // bit j: row j holds a valid token with a valid block
  int bad;  // bit j: row j is a valid token whose block id is out of range
  long long app;  // append variant: byte offset of the new row in the kv head's cache, or -1
};

// One (kv head, sequence) unit as a wavefront sees it.  Lane i of win0 /
// win1 holds table entry wbase + i / wbase + 64 + i (-1 past the context).
template <typename T, int D, int G>
struct Unit {
  const char* kb;  // k_cache + kv head offset (bytes)
  const char* vb;
  const int32_t* trow;
  int h, s, ctx, n, g0;  // n chunks, the first of which is global chunk g0
  int lo, cf;            // first attended token (sliding window) and its chunk
  int nblk, wbase;
  int win0, win1;
  const char* kn;  // append variant: this unit's new K and V rows (null: none)
  const char* vn;
  uint4 qv[G];
};

template <typename T, int D, int G>
__device__ __forceinline__ int load_window(const Unit<T, D, G>& u, int base, int lane) {
  const int lb = base + lane;
  return lb < u.nblk ? u.trow[lb] : -1;
}

// Set up unit (h, s) starting at global chunk g0: issue the loads of its
// table window and query rows (nothing waits for them here).
template <typename T, int D, int G, bool APP>
__device__ __forceinline__ void open_unit(Unit<T, D, G>& u, const DecodeArgs& a, int h, int s, int ctx, int g0,
                                          int c0, int lane) {
  using SH = DShape<T, D, G>;
  const size_t rowb = (size_t)D * SH::ES;
  u.h = h;
  u.s = s;
  u.ctx = ctx;
  u.lo = a.window > 0 ? max(0, ctx - a.window) : 0;
  u.cf = u.lo / SH::NT;
  u.n = (ctx + SH::NT - 1) / SH::NT - u.cf;
  u.g0 = g0;
  u.nblk = (ctx + (1 << a.log2B) - 1) >> a.log2B;
  u.trow = a.tables + (size_t)s * a.max_blocks;
  u.kb = (const char*)a.k_cache + (size_t)h * ((size_t)1 << a.log2B) * rowb;
  u.vb = (const char*)a.v_cache + (size_t)h * ((size_t)1 << a.log2B) * rowb;
  u.wbase = ((c0 + u.cf) * SH::NT) >> a.log2B;
  u.win0 = load_window(u, u.wbase, lane);
  u.win1 = load_window(u, u.wbase + 64, lane);
  if constexpr (APP) {
    const size_t no = ((size_t)s * a.Hkv + h) * rowb;
    u.kn = (const char*)a.k_new + no;
    u.vn = (const char*)a.v_new + no;
    // a context longer than the table (clamped to it for the attention) has
    // no slot for its new token: nothing is taken from the new rows or stored
    if (a.ctx_lens[s] > (a.max_blocks << a.log2B)) u.kn = u.vn = nullptr;
  }
  const char* qp = (const char*)a.q + ((size_t)s * a.Hq + (size_t)h * G) * rowb + (lane % SH::LR) * 16;
#pragma unroll
  for (int g = 0; g < G; ++g) u.qv[g] = *(const uint4*)(qp + g * rowb);
}

// Issue the loads of chunk c (counted from the unit's first attended chunk)
// of unit u.  Rows outside [lo, ctx), or whose block id is out of range, are
// zero; the latter are flagged so that the output turns into NaN instead of
// reading outside the pool.  Table entries of blocks wholly before lo are
// never read (a sliding window may have released them).  In the append
// variant the row of position ctx - 1 comes from the unit's new K/V row
// instead of the cache, and the chunk notes where that row goes in the
// cache (stored once the chunk has been computed).
template <typename T, int D, int G, bool APP>
__device__ __forceinline__ void load_chunk(Chunk<T, D, G>& ch, Unit<T, D, G>& u, const DecodeArgs& a, int c,
                                           int lane) {
  using SH = DShape<T, D, G>;
  const int rg = lane / SH::LR;
  const int cl = lane % SH::LR;
  const int t0 = (c + u.cf) * SH::NT;
  const int B = 1 << a.log2B;
  const int lb0 = t0 >> a.log2B;
  // slide the window once the chunk has moved into its upper half; the new
  // upper half is needed only 64 blocks later
  if (lb0 >= u.wbase + 64) {
    if (lb0 >= u.wbase + 128) {  // jumped past both halves
      u.wbase = lb0;
      u.win0 = load_window(u, u.wbase, lane);
    } else {
      u.wbase += 64;
      u.win0 = u.win1;
    }
    u.win1 = load_window(u, u.wbase + 64, lane);
  }
  const size_t rowb = (size_t)D * SH::ES;
  const size_t blkb = (size_t)a.Hkv << a.log2B;  // rows per physical block (all heads)
  ch.ok = 0;
  ch.bad = 0;
  // row of the new token, in this chunk if below NT (the same for every lane)
  const int rnew = APP && u.kn != nullptr ? u.ctx - 1 - t0 : SH::NT;
  if constexpr (APP) ch.app = -1;
  if (SH::NT <= B) {
    // the whole chunk lies in one block: one uniform table entry, one
    // uniform base address, a 32-bit offset per lane
    const int wi = lb0 - u.wbase;
    const int blk = wi < 64 ? __builtin_amdgcn_readlane(u.win0, wi) : __builtin_amdgcn_readlane(u.win1, wi - 64);
    const bool bok = (unsigned)blk < (unsigned)a.num_blocks;
    const size_t ub = ((size_t)blk * blkb + (size_t)(t0 & (B - 1))) * rowb;
    const char* kp = u.kb + ub;
    const char* vp = u.vb + ub;
    const int full = t0 >= u.lo && t0 + SH::NT <= u.ctx;
    if constexpr (APP) {
      if (bok && rnew < SH::NT) ch.app = (long long)(ub + (size_t)rnew * rowb);
    }
    const unsigned loff = (unsigned)(rg * D * SH::ES + cl * 16);
#pragma unroll
    for (int j = 0; j < SH::J; ++j) {
      const int r = rg + j * SH::RW;
      const unsigned off = loff + (unsigned)(j * SH::RW * D * SH::ES);
      const bool in = t0 + r >= u.lo && t0 + r < u.ctx;
      if (bok && (full || in)) {
        const char* ks = kp + off;
        const char* vs = vp + off;
        if constexpr (APP) {
          if (r == rnew) {
            ks = u.kn + cl * 16;
            vs = u.vn + cl * 16;
          }
        }
        ch.k[j] = load_stream(ks);
        ch.v[j] = load_stream(vs);
        ch.ok |= 1 << j;
      } else {
        ch.k[j] = make_uint4(0, 0, 0, 0);
        ch.v[j] = make_uint4(0, 0, 0, 0);
        if (in) ch.bad |= 1 << j;
      }
    }
  } else {
    if constexpr (APP) {
      if (rnew < SH::NT) {
        const int wn = ((u.ctx - 1) >> a.log2B) - u.wbase;  // the chunk holds it, so it is in the window
        const int bn = wn < 64 ? __builtin_amdgcn_readlane(u.win0, wn) : __builtin_amdgcn_readlane(u.win1, wn - 64);
        if ((unsigned)bn < (unsigned)a.num_blocks)
          ch.app = (long long)(((size_t)bn * blkb + ((u.ctx - 1) & (B - 1))) * rowb);
      }
    }
#pragma unroll
    for (int j = 0; j < SH::J; ++j) {
      const int t = t0 + rg + j * SH::RW;
      const int wi = (t >> a.log2B) - u.wbase;  // 0 .. 127 for rows inside the context
      const int b0 = __builtin_amdgcn_ds_bpermute((wi & 63) << 2, u.win0);
      const int b1 = __builtin_amdgcn_ds_bpermute((wi & 63) << 2, u.win1);
      const int blk = wi < 64 ? b0 : b1;
      ch.k[j] = make_uint4(0, 0, 0, 0);
      ch.v[j] = make_uint4(0, 0, 0, 0);
      if (t >= u.lo && t < u.ctx) {
        if ((unsigned)blk < (unsigned)a.num_blocks) {
          const size_t off = ((size_t)blk * blkb + (t & (B - 1))) * rowb + cl * 16;
          const char* ks = u.kb + off;
          const char* vs = u.vb + off;
          if constexpr (APP) {
            if (t - t0 == rnew) {
              ks = u.kn + cl * 16;
              vs = u.vn + cl * 16;
            }
          }
          ch.k[j] = load_stream(ks);
          ch.v[j] = load_stream(vs);
          ch.ok |= 1 << j;
        } else {
          ch.bad |= 1 << j;
        }
      }
    }
  }
}

// Online-softmax update with one chunk: scores of the chunk's rows for the
// G heads, running max m and sum lsum per (row group, head), and the
// rescaled P.V accumulation.
template <typename T, int D, int G>
__device__ __forceinline__ void compute_chunk(const Chunk<T, D, G>& ch, const uint4 (&qv)[G], int lane,
                                              float scale_log2, float& m, float& lsum,
                                              float (&acc)[G][16 / sizeof(T)], float* L) {
  using SH = DShape<T, D, G>;
  constexpr int E = SH::E;
  constexpr int LR = SH::LR;
  constexpr int NS = SH::NS;
  const int rg = lane / LR;
  const int cl = lane % LR;
  // QK^T partial sums over this lane's 16-byte piece: index j*G + g
  float part[NS];
#pragma unroll
  for (int j = 0; j < SH::J; ++j)
#pragma unroll
    for (int g = 0; g < G; ++g) part[j * G + g] = dot16<T>(qv[g], ch.k[j]);
  const float sc = transpose_reduce<NS, LR>(part, cl);
  // this lane now holds score k = cl >> SH: row j = k / G, head g = k % G
  const int k = cl >> SH::SH;
  const int jj = k / G;
  const bool valid = (ch.ok >> jj) & 1;
  const bool bad = (ch.bad >> jj) & 1;
  const float s = valid ? sc * scale_log2 : -INFINITY;
  const float cmax = group_max<SH::SH + ilog2(G), ilog2(LR), SH::FULL_ROWS>(s);
  // Lazy running max: the reference m moves only when the chunk's max
  // exceeds it by more than 2^8 (or on the first valid chunk), so the
  // accumulators are rescaled rarely; weights stay below 256 and the final
  // division by the sum taken against the same reference cancels it.
  const bool move = cmax > m + 8.f;  // m = -inf: moves on the first valid score
  const float mnew = move ? cmax : m;
  const float alpha = move ? __builtin_amdgcn_exp2f(m - mnew) : 1.f;
  const float p = valid ? __builtin_amdgcn_exp2f(s - mnew) : 0.f;
  lsum = lsum * alpha + p + (bad ? __builtin_nanf("") : 0.f);
  m = mnew;
  // any head of any row group whose reference moved?
  const bool rescale = __ballot(move) != 0;
  if ((cl & ((1 << SH::SH) - 1)) == 0) {
    L[rg * NS + k] = p;
    if (k < G) L[SH::OFF_ALPHA + rg * G + k] = alpha;
  }
  wave_lds_sync();
  float pp[NS];
  const float* prow = L + rg * NS;
  if constexpr (NS % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NS; i += 4) {
      const float4 x = *(const float4*)(prow + i);
      pp[i] = x.x; pp[i + 1] = x.y; pp[i + 2] = x.z; pp[i + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NS; ++i) pp[i] = prow[i];
  }
  if (rescale) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float al = L[SH::OFF_ALPHA + rg * G + g];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[g][e] *= al;
    }
  }
  wave_lds_sync();
#pragma unroll
  for (int j = 0; j < SH::J; ++j) {
    float vf[E];
    unpack16<T>(ch.v[j], vf);
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[g][e] = fmaf(pp[j * G + g], vf[e], acc[g][e]);
  }
}

// End of a segment: combine the row groups' (m, lsum, acc) and write either
// the normalised output (mode 0) or an unnormalised partial with its max and
// sum into slot 0 (mode 1) or slot 1 (mode 2) of wavefront w.
template <typename T, int D, int G>
__device__ __forceinline__ void finish_segment(const DecodeArgs& a, float* L, int lane, int w, int h, int s,
                                               int mode, float m, float lsum, const float (&acc)[G][16 / sizeof(T)]) {
  using SH = DShape<T, D, G>;
  constexpr int E = SH::E;
  const int rg = lane / SH::LR;
  const int cl = lane % SH::LR;
  const float lt = group_sum<SH::SH + ilog2(G), ilog2(SH::LR), SH::FULL_ROWS>(lsum);
  if (cl < (G << SH::SH) && (cl & ((1 << SH::SH) - 1)) == 0) {
    L[SH::OFF_M + rg * G + (cl >> SH::SH)] = m;
    L[SH::OFF_L + rg * G + (cl >> SH::SH)] = lt;
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float* dst = L + SH::OFF_ACC + (rg * G + g) * D + cl * E;
#pragma unroll
    for (int e = 0; e < E; e += 4) *(float4*)(dst + e) = make_float4(acc[g][e], acc[g][e + 1], acc[g][e + 2], acc[g][e + 3]);
  }
  wave_lds_sync();
  if (lane < SH::OUT_LANES) {
    constexpr int OPL = SH::OPL;
    const int o0 = lane * OPL;
    const int g = o0 / D;
    const int d0 = o0 % D;
    float M = -INFINITY;
#pragma unroll
    for (int r = 0; r < SH::RW; ++r) M = fmaxf(M, L[SH::OFF_M + r * G + g]);
    float res[OPL];
#pragma unroll
    for (int i = 0; i < OPL; ++i) res[i] = 0.f;
    float lt_all = 0.f;
#pragma unroll
    for (int r = 0; r < SH::RW; ++r) {
      const float mr = L[SH::OFF_M + r * G + g];
      const float wr = (mr == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mr - M);
      lt_all = fmaf(wr, L[SH::OFF_L + r * G + g], lt_all);
      const float* src = L + SH::OFF_ACC + (r * G + g) * D + d0;
#pragma unroll
      for (int i = 0; i < OPL; ++i) res[i] = fmaf(wr, src[i], res[i]);
    }
    if (mode == 0) {
#pragma unroll
      for (int i = 0; i < OPL; ++i) res[i] = res[i] / lt_all;
      store_out<T>(a.out, ((size_t)s * a.Hq + (size_t)h * G) * D + o0, res, OPL);
    } else {
      float* pp = a.part + ((size_t)w * 2 + (mode - 1)) * SH::PSZ;
      if constexpr (OPL % 4 == 0) {
#pragma unroll
        for (int i = 0; i < OPL; i += 4) *(float4*)(pp + o0 + i) = make_float4(res[i], res[i + 1], res[i + 2], res[i + 3]);
      } else {
#pragma unroll
        for (int i = 0; i < OPL; ++i) pp[o0 + i] = res[i];
      }
      if (d0 == 0) {
        pp[G * D + g] = M;
        pp[G * D + G + g] = lt_all;
      }
    }
  }
  wave_lds_sync();
}

// Chunks a unit of context ctx contributes: from the chunk of its first
// attended token to the chunk of its last.
__device__ __forceinline__ int chunks_of(int ctx, int maxctx, int nt, int window) {
  ctx = min(ctx, maxctx);
  if (ctx <= 0) return 0;
  const int lo = window > 0 ? max(0, ctx - window) : 0;
  return (ctx + nt - 1) / nt - lo / nt;
}

// Context lengths of batches up to this size are kept in LDS by every
// wavefront after its first read, so that later look-ups (the sequence
// holding the share's first chunk, the next unit) cost no memory round trip.
constexpr int kCtxCache = 512;

// Context length of sequence s, clamped to the table's capacity.
__device__ __forceinline__ int ctx_of(const DecodeArgs& a, const int* lc, int maxctx, int s) {
  return a.S <= kCtxCache ? lc[s] : min(a.ctx_lens[s], maxctx);
}

// Next non-empty unit after (h, s) in kv-head-major order; false at the end.
__device__ __forceinline__ bool next_unit(const DecodeArgs& a, const int* lc, int maxctx, int& h, int& s,
                                          int& ctx) {
  for (;;) {
    if (++s == a.S) {
      s = 0;
      if (++h == a.Hkv) return false;
    }
    ctx = ctx_of(a, lc, maxctx, s);
    if (ctx > 0) return true;
  }
}

// Store the new row of the unit's last chunk into the cache (append
// variant): the lanes that loaded it from the new K/V hold it in the chunk's
// registers, which the computation has already waited for.
template <typename T, int D, int G>
__device__ __forceinline__ void store_new_row(const Chunk<T, D, G>& ch, const Unit<T, D, G>& u, int c, int lane) {
  using SH = DShape<T, D, G>;
  if (ch.app < 0) return;
  const int rnew = u.ctx - 1 - (c + u.cf) * SH::NT;
  const int rg = lane / SH::LR;
  const size_t o = (size_t)ch.app + (lane % SH::LR) * 16;
  // a test per lane and load (not an index computed once), so that the
  // registers are never indexed at run time
#pragma unroll
  for (int j = 0; j < SH::J; ++j)
    if (rg + j * SH::RW == rnew) {
      *(uint4*)(const_cast<char*>(u.kb) + o) = ch.k[j];
      *(uint4*)(const_cast<char*>(u.vb) + o) = ch.v[j];
    }
}

template <typename T, int D, int G, bool APP>
__global__ __launch_bounds__(256) void decode_main(DecodeArgs a) {
  using SH = DShape<T, D, G>;
  constexpr int E = SH::E;
  __shared__ __attribute__((aligned(16))) float lds[kWavesPerWG][SH::LDS_FLOATS];
  __shared__ int lds_ctx[kWavesPerWG][kCtxCache];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  int wg = blockIdx.x;
  const int nwg = gridDim.x;
  // Consecutive work shares go to workgroups on the same XCD (workgroups are
  // dealt to the 8 XCDs round robin), so sequences adjacent in the batch,
  // e.g. branches sharing a prompt, meet in one L2.
  if ((nwg & 7) == 0) wg = (wg & 7) * (nwg >> 3) + (wg >> 3);
  const int w = wg * kWavesPerWG + wid;
  float* L = lds[wid];
  int* lc = lds_ctx[wid];
  constexpr int NT = SH::NT;
  const int maxctx = a.max_blocks << a.log2B;
  const int S = a.S;
  if (w >= a.nW) return;
  if (lane == 0) a.jobs[w] = make_int2(-1, 0);

  // Chunks per kv head, and this wavefront's share [gstart, gend), in one
  // round trip whatever the batch size: lane l sums the chunks of its own
  // contiguous segment of sequences (all of its loads in flight at once),
  // and a scan over the 64 segments finds the one holding chunk gstart.
  // Batches up to kCtxCache sequences (segments of at most 8) keep every
  // length in LDS; longer segments are walked again from memory.
  const int seg = (S + 63) / 64;  // sequences per lane segment
  const int sbeg = min(lane * seg, S), send = min(sbeg + seg, S);
  int my_n = 0;
  for (int si = sbeg; si < send; si += 8) {
    int cx[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) cx[j] = si + j < send ? a.ctx_lens[si + j] : 0;  // all eight loads in flight
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      my_n += chunks_of(cx[j], maxctx, NT, a.window);
      if (S <= kCtxCache && si + j < send) lc[si + j] = min(cx[j], maxctx);
    }
  }
  if (S <= kCtxCache) wave_lds_sync();

  // zero the outputs of empty sequences
  for (int s = w; s < S; s += a.nW) {
    if (ctx_of(a, lc, maxctx, s) <= 0) {
      const size_t n = (size_t)a.Hq * D;
      for (size_t i = lane; i < n; i += 64) {
        float z = 0.f;
        store_out<T>(a.out, (size_t)s * n + i, &z, 1);
      }
    }
  }

  const int seg_incl = wave_incl_scan_i(my_n, lane);
  const int W1 = __builtin_amdgcn_readlane(seg_incl, 63);
  const int Wtot = a.Hkv * W1;
  const int cpw = (Wtot + a.nW - 1) / max(a.nW, 1);
  const int gstart = w * cpw;
  const int gend = min(Wtot, gstart + cpw);
  if (gstart >= gend) return;
  // locate the unit holding chunk gstart
  int h = gstart / W1;
  const int rem = gstart - h * W1;
  int s = 0, P = 0;
  {
    const unsigned long long seg_hit = __ballot(seg_incl > rem);
    if (!seg_hit) return;  // context lengths changed under the kernel: do nothing
    const int ls = __ffsll((long long)seg_hit) - 1;  // lane whose segment holds it
    const int base = ls * seg;
    const int bend = min(base + seg, S);
    P = __builtin_amdgcn_readlane(seg_incl - my_n, ls);
    bool found = false;
    if (S <= kCtxCache) {
      // the segment's lengths are in LDS (at most 8)
      for (int si = base; si < bend && !found; ++si) {
        const int n = chunks_of(lc[si], maxctx, NT, a.window);
        if (P + n > rem) {
          s = si;
          found = true;
        } else {
          P += n;
        }
      }
    } else {
      // walked 64 sequences at a time
      for (int b0 = base; b0 < bend && !found; b0 += 64) {
        const int si = b0 + lane;
        const int n = si < bend ? chunks_of(a.ctx_lens[si], maxctx, NT, a.window) : 0;
        const int incl = wave_incl_scan_i(n, lane);
        const unsigned long long hit = __ballot(P + incl > rem);
        if (hit) {
          const int first = __ffsll((long long)hit) - 1;
          s = b0 + first;
          P += __builtin_amdgcn_readlane(incl - n, first);
          found = true;
        } else {
          P += __builtin_amdgcn_readlane(incl, 63);
        }
      }
    }
    if (!found) return;
  }

  Unit<T, D, G> cur, nxt;
  int c = rem - P;  // chunk of `cur` being computed
  open_unit<T, D, G, APP>(cur, a, h, s, ctx_of(a, lc, maxctx, s), gstart - c, c, lane);
  int seg_c0 = c;  // first chunk of cur in this wavefront's share
  bool have_next = false;
  {
    int h2 = h, s2 = s, ctx2 = 0;
    if (cur.g0 + cur.n < gend && next_unit(a, lc, maxctx, h2, s2, ctx2)) {
      open_unit<T, D, G, APP>(nxt, a, h2, s2, ctx2, cur.g0 + cur.n, 0, lane);
      have_next = true;
    }
  }

  float m = -INFINITY, lsum = 0.f;
  float acc[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[g][e] = 0.f;

  // One step: prefetch the chunk after `i` into `nb`, compute chunk i from
  // `cb`, and close the unit when its last chunk (or the share) ends.
  // Returns false when the share is done.
  auto step = [&](Chunk<T, D, G>& cb, Chunk<T, D, G>& nb, int i) -> bool {
    if (i + 1 < gend) {
      if (c + 1 < cur.n) load_chunk<T, D, G, APP>(nb, cur, a, c + 1, lane);
      else load_chunk<T, D, G, APP>(nb, nxt, a, 0, lane);
    }
    compute_chunk<T, D, G>(cb, cur.qv, lane, a.scale_log2, m, lsum, acc, L);
    if constexpr (APP) {
      if (c == cur.n - 1) store_new_row<T, D, G>(cb, cur, c, lane);
    }
    ++c;
    if (c < cur.n && i + 1 < gend) return true;
    const int mode = seg_c0 > 0 ? 1 : (c < cur.n ? 2 : 0);
    finish_segment<T, D, G>(a, L, lane, w, cur.h, cur.s, mode, m, lsum, acc);
    if (mode == 2 && lane == 0) a.jobs[w] = make_int2(cur.h * S + cur.s, (cur.g0 + cur.n - 1) / cpw);
    if (i + 1 >= gend || !have_next) return false;
    cur = nxt;
    c = 0;
    seg_c0 = 0;
    have_next = false;
    int h2 = cur.h, s2 = cur.s, ctx2 = 0;
    if (cur.g0 + cur.n < gend && next_unit(a, lc, maxctx, h2, s2, ctx2)) {
      open_unit<T, D, G, APP>(nxt, a, h2, s2, ctx2, cur.g0 + cur.n, 0, lane);
      have_next = true;
    }
    m = -INFINITY;
    lsum = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[g][e] = 0.f;
    return true;
  };

  Chunk<T, D, G> ca, cb;
  load_chunk<T, D, G, APP>(ca, cur, a, c, lane);
  for (int i = gstart; i < gend; i += 2) {
    if (!step(ca, cb, i)) break;
    if (i + 1 >= gend || !step(cb, ca, i + 1)) break;
  }
}

// Second pass: log-sum-exp merge of the partials of every (kv head,
// sequence) that spans several wavefronts.  Job w names the unit whose first
// partial wavefront w wrote into slot 1 and the last wavefront holding one;
// the wavefronts in between wrote theirs into slot 0.  All loads of a pass
// are issued before any is used.
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void decode_merge(DecodeArgs a) {
  using SH = DShape<T, D, G>;
  const int lane = threadIdx.x & 63;
  // the main pass's mapping of workgroups to XCDs, so that a job's merge
  // runs on the XCD whose L2 holds most of its partials
  int wg = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) wg = (wg & 7) * (nwg >> 3) + (wg >> 3);
  const int w = wg * kWavesPerWG + (threadIdx.x >> 6);
  if (w >= a.nW) return;
  const int2 job = a.jobs[w];
  if (job.x < 0 || lane >= SH::OUT_LANES) return;
  const int h = job.x / a.S;
  const int s = job.x - h * a.S;
  constexpr int OPL = SH::OPL;
  const int o0 = lane * OPL;
  const int g = o0 / D;
  const int K = job.y - w + 1;
  auto slot = [&](int k) -> const float* {
    return a.part + ((size_t)(w + k) * 2 + (k == 0 ? 1 : 0)) * SH::PSZ;
  };
  // Batches of KB partials: all loads of a batch are issued before any is
  // used; the running max across batches rescales what was summed so far.
  constexpr int KB = 8;
  float M = -INFINITY, lt = 0.f;
  float res[OPL];
#pragma unroll
  for (int i = 0; i < OPL; ++i) res[i] = 0.f;
  for (int k0 = 0; k0 < K; k0 += KB) {
    float x[KB][OPL], mk[KB], lk[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      if (k0 + k < K) {
        const float* p = slot(k0 + k);
        mk[k] = p[G * D + g];
        lk[k] = p[G * D + G + g];
        if constexpr (OPL % 4 == 0) {
#pragma unroll
          for (int i = 0; i < OPL; i += 4) {
            const float4 v = *(const float4*)(p + o0 + i);
            x[k][i] = v.x; x[k][i + 1] = v.y; x[k][i + 2] = v.z; x[k][i + 3] = v.w;
          }
        } else {
#pragma unroll
          for (int i = 0; i < OPL; ++i) x[k][i] = p[o0 + i];
        }
      } else {
        mk[k] = -INFINITY;
        lk[k] = 0.f;
#pragma unroll
        for (int i = 0; i < OPL; ++i) x[k][i] = 0.f;
      }
    }
    float Mb = M;
#pragma unroll
    for (int k = 0; k < KB; ++k) Mb = fmaxf(Mb, mk[k]);
    const float r = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - Mb);
    lt *= r;
#pragma unroll
    for (int i = 0; i < OPL; ++i) res[i] *= r;
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const float wk = (mk[k] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mk[k] - Mb);
      lt = fmaf(wk, lk[k], lt);
#pragma unroll
      for (int i = 0; i < OPL; ++i) res[i] = fmaf(wk, x[k][i], res[i]);
    }
    M = Mb;
  }
#pragma unroll
  for (int i = 0; i < OPL; ++i) res[i] = res[i] / lt;
  store_out<T>(a.out, ((size_t)s * a.Hq + (size_t)h * G) * D + o0, res, OPL);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct DecodeKernels {
  const void* main;
  const void* main_app;  // the append variant
  const void* merge;
  int nt;
  int psz;
};

template <typename T, int D, int G>
static DecodeKernels kernels_for() {
  using SH = DShape<T, D, G>;
  return {(const void*)decode_main<T, D, G, false>, (const void*)decode_main<T, D, G, true>,
          (const void*)decode_merge<T, D, G>, SH::NT, SH::PSZ};
}
static bool pick(int dtype, int D, int G, DecodeKernels* k) {
#define PKV_CASE(TT, DD, GG)                      \
  if (D == DD && G == GG) {                       \
    *k = kernels_for<TT, DD, GG>();               \
    return true;                                  \
  }
  if (dtype == 1) {
    PKV_CASE(bf16_t, 16, 1) PKV_CASE(bf16_t, 16, 2)
    PKV_CASE(bf16_t, 32, 1) PKV_CASE(bf16_t, 32, 2) PKV_CASE(bf16_t, 32, 4)
    PKV_CASE(bf16_t, 64, 1) PKV_CASE(bf16_t, 64, 2) PKV_CASE(bf16_t, 64, 4) PKV_CASE(bf16_t, 64, 8)
    PKV_CASE(bf16_t, 128, 1) PKV_CASE(bf16_t, 128, 2) PKV_CASE(bf16_t, 128, 4) PKV_CASE(bf16_t, 128, 8)
  } else if (dtype == 0) {
    PKV_CASE(float, 16, 1) PKV_CASE(float, 16, 2) PKV_CASE(float, 16, 4)
    PKV_CASE(float, 32, 1) PKV_CASE(float, 32, 2) PKV_CASE(float, 32, 4) PKV_CASE(float, 32, 8)
    PKV_CASE(float, 64, 1) PKV_CASE(float, 64, 2) PKV_CASE(float, 64, 4) PKV_CASE(float, 64, 8)
    PKV_CASE(float, 128, 1) PKV_CASE(float, 128, 2) PKV_CASE(float, 128, 4) PKV_CASE(float, 128, 8)
  }
#undef PKV_CASE
  return false;
}

bool decode_supported(int dtype, int head_dim, int group) {
  DecodeKernels k;
  return pick(dtype, head_dim, group, &k);
}

// Number of wavefronts of the persistent grid: a fixed number of
// workgroups per compute unit (PKV_DECODE_WG_PER_CU overrides the device's
// occupancy limit), never more than the chunks there can be.  The append
// variant runs on the plain decode's grid, so that both split the chunks at
// the same points and round alike; where it fits fewer workgroups per
// compute unit (some small head dims), the rest wait for a slot, which is
// safe because no workgroup of the pass waits for another.
static int decode_waves(const DecodeKernels& k, int S, int Hkv, int max_blocks, int B) {
  const DeviceInfo& dev = device_info();
  int per_cu = occupancy(k.main, 64 * kWavesPerWG);
  const int force = tuning_int("PKV_DECODE_WG_PER_CU", 0);
  if (force > 0) per_cu = std::min(force, 8);
  long long wgs = (long long)per_cu * std::max(dev.num_cus, 1);
  const long long maxctx = (long long)max_blocks * B;
  const long long upper = (long long)Hkv * S * ((maxctx + k.nt - 1) / k.nt);
  long long need_wg = (upper + kWavesPerWG - 1) / kWavesPerWG;
  if (need_wg < wgs) wgs = need_wg;
  if (wgs < 1) wgs = 1;
  if (wgs > 8) wgs = wgs / 8 * 8;
  return (int)(wgs * kWavesPerWG);
}

// Workspace: two partial slots per wavefront, then one job entry per
// wavefront.
static size_t workspace_layout(const DecodeKernels& k, int nW, size_t* jobs_off) {
  const size_t part = (size_t)nW * 2 * k.psz * sizeof(float);
  *jobs_off = ((part + 255) / 256) * 256;
  return *jobs_off + (size_t)nW * sizeof(int2);
}

size_t decode_workspace_bytes(int dtype, int D, int G, int S, int Hkv, int max_blocks, int B) {
  DecodeKernels k;
  if (!pick(dtype, D, G, &k)) return 0;
  size_t off;
  return workspace_layout(k, decode_waves(k, S, Hkv, max_blocks, B), &off);
}

int launch_decode(void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* tables,
                  int max_blocks, const int32_t* ctx, int S, int Hq, int Hkv, int D, int B, int num_blocks,
                  int window, float scale, int dtype, void* ws, size_t ws_bytes, hipStream_t stream,
                  const void* k_new, const void* v_new) {
  DecodeKernels k;
  if (!pick(dtype, D, Hq / Hkv, &k)) return -2;
  if (k_new != nullptr && window > 0) return -2;
  const int nW = decode_waves(k, S, Hkv, max_blocks, B);
  size_t jobs_off;
  const size_t need = workspace_layout(k, nW, &jobs_off);
  if (ws == nullptr || ws_bytes < need) return -7;
  DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.tables = tables;
  a.ctx_lens = ctx;
  a.part = (float*)ws;
  a.jobs = (int2*)((char*)ws + jobs_off);
  a.k_new = k_new;
  a.v_new = v_new;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.max_blocks = max_blocks;
  a.num_blocks = num_blocks;
  a.log2B = 0;
  while ((1 << a.log2B) < B) ++a.log2B;
  a.nW = nW;
  a.window = window > 0 ? window : 0;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  const int grid = nW / kWavesPerWG;
  const void* main = k_new != nullptr ? k.main_app : k.main;
  hipLaunchKernelGGL((void (*)(DecodeArgs))main, dim3(grid), dim3(64 * kWavesPerWG), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return -6;
  hipLaunchKernelGGL((void (*)(DecodeArgs))k.merge, dim3(grid), dim3(64 * kWavesPerWG), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return -6;
  return 0;
}

// ---------------------------------------------------------------------------
// Decode without a caller workspace: the partials and merge jobs live in a
// fixed device array of this library (one copy per GPU, held until the
// process ends).  In host code the array's name is only a stand-in for the
// symbol; its device address, which differs per GPU, is looked up once per
// device and that address is what the kernels receive.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

static void* scratch_address(int dev) {
  static void* addr[64] = {};
  static std::mutex mu;
  if (dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

int launch_decode_scratch(void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* tables,
                          int max_blocks, const int32_t* ctx, int S, int Hq, int Hkv, int D, int B, int num_blocks,
                          float scale, int dtype, hipStream_t stream) {
  DecodeKernels k;
  if (!pick(dtype, D, Hq / Hkv, &k)) return -2;
  size_t jobs_off;
  if (workspace_layout(k, decode_waves(k, S, Hkv, max_blocks, B), &jobs_off) > (size_t)kDecodeScratchBytes)
    return -7;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return -6;
  void* ws = scratch_address(dev);
  if (ws == nullptr) return -6;
  return launch_decode(out, q, k_cache, v_cache, tables, max_blocks, ctx, S, Hq, Hkv, D, B, num_blocks, 0, scale,
                       dtype, ws, (size_t)kDecodeScratchBytes, stream);
}

}  // namespace pkv
