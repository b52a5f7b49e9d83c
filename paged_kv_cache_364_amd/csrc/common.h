// Shared device helpers for the gfx950 kernels: element conversions, 16-byte
// vector moves and cross-lane primitives of a 64-lane wavefront.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }

// bf16 is handled as raw 16-bit patterns.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// float -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return f32_to_bf16(a) | (f32_to_bf16(b) << 16);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

// fp32 += a.lo*b.lo + a.hi*b.hi on packed bf16 pairs (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// ---- cross-lane moves ------------------------------------------------------
// DPP controls (gfx9 encoding).
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppQuadRev = 0x1B;   // quad_perm [3,2,1,0]  (lane ^ 3)
constexpr int kDppRowHalfMirror = 0x141;  // lane ^ 7 inside 8 lanes
constexpr int kDppRowMirror = 0x140;      // lane ^ 15 inside 16 lanes

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// ds_swizzle in bit-mask mode: partner = lane ^ XOR inside groups of 32.
template <int XOR>
__device__ __forceinline__ float swizzle_xor(float v) {
  static_assert(XOR > 0 && XOR < 32, "swizzle xor mask");
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x1F | (XOR << 10)));
}

__device__ __forceinline__ float bpermute(float v, int src_lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src_lane << 2, __builtin_bit_cast(int, v)));
}

// Value of lane ^ MASK (MASK a power of two).
template <int MASK>
__device__ __forceinline__ float xor_lane(float v) {
  if constexpr (MASK == 1) {
    return dpp<kDppQuadXor1>(v);
  } else if constexpr (MASK == 2) {
    return dpp<kDppQuadXor2>(v);
  } else if constexpr (MASK < 32) {
    return swizzle_xor<MASK>(v);
  } else {
    return bpermute(v, (int)(threadIdx.x & 63) ^ MASK);
  }
}

// Partner used by stage B of a transpose-reduce: any lane whose bits above B
// equal ours and whose bit B differs.  Mirrors inside rows are cheaper than
// exact xors on gfx9 DPP.
template <int B>
__device__ __forceinline__ float stage_partner(float v) {
  if constexpr (B == 0) {
    return dpp<kDppQuadXor1>(v);
  } else if constexpr (B == 1) {
    return dpp<kDppQuadRev>(v);
  } else if constexpr (B == 2) {
    return dpp<kDppRowHalfMirror>(v);
  } else if constexpr (B == 3) {
    return dpp<kDppRowMirror>(v);
  } else if constexpr (B == 4) {
    return swizzle_xor<16>(v);
  } else {
    return bpermute(v, (int)(threadIdx.x & 63) ^ 32);
  }
}

// Transpose-reduce of N partial sums over aligned groups of LR lanes
// (N <= LR, both powers of two).  On entry each lane holds v[0..N-1], its
// partial sums of N different outputs; on exit every lane holds the full sum
// over its group of output index (lane_in_group >> log2(LR / N)).  The top
// log2(N) lane bits are transposed (each stage keeps half the outputs and
// ships the other half to the partner), the remaining low bits are summed.
template <int N, int B, int SHIFT>
__device__ __forceinline__ void transpose_stage(float (&v)[N], int lane_in_group) {
  constexpr int HALF = 1 << (B - SHIFT);
  const bool up = (lane_in_group >> B) & 1;
#pragma unroll
  for (int m = 0; m < HALF; ++m) {
    const float keep = up ? v[m + HALF] : v[m];
    const float send = up ? v[m] : v[m + HALF];
    v[m] = keep + stage_partner<B>(send);
  }
}

template <int N, int LR, int B>
__device__ __forceinline__ void transpose_stages(float (&v)[N], int lane_in_group) {
  constexpr int SHIFT = ilog2(LR) - ilog2(N);
  if constexpr (B >= SHIFT && B >= 0) {
    transpose_stage<N, B, SHIFT>(v, lane_in_group);
    transpose_stages<N, LR, B - 1>(v, lane_in_group);
  }
}

template <int B>
__device__ __forceinline__ float sum_stages(float x) {
  if constexpr (B >= 0) {
    x += stage_partner<B>(x);
    return sum_stages<B - 1>(x);
  } else {
    return x;
  }
}

template <int N, int LR>
__device__ __forceinline__ float transpose_reduce(float (&v)[N], int lane_in_group) {
  static_assert((N & (N - 1)) == 0 && (LR & (LR - 1)) == 0 && N >= 1 && N <= LR && LR <= 64, "group size");
  transpose_stages<N, LR, ilog2(LR) - 1>(v, lane_in_group);
  return sum_stages<ilog2(LR) - ilog2(N) - 1>(v[0]);
}

// Value of lane ^ (1 << B) for reductions; inside full 16-lane rows a row
// rotation by 1 << B reaches the same set of lanes and stays on DPP.
template <int B, bool FULL_ROWS>
__device__ __forceinline__ float reduce_partner(float v) {
  if constexpr (FULL_ROWS && (B == 2 || B == 3)) {
    return dpp<0x120 + (1 << B)>(v);  // row_ror
  } else {
    return xor_lane<(1 << B)>(v);
  }
}

// Reduce over lane-index bits [LO, HI): every lane gets the result of its
// group (lanes that agree on all other bits).  FULL_ROWS: the bits
// [LO, HI) together with the bits below LO cover whole 16-lane rows, so a
// row rotation keeps the lower bits unchanged modulo the group.
template <int LO, int HI, bool FULL_ROWS = false>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (LO < HI) {
    v = fmaxf(v, reduce_partner<LO, FULL_ROWS>(v));
    return group_max<LO + 1, HI, FULL_ROWS>(v);
  } else {
    return v;
  }
}

template <int LO, int HI, bool FULL_ROWS = false>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LO < HI) {
    v = v + reduce_partner<LO, FULL_ROWS>(v);
    return group_sum<LO + 1, HI, FULL_ROWS>(v);
  } else {
    return v;
  }
}

// Intra-wavefront LDS hand-off: the LDS unit runs one wavefront's
// instructions in order, so only the compiler has to be kept from moving
// memory operations across this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace pkv
