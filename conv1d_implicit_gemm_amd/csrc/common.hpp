// Device-side building blocks shared by the gfx950 kernels of the conv1d ->
// GroupNorm library: vector types, MFMA wrappers, wave reductions and the
// pairwise (count, mean, M2) merge used by every statistics reduction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace c1g {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// v_mfma_f32_16x16x4_f32.  Lane l supplies A[l%16][l/16] and B[l/16][l%16];
// the 16x16 result lives in lane (j + 16*(i/4)), register i%4.
__device__ __forceinline__ f32x4 mfma16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16 (gfx950).  Lane l supplies A[l%16][8*(l/16)+0..7]
// and B[8*(l/16)+0..7][l%16]; result layout as above.
__device__ __forceinline__ f32x4 mfma16x16x32bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Cross-lane exchanges that stay in the vector ALU (no LDS crossbar round
// trip): DPP within rows of 16 lanes, and gfx950's permlane swaps across rows.
// Every lane must be active.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i within 16
// (v of lane l, v of lane l ^ 16) and (v of lane l, v of lane l ^ 32), in
// lane order within each pair (the lower lane's value first)
__device__ __forceinline__ f32x2 pair16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ f32x2 pair32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Sum over the lanes whose indices differ only in the MASK bits; the low four
// mask bits must be contiguous from bit 0 (the row reduction pairs quads, then
// halves, then mirrored halves of a row).  Every lane of a group ends with the
// same bits (each step adds the same two partial sums; a + b == b + a).
template <int MASK>
__device__ __forceinline__ float lane_sum(float v) {
  static_assert(((MASK & 15) & ((MASK & 15) + 1)) == 0, "row bits contiguous from bit 0");
  if (MASK & 1) v += dpp<kDppXor1>(v);
  if (MASK & 2) v += dpp<kDppXor2>(v);
  if (MASK & 4) v += dpp<kDppHalfMirror>(v);
  if (MASK & 8) v += dpp<kDppMirror>(v);
  if (MASK & 16) { const f32x2 p = pair16(v); v = p[0] + p[1]; }
  if (MASK & 32) { const f32x2 p = pair32(v); v = p[0] + p[1]; }
  return v;
}
// lane_sum of the four elements of v at once: four independent chains per
// cross-lane step, so no step waits on the one before it.
template <int MASK>
__device__ __forceinline__ f32x4 lane_sum4(f32x4 v) {
  static_assert(((MASK & 15) & ((MASK & 15) + 1)) == 0, "row bits contiguous from bit 0");
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (MASK & 1) v[k] += dpp<kDppXor1>(v[k]);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (MASK & 2) v[k] += dpp<kDppXor2>(v[k]);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (MASK & 4) v[k] += dpp<kDppHalfMirror>(v[k]);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (MASK & 8) v[k] += dpp<kDppMirror>(v[k]);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (MASK & 16) { const f32x2 p = pair16(v[k]); v[k] = p[0] + p[1]; }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (MASK & 32) { const f32x2 p = pair32(v[k]); v[k] = p[0] + p[1]; }
  }
  return v;
}

// The smaller of a and b, or NaN if either is NaN: the row-min reduces like
// PyTorch's min over a dimension, which returns NaN for a row holding one
// (fminf would drop it).  One v_minimum3_f32 on gfx950.
__device__ __forceinline__ float min_nan(float a, float b) {
  return __builtin_elementwise_minimum(a, b);
}

// Minimum over lanes differing in bits 16 and 32 of the lane index (NaN if
// any of them holds one).
__device__ __forceinline__ float lane_min48(float v) {
  f32x2 p = pair16(v);
  v = min_nan(p[0], p[1]);
  p = pair32(v);
  return min_nan(p[0], p[1]);
}

// Running statistics of a set of values: count, mean and the sum of squared
// deviations from the mean (M2).  merge() is the pairwise update for two
// disjoint sets (Chan, Golub and LeVeque); it is exact in real arithmetic and
// its result does not depend on how a set was split, only the rounding does.
struct Stats {
  float n, mean, m2;
};

__device__ __forceinline__ Stats stats_merge(Stats a, Stats b) {
  float n = a.n + b.n;
  if (b.n == 0.f) return a;
  if (a.n == 0.f) return b;
  float delta = b.mean - a.mean;
  float fb = b.n / n;
  Stats r;
  r.n = n;
  r.mean = a.mean + delta * fb;
  r.m2 = a.m2 + b.m2 + delta * delta * a.n * fb;
  return r;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// fp32 -> bf16 bits, round to nearest even (gfx950 converts in hardware,
// v_cvt_pk_bf16_f32, two values per instruction).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ u32x2 f32x4_to_bf16(f32x4 v) {
  return __builtin_bit_cast(u32x2, __builtin_convertvector(v, bf16x4));
}

// Element access for the two output types: float, or bf16 held as its bits
// in uint16_t.  Values are always computed in fp32 and rounded on the store.
__device__ __forceinline__ float load_elem(const float* p) { return *p; }
__device__ __forceinline__ float load_elem(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void store_elem(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_elem(uint16_t* p, float v) { *p = f32_to_bf16(v); }
// four consecutive elements; p aligned to 4 elements
__device__ __forceinline__ void store_elem4(float* p, f32x4 v) { *(f32x4*)p = v; }
__device__ __forceinline__ void store_elem4(uint16_t* p, f32x4 v) { *(u32x2*)p = f32x4_to_bf16(v); }
// the same as non-temporal (streaming) stores, for final outputs that no
// later kernel of the call reads back
__device__ __forceinline__ void store_elem4_nt(float* p, f32x4 v) {
  __builtin_nontemporal_store(v, (f32x4*)p);
}
__device__ __forceinline__ void store_elem4_nt(uint16_t* p, f32x4 v) {
  __builtin_nontemporal_store(f32x4_to_bf16(v), (u32x2*)p);
}

}  // namespace c1g
