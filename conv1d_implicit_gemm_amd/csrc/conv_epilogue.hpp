// Epilogue shared by the split-path implicit-GEMM convolution kernels.
//
// The workgroup tile is TM = WGM*WM*16 output positions x TN = WGN*WN*16
// output channels; wave (wm, wn) owns WM x WN MFMA 16x16 tiles, lane
// (lr = lane%16, kq = lane/16) holding rows t = 4*kq + r (r = 0..3) of column
// c = lr of each tile.
//
//   EPI_STORE    y = acc + bias, stored as fp32 or (y_bf16) rounded to bf16
//   EPI_GN_PART  also, per channel, (mean, M2) over the tile's valid
//                positions -> part[(n*C_out + c)*n_ttiles + ttile]
//   EPI_LN_PART  also, per position, (mean, M2) over the tile's valid
//                channels  -> part[(n*n_ctiles + ctile)*T_out + t]
//
// Partial statistics are taken from the fp32 values, before any rounding of
// the stored y.  Two passes over the registers (mean, then squared
// deviations), cross-lane sums (DPP and lane swaps), then a fixed-order pairwise
// merge across waves through LDS; every partial has one fixed slot (no
// atomics), so the later merge is deterministic.
//
// Waves with active == false (extra waves of a workgroup whose results were
// already folded into the active ones) store nothing but reach every barrier.
// With store_y == false only the bias is added and the partials written (the
// persistent kernel normalises the registers afterwards).
#pragma once

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace c1g {

// A partial (mean, M2) pair.  coherent: written as one device-scope atomic
// 64-bit store, which goes to the point of coherence of all XCDs (the
// persistent kernel's workgroups on other XCDs read it right after a barrier,
// with no cache-wide flush in between).
__device__ __forceinline__ void store_partial(float* p, float mean, float m2, bool coherent) {
  if (coherent) {
    const uint64_t bits = (uint64_t)__float_as_uint(mean) | ((uint64_t)__float_as_uint(m2) << 32);
    __hip_atomic_store((uint64_t*)p, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    *(f32x2*)p = f32x2{mean, m2};
  }
}
__device__ __forceinline__ f32x2 load_partial_coherent(const float* p) {
  const uint64_t bits = __hip_atomic_load((const uint64_t*)p, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
  return f32x2{__uint_as_float((uint32_t)bits), __uint_as_float((uint32_t)(bits >> 32))};
}

// y = acc (bias already added) in the output type TO (float, or bf16 bits);
// four consecutive positions of one channel per lane and tile.
template <typename TO, int WM, int WN, int WGM, int WGN>
__device__ __forceinline__ void conv_store(const ConvArgs& a, const f32x4 (&acc)[WM][WN],
                                           int64_t n, int64_t t0, int c0, int wm, int wn) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, kq = lane >> 4;
  const int64_t T_out = a.T_out;
  TO* y = (TO*)a.y;
  const bool vec_ok = ((T_out & 3) == 0) && ((((uintptr_t)y) & (4 * sizeof(TO) - 1)) == 0);
#pragma unroll
  for (int jn = 0; jn < WN; ++jn) {
    const int c = c0 + wn * WN * 16 + jn * 16 + lr;
    if (c >= a.C_out) continue;
    TO* dst = y + (n * a.C_out + c) * T_out;
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      const int64_t t = t0 + wm * WM * 16 + i * 16 + 4 * kq;
      if (vec_ok && t + 3 < T_out) {
        store_elem4(dst + t, acc[i][jn]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t + r < T_out) store_elem(dst + t + r, acc[i][jn][r]);
      }
    }
  }
}

// GroupNorm statistics of this wave's positions, per channel: lane (lr, kq == 0)
// of wave (wm, wn) writes red[wm * TN + channel-in-tile] = (count, mean, M2)
// over the wave's valid positions (two passes over the registers, cross-lane
// sums).  The caller synchronises before reading red.
template <int WM, int WN, int WGM, int WGN>
__device__ __forceinline__ void gn_wave_channel_stats(const ConvArgs& a,
                                                      const f32x4 (&acc)[WM][WN], int64_t t0,
                                                      int wm, int wn, Stats* red, bool active) {
  constexpr int TN = WGN * WN * 16;
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, kq = lane >> 4;
  const int64_t T_out = a.T_out;
  // the wave's valid positions: the same count for every channel
  const int64_t vt64 = T_out - (t0 + wm * WM * 16);
  const int vt = (int)(vt64 < 0 ? 0 : (vt64 < WM * 16 ? vt64 : WM * 16));
  const float cnt = (float)vt;
  // The sums of the four channel columns of a lane at once, their cross-lane
  // sums together (four independent chains per step), then the squared
  // deviations the same way.  FULL: every position of the wave valid (all but
  // the last position tile), no masks.
  auto cols = [&](auto full_tag) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (FULL || i * 16 + 4 * kq + r < vt) {
#pragma unroll
          for (int jn = 0; jn < WN; ++jn) sum[jn] += acc[i][jn][r];
        }
    const f32x4 mean = cnt > 0.f ? lane_sum4<48>(sum) / cnt : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 m2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (FULL || i * 16 + 4 * kq + r < vt) {
#pragma unroll
          for (int jn = 0; jn < WN; ++jn) {
            const float dv = acc[i][jn][r] - mean[jn];
            m2[jn] += dv * dv;
          }
        }
    m2 = lane_sum4<48>(m2);
    if (active && kq == 0) {
#pragma unroll
      for (int jn = 0; jn < WN; ++jn)
        red[wm * TN + wn * WN * 16 + jn * 16 + lr] = Stats{cnt, mean[jn], m2[jn]};
    }
  };
  static_assert(WN == 4, "four channel columns per lane");
  if (vt == WM * 16)
    cols(std::true_type{});
  else
    cols(std::false_type{});
}

template <int WM, int WN, int WGM, int WGN>
__device__ __forceinline__ void conv_epilogue(const ConvArgs& a, int epi,
                                              f32x4 (&acc)[WM][WN], int64_t n, int64_t t0,
                                              int c0, int ttile, int ctile, int wm, int wn,
                                              Stats* red, bool active = true,
                                              bool store_y = true) {
  const bool coherent = !store_y;  // the persistent kernel's partials
  constexpr int TM = WGM * WM * 16, TN = WGN * WN * 16;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int lr = lane & 15, kq = lane >> 4;
  const int64_t T_out = a.T_out;
  // all bias loads before the first store: a load issued between stores would
  // make its wait also wait for every store before it
  float bias[WN];
#pragma unroll
  for (int jn = 0; jn < WN; ++jn) {
    const int c = c0 + wn * WN * 16 + jn * 16 + lr;
    bias[jn] = (a.bias != nullptr && c < a.C_out) ? a.bias[c] : 0.f;
  }
#pragma unroll
  for (int jn = 0; jn < WN; ++jn)
#pragma unroll
    for (int i = 0; i < WM; ++i) acc[i][jn] += bias[jn];
  if (active && store_y) {
    if (a.y_bf16)
      conv_store<uint16_t, WM, WN, WGM, WGN>(a, acc, n, t0, c0, wm, wn);
    else
      conv_store<float, WM, WN, WGM, WGN>(a, acc, n, t0, c0, wm, wn);
  }
  if (epi == EPI_STORE) return;

  __syncthreads();  // the staging LDS is free again: reuse it for the cross-wave merge

  if (epi == EPI_GN_PART) {
    gn_wave_channel_stats<WM, WN, WGM, WGN>(a, acc, t0, wm, wn, red, active);
    __syncthreads();
    for (int cl = tid; cl < TN; cl += blockDim.x) {
      const int c = c0 + cl;
      if (c < a.C_out) {
        Stats st = red[cl];
#pragma unroll
        for (int w = 1; w < WGM; ++w) st = stats_merge(st, red[w * TN + cl]);
        store_partial(a.part + ((n * a.C_out + c) * a.n_ttiles + ttile) * 2, st.mean, st.m2,
                      coherent);
      }
    }
  } else {  // EPI_LN_PART
    // the wave's valid channels: the same count for every position
    const int vc = a.C_out - (c0 + wn * WN * 16);
    const float cnt = (float)(vc < 0 ? 0 : (vc < WN * 16 ? vc : WN * 16));
    const float inv = cnt > 0.f ? 1.0f / cnt : 0.f;
    // Per MFMA row block, the four positions of a lane at once: their sums
    // over the lane's channels, cross-lane sums of all four together (four
    // independent chains per step), then the same for the squared deviations.
    // FULL: every channel of the wave inside C_out (all but a ragged last
    // channel tile), no masks.
    auto rows = [&](auto full_tag) __attribute__((always_inline)) {
      constexpr bool FULL = decltype(full_tag)::value;
      bool cin[WN];
#pragma unroll
      for (int jn = 0; jn < WN; ++jn) cin[jn] = FULL || (jn * 16 + lr < vc);
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jn = 0; jn < WN; ++jn)
          if (cin[jn]) sum += acc[i][jn];
        const f32x4 mean = lane_sum4<15>(sum) * inv;
        f32x4 m2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jn = 0; jn < WN; ++jn)
          if (cin[jn]) {
            const f32x4 dv = acc[i][jn] - mean;
            m2 += dv * dv;
          }
        m2 = lane_sum4<15>(m2);
        if (active && lr == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            red[wn * TM + wm * WM * 16 + i * 16 + 4 * kq + r] = Stats{cnt, mean[r], m2[r]};
        }
      }
    };
    if (vc >= WN * 16)
      rows(std::true_type{});
    else
      rows(std::false_type{});
    __syncthreads();
    for (int tl = tid; tl < TM; tl += blockDim.x) {
      const int64_t t = t0 + tl;
      if (t < T_out) {
        Stats st = red[tl];
#pragma unroll
        for (int w = 1; w < WGN; ++w) st = stats_merge(st, red[w * TM + tl]);
        store_partial(a.part + ((n * a.n_ctiles + ctile) * T_out + t) * 2, st.mean, st.m2,
                      coherent);
      }
    }
  }
}

}  // namespace c1g
