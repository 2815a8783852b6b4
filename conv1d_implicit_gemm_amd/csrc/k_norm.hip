// Normalisation kernels of the split path (all HBM- or latency-bound):
//   gn_merge   per-(n, c, t-tile) partials -> GroupNorm mean/rstd per (n, g)
//   gn_stats   GroupNorm mean/rstd straight from an fp32 y (slices of each
//              group in parallel, then a fixed-order merge)
//   gn_apply   out = (y - mean) * rstd * gamma + beta, per (n, g) statistics
//              (y and out fp32 or bf16; arithmetic in fp32)
//   ln_merge   per-(n, c-tile, t) partials -> LayerNorm-over-channels mean/rstd
//   ln_apply   the same affine with per-(n, t) statistics
//   rowmin     min over channels of the normalised value, plus bias2 broadcast
//
// Statistics follow "Kimi-K2.6 l2_p35" (GroupNorm over C/G channels x L per
// (n, g), population variance, eps inside the square root) and the
// statistics-then-apply split of "Kimi-K2.6 l2_p3"; the row-min epilogue is
// "Kimi-K2.6 l2_p75" (min over channels after the affine, bias2 broadcast).
// Every reduction runs in a fixed order (sequential per thread, then a fixed
// tree), so results are bit-identical from run to run.
#include "common.hpp"
#include "launch.hpp"

namespace c1g {
namespace {

constexpr int NT = 256;

__device__ __forceinline__ Stats block_merge(Stats st, Stats* sh) {
  const int tid = threadIdx.x;
  sh[tid] = st;
  __syncthreads();
#pragma unroll
  for (int s = NT / 2; s > 0; s >>= 1) {
    if (tid < s) sh[tid] = stats_merge(sh[tid], sh[tid + s]);
    __syncthreads();
  }
  return sh[0];
}

// Unsigned 32-bit division by a run-time constant (Granlund & Montgomery,
// round-up multiplier): q = (mulhi(m, n) + n) >> l with l = ceil(log2(d)).
struct FastDiv {
  uint32_t d, m, l;
  static FastDiv make(uint32_t d) {
    FastDiv f;
    f.d = d;
    uint32_t l = 0;
    while (l < 32 && (1ull << l) < d) ++l;
    f.l = l;
    f.m = (uint32_t)((((1ull << l) - d) << 32) / d + 1);
    return f;
  }
  __device__ __forceinline__ uint32_t div(uint32_t n) const {
    const uint64_t t = ((uint64_t)n * m) >> 32;
    return (uint32_t)((t + n) >> l);
  }
};

__global__ __launch_bounds__(NT) void gn_merge_kernel(const float* __restrict__ part, int64_t C,
                                                      int64_t L, int32_t G, int32_t n_ttiles,
                                                      int32_t tm, float eps, float* mean,
                                                      float* rstd) {
  __shared__ Stats sh[NT];
  const int64_t ng = blockIdx.x;
  const int64_t n = ng / G, g = ng - n * G;
  const int64_t cpg = C / G;
  const int64_t P = cpg * n_ttiles;
  const float* base = part + ((n * C + g * cpg) * n_ttiles) * 2;
  Stats st = {0.f, 0.f, 0.f};
  for (int64_t p = threadIdx.x; p < P; p += NT) {
    const int tt = (int)(p % n_ttiles);
    const int64_t cntl = L - (int64_t)tt * tm;
    const float cnt = (float)(cntl < tm ? cntl : tm);
    const f32x2 v = *(const f32x2*)(base + 2 * p);
    st = stats_merge(st, Stats{cnt, v[0], v[1]});
  }
  st = block_merge(st, sh);
  if (threadIdx.x == 0) {
    mean[ng] = st.mean;
    rstd[ng] = 1.0f / sqrtf(st.m2 / st.n + eps);
  }
}

// Statistics of 16 values as one batch (two passes over registers).
__device__ __forceinline__ Stats batch16(const f32x4 v[4]) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
  const float mu = s * (1.0f / 16.0f);
  float m2 = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float dv = v[i][e] - mu;
      m2 += dv * dv;
    }
  return Stats{16.f, mu, m2};
}

// Fold the statistics of all 64 lanes of a wave into lane 0 (a fixed xor
// tree: every run merges the same pairs in the same order).
__device__ __forceinline__ Stats wave_merge(Stats st) {
#pragma unroll
  for (int h = 32; h >= 1; h >>= 1) {
    const Stats o = {__shfl_xor(st.n, h), __shfl_xor(st.mean, h), __shfl_xor(st.m2, h)};
    st = stats_merge(st, o);
  }
  return st;
}

// GroupNorm statistics straight from an fp32 y, in two stages, so that any
// number of (n, g) groups fills the GPU.  The values of group (n, g) are one
// contiguous run of len = (C/G) * L elements ("Kimi-K2.6 l2_p35": statistics
// over the C/G channels x L positions of a group), cut into S slices of
// kStatSlice elements (the last one shorter).
// Stage 1 (gn_stats_slice_kernel): one workgroup per (n, g, slice) reduces
// its slice to (mean, M2) at part[((n*G + g)*S + s)*2] (the count follows from
// the geometry); with S == 1 it writes mean/rstd itself.
// Stage 2 (gn_stats_merge_kernel): one wave per (n, g) folds the S partials
// in a fixed order.  Every reduction order is fixed, so results are bit
// identical from run to run.
constexpr int64_t kStatSlice = 32768;  // elements per stage-1 workgroup (128 KB)

int64_t stat_slices(int64_t len, bool two_stage) {
  return two_stage ? (len + kStatSlice - 1) / kStatSlice : 1;
}

// VEC: y 16-byte aligned and len % 4 == 0 (every slice starts aligned)
template <bool VEC>
__global__ __launch_bounds__(NT) void gn_stats_slice_kernel(const float* __restrict__ y,
                                                            int64_t len, int64_t S,
                                                            float eps,
                                                            float* __restrict__ part,
                                                            float* mean, float* rstd) {
  __shared__ Stats wsh[NT / 64];
  const int64_t gs = blockIdx.x;           // (n*G + g)*S + s
  const int64_t ng = gs / S, sl = gs - ng * S;
  const int64_t off = sl * kStatSlice;
  const int64_t rem = len - off;
  const int64_t cnt = rem < kStatSlice ? rem : kStatSlice;
  const float* p = y + ng * len + off;
  const int tid = threadIdx.x;
  Stats st = {0.f, 0.f, 0.f};
  // full batches: 16 values per thread per iteration, all loads issued first
  constexpr int64_t BATCH = 16 * NT;
  const int64_t nfull = cnt / BATCH;
  for (int64_t it = 0; it < nfull; ++it) {
    f32x4 v[4];
    if (VEC) {
      const f32x4* pv = (const f32x4*)(p + it * BATCH);
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(pv + u * NT + tid);
    } else {
      const float* pb = p + it * BATCH;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[u][e] = pb[(4 * u + e) * NT + tid];
    }
    st = stats_merge(st, batch16(v));
  }
  // the tail of the slice, value by value
  for (int64_t e = nfull * BATCH + tid; e < cnt; e += NT) st = stats_merge(st, Stats{1.f, p[e], 0.f});
  st = wave_merge(st);
  const int lane = tid & 63, wave = tid >> 6;
  if (lane == 0) wsh[wave] = st;
  __syncthreads();
  if (tid == 0) {
    Stats r = wsh[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) r = stats_merge(r, wsh[w]);
    if (S == 1) {
      mean[ng] = r.mean;
      rstd[ng] = 1.0f / sqrtf(r.m2 / r.n + eps);
    } else {
      *(f32x2*)(part + 2 * gs) = f32x2{r.mean, r.m2};
    }
  }
}

__global__ __launch_bounds__(NT) void gn_stats_merge_kernel(const float* __restrict__ part,
                                                            int64_t NG, int64_t len, int64_t S,
                                                            float eps, float* mean,
                                                            float* rstd) {
  const int lane = threadIdx.x & 63;
  const int64_t ng = (int64_t)blockIdx.x * (NT / 64) + (threadIdx.x >> 6);
  if (ng >= NG) return;  // whole wave
  Stats st = {0.f, 0.f, 0.f};
  for (int64_t s = lane; s < S; s += 64) {
    const int64_t rem = len - s * kStatSlice;
    const float cnt = (float)(rem < kStatSlice ? rem : kStatSlice);
    const f32x2 v = *(const f32x2*)(part + 2 * (ng * S + s));
    st = stats_merge(st, Stats{cnt, v[0], v[1]});
  }
  st = wave_merge(st);
  if (lane == 0) {
    mean[ng] = st.mean;
    rstd[ng] = 1.0f / sqrtf(st.m2 / st.n + eps);
  }
}

// The 4 values of unit u of a raw 16-byte vector of TI (fp32: one unit;
// bf16: two units, element order preserved).
template <typename TI>
__device__ __forceinline__ f32x4 unit_values(u32x4 raw, int u) {
  if constexpr (sizeof(TI) == 4) {
    return __builtin_bit_cast(f32x4, raw);
  } else {
    const uint32_t lo = raw[2 * u], hi = raw[2 * u + 1];
    return f32x4{__uint_as_float(lo << 16), __uint_as_float(lo & 0xffff0000u),
                 __uint_as_float(hi << 16), __uint_as_float(hi & 0xffff0000u)};
  }
}

// Store VU units (4 * VU consecutive elements) of the output type TO.
template <int VU>
__device__ __forceinline__ void store_units(float* p, const f32x4 (&z)[VU]) {
#pragma unroll
  for (int u = 0; u < VU; ++u) __builtin_nontemporal_store(z[u], (f32x4*)(p + 4 * u));
}
template <int VU>
__device__ __forceinline__ void store_units(uint16_t* p, const f32x4 (&z)[VU]) {
  if constexpr (VU == 2) {
    const u32x2 a = f32x4_to_bf16(z[0]), b = f32x4_to_bf16(z[1]);
    __builtin_nontemporal_store(u32x4{a[0], a[1], b[0], b[1]}, (u32x4*)p);
  } else {
#pragma unroll
    for (int u = 0; u < VU; ++u)
      __builtin_nontemporal_store(f32x4_to_bf16(z[u]), (u32x2*)(p + 4 * u));
  }
}

// mode 1: statistics per (n, g); mode 2: per (n, l).  TI / TO: element types
// of y and out (float, or bf16 bits in uint16_t); arithmetic in fp32, out
// rounded to nearest even when bf16.
template <int MODE, bool VEC, typename TI, typename TO>
__global__ __launch_bounds__(NT) void apply_kernel(const TI* __restrict__ y,
                                                   const float* __restrict__ mean,
                                                   const float* __restrict__ rstd,
                                                   const float* __restrict__ gamma,
                                                   const float* __restrict__ beta, TO* out,
                                                   uint32_t total, FastDiv divL, FastDiv divC,
                                                   uint32_t C, uint32_t L, uint32_t G,
                                                   uint32_t cpg) {
  const uint32_t step = gridDim.x * NT;
  // one element, all index math from scratch
  auto scalar = [&](uint32_t e) __attribute__((always_inline)) {
    const uint32_t row = divL.div(e);
    const uint32_t l = e - row * L;
    const uint32_t n = divC.div(row);
    const uint32_t c = row - n * C;
    const float ga = gamma ? gamma[c] : 1.f, be = beta ? beta[c] : 0.f;
    float mu, rs;
    if (MODE == 1) {
      mu = mean[n * G + c / cpg];
      rs = rstd[n * G + c / cpg];
    } else {
      mu = mean[(size_t)n * L + l];
      rs = rstd[(size_t)n * L + l];
    }
    store_elem(out + e, (load_elem(y + e) - mu) * (rs * ga) + be);
  };
  if (VEC) {
    // 16-byte vectors of y: EPV elements, VU units of 4 (a unit never
    // crosses a row: L % 4 == 0)
    constexpr uint32_t EPV = 16 / sizeof(TI), VU = EPV / 4;
    const uint32_t nv = total / EPV;
    auto unit = [&](uint32_t e, const f32x4& yv) __attribute__((always_inline)) {
      const uint32_t row = divL.div(e);
      const uint32_t l = e - row * L;
      const uint32_t n = divC.div(row);
      const uint32_t c = row - n * C;
      const float ga = gamma ? gamma[c] : 1.f, be = beta ? beta[c] : 0.f;
      f32x4 z;
      if (MODE == 1) {
        const uint32_t sidx = n * G + c / cpg;
        const float mu = mean[sidx], sc = rstd[sidx] * ga;
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = (yv[i] - mu) * sc + be;
      } else {
        const f32x4 mu = *(const f32x4*)(mean + (size_t)n * L + l);
        const f32x4 rs = *(const f32x4*)(rstd + (size_t)n * L + l);
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = (yv[i] - mu[i]) * (rs[i] * ga) + be;
      }
      return z;
    };
    auto one = [&](uint32_t v, const u32x4& raw) __attribute__((always_inline)) {
      const uint32_t e = v * EPV;
      f32x4 z[VU];
#pragma unroll
      for (uint32_t u = 0; u < VU; ++u) z[u] = unit(e + 4 * u, unit_values<TI>(raw, u));
      store_units<VU>(out + e, z);
    };
    auto load = [&](uint32_t v) __attribute__((always_inline)) {
      return __builtin_nontemporal_load((const u32x4*)(y + (size_t)v * EPV));
    };
    // elements past the last whole vector (bf16 y with total % 8 == 4); a
    // 64-bit counter, so the stride cannot wrap past 2^32 near the size limit
    for (uint64_t e = (uint64_t)nv * EPV + blockIdx.x * NT + threadIdx.x; e < total; e += step)
      scalar((uint32_t)e);
    if (MODE == 2) {
      // three loads per unit (y, mean, rstd): a grid-strided loop with four
      // vectors in flight per thread measured faster here
      constexpr int U2 = 4;
      uint32_t v = blockIdx.x * NT + threadIdx.x;
      for (; v + (U2 - 1) * step < nv; v += U2 * step) {
        u32x4 yv[U2];
#pragma unroll
        for (int u = 0; u < U2; ++u) yv[u] = load(v + u * step);
#pragma unroll
        for (int u = 0; u < U2; ++u) one(v + u * step, yv[u]);
      }
      for (; v < nv; v += step) one(v, load(v));
      return;
    }
    // Block-contiguous batches: per iteration a workgroup owns UNR * NT
    // consecutive 16-byte vectors (UNR loads in flight per thread, all before
    // any store); measured on this GPU, contiguous per-workgroup spans stream
    // ~10% faster than a grid-strided interleave.
    constexpr int UNR = 2;
    const uint32_t batch = UNR * NT;
    for (uint32_t base = blockIdx.x * batch; base < nv; base += gridDim.x * batch) {
      u32x4 yv[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const uint32_t v = base + u * NT + threadIdx.x;
        if (v < nv) yv[u] = load(v);
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const uint32_t v = base + u * NT + threadIdx.x;
        if (v < nv) one(v, yv[u]);
      }
    }
  } else {
    for (uint64_t e = (uint64_t)blockIdx.x * NT + threadIdx.x; e < total; e += step)
      scalar((uint32_t)e);
  }
}

__global__ __launch_bounds__(NT) void ln_merge_kernel(const float* __restrict__ part, int64_t N,
                                                      int64_t C, int64_t L, int32_t n_ctiles,
                                                      int32_t tn, float eps, float* mean,
                                                      float* rstd) {
  const int64_t idx = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (idx >= N * L) return;
  const int64_t n = idx / L, l = idx - n * L;
  Stats st = {0.f, 0.f, 0.f};
  for (int ct = 0; ct < n_ctiles; ++ct) {
    const int64_t rem = C - (int64_t)ct * tn;
    const float cnt = (float)(rem < tn ? rem : tn);
    const f32x2 v = *(const f32x2*)(part + ((n * n_ctiles + ct) * L + l) * 2);
    st = stats_merge(st, Stats{cnt, v[0], v[1]});
  }
  mean[idx] = st.mean;
  rstd[idx] = 1.0f / sqrtf(st.m2 / st.n + eps);
}

template <int KIND>
__device__ __forceinline__ float normed(float v, const float* mean, const float* rstd,
                                        const float* gamma, const float* beta, int64_t n,
                                        int64_t c, int64_t l, int64_t L, int64_t G,
                                        int64_t cpg) {
  if (KIND == 0) return v;
  const float ga = gamma ? gamma[c] : 1.f, be = beta ? beta[c] : 0.f;
  const int64_t si = (KIND == 1) ? n * G + c / cpg : n * L + l;
  return (v - mean[si]) * (rstd[si] * ga) + be;
}

// one thread per (n, l): two passes over the channels
template <int KIND, typename TI, typename TO>
__global__ __launch_bounds__(NT) void rowmin_kernel(const TI* __restrict__ y,
                                                    const float* mean, const float* rstd,
                                                    const float* gamma, const float* beta,
                                                    const float* __restrict__ bias2, TO* out,
                                                    int64_t N, int64_t C, int64_t L, int64_t G) {
  const int64_t idx = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (idx >= N * L) return;
  const int64_t n = idx / L, l = idx - n * L;
  const int64_t cpg = G > 0 ? C / G : 1;
  float m = __builtin_inff();
  for (int64_t c = 0; c < C; ++c) {
    const float z = normed<KIND>(load_elem(y + (n * C + c) * L + l), mean, rstd, gamma, beta, n,
                                 c, l, L, G, cpg);
    m = min_nan(m, z);
  }
  for (int64_t c = 0; c < C; ++c) store_elem(out + (n * C + c) * L + l, m + bias2[c]);
}

// L == 1: one workgroup per row n, threads over channels
template <int KIND, typename TI, typename TO>
__global__ __launch_bounds__(NT) void rowmin_l1_kernel(const TI* __restrict__ y,
                                                       const float* mean, const float* rstd,
                                                       const float* gamma, const float* beta,
                                                       const float* __restrict__ bias2,
                                                       TO* out, int64_t C, int64_t G) {
  __shared__ float sh[NT];
  const int64_t n = blockIdx.x;
  const int64_t cpg = G > 0 ? C / G : 1;
  float m = __builtin_inff();
  for (int64_t c = threadIdx.x; c < C; c += NT) {
    const float z = normed<KIND>(load_elem(y + n * C + c), mean, rstd, gamma, beta, n, c, 0, 1,
                                 G, cpg);
    m = min_nan(m, z);
  }
  sh[threadIdx.x] = m;
  __syncthreads();
  for (int s = NT / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) sh[threadIdx.x] = min_nan(sh[threadIdx.x], sh[threadIdx.x + s]);
    __syncthreads();
  }
  m = sh[0];
  for (int64_t c = threadIdx.x; c < C; c += NT) store_elem(out + n * C + c, m + bias2[c]);
}

unsigned grid_for(uint64_t work) {
  uint64_t b = (work + NT - 1) / NT;
  const uint64_t cap = 256ull * 64;  // enough resident waves to saturate HBM
  return (unsigned)(b < 1 ? 1 : (b > cap ? cap : b));
}

template <int MODE, typename TI, typename TO>
hipError_t apply_launch_t(const TI* y, const float* mean, const float* rstd, const float* gamma,
                          const float* beta, TO* out, int64_t N, int64_t C, int64_t L,
                          int32_t G, hipStream_t s) {
  const uint64_t total = (uint64_t)N * C * L;
  if (total >= (1ull << 32)) return hipErrorInvalidValue;
  const FastDiv dl = FastDiv::make((uint32_t)L), dc = FastDiv::make((uint32_t)C);
  const uint32_t cpg = (MODE == 1) ? (uint32_t)(C / G) : 1u;
  // out is written VU units of 4 at a time per 16-byte vector of y
  constexpr uintptr_t out_align = (16 / sizeof(TI) / 4) * 4 * sizeof(TO);
  const bool vec = (L % 4 == 0) && ((((uintptr_t)y) & 15) == 0) &&
                   ((((uintptr_t)out) & (out_align - 1)) == 0) &&
                   (MODE == 1 || ((((uintptr_t)mean) & 15) == 0 && (((uintptr_t)rstd) & 15) == 0));
  if (vec) {
    const uint64_t nvec = total / (16 / sizeof(TI));
    const uint64_t batches = (nvec + 2 * NT - 1) / (2 * NT);
    const unsigned grid = MODE == 2 ? grid_for(nvec)
                                    : (unsigned)(batches < 8192 ? (batches < 1 ? 1 : batches) : 8192);
    hipLaunchKernelGGL((apply_kernel<MODE, true, TI, TO>), dim3(grid), dim3(NT), 0, s, y, mean,
                       rstd, gamma, beta, out, (uint32_t)total, dl, dc, (uint32_t)C,
                       (uint32_t)L, (uint32_t)G, cpg);
  } else {
    hipLaunchKernelGGL((apply_kernel<MODE, false, TI, TO>), dim3(grid_for(total)), dim3(NT), 0,
                       s, y, mean, rstd, gamma, beta, out, (uint32_t)total, dl, dc, (uint32_t)C,
                       (uint32_t)L, (uint32_t)G, cpg);
  }
  return hipGetLastError();
}

// element types: 0 fp32, 1 bf16 (enum c1g_dtype)
template <int MODE>
hipError_t apply_launch(const void* y, int y_dt, const float* mean, const float* rstd,
                        const float* gamma, const float* beta, void* out, int out_dt, int64_t N,
                        int64_t C, int64_t L, int32_t G, hipStream_t s) {
  if (y_dt == 0 && out_dt == 0)
    return apply_launch_t<MODE>((const float*)y, mean, rstd, gamma, beta, (float*)out, N, C, L,
                                G, s);
  if (y_dt == 1 && out_dt == 1)
    return apply_launch_t<MODE>((const uint16_t*)y, mean, rstd, gamma, beta, (uint16_t*)out, N,
                                C, L, G, s);
  if (y_dt == 0 && out_dt == 1)
    return apply_launch_t<MODE>((const float*)y, mean, rstd, gamma, beta, (uint16_t*)out, N, C,
                                L, G, s);
  return hipErrorInvalidValue;
}

template <typename TI, typename TO>
void rowmin_launch_t(const TI* y, const float* mean, const float* rstd, const float* gamma,
                     const float* beta, const float* bias2, TO* out, int64_t N, int64_t C,
                     int64_t L, int32_t G, int norm_kind, hipStream_t s) {
  if (L == 1) {
    dim3 grid((unsigned)N);
    if (norm_kind == 1)
      hipLaunchKernelGGL((rowmin_l1_kernel<1, TI, TO>), grid, dim3(NT), 0, s, y, mean, rstd,
                         gamma, beta, bias2, out, C, (int64_t)G);
    else if (norm_kind == 2)
      hipLaunchKernelGGL((rowmin_l1_kernel<2, TI, TO>), grid, dim3(NT), 0, s, y, mean, rstd,
                         gamma, beta, bias2, out, C, (int64_t)G);
    else
      hipLaunchKernelGGL((rowmin_l1_kernel<0, TI, TO>), grid, dim3(NT), 0, s, y, mean, rstd,
                         gamma, beta, bias2, out, C, (int64_t)G);
  } else {
    dim3 grid((unsigned)((N * L + NT - 1) / NT));
    if (norm_kind == 1)
      hipLaunchKernelGGL((rowmin_kernel<1, TI, TO>), grid, dim3(NT), 0, s, y, mean, rstd, gamma,
                         beta, bias2, out, N, C, L, (int64_t)G);
    else if (norm_kind == 2)
      hipLaunchKernelGGL((rowmin_kernel<2, TI, TO>), grid, dim3(NT), 0, s, y, mean, rstd, gamma,
                         beta, bias2, out, N, C, L, (int64_t)G);
    else
      hipLaunchKernelGGL((rowmin_kernel<0, TI, TO>), grid, dim3(NT), 0, s, y, mean, rstd, gamma,
                         beta, bias2, out, N, C, L, (int64_t)G);
  }
}

}  // namespace

hipError_t gn_merge_launch(const float* part, int64_t N, int64_t C, int64_t L, int32_t G,
                           int32_t n_ttiles, int32_t tm, float eps, float* mean, float* rstd,
                           hipStream_t s) {
  hipLaunchKernelGGL(gn_merge_kernel, dim3((unsigned)(N * G)), dim3(NT), 0, s, part, C, L, G,
                     n_ttiles, tm, eps, mean, rstd);
  return hipGetLastError();
}

size_t gn_stats_workspace_bytes(int64_t N, int64_t C, int64_t L, int32_t G) {
  const int64_t S = stat_slices(C / G * L, true);
  return S > 1 ? (size_t)(N * G * S) * 2 * sizeof(float) : 0;
}

hipError_t gn_stats_launch(const float* y, int64_t N, int64_t C, int64_t L, int32_t G,
                           float eps, float* mean, float* rstd, float* part, hipStream_t s) {
  const int64_t len = C / G * L, NG = N * G;
  // without a workspace: one workgroup per group
  const int64_t S = stat_slices(len, part != nullptr);
  const bool vec = (len % 4 == 0) && ((((uintptr_t)y) & 15) == 0);
  const dim3 grid((unsigned)(NG * S));
  if (vec)
    hipLaunchKernelGGL(gn_stats_slice_kernel<true>, grid, dim3(NT), 0, s, y, len, S, eps,
                       part, mean, rstd);
  else
    hipLaunchKernelGGL(gn_stats_slice_kernel<false>, grid, dim3(NT), 0, s, y, len, S, eps,
                       part, mean, rstd);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  hipLaunchKernelGGL(gn_stats_merge_kernel, dim3((unsigned)((NG + NT / 64 - 1) / (NT / 64))),
                     dim3(NT), 0, s, part, NG, len, S, eps, mean, rstd);
  return hipGetLastError();
}

hipError_t gn_apply_launch(const void* y, int y_dt, const float* mean, const float* rstd,
                           const float* gamma, const float* beta, void* out, int out_dt,
                           int64_t N, int64_t C, int64_t L, int32_t G, hipStream_t s) {
  return apply_launch<1>(y, y_dt, mean, rstd, gamma, beta, out, out_dt, N, C, L, G, s);
}

hipError_t ln_merge_launch(const float* part, int64_t N, int64_t C, int64_t L,
                           int32_t n_ctiles, int32_t tn, float eps, float* mean, float* rstd,
                           hipStream_t s) {
  const int64_t work = N * L;
  hipLaunchKernelGGL(ln_merge_kernel, dim3((unsigned)((work + NT - 1) / NT)), dim3(NT), 0, s,
                     part, N, C, L, n_ctiles, tn, eps, mean, rstd);
  return hipGetLastError();
}

hipError_t ln_apply_launch(const void* y, int y_dt, const float* mean, const float* rstd,
                           const float* gamma, const float* beta, void* out, int out_dt,
                           int64_t N, int64_t C, int64_t L, hipStream_t s) {
  return apply_launch<2>(y, y_dt, mean, rstd, gamma, beta, out, out_dt, N, C, L, 1, s);
}

hipError_t rowmin_bias_launch(const void* y, int y_dt, const float* mean, const float* rstd,
                              const float* gamma, const float* beta, const float* bias2,
                              void* out, int out_dt, int64_t N, int64_t C, int64_t L,
                              int32_t G, int norm_kind, hipStream_t s) {
  if (y_dt == 0 && out_dt == 0)
    rowmin_launch_t((const float*)y, mean, rstd, gamma, beta, bias2, (float*)out, N, C, L, G,
                    norm_kind, s);
  else if (y_dt == 1 && out_dt == 1)
    rowmin_launch_t((const uint16_t*)y, mean, rstd, gamma, beta, bias2, (uint16_t*)out, N, C,
                    L, G, norm_kind, s);
  else if (y_dt == 0 && out_dt == 1)
    rowmin_launch_t((const float*)y, mean, rstd, gamma, beta, bias2, (uint16_t*)out, N, C, L,
                    G, norm_kind, s);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace c1g
