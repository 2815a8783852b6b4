// Fused conv1d + GroupNorm in one pass, fp32, for slabs that fit on chip.
//
// One workgroup owns one sample n and a block of 16 output channels made of
// whole groups (C_out/G divides 16), over every output position: the complete
// GroupNorm slab of its groups ("Kimi-K2.6 l2_p35": statistics over C_out/G
// channels x T_out per (n, group); its single-pass design keeps a group's
// whole output on chip so the normalised result is written once).  Here the
// slab stays in MFMA accumulator registers: 8 waves, each owning MQ 16-row
// subtiles of positions x 16 channels (v_mfma_f32_16x16x4_f32), so y never
// goes to HBM and is never re-read.
//
// Per K-chunk (8 input channels, all taps) the input halo window of the whole
// sequence is staged in LDS once and read by every tap at a shifted offset;
// the next chunk is fetched into registers while the current one is consumed.
// After the K loop the group statistics are taken in two passes over the
// registers (sum -> mean, then sum of squared deviations -> variance), reduced
// across lanes with xor shuffles and across waves in a fixed order through LDS
// (deterministic), then each value is normalised, scaled and written once.
//
// blockIdx -> (n, channel block) is remapped so that the workgroups of one
// sample land on the same XCD and share its L2 copy of x[n].
#include "common.hpp"
#include "launch.hpp"

namespace c1g {
namespace {

constexpr int NW = 8;              // waves per workgroup
constexpr int NTHR = NW * 64;
constexpr int CB = 16;             // channels per workgroup
constexpr int CK = 8;              // input channels per K-chunk
constexpr int KMAX = 8;
constexpr int HALO_MAX = 28;       // (K-1)*dilation supported

template <int MQ>
struct FusedGeom {
  static constexpr int TCOV = NW * MQ * 16;          // positions covered
  static constexpr int XL = TCOV + 32;               // staged window width
  static constexpr int XS = XL + 16;                 // LDS row stride (== 16 mod 32)
  static constexpr int XQ = XL / 4;
  static constexpr int XV = (CK * XQ + NTHR - 1) / NTHR;
  static constexpr int WV = (KMAX * CK * CB + NTHR - 1) / NTHR;
};

template <int MQ>
__global__ __launch_bounds__(NTHR) void fused_conv_gn_kernel(FusedArgs a) {
  using Gm = FusedGeom<MQ>;
  __shared__ float Xs[CK * Gm::XS];
  __shared__ float Ws[KMAX * CK * CB];
  __shared__ float red[NW * CB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, kq = lane >> 4;

  // XCD-aware mapping: consecutive workgroup ids round-robin over the 8 XCDs;
  // give each XCD a contiguous range of (n, block) so one sample's blocks share an L2.
  const int nblk = (int)((a.C_out + CB - 1) / CB);
  const int total = (int)(a.N * nblk);
  int lin = blockIdx.x;
  if ((total & 7) == 0) lin = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int64_t n = lin / nblk;
  const int cb = lin - (int)n * nblk;
  const int cbase = cb * CB;

  const int K = a.K, d = a.dilation;
  const int64_t T = a.T, T_out = a.T_out;
  const int64_t tbase = -(int64_t)a.pad_left;
  const int64_t tal = (tbase >= 0) ? (tbase & ~(int64_t)3) : -(((-tbase) + 3) & ~(int64_t)3);
  const int shift = (int)(tbase - tal);
  const int n_chunks = (int)((a.C_in + CK - 1) / CK);

  const float* __restrict__ x = a.x;
  const float* __restrict__ w = a.w;

  f32x4 xr[Gm::XV];
  float wr[Gm::WV];

  auto fetch = [&](int chunk) {
    const int64_t ci0 = (int64_t)chunk * CK;
#pragma unroll
    for (int i = 0; i < Gm::XV; ++i) {
      const int q = tid + NTHR * i;
      const int row = q / Gm::XQ, c4 = q - row * Gm::XQ;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      const int64_t ci = ci0 + row;
      if (row < CK && ci < a.C_in) {
        const int64_t t = tal + 4 * c4;
        const float* src = x + (n * a.C_in + ci) * T;
        if (t >= 0 && t + 3 < T && ((((uintptr_t)(src + t)) & 15) == 0)) {
          v = *(const f32x4*)(src + t);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (t + e >= 0 && t + e < T) v[e] = src[t + e];
        }
      }
      xr[i] = v;
    }
    // weight chunk image [j][cl][c], c fastest
#pragma unroll
    for (int i = 0; i < Gm::WV; ++i) {
      const int e = tid + NTHR * i;
      const int c = e & (CB - 1);
      const int rest = e >> 4;
      const int cl = rest % CK, j = rest / CK;
      float v = 0.f;
      const int64_t co = cbase + c, ci = ci0 + cl;
      if (j < K && co < a.C_out && ci < a.C_in) v = w[(co * a.C_in + ci) * K + j];
      wr[i] = v;
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < Gm::XV; ++i) {
      const int q = tid + NTHR * i;
      const int row = q / Gm::XQ, c4 = q - row * Gm::XQ;
      if (row < CK) *(f32x4*)(Xs + row * Gm::XS + 4 * c4) = xr[i];
    }
#pragma unroll
    for (int i = 0; i < Gm::WV; ++i) {
      const int e = tid + NTHR * i;
      if (e < KMAX * CK * CB) Ws[e] = wr[i];
    }
  };

  f32x4 acc[MQ];
#pragma unroll
  for (int m = 0; m < MQ; ++m) acc[m] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int abase = kq * Gm::XS + shift + wave * MQ * 16 + lr;  // stride 1
  const int bbase = kq * CB + lr;

  fetch(0);
  stash();
  __syncthreads();
  for (int chunk = 0; chunk < n_chunks; ++chunk) {
    if (chunk + 1 < n_chunks) fetch(chunk + 1);
    for (int j = 0; j < K; ++j) {
#pragma unroll
      for (int h = 0; h < CK / 4; ++h) {
        const float bv = Ws[bbase + (j * CK + 4 * h) * CB];
        const int ao = abase + 4 * h * Gm::XS + j * d;
#pragma unroll
        for (int m = 0; m < MQ; ++m) acc[m] = mfma16x16x4(Xs[ao + m * 16], bv, acc[m]);
      }
    }
    __syncthreads();
    if (chunk + 1 < n_chunks) {
      stash();
      __syncthreads();
    }
  }

  // ---------------------------------------------------------------- epilogue
  const int c = cbase + lr;
  const bool cvalid = c < a.C_out;
  const float bias = (a.bias != nullptr && cvalid) ? a.bias[c] : 0.f;
  const int cpg = (int)(a.C_out / a.G);
  const int gl = lr / cpg;                 // group within the block
  const int ngl = CB / cpg;
  const int t_lane = wave * MQ * 16 + 4 * kq;

  float sum = 0.f;
#pragma unroll
  for (int m = 0; m < MQ; ++m) {
    acc[m] += bias;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (t_lane + m * 16 + r < T_out) sum += acc[m][r];
  }
  // lanes of one group differ in the low log2(cpg) bits of lr and in kq
  auto group_reduce = [&](float v) {
#pragma unroll
    for (int msk = 1; msk < 16; msk <<= 1)
      if (msk < cpg) v += shfl_xor(v, msk);
    v += shfl_xor(v, 16);
    v += shfl_xor(v, 32);
    return v;
  };
  auto block_total = [&](float v) {
    v = group_reduce(v);
    if (kq == 0 && (lr % cpg) == 0) red[wave * CB + gl] = v;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) tot += red[wv * CB + gl];
    __syncthreads();
    return tot;
  };
  const float cnt = (float)cpg * (float)T_out;
  const float mean = block_total(sum) / cnt;
  float ss = 0.f;
#pragma unroll
  for (int m = 0; m < MQ; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (t_lane + m * 16 + r < T_out) {
        const float dv = acc[m][r] - mean;
        ss += dv * dv;
      }
  const float var = block_total(ss) / cnt;
  const float rstd = 1.0f / sqrtf(var + a.eps);

  if (cvalid) {
    const float ga = a.gamma ? a.gamma[c] : 1.f;
    const float be = a.beta ? a.beta[c] : 0.f;
    const float sc = rstd * ga;
    float* dst = a.out + (n * a.C_out + c) * T_out;
    const bool vec_ok = ((T_out & 3) == 0) && ((((uintptr_t)a.out) & 15) == 0);
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      const int64_t t = t_lane + m * 16;
      f32x4 z;
#pragma unroll
      for (int r = 0; r < 4; ++r) z[r] = (acc[m][r] - mean) * sc + be;
      if (vec_ok && t + 3 < T_out) {
        *(f32x4*)(dst + t) = z;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t + r < T_out) dst[t + r] = z[r];
      }
    }
    if (wave == 0 && kq == 0 && (lr % cpg) == 0) {
      const int64_t g = c / cpg;
      if (a.mean_out) a.mean_out[n * a.G + g] = mean;
      if (a.rstd_out) a.rstd_out[n * a.G + g] = rstd;
    }
  }
  (void)ngl;
}

template <int MQ>
hipError_t launch_mq(const FusedArgs& a, hipStream_t s) {
  const int nblk = (int)((a.C_out + CB - 1) / CB);
  dim3 grid((unsigned)(a.N * nblk));
  hipLaunchKernelGGL(fused_conv_gn_kernel<MQ>, grid, dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int fused_gn_max_tout(int stride, int K, int dilation) {
  if (stride != 1 || K < 1 || K > KMAX || (int64_t)(K - 1) * dilation > HALO_MAX) return 0;
  return NW * 8 * 16;
}

bool fused_gn_supported(int64_t C_out, int32_t G, int64_t T_out, int stride, int K,
                        int dilation) {
  if (G < 1 || C_out % G) return false;
  const int64_t cpg = C_out / G;
  if (cpg > CB || (CB % cpg) != 0) return false;
  return T_out >= 1 && T_out <= fused_gn_max_tout(stride, K, dilation);
}

hipError_t fused_gn_launch(const FusedArgs& a, hipStream_t s) {
  const int64_t t = a.T_out;
  if (t <= NW * 16 * 1) return launch_mq<1>(a, s);
  if (t <= NW * 16 * 2) return launch_mq<2>(a, s);
  if (t <= NW * 16 * 4) return launch_mq<4>(a, s);
  if (t <= NW * 16 * 8) return launch_mq<8>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace c1g
