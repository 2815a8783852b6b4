// fp32 implicit-GEMM 1-D convolution for gfx950 (split path).
//
// GEMM view ("Kimi-K2.6 l1_p5", the implicit-GEMM shape M = N*T_out,
// N = C_out, K = C_in*K): row m = (n, t), column = output channel c,
// reduction over (tap j, input channel ci).  The im2col matrix is never built:
// each workgroup stages the input halo window x[n, ci0:ci0+CK, tbase : tbase+XW]
// (zero outside [0,T)) in LDS once per K-chunk, and every tap reads it at a
// shifted offset, so one staged x value feeds K MFMA operands.  Weights are
// repacked once per call into the exact LDS image of each (c-tile, K-chunk),
// so their staging is a straight 16-byte copy.
//
// Workgroup: 256 threads = 4 waves in a 2x2 grid; tile 128 (t) x 128 (c);
// each wave owns 64 x 64 = 4x4 MFMA 16x16 tiles (v_mfma_f32_16x16x4_f32), so
// per K-step it reads 4 A and 4 B scalars from LDS and issues 16 MFMAs.
// The next chunk is fetched into registers while the current one is consumed.
//
// Epilogues: store y (+bias); or also reduce the tile into per-(n, c, t-tile)
// (mean, M2) partials for GroupNorm; or into per-(n, c-tile, t) partials for
// LayerNorm over channels.  Partials are written to fixed slots (no atomics),
// so the later merge is deterministic.
#include "common.hpp"
#include "conv_epilogue.hpp"
#include "launch.hpp"

namespace c1g {
namespace {

constexpr int TM = ConvF32Cfg::TM;   // 128 output positions per tile
constexpr int TN = ConvF32Cfg::TN;   // 128 output channels per tile
constexpr int CK = ConvF32Cfg::CK;   // 8 input channels per K-chunk
constexpr int KMAX = 8;              // taps supported (LDS budget)
constexpr int TNS = TN + 16;         // padded LDS row of the weight image
constexpr int NTHR = 256;
constexpr int WM = 4, WN = 4;        // MFMA tiles per wave (t, c)

__host__ __device__ constexpr int xs_stride(int xcap) { return xcap + 16; }

template <int XCAP>
__global__ __launch_bounds__(NTHR) void conv_f32_kernel(ConvArgs a, int epi) {
  extern __shared__ float lds[];
  constexpr int XS = xs_stride(XCAP);
  float* Xs = lds;                      // [CK][XS]
  float* Ws = lds + CK * XS;            // [K*CK][TNS]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int lr = lane & 15, kq = lane >> 4;

  // 1-D grid, XCD-aware: workgroup ids round-robin over the 8 XCDs; XCD x
  // takes a contiguous range of tiles ordered (n, t-tile, c-tile) with the
  // c-tile fastest, so the channel tiles of one input window share an L2
  // (and x comes from HBM once)
  const int total = (int)gridDim.x;
  int lin = blockIdx.x;
  if ((total & 7) == 0) lin = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int ctile = lin % a.n_ctiles;
  const int ttile = (lin / a.n_ctiles) % a.n_ttiles;
  const int64_t n = lin / (a.n_ctiles * a.n_ttiles);
  const int64_t t0 = (int64_t)ttile * TM;
  const int c0 = ctile * TN;
  const int K = a.K, s = a.stride, d = a.dilation;

  const float* __restrict__ x = (const float*)a.x;
  const float* __restrict__ wp = (const float*)a.wp;

  // input window of this tile, aligned down to 4 elements for 16-byte loads
  const int64_t tbase = t0 * s - a.pad_left;
  const int64_t tal = (tbase >= 0) ? (tbase & ~(int64_t)3) : -(((-tbase) + 3) & ~(int64_t)3);
  const int shift = (int)(tbase - tal);

  constexpr int XQ = XCAP / 4;                            // float4 per window row
  constexpr int XV = (CK * XQ + NTHR - 1) / NTHR;         // float4 slots per thread
  const int wrows = K * CK;                               // weight-image rows
  const int WV = wrows * (TN / 4) / NTHR;                 // = K float4 per thread

  f32x4 xr[XV];
  f32x4 wr[KMAX];

  auto fetch = [&](int chunk) {
    const int64_t ci0 = (int64_t)chunk * CK;
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      const int q = tid + NTHR * i;
      const int row = q / XQ, c4 = q - row * XQ;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      const int64_t ci = ci0 + row;
      if (row < CK && ci < a.C_in) {
        const int64_t t = tal + 4 * c4;
        const float* src = x + (n * a.C_in + ci) * a.T;
        if (t >= 0 && t + 3 < a.T && ((((uintptr_t)(src + t)) & 15) == 0)) {
          v = *(const f32x4*)(src + t);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (t + e >= 0 && t + e < a.T) v[e] = src[t + e];
        }
      }
      xr[i] = v;
    }
    const float* wsrc = wp + ((int64_t)ctile * a.n_chunks + chunk) * (int64_t)wrows * TN;
#pragma unroll
    for (int i = 0; i < KMAX; ++i)
      if (i < WV) wr[i] = *(const f32x4*)(wsrc + 4 * (tid + NTHR * i));
  };

  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      const int q = tid + NTHR * i;
      const int row = q / XQ, c4 = q - row * XQ;
      if (row < CK) *(f32x4*)(Xs + row * XS + 4 * c4) = xr[i];
    }
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      if (i < WV) {
        const int q = tid + NTHR * i;
        const int row = q >> 5, c4 = q & 31;
        *(f32x4*)(Ws + row * TNS + 4 * c4) = wr[i];
      }
    }
  };

  f32x4 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // per-lane LDS bases of the A (window) and B (weight image) operands
  const int abase = kq * XS + shift + (wm * WM * 16 + lr) * s;
  const int bbase = kq * TNS + wn * WN * 16 + lr;

  fetch(0);
  stash();
  __syncthreads();
  for (int chunk = 0; chunk < a.n_chunks; ++chunk) {
    if (chunk + 1 < a.n_chunks) fetch(chunk + 1);
    for (int j = 0; j < K; ++j) {
#pragma unroll
      for (int h = 0; h < CK / 4; ++h) {
        float av[WM], bv[WN];
#pragma unroll
        for (int i = 0; i < WM; ++i) av[i] = Xs[abase + 4 * h * XS + j * d + i * 16 * s];
#pragma unroll
        for (int jn = 0; jn < WN; ++jn) bv[jn] = Ws[bbase + (j * CK + 4 * h) * TNS + jn * 16];
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int jn = 0; jn < WN; ++jn) acc[i][jn] = mfma16x16x4(av[i], bv[jn], acc[i][jn]);
      }
    }
    __syncthreads();
    if (chunk + 1 < a.n_chunks) {
      stash();
      __syncthreads();
    }
  }

  conv_epilogue<WM, WN, 2, 2>(a, epi, acc, n, t0, c0, ttile, ctile, wm, wn, (Stats*)lds);
}

// Weight image: wp[((ctile*n_chunks + chunk)*K*CK + j*CK + cl)*TN + c]
//             = w[ctile*TN + c][chunk*CK + cl][j]   (0 outside the tensor)
__global__ void conv_f32_pack_kernel(const float* __restrict__ w, float* __restrict__ wp,
                                     int64_t C_in, int64_t C_out, int K, int n_chunks,
                                     int64_t total) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int c = (int)(idx % TN);
  int64_t rest = idx / TN;
  const int cl = (int)(rest % CK);
  rest /= CK;
  const int j = (int)(rest % K);
  rest /= K;
  const int chunk = (int)(rest % n_chunks);
  const int64_t ctile = rest / n_chunks;
  const int64_t co = ctile * TN + c;
  const int64_t ci = (int64_t)chunk * CK + cl;
  wp[idx] = (co < C_out && ci < C_in) ? w[(co * C_in + ci) * K + j] : 0.f;
}

template <int XCAP>
hipError_t launch_xcap(const ConvArgs& a, int epi, hipStream_t s) {
  const size_t lds = (size_t)(CK * xs_stride(XCAP) + a.K * CK * TNS) * sizeof(float);
  dim3 grid((unsigned)(a.N * a.n_ttiles * a.n_ctiles));
  hipLaunchKernelGGL(conv_f32_kernel<XCAP>, grid, dim3(NTHR), lds, s, a, epi);
  return hipGetLastError();
}

}  // namespace

int conv_f32_window_cap(int stride) {
  (void)stride;
  return 544 - 3;  // widest window (incl. 16-byte alignment shift) of any instantiation
}

size_t conv_f32_packed_bytes(int64_t C_in, int64_t C_out, int K) {
  const int64_t n_chunks = (C_in + CK - 1) / CK, n_ctiles = (C_out + TN - 1) / TN;
  return (size_t)(n_ctiles * n_chunks * K * CK * TN) * sizeof(float);
}

hipError_t conv_f32_pack(const float* w, float* wp, int64_t C_in, int64_t C_out, int K,
                         hipStream_t s) {
  const int n_chunks = (int)((C_in + CK - 1) / CK);
  const int64_t total = (int64_t)conv_f32_packed_bytes(C_in, C_out, K) / sizeof(float);
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(conv_f32_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, wp,
                     C_in, C_out, K, n_chunks, total);
  return hipGetLastError();
}

hipError_t conv_f32_launch(const ConvArgs& a, int epi, hipStream_t s) {
  if (a.K > KMAX) return hipErrorInvalidValue;
  const int64_t xw = (int64_t)(TM - 1) * a.stride + (int64_t)(a.K - 1) * a.dilation + 1 + 3;
  if (xw <= 160) return launch_xcap<160>(a, epi, s);
  if (xw <= 288) return launch_xcap<288>(a, epi, s);
  if (xw <= 544) return launch_xcap<544>(a, epi, s);
  return hipErrorInvalidValue;
}

}  // namespace c1g
