// bf16 implicit-GEMM 1-D convolution for gfx950 (split path), fp32 accumulate.
//
// GEMM view ("Kimi-K2.6 l1_p5", the implicit-GEMM shape M = N*T_out,
// N = C_out, K = C_in*K): row m = (n, t), column = output channel c; the
// reduction runs over (tap j, input channel ci) in chunks of 32 input channels,
// one v_mfma_f32_16x16x32_bf16 K-step per tap.  The MFMA wants 8 consecutive
// reduction values per lane, i.e. 8 consecutive input channels at one position,
// while x is stored position-contiguous, so the input halo window of a tile is
// transposed while it is staged: each thread loads an 8 (channels) x 8
// (positions) block with 16-byte loads along t, transposes it in registers and
// writes 8 rows of the LDS window Xt[t][ci] (80-byte rows: the 16-byte MFMA
// operand reads of 8 consecutive rows hit 8 distinct bank groups).  Every tap
// then reads the same window at a shifted row offset.  The weights are repacked
// once per call into the exact LDS image of each (c-tile, chunk) and streamed
// with direct global->LDS loads.
//
// Workgroup: WGM x 2 waves; tile TM = WGM*WM*16 (t) x 128 (c); wave tile
// WM x 4 MFMA tiles (256 x 128 with 8 waves of 64 x 64 for unit stride and
// short halos, 64 x 128 with 4 waves otherwise).  Two LDS stages: the next chunk's weights
// stream in and its window is fetched into registers while the current chunk
// is consumed.  Epilogue: shared with the fp32 kernel (store y, GroupNorm or
// channel-LayerNorm partial statistics).
#include "common.hpp"
#include "conv_epilogue.hpp"
#include "launch.hpp"

namespace c1g {
namespace {

constexpr int TN = ConvBf16Cfg::TN;  // 128 output channels per tile
constexpr int CK = ConvBf16Cfg::CK;  // 32 input channels per chunk
constexpr int RS = CK + 8;           // LDS row stride in bf16 (80 bytes)
constexpr int KMAX = 5;              // taps (LDS budget of the weight stages)
constexpr int WN = 4;                // MFMA tiles per wave along c
constexpr int WGN = 2;               // waves along c (TN = WGN * WN * 16)
constexpr int XCAP = 288;            // window positions per stage
constexpr int XTG = XCAP / 8;        // 8-position groups per window
constexpr int XBLK = XTG * (CK / 8); // 8x8 blocks per window

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef uint16_t u16;

__device__ __forceinline__ void dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_wave_base, 16, 0, 0);
}

// 8x8 transpose of 16-bit values: in[r] holds row r (4 dwords, element 2k in
// the low half of dword k); out[e] receives column e.
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = e >> 1;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t lo = in[2 * m][k], hi = in[2 * m + 1][k];
      out[e][m] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
  }
}

template <int WGM, int WM, int KT, bool FAST>
__global__ __launch_bounds__(WGM * WGN * 64) void conv_bf16_kernel(ConvArgs a, int epi) {
  constexpr int NTHR = WGM * WGN * 64, NWAVE = WGM * WGN;
  constexpr int TM = WGM * WM * 16;
  constexpr int XB = (XBLK + NTHR - 1) / NTHR;
  __shared__ __attribute__((aligned(16))) u16 Xs0[XCAP * RS];
  __shared__ __attribute__((aligned(16))) u16 Xs1[XCAP * RS];
  __shared__ __attribute__((aligned(16))) u16 Ws0[KMAX * TN * RS];
  __shared__ __attribute__((aligned(16))) u16 Ws1[KMAX * TN * RS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WGM, wn = wave / WGM;
  const int lr = lane & 15, kq = lane >> 4;
  // 1-D grid, XCD-aware: workgroup ids round-robin over the 8 XCDs; XCD x
  // takes a contiguous range of tiles ordered (n, t-tile, c-tile) with the
  // c-tile fastest, so the channel tiles of one input window share an L2.
  const int total = a.n_ttiles * a.n_ctiles * (int)a.N;
  int lin = blockIdx.x;
  if ((total & 7) == 0) lin = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int ctile = lin % a.n_ctiles;
  const int ttile = (lin / a.n_ctiles) % a.n_ttiles;
  const int64_t n = lin / (a.n_ctiles * a.n_ttiles);
  const int64_t t0 = (int64_t)ttile * TM;
  const int c0 = ctile * TN;
  const int s = a.stride, d = a.dilation;
  const int64_t T = a.T;

  const u16* __restrict__ x = (const u16*)a.x;
  const u16* __restrict__ wp = (const u16*)a.wp;
  const u16* xn = x + n * a.C_in * T;

  // window of this tile, aligned down to 8 positions (16 bytes)
  const int64_t tbase = t0 * s - a.pad_left;
  const int64_t tal = (tbase >= 0) ? (tbase & ~(int64_t)7) : -(((-tbase) + 7) & ~(int64_t)7);
  const int shift = (int)(tbase - tal);

  // ---- input window: thread -> 8x8 block (position group fastest)
  u32x4 xr[XB][8];
  auto fetch_x = [&](int chunk) {
    const int64_t ci0 = (int64_t)chunk * CK;
#pragma unroll
    for (int b = 0; b < XB; ++b) {
      const int blk = tid + NTHR * b;
      const int tg = blk % XTG, cg = blk / XTG;
      const int64_t t = tal + 8 * tg;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int64_t ci = ci0 + 8 * cg + r;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (blk < XBLK && ci < a.C_in) {
          const u16* src = xn + ci * T;
          if (FAST) {
            if (t >= 0 && t + 7 < T) v = *(const u32x4*)(src + t);
          } else {
            u16 e8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) e8[e] = (t + e >= 0 && t + e < T) ? src[t + e] : (u16)0;
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] = (uint32_t)e8[2 * k] | ((uint32_t)e8[2 * k + 1] << 16);
          }
        }
        xr[b][r] = v;
      }
    }
  };
  auto stash_x = [&](u16* xs) {
#pragma unroll
    for (int b = 0; b < XB; ++b) {
      const int blk = tid + NTHR * b;
      if (blk < XBLK) {
        const int tg = blk % XTG, cg = blk / XTG;
        u32x4 tr[8];
        transpose8x8(xr[b], tr);
#pragma unroll
        for (int e = 0; e < 8; ++e) *(u32x4*)(xs + (8 * tg + e) * RS + 8 * cg) = tr[e];
      }
    }
  };
  // ---- weights: direct copy of the packed LDS image of (ctile, chunk)
  const int wbytes = KT * TN * RS * 2;
  auto dma_w = [&](int chunk, u16* ws) {
    const char* src = (const char*)(wp + ((int64_t)ctile * a.n_chunks + chunk) * (int64_t)(KT * TN * RS));
    for (int p = wave; p * 1024 < wbytes; p += NWAVE)
      dma16(src + p * 1024 + lane * 16, (char*)ws + p * 1024);
  };

  f32x4 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int arow = (wm * WM * 16 + lr) * s + shift;   // window row of subtile 0, tap 0
  const int brow = wn * WN * 16 + lr;
  auto compute = [&](const u16* xs, const u16* ws) {
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      bf16x8 av[WM], bv[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i)
        av[i] = *(const bf16x8*)(xs + (arow + i * 16 * s + j * d) * RS + 8 * kq);
#pragma unroll
      for (int jn = 0; jn < WN; ++jn)
        bv[jn] = *(const bf16x8*)(ws + (j * TN + brow + jn * 16) * RS + 8 * kq);
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int jn = 0; jn < WN; ++jn) acc[i][jn] = mfma16x16x32bf16(av[i], bv[jn], acc[i][jn]);
      // one tap's operands live at a time (keeps the 256-position tile in registers)
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int n_chunks = a.n_chunks;
  dma_w(0, Ws0);
  fetch_x(0);
  stash_x(Xs0);
  __syncthreads();
  for (int c = 0; c < n_chunks; c += 2) {
    if (c + 1 < n_chunks) {
      dma_w(c + 1, Ws1);
      fetch_x(c + 1);
    }
    compute(Xs0, Ws0);
    if (c + 1 < n_chunks) stash_x(Xs1);
    __syncthreads();
    if (c + 1 >= n_chunks) break;
    if (c + 2 < n_chunks) {
      dma_w(c + 2, Ws0);
      fetch_x(c + 2);
    }
    compute(Xs1, Ws1);
    if (c + 2 < n_chunks) stash_x(Xs0);
    __syncthreads();
  }

  conv_epilogue<WM, WN, WGM, WGN>(a, epi, acc, n, t0, c0, ttile, ctile, wm, wn, (Stats*)Ws0);
}

// Weight image: one block of KT*TN*RS bf16 per (ctile, chunk), laid out
// [j][c][r] with r < 32 the input channel inside the chunk and r >= 32 padding:
//   wp[(((ctile*n_chunks + chunk)*K + j)*TN + c)*RS + r] = w[ctile*TN + c][chunk*32 + r][j]
__global__ void conv_bf16_pack_kernel(const u16* __restrict__ w, u16* __restrict__ wp,
                                      int64_t C_in, int64_t C_out, int K, int n_chunks,
                                      int64_t total) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int r = (int)(idx % RS);
  int64_t rest = idx / RS;
  const int c = (int)(rest % TN);
  rest /= TN;
  const int j = (int)(rest % K);
  rest /= K;
  const int chunk = (int)(rest % n_chunks);
  const int64_t ctile = rest / n_chunks;
  const int64_t co = ctile * TN + c;
  const int64_t ci = (int64_t)chunk * CK + r;
  wp[idx] = (r < CK && co < C_out && ci < C_in) ? w[(co * C_in + ci) * K + j] : (u16)0;
}

template <int WGM, int WM, int KT>
hipError_t launch_wk(const ConvArgs& a, int epi, hipStream_t st) {
  dim3 grid((unsigned)(a.n_ttiles * a.n_ctiles * a.N));
  constexpr int nthr = WGM * WGN * 64;
  const bool fast = (a.T % 8 == 0) && ((((uintptr_t)a.x) & 15) == 0);
  if (fast)
    hipLaunchKernelGGL((conv_bf16_kernel<WGM, WM, KT, true>), grid, dim3(nthr), 0, st, a, epi);
  else
    hipLaunchKernelGGL((conv_bf16_kernel<WGM, WM, KT, false>), grid, dim3(nthr), 0, st, a, epi);
  return hipGetLastError();
}

template <int WGM, int WM>
hipError_t launch_w(const ConvArgs& a, int epi, hipStream_t st) {
  switch (a.K) {
    case 1: return launch_wk<WGM, WM, 1>(a, epi, st);
    case 2: return launch_wk<WGM, WM, 2>(a, epi, st);
    case 3: return launch_wk<WGM, WM, 3>(a, epi, st);
    case 4: return launch_wk<WGM, WM, 4>(a, epi, st);
    case 5: return launch_wk<WGM, WM, 5>(a, epi, st);
    default: return hipErrorInvalidValue;
  }
}

// window (incl. the 8-position alignment shift) a TM-position tile needs
int64_t window(int tm, int stride, int K, int dilation) {
  return (int64_t)(tm - 1) * stride + (int64_t)(K - 1) * dilation + 1 + 7;
}

}  // namespace

int conv_bf16_tile_m(int stride, int K, int dilation) {
  if (K < 1 || K > KMAX) return 0;
  if (window(256, stride, K, dilation) <= XCAP) return 256;
  if (window(64, stride, K, dilation) <= XCAP) return 64;
  return 0;
}

size_t conv_bf16_packed_bytes(int64_t C_in, int64_t C_out, int K) {
  const int64_t n_chunks = (C_in + CK - 1) / CK, n_ctiles = (C_out + TN - 1) / TN;
  return (size_t)(n_ctiles * n_chunks * K * TN * RS) * sizeof(u16);
}

hipError_t conv_bf16_pack(const uint16_t* w, uint16_t* wp, int64_t C_in, int64_t C_out, int K,
                          hipStream_t s) {
  const int n_chunks = (int)((C_in + CK - 1) / CK);
  const int64_t total = (int64_t)(conv_bf16_packed_bytes(C_in, C_out, K) / sizeof(u16));
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(conv_bf16_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, wp, C_in,
                     C_out, K, n_chunks, total);
  return hipGetLastError();
}

hipError_t conv_bf16_launch(const ConvArgs& a, int epi, hipStream_t s) {
  const int tm = conv_bf16_tile_m(a.stride, a.K, a.dilation);
  if (tm == 256) return launch_w<4, 4>(a, epi, s);  // 8 waves, 64 x 64 each
  if (tm == 64) return launch_w<2, 2>(a, epi, s);   // 4 waves, 32 x 64 each
  return hipErrorInvalidValue;
}

}  // namespace c1g
