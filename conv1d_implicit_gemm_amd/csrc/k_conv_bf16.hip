// bf16 implicit-GEMM 1-D convolution for gfx950 (split path), fp32 accumulate.
//
// GEMM view ("Kimi-K2.6 l1_p5", the implicit-GEMM shape M = N*T_out,
// N = C_out, K = C_in*K): row m = (n, t), column = output channel c; the
// reduction runs over (tap j, input channel ci) in chunks of 32 input channels,
// one v_mfma_f32_16x16x32_bf16 K-step per tap.  The MFMA wants 8 consecutive
// reduction values per lane, i.e. 8 consecutive input channels at one position,
// while x is stored position-contiguous, so the input halo window of a tile is
// transposed while it is staged: a lane loads an 8 (channels) x 8 (positions)
// block with 16-byte loads along t, transposes it in registers and writes 8
// rows of the LDS window Xt[t][ci].  Every tap then reads the same window at a
// shifted row offset.  The weights are repacked once per call into the exact
// LDS image of each (c-tile, chunk) and streamed with direct global->LDS loads.
//
// LDS rows are 64 bytes (32 bf16) with no padding; the 16-byte column of a row
// is XOR-ed with 2 when bit 2 of the row index is set.  The LDS has 64
// four-byte banks and serves a 16-byte-per-lane read in four passes of 16
// lanes (lanes 0-7 with 16-23, and so on), so an operand read of rows r..r+7
// and two adjacent columns touches 16 distinct groups of 4 banks for any r
// (unit stride); without the XOR, rows r and r+4 would collide.
//
// Workgroup: 512 threads; tile TM (512 or 128) positions x 128 channels.  The
// eight waves form a 4 x 2 grid of wave tiles of WM x 4 MFMA tiles (128 x 64
// for TM = 512), each running every tap, so a wave reads 12 KB of operands per
// 32 MFMAs and two waves per SIMD hide LDS latency.  The tile is tall because
// the L2 -> LDS path moves ~40 bytes per clock per CU (measured, the same for
// direct loads and for register staging): a 512-position tile stages 75 KB per
// chunk for 21 MFLOP, where a 256-position one needs 58 KB for half the work.
// Two LDS stages: the next chunk's weights stream in and its window is loaded
// into registers while the current chunk is consumed; every wave takes a
// share of the staging.  Window blocks go to lanes channel-group fastest, so
// the 8 lanes of one 16-byte LDS write pass (32 banks, 8 consecutive lanes per
// pass for writes) cover two rows and all four columns: a 2-way conflict, the
// least possible for rows that share their index modulo 8.  Epilogue: shared with
// the fp32 kernel (store y, GroupNorm or channel-LayerNorm partial statistics).
#include "common.hpp"
#include "conv_epilogue.hpp"
#include "launch.hpp"

namespace c1g {
namespace {

constexpr int TN = ConvBf16Cfg::TN;  // 128 output channels per tile
constexpr int CK = ConvBf16Cfg::CK;  // 32 input channels per chunk
constexpr int RW = CK;               // LDS row: 32 bf16 (64 bytes)
constexpr int KMAX = 8;              // taps: up to 5 on 512-position tiles, 8 on 128
constexpr int WN = 4;                // MFMA tiles per wave along c
constexpr int WGN = 2;               // waves along c (TN = WGN * WN * 16)
constexpr int WGM = 4;               // waves along t
constexpr int NWAVE = WGM * WGN;
constexpr int NTHR = NWAVE * 64;
// LDS per workgroup: two stages of (window XC rows + weight image of the taps)
// of 64-byte rows.  XC = 544 rows with up to 5 taps (150 KB), or 224 rows with
// 6 to 8 taps on 128-position tiles (156 KB); gfx950 allows 160 KB.
constexpr int XCAP_WIDE = 544, XCAP_TAPS = 224;
template <int XC>
struct XGeom {
  static constexpr int XTG = XC / 8;        // 8-position groups per window
  static constexpr int XBLK = XTG * (CK / 8); // 8x8 blocks per window
  static constexpr int XLANES = XBLK / NWAVE; // lanes per wave that stage one block each
  static_assert(XBLK % NWAVE == 0 && XLANES <= 64, "window blocks spread over the waves");
};
static_assert(TN == 128, "weight rows keep bit 2 of c across taps");

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef uint16_t u16;

__device__ __forceinline__ void dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_wave_base, 16, 0, 0);
}

// 16-byte column swizzle of LDS row `row`
__host__ __device__ __forceinline__ int swz(int row) { return (row >> 1) & 2; }

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

template <int WM, int KT, bool FAST, int XC>
__global__ __launch_bounds__(NTHR) void conv_bf16_kernel(ConvArgs a, int epi) {
  constexpr int XLANES = XGeom<XC>::XLANES;
  // the weight stage also holds the epilogue's cross-wave merge (<= 12 KB)
  constexpr int WSK = KT < 2 ? 2 : KT;
  constexpr int TM = WGM * WM * 16;
  __shared__ __attribute__((aligned(16))) u16 Xs0[XC * RW];
  __shared__ __attribute__((aligned(16))) u16 Xs1[XC * RW];
  __shared__ __attribute__((aligned(16))) u16 Ws0[WSK * TN * RW];
  __shared__ __attribute__((aligned(16))) u16 Ws1[WSK * TN * RW];

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

  // ---- input window: lanes 0..XLANES-1 of every wave own one 8x8 block
  // (8 positions of 8 channels), channel group fastest
  const bool xown = lane < XLANES;
  const int blk = wave * XLANES + (xown ? lane : 0);
  const int tg = blk >> 2, cg = blk & 3;
  const int64_t tx = tal + 8 * tg;
  u32x4 xr[8];
  auto fetch_x = [&](int chunk) __attribute__((always_inline)) {
    const int64_t ci0 = (int64_t)chunk * CK + 8 * cg;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t ci = ci0 + r;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (xown && ci < a.C_in) {
        const u16* src = xn + ci * T;
        if (FAST) {
          // T % 8 == 0 and the group is 8-aligned: wholly inside or outside
          if (tx >= 0 && tx < T) v = *(const u32x4*)(src + tx);
        } else {
          u16 e8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) e8[e] = (tx + e >= 0 && tx + e < T) ? src[tx + e] : (u16)0;
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = (uint32_t)e8[2 * k] | ((uint32_t)e8[2 * k + 1] << 16);
        }
      }
      xr[r] = v;
    }
  };
  auto stash_x = [&](u16* xs) __attribute__((always_inline)) {
    if (xown) {
      u32x4 tr[8];
      transpose8x8(xr, tr);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = 8 * tg + e;
        *(u32x4*)(xs + row * RW + 8 * (cg ^ swz(row))) = tr[e];
      }
    }
  };
  // ---- weights: direct copy of the packed LDS image of (ctile, chunk),
  // KT * 8 pieces of 1 KB spread over the waves
  auto dma_w = [&](int chunk, u16* ws) __attribute__((always_inline)) {
    const char* src = (const char*)(wp + ((int64_t)ctile * a.n_chunks + chunk) * (int64_t)(KT * TN * RW));
#pragma unroll
    for (int p = 0; p < (KT * 8 + NWAVE - 1) / NWAVE; ++p) {
      const int piece = wave + NWAVE * p;
      if (piece < KT * 8) dma16(src + piece * 1024 + lane * 16, (char*)ws + piece * 1024);
    }
  };

  f32x4 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int arow0 = (wm * WM * 16 + lr) * s + shift;  // window row of subtile 0, tap 0
  const int bcol = 8 * (kq ^ swz(lr));                // weight rows: bit 2 of c = bit 2 of lr
  auto tap = [&](const u16* xs, const u16* ws, int j) __attribute__((always_inline)) {
    const int r0 = arow0 + j * d;                       // rows r0 + 16*s*i keep bit 2
    const u16* xa = xs + r0 * RW + 8 * (kq ^ swz(r0));
    const u16* wb = ws + (j * TN + wn * WN * 16 + lr) * RW + bcol;
    bf16x8 av[WM], bv[WN];
#pragma unroll
    for (int jn = 0; jn < WN; ++jn) bv[jn] = *(const bf16x8*)(wb + jn * 16 * RW);
#pragma unroll
    for (int i = 0; i < WM; ++i) av[i] = *(const bf16x8*)(xa + i * 16 * s * RW);
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int jn = 0; jn < WN; ++jn) acc[i][jn] = mfma16x16x32bf16(av[i], bv[jn], acc[i][jn]);
    __builtin_amdgcn_sched_group_barrier(0x100, WM + WN, 0);  // all operand reads first
    __builtin_amdgcn_sched_group_barrier(0x008, WM * WN, 0);  // then the MFMAs
    __builtin_amdgcn_sched_barrier(0);  // one tap's operands live at a time
  };
  // every tap of the chunk; one tap body in a runtime loop keeps a single copy
  // of it in registers
  auto compute = [&](const u16* xs, const u16* ws) __attribute__((always_inline)) {
#pragma nounroll
    for (int j = 0; j < KT; ++j) tap(xs, ws, j);
  };

  // Pairs of chunks per iteration, loads clamped to the last chunk and issued
  // unconditionally (surplus copies land in a stage nobody reads again), so
  // the loop body is one block; every load of a chunk completes before the
  // barrier that ends the half in which it was issued.
  const int n_chunks = a.n_chunks, last = n_chunks - 1;
  auto cl = [&](int c) { return c < last ? c : last; };
  dma_w(0, Ws0);
  fetch_x(0);
  stash_x(Xs0);
  __syncthreads();
  int c = 0;
  for (; c + 1 < n_chunks; c += 2) {
    // stage 0 holds chunk c
    dma_w(c + 1, Ws1);
    fetch_x(c + 1);
    compute(Xs0, Ws0);
    stash_x(Xs1);
    __syncthreads();
    // stage 1 holds chunk c+1
    dma_w(cl(c + 2), Ws0);
    fetch_x(cl(c + 2));
    compute(Xs1, Ws1);
    stash_x(Xs0);
    __syncthreads();
  }
  if (c < n_chunks) {  // odd count: the last chunk is in stage 0
    compute(Xs0, Ws0);
    __syncthreads();
  }

  conv_epilogue<WM, WN, WGM, WGN>(a, epi, acc, n, t0, c0, ttile, ctile, wm, wn, (Stats*)Ws0);
}

// Weight image: one block of K*TN*RW bf16 per (ctile, chunk), laid out
// [j][c][32] with the input channels of the chunk in four 16-byte columns,
// column q of row c stored at column q ^ swz(c):
//   wp[(((ctile*n_chunks + chunk)*K + j)*TN + c)*RW + 8*(q ^ swz(c)) + e]
//     = w[ctile*TN + c][chunk*32 + 8*q + e][j]      (0 outside the tensor)
__global__ void conv_bf16_pack_kernel(const u16* __restrict__ w, u16* __restrict__ wp,
                                      int64_t C_in, int64_t C_out, int K, int n_chunks,
                                      int64_t total) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int e = (int)(idx % 8);
  const int pq = (int)((idx / 8) % (RW / 8));
  int64_t rest = idx / RW;
  const int c = (int)(rest % TN);
  rest /= TN;
  const int j = (int)(rest % K);
  rest /= K;
  const int chunk = (int)(rest % n_chunks);
  const int64_t ctile = rest / n_chunks;
  const int q = pq ^ swz(c);
  const int64_t co = ctile * TN + c;
  const int64_t ci = (int64_t)chunk * CK + 8 * q + e;
  wp[idx] = (co < C_out && ci < C_in) ? w[(co * C_in + ci) * K + j] : (u16)0;
}

template <int WM, int KT, int XC>
hipError_t launch_wk(const ConvArgs& a, int epi, hipStream_t st) {
  dim3 grid((unsigned)(a.n_ttiles * a.n_ctiles * a.N));
  const bool fast = (a.T % 8 == 0) && ((((uintptr_t)a.x) & 15) == 0);
  if (fast)
    hipLaunchKernelGGL((conv_bf16_kernel<WM, KT, true, XC>), grid, dim3(NTHR), 0, st, a, epi);
  else
    hipLaunchKernelGGL((conv_bf16_kernel<WM, KT, false, XC>), grid, dim3(NTHR), 0, st, a, epi);
  return hipGetLastError();
}

template <int WM>
hipError_t launch_w(const ConvArgs& a, int epi, hipStream_t st) {
  switch (a.K) {
    case 1: return launch_wk<WM, 1, XCAP_WIDE>(a, epi, st);
    case 2: return launch_wk<WM, 2, XCAP_WIDE>(a, epi, st);
    case 3: return launch_wk<WM, 3, XCAP_WIDE>(a, epi, st);
    case 4: return launch_wk<WM, 4, XCAP_WIDE>(a, epi, st);
    case 5: return launch_wk<WM, 5, XCAP_WIDE>(a, epi, st);
    default: break;
  }
  if (WM != 2) return hipErrorInvalidValue;
  switch (a.K) {
    case 6: return launch_wk<2, 6, XCAP_TAPS>(a, epi, st);
    case 7: return launch_wk<2, 7, XCAP_TAPS>(a, epi, st);
    case 8: return launch_wk<2, 8, XCAP_TAPS>(a, epi, st);
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
  if (K <= 5 && window(512, stride, K, dilation) <= XCAP_WIDE) return 512;
  if (window(128, stride, K, dilation) <= (K <= 5 ? XCAP_WIDE : XCAP_TAPS)) return 128;
  return 0;
}

size_t conv_bf16_packed_bytes(int64_t C_in, int64_t C_out, int K) {
  const int64_t n_chunks = (C_in + CK - 1) / CK, n_ctiles = (C_out + TN - 1) / TN;
  return (size_t)(n_ctiles * n_chunks * K * TN * RW) * sizeof(u16);
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
  if (tm == 512) return launch_w<8>(a, epi, s);  // wave tiles 128 x 64
  if (tm == 128) return launch_w<2>(a, epi, s);  // wave tiles 32 x 64
  return hipErrorInvalidValue;
}

}  // namespace c1g
