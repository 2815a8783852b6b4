// bf16 GEMM for the K = 1, T = 1 convolution (a Linear layer):
//   y[n][c] = sum_ci x[n][ci] * w[c][ci]      (x [N, C_in], w [C_out, C_in])
// with an optional fused GroupNorm + per-row min epilogue ("Kimi-K2.6 l2_p75":
// Linear -> GroupNorm -> min over channels -> + bias broadcast; with T = 1 a
// GroupNorm group is C_out/G consecutive channels of one row).
//
// MFMA view (v_mfma_f32_16x16x32_bf16): A = w (rows c), B = x^T (columns n);
// both operands are contiguous along the reduction, so each 64-element chunk
// of a row is loaded with 16-byte loads (two chunks ahead, into registers) and
// written to LDS rows of 160 bytes (80 bf16, the last 32 bytes unused).  The
// LDS has 64 four-byte banks and serves a 16-byte-per-lane read in four passes
// of 16 lanes (lanes 0-7 with 16-23, 8-15 with 24-31, and so on); an operand
// read puts rows r..r+7 and two adjacent 16-byte columns in one pass, and with
// a 160-byte stride those 16 pieces fall on 16 disjoint groups of 4 banks
// (a 144-byte stride would make two of them collide).
// Workgroup: 512 threads, tile 256 (c) x 128 (n), two LDS stages (one is read
// while the other is written from registers).  The eight waves form a 2 x 2
// grid of 128 x 64 wave tiles (8 x 4 MFMA tiles) times two halves of each
// chunk's reduction: the two waves of a SIMD own the same output tile and take
// alternate 32-wide K-steps, so each wave reads 12 KB of operands from LDS per
// 32 MFMAs (a 64 x 64 wave tile would need 16 KB per 16) while a second wave
// per SIMD still hides LDS latency.  The two halves are summed through LDS once
// at the end, in a fixed order.
// Workgroups are mapped so that each XCD works on a compact block of tiles and
// its L2 serves the shared rows of w and x.
//
// Result layout: lane (lr, kq), register r of tile (i, j) holds
// c = c0 + 16 i + 4 kq + r, n = n0 + 16 j + lr, so a 16-channel group of one
// row is exactly one MFMA tile column (4 registers x 4 lanes).
//
// Epilogues: GEMM_STORE writes y (+bias).  GEMM_GN_ROWMIN (C_out/G == 16)
// normalises each group in registers (two-pass mean/variance over its 16
// values), applies gamma/beta, and reduces min over the tile's channels into
// one partial per (n, c-tile) (fixed slots, no atomics); optional mean/rstd
// outputs.  rowmin_bcast then folds the partials in a fixed order and writes
// out[n][c] = min + bias2[c].
#include "common.hpp"
#include "launch.hpp"

namespace c1g {
namespace {

constexpr int WGC = 2, WGNN = 2;  // spatial waves along c and along n
constexpr int KSPLIT = 2;         // waves sharing one output tile (one per K-step)
constexpr int NWAVE = WGC * WGNN * KSPLIT;
constexpr int NTHR = NWAVE * 64;
constexpr int BM = 256;        // channels per tile (A rows)
constexpr int BN = 128;        // samples per tile (B rows)
constexpr int KC = 64;         // reduction chunk (two MFMA K-steps)
constexpr int RS = KC + 16;    // LDS row stride in bf16 (160 bytes)
constexpr int QPR = KC / 8;    // 16-byte slots of data per row
constexpr int NSLOT = (BM + BN) * QPR;           // slots per chunk (A rows, then B rows)
constexpr int SPT = NSLOT / NTHR;                // slots per thread
static_assert(NSLOT % NTHR == 0, "whole slots per thread");
static_assert(KC / 32 == KSPLIT, "one K-step per wave per chunk");
constexpr int WMT = BM / (16 * WGC), WNT = BN / (16 * WGNN);  // 8 x 4 MFMA tiles per wave
constexpr int STAGE = (BM + BN) * RS;            // bf16 per LDS stage
// the K-half reduction moves half of a wave's accumulators per round
constexpr int RED_ROUND_BYTES = WGC * WGNN * (WMT / 2) * WNT * 64 * 16;
static_assert(RED_ROUND_BYTES <= 2 * STAGE * 2, "reduction round fits in the stages");

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef uint16_t u16;


template <int EPI>
__global__ __launch_bounds__(NTHR) void gemm_bf16_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) u16 smem[2 * STAGE];
  u16* const As0 = smem;
  u16* const Bs0 = smem + BM * RS;
  u16* const As1 = smem + STAGE;
  u16* const Bs1 = smem + STAGE + BM * RS;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wslot = wave & 3;                 // spatial position of the wave
  const int kh = wave >> 2;                   // K-step of each chunk it takes
  const int wc = wslot % WGC, wnn = wslot / WGC;
  const int lr = lane & 15, kq = lane >> 4;

  // XCD-aware tile order: blocks round-robin over 8 XCDs; give XCD x the
  // contiguous tile range [x*tiles/8, (x+1)*tiles/8), enumerated n-tile fastest
  // so the c-tiles (rows of w) it touches are few and shared in its L2.
  const int tiles = a.n_ctiles * a.n_ntiles;
  int lin = blockIdx.x;
  if ((tiles & 7) == 0) lin = (blockIdx.x & 7) * (tiles >> 3) + (blockIdx.x >> 3);
  const int ntile = lin % a.n_ntiles, ctile = lin / a.n_ntiles;
  const int64_t c0 = (int64_t)ctile * BM, n0 = (int64_t)ntile * BN;

  const u16* __restrict__ w = (const u16*)a.w;
  const u16* __restrict__ x = (const u16*)a.x;
  const int n_chunks = (int)((a.C_in + KC - 1) / KC);

  f32x4 acc[WMT][WNT];
#pragma unroll
  for (int i = 0; i < WMT; ++i)
#pragma unroll
    for (int j = 0; j < WNT; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int arow = wc * WMT * 16 + lr, brow = wnn * WNT * 16 + lr;
  auto compute = [&](const u16* as, const u16* bs) {
    bf16x8 av[WMT], bv[WNT];
#pragma unroll
    for (int j = 0; j < WNT; ++j)
      bv[j] = *(const bf16x8*)(bs + (brow + 16 * j) * RS + 32 * kh + 8 * kq);
#pragma unroll
    for (int i = 0; i < WMT; ++i)
      av[i] = *(const bf16x8*)(as + (arow + 16 * i) * RS + 32 * kh + 8 * kq);
#pragma unroll
    for (int i = 0; i < WMT; ++i)
#pragma unroll
      for (int j = 0; j < WNT; ++j) acc[i][j] = mfma16x16x32bf16(av[i], bv[j], acc[i][j]);
  };
  // Staging: thread tid owns slots tid + NTHR*i of a chunk (A rows first, then
  // B rows; slot = row * QPR + 16-byte column group), so slot i of every thread
  // is an A slot for i < SPT_A and a B slot after.  Rows past the matrix read
  // its last row (their products land in outputs that are never stored).  Each
  // slot keeps a 32-bit byte offset from the matrix base (rows * C_in < 2^31
  // elements on this route), so a load is one uniform base plus one register.
  constexpr int SPT_A = BM * QPR / NTHR;
  static_assert(BM * QPR % NTHR == 0, "A slots fill whole thread rounds");
  const int q = tid % QPR;
  const int rbase = tid / QPR;                 // row of slot 0 (A) / slot SPT_A (B)
  constexpr int RSTEP = NTHR / QPR;            // rows between a thread's slots
  uint32_t soff[SPT];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const bool b = i >= SPT_A;
    const int row = rbase + RSTEP * (b ? i - SPT_A : i);
    int64_t gr = (b ? n0 : c0) + row;
    const int64_t R = b ? a.N : a.C_out;
    if (gr > R - 1) gr = R - 1;
    soff[i] = (uint32_t)((gr * a.C_in + 8 * q) * 2);
  }
  const char* const wbytes = (const char*)w;
  const char* const xbytes = (const char*)x;
  // whole chunks only (the reduction tail, if any, is handled after the loop)
  auto fetch = [&](int chunk, u32x4 (&r)[SPT]) {
    const int64_t kb = (int64_t)chunk * KC * 2;
#pragma unroll
    for (int i = 0; i < SPT; ++i)
      r[i] = *(const u32x4*)((i >= SPT_A ? xbytes : wbytes) + kb + soff[i]);
  };
  auto stash = [&](const u32x4 (&r)[SPT], u16* as, u16* bs) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const bool b = i >= SPT_A;
      const int row = rbase + RSTEP * (b ? i - SPT_A : i);
      *(u32x4*)((b ? bs : as) + row * RS + 8 * q) = r[i];
    }
  };

  // Issue order within a chunk: the 12 operand reads, then the MFMAs with one
  // global load and one LDS write (of the other stage, free since the last
  // barrier) after every 4 MFMAs, so the loads reach the address unit spread
  // over the chunk instead of in one burst that stalls the issuing waves.
  auto schedule = [] {
    __builtin_amdgcn_sched_group_barrier(0x100, WMT + WNT, 0);  // DS reads
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);        // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);        // VMEM read
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);        // DS write
    }
    __builtin_amdgcn_sched_group_barrier(0x008, WMT * WNT - 4 * SPT, 0);
  };

  // Main loop over pairs of whole chunks.  The prefetch and stash run
  // unconditionally, on chunk indices clamped to the last whole chunk (the
  // surplus copies land in a stage nobody reads again), and the loop body is
  // one block with one back edge: the compiler then counts the loads in
  // flight exactly, so each write of a staged chunk waits only for its own
  // loads while the next chunk's loads stay in flight.
  const int n_full = (int)(a.C_in / KC);
  if (n_full > 0) {
    const int last = n_full - 1;
    auto cl = [&](int c) { return c < last ? c : last; };
    u32x4 ra[SPT], rb[SPT];
    fetch(0, ra);
    fetch(cl(1), rb);
    stash(ra, As0, Bs0);
    __syncthreads();
    int c = 0;
    for (; c + 1 < n_full; c += 2) {
      // stage 0 holds chunk c; rb holds chunk c+1
      fetch(cl(c + 2), ra);
      compute(As0, Bs0);
      stash(rb, As1, Bs1);
      schedule();
      __syncthreads();
      // stage 1 holds chunk c+1; ra holds chunk c+2
      fetch(cl(c + 3), rb);
      compute(As1, Bs1);
      stash(ra, As0, Bs0);
      schedule();
      __syncthreads();
    }
    if (c < n_full) {  // odd count: the last whole chunk is in stage 0
      compute(As0, Bs0);
      __syncthreads();
    }
  }
  // Reduction tail (C_in % 64 != 0; C_in % 8 == 0, so a 16-byte slot lies
  // wholly inside or wholly past C_in): slots past C_in load column 0 of their
  // row (in bounds) and are written as zeros.  Every stage is free here.
  if (a.C_in % KC != 0) {
    const int64_t k0 = (int64_t)n_full * KC;
    const bool inside = k0 + 8 * q < a.C_in;
    const int64_t kb = inside ? k0 * 2 : -(int64_t)(8 * q) * 2;
    u32x4 rt[SPT];
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const u32x4 v = *(const u32x4*)((i >= SPT_A ? xbytes : wbytes) + kb + soff[i]);
      rt[i] = inside ? v : (u32x4){0u, 0u, 0u, 0u};
    }
    stash(rt, As0, Bs0);
    __syncthreads();
    compute(As0, Bs0);
    __syncthreads();
  }

  // K-half reduction: the kh = 1 wave of each spatial slot adds its partial
  // sums into the kh = 0 wave's, half of the tile per round (lane-contiguous
  // 16-byte slots, so the LDS traffic is conflict-free).
  {
    f32x4* red = (f32x4*)smem;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < WMT / 2; ++i)
#pragma unroll
        for (int j = 0; j < WNT; ++j) {
          f32x4* slot = red + ((wslot * (WMT / 2) + i) * WNT + j) * 64 + lane;
          if (kh == 1) *slot = acc[h * (WMT / 2) + i][j];
        }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < WMT / 2; ++i)
#pragma unroll
        for (int j = 0; j < WNT; ++j) {
          const f32x4* slot = red + ((wslot * (WMT / 2) + i) * WNT + j) * 64 + lane;
          if (kh == 0) acc[h * (WMT / 2) + i][j] += *slot;
        }
      __syncthreads();
    }
  }

  // ------------------------------------------------------------------ epilogue
  // (kh = 0 waves hold the complete tile; kh = 1 waves only join the barriers)
  if (EPI == GEMM_STORE) {
    if (kh != 0) return;
    // y as fp32, or rounded to bf16 (y_bf16)
    auto store = [&](auto* y) __attribute__((always_inline)) {
      const bool vec = (a.C_out % 4 == 0) && ((((uintptr_t)y) & (4 * sizeof(*y) - 1)) == 0);
#pragma unroll
      for (int i = 0; i < WMT; ++i) {
        const int64_t c = c0 + wc * WMT * 16 + 16 * i + 4 * kq;
        f32x4 b = {0.f, 0.f, 0.f, 0.f};
        if (a.bias)
#pragma unroll
          for (int r = 0; r < 4; ++r) b[r] = (c + r < a.C_out) ? a.bias[c + r] : 0.f;
#pragma unroll
        for (int j = 0; j < WNT; ++j) {
          const int64_t nn = n0 + wnn * WNT * 16 + 16 * j + lr;
          if (nn >= a.N) continue;
          const f32x4 v = acc[i][j] + b;
          auto* dst = y + nn * a.C_out + c;
          if (vec && c + 3 < a.C_out) {
            store_elem4(dst, v);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (c + r < a.C_out) store_elem(dst + r, v[r]);
          }
        }
      }
    };
    if (a.y_bf16)
      store((uint16_t*)a.y);
    else
      store((float*)a.y);
  } else {  // GEMM_GN_ROWMIN: groups of 16 channels = one tile column block
    float* red = (float*)smem;  // free after the reduction's last barrier
    float rmin[WNT];
#pragma unroll
    for (int j = 0; j < WNT; ++j) rmin[j] = __builtin_inff();
#pragma unroll
    for (int i = 0; i < WMT; ++i) {
      const int64_t cg = c0 + wc * WMT * 16 + 16 * i;  // first channel of the group
      const bool gvalid = cg < a.C_out && kh == 0;
      const int64_t c = cg + 4 * kq;
      f32x4 ga = {1.f, 1.f, 1.f, 1.f}, be = {0.f, 0.f, 0.f, 0.f}, bi = {0.f, 0.f, 0.f, 0.f};
      if (gvalid) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (a.gamma) ga[r] = a.gamma[c + r];
          if (a.beta) be[r] = a.beta[c + r];
          if (a.bias) bi[r] = a.bias[c + r];
        }
      }
#pragma unroll
      for (int j = 0; j < WNT; ++j) {
        const f32x4 v = acc[i][j] + bi;
        float s = (v[0] + v[1]) + (v[2] + v[3]);
        s += shfl_xor(s, 16);
        s += shfl_xor(s, 32);
        const float mean = s * (1.0f / 16.0f);
        float q = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) { const float dv = v[r] - mean; q += dv * dv; }
        q += shfl_xor(q, 16);
        q += shfl_xor(q, 32);
        const float rstd = 1.0f / sqrtf(q * (1.0f / 16.0f) + a.eps);
        float m = __builtin_inff();
#pragma unroll
        for (int r = 0; r < 4; ++r) m = fminf(m, (v[r] - mean) * (rstd * ga[r]) + be[r]);
        if (gvalid) rmin[j] = fminf(rmin[j], m);
        const int64_t nn = n0 + wnn * WNT * 16 + 16 * j + lr;
        if (gvalid && kq == 0 && nn < a.N) {
          const int64_t g = cg / 16;
          if (a.mean_out) a.mean_out[nn * a.G + g] = mean;
          if (a.rstd_out) a.rstd_out[nn * a.G + g] = rstd;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < WNT; ++j) {
      float m = rmin[j];
      m = fminf(m, shfl_xor(m, 16));
      m = fminf(m, shfl_xor(m, 32));
      if (kq == 0 && kh == 0) red[wc * BN + wnn * WNT * 16 + 16 * j + lr] = m;
    }
    __syncthreads();
    if (tid < BN) {
      const int64_t nn = n0 + tid;
      float m = red[tid];
#pragma unroll
      for (int w = 1; w < WGC; ++w) m = fminf(m, red[w * BN + tid]);
      if (nn < a.N) a.part[nn * a.n_ctiles + ctile] = m;
    }
  }
}

// out[n][c] = min over c-tiles of part[n][*] + bias2[c]; one workgroup per row;
// TO is float, or bf16 bits (rounded to nearest even)
template <typename TO>
__global__ __launch_bounds__(NTHR) void rowmin_bcast_kernel(const float* __restrict__ part,
                                                            int n_ctiles,
                                                            const float* __restrict__ bias2,
                                                            TO* out, int64_t C) {
  const int64_t n = blockIdx.x;
  float m = __builtin_inff();
  for (int t = 0; t < n_ctiles; ++t) m = fminf(m, part[n * n_ctiles + t]);
  TO* row = out + n * C;
  if ((C % 4) == 0 && (((uintptr_t)out) & (4 * sizeof(TO) - 1)) == 0 &&
      (((uintptr_t)bias2) & 15) == 0) {
    for (int64_t q = threadIdx.x; q < C / 4; q += NTHR) {
      const f32x4 b = *(const f32x4*)(bias2 + 4 * q);
      store_elem4(row + 4 * q, b + m);
    }
  } else {
    for (int64_t c = threadIdx.x; c < C; c += NTHR) store_elem(row + c, m + bias2[c]);
  }
}

}  // namespace

hipError_t gemm_bf16_launch(const GemmArgs& a, int epi, hipStream_t s) {
  dim3 grid((unsigned)(a.n_ctiles * a.n_ntiles));
  if (epi == GEMM_STORE)
    hipLaunchKernelGGL(gemm_bf16_kernel<GEMM_STORE>, grid, dim3(NTHR), 0, s, a);
  else
    hipLaunchKernelGGL(gemm_bf16_kernel<GEMM_GN_ROWMIN>, grid, dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

hipError_t rowmin_bcast_launch(const float* part, int64_t N, int n_ctiles, const float* bias2,
                               void* out, bool out_bf16, int64_t C, hipStream_t s) {
  if (out_bf16)
    hipLaunchKernelGGL(rowmin_bcast_kernel<uint16_t>, dim3((unsigned)N), dim3(NTHR), 0, s, part,
                       n_ctiles, bias2, (uint16_t*)out, C);
  else
    hipLaunchKernelGGL(rowmin_bcast_kernel<float>, dim3((unsigned)N), dim3(NTHR), 0, s, part,
                       n_ctiles, bias2, (float*)out, C);
  return hipGetLastError();
}

int gemm_bf16_tile_c() { return BM; }
int gemm_bf16_tile_n() { return BN; }

}  // namespace c1g
