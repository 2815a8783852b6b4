// bf16 GEMM for the K = 1, T = 1 convolution (a Linear layer):
//   y[n][c] = sum_ci x[n][ci] * w[c][ci]      (x [N, C_in], w [C_out, C_in])
// with an optional fused GroupNorm + per-row min epilogue ("Kimi-K2.6 l2_p75":
// Linear -> GroupNorm -> min over channels -> + bias broadcast; with T = 1 a
// GroupNorm group is C_out/G consecutive channels of one row).
//
// MFMA view (v_mfma_f32_16x16x32_bf16): A = w (rows c), B = x^T (columns n);
// both operands are contiguous along the reduction.  Workgroup: 512 threads,
// tile 256 (c) x 128 (n), reduction chunks of 64 (128 bytes of each row).
// Staging: direct global -> LDS copies (global_load_lds, 16 bytes per lane,
// 1 KB = 8 rows per instruction, no registers), three LDS stages of 48 KB,
// copies two chunks ahead.  Rows are 128 bytes with no padding; the 16-byte
// column q of row r sits at column q ^ (r & 6), which keeps the operand reads
// conflict-free: the LDS has 64 four-byte banks and serves a 16-byte-per-lane
// read in four passes of 16 lanes (lanes 0-7 with 16-23, 8-15 with 24-31, and
// so on), and a pass reads rows r..r+7 at two adjacent columns, which the
// swizzle spreads over 16 disjoint groups of 4 banks.
// The eight waves form a 2 x 2 grid of 128 x 64 wave tiles (8 x 4 MFMA tiles)
// times two halves of each chunk's reduction: the two waves of a SIMD own the
// same output tile and take alternate 32-wide K-steps, so each wave reads 12
// KB of operands from LDS per 32 MFMAs (a 64 x 64 wave tile would need 16 KB
// per 16).  A wave reads the next chunk's operands while its MFMAs run on the
// current ones (the B fragments into a second set, each A fragment into the
// register whose last MFMA has issued), so the LDS reads overlap the matrix
// work; one barrier per chunk.  At the end the two waves of a slot swap
// halves of their partial sums through LDS, each finishing half the rows.
// Workgroups are mapped so that each XCD works on a compact block of tiles and
// its L2 serves the shared rows of w and x.
//
// Result layout: lane (lr, kq), register r of tile (i, j) holds
// c = c0 + 16 i + 4 kq + r, n = n0 + 16 j + lr, so a 16-channel group of one
// row is exactly one MFMA tile column (4 registers x 4 lanes).
//
// Epilogues: GEMM_STORE writes y (+bias).  GEMM_GN_ROWMIN (C_out/G == 16)
// normalises each group in registers (two-pass mean/variance over its 16
// values, reduced across lanes with lane swaps; rstd by the hardware
// reciprocal square root), applies gamma/beta, and reduces min over the
// tile's channels into
// one partial per (n, c-tile) (fixed slots, no atomics); optional mean/rstd
// outputs.  rowmin_bcast then folds the partials in a fixed order and writes
// out[n][c] = min + bias2[c].  GEMM_GN_ROWMIN_ONE does that last step inside
// the same launch, whose grid fits what the device keeps resident at once
// (an ordinary launch, or a cooperative one on request): each workgroup publishes its partials, waits until the other c-tiles of its
// rows have published theirs, folds them (min is exact, so any order gives the
// same bits) and writes its own 256 x 128 block of the broadcast output.
#include "common.hpp"
#include "grid_sync.hpp"
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
constexpr int RB = KC * 2;     // bytes of one staged row (128: no padding)
constexpr int ROWS = BM + BN;  // staged rows per chunk (A rows, then B rows)
constexpr int PIECES = ROWS / 8;                 // 1 KB copies (8 rows) per chunk
constexpr int PPW = PIECES / NWAVE;              // copies per wave per chunk
constexpr int PPW_A = BM / 8 / NWAVE;            // of which A rows
constexpr int STAGE_B = ROWS * RB;               // bytes per LDS stage
static_assert(PIECES % NWAVE == 0 && (BM / 8) % NWAVE == 0, "whole copies per wave");
static_assert(KC / 32 == KSPLIT, "one K-step per wave per chunk");
constexpr int WMT = BM / (16 * WGC), WNT = BN / (16 * WGNN);  // 8 x 4 MFMA tiles per wave
// the epilogue's K-half exchange puts three waves' outgoing halves in a stage
static_assert(3 * (WMT / 2) * WNT * 64 * 16 <= STAGE_B, "three outgoing halves fit a stage");

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef uint16_t u16;

__device__ __forceinline__ void dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_wave_base, 16, 0, 0);
}

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their
// maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// vmcnt <= N and every LDS access of this wave complete (lgkmcnt 0), written
// as a compiler builtin so the compiler knows those reads have landed
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// Workgroup barrier without the waits of __syncthreads() (which would also
// wait for every outstanding global access, including the copies of the
// chunks still in flight): the caller waits first for what the barrier must
// cover (wait_vm_lds); the memory clobber keeps the compiler from moving any
// memory access across the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int EPI>
__global__ __launch_bounds__(NTHR) void gemm_bf16_kernel(GemmArgs a) {
  // three stages, each [A rows (256) | B rows (128)] x 128 bytes; the 16-byte
  // column q of row r sits at column q ^ (r & 6)
  __shared__ __attribute__((aligned(1024))) char S0[STAGE_B];
  __shared__ __attribute__((aligned(1024))) char S1[STAGE_B];
  __shared__ __attribute__((aligned(1024))) char S2[STAGE_B];

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

  const char* const wbytes = (const char*)a.w;
  const char* const xbytes = (const char*)a.x;

  f32x4 acc[WMT][WNT];
#pragma unroll
  for (int i = 0; i < WMT; ++i)
#pragma unroll
    for (int j = 0; j < WNT; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // operand reads: row arow + 16 i (A) or brow + 16 j (B), logical 16-byte
  // column 4 kh + kq; every such row has (row & 6) == (lr & 6)
  const int arow = wc * WMT * 16 + lr, brow = wnn * WNT * 16 + lr;
  const int pcol = ((4 * kh + kq) ^ (lr & 6)) * 16;
  // operand sets: the next chunk's operands are read into one while the
  // MFMAs consume the other
  struct Ops {
    bf16x8 a[WMT], b[WNT];
  };
  auto read_ops = [&](const char* st, Ops& o) __attribute__((always_inline)) {
    const char* as = st + arow * RB + pcol;
    const char* bs = st + BM * RB + brow * RB + pcol;
#pragma unroll
    for (int j = 0; j < WNT; ++j) o.b[j] = *(const bf16x8*)(bs + 16 * j * RB);
#pragma unroll
    for (int i = 0; i < WMT; ++i) o.a[i] = *(const bf16x8*)(as + 16 * i * RB);
  };
  auto mfma_ops = [&](const Ops& o) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < WMT; ++i)
#pragma unroll
      for (int j = 0; j < WNT; ++j) acc[i][j] = mfma16x16x32bf16(o.a[i], o.b[j], acc[i][j]);
  };
  auto compute = [&](const char* st) __attribute__((always_inline)) {
    Ops o;
    read_ops(st, o);
    mfma_ops(o);
  };

  // Staging by direct global -> LDS copies (no registers): copy k of a wave
  // moves 8 staged rows (P = wave + NWAVE k; A rows first, then B rows); lane
  // l fetches row 8 P + l/8 at logical column (l % 8) ^ (row & 6), which the
  // copy drops at physical column l % 8.  Rows past the matrix read its last
  // row (their products land in outputs that are never stored).  Offsets are
  // 32-bit (rows * C_in < 2^31 elements on this route).
  uint32_t doff[PPW];
#pragma unroll
  for (int k = 0; k < PPW; ++k) {
    const int P = wave + NWAVE * k;
    const bool b = k >= PPW_A;
    const int r = 8 * (b ? P - BM / 8 : P) + (lane >> 3);
    int64_t gr = (b ? n0 : c0) + r;
    const int64_t R = b ? a.N : a.C_out;
    if (gr > R - 1) gr = R - 1;
    const int q = (lane & 7) ^ ((lane >> 3) & 6);
    doff[k] = (uint32_t)((gr * a.C_in + 8 * q) * 2);
  }
  auto dma = [&](int chunk, char* st) __attribute__((always_inline)) {
    const uint32_t kb = (uint32_t)chunk * RB;
#pragma unroll
    for (int k = 0; k < PPW; ++k)
      dma16((k >= PPW_A ? xbytes : wbytes) + (kb + doff[k]), st + (wave + NWAVE * k) * 1024);
  };
  // Chunk c: wait for this wave's copies of chunk c (chunk c+1 may stay in
  // flight); barrier (everyone's copies of c landed; every wave's operand
  // reads of chunk c-1 completed, so its stage is free); start the copies of
  // chunk c+2 into that stage; then the MFMAs of chunk c-1 with chunk c's
  // operands read in behind them: chunk c's B fragments into a second set
  // first, then each A fragment of chunk c into the register of chunk c-1's
  // A fragment i as soon as its row of MFMAs has issued.  Issue order: the B
  // reads, then per A row 4 MFMAs and one A read, with one copy after each
  // of the first six rows.
  auto step = [&](const char* rd, char* wr, int next, Ops& o, Ops& nb)
      __attribute__((always_inline)) {
    wait_vm_lds<PPW>();
    lds_barrier();
    dma(next, wr);
    const char* as = rd + arow * RB + pcol;
    const char* bs = rd + BM * RB + brow * RB + pcol;
#pragma unroll
    for (int j = 0; j < WNT; ++j) nb.b[j] = *(const bf16x8*)(bs + 16 * j * RB);
#pragma unroll
    for (int i = 0; i < WMT; ++i) {
#pragma unroll
      for (int j = 0; j < WNT; ++j) acc[i][j] = mfma16x16x32bf16(o.a[i], o.b[j], acc[i][j]);
      o.a[i] = *(const bf16x8*)(as + 16 * i * RB);
    }
#pragma unroll
    for (int j = 0; j < WNT; ++j) o.b[j] = nb.b[j];
    __builtin_amdgcn_sched_group_barrier(0x100, WNT, 0);         // DS reads (B)
#pragma unroll
    for (int i = 0; i < WMT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, WNT, 0);       // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);         // DS read (A)
      if (i < PPW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
    }
  };

  // Chunk c sits in stage c % 3, so the main loop takes three chunks per
  // iteration.  Copies run unconditionally on chunk indices clamped to the
  // last whole chunk (surplus copies land in stages nobody reads again), so
  // the loop body is one block with one back edge.
  const int n_full = (int)(a.C_in / KC);
  if (n_full > 0) {
    const int last = n_full - 1;
    auto cl = [&](int c) { return c < last ? c : last; };
    Ops o, nb;
    dma(0, S0);
    dma(cl(1), S1);
    wait_vm_lds<PPW>();
    lds_barrier();
    dma(cl(2), S2);
    read_ops(S0, o);
    int c = 1;
    for (; c + 2 < n_full; c += 3) {
      step(S1, S0, cl(c + 2), o, nb);
      step(S2, S1, cl(c + 3), o, nb);
      step(S0, S2, cl(c + 4), o, nb);
    }
    // up to two chunks left (c % 3 == 1 here)
    if (c < n_full) step(S1, S0, cl(c + 2), o, nb);
    if (c + 1 < n_full) step(S2, S1, cl(c + 3), o, nb);
    mfma_ops(o);  // the last chunk
    wait_vmcnt<0>();  // surplus copies
    __syncthreads();
  }
  // Reduction tail (C_in % 64 != 0; C_in % 8 == 0, so a 16-byte piece lies
  // wholly inside or wholly past C_in), staged through registers: pieces past
  // C_in load column 0 of their row (in bounds) and are written as zeros.
  // Every stage is free here.
  if (a.C_in % KC != 0) {
    const int64_t k0 = (int64_t)n_full * KC;
#pragma unroll
    for (int k = 0; k < PPW; ++k) {
      const int q = (lane & 7) ^ ((lane >> 3) & 6);
      const bool inside = k0 + 8 * q < a.C_in;
      const int64_t kb = inside ? k0 * 2 : -(int64_t)(8 * q) * 2;
      const u32x4 v = *(const u32x4*)((k >= PPW_A ? xbytes : wbytes) + kb + doff[k]);
      *(u32x4*)(S0 + (wave + NWAVE * k) * 1024 + lane * 16) = inside ? v : (u32x4){0u, 0u, 0u, 0u};
    }
    __syncthreads();
    compute(S0);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  // The two waves of a spatial slot (kh = 0, 1) each hold half of the K-sum of
  // every tile.  They swap halves through LDS so that each ends with complete
  // sums of half the tile rows: kh = 0 keeps rows i < WMT/2, kh = 1 the rest.
  // (Both orders of the one addition give the same bits.)  Both waves then run
  // the epilogue on their rows.
  constexpr int HALF = WMT / 2;
  const int row0 = kh * HALF;  // first tile row this wave finishes
  // per-channel parameters of this wave's rows (channels c = cg + 4 kq + r),
  // loaded here so that one memory latency, overlapped with the exchange,
  // covers them
  f32x4 gam[HALF], bet[HALF], bis[HALF];
  {
    const bool vec = ((((uintptr_t)a.gamma) | ((uintptr_t)a.beta) | ((uintptr_t)a.bias)) & 15) == 0;
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
      const int64_t cg = c0 + wc * WMT * 16 + 16 * (row0 + i);
      const int64_t c = cg + 4 * kq;
      gam[i] = (f32x4){1.f, 1.f, 1.f, 1.f};
      bet[i] = bis[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (EPI != GEMM_STORE) {
        // whole groups of 16: a group either lies inside C_out or past it
        const int64_t cc = cg < a.C_out ? c : 4 * kq;
        if (vec) {
          if (a.gamma) gam[i] = *(const f32x4*)(a.gamma + cc);
          if (a.beta) bet[i] = *(const f32x4*)(a.beta + cc);
          if (a.bias) bis[i] = *(const f32x4*)(a.bias + cc);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (a.gamma) gam[i][r] = a.gamma[cc + r];
            if (a.beta) bet[i][r] = a.beta[cc + r];
            if (a.bias) bis[i][r] = a.bias[cc + r];
          }
        }
      } else if (a.bias) {
#pragma unroll
        for (int r = 0; r < 4; ++r) bis[i][r] = (c + r < a.C_out) ? a.bias[c + r] : 0.f;
      }
    }
  }
  {
    // wave w's outgoing half: 16 KB at slot w of the three stages (3 + 3 + 2)
    auto region = [&](int w) {
      char* st = w < 3 ? S0 : (w < 6 ? S1 : S2);
      return (f32x4*)(st + (w % 3) * (HALF * WNT * 64 * 16));
    };
    f32x4* out_r = region(wave);
    const f32x4* in_r = region(wave ^ 4);  // the other kh of the same slot
    auto send = [&](const f32x4 (&t)[WNT], int i) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < WNT; ++j) out_r[(i * WNT + j) * 64 + lane] = t[j];
    };
    auto recv = [&](f32x4 (&t)[WNT], int i) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < WNT; ++j) t[j] += in_r[(i * WNT + j) * 64 + lane];
    };
    if (kh == 0) {
#pragma unroll
      for (int i = 0; i < HALF; ++i) send(acc[HALF + i], i);
    } else {
#pragma unroll
      for (int i = 0; i < HALF; ++i) send(acc[i], i);
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int i = 0; i < HALF; ++i) recv(acc[i], i);
    } else {
#pragma unroll
      for (int i = 0; i < HALF; ++i) recv(acc[HALF + i], i);
    }
    __syncthreads();  // the stages are free again
  }

  if (EPI == GEMM_STORE) {
    // y (+ bias) as fp32, or rounded to bf16 (y_bf16)
    auto store_row = [&](auto* y, const f32x4 (&t)[WNT], int i) __attribute__((always_inline)) {
      const bool vec = (a.C_out % 4 == 0) && ((((uintptr_t)y) & (4 * sizeof(*y) - 1)) == 0);
      const int64_t c = c0 + wc * WMT * 16 + 16 * (row0 + i) + 4 * kq;
#pragma unroll
      for (int j = 0; j < WNT; ++j) {
        const int64_t nn = n0 + wnn * WNT * 16 + 16 * j + lr;
        if (nn >= a.N) continue;
        const f32x4 v = t[j] + bis[i];
        auto* dst = y + nn * a.C_out + c;
        if (vec && c + 3 < a.C_out) {
          store_elem4(dst, v);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (c + r < a.C_out) store_elem(dst + r, v[r]);
        }
      }
    };
    auto store = [&](auto* y) __attribute__((always_inline)) {
      if (kh == 0) {
#pragma unroll
        for (int i = 0; i < HALF; ++i) store_row(y, acc[i], i);
      } else {
#pragma unroll
        for (int i = 0; i < HALF; ++i) store_row(y, acc[HALF + i], i);
      }
    };
    if (a.y_bf16)
      store((uint16_t*)a.y);
    else
      store((float*)a.y);
  } else {  // GEMM_GN_ROWMIN: groups of 16 channels = one tile column block
    float* red = (float*)S0;
    float rmin[WNT];
#pragma unroll
    for (int j = 0; j < WNT; ++j) rmin[j] = __builtin_inff();
    // one row of group blocks: normalise each 16-channel group of each row n
    // (two-pass mean / variance over its 16 values), affine, min
    auto gn_row = [&](const f32x4 (&t)[WNT], int i) __attribute__((always_inline)) {
      const int64_t cg = c0 + wc * WMT * 16 + 16 * (row0 + i);  // first channel of the group
      const bool gvalid = cg < a.C_out;
      const f32x4 ga = gam[i], be = bet[i], bi = bis[i];
#pragma unroll
      for (int j = 0; j < WNT; ++j) {
        const f32x4 v = t[j] + bi;
        float s = (v[0] + v[1]) + (v[2] + v[3]);
        s = lane_sum<48>(s);
        const float mean = s * (1.0f / 16.0f);
        float q = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) { const float dv = v[r] - mean; q += dv * dv; }
        q = lane_sum<48>(q);
        const float rstd = __builtin_amdgcn_rsqf(q * (1.0f / 16.0f) + a.eps);
        float m = __builtin_inff();
#pragma unroll
        for (int r = 0; r < 4; ++r) m = min_nan(m, (v[r] - mean) * (rstd * ga[r]) + be[r]);
        if (gvalid) rmin[j] = min_nan(rmin[j], m);
        const int64_t nn = n0 + wnn * WNT * 16 + 16 * j + lr;
        if (gvalid && kq == 0 && nn < a.N) {
          const int64_t g = cg / 16;
          if (a.mean_out) a.mean_out[nn * a.G + g] = mean;
          if (a.rstd_out) a.rstd_out[nn * a.G + g] = rstd;
        }
      }
    };
    if (kh == 0) {
#pragma unroll
      for (int i = 0; i < HALF; ++i) gn_row(acc[i], i);
    } else {
#pragma unroll
      for (int i = 0; i < HALF; ++i) gn_row(acc[HALF + i], i);
    }
#pragma unroll
    for (int j = 0; j < WNT; ++j) {
      const float m = lane_min48(rmin[j]);
      if (kq == 0) red[(kh * WGC + wc) * BN + wnn * WNT * 16 + 16 * j + lr] = m;
    }
    __syncthreads();
    if (tid < BN) {
      const int64_t nn = n0 + tid;
      float m = red[tid];
#pragma unroll
      for (int w = 1; w < KSPLIT * WGC; ++w) m = min_nan(m, red[w * BN + tid]);
      if (nn < a.N) {
        float* p = a.part + nn * a.n_ctiles + ctile;
        if (EPI == GEMM_GN_ROWMIN_ONE)  // read by the other c-tiles' workgroups
          __hip_atomic_store((unsigned*)p, __float_as_uint(m), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        else
          *p = m;
      }
    }
    if constexpr (EPI == GEMM_GN_ROWMIN_ONE) {
      const bool ok = sample_barrier(a.sync + ntile, (unsigned)a.n_ctiles, a.fault, a.polls);
      // the rows' minima over all c-tiles (NaN if a wait gave up)
      float* rowm = red + KSPLIT * WGC * BN;
      if (tid < BN) {
        const int64_t nn = n0 + tid;
        float m = __builtin_inff();
        if (nn < a.N)
          for (int t = 0; t < a.n_ctiles; ++t)
            m = min_nan(m, __uint_as_float(__hip_atomic_load(
                             (const unsigned*)(a.part + nn * a.n_ctiles + t), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT)));
        rowm[tid] = ok ? m : __builtin_nanf("");
      }
      __syncthreads();
      // this tile's block of out[n][c] = min[n] + bias2[c]: a wave writes whole
      // 256-channel row segments, four channels per lane
      const int64_t c = c0 + 4 * lane;
      f32x4 b = {0.f, 0.f, 0.f, 0.f};
      const bool vec = (a.C_out % 4 == 0) &&
                       ((((uintptr_t)a.out) & (a.out_bf16 ? 7 : 15)) == 0) &&
                       ((((uintptr_t)a.bias2) & 15) == 0);
      if (a.bias2) {
        if (vec && c + 3 < a.C_out) {
          b = *(const f32x4*)(a.bias2 + c);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) b[r] = c + r < a.C_out ? a.bias2[c + r] : 0.f;
        }
      }
      auto bcast = [&](auto* out) __attribute__((always_inline)) {
        for (int r = wave; r < BN; r += NWAVE) {
          const int64_t nn = n0 + r;
          if (nn >= a.N) break;
          const f32x4 v = b + rowm[r];
          auto* dst = out + nn * a.C_out + c;
          if (vec && c + 3 < a.C_out) {
            store_elem4(dst, v);
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (c + q < a.C_out) store_elem(dst + q, v[q]);
          }
        }
      };
      if (a.out_bf16)
        bcast((uint16_t*)a.out);
      else
        bcast((float*)a.out);
    }
  }
}

// out[n][c] = min over c-tiles of part[n][*] + bias2[c]; one workgroup per row;
// TO is float, or bf16 bits (rounded to nearest even).  Each wave takes the
// row's minimum itself: one partial per lane, then a min across the lanes
// (not a chain of dependent loads per thread).  Streaming stores.
template <typename TO>
__global__ __launch_bounds__(NTHR) void rowmin_bcast_kernel(const float* __restrict__ part,
                                                            int n_ctiles,
                                                            const float* __restrict__ bias2,
                                                            TO* out, int64_t C) {
  const int64_t n = blockIdx.x;
  const int lane = threadIdx.x & 63;
  float m = __builtin_inff();
  for (int t = lane; t < n_ctiles; t += 64) m = min_nan(m, part[n * n_ctiles + t]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = min_nan(m, __shfl_xor(m, off));
  TO* row = out + n * C;
  if ((C % 4) == 0 && (((uintptr_t)out) & (4 * sizeof(TO) - 1)) == 0 &&
      (((uintptr_t)bias2) & 15) == 0) {
    for (int64_t q = threadIdx.x; q < C / 4; q += NTHR) {
      const f32x4 b = *(const f32x4*)(bias2 + 4 * q);
      store_elem4_nt(row + 4 * q, b + m);  // whole 1 KB runs, never read back here
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

int gemm_bf16_rowmin_capacity() {
  return resident_capacity((const void*)gemm_bf16_kernel<GEMM_GN_ROWMIN_ONE>, NTHR);
}

hipError_t gemm_bf16_rowmin_one_launch(GemmArgs a, bool cooperative, hipStream_t s) {
  const int64_t tiles = (int64_t)a.n_ctiles * a.n_ntiles;
  if (tiles < 1 || tiles > gemm_bf16_rowmin_capacity()) return hipErrorInvalidValue;
  // one arrival counter per row block, then the fault word
  const int64_t words = (int64_t)a.n_ntiles + 1;
  a.fault = a.sync + a.n_ntiles;
  a.polls = barrier_poll_limit();
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s,
                     a.sync, words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  void* args[] = {(void*)&a};
  return launch_coresident((const void*)gemm_bf16_kernel<GEMM_GN_ROWMIN_ONE>, (unsigned)tiles,
                           NTHR, args, cooperative, s);
}

int gemm_bf16_tile_c() { return BM; }
int gemm_bf16_tile_n() { return BN; }

}  // namespace c1g
