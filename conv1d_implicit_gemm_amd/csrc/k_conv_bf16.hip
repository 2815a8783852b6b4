// bf16 implicit-GEMM 1-D convolution for gfx950, fp32 accumulate: the
// convolution of the split route (y plus partial statistics) and, as a
// persistent kernel whose workgroups wait on each other, the whole conv +
// GroupNorm / channel LayerNorm of the fused_persistent route.
//
// GEMM view ("Kimi-K2.6 l1_p5", the implicit-GEMM shape M = N*T_out,
// N = C_out, K = C_in*K): row m = (n, t), column = output channel c; the
// reduction runs over (tap j, input channel ci) in chunks of 32 input channels,
// one v_mfma_f32_16x16x32_bf16 K-step per tap.  The MFMA wants 8 consecutive
// reduction values per lane, i.e. 8 consecutive input channels at one
// position, while x is stored position-contiguous.  So x is first repacked
// into a channels-last image in the workspace: per sample, rows of padded
// position tp = t + pad_left, each row the channels of one position padded to
// whole chunks, zero outside the tensor (the padding and the tail of the last
// tile are explicit zero rows).  A tile's input window is then a contiguous
// run of image rows, and both operands reach LDS by direct global -> LDS
// copies (global_load_lds, 16 bytes per lane, no registers).  Every tap reads
// the same window at a shifted row offset; the weights are repacked once per
// call into the exact LDS image of each (c-tile, chunk).
//
// LDS rows are 64 bytes (32 bf16) with no padding; the 16-byte column of a row
// is XOR-ed with 2 when bit 2 of the row index is set.  The LDS has 64
// four-byte banks and serves a 16-byte-per-lane read in four passes of 16
// lanes (lanes 0-7 with 16-23, and so on), so an operand read of rows r..r+7
// and two adjacent columns touches 16 distinct groups of 4 banks for any r
// (unit stride); without the XOR, rows r and r+4 would collide.  The copies
// write whole 1 KB runs, so a lane fetches the logical column that lands at
// its physical slot.
//
// Workgroup: 512 threads; tile TM (512, 256 or 128) positions x 128
// channels.  The eight waves form a 4 x 2 grid of wave tiles of WM x 4 MFMA
// tiles (128 x 64 for TM = 512, 64 x 64 for 256, 32 x 64 for 128), each
// running every tap, so a wave reads 12 KB of operands per 32 MFMAs at
// TM = 512 (8 KB per 16 at 256, 6 KB per 8 at 128).  The largest tile whose
// input window fits the LDS is used: the window of TM positions spans
// (TM - 1) * stride + (K - 1) * dilation + 1 input rows.  Two LDS stages, one barrier per chunk: the next chunk's copies
// run while the current chunk is consumed, issued in groups behind its first
// tap steps.  Within a chunk a wave reads each
// tap's fragments while the previous tap's MFMAs run (a fragment register is
// reloaded as soon as its last MFMA has issued), and across chunks the last
// tap's MFMAs run after the barrier while the next chunk's first tap is read.
// Epilogue: shared with the fp32 kernel (store y, GroupNorm or channel-
// LayerNorm partial statistics), or in the persistent kernel the sample-wide
// statistics and the normalised output (fused_norm_epilogue).
#include <type_traits>

#include "common.hpp"
#include "conv_epilogue.hpp"
#include "grid_sync.hpp"
#include "launch.hpp"

namespace c1g {
namespace {

constexpr int TN = ConvBf16Cfg::TN;  // 128 output channels per tile
constexpr int CK = ConvBf16Cfg::CK;  // 32 input channels per chunk
constexpr int RW = CK;               // LDS row: 32 bf16 (64 bytes)
constexpr int KMAX = 8;              // taps (512-position tiles: up to 5 per pass)
constexpr int WN = 4;                // MFMA tiles per wave along c
constexpr int WGN = 2;               // waves along c (TN = WGN * WN * 16)
constexpr int WGM = 4;               // waves along t
constexpr int NWAVE = WGM * WGN;
constexpr int NTHR = NWAVE * 64;
// LDS per workgroup: two stages of (window XR rows + weight image of the
// taps) of 64-byte rows.  XR = 544 rows with up to 5 taps (150 KB); on
// 256-position tiles 496 rows with 6 taps or 368 with 7 (158 KB each); on
// 128-position tiles 224 rows with 6 to 8 taps (156 KB); gfx950 allows 160 KB.
// A window of XR rows is 16-row copies (1 KB each).
constexpr int XCAP_WIDE = 544, XCAP_T6 = 496, XCAP_T7 = 368, XCAP_TAPS = 224;
static_assert(XCAP_WIDE % 16 == 0 && XCAP_T6 % 16 == 0 && XCAP_T7 % 16 == 0 &&
                  XCAP_TAPS % 16 == 0, "whole 16-row copies");
static_assert(2 * (XCAP_T6 + 6 * 128) * 64 <= 160 * 1024 - 2048 &&
                  2 * (XCAP_T7 + 7 * 128) * 64 <= 160 * 1024 - 2048,
              "two stages fit the LDS");
static_assert(TN == 128, "weight rows keep bit 2 of c across taps");

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef uint16_t u16;

// Direct global -> LDS copy of 16 bytes per lane: lane i reads base +
// lane_off and writes M0 + 16 i.  Issued as inline assembly so that the
// wave-uniform part of the address stays in scalar registers (one VGPR per
// copy however many are in flight) and the compiler adds no waits of its own
// before LDS reads: every read of a copied stage is ordered by the kernel's
// explicit wait_all_mem before the workgroup barrier.  The memory clobber
// keeps all memory accesses on their side of the copy.
__device__ __forceinline__ void dma16(const void* base, uint32_t lane_off, const void* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(lane_off), "s"(base), "s"(m0)
               : "memory", "m0");
}

// s_waitcnt vmcnt(0) lgkmcnt(0) as a compiler builtin (gfx9 encoding, expcnt
// left at its maximum), so the compiler knows every copy and LDS access of
// this wave has completed
__device__ __forceinline__ void wait_all_mem() { __builtin_amdgcn_s_waitcnt(7 << 4); }

// Workgroup barrier without the waits of __syncthreads() (which would also
// wait for the copies of the next chunk issued after it in program order):
// the caller waits first for what the barrier must cover; the memory clobber
// keeps the compiler from moving any memory access across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// 16-byte column swizzle of LDS row `row`
__host__ __device__ __forceinline__ int swz(int row) { return (row >> 1) & 2; }

// The kernel's arguments, read afresh from the argument segment: the pointer
// is made opaque, so the fields are loaded inside each round of the
// persistent loop instead of being hoisted out of it and held in scalar
// registers (spilled) across every round.  ConvArgs is the first argument.
__device__ __forceinline__ const ConvArgs& round_args() {
  typedef const __attribute__((address_space(4))) char* kptr;
  kptr p = (kptr)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return *(const ConvArgs*)p;
}

// Channels per GroupNorm partial of the persistent kernel: the largest power
// of two dividing the group width cpg, at most 64 (so it divides the
// 128-channel tile too)
__host__ __device__ __forceinline__ int gn_partial_width(int cpg) {
  const int low = cpg & -cpg;
  return low < 64 ? low : 64;
}

// Sum over aligned groups of w lanes (w a power of two up to 64, uniform)
__device__ __forceinline__ float group_lane_sum(float v, int w) {
  switch (w) {
    case 2: return lane_sum<1>(v);
    case 4: return lane_sum<3>(v);
    case 8: return lane_sum<7>(v);
    case 16: return lane_sum<15>(v);
    case 32: return lane_sum<31>(v);
    case 64: return lane_sum<63>(v);
    default: return v;
  }
}

// Persistent-kernel epilogue: bias and partial statistics, the sample
// barrier, the fixed-order merge of the sample's partials for this tile's
// groups (GroupNorm) or positions (LayerNorm over channels), then normalise +
// affine in registers and write the output once.  Every workgroup that needs
// a group's statistics merges the same partials in the same order.
//
// GroupNorm partials: one (mean, M2) per chunk of pg channels of a group per
// position tile, pg the largest power of two dividing C_out/G, at most 64 (so
// a chunk never straddles a group or a 128-channel tile), at
// part[((n * C_out/pg + chunk) *
// n_ttiles + ttile) * 2], so a group's partials are one contiguous run.  Every
// channel of a tile has the same count (the tile's valid positions), so the
// chunk's mean is the mean of its channel means and its M2 the sum of the
// channel M2s plus count * (channel mean - chunk mean)^2 (exact).
// LayerNorm partials: as on the split path, per position and channel tile.
//
// between(): issued after this workgroup has published its partials and
// counted itself in, before it waits for the others (the caller's prefetch of
// its next round's first chunk, into LDS the rest of the epilogue leaves
// alone: the window stage 0 and the weight stage 0, which held `red`).
template <int WM, int EPI, typename Between>
__device__ __forceinline__ void fused_norm_epilogue(const ConvArgs& a,
                                                    f32x4 (&acc)[WM][WN], int64_t n,
                                                    int64_t t0, int c0, int ttile, int ctile,
                                                    int wm, int wn, int round, int slot,
                                                    int tps, Stats* red, float* lds,
                                                    Between between) {
  constexpr int TM = WGM * WM * 16;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int lr = lane & 15, kq = lane >> 4;
  const int64_t T_out = a.T_out;
  constexpr bool gn = EPI == EPI_GN_FUSED;
  const int cpg = gn ? (int)(a.C_out / a.G) : 0;
  const int pg = gn_partial_width(cpg);  // channels per GroupNorm partial
  if constexpr (gn) {
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
    gn_wave_channel_stats<WM, WN, WGM, WGN>(a, acc, t0, wm, wn, red, true);
    __syncthreads();
    if (tid < TN) {  // two whole waves: every lane takes part in the lane sums
      const int c = c0 + tid;
      Stats st = red[tid];
#pragma unroll
      for (int w = 1; w < WGM; ++w) st = stats_merge(st, red[w * TN + tid]);
      const float mg = group_lane_sum(st.mean, pg) / (float)pg;
      const float dv = st.mean - mg;
      const float q = group_lane_sum(st.m2 + st.n * dv * dv, pg);
      if ((tid % pg) == 0 && c < a.C_out)
        store_partial(a.part + ((n * (a.C_out / pg) + c / pg) * a.n_ttiles + ttile) * 2, mg, q,
                      true);
    }
  } else {
    conv_epilogue<WM, WN, WGM, WGN>(a, EPI_LN_PART, acc, n, t0, c0, ttile, ctile, wm, wn, red,
                                    true, false);
  }
  // Wait only for the workgroups whose partials this tile's statistics need:
  // GroupNorm, the position tiles of its groups' channel tiles; LayerNorm,
  // the channel tiles of its position tile (fused_barrier_groups).  An
  // incomplete set of partials (a wait that gave up) yields NaN statistics,
  // hence a NaN output, never a plausible wrong one.
  int nsub, sub, expect;
  if constexpr (gn) {
    if (TN % cpg == 0 || cpg % TN == 0) {
      const int cpt = cpg > TN ? cpg / TN : 1;  // channel tiles per group
      nsub = a.n_ctiles / cpt;
      sub = ctile / cpt;
      expect = a.n_ttiles * cpt;
    } else {  // groups straddle channel tiles: the whole sample
      nsub = 1;
      sub = 0;
      expect = a.n_ttiles * a.n_ctiles;
    }
  } else {
    nsub = a.n_ttiles;
    sub = ttile;
    expect = a.n_ctiles;
  }
  (void)tps;
  unsigned* const ctr = a.sync + ((int64_t)round * a.spr + slot) * nsub + sub;
  barrier_arrive(ctr);
  between();
  const float poison =
      barrier_wait(ctr, (unsigned)expect, a.fault, a.polls) ? 0.f : __builtin_nanf("");

  float* mean_s = lds;        // merged statistics of this tile
  float* rstd_s = lds + 512;
  if constexpr (gn) {
    // ng groups meet this tile (the first, g0, may have begun in an earlier
    // channel tile and the last may go on in a later one), P partials per
    // group, S lanes of one wave per
    // group (a power of two): lane u folds partials u, u + S, ... in order,
    // then a fixed tree over the S lanes (lane u takes lane u + h)
    const int64_t cend = c0 + TN < a.C_out ? c0 + TN : a.C_out;
    const int g0 = c0 / cpg;
    const int ng = (int)((cend - 1) / cpg) - g0 + 1;
    const int P = (cpg / pg) * a.n_ttiles;
    int S = 1;
    while (S < P && S < 64 && 2 * S * ng <= NTHR) S *= 2;
    const int k = tid / S, u = tid - k * S;
    const int64_t g = (int64_t)g0 + k;
    Stats st = {0.f, 0.f, 0.f};
    if (k < ng && g < a.G) {
      const float* base = a.part + ((n * (a.C_out / pg) + g * (cpg / pg)) * a.n_ttiles) * 2;
      for (int p = u; p < P; p += S) {
        const int tt = p % a.n_ttiles;
        const int64_t cntl = T_out - (int64_t)tt * TM;
        const float cnt = (float)pg * (float)(cntl < TM ? cntl : TM);
        const f32x2 v = load_partial_coherent(base + 2 * p);
        st = stats_merge(st, Stats{cnt, v[0], v[1]});
      }
    }
    for (int h = S / 2; h > 0; h >>= 1) {
      const Stats o = {__shfl_xor(st.n, h), __shfl_xor(st.mean, h), __shfl_xor(st.m2, h)};
      if (u < h) st = stats_merge(st, o);
    }
    if (u == 0 && k < ng) {
      const Stats r = st;
      const float mu = r.mean + poison, rs = 1.0f / sqrtf(r.m2 / r.n + a.eps) + poison;
      mean_s[k] = mu;
      rstd_s[k] = rs;
      if (ttile == 0 && g < a.G) {
        if (a.mean_out) a.mean_out[n * a.G + g] = mu;
        if (a.rstd_out) a.rstd_out[n * a.G + g] = rs;
      }
    }
  } else {
    // one position per thread: the channel tiles' partials at (n, t)
    for (int tl = tid; tl < TM; tl += NTHR) {
      const int64_t t = t0 + tl;
      float mu = 0.f, rs = 0.f;
      if (t < T_out) {
        // the channel tiles' partials of (n, t), eight loads in flight at a
        // time (one by one, each load's round trip to the point of coherence
        // was paid in sequence), merged in channel-tile order
        Stats st = {0.f, 0.f, 0.f};
        const float* pp = a.part + (n * a.n_ctiles * T_out + t) * 2;
        const int nct = a.n_ctiles;
        const int crem = (int)(a.C_out - (int64_t)(nct - 1) * TN);  // last tile's channels
        for (int ct0 = 0; ct0 < nct; ct0 += 8) {
          f32x2 v[8];
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (ct0 + k < nct) v[k] = load_partial_coherent(pp + (int64_t)(ct0 + k) * T_out * 2);
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (ct0 + k < nct)
              st = stats_merge(st, Stats{(float)(ct0 + k == nct - 1 ? crem : TN), v[k][0], v[k][1]});
        }
        mu = st.mean + poison;
        rs = 1.0f / sqrtf(st.m2 / st.n + a.eps) + poison;
        if (ctile == 0) {
          if (a.mean_out) a.mean_out[n * T_out + t] = mu;
          if (a.rstd_out) a.rstd_out[n * T_out + t] = rs;
        }
      }
      mean_s[tl] = mu;
      rstd_s[tl] = rs;
    }
  }
  __syncthreads();

  // normalise + affine in registers (channel c, position t of each lane)
  float ga[WN], be[WN];
#pragma unroll
  for (int jn = 0; jn < WN; ++jn) {
    const int c = c0 + wn * WN * 16 + jn * 16 + lr;
    ga[jn] = (a.gamma != nullptr && c < a.C_out) ? a.gamma[c] : 1.f;
    be[jn] = (a.beta != nullptr && c < a.C_out) ? a.beta[c] : 0.f;
  }
  if constexpr (gn) {
    const int cpg = (int)(a.C_out / a.G);
#pragma unroll
    for (int jn = 0; jn < WN; ++jn) {
      const int k = (c0 + wn * WN * 16 + jn * 16 + lr) / cpg - c0 / cpg;
      const float mu = mean_s[k], sc = rstd_s[k] * ga[jn], b = be[jn];
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][jn][r] = (acc[i][jn][r] - mu) * sc + b;
    }
  } else {
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tl = wm * WM * 16 + i * 16 + 4 * kq + r;
        const float mu = mean_s[tl], rs = rstd_s[tl];
#pragma unroll
        for (int jn = 0; jn < WN; ++jn)
          acc[i][jn][r] = (acc[i][jn][r] - mu) * (rs * ga[jn]) + be[jn];
      }
  }
  if (a.y_bf16)
    conv_store<uint16_t, WM, WN, WGM, WGN>(a, acc, n, t0, c0, wm, wn);
  else
    conv_store<float, WM, WN, WGM, WGN>(a, acc, n, t0, c0, wm, wn);
}

// FUSE: 0 (one tile per workgroup, epilogue epi), or EPI_GN_FUSED /
// EPI_LN_FUSED (persistent rounds of whole samples, normalised output).
// NP: passes over the chunks.  IL = 0: K = NP * KT consecutive taps per
// pass (NP = 2 for eight or six taps on 512-position tiles, whose window and
// weights for all taps do not fit).  IL = 1 (strided convolutions): pass p
// takes the taps p, p + s, p + 2s, ... (at most KT of them; strides 2 to 5)
// and its window
// gathers every s-th image row from row s*t0 + p*d, so that within a pass
// the output positions advance one window row each and the taps d rows: a
// stride-1 window of TM + (KT - 1)*d rows where the direct one would need
// (TM - 1)*s + (K - 1)*d + 1.  IL = 2: consecutive taps, the last pass with
// fewer (seven taps as four and three).  With IL != 0 a step's tap count
// follows its pass, and weight slots past a pass's last tap copy the last
// tap (their MFMAs are skipped).
template <int WM, int KT, int XR, int FUSE, int NP = 1, int IL = 0>
__global__ __launch_bounds__(NTHR) void conv_bf16_kernel(ConvArgs a_, int epi) {
  const ConvArgs& a = a_;
  // the weight stage also holds the epilogue's cross-wave merge (<= 12 KB)
  constexpr int WSK = KT < 2 ? 2 : KT;
  constexpr int TM = WGM * WM * 16;
  constexpr int XP = XR / 16;                         // window copies per chunk
  constexpr int NPIECE = XP + KT * 8;                 // window + weight copies
  constexpr int PPW = (NPIECE + NWAVE - 1) / NWAVE;   // copies per wave per chunk
  __shared__ __attribute__((aligned(16))) u16 Xs0[XR * RW];
  __shared__ __attribute__((aligned(16))) u16 Xs1[XR * RW];
  __shared__ __attribute__((aligned(16))) u16 Ws0[WSK * TN * RW];
  __shared__ __attribute__((aligned(16))) u16 Ws1[WSK * TN * RW];

  const int tid = threadIdx.x;
  // the wave index is uniform: in a scalar register, everything derived from
  // it (copy slots, wave-tile origin) stays scalar too
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WGM, wn = wave / WGM;
  const int lr = lane & 15, kq = lane >> 4;
  const int s = a.stride, d = a.dilation;
  const int sw = IL == 1 ? 1 : s;  // window rows per output position
  const int sg = IL == 1 ? s : 1;  // image rows per window row
  // 1-D grid, XCD-aware: workgroup ids round-robin over the 8 XCDs; XCD x
  // takes a contiguous range of tiles ordered (n, t-tile, c-tile) with the
  // c-tile fastest, so the channel tiles of one input window share an L2.
  // The persistent kernel (FUSE) runs rounds of spr whole samples.
  const int tps = a.n_ttiles * a.n_ctiles;  // tiles per sample
  const int total = FUSE != 0 ? (int)gridDim.x : tps * (int)a.N;
  int lin = blockIdx.x;
  if ((total & 7) == 0) lin = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  // (The persistent GroupNorm kernel orders the tiles of a sample with the
  // t-tile fastest instead, so that the position tiles of a channel tile,
  // which wait for each other, share an XCD.)
  const bool tfast = FUSE == EPI_GN_FUSED;
  const int ctile = tfast ? (lin / a.n_ttiles) % a.n_ctiles : lin % a.n_ctiles;
  const int ttile = tfast ? lin % a.n_ttiles : (lin / a.n_ctiles) % a.n_ttiles;
  const int slot = lin / tps;  // FUSE: sample slot within a round
  const int64_t t0_ = (int64_t)ttile * TM;
  const int c0_ = ctile * TN;
  const int rounds = FUSE != 0 ? a.rounds : 1;
  bool prefetched = false;  // this round's chunk 0 already issued
  for (int round = 0; round < rounds; ++round) {
  const ConvArgs& a = FUSE != 0 ? round_args() : a_;
  const int64_t n = FUSE != 0 ? (int64_t)round * a.spr + slot : (int64_t)slot;
  // the tile origin, opaque per round: nothing derived from it (masks,
  // offsets of the epilogue) is hoisted out of the round loop
  int64_t t0 = t0_;
  int c0 = c0_;
  if constexpr (FUSE != 0) asm volatile("" : "+s"(t0), "+s"(c0));
  if (n >= a.N) break;  // whole workgroup: the samples of later rounds are none

  // ---- copies of one chunk: pieces 0..XP-1 are 16-row runs of the window,
  // XP.. the weight image (KT*8 runs of 16 rows); piece = wave + NWAVE * p.
  // Every wave issues PPW copies per chunk (surplus slots repeat the last
  // piece, writing the same bytes again).
  const int64_t row_bytes = (int64_t)a.n_chunks * CK * 2;  // one image row
  const char* const xwin = (const char*)a.ximg + (n * a.T_img + t0 * s) * row_bytes;
  // NP passes over the chunks, pass p with taps p*KT .. p*KT + KT - 1: its
  // window starts p*KT*d rows further down the image and its weights are
  // those taps of each (c-tile, chunk) block
  static_assert(NP >= 1 && NP <= (IL == 1 ? 5 : 2), "passes");
  const int64_t wblk = IL ? (int64_t)a.K * (TN * RW * 2)        // bytes of a (c-tile, chunk)
                          : (int64_t)NP * KT * (TN * RW * 2);  // block of the weight image
  const char* const wimg = (const char*)a.wp + (int64_t)ctile * a.n_chunks * wblk;
  // A copy's source offset is a wave-uniform part (its piece) plus one of two
  // lane offsets: window row 16 * piece + lane / 4 at logical column
  // (lane % 4) ^ swz(row) (the column landing at slot lane % 4; swz of the
  // row depends only on the lane), or weight bytes 16 * lane.
  const uint32_t lane_x =
      (uint32_t)((lane >> 2) * sg * row_bytes + 16 * ((lane & 3) ^ swz(lane >> 2)));
  const uint32_t lane_w = (uint32_t)(16 * lane);
  // q: pass * n_chunks + chunk
  auto pass_of = [&](int q) __attribute__((always_inline)) {
    if constexpr (NP > 3) return q / a.n_chunks;
    return NP >= 3 && q >= 2 * a.n_chunks ? 2 : (NP >= 2 && q >= a.n_chunks ? 1 : 0);
  };
  auto copy_from = [&](const char* xw, int p, int q, u16* xs, u16* ws)
      __attribute__((always_inline)) {
    int piece = wave + NWAVE * p;
    if (piece >= NPIECE) piece = NPIECE - 1;
    const int pass = pass_of(q);
    const int chunk = q - pass * a.n_chunks;
    if (piece < XP) {
      dma16(xw + (int64_t)pass * (IL == 1 ? 1 : KT) * d * row_bytes + (int64_t)chunk * (CK * 2) +
                (int64_t)16 * piece * sg * row_bytes,
            lane_x, (char*)xs + piece * 1024);
    } else if constexpr (IL) {
      // weight slot k of the pass: tap pass + s*k (IL 1) or pass*KT + k (IL
      // 2); slots past the last tap, whose MFMAs are skipped, copy the last
      // tap: no read leaves the block
      const int k = (piece - XP) >> 3;
      int tap = IL == 1 ? pass + s * k : pass * KT + k;
      if (tap > a.K - 1) tap = a.K - 1;
      // uniform (chunk step, piece and kernel arguments): kept in a scalar
      // register, as the copy's base operand requires
      tap = __builtin_amdgcn_readfirstlane(tap);
      dma16(wimg + (int64_t)chunk * wblk + (int64_t)tap * (TN * RW * 2) +
                ((piece - XP) & 7) * 1024,
            lane_w, (char*)ws + (piece - XP) * 1024);
    } else {
      dma16(wimg + (int64_t)chunk * wblk + (int64_t)pass * (KT * TN * RW * 2) +
                (piece - XP) * 1024,
            lane_w, (char*)ws + (piece - XP) * 1024);
    }
  };
  auto copy = [&](int p, int chunk, u16* xs, u16* ws) __attribute__((always_inline)) {
    copy_from(xwin, p, chunk, xs, ws);
  };
  auto stage = [&](int chunk, u16* xs, u16* ws) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < PPW; ++p) copy(p, chunk, xs, ws);
  };
  // The copies of the next chunk are issued in NG groups, one after each of
  // the first NG tap steps of the current chunk, not all at once after the
  // barrier: the copy path takes ~64 bytes per clock per CU, so a wave that
  // issues all its copies at once stalls for ~1.2 K cycles, and with both
  // waves of a SIMD doing so right after the barrier the MFMA pipe idles.
  // The last tap step issues none, leaving it for the copies to land.
  constexpr int NG = IL ? 1 : (KT > 2 ? KT - 1 : 1);  // IL: a pass may have fewer taps
  auto stage_group = [&](int chunk, u16* xs, u16* ws, int g) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < PPW; ++p)
      if ((p * NG) / PPW == g) copy(p, chunk, xs, ws);
  };

  f32x4 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // Operand fragments of one tap: A = 16 output positions x 32 channels
  // (window rows (t - t0) * s + j * d), B = 32 channels x 16 output channels.
  const int arow0 = (wm * WM * 16 + lr) * sw;
  const int bcol = 8 * (kq ^ swz(lr));  // weight rows: bit 2 of c = bit 2 of lr
  bf16x8 av[WM], bv[WN];
  auto xa_of = [&](const u16* xs, int j) __attribute__((always_inline)) {
    const int r0 = arow0 + j * d;  // rows r0 + 16*s*i keep bit 2
    return xs + r0 * RW + 8 * (kq ^ swz(r0));
  };
  auto wb_of = [&](const u16* ws, int j) __attribute__((always_inline)) {
    return ws + (j * TN + wn * WN * 16 + lr) * RW + bcol;
  };
  auto read_tap = [&](const u16* xs, const u16* ws, int j) __attribute__((always_inline)) {
    const u16* xa = xa_of(xs, j);
    const u16* wb = wb_of(ws, j);
#pragma unroll
    for (int jn = 0; jn < WN; ++jn) bv[jn] = *(const bf16x8*)(wb + jn * 16 * RW);
#pragma unroll
    for (int i = 0; i < WM; ++i) av[i] = *(const bf16x8*)(xa + i * 16 * sw * RW);
  };
  // The MFMAs of the tap whose fragments are in av/bv, each fragment replaced
  // by its counterpart of tap j of (xs, ws) as soon as its last MFMA has
  // issued (A row by row, then B within the last row).
  auto mfma_reload = [&](const u16* xs, const u16* ws, int j) __attribute__((always_inline)) {
    const u16* xa = xa_of(xs, j);
    const u16* wb = wb_of(ws, j);
#pragma unroll
    for (int i = 0; i < WM - 1; ++i) {
#pragma unroll
      for (int jn = 0; jn < WN; ++jn) acc[i][jn] = mfma16x16x32bf16(av[i], bv[jn], acc[i][jn]);
      av[i] = *(const bf16x8*)(xa + i * 16 * sw * RW);
    }
#pragma unroll
    for (int jn = 0; jn < WN; ++jn) {
      acc[WM - 1][jn] = mfma16x16x32bf16(av[WM - 1], bv[jn], acc[WM - 1][jn]);
      bv[jn] = *(const bf16x8*)(wb + jn * 16 * RW);
    }
    av[WM - 1] = *(const bf16x8*)(xa + (WM - 1) * 16 * sw * RW);
#pragma unroll
    for (int i = 0; i < WM - 1; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, WN, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
    }
#pragma unroll
    for (int jn = 0; jn < WN; ++jn) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto mfma_only = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int jn = 0; jn < WN; ++jn) acc[i][jn] = mfma16x16x32bf16(av[i], bv[jn], acc[i][jn]);
  };
  // the MFMAs of taps 0..KT-2 of the chunk in (xs, ws) (tap 0's fragments
  // already loaded), reading taps 1..KT-1 behind them; a runtime loop keeps
  // one copy of the body
  int kt = KT;  // with two taps, opaque: the one-trip loop stays a loop (its
                // unrolled form spills in the persistent kernel)
  if constexpr (KT == 2) asm volatile("" : "+s"(kt));
  // ... and issue copy groups 1 .. NG-1 of chunk cc into (cxs, cws) behind
  // the first tap steps
  // 512-position tiles: the two waves of a SIMD (wave w and w + 4) take
  // turns at the higher issue priority, one tap each, so that they progress
  // together instead of oldest first (which leaves the younger wave running
  // alone, its LDS latency uncovered, while the older one waits at the chunk
  // barrier).  Measured faster on 512-position tiles only; the 128-position
  // tiles (short taps) run 2-5% slower with it and keep the default order.
  const int prio_par = (wave >> 2) & 1;
  auto set_prio = [&](int j) __attribute__((always_inline)) {
    if constexpr (WM >= 8) {
      if (((j + prio_par) & 1) != 0)
        __builtin_amdgcn_s_setprio(1);
      else
        __builtin_amdgcn_s_setprio(0);
    }
  };
  // taps of (pass, chunk) step q: KT, or with IL those of its pass
  auto kt_of = [&](int q) __attribute__((always_inline)) {
    if constexpr (IL == 1) return (a.K - pass_of(q) + s - 1) / s;
    if constexpr (IL == 2) {
      const int left = a.K - pass_of(q) * KT;
      return left < KT ? left : KT;
    }
    return kt;
  };
  auto taps = [&](const u16* xs, const u16* ws, int ktq, int cc, u16* cxs, u16* cws)
      __attribute__((always_inline)) {
#pragma nounroll
    for (int j = 1; j < ktq; ++j) {
      set_prio(j);
      mfma_reload(xs, ws, j);
      if (j < NG) stage_group(cc, cxs, cws, j);
    }
  };

  // Pairs of chunks per iteration.  Copies run unconditionally on chunk
  // indices clamped to the last chunk (surplus copies land in a stage nobody
  // reads again), so the loop body is one block.  Before each barrier every
  // wave waits for all its copies: those of the next chunk, issued one chunk
  // earlier.
  const int n_chunks = NP * a.n_chunks, last = n_chunks - 1;  // (pass, chunk) steps
  auto cl = [&](int c) { return c < last ? c : last; };
  // the persistent kernel's later rounds find chunk 0 already copied (issued
  // by the previous round while it waited at its barrier)
  if (!prefetched) stage(0, Xs0, Ws0);
  wait_all_mem();
  lds_barrier();
  read_tap(Xs0, Ws0, 0);
  stage_group(cl(1), Xs1, Ws1, 0);
  int c = 0;
  for (; c + 1 < n_chunks; c += 2) {
    // stage 0 holds chunk c, its tap 0 in the fragments; stage 1 is loading c+1
    taps(Xs0, Ws0, kt_of(c), cl(c + 1), Xs1, Ws1);
    wait_all_mem();
    lds_barrier();
    set_prio(0);
    mfma_reload(Xs1, Ws1, 0);  // chunk c's last tap; chunk c+1's tap 0
    stage_group(cl(c + 2), Xs0, Ws0, 0);
    // stage 1 holds chunk c+1; stage 0 is loading c+2
    taps(Xs1, Ws1, kt_of(c + 1), cl(c + 2), Xs0, Ws0);
    wait_all_mem();
    lds_barrier();
    set_prio(0);
    mfma_reload(Xs0, Ws0, 0);
    stage_group(cl(c + 3), Xs1, Ws1, 0);
  }
  if (c < n_chunks) {  // odd count: the last chunk is in stage 0
    taps(Xs0, Ws0, kt_of(c), cl(c + 1), Xs1, Ws1);
    mfma_only();
  }
  __builtin_amdgcn_s_setprio(0);
  wait_all_mem();  // surplus copies land before the epilogue reuses the LDS
  __syncthreads();

  if constexpr (FUSE == 0) {
    conv_epilogue<WM, WN, WGM, WGN>(a, epi, acc, n, t0, c0, ttile, ctile, wm, wn, (Stats*)Ws0);
  } else {
    // while this round waits at its barrier: the next round's chunk 0
    const int64_t n_next = n + a.spr;
    prefetched = n_next < a.N;
    fused_norm_epilogue<WM, FUSE>(a, acc, n, t0, c0, ttile, ctile, wm, wn, round, slot, tps,
                                  (Stats*)Ws0, (float*)Ws1, [&]() __attribute__((always_inline)) {
                                    if (n_next < a.N) {
                                      const char* xw = (const char*)a.ximg +
                                                       (n_next * a.T_img + t0 * s) * row_bytes;
#pragma unroll
                                      for (int p = 0; p < PPW; ++p) copy_from(xw, p, 0, Xs0, Ws0);
                                    }
                                  });
    __syncthreads();  // the LDS is reused by the next round
  }
  }  // rounds
}

// Weight image: one block of K*TN*RW bf16 per (ctile, chunk), laid out
// [j][c][32] with the input channels of the chunk in four 16-byte columns,
// column q of row c stored at column q ^ swz(c):
//   wp[(((ctile*n_chunks + chunk)*K + j)*TN + c)*RW + 8*(q ^ swz(c)) + e]
//     = w[ctile*TN + c][chunk*32 + 8*q + e][j]      (0 outside the tensor)
// A thread reads the 8 * K contiguous weights of 8 input channels of one
// output channel (every tap) once, as K 16-byte loads when C_in % 8 == 0 and
// w is 16-byte aligned (vec; element by element otherwise, and at the edges),
// and writes the K 16-byte pieces they form.
// Also zeroes `zero_words` words at `zero` (the persistent kernel's arrival
// counters and fault word), so they need no launch of their own.
template <int K>
__global__ void conv_bf16_pack_kernel(const u16* __restrict__ w, u16* __restrict__ wp,
                                      int64_t C_in, int64_t C_out, int n_chunks,
                                      int64_t total, unsigned* zero, int64_t zero_words,
                                      int vec) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx < zero_words) zero[idx] = 0u;
  if (idx >= total / (8 * K)) return;
  const int pq = (int)(idx % (RW / 8));
  int64_t rest = idx / (RW / 8);
  const int c = (int)(rest % TN);
  rest /= TN;
  const int chunk = (int)(rest % n_chunks);
  const int64_t ctile = rest / n_chunks;
  const int q = pq ^ swz(c);
  const int64_t co = ctile * TN + c;
  const int64_t ci0 = (int64_t)chunk * CK + 8 * q;
  // v[e * K + j]: input channel ci0 + e, tap j (w's own order within the run)
  u16 v[8 * K];
  if (vec && co < C_out && ci0 + 8 <= C_in) {
    const u32x4* src = (const u32x4*)(w + (co * C_in + ci0) * K);
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const u32x4 r = src[i];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[8 * i + 2 * k] = (u16)(r[k] & 0xffffu);
        v[8 * i + 2 * k + 1] = (u16)(r[k] >> 16);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int j = 0; j < K; ++j)
        v[e * K + j] =
            (co < C_out && ci0 + e < C_in) ? w[(co * C_in + ci0 + e) * K + j] : (u16)0;
  }
  u16* dst = wp + ((((ctile * n_chunks + chunk) * K) * TN + c) * RW + 8 * pq);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      o[k] = (uint32_t)v[2 * k * K + j] | ((uint32_t)v[(2 * k + 1) * K + j] << 16);
    *(u32x4*)(dst + (int64_t)j * TN * RW) = o;
  }
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

// Input image: ximg[n][tp][cp] = x[n][cp][tp - pad_left] for 0 <= tp - pad_left
// < T and cp < C_in, else 0; rows of cpad = n_chunks * 32 channels, T_img rows
// per sample.  A lane moves one 8 (channels) x 8 (positions) block: eight
// 16-byte loads along t, a register transpose, eight 16-byte stores along the
// channels.  Lane l of a wave takes channel group l % 8 and position group
// l / 8 of a 64 x 64 tile, so both the loads (8 lanes per channel row) and the
// stores (8 lanes per image row) come in 128-byte runs.  The tile's input
// positions start at a multiple of 64 (t0 = 64 * bx - A, A = pad_left rounded
// up to 64), so in-range blocks load with aligned 16-byte loads when T % 8 == 0
// and, when T % 64 == 0, each 128-byte run is one whole 128-byte line (a run
// straddling two lines would fetch both: twice the bytes of x).
__global__ __launch_bounds__(256) void conv_bf16_pack_x_kernel(const u16* __restrict__ x,
                                                              u16* __restrict__ ximg,
                                                              int64_t C_in, int64_t T,
                                                              int64_t cpad, int64_t T_img,
                                                              int pad_left, int64_t A,
                                                              int fast) {
  const int64_t n = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t ci0 = (int64_t)blockIdx.y * 256 + 64 * wave + 8 * (lane & 7);
  const int64_t tb = (int64_t)blockIdx.x * 64 - A + 8 * (lane >> 3);
  if (ci0 >= cpad) return;
  u32x4 in[8], out[8];
  const bool vec = fast && tb >= 0 && tb + 8 <= T;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int64_t ci = ci0 + r;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (ci < C_in) {
      const u16* src = x + (n * C_in + ci) * T;
      if (vec) {
        // x is read once here: streaming loads keep it from evicting the
        // image (which the conv reads next) from the caches
        v = __builtin_nontemporal_load((const u32x4*)(src + tb));
      } else {
        u16 e8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) e8[e] = (tb + e >= 0 && tb + e < T) ? src[tb + e] : (u16)0;
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = (uint32_t)e8[2 * k] | ((uint32_t)e8[2 * k + 1] << 16);
      }
    }
    in[r] = v;
  }
  transpose8x8(in, out);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int64_t tp = tb + e + pad_left;
    if (tp >= 0 && tp < T_img) *(u32x4*)(ximg + (n * T_img + tp) * cpad + ci0) = out[e];
  }
}

// The same image from a channels-last x [N, T, C_in]: every in-range image
// row is one input row padded with zeros to cpad channels, the others are
// zero.  A thread writes 8 channels (16 bytes) of a row, so consecutive lanes
// read and write consecutive 16-byte pieces of the same rows.  vec: C_in % 8
// == 0 and x 16-byte aligned (every piece is one aligned load).
__global__ __launch_bounds__(256) void conv_bf16_pack_x_nlc_kernel(const u16* __restrict__ x,
                                                                  u16* __restrict__ ximg,
                                                                  int64_t C_in, int64_t T,
                                                                  int64_t cpad, int64_t T_img,
                                                                  int pad_left, int64_t total,
                                                                  int vec) {
  const int64_t per_row = cpad / 8;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = idx / per_row;  // n * T_img + tp
    const int64_t c = 8 * (idx - row * per_row);
    const int64_t n = row / T_img, t = row - n * T_img - pad_left;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (t >= 0 && t < T && c < C_in) {
      const u16* src = x + (n * T + t) * C_in + c;
      if (vec) {
        v = __builtin_nontemporal_load((const u32x4*)src);  // read once
      } else {
        u16 e8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) e8[e] = c + e < C_in ? src[e] : (u16)0;
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = (uint32_t)e8[2 * k] | ((uint32_t)e8[2 * k + 1] << 16);
      }
    }
    *(u32x4*)(ximg + row * cpad + c) = v;
  }
}

template <int WM, int KT, int XR, int NP = 1, int IL = 0>
hipError_t launch_wk(const ConvArgs& a, int epi, hipStream_t st, bool coop = false) {
  if (epi == EPI_GN_FUSED || epi == EPI_LN_FUSED) {
    // one round: spr whole samples, every workgroup resident at once
    ConvArgs ac = a;
    int ep = epi;
    void* args[] = {(void*)&ac, (void*)&ep};
    const void* k = epi == EPI_GN_FUSED
                        ? (const void*)conv_bf16_kernel<WM, KT, XR, EPI_GN_FUSED, NP, IL>
                        : (const void*)conv_bf16_kernel<WM, KT, XR, EPI_LN_FUSED, NP, IL>;
    return launch_coresident(k, (unsigned)(a.spr * a.n_ttiles * a.n_ctiles), NTHR, args, coop,
                             st);
  }
  dim3 grid((unsigned)(a.n_ttiles * a.n_ctiles * a.N));
  hipLaunchKernelGGL((conv_bf16_kernel<WM, KT, XR, 0, NP, IL>), grid, dim3(NTHR), 0, st, a,
                     epi);
  return hipGetLastError();
}

// How the bf16 conv runs (stride s, K taps, dilation d): tiles of tm
// positions, np passes over the chunks of at most kt taps each, interleaved
// (il, strided convolutions) or of consecutive taps, xr window rows.  The
// first that fits: 512 positions with all taps in one pass; 512 with eight,
// six or seven taps in two passes; 512 with a stride of 2 to 5 in
// interleaved passes; 256; 128.  tm == 0: not built.
struct Geo {
  int tm, kt, np, il, xr;
};
Geo geo_of(int s, int K, int d) {
  if (K < 1 || K > KMAX || s < 1 || d < 1) return Geo{0, 0, 0, 0, 0};
  auto fits = [&](int tm, int kt, int rows_per_pos, int xr) {
    return (int64_t)(tm - 1) * rows_per_pos + (int64_t)(kt - 1) * d + 1 <= xr;
  };
  if (K <= 5 && fits(512, K, s, XCAP_WIDE)) return Geo{512, K, 1, 0, XCAP_WIDE};
  if ((K == 8 || K == 6) && fits(512, K / 2, s, XCAP_WIDE))
    return Geo{512, K / 2, 2, 0, XCAP_WIDE};
  if (K == 7 && fits(512, 4, s, XCAP_WIDE)) return Geo{512, 4, 2, 2, XCAP_WIDE};  // 4 + 3
  if (s >= 2 && s <= 5) {
    const int kt = (K + s - 1) / s, np = K < s ? K : s;
    if (kt <= 4 && fits(512, kt, 1, XCAP_WIDE)) return Geo{512, kt, np, 1, XCAP_WIDE};
  }
  const int cap256 = K <= 5 ? XCAP_WIDE : K == 6 ? XCAP_T6 : K == 7 ? XCAP_T7 : 0;
  if (cap256 > 0 && fits(256, K, s, cap256)) return Geo{256, K, 1, 0, cap256};
  const int cap128 = K <= 5 ? XCAP_WIDE : XCAP_TAPS;
  if (fits(128, K, s, cap128)) return Geo{128, K, 1, 0, cap128};
  return Geo{0, 0, 0, 0, 0};
}

// the interleaved instances of 512-position tiles: (kt, np) of strides 2 to 5
// (kt = ceil(K / s) taps per pass, np = min(s, K) passes)
template <typename F>
hipError_t il_dispatch(const Geo& g, F&& f) {
  using std::integral_constant;
#define C1G_IL(KT_, NP_) \
  case KT_ * 8 + NP_: return f(integral_constant<int, KT_>{}, integral_constant<int, NP_>{});
  switch (g.kt * 8 + g.np) {
    C1G_IL(1, 1) C1G_IL(1, 2) C1G_IL(1, 3) C1G_IL(1, 4) C1G_IL(1, 5)
    C1G_IL(2, 2) C1G_IL(2, 3) C1G_IL(2, 4) C1G_IL(2, 5)
    C1G_IL(3, 2) C1G_IL(3, 3)
    C1G_IL(4, 2)
    default: return hipErrorInvalidValue;
  }
#undef C1G_IL
}

template <int WM>
hipError_t launch_w(const ConvArgs& a, int epi, hipStream_t st, bool coop = false) {
  if constexpr (WM == 8) {
    const Geo g = geo_of(a.stride, a.K, a.dilation);
    if (g.il == 2) return launch_wk<8, 4, XCAP_WIDE, 2, 2>(a, epi, st, coop);
    if (g.il)
      return il_dispatch(g, [&](auto kt, auto np) {
        return launch_wk<8, decltype(kt)::value, XCAP_WIDE, decltype(np)::value, 1>(a, epi, st,
                                                                                    coop);
      });
  }
  switch (a.K) {
    case 1: return launch_wk<WM, 1, XCAP_WIDE>(a, epi, st, coop);
    case 2: return launch_wk<WM, 2, XCAP_WIDE>(a, epi, st, coop);
    case 3: return launch_wk<WM, 3, XCAP_WIDE>(a, epi, st, coop);
    case 4: return launch_wk<WM, 4, XCAP_WIDE>(a, epi, st, coop);
    case 5: return launch_wk<WM, 5, XCAP_WIDE>(a, epi, st, coop);
    default: break;
  }
  if (WM == 8) {  // eight or six taps: two passes of four or three
    if (a.K == 8) return launch_wk<8, 4, XCAP_WIDE, 2>(a, epi, st, coop);
    if (a.K == 6) return launch_wk<8, 3, XCAP_WIDE, 2>(a, epi, st, coop);
    return hipErrorInvalidValue;
  }
  if (WM == 4) {
    switch (a.K) {
      case 6: return launch_wk<4, 6, XCAP_T6>(a, epi, st, coop);
      case 7: return launch_wk<4, 7, XCAP_T7>(a, epi, st, coop);
      default: return hipErrorInvalidValue;
    }
  }
  if (WM != 2) return hipErrorInvalidValue;
  switch (a.K) {
    case 6: return launch_wk<2, 6, XCAP_TAPS>(a, epi, st, coop);
    case 7: return launch_wk<2, 7, XCAP_TAPS>(a, epi, st, coop);
    case 8: return launch_wk<2, 8, XCAP_TAPS>(a, epi, st, coop);
    default: return hipErrorInvalidValue;
  }
}


}  // namespace

int conv_bf16_tile_m(int stride, int K, int dilation) { return geo_of(stride, K, dilation).tm; }

int conv_bf16_passes(int stride, int K, int dilation, int* interleaved) {
  const Geo g = geo_of(stride, K, dilation);
  if (interleaved) *interleaved = g.il == 1;
  return g.np;
}

int64_t conv_bf16_image_rows(int64_t T_out, int stride, int K, int dilation) {
  const int tm = conv_bf16_tile_m(stride, K, dilation);
  if (tm == 0) return 0;
  const Geo g = geo_of(stride, K, dilation);
  const int64_t n_tt = (T_out + tm - 1) / tm;
  const int64_t first = (n_tt - 1) * tm * stride;  // the last tile's first input row
  // its last pass copies xr rows from (np - 1) * kt * dilation rows further,
  // or (interleaved) every stride-th row from (np - 1) * dilation further
  if (g.il == 1)
    return first + (int64_t)(g.np - 1) * dilation + (int64_t)stride * (g.xr - 1) + 1;
  return first + (int64_t)(g.np - 1) * g.kt * dilation + g.xr;
}

size_t conv_bf16_image_bytes(int64_t N, int64_t C_in, int64_t T_img) {
  const int64_t cpad = (C_in + CK - 1) / CK * CK;
  return (size_t)(N * T_img * cpad) * sizeof(u16);
}

size_t conv_bf16_packed_bytes(int64_t C_in, int64_t C_out, int K) {
  const int64_t n_chunks = (C_in + CK - 1) / CK, n_ctiles = (C_out + TN - 1) / TN;
  return (size_t)(n_ctiles * n_chunks * K * TN * RW) * sizeof(u16);
}

hipError_t conv_bf16_pack(const uint16_t* w, uint16_t* wp, int64_t C_in, int64_t C_out, int K,
                          hipStream_t s, unsigned* zero, int64_t zero_words) {
  const int n_chunks = (int)((C_in + CK - 1) / CK);
  const int64_t total = (int64_t)(conv_bf16_packed_bytes(C_in, C_out, K) / sizeof(u16));
  int64_t threads = total / (8 * K);
  if (threads < zero_words) threads = zero_words;
  const int64_t blocks = (threads + 255) / 256;
  const int vec = (C_in % 8 == 0) && ((((uintptr_t)w) & 15) == 0);
#define C1G_PACK_K(KK)                                                                        \
  case KK:                                                                                    \
    hipLaunchKernelGGL(conv_bf16_pack_kernel<KK>, dim3((unsigned)blocks), dim3(256), 0, s, w, \
                       wp, C_in, C_out, n_chunks, total, zero, zero_words, vec);              \
    break;
  switch (K) {
    C1G_PACK_K(1) C1G_PACK_K(2) C1G_PACK_K(3) C1G_PACK_K(4)
    C1G_PACK_K(5) C1G_PACK_K(6) C1G_PACK_K(7) C1G_PACK_K(8)
    default: return hipErrorInvalidValue;
  }
#undef C1G_PACK_K
  return hipGetLastError();
}

hipError_t conv_bf16_pack_x(const uint16_t* x, uint16_t* ximg, int64_t N, int64_t C_in,
                            int64_t T, int pad_left, int64_t T_img, bool nlc, hipStream_t s) {
  const int64_t cpad = (C_in + CK - 1) / CK * CK;
  if (nlc) {
    const int64_t total = N * T_img * (cpad / 8);
    const int64_t blocks = (total + 255) / 256;
    const int vec = (C_in % 8 == 0) && ((((uintptr_t)x) & 15) == 0);
    hipLaunchKernelGGL(conv_bf16_pack_x_nlc_kernel,
                       dim3((unsigned)(blocks < 1048576 ? blocks : 1048576)), dim3(256), 0, s, x,
                       ximg, C_in, T, cpad, T_img, pad_left, total, vec);
    return hipGetLastError();
  }
  // first input position of tile 0: -A, a multiple of 64 positions, so each
  // lane group's 128-byte run of a channel row is one whole 128-byte line
  const int64_t A = (pad_left + 63) / 64 * 64;
  const int fast = (T % 8 == 0) && ((((uintptr_t)x) & 15) == 0);
  // tiles of 64 positions cover input positions -A .. T_img - 1 - pad_left
  dim3 grid((unsigned)((T_img - pad_left + A + 63) / 64), (unsigned)((cpad + 255) / 256),
            (unsigned)N);
  hipLaunchKernelGGL(conv_bf16_pack_x_kernel, grid, dim3(256), 0, s, x, ximg, C_in, T, cpad,
                     T_img, pad_left, A, fast);
  return hipGetLastError();
}

hipError_t conv_bf16_launch(const ConvArgs& a, int epi, hipStream_t s) {
  const int tm = conv_bf16_tile_m(a.stride, a.K, a.dilation);
  if (tm == 512) return launch_w<8>(a, epi, s);  // wave tiles 128 x 64
  if (tm == 256) return launch_w<4>(a, epi, s);  // wave tiles 64 x 64
  if (tm == 128) return launch_w<2>(a, epi, s);  // wave tiles 32 x 64
  return hipErrorInvalidValue;
}

namespace {
// the GroupNorm and LayerNorm instances share their resources (same LDS,
// launch bounds), so either stands for both
template <int WM, int KT, int XR, int NP = 1, int IL = 0>
int capacity_wk() {
  return resident_capacity((const void*)conv_bf16_kernel<WM, KT, XR, EPI_GN_FUSED, NP, IL>,
                           NTHR);
}
template <int WM>
int capacity_w(int K) {
  switch (K) {
    case 1: return capacity_wk<WM, 1, XCAP_WIDE>();
    case 2: return capacity_wk<WM, 2, XCAP_WIDE>();
    case 3: return capacity_wk<WM, 3, XCAP_WIDE>();
    case 4: return capacity_wk<WM, 4, XCAP_WIDE>();
    case 5: return capacity_wk<WM, 5, XCAP_WIDE>();
    default: break;
  }
  if (WM == 8) {  // two passes
    if (K == 8) return capacity_wk<8, 4, XCAP_WIDE, 2>();
    if (K == 6) return capacity_wk<8, 3, XCAP_WIDE, 2>();
    return 0;
  }
  if (WM == 4) {
    switch (K) {
      case 6: return capacity_wk<4, 6, XCAP_T6>();
      case 7: return capacity_wk<4, 7, XCAP_T7>();
      default: return 0;
    }
  }
  if (WM != 2) return 0;
  switch (K) {
    case 6: return capacity_wk<2, 6, XCAP_TAPS>();
    case 7: return capacity_wk<2, 7, XCAP_TAPS>();
    case 8: return capacity_wk<2, 8, XCAP_TAPS>();
    default: return 0;
  }
}
}  // namespace

int fused_barrier_groups(int epi, int64_t C_out, int G, int n_ttiles, int n_ctiles) {
  if (epi == EPI_LN_FUSED) return n_ttiles;
  const int64_t cpg = C_out / G;
  if (TN % cpg != 0 && cpg % TN != 0) return 1;  // groups straddle tiles: per sample
  const int64_t cpt = cpg > TN ? cpg / TN : 1;
  return (int)(n_ctiles / cpt);
}

int conv_bf16_fused_capacity(int stride, int K, int dilation) {
  const Geo g = geo_of(stride, K, dilation);
  const int tm = g.tm;
  if (tm == 512 && g.il == 2) return capacity_wk<8, 4, XCAP_WIDE, 2, 2>();
  if (tm == 512 && g.il) {
    int cap = 0;
    il_dispatch(g, [&](auto kt, auto np) {
      cap = capacity_wk<8, decltype(kt)::value, XCAP_WIDE, decltype(np)::value, 1>();
      return hipSuccess;
    });
    return cap;
  }
  if (tm == 512) return capacity_w<8>(K);
  if (tm == 256) return capacity_w<4>(K);
  if (tm == 128) return capacity_w<2>(K);
  return 0;
}

int64_t conv_bf16_fused_sync_words(int64_t N, int tiles_per_sample, int stride, int K,
                                   int dilation, int epi, int64_t C_out, int G, int n_ttiles,
                                   int n_ctiles) {
  const int cap = conv_bf16_fused_capacity(stride, K, dilation);
  if (tiles_per_sample < 1 || cap < tiles_per_sample) return 0;
  int64_t spr = cap / tiles_per_sample;
  if (spr > N) spr = N;
  const int64_t rounds = (N + spr - 1) / spr;
  return spr * rounds * fused_barrier_groups(epi, C_out, G, n_ttiles, n_ctiles) + 1;
}

hipError_t conv_bf16_fused_launch(ConvArgs a, int epi, bool cooperative, hipStream_t s) {
  const int tps = a.n_ttiles * a.n_ctiles;
  const int cap = conv_bf16_fused_capacity(a.stride, a.K, a.dilation);
  if (tps < 1 || cap < tps) return hipErrorInvalidValue;
  int64_t spr = cap / tps;
  if (spr > a.N) spr = a.N;
  a.spr = (int32_t)spr;
  a.rounds = (int32_t)((a.N + spr - 1) / spr);
  // the counters (and the fault word just after them), zeroed by the weight
  // pack launched before this (conv_bf16_fused_sync_words of them)
  const int64_t words = conv_bf16_fused_sync_words(a.N, tps, a.stride, a.K, a.dilation, epi,
                                                   a.C_out, a.G, a.n_ttiles, a.n_ctiles);
  if (words < 1) return hipErrorInvalidValue;
  a.fault = a.sync + (words - 1);
  a.polls = barrier_poll_limit();
  const int tm = conv_bf16_tile_m(a.stride, a.K, a.dilation);
  if (tm == 512) return launch_w<8>(a, epi, s, cooperative);
  if (tm == 256) return launch_w<4>(a, epi, s, cooperative);
  return launch_w<2>(a, epi, s, cooperative);
}

}  // namespace c1g
