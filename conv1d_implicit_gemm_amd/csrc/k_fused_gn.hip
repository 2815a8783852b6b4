// Fused conv1d + GroupNorm in one pass, fp32, for slabs that fit on chip.
//
// One workgroup owns one sample n and a block of 16 output channels made of
// whole groups (C_out/G divides 16), over every output position: the complete
// GroupNorm slab of its groups ("Kimi-K2.6 l2_p35": statistics over C_out/G
// channels x T_out per (n, group); its single-pass design keeps a group's
// whole output on chip so the normalised result is written once).  Here the
// slab stays in MFMA accumulator registers: 16 waves (4 per SIMD, which
// measured faster than 2), each owning MQ 16-row subtiles of positions x 16
// channels (v_mfma_f32_16x16x4_f32), so y never goes to HBM and is never
// re-read.
//
// K loop: per chunk of 16 input channels (all taps) the input halo window of
// the whole sequence and the chunk's weights are staged in LDS, and every tap
// reads the window at a shifted offset.  Two LDS stages: while one chunk is
// consumed, the next one streams in with gfx950's direct global->LDS loads
// (global_load_lds_dwordx4 / _dword), which bypass VGPRs and do not occupy the
// waves' LDS instruction queues, so the MFMA operand reads are never stuck
// behind staging writes.  Window slots in the zero padding are zeroed once and
// never loaded.  A register-staged variant serves inputs whose rows are not
// 16-byte aligned.
//
// Each K-step (4 input channels at one tap) reads the A operands of the next
// step from LDS before issuing its own MQ independent MFMAs; scheduling fences
// keep that order and keep each step's accumulators apart.
//
// Epilogue: each wave takes the exact statistics of its part of each group
// (two passes over its registers: sum -> mean, then squared deviations from
// it), reduced across lanes with DPP and lane swaps; one exchange through LDS
// merges the waves' (mean, M2) in a fixed order (deterministic); each value is
// then normalised, scaled and written once.
//
// blockIdx -> (n, channel block) is remapped so that the workgroups of one
// sample land on the same XCD and share its L2 copy of x[n].
#include "common.hpp"
#include "launch.hpp"

namespace c1g {
namespace {

constexpr int NW = 16;             // waves per workgroup (4 per SIMD)
constexpr int NTHR = NW * 64;
constexpr int CB = 16;             // channels per workgroup
constexpr int CK = 16;             // input channels per K-chunk
constexpr int KMAX = 8;
constexpr int HALO_MAX = 28;       // (K-1)*dilation supported

template <int MQ>
struct FusedGeom {
  static constexpr int TCOV = NW * MQ * 16;          // positions covered
  static constexpr int XL = TCOV + 32;               // staged window width
  static constexpr int XS = XL + 16;                 // LDS row stride (== 16 mod 32)
  static constexpr int XQ = XL / 4;                  // 16-byte slots per row
  static constexpr int XV = (CK * XQ + NTHR - 1) / NTHR;
  static constexpr int WV = (KMAX * CK * CB + NTHR - 1) / NTHR;
  static constexpr int DPR = (XQ + 63) / 64;         // direct-load instructions per row
};

// Direct global->LDS copies: lane i of the wave writes lds_wave_base + i*size
// (M0 holds the wave's LDS base).  Written as inline assembly: the compiler
// treats its own LDS-DMA builtin like a flat access that may complete out of
// order with the LDS reads, and then waits for every LDS read in flight
// (lgkmcnt(0)) at each K-step of a chunk during which copies are pending,
// instead of only for the reads that step consumes.  Here the compiler does
// not know about the copies, so the kernel waits for them itself
// (wait_all_mem) before each workgroup barrier that publishes a stage; the
// memory clobber keeps every memory access on its side of a copy.
__device__ __forceinline__ uint32_t lds_addr(const float* lds) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds);
}
__device__ __forceinline__ void dma16(const float* src, float* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_addr(lds_wave_base))
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const float* src, float* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(src), "s"(lds_addr(lds_wave_base))
               : "memory", "m0");
}
// s_waitcnt vmcnt(0) lgkmcnt(0) (gfx9 encoding, expcnt at its maximum)
__device__ __forceinline__ void wait_all_mem() { __builtin_amdgcn_s_waitcnt(7 << 4); }

struct Coord {
  int64_t n;
  int cbase;
};

__device__ __forceinline__ Coord wg_coord(const FusedArgs& a) {
  // XCD-aware mapping: consecutive workgroup ids round-robin over the 8 XCDs;
  // give each XCD a contiguous range of (n, block) so one sample's blocks share an L2.
  const int nblk = (int)((a.C_out + CB - 1) / CB);
  const int total = (int)(a.N * nblk);
  int lin = blockIdx.x;
  if ((total & 7) == 0) lin = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  Coord r;
  r.n = lin / nblk;
  r.cbase = (lin - (int)r.n * nblk) * CB;
  return r;
}

// One chunk of MFMA work on a staged (window, weight) pair.
template <int MQ, int KT>
__device__ __forceinline__ void compute_chunk(const float* xs, const float* ws,
                                              f32x4 (&acc)[MQ], int abase, int bbase, int d) {
  using Gm = FusedGeom<MQ>;
  constexpr int HS = CK / 4;          // K-steps per tap
  constexpr int NSTEP = KT * HS;
  float av[2][MQ], bv[NSTEP];
#pragma unroll
  for (int st = 0; st < NSTEP; ++st) bv[st] = ws[bbase + ((st / HS) * CK + 4 * (st % HS)) * CB];
#pragma unroll
  for (int m = 0; m < MQ; ++m) av[0][m] = xs[abase + m * 16];
#pragma unroll
  for (int st = 0; st < NSTEP; ++st) {
    if (st + 1 < NSTEP) {
      const int j = (st + 1) / HS, h = (st + 1) % HS;
      const int ao = abase + 4 * h * Gm::XS + j * d;
#pragma unroll
      for (int m = 0; m < MQ; ++m) av[(st + 1) & 1][m] = xs[ao + m * 16];
    }
#pragma unroll
    for (int m = 0; m < MQ; ++m) acc[m] = mfma16x16x4(av[st & 1][m], bv[st], acc[m]);
    // keep the order: the next step's LDS reads before this step's MFMAs,
    // and no instruction crossing a step boundary
    if (st + 1 < NSTEP) __builtin_amdgcn_sched_group_barrier(0x100, MQ, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, MQ, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The channel's bias, gamma and beta, loaded at the start of the kernel so
// that their latency hides under the K loop (0 / 1 / 0 past C_out or absent).
struct ChanParams {
  float bias, ga, be;
};

__device__ __forceinline__ ChanParams load_params(const FusedArgs& a, int c) {
  const bool ok = c < a.C_out;
  return ChanParams{(a.bias != nullptr && ok) ? a.bias[c] : 0.f,
                    (a.gamma != nullptr && ok) ? a.gamma[c] : 1.f,
                    (a.beta != nullptr && ok) ? a.beta[c] : 0.f};
}

// Statistics, normalisation and the single write of the output slab.  lo /
// hi: LDS no longer in use (waves 0-7 / 8-15, 16 x (P + 4) floats each) in
// which a wave re-lays its normalised fp32 tile so that each streaming store
// writes whole channel-row runs (16 lanes x 16 bytes) instead of the 64-byte
// halves of lines the MFMA layout gives (which the streaming path does not
// merge: 1.5x the output's bytes reached HBM); nullptr: direct stores.
template <int MQ>
__device__ __forceinline__ void epilogue(const FusedArgs& a, const Coord& co,
                                         f32x4 (&acc)[MQ], const ChanParams& prm, f32x2* red,
                                         float* lo = nullptr, float* hi = nullptr) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, kq = lane >> 4;
  const int64_t n = co.n, T_out = a.T_out;
  const int c = co.cbase + lr;
  const bool cvalid = c < a.C_out;
  const int cpg = (int)(a.C_out / a.G);
  const int gl = lr / cpg;                 // group within the block
  const int t_lane = wave * MQ * 16 + 4 * kq;
  const bool full = FusedGeom<MQ>::TCOV == T_out;

  // lanes of one group differ in the low log2(cpg) bits of lr and in kq
  // (cpg is 1, 2, 4, 8 or 16: a group is an aligned run of lr values)
  auto group_reduce = [&](float v) {
    if (cpg > 1) v += dpp<kDppXor1>(v);
    if (cpg > 2) v += dpp<kDppXor2>(v);
    if (cpg > 4) v += dpp<kDppHalfMirror>(v);
    if (cpg > 8) v += dpp<kDppMirror>(v);
    return lane_sum<48>(v);
  };
  // Each wave first takes the exact statistics of its own part of each group
  // (two passes over its registers: the mean, then the squared deviations
  // from it), then one exchange through LDS merges the 16 waves' (mean, M2)
  // in a fixed order.  The wave's valid positions, hence its count per group:
  const int64_t vt64 = T_out - (int64_t)wave * MQ * 16;
  const int vt = (int)(vt64 < 0 ? 0 : (vt64 < MQ * 16 ? vt64 : MQ * 16));
  const float cnt_w = (float)(cpg * vt);
  float sum = 0.f;
#pragma unroll
  for (int m = 0; m < MQ; ++m) {
    acc[m] += prm.bias;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (full || t_lane + m * 16 + r < T_out) sum += acc[m][r];
  }
  const float mean_w = cnt_w > 0.f ? group_reduce(sum) / cnt_w : 0.f;
  float ss = 0.f;
#pragma unroll
  for (int m = 0; m < MQ; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (full || t_lane + m * 16 + r < T_out) {
        const float dv = acc[m][r] - mean_w;
        ss += dv * dv;
      }
  const float m2_w = group_reduce(ss);
  if (kq == 0 && (lr % cpg) == 0) red[wave * CB + gl] = f32x2{mean_w, m2_w};
  __syncthreads();
  float mean, var;
  if (full) {
    // every wave holds the same count n_w of each group: the mean of the
    // group is the mean of the wave means and M2 = sum M2_w + n_w * sum
    // (mean_w - mean)^2, exactly
    float sm = 0.f;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) sm += red[wv * CB + gl][0];
    mean = sm * (1.0f / NW);
    float m2 = 0.f, dd = 0.f;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) {
      const f32x2 e = red[wv * CB + gl];
      const float dm = e[0] - mean;
      m2 += e[1];
      dd += dm * dm;
    }
    var = (m2 + cnt_w * dd) / (cnt_w * NW);
  } else {
    // unequal counts (the sequence ends inside the last waves' rows): the
    // pairwise merge in wave order
    Stats st = {0.f, 0.f, 0.f};
    for (int wv = 0; wv < NW; ++wv) {
      const int64_t v64 = T_out - (int64_t)wv * MQ * 16;
      const int v = (int)(v64 < 0 ? 0 : (v64 < MQ * 16 ? v64 : MQ * 16));
      const f32x2 e = red[wv * CB + gl];
      st = stats_merge(st, Stats{(float)(cpg * v), e[0], e[1]});
    }
    mean = st.mean;
    var = st.m2 / st.n;
  }
  const float rstd = 1.0f / sqrtf(var + a.eps);

  // fp32 out, whole wave tile inside [0, T_out), aligned: through LDS
  constexpr int P = MQ * 16, RS = P + 4;  // positions per wave; LDS row stride
  constexpr int LPC = P / 4, CPI = 64 / LPC;  // lanes per channel row; rows per store
  if (lo != nullptr && !a.out_bf16 && (T_out & 3) == 0 &&
      (((uintptr_t)a.out) & 15) == 0 && (int64_t)(wave + 1) * P <= T_out) {
    const float be = prm.be;
    const float sc = rstd * prm.ga;
    float* tile = (wave < NW / 2 ? lo : hi) + (wave % (NW / 2)) * (CB * RS);
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      f32x4 z;
#pragma unroll
      for (int r = 0; r < 4; ++r) z[r] = (acc[m][r] - mean) * sc + be;
      *(f32x4*)(tile + lr * RS + m * 16 + 4 * kq) = z;
    }
    float* outp = (float*)a.out;
#pragma unroll
    for (int k = 0; k < CB / CPI; ++k) {
      const int ch = lane / LPC + CPI * k;
      const f32x4 v = *(const f32x4*)(tile + ch * RS + 4 * (lane % LPC));
      if (co.cbase + ch < a.C_out)
        store_elem4_nt(outp + (n * a.C_out + co.cbase + ch) * T_out + (int64_t)wave * P +
                           4 * (lane % LPC),
                       v);
    }
    if (cvalid && wave == 0 && kq == 0 && (lr % cpg) == 0) {
      const int64_t g = c / cpg;
      if (a.mean_out) a.mean_out[n * a.G + g] = mean;
      if (a.rstd_out) a.rstd_out[n * a.G + g] = rstd;
    }
    return;
  }

  if (cvalid) {
    const float be = prm.be;
    const float sc = rstd * prm.ga;
    // out as fp32, or rounded to bf16 (out_bf16)
    auto store = [&](auto* out) __attribute__((always_inline)) {
      auto* dst = out + (n * a.C_out + c) * T_out;
      const bool vec_ok =
          ((T_out & 3) == 0) && ((((uintptr_t)out) & (4 * sizeof(*out) - 1)) == 0);
#pragma unroll
      for (int m = 0; m < MQ; ++m) {
        const int64_t t = t_lane + m * 16;
        f32x4 z;
#pragma unroll
        for (int r = 0; r < 4; ++r) z[r] = (acc[m][r] - mean) * sc + be;
        if (vec_ok && t + 3 < T_out) {
          store_elem4_nt(dst + t, z);  // the final output: streaming stores
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (t + r < T_out) store_elem(dst + t + r, z[r]);
        }
      }
    };
    if (a.out_bf16)
      store((uint16_t*)a.out);
    else
      store((float*)a.out);
    if (wave == 0 && kq == 0 && (lr % cpg) == 0) {
      const int64_t g = c / cpg;
      if (a.mean_out) a.mean_out[n * a.G + g] = mean;
      if (a.rstd_out) a.rstd_out[n * a.G + g] = rstd;
    }
  }
}

// ------------------------------------------------------------ direct-load variant
// Requires T % 4 == 0 and a 16-byte aligned x: every 16-byte window slot then
// lies entirely inside [0,T) or entirely in the padding.
template <int MQ, int KT>
__global__ __launch_bounds__(NTHR) void fused_gn_dma_kernel(FusedArgs a) {
  using Gm = FusedGeom<MQ>;
  // two stages; distinct arrays so the compiler can tell a stage being read
  // from the stage being filled (gfx950 allows 160 KB of LDS per workgroup)
  __shared__ __attribute__((aligned(16))) float Xs0[CK * Gm::XS];
  __shared__ __attribute__((aligned(16))) float Xs1[CK * Gm::XS];
  __shared__ __attribute__((aligned(16))) float Ws0[KT * CK * CB];
  __shared__ __attribute__((aligned(16))) float Ws1[KT * CK * CB];
  __shared__ f32x2 red[NW * CB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, kq = lane >> 4;
  const Coord co = wg_coord(a);
  const int64_t n = co.n;
  const int cbase = co.cbase;
  const int d = a.dilation;
  const int64_t T = a.T;
  const int64_t tbase = -(int64_t)a.pad_left;
  const int64_t tal = (tbase >= 0) ? (tbase & ~(int64_t)3) : -(((-tbase) + 3) & ~(int64_t)3);
  const int shift = (int)(tbase - tal);
  const int n_chunks = (int)((a.C_in + CK - 1) / CK);
  const float* xn = a.x + n * a.C_in * T;
  constexpr int K = KT;

  // Zero the padding slots of both window stages (slots q < qlo and q >= qhi
  // of every row hold positions outside [0, T)) and, for a partial channel
  // block, the weight entries of channels past C_out.  The copies never touch
  // these slots, so the zero fill runs while the first chunk's copies land.
  auto zero_fill = [&]() {
    const int64_t qlo64 = (-tal + 3) / 4;  // first slot with t >= 0 (tal <= 0)
    const int qlo = (int)(qlo64 < Gm::XQ ? qlo64 : Gm::XQ);
    const int64_t qhi64 = (T - tal) / 4;   // first slot with t + 3 >= T
    const int qhi = (int)(qhi64 < qlo ? qlo : (qhi64 < Gm::XQ ? qhi64 : Gm::XQ));
    const int npad = qlo + (Gm::XQ - qhi);  // padding slots per row
    for (int e = tid; e < 2 * CK * npad; e += NTHR) {
      const int row = e / npad, k = e - row * npad;  // row: stage * CK + channel
      const int q = k < qlo ? k : qhi + (k - qlo);
      float* xs = row < CK ? Xs0 : Xs1;
      *(f32x4*)(xs + (row % CK) * Gm::XS + 4 * q) = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    if (cbase + CB > a.C_out)
      for (int e = tid; e < 2 * K * CK * CB; e += NTHR) {
        const int b = e / (K * CK * CB), p = e - b * (K * CK * CB);
        if (cbase + (p & (CB - 1)) >= a.C_out) (b ? Ws1 : Ws0)[p] = 0.f;
      }
  };

  // issue the direct loads of one chunk into a stage (window rows wave,
  // wave + NW, ...; weight instructions wave, wave + NW, ...)
  auto stage = [&](int chunk, float* xs, float* ws) {
    const int64_t ci0 = (int64_t)chunk * CK;
    for (int r = wave; r < CK; r += NW) {
      const bool row_ok = ci0 + r < a.C_in;
      const float* src_row = xn + (ci0 + r) * T + tal;
#pragma unroll
      for (int p = 0; p < Gm::DPR; ++p) {
        const int q = 64 * p + lane;
        const int64_t t = tal + 4 * q;
        float* dst = xs + r * Gm::XS + 4 * 64 * p;       // wave-uniform base
        if (row_ok && q < Gm::XQ && t >= 0 && t + 3 < T) dma16(src_row + 4 * q, dst);
      }
      if (!row_ok)  // partial last chunk: rows past C_in are zero
        for (int q = lane; q < Gm::XQ; q += 64)
          *(f32x4*)(xs + r * Gm::XS + 4 * q) = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    constexpr int NWI = K * CK * CB / 64;                // weight instructions
    for (int p = wave; p < NWI; p += NW) {
      const int e = 64 * p + lane;                       // LDS position
      const int c = e & (CB - 1), jc = e >> 4;
      const int j = jc / CK, cl = jc - j * CK;
      float* dst = ws + 64 * p;
      const bool cok = cbase + c < a.C_out;
      if (cok && ci0 + cl < a.C_in)
        dma4(a.w + ((int64_t)(cbase + c) * a.C_in + ci0 + cl) * K + j, dst);
      else if (cok)
        ws[e] = 0.f;
    }
  };

  const ChanParams prm = load_params(a, cbase + lr);
  f32x4 acc[MQ];
#pragma unroll
  for (int m = 0; m < MQ; ++m) acc[m] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int abase = kq * Gm::XS + shift + wave * MQ * 16 + lr;  // stride 1
  const int bbase = kq * CB + lr;

  stage(0, Xs0, Ws0);
  zero_fill();
  wait_all_mem();
  __syncthreads();
  // Each wave issues the next stage's copies at the highest issue priority,
  // so that the younger waves' copies are not held behind the older waves'
  // MFMAs (the SIMD otherwise serves its waves oldest first).
  for (int c = 0; c < n_chunks; c += 2) {
    __builtin_amdgcn_s_setprio(3);
    if (c + 1 < n_chunks) stage(c + 1, Xs1, Ws1);
    __builtin_amdgcn_s_setprio(0);
    compute_chunk<MQ, KT>(Xs0, Ws0, acc, abase, bbase, d);
    wait_all_mem();  // this wave's copies of the next stage have landed
    __syncthreads();
    if (c + 1 >= n_chunks) break;
    __builtin_amdgcn_s_setprio(3);
    if (c + 2 < n_chunks) stage(c + 2, Xs0, Ws0);
    __builtin_amdgcn_s_setprio(0);
    compute_chunk<MQ, KT>(Xs1, Ws1, acc, abase, bbase, d);
    wait_all_mem();
    __syncthreads();
  }
  epilogue<MQ>(a, co, acc, prm, red, Xs0, Xs1);
}

// ------------------------------------------------------------ register-staged variant
// Any T and alignment: each thread loads its window slots element by element
// (zero outside [0,T)) into registers one chunk ahead and writes them to LDS.
template <int MQ, int KT>
__global__ __launch_bounds__(NTHR) void fused_gn_regs_kernel(FusedArgs a) {
  using Gm = FusedGeom<MQ>;
  __shared__ __attribute__((aligned(16))) float Xs[CK * Gm::XS];
  __shared__ __attribute__((aligned(16))) float Ws[KT * CK * CB];
  __shared__ f32x2 red[NW * CB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, kq = lane >> 4;
  const Coord co = wg_coord(a);
  const int64_t n = co.n;
  const int cbase = co.cbase;
  const int d = a.dilation;
  const int64_t T = a.T;
  const int64_t tbase = -(int64_t)a.pad_left;
  const int64_t tal = (tbase >= 0) ? (tbase & ~(int64_t)3) : -(((-tbase) + 3) & ~(int64_t)3);
  const int shift = (int)(tbase - tal);
  const int n_chunks = (int)((a.C_in + CK - 1) / CK);
  const float* xn = a.x + n * a.C_in * T;
  constexpr int K = KT;

  f32x4 xr[Gm::XV];
  float wr[Gm::WV];
  auto fetch = [&](int chunk) {
    const int64_t ci0 = (int64_t)chunk * CK;
#pragma unroll
    for (int i = 0; i < Gm::XV; ++i) {
      const int q = tid + NTHR * i;
      const int row = q / Gm::XQ, c4 = q - row * Gm::XQ;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (row < CK && ci0 + row < a.C_in) {
        const int64_t t = tal + 4 * c4;
        const float* src = xn + (ci0 + row) * T;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (t + e >= 0 && t + e < T) v[e] = src[t + e];
      }
      xr[i] = v;
    }
#pragma unroll
    for (int i = 0; i < Gm::WV; ++i) {
      const int e = tid + NTHR * i;
      const int c = e & (CB - 1), jc = e >> 4;
      const int j = jc / CK, cl = jc - j * CK;
      float v = 0.f;
      if (j < K && cbase + c < a.C_out && ci0 + cl < a.C_in)
        v = a.w[((int64_t)(cbase + c) * a.C_in + ci0 + cl) * K + j];
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
      if (e < K * CK * CB) Ws[e] = wr[i];
    }
  };

  const ChanParams prm = load_params(a, cbase + lr);
  f32x4 acc[MQ];
#pragma unroll
  for (int m = 0; m < MQ; ++m) acc[m] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int abase = kq * Gm::XS + shift + wave * MQ * 16 + lr;
  const int bbase = kq * CB + lr;

  fetch(0);
  stash();
  __syncthreads();
  for (int chunk = 0; chunk < n_chunks; ++chunk) {
    if (chunk + 1 < n_chunks) fetch(chunk + 1);
    compute_chunk<MQ, KT>(Xs, Ws, acc, abase, bbase, d);
    __syncthreads();
    if (chunk + 1 < n_chunks) {
      stash();
      __syncthreads();
    }
  }
  epilogue<MQ>(a, co, acc, prm, red);
}

template <int MQ, int KT>
hipError_t launch_mqk(const FusedArgs& a, hipStream_t s) {
  const int nblk = (int)((a.C_out + CB - 1) / CB);
  dim3 grid((unsigned)(a.N * nblk));
  const bool direct = (a.T % 4 == 0) && ((((uintptr_t)a.x) & 15) == 0);
  if (direct)
    hipLaunchKernelGGL((fused_gn_dma_kernel<MQ, KT>), grid, dim3(NTHR), 0, s, a);
  else
    hipLaunchKernelGGL((fused_gn_regs_kernel<MQ, KT>), grid, dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

template <int MQ>
hipError_t launch_mq(const FusedArgs& a, hipStream_t s) {
  switch (a.K) {
    case 1: return launch_mqk<MQ, 1>(a, s);
    case 2: return launch_mqk<MQ, 2>(a, s);
    case 3: return launch_mqk<MQ, 3>(a, s);
    case 4: return launch_mqk<MQ, 4>(a, s);
    case 5: return launch_mqk<MQ, 5>(a, s);
    case 6: return launch_mqk<MQ, 6>(a, s);
    case 7: return launch_mqk<MQ, 7>(a, s);
    case 8: return launch_mqk<MQ, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int fused_gn_max_tout(int stride, int K, int dilation) {
  if (stride != 1 || K < 1 || K > KMAX || (int64_t)(K - 1) * dilation > HALO_MAX) return 0;
  return NW * 4 * 16;
}

bool fused_gn_supported(int64_t C_in, int64_t C_out, int32_t G, int64_t T_out, int stride,
                        int K, int dilation) {
  if (G < 1 || C_out % G) return false;
  if (C_out * C_in * K >= (1ll << 31)) return false;  // 32-bit weight offsets
  const int64_t cpg = C_out / G;
  if (cpg > CB || (CB % cpg) != 0) return false;
  return T_out >= 1 && T_out <= fused_gn_max_tout(stride, K, dilation);
}

hipError_t fused_gn_launch(const FusedArgs& a, hipStream_t s) {
  const int64_t t = a.T_out;
  if (t <= NW * 16 * 1) return launch_mq<1>(a, s);
  if (t <= NW * 16 * 2) return launch_mq<2>(a, s);
  if (t <= NW * 16 * 4) return launch_mq<4>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace c1g
