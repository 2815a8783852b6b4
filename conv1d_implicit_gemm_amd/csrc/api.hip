// C ABI of the conv1d -> GroupNorm library: validation, planning (output
// length, route, workspace layout) and launches on the caller's stream.
// Declarations and the contract of every entry point: include/conv1d_gn.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/conv1d_gn.h"
#include "launch.hpp"

using namespace c1g;

namespace {

enum Route { R_INVALID = 0, R_CONV_ONLY, R_FUSED, R_SPLIT, R_GEMM, R_PERSIST, R_EMPTY };

// Workgroups of the bf16 conv that one full MI355X keeps resident at once
// (one per compute unit); the persistent route needs a sample's tiles to fit.
constexpr int64_t kResidentTiles = 256;

struct Plan {
  int status = C1G_OK;
  const char* why = "";   // what made the planner refuse (for the C1G_LOG log)
  int route = R_INVALID;
  int64_t T_out = -1;
  bool bf16 = false;      // x and w are bf16
  bool out_bf16 = false;  // y / out are bf16
  int norm = C1G_NORM_NONE, epi = C1G_EPI_NONE;
  int n_chunks = 0, n_ttiles = 0, n_ctiles = 0, tm = 0, tn = 0;
  bool gemm_fused = false;  // R_GEMM: GroupNorm + row-min inside the GEMM epilogue
  size_t off_pack = 0, off_part = 0, off_mean = 0, off_rstd = 0, off_y = 0, total = 0;
  size_t off_ximg = 0;  // bf16 conv: channels-last input image
  size_t off_sync = 0;  // persistent route: per-round arrival counters
  bool x_nlc = false;   // channels-last x with T > 1 (T == 1: the same bytes as [N, C_in, 1])
  size_t off_xt = 0;    // fp32 and x_nlc: x transposed to [N, C_in, T] (at offset 0)
  int64_t T_img = 0;
};

Plan& refuse(Plan& p, int status, const char* why) {
  p.status = status;
  p.why = why;
  return p;
}

// C1G_FORCE_PATH=split (read at each call; for tests): problems the planner
// would give a single-kernel route (fused_single_pass, fused_persistent) take
// the split route instead, so one problem can be run down both.
bool force_split() {
  const char* e = std::getenv("C1G_FORCE_PATH");
  return e != nullptr && std::strcmp(e, "split") == 0;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int64_t out_len(const c1g_conv_desc* d) {
  if (!d) return -1;
  // (a T past 2^62 is no length: the span below must not overflow)
  if (d->N < 0 || d->C_in < 1 || d->C_out < 1 || d->T < 1 || d->T > (1ll << 62)) return -1;
  if (d->K < 1 || d->stride < 1 || d->dilation < 1 || d->pad_left < 0 || d->pad_right < 0)
    return -1;
  const int64_t span =
      d->T + d->pad_left + d->pad_right - (int64_t)d->dilation * (d->K - 1) - 1;
  if (span < 0) return -1;
  return span / d->stride + 1;
}

// Everything the entry points need to know before touching the device.
Plan make_plan(const c1g_conv_desc* d, const c1g_norm_desc* nd) {
  Plan p;
  p.T_out = out_len(d);
  if (p.T_out < 1)
    return refuse(p, C1G_ERR_INVALID_ARG,
                  "a size, tap, stride, dilation or padding out of range, or no output position");
  if (d->dtype != C1G_F32 && d->dtype != C1G_BF16)
    return refuse(p, C1G_ERR_UNSUPPORTED, "dtype is neither fp32 nor bf16");
  p.bf16 = d->dtype == C1G_BF16;
  if (d->out_dtype != C1G_F32 && d->out_dtype != C1G_BF16)
    return refuse(p, C1G_ERR_UNSUPPORTED, "out_dtype is neither fp32 nor bf16");
  p.out_bf16 = d->out_dtype == C1G_BF16;
  if (d->x_layout != C1G_LAYOUT_NCL && d->x_layout != C1G_LAYOUT_NLC)
    return refuse(p, C1G_ERR_INVALID_ARG, "x_layout is neither NCL nor NLC");
  // sizes far past any device's memory are refused before a byte count is
  // formed from them: N up to 65535, C_in and C_out up to 2^30, T up to 2^40,
  // x and w below 2^46 elements each (the products are taken in 128 bits)
  typedef unsigned __int128 u128;
  if (d->N > 65535 || d->C_in > (1ll << 30) || d->C_out > (1ll << 30) || d->T > (1ll << 40) ||
      (u128)(uint64_t)d->N * (uint64_t)d->C_in * (uint64_t)d->T >= ((u128)1 << 46) ||
      (u128)(uint64_t)d->C_out * (uint64_t)d->C_in * (uint64_t)d->K >= ((u128)1 << 46))
    return refuse(p, C1G_ERR_UNSUPPORTED,
                  "past the size limits (N 65535, C 2^30, T 2^40, x and w 2^46 elements)");
  p.x_nlc = d->x_layout == C1G_LAYOUT_NLC && d->T > 1;
  // fp32 kernels read x position-contiguous: a channels-last x is transposed
  // into the front of the workspace first
  const size_t xt_bytes =
      (p.x_nlc && !p.bf16) ? align_up((size_t)d->N * d->C_in * d->T * sizeof(float)) : 0;
  if (xt_bytes && (d->C_in + 63) / 64 > 65535)
    return refuse(p, C1G_ERR_UNSUPPORTED, "channels-last fp32 x with C_in past 65535 * 64");
  if (nd) {
    p.norm = nd->norm;
    p.epi = nd->epilogue;
    if (p.norm < C1G_NORM_NONE || p.norm > C1G_NORM_LAYER_CHANNELS ||
        p.epi < C1G_EPI_NONE || p.epi > C1G_EPI_ROWMIN_BIAS)
      return refuse(p, C1G_ERR_INVALID_ARG, "unknown norm or epilogue");
    if (p.norm == C1G_NORM_GROUP && (nd->G < 1 || d->C_out % nd->G != 0))
      return refuse(p, C1G_ERR_INVALID_ARG, "G < 1 or C_out % G != 0");
    if (p.norm != C1G_NORM_NONE && !(nd->eps > 0.f && std::isfinite(nd->eps)))
      return refuse(p, C1G_ERR_INVALID_ARG, "eps not finite and > 0");
  }
  // an empty batch: nothing to read, write or launch
  if (d->N == 0) {
    p.route = R_EMPTY;
    p.total = 0;
    return p;
  }
  // size limits of the kernels' index arithmetic and grids
  const uint64_t n_out = (uint64_t)d->N * (uint64_t)d->C_out * (uint64_t)p.T_out;
  if (n_out >= (1ull << 32))
    return refuse(p, C1G_ERR_UNSUPPORTED, "N * C_out * T_out >= 2^32");

  // route
  const bool want_gn = p.norm == C1G_NORM_GROUP, want_ln = p.norm == C1G_NORM_LAYER_CHANNELS;
  const bool conv_only = p.norm == C1G_NORM_NONE && p.epi == C1G_EPI_NONE;
  if (!p.bf16 && want_gn && p.epi == C1G_EPI_NONE && !force_split() &&
      fused_gn_supported(d->C_in, d->C_out, nd->G, p.T_out, d->stride, d->K, d->dilation)) {
    p.route = R_FUSED;
    p.total = xt_bytes;
    return p;
  }
  // K = 1, T = 1 (a Linear layer) in bf16: plain GEMM over rows n
  if (p.bf16 && d->K == 1 && d->T == 1 && d->pad_left == 0 && d->pad_right == 0 &&
      d->C_in % 8 == 0 && (d->N > d->C_out ? d->N : d->C_out) * d->C_in < (1ll << 31)) {
    p.route = R_GEMM;
    p.tn = gemm_bf16_tile_c();
    p.n_ctiles = (int)((d->C_out + p.tn - 1) / p.tn);
    p.n_ttiles = (int)((d->N + gemm_bf16_tile_n() - 1) / gemm_bf16_tile_n());
    p.gemm_fused = want_gn && p.epi == C1G_EPI_ROWMIN_BIAS && d->C_out / nd->G == 16;
    size_t off = 0;
    p.off_part = off;
    off = align_up(off + (p.gemm_fused ? (size_t)d->N * p.n_ctiles * sizeof(float) : 0));
    const size_t stat = want_gn ? (size_t)d->N * nd->G : want_ln ? (size_t)d->N : 0;
    p.off_mean = off;
    off = align_up(off + stat * sizeof(float));
    p.off_rstd = off;
    off = align_up(off + stat * sizeof(float));
    // a bf16 out of the unfused epilogues: fp32 y in the workspace, so the
    // statistics and the affine read unrounded values
    p.off_y = off;
    if (p.out_bf16 && !p.gemm_fused) off = align_up(off + (size_t)d->N * d->C_out * sizeof(float));
    // the one-launch form of the fused epilogue: an arrival counter per row
    // block and a fault word
    p.off_sync = off;
    if (p.gemm_fused) off = align_up(off + (size_t)(p.n_ttiles + 1) * sizeof(unsigned));
    p.total = conv_only ? 0 : off;
    return p;
  }
  p.route = conv_only ? R_CONV_ONLY : R_SPLIT;

  size_t pack_bytes, ximg_bytes = 0;
  if (p.bf16) {
    const int tm = conv_bf16_tile_m(d->stride, d->K, d->dilation);
    if (tm == 0)
      return refuse(p, C1G_ERR_UNSUPPORTED,
                    "bf16: K > 8, or the input window wider than any tile's");
    p.tm = tm;
    p.tn = ConvBf16Cfg::TN;
    p.n_chunks = (int)((d->C_in + ConvBf16Cfg::CK - 1) / ConvBf16Cfg::CK);
    pack_bytes = conv_bf16_packed_bytes(d->C_in, d->C_out, d->K);
    p.T_img = conv_bf16_image_rows(p.T_out, d->stride, d->K, d->dilation);
    // row offsets into the image are 32-bit within a tile's window
    if ((int64_t)p.n_chunks * ConvBf16Cfg::CK * 2 * 1024 >= (1ll << 31))
      return refuse(p, C1G_ERR_UNSUPPORTED, "bf16: C_in too large for 32-bit image offsets");
    ximg_bytes = conv_bf16_image_bytes(d->N, d->C_in, p.T_img);
  } else {
    if (d->K > 8) return refuse(p, C1G_ERR_UNSUPPORTED, "fp32: K > 8");
    const int64_t xw = (int64_t)(ConvF32Cfg::TM - 1) * d->stride +
                       (int64_t)(d->K - 1) * d->dilation + 1;
    if (xw > conv_f32_window_cap(d->stride))
      return refuse(p, C1G_ERR_UNSUPPORTED, "fp32: the input window is wider than a tile's");
    p.tm = ConvF32Cfg::TM;
    p.tn = ConvF32Cfg::TN;
    p.n_chunks = (int)((d->C_in + ConvF32Cfg::CK - 1) / ConvF32Cfg::CK);
    pack_bytes = conv_f32_packed_bytes(d->C_in, d->C_out, d->K);
  }
  const int64_t n_tt = (p.T_out + p.tm - 1) / p.tm, n_ct = (d->C_out + p.tn - 1) / p.tn;
  if (n_tt > (1ll << 31) - 1 || n_ct > 65535)
    return refuse(p, C1G_ERR_UNSUPPORTED, "too many tiles for the grid");
  p.n_ttiles = (int)n_tt;
  p.n_ctiles = (int)n_ct;
  // bf16 GroupNorm or channel LayerNorm without the row-min: normalise
  // inside the persistent conv
  if (p.bf16 && (want_gn || want_ln) && p.epi == C1G_EPI_NONE &&
      !(nd->flags & C1G_FLAG_NO_PERSISTENT) && !force_split() && n_tt * n_ct <= kResidentTiles)
    p.route = R_PERSIST;

  size_t off = xt_bytes;
  p.off_pack = off;
  off = align_up(off + pack_bytes);
  p.off_ximg = off;
  off = align_up(off + ximg_bytes);
  const size_t conv_bytes = off;  // what the convolution alone needs
  size_t part_bytes = 0, stat_elems = 0;
  if (want_gn) {
    part_bytes = (size_t)d->N * d->C_out * p.n_ttiles * 2 * sizeof(float);
    stat_elems = (size_t)d->N * nd->G;
  } else if (want_ln) {
    part_bytes = (size_t)d->N * p.n_ctiles * p.T_out * 2 * sizeof(float);
    stat_elems = (size_t)d->N * p.T_out;
  }
  p.off_part = off;
  off = align_up(off + part_bytes);
  p.off_mean = off;
  off = align_up(off + stat_elems * sizeof(float));
  p.off_rstd = off;
  off = align_up(off + stat_elems * sizeof(float));
  // rounds * samples-per-round * barrier groups counters + 1 fault word
  // (rounds * samples-per-round < 2N; groups <= the tiles along one axis)
  p.off_sync = off;
  if (p.route == R_PERSIST) {
    const int64_t groups = p.n_ttiles > p.n_ctiles ? p.n_ttiles : p.n_ctiles;
    off = align_up(off + (size_t)(2 * d->N * groups + 2) * sizeof(unsigned));
  }
  p.total = (p.route == R_CONV_ONLY) ? conv_bytes : off;
  return p;
}

bool aligned(const void* p, size_t a) { return (((uintptr_t)p) % a) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? C1G_OK : C1G_ERR_HIP; }

// What a call did beyond its plan (a fallback it took), for its log line;
// set by the run paths, cleared by each entry point.
thread_local const char* t_note = nullptr;

// Records what made a call refuse (for its log line) and returns the status.
int refused(const char*& why, int status, const char* reason) {
  why = reason;
  return status;
}

ConvArgs conv_args(const Plan& p, const c1g_conv_desc* d, const void* x, const float* bias,
                   void* y, char* ws) {
  ConvArgs a = {};
  a.x = x;
  a.wp = ws + p.off_pack;
  a.ximg = ws + p.off_ximg;
  a.T_img = p.T_img;
  a.bias = bias;
  a.y = y;
  a.part = (float*)(ws + p.off_part);
  a.N = d->N;
  a.C_in = d->C_in;
  a.C_out = d->C_out;
  a.T = d->T;
  a.T_out = p.T_out;
  a.K = d->K;
  a.stride = d->stride;
  a.dilation = d->dilation;
  a.pad_left = d->pad_left;
  a.n_chunks = p.n_chunks;
  a.n_ttiles = p.n_ttiles;
  a.n_ctiles = p.n_ctiles;
  a.y_bf16 = p.out_bf16;
  return a;
}

// Convolution into y (with the requested statistics epilogue); packs weights
// (and, for bf16, the input image) first.  norm: the persistent route's
// normalisation (epi EPI_GN_FUSED / EPI_LN_FUSED), else nullptr.
int run_conv(const Plan& p, const c1g_conv_desc* d, const void* x, const void* w,
             const float* bias, void* y, char* ws, int epi, hipStream_t s,
             const c1g_norm_desc* nd = nullptr, const float* gamma = nullptr,
             const float* beta = nullptr, float* mean_out = nullptr, float* rstd_out = nullptr) {
  hipError_t e;
  if (p.x_nlc && !p.bf16) {
    e = transpose_nlc_f32((const float*)x, (float*)(ws + p.off_xt), d->N, d->T, d->C_in, s);
    if (e != hipSuccess) return C1G_ERR_HIP;
    x = ws + p.off_xt;
  }
  ConvArgs a = conv_args(p, d, x, bias, y, ws);
  if (p.bf16) {
    const bool fused = epi == EPI_GN_FUSED || epi == EPI_LN_FUSED;
    // the persistent kernel's arrival counters, zeroed by the weight pack
    const int64_t zw =
        fused ? conv_bf16_fused_sync_words(d->N, p.n_ttiles * p.n_ctiles, d->stride, d->K,
                                           d->dilation, epi, d->C_out, nd->G, p.n_ttiles,
                                           p.n_ctiles)
              : 0;
    if (fused && zw < 1) return C1G_ERR_HIP;
    e = conv_bf16_pack((const uint16_t*)w, (uint16_t*)(ws + p.off_pack), d->C_in, d->C_out,
                       d->K, s, fused ? (unsigned*)(ws + p.off_sync) : nullptr, zw);
    if (e != hipSuccess) return C1G_ERR_HIP;
    e = conv_bf16_pack_x((const uint16_t*)x, (uint16_t*)(ws + p.off_ximg), d->N, d->C_in, d->T,
                         d->pad_left, p.T_img, p.x_nlc, s);
    if (e != hipSuccess) return C1G_ERR_HIP;
    if (epi == EPI_GN_FUSED || epi == EPI_LN_FUSED) {
      a.gamma = gamma;
      a.beta = beta;
      a.mean_out = mean_out;
      a.rstd_out = rstd_out;
      a.eps = nd->eps;
      a.G = nd->G;
      a.sync = (unsigned*)(ws + p.off_sync);
      return hip_status(
          conv_bf16_fused_launch(a, epi, (nd->flags & C1G_FLAG_COOPERATIVE) != 0, s));
    }
    return hip_status(conv_bf16_launch(a, epi, s));
  }
  e = conv_f32_pack((const float*)w, (float*)(ws + p.off_pack), d->C_in, d->C_out, d->K, s);
  if (e != hipSuccess) return C1G_ERR_HIP;
  return hip_status(conv_f32_launch(a, epi, s));
}

// K = 1, T = 1 bf16 GEMM route: y[n][c] (== out viewed as [N, C_out, 1]).
int run_gemm(const Plan& p, const c1g_conv_desc* d, const c1g_norm_desc* nd, const void* x,
             const void* w, const float* bias, const float* gamma, const float* beta,
             const float* bias2, void* out, float* mean_out, float* rstd_out, char* ws,
             hipStream_t s) {
  if (!aligned(x, 16) || !aligned(w, 16)) {
    t_note = "gemm_rows: x or w not 16-byte aligned";
    return C1G_ERR_MISALIGNED;
  }
  const bool conv_only = !nd || (p.norm == C1G_NORM_NONE && p.epi == C1G_EPI_NONE);
  const int out_dt = p.out_bf16 ? C1G_BF16 : C1G_F32;
  GemmArgs g{};
  g.x = x;
  g.w = w;
  g.bias = bias;
  g.gamma = gamma;
  g.beta = beta;
  // y: out itself, except ahead of an unfused epilogue into a bf16 out (then
  // fp32 y in the workspace)
  float* y = (!conv_only && p.out_bf16) ? (float*)(ws + p.off_y) : (float*)out;
  g.y = conv_only ? out : (void*)y;
  g.y_bf16 = conv_only && p.out_bf16;
  g.part = (float*)(ws + p.off_part);
  g.mean_out = mean_out;
  g.rstd_out = rstd_out;
  g.N = d->N;
  g.C_in = d->C_in;
  g.C_out = d->C_out;
  g.G = nd ? nd->G : 0;
  g.n_ctiles = p.n_ctiles;
  g.n_ntiles = p.n_ttiles;
  g.eps = nd ? nd->eps : 0.f;
  if (p.gemm_fused) {
    // one launch (cooperative with C1G_FLAG_COOPERATIVE) on request when every
    // tile can be resident at once, else the GEMM and a broadcast kernel
    const bool one = (nd->flags & C1G_FLAG_ROWMIN_ONE_LAUNCH) && !(nd->flags & C1G_FLAG_NO_PERSISTENT);
    if (one && (int64_t)p.n_ctiles * p.n_ttiles > gemm_bf16_rowmin_capacity())
      t_note = "one launch requested, more tiles than the device keeps resident: two launches";
    if (one && (int64_t)p.n_ctiles * p.n_ttiles <= gemm_bf16_rowmin_capacity()) {
      g.bias2 = bias2;
      g.out = out;
      g.out_bf16 = p.out_bf16;
      g.sync = (unsigned*)(ws + p.off_sync);
      return hip_status(
          gemm_bf16_rowmin_one_launch(g, (nd->flags & C1G_FLAG_COOPERATIVE) != 0, s));
    }
    hipError_t e = gemm_bf16_launch(g, GEMM_GN_ROWMIN, s);
    if (e != hipSuccess) return C1G_ERR_HIP;
    return hip_status(
        rowmin_bcast_launch(g.part, d->N, p.n_ctiles, bias2, out, p.out_bf16, d->C_out, s));
  }
  hipError_t e = gemm_bf16_launch(g, GEMM_STORE, s);
  if (e != hipSuccess) return C1G_ERR_HIP;
  if (conv_only) return C1G_OK;
  // y is [N, C_out, 1]: a group's values are contiguous, as are a row's channels
  float* mean = mean_out ? mean_out : (float*)(ws + p.off_mean);
  float* rstd = rstd_out ? rstd_out : (float*)(ws + p.off_rstd);
  if (p.norm == C1G_NORM_GROUP) {
    e = gn_stats_launch(y, d->N, d->C_out, 1, nd->G, nd->eps, mean, rstd, nullptr, s);
    if (e != hipSuccess) return C1G_ERR_HIP;
    e = (p.epi == C1G_EPI_NONE)
            ? gn_apply_launch(y, C1G_F32, mean, rstd, gamma, beta, out, out_dt, d->N, d->C_out,
                              1, nd->G, s)
            : rowmin_bias_launch(y, C1G_F32, mean, rstd, gamma, beta, bias2, out, out_dt, d->N,
                                 d->C_out, 1, nd->G, 1, s);
  } else if (p.norm == C1G_NORM_LAYER_CHANNELS) {
    // LayerNorm over the channels of one position == GroupNorm with one group
    e = gn_stats_launch(y, d->N, d->C_out, 1, 1, nd->eps, mean, rstd, nullptr, s);
    if (e != hipSuccess) return C1G_ERR_HIP;
    e = (p.epi == C1G_EPI_NONE)
            ? ln_apply_launch(y, C1G_F32, mean, rstd, gamma, beta, out, out_dt, d->N, d->C_out,
                              1, s)
            : rowmin_bias_launch(y, C1G_F32, mean, rstd, gamma, beta, bias2, out, out_dt, d->N,
                                 d->C_out, 1, 0, 2, s);
  } else {
    e = rowmin_bias_launch(y, C1G_F32, nullptr, nullptr, nullptr, nullptr, bias2, out, out_dt,
                           d->N, d->C_out, 1, 0, 0, s);
  }
  return hip_status(e);
}

const char* route_name(int r) {
  switch (r) {
    case R_CONV_ONLY: return "conv_only";
    case R_FUSED: return "fused_single_pass";
    case R_SPLIT: return "split";
    case R_GEMM: return "gemm_rows";
    case R_PERSIST: return "fused_persistent";
    case R_EMPTY: return "empty";
    default: return "invalid";
  }
}

// ---- host-side log: with the environment variable C1G_LOG=1 (read at each
// call) every entry point writes one line to stderr: its arguments' sizes,
// the plan (route, tiles, workspace), the status and, for a refusal, what
// caused it.  Nothing is logged otherwise, and never from the device.
bool log_enabled() {
  const char* e = std::getenv("C1G_LOG");
  return e != nullptr && std::strcmp(e, "1") == 0;
}

const char* dtype_name(int32_t t) { return t == C1G_F32 ? "fp32" : t == C1G_BF16 ? "bf16" : "?"; }

// one fputs per line, so lines of concurrent calls do not interleave
void log_line(const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  std::fputs(buf, stderr);
}

int log_conv(const char* entry, const c1g_conv_desc* d, const c1g_norm_desc* nd, const Plan& p,
             int status, const char* why) {
  if (!log_enabled()) return status;
  char geo[320] = "(no descriptor)", nrm[128] = "", plan[160] = "";
  if (d)
    std::snprintf(geo, sizeof(geo),
                  "N=%lld C_in=%lld C_out=%lld T=%lld K=%d stride=%d dilation=%d pad=%d/%d "
                  "%s->%s%s",
                  (long long)d->N, (long long)d->C_in, (long long)d->C_out, (long long)d->T,
                  d->K, d->stride, d->dilation, d->pad_left, d->pad_right,
                  dtype_name(d->dtype), dtype_name(d->out_dtype),
                  d->x_layout == C1G_LAYOUT_NLC ? " channels-last" : "");
  if (nd)
    std::snprintf(nrm, sizeof(nrm), " norm=%s G=%d eps=%g%s flags=%d",
                  nd->norm == C1G_NORM_GROUP ? "group"
                  : nd->norm == C1G_NORM_LAYER_CHANNELS ? "layer_channels"
                  : nd->norm == C1G_NORM_NONE ? "none" : "?",
                  nd->G, (double)nd->eps, nd->epilogue == C1G_EPI_ROWMIN_BIAS ? " rowmin" : "",
                  nd->flags);
  if (p.status == C1G_OK && p.route != R_INVALID) {
    // bf16 convolutions: the tile's positions and, beyond one, the passes
    char conv[64] = "";
    if (p.bf16 && d && (p.route == R_SPLIT || p.route == R_CONV_ONLY || p.route == R_PERSIST)) {
      int il = 0;
      const int np = conv_bf16_passes(d->stride, d->K, d->dilation, &il);
      if (np > 1)
        std::snprintf(conv, sizeof(conv), " tile=%d passes=%d%s", p.tm, np,
                      il ? " interleaved" : "");
      else
        std::snprintf(conv, sizeof(conv), " tile=%d", p.tm);
    }
    std::snprintf(plan, sizeof(plan), " | %s T_out=%lld tiles=%dx%d ws=%zu%s",
                  route_name(p.route), (long long)p.T_out, p.n_ttiles, p.n_ctiles, p.total,
                  conv);
  }
  const char* reason = (why && *why) ? why : (t_note ? t_note : "");
  log_line("c1g: %s %s%s%s -> %s%s%s\n", entry, geo, nrm, plan, c1g_status_string(status),
           *reason ? ": " : "", reason);
  return status;
}

int log_norm(const char* entry, int64_t N, int64_t C, int64_t L, int32_t G, int status,
             const char* why) {
  if (!log_enabled()) return status;
  log_line("c1g: %s N=%lld C=%lld L=%lld G=%d -> %s%s%s\n", entry, (long long)N, (long long)C,
           (long long)L, G, c1g_status_string(status), (why && *why) ? ": " : "",
           why ? why : "");
  return status;
}

}  // namespace

extern "C" {

int64_t c1g_out_len(const c1g_conv_desc* d) { return out_len(d); }

int c1g_check(const c1g_conv_desc* d, const c1g_norm_desc* norm, size_t ws_bytes) {
  if (!d) return C1G_ERR_INVALID_ARG;
  const Plan p = make_plan(d, norm);
  if (p.status != C1G_OK) return p.status;
  if (ws_bytes < p.total) return C1G_ERR_WORKSPACE;
  return C1G_OK;
}

const char* c1g_route(const c1g_conv_desc* d, const c1g_norm_desc* norm) {
  if (!d) return "invalid";
  const Plan p = make_plan(d, norm);
  return p.status == C1G_OK ? route_name(p.route) : "invalid";
}

size_t c1g_conv1d_workspace_size(const c1g_conv_desc* d) {
  if (!d) return 0;
  const Plan p = make_plan(d, nullptr);
  return p.status == C1G_OK ? p.total : 0;
}

size_t c1g_conv1d_gn_workspace_size(const c1g_conv_desc* d, const c1g_norm_desc* norm) {
  if (!d) return 0;
  const Plan p = make_plan(d, norm);
  return p.status == C1G_OK ? p.total : 0;
}

int conv1d_forward(const c1g_conv_desc* d, const void* x, const void* w, const float* bias,
                   void* y, void* ws, size_t ws_bytes, void* stream) {
  t_note = nullptr;
  Plan p;
  const char* why = "";
  const int st = [&]() -> int {
    if (!d) return refused(why, C1G_ERR_INVALID_ARG, "no descriptor");
    p = make_plan(d, nullptr);
    if (p.status != C1G_OK) return refused(why, p.status, p.why);
    if (p.route == R_EMPTY) return C1G_OK;
    if (!x || !w || !y) return refused(why, C1G_ERR_INVALID_ARG, "x, w or y is NULL");
    const size_t es = p.bf16 ? 2 : 4, os = p.out_bf16 ? 2 : 4;
    if (!aligned(x, es) || !aligned(w, es) || !aligned(y, os) || (bias && !aligned(bias, 4)))
      return refused(why, C1G_ERR_MISALIGNED, "a tensor not aligned to its element size");
    if (p.total > 0 && (!ws || ws_bytes < p.total))
      return refused(why, C1G_ERR_WORKSPACE, "workspace NULL or below the size query");
    if (p.total > 0 && !aligned(ws, kAlign))
      return refused(why, C1G_ERR_MISALIGNED, "workspace not 256-byte aligned");
    if (p.route == R_GEMM)
      return run_gemm(p, d, nullptr, x, w, bias, nullptr, nullptr, nullptr, y, nullptr, nullptr,
                      (char*)ws, (hipStream_t)stream);
    return run_conv(p, d, x, w, bias, y, (char*)ws, EPI_STORE, (hipStream_t)stream);
  }();
  return log_conv("conv1d_forward", d, nullptr, p, st, why);
}

namespace {
bool gn_stats_args_ok(int64_t N, int64_t C, int64_t L, int32_t G) {
  return N >= 0 && C >= 1 && L >= 1 && G >= 1 && C % G == 0;
}
// grid of the first stage: one workgroup per slice of 32768 values of a
// group, at most 2^31 - 1 of them; the products are taken in 128 bits with
// each factor bounded first, so no size wraps into an accepted one (and every
// offset, below 32768 * 2^31 values, fits 64 bits)
bool gn_stats_fits(int64_t N, int64_t C, int64_t L, int32_t G) {
  typedef unsigned __int128 u128;
  const u128 len = (u128)(uint64_t)(C / G) * (uint64_t)L;
  const u128 slices = (len + 32767) / 32768;
  const u128 ng = (u128)(uint64_t)N * (uint64_t)G;
  return slices <= 0x7fffffff && ng <= 0x7fffffff && ng * slices <= 0x7fffffff;
}
// N * C * L < 2^32 (C and L at most 2^31), without a product that could wrap
bool apply_fits(int64_t N, int64_t C, int64_t L) {
  if (C > (1ll << 31) || L > (1ll << 31)) return false;
  const uint64_t cl = (uint64_t)C * (uint64_t)L;
  return cl < (1ull << 32) && (uint64_t)N < (1ull << 32) && (uint64_t)N * cl < (1ull << 32);
}
}  // namespace

size_t c1g_gn_stats_workspace_size(int64_t N, int64_t C, int64_t L, int32_t G) {
  if (!gn_stats_args_ok(N, C, L, G) || !gn_stats_fits(N, C, L, G)) return 0;
  const size_t b = gn_stats_workspace_bytes(N, C, L, G);
  return b ? align_up(b) : 0;
}

int gn_stats(int64_t N, int64_t C, int64_t L, int32_t G, float eps, const float* y, float* mean,
             float* rstd, void* ws, size_t ws_bytes, void* stream) {
  const char* why = "";
  const int st = [&]() -> int {
    if (!gn_stats_args_ok(N, C, L, G))
      return refused(why, C1G_ERR_INVALID_ARG, "a size out of range, G < 1 or C % G != 0");
    if (!(eps > 0.f && std::isfinite(eps)))
      return refused(why, C1G_ERR_INVALID_ARG, "eps not finite and > 0");
    if (N == 0) return C1G_OK;  // an empty batch
    if (!y || !mean || !rstd) return refused(why, C1G_ERR_INVALID_ARG, "y, mean or rstd is NULL");
    if (!gn_stats_fits(N, C, L, G))
      return refused(why, C1G_ERR_UNSUPPORTED, "more than 2^31 - 1 slices of 32768 values");
    if (!aligned(y, 4) || !aligned(mean, 4) || !aligned(rstd, 4))
      return refused(why, C1G_ERR_MISALIGNED, "a tensor not 4-byte aligned");
    // the size the query reports (rounded up to the workspace alignment)
    const size_t need = c1g_gn_stats_workspace_size(N, C, L, G);
    if (need > 0 && (!ws || ws_bytes < need))
      return refused(why, C1G_ERR_WORKSPACE, "workspace NULL or below the size query");
    if (need > 0 && !aligned(ws, kAlign))
      return refused(why, C1G_ERR_MISALIGNED, "workspace not 256-byte aligned");
    return hip_status(gn_stats_launch(y, N, C, L, G, eps, mean, rstd,
                                      need > 0 ? (float*)ws : nullptr, (hipStream_t)stream));
  }();
  return log_norm("gn_stats", N, C, L, G, st, why);
}

int gn_apply(int64_t N, int64_t C, int64_t L, int32_t G, const float* y, const float* mean,
             const float* rstd, const float* gamma, const float* beta, float* out,
             void* stream) {
  const char* why = "";
  const int st = [&]() -> int {
    if (N < 0 || C < 1 || L < 1 || G < 1 || C % G != 0)
      return refused(why, C1G_ERR_INVALID_ARG, "a size out of range, G < 1 or C % G != 0");
    if (N == 0) return C1G_OK;  // an empty batch
    if (!y || !mean || !rstd || !out)
      return refused(why, C1G_ERR_INVALID_ARG, "y, mean, rstd or out is NULL");
    if (!apply_fits(N, C, L))
      return refused(why, C1G_ERR_UNSUPPORTED, "N * C * L >= 2^32, or C or L past 2^31");
    if (!aligned(y, 4) || !aligned(out, 4) || !aligned(mean, 4) || !aligned(rstd, 4) ||
        (gamma && !aligned(gamma, 4)) || (beta && !aligned(beta, 4)))
      return refused(why, C1G_ERR_MISALIGNED, "a tensor not aligned to its element size");
    return hip_status(gn_apply_launch(y, C1G_F32, mean, rstd, gamma, beta, out, C1G_F32, N, C,
                                     L, G, (hipStream_t)stream));
  }();
  return log_norm("gn_apply", N, C, L, G, st, why);
}

int gn_apply_bf16(int64_t N, int64_t C, int64_t L, int32_t G, const uint16_t* y,
                  const float* mean, const float* rstd, const float* gamma, const float* beta,
                  uint16_t* out, void* stream) {
  const char* why = "";
  const int st = [&]() -> int {
    if (N < 0 || C < 1 || L < 1 || G < 1 || C % G != 0)
      return refused(why, C1G_ERR_INVALID_ARG, "a size out of range, G < 1 or C % G != 0");
    if (N == 0) return C1G_OK;  // an empty batch
    if (!y || !mean || !rstd || !out)
      return refused(why, C1G_ERR_INVALID_ARG, "y, mean, rstd or out is NULL");
    if (!apply_fits(N, C, L))
      return refused(why, C1G_ERR_UNSUPPORTED, "N * C * L >= 2^32, or C or L past 2^31");
    if (!aligned(y, 2) || !aligned(out, 2) || !aligned(mean, 4) || !aligned(rstd, 4) ||
        (gamma && !aligned(gamma, 4)) || (beta && !aligned(beta, 4)))
      return refused(why, C1G_ERR_MISALIGNED, "a tensor not aligned to its element size");
    return hip_status(gn_apply_launch(y, C1G_BF16, mean, rstd, gamma, beta, out, C1G_BF16, N,
                                     C, L, G, (hipStream_t)stream));
  }();
  return log_norm("gn_apply_bf16", N, C, L, G, st, why);
}

}  // extern "C"

namespace {

// The pointer checks of conv1d_gn_forward (everything but the workspace);
// *why names a refusal's cause.
int check_forward_ptrs(const Plan& p, const void* x, const void* w, const float* bias,
                       const float* gamma, const float* beta, const float* bias2,
                       const void* out, const float* mean_out, const float* rstd_out,
                       const char** why) {
  if (!x || !w || !out) return refused(*why, C1G_ERR_INVALID_ARG, "x, w or out is NULL");
  if (p.epi == C1G_EPI_ROWMIN_BIAS && !bias2)
    return refused(*why, C1G_ERR_INVALID_ARG, "the row-min epilogue without bias2");
  const size_t es = p.bf16 ? 2 : 4, os = p.out_bf16 ? 2 : 4;
  if (!aligned(x, es) || !aligned(w, es) || !aligned(out, os) || (bias && !aligned(bias, 4)) ||
      (gamma && !aligned(gamma, 4)) || (beta && !aligned(beta, 4)) ||
      (bias2 && !aligned(bias2, 4)) || (mean_out && !aligned(mean_out, 4)) ||
      (rstd_out && !aligned(rstd_out, 4)))
    return refused(*why, C1G_ERR_MISALIGNED, "a tensor not aligned to its element size");
  return C1G_OK;
}

// Device scratch of conv1d_gn_forward_noalloc, the workspace of callers that
// cannot allocate; each device the library runs on holds its own copy until
// the process ends.  In host code `scratch` names the runtime's host-side
// handle of the symbol, not device memory: the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current,
// and only that address is ever given to kernels.
static __device__ __align__(256) unsigned char scratch[C1G_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_addr[kMaxDevices];  // per device; null until looked up

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return C1G_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return C1G_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_addr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return C1G_ERR_HIP;
    scratch_addr[dev] = ptr;
  }
  *out = scratch_addr[dev];
  return C1G_OK;
}

// The work of conv1d_gn_forward, for it and the allocation-free entry point:
// p is the plan (filled in), why the cause of a refusal.
int forward_impl(const c1g_conv_desc* d, const c1g_norm_desc* nd, const void* x, const void* w,
                 const float* bias, const float* gamma, const float* beta, const float* bias2,
                 void* out, float* mean_out, float* rstd_out, void* ws, size_t ws_bytes,
                 void* stream, Plan& p, const char*& why) {
  if (!d || !nd) return refused(why, C1G_ERR_INVALID_ARG, "no descriptor");
  p = make_plan(d, nd);
  if (p.status != C1G_OK) return refused(why, p.status, p.why);
  if (p.route == R_EMPTY) return C1G_OK;
  const int pst =
      check_forward_ptrs(p, x, w, bias, gamma, beta, bias2, out, mean_out, rstd_out, &why);
  if (pst != C1G_OK) return pst;
  if (p.total > 0 && (!ws || ws_bytes < p.total))
    return refused(why, C1G_ERR_WORKSPACE, "workspace NULL or below the size query");
  if (p.total > 0 && !aligned(ws, kAlign))
    return refused(why, C1G_ERR_MISALIGNED, "workspace not 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  char* wsb = (char*)ws;

  if (p.route == R_FUSED) {
    if (p.x_nlc) {
      if (transpose_nlc_f32((const float*)x, (float*)(wsb + p.off_xt), d->N, d->T, d->C_in, s) !=
          hipSuccess)
        return C1G_ERR_HIP;
      x = wsb + p.off_xt;
    }
    FusedArgs a;
    a.x = (const float*)x;
    a.w = (const float*)w;
    a.bias = bias;
    a.gamma = gamma;
    a.beta = beta;
    a.out = out;
    a.mean_out = mean_out;
    a.rstd_out = rstd_out;
    a.N = d->N;
    a.C_in = d->C_in;
    a.C_out = d->C_out;
    a.T = d->T;
    a.T_out = p.T_out;
    a.K = d->K;
    a.stride = d->stride;
    a.dilation = d->dilation;
    a.pad_left = d->pad_left;
    a.G = nd->G;
    a.eps = nd->eps;
    a.out_bf16 = p.out_bf16;
    return hip_status(fused_gn_launch(a, s));
  }
  if (p.route == R_GEMM)
    return run_gemm(p, d, nd, x, w, bias, gamma, beta, bias2, out, mean_out, rstd_out, wsb, s);
  if (p.route == R_CONV_ONLY)
    return run_conv(p, d, x, w, bias, out, wsb, EPI_STORE, s);

  // persistent route: the conv kernel normalises in registers and writes out
  // once; on a device that cannot keep a sample's tiles resident together
  // (a partitioned GPU) the split route runs instead, in the same workspace
  if (p.route == R_PERSIST &&
      conv_bf16_fused_capacity(d->stride, d->K, d->dilation) >= p.n_ttiles * p.n_ctiles)
    return run_conv(p, d, x, w, bias, out, wsb,
                    p.norm == C1G_NORM_GROUP ? EPI_GN_FUSED : EPI_LN_FUSED, s, nd, gamma, beta,
                    mean_out, rstd_out);

  if (p.route == R_PERSIST)
    t_note = "fused_persistent planned, more tiles per sample than the device keeps "
             "resident: the split route ran";

  // split route: conv (+ partial statistics from the fp32 accumulators) into
  // out in out's type, merge, then in-place passes
  const int conv_epi = p.norm == C1G_NORM_GROUP ? EPI_GN_PART
                       : p.norm == C1G_NORM_LAYER_CHANNELS ? EPI_LN_PART : EPI_STORE;
  int st = run_conv(p, d, x, w, bias, out, wsb, conv_epi, s);
  if (st != C1G_OK) return st;
  float* mean = mean_out ? mean_out : (float*)(wsb + p.off_mean);
  float* rstd = rstd_out ? rstd_out : (float*)(wsb + p.off_rstd);
  const float* part = (const float*)(wsb + p.off_part);
  const int dt = p.out_bf16 ? C1G_BF16 : C1G_F32;
  hipError_t e = hipSuccess;
  if (p.norm == C1G_NORM_GROUP) {
    e = gn_merge_launch(part, d->N, d->C_out, p.T_out, nd->G, p.n_ttiles, p.tm, nd->eps, mean,
                        rstd, s);
    if (e != hipSuccess) return C1G_ERR_HIP;
    if (p.epi == C1G_EPI_NONE)
      e = gn_apply_launch(out, dt, mean, rstd, gamma, beta, out, dt, d->N, d->C_out, p.T_out,
                          nd->G, s);
    else
      e = rowmin_bias_launch(out, dt, mean, rstd, gamma, beta, bias2, out, dt, d->N, d->C_out,
                             p.T_out, nd->G, 1, s);
  } else if (p.norm == C1G_NORM_LAYER_CHANNELS) {
    e = ln_merge_launch(part, d->N, d->C_out, p.T_out, p.n_ctiles, p.tn, nd->eps, mean, rstd, s);
    if (e != hipSuccess) return C1G_ERR_HIP;
    if (p.epi == C1G_EPI_NONE)
      e = ln_apply_launch(out, dt, mean, rstd, gamma, beta, out, dt, d->N, d->C_out, p.T_out,
                          s);
    else
      e = rowmin_bias_launch(out, dt, mean, rstd, gamma, beta, bias2, out, dt, d->N, d->C_out,
                             p.T_out, 0, 2, s);
  } else {  // no norm, row-min epilogue only
    e = rowmin_bias_launch(out, dt, nullptr, nullptr, nullptr, nullptr, bias2, out, dt, d->N,
                           d->C_out, p.T_out, 0, 0, s);
  }
  return hip_status(e);
}

}  // namespace

extern "C" {

int conv1d_gn_forward(const c1g_conv_desc* d, const c1g_norm_desc* nd, const void* x,
                      const void* w, const float* bias, const float* gamma, const float* beta,
                      const float* bias2, void* out, float* mean_out, float* rstd_out,
                      void* ws, size_t ws_bytes, void* stream) {
  t_note = nullptr;
  Plan p;
  const char* why = "";
  const int st = forward_impl(d, nd, x, w, bias, gamma, beta, bias2, out, mean_out, rstd_out,
                              ws, ws_bytes, stream, p, why);
  return log_conv("conv1d_gn_forward", d, nd, p, st, why);
}

int conv1d_gn_forward_noalloc(const c1g_conv_desc* d, const c1g_norm_desc* nd, const void* x,
                              const void* w, const float* bias, const float* gamma,
                              const float* beta, const float* bias2, void* out,
                              float* mean_out, float* rstd_out, void* stream) {
  t_note = nullptr;
  Plan p;
  const char* why = "";
  const int st = [&]() -> int {
    if (!d || !nd) return refused(why, C1G_ERR_INVALID_ARG, "no descriptor");
    p = make_plan(d, nd);
    if (p.status != C1G_OK) return refused(why, p.status, p.why);
    if (p.route == R_EMPTY) return C1G_OK;
    const int pst =
        check_forward_ptrs(p, x, w, bias, gamma, beta, bias2, out, mean_out, rstd_out, &why);
    if (pst != C1G_OK) return pst;
    if (p.total > C1G_NOALLOC_SCRATCH_BYTES)
      return refused(why, C1G_ERR_WORKSPACE, "workspace past the static scratch");
    void* ws = nullptr;
    if (p.total > 0) {
      const int sst = scratch_address(&ws);
      if (sst != C1G_OK) return refused(why, sst, "no device scratch address");
    }
    return forward_impl(d, nd, x, w, bias, gamma, beta, bias2, out, mean_out, rstd_out, ws,
                        p.total > 0 ? C1G_NOALLOC_SCRATCH_BYTES : 0, stream, p, why);
  }();
  return log_conv("conv1d_gn_forward_noalloc", d, nd, p, st, why);
}

const char* c1g_status_string(int status) {
  switch (status) {
    case C1G_OK: return "ok";
    case C1G_ERR_INVALID_ARG: return "invalid argument";
    case C1G_ERR_UNSUPPORTED: return "unsupported configuration";
    case C1G_ERR_WORKSPACE: return "workspace missing or too small";
    case C1G_ERR_MISALIGNED: return "misaligned pointer";
    case C1G_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

}  // extern "C"
