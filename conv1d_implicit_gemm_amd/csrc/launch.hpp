// Host-side launch interface between the C ABI (api.cpp) and the kernel
// translation units.  Every launcher enqueues on the given stream, assumes
// its arguments were validated by the planner, and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace c1g {

// Epilogue of the split-path convolution kernels.
enum ConvEpi : int {
  EPI_STORE = 0,      // y = acc + bias
  EPI_GN_PART = 1,    // y, plus per-(n, channel, t-tile) (mean, M2) partials
  EPI_LN_PART = 2,    // y, plus per-(n, c-tile, t) (mean, M2) partials
  // bf16 persistent kernel: partials, a barrier among the workgroups of each
  // sample, the merge, and the normalised output written once (no y)
  EPI_GN_FUSED = 3,
  EPI_LN_FUSED = 4,
};

// Geometry + pointers of one implicit-GEMM convolution launch.
struct ConvArgs {
  const void* x;       // [N, C_in, T] fp32 or bf16
  const void* wp;      // packed weights (layout owned by the kernel file)
  const void* ximg;    // bf16: channels-last input image (conv_bf16_pack_x)
  int64_t T_img;       // bf16: rows per sample of the input image
  const float* bias;   // [C_out] or nullptr
  void* y;             // [N, C_out, T_out], fp32 or (y_bf16) bf16
  float* part;         // partial statistics (EPI_GN_PART / EPI_LN_PART), from fp32 values
  int64_t N, C_in, C_out, T, T_out;
  int32_t K, stride, dilation, pad_left;
  int32_t n_chunks;    // ceil(C_in / CK)
  int32_t n_ttiles;    // ceil(T_out / TM)
  int32_t n_ctiles;    // ceil(C_out / TN)
  int32_t y_bf16;      // y is stored as bf16 (rounded to nearest even)
  // EPI_GN_FUSED / EPI_LN_FUSED (y is then the normalised output)
  const float* gamma;  // [C_out] or nullptr
  const float* beta;
  float* mean_out;     // [N, G] (GroupNorm) or [N, T_out] (LayerNorm), or nullptr
  float* rstd_out;
  float eps;
  int32_t G;
  unsigned* sync;      // [rounds * spr * barrier groups] arrival counters, zero at launch
  int32_t spr;         // samples per round (spr * tiles per sample workgroups)
  int32_t rounds;      // ceil(N / spr)
  unsigned* fault;     // set when a barrier wait gives up (never on a full GPU)
  uint32_t polls;      // polls before a barrier wait gives up (set by the launcher)
};

// ---- kernels whose workgroups wait on each other (residency.hip)
// Workgroups of `kernel` (`threads` per workgroup, no dynamic LDS) the
// current device keeps resident at once, 0 if unknown; queried once per
// (device, kernel) and cached.
int resident_capacity(const void* kernel, int threads);
// Launch with grid <= resident_capacity (hipErrorInvalidValue otherwise): an
// ordinary launch, or (cooperative) hipLaunchCooperativeKernel, whose
// co-residency guarantee also holds while other work shares the device.
hipError_t launch_coresident(const void* kernel, unsigned grid, int threads, void** args,
                             bool cooperative, hipStream_t s);

// ---- fp32 split-path convolution (k_conv_f32.hip)
// Tile geometry: TM output positions x TN output channels, CK input channels
// per K-chunk.  xcap is the widest input window one tile may need.
struct ConvF32Cfg {
  static constexpr int TM = 128, TN = 128, CK = 8;
};
int conv_f32_window_cap(int stride);  // largest input window a tile supports
size_t conv_f32_packed_bytes(int64_t C_in, int64_t C_out, int K);
hipError_t conv_f32_pack(const float* w, float* wp, int64_t C_in, int64_t C_out, int K,
                         hipStream_t s);
hipError_t conv_f32_launch(const ConvArgs& a, int epi, hipStream_t s);

// ---- bf16 split-path convolution (k_conv_bf16.hip)
// Tile: TM (512, 256 or 128, chosen from stride/K/dilation) positions x TN
// channels, CK input channels per chunk; taps K <= 8.
struct ConvBf16Cfg {
  static constexpr int TN = 128, CK = 32;
};
int conv_bf16_tile_m(int stride, int K, int dilation);  // 0 if unsupported
// passes over the input channels (1 to 5); *interleaved: the passes take
// every stride-th tap (strided convolutions) rather than consecutive ones
int conv_bf16_passes(int stride, int K, int dilation, int* interleaved);
// channels-last input image: rows per sample, bytes, and the repack of x
int64_t conv_bf16_image_rows(int64_t T_out, int stride, int K, int dilation);
size_t conv_bf16_image_bytes(int64_t N, int64_t C_in, int64_t T_img);
// x [N, C_in, T], or (nlc) channels-last x [N, T, C_in]
hipError_t conv_bf16_pack_x(const uint16_t* x, uint16_t* ximg, int64_t N, int64_t C_in,
                            int64_t T, int pad_left, int64_t T_img, bool nlc, hipStream_t s);
size_t conv_bf16_packed_bytes(int64_t C_in, int64_t C_out, int K);
// also zeroes zero_words 32-bit words at zero (nullptr / 0: none)
hipError_t conv_bf16_pack(const uint16_t* w, uint16_t* wp, int64_t C_in, int64_t C_out, int K,
                          hipStream_t s, unsigned* zero = nullptr, int64_t zero_words = 0);
hipError_t conv_bf16_launch(const ConvArgs& a, int epi, hipStream_t s);
// Persistent conv + normalisation (EPI_GN_FUSED / EPI_LN_FUSED): workgroups
// that can be resident at once on the current device for this geometry (0 if
// unknown); the launch fills spr/rounds and launches (cooperatively on
// request).
int conv_bf16_fused_capacity(int stride, int K, int dilation);
// Workgroups of a persistent round wait for each other in groups: GroupNorm,
// the position tiles of a group's channel tiles; LayerNorm over channels, the
// channel tiles of a position tile.  Groups per sample (one arrival counter
// each per round and sample slot):
int fused_barrier_groups(int epi, int64_t C_out, int G, int n_ttiles, int n_ctiles);
// Words of arrival counters + fault word the persistent launch expects zeroed
// at a.sync (0 when the geometry does not fit the device); the weight pack
// zeroes them (conv_bf16_pack's zero / zero_words).
int64_t conv_bf16_fused_sync_words(int64_t N, int tiles_per_sample, int stride, int K,
                                   int dilation, int epi, int64_t C_out, int G, int n_ttiles,
                                   int n_ctiles);
hipError_t conv_bf16_fused_launch(ConvArgs a, int epi, bool cooperative, hipStream_t s);

// ---- bf16 GEMM for K = 1, T = 1 (k_gemm_bf16.hip)
// GEMM_GN_ROWMIN writes per-tile row minima for rowmin_bcast;
// GEMM_GN_ROWMIN_ONE (every tile resident at once) also waits for
// the other c-tiles of its rows and writes its block of the broadcast output
enum GemmEpi : int { GEMM_STORE = 0, GEMM_GN_ROWMIN = 1, GEMM_GN_ROWMIN_ONE = 2 };
struct GemmArgs {
  const void* x;       // [N, C_in] bf16, 16-byte aligned, C_in % 8 == 0
  const void* w;       // [C_out, C_in] bf16, 16-byte aligned
  const float* bias;   // [C_out] or nullptr
  const float* gamma;  // GN_ROWMIN: [C_out] or nullptr
  const float* beta;
  void* y;             // STORE: [N, C_out], fp32 or (y_bf16) bf16
  float* part;         // GN_ROWMIN: [N, n_ctiles] per-tile row minima
  float* mean_out;     // GN_ROWMIN: [N, G] or nullptr
  float* rstd_out;
  const float* bias2;  // GN_ROWMIN_ONE: [C_out] or nullptr
  void* out;           // GN_ROWMIN_ONE: [N, C_out], fp32 or (out_bf16) bf16
  unsigned* sync;      // GN_ROWMIN_ONE: n_ntiles arrival counters, zeroed by the launcher
  unsigned* fault;     // set when a barrier wait gives up (never on a full GPU)
  uint32_t polls;      // polls before a barrier wait gives up (set by the launcher)
  int64_t N, C_in, C_out;
  int32_t G, n_ctiles, n_ntiles;
  float eps;
  int32_t y_bf16, out_bf16;
};
int gemm_bf16_tile_c();
int gemm_bf16_tile_n();
hipError_t gemm_bf16_launch(const GemmArgs& a, int epi, hipStream_t s);
// channels-last fp32 x [N, T, C] -> xt [N, C, T] (k_layout.hip); needs
// ceil(C / 64) <= 65535
hipError_t transpose_nlc_f32(const float* x, float* xt, int64_t N, int64_t T, int64_t C,
                             hipStream_t s);
// GEMM + GroupNorm + row-min + bias2 in one launch whose workgroups wait on
// each other: workgroups the
// device keeps resident at once with the GN_ROWMIN_ONE kernel (0 on error);
// the launch needs n_ctiles * n_ntiles of them and n_ntiles + 1 zeroed
// words at a.sync (zeroed here); cooperative: see launch_coresident
int gemm_bf16_rowmin_capacity();
hipError_t gemm_bf16_rowmin_one_launch(GemmArgs a, bool cooperative, hipStream_t s);
// out[n][c] = min_t part[n][t] + bias2[c]; out fp32 or (out_bf16) bf16
hipError_t rowmin_bcast_launch(const float* part, int64_t N, int n_ctiles, const float* bias2,
                               void* out, bool out_bf16, int64_t C, hipStream_t s);

// ---- fp32 fused conv + GroupNorm, one workgroup per (n, 16-channel block)
// (k_fused_gn.hip).  Supported when C_out/G divides 16 and the whole
// T_out fits the workgroup's registers.
struct FusedArgs {
  const float* x;
  const float* w;      // unpacked [C_out, C_in, K]
  const float* bias;
  const float* gamma;
  const float* beta;
  void* out;           // fp32 or (out_bf16) bf16
  float* mean_out;     // [N, G] or nullptr
  float* rstd_out;
  int64_t N, C_in, C_out, T, T_out;
  int32_t K, stride, dilation, pad_left, G;
  float eps;
  int32_t out_bf16;
};
int fused_gn_max_tout(int stride, int K, int dilation);  // 0 if unsupported
bool fused_gn_supported(int64_t C_in, int64_t C_out, int32_t G, int64_t T_out, int stride,
                        int K, int dilation);
hipError_t fused_gn_launch(const FusedArgs& a, hipStream_t s);

// ---- normalisation kernels (k_norm.hip)
// GroupNorm: partials [N, C, n_ttiles] (mean, M2) with tile length tm -> mean/rstd [N, G]
hipError_t gn_merge_launch(const float* part, int64_t N, int64_t C, int64_t L, int32_t G,
                           int32_t n_ttiles, int32_t tm, float eps, float* mean, float* rstd,
                           hipStream_t s);
// GroupNorm statistics straight from y [N, C, L] -> mean/rstd [N, G]: each
// group's values in slices, one workgroup per slice, then a fixed-order merge
// of the slice partials held in `part` (gn_stats_workspace_bytes of it);
// part == nullptr: one workgroup per group, no workspace
size_t gn_stats_workspace_bytes(int64_t N, int64_t C, int64_t L, int32_t G);
hipError_t gn_stats_launch(const float* y, int64_t N, int64_t C, int64_t L, int32_t G,
                           float eps, float* mean, float* rstd, float* part, hipStream_t s);
// Element types of y and out in the passes below (values of enum c1g_dtype):
// fp32 -> fp32, bf16 -> bf16 and fp32 -> bf16 are built; out may equal y.
// out = (y - mean[n,g]) * rstd[n,g] * gamma[c] + beta[c]
hipError_t gn_apply_launch(const void* y, int y_dt, const float* mean, const float* rstd,
                           const float* gamma, const float* beta, void* out, int out_dt,
                           int64_t N, int64_t C, int64_t L, int32_t G, hipStream_t s);
// LayerNorm over channels: partials [N, n_ctiles, L] (mean, M2), tile width tn
hipError_t ln_merge_launch(const float* part, int64_t N, int64_t C, int64_t L,
                           int32_t n_ctiles, int32_t tn, float eps, float* mean, float* rstd,
                           hipStream_t s);
hipError_t ln_apply_launch(const void* y, int y_dt, const float* mean, const float* rstd,
                           const float* gamma, const float* beta, void* out, int out_dt,
                           int64_t N, int64_t C, int64_t L, hipStream_t s);
// Row-min epilogue: z = (y - mean) * rstd * gamma + beta with statistics per
// (n, group) (norm_kind 1), per (n, l) (norm_kind 2) or none (norm_kind 0);
// out[n,c,l] = min_c z[n,c,l] + bias2[c].
hipError_t rowmin_bias_launch(const void* y, int y_dt, const float* mean, const float* rstd,
                              const float* gamma, const float* beta, const float* bias2,
                              void* out, int out_dt, int64_t N, int64_t C, int64_t L,
                              int32_t G, int norm_kind, hipStream_t s);

}  // namespace c1g
