// extern "C" entry points of libbtq: host-side argument checks, then the
// launchers in calib.hip, select.hip, compress.hip and decompress.hip.
// The contract of each call is documented in include/btq.h.
#include <math.h>

#include <mutex>

#include "btq.h"
#include "common.hpp"

// Scratch of btq_calib_update_noalloc: a file-scope device array, one copy
// on each GPU the library runs on, held until the process ends. Host code
// never uses this name as an address (on the host it is only a stand-in);
// it passes the device address that hipGetSymbolAddress returns for the
// current device.
static __device__ __align__(256) float scratch[BTQ_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int64_t kMaxP = 65535;
constexpr int64_t kMaxH = int64_t(1) << 30;
constexpr int64_t kMaxElems = int64_t(1) << 62;

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// P in [1,kMaxP], H in [1,kMaxH], T >= t_min, P*T*H < 2^62.
int check_dims(int64_t P, int64_t T, int64_t H, int64_t t_min) {
  if (P < 1 || P > kMaxP || H < 1 || H > kMaxH || T < t_min) return BTQ_ERR_SHAPE;
  if (T > 0 && T > kMaxElems / (P * H)) return BTQ_ERR_SHAPE;
  return BTQ_OK;
}

int check_k(int64_t H, int64_t k) { return (k < 0 || k > H) ? BTQ_ERR_SHAPE : BTQ_OK; }

int hip_status(hipError_t e) { return e == hipSuccess ? BTQ_OK : BTQ_ERR_HIP; }

// Packed row pitch: at least the row's code bytes, and P*T*pitch < 2^62.
int check_pitch(int64_t P, int64_t T, int64_t H, int64_t k, int64_t pitch) {
  if (pitch < (H - k + 1) / 2 || pitch > kMaxElems) return BTQ_ERR_SHAPE;
  if (T > 0 && pitch > 0 && T > kMaxElems / (P * pitch)) return BTQ_ERR_SHAPE;
  return BTQ_OK;
}

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];   // `scratch` on each device, looked up once

// The current device's address of `scratch`: looked up on the first call on
// that device, with it current, and kept.
int scratch_address(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BTQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return BTQ_ERR_HIP;
    }
    g_scratch_addr[dev] = p;
  }
  *out = static_cast<float*>(g_scratch_addr[dev]);
  return BTQ_OK;
}

}  // namespace

extern "C" {

int64_t btq_packed_row_bytes(int64_t H, int64_t k) {
  if (H < 1 || k < 0 || k > H) return -1;
  return (H - k + 1) / 2;
}

int64_t btq_packed_pitch(int64_t H, int64_t k) {
  const int64_t b = btq_packed_row_bytes(H, k);
  return b < 0 ? -1 : (b + 127) / 128 * 128;
}

size_t btq_calib_workspace_bytes(int64_t P, int64_t T, int64_t H) {
  if (check_dims(P, T, H, 1) != BTQ_OK) return 0;
  const btq::CalibPlan plan = btq::calib_plan(P, T, H);
  return (size_t)(2 * plan.nchunk * P * H) * sizeof(float);
}

size_t btq_select_workspace_bytes(int64_t P, int64_t H, int64_t k) {
  if (P < 1 || P > kMaxP || H < 1 || H > kMaxH || check_k(H, k) != BTQ_OK) return 0;
  return (size_t)(P * H) * sizeof(float);   // per-shard widths; the shared score uses H
}

int btq_calib_update(const uint16_t* x, int64_t P, int64_t T, int64_t H, float momentum,
                     int first_batch, float* run_min, float* run_max, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int st = check_dims(P, T, H, 1);
  if (st != BTQ_OK) return st;
  if (!x || !run_min || !run_max) return BTQ_ERR_ARG;
  if (!(momentum >= 0.0f && momentum < 1.0f)) return BTQ_ERR_ARG;   // also rejects NaN
  if (!aligned(x, 2) || !aligned(run_min, 4) || !aligned(run_max, 4)) return BTQ_ERR_ALIGN;
  const size_t need = btq_calib_workspace_bytes(P, T, H);
  if (need > 0 && !workspace) return BTQ_ERR_ARG;
  if (workspace_bytes < need) return BTQ_ERR_WORKSPACE;
  if (!aligned(workspace, 4)) return BTQ_ERR_ALIGN;
  const float a = momentum;
  const float c = 1.0f - a;   // one fp32 subtraction
  return hip_status(btq::launch_calib(x, P, T, H, a, c, first_batch != 0, run_min, run_max,
                                      (float*)workspace, (hipStream_t)stream));
}

int btq_calib_update_noalloc(const uint16_t* x, int64_t P, int64_t T, int64_t H, float momentum,
                             int first_batch, float* run_min, float* run_max, void* stream) {
  int st = check_dims(P, T, H, 1);
  if (st != BTQ_OK) return st;
  if (!x || !run_min || !run_max) return BTQ_ERR_ARG;
  if (!(momentum >= 0.0f && momentum < 1.0f)) return BTQ_ERR_ARG;   // also rejects NaN
  if (!aligned(x, 2) || !aligned(run_min, 4) || !aligned(run_max, 4)) return BTQ_ERR_ALIGN;
  // the same kernels with as many token chunks as the scratch holds partials for
  const btq::CalibPlan plan =
      btq::calib_plan_capped(P, T, H, (int64_t)(BTQ_NOALLOC_SCRATCH_BYTES / sizeof(float)));
  if (plan.nchunk < 1) return BTQ_ERR_SCRATCH;
  float* ws = nullptr;
  st = scratch_address(&ws);
  if (st != BTQ_OK) return st;
  const float a = momentum;
  const float c = 1.0f - a;
  return hip_status(btq::launch_calib_plan(x, P, T, H, a, c, first_batch != 0, run_min, run_max,
                                           ws, plan, (hipStream_t)stream));
}

namespace {

// Shared checks of the selection calls' parameter and map outputs.
int check_select_outputs(const float* run_min, const float* run_max, int64_t P, int64_t H,
                         int64_t k, const float* scale, const float* rscale,
                         const uint8_t* zero_point, const int32_t* outlier_idx,
                         const int32_t* fmap, const int32_t* cmap) {
  if (P < 1 || P > kMaxP || H < 1 || H > kMaxH) return BTQ_ERR_SHAPE;
  int st = check_k(H, k);
  if (st != BTQ_OK) return st;
  if (!run_min || !run_max || !scale || !rscale || !zero_point || !fmap) return BTQ_ERR_ARG;
  if ((k > 0 && !outlier_idx) || (k < H && !cmap)) return BTQ_ERR_ARG;
  if (!aligned(run_min, 4) || !aligned(run_max, 4) || !aligned(scale, 4) ||
      !aligned(rscale, 4) || !aligned(outlier_idx, 4) || !aligned(fmap, 4) || !aligned(cmap, 4))
    return BTQ_ERR_ALIGN;
  return BTQ_OK;
}

int check_workspace(int64_t P, int64_t H, int64_t k, const void* workspace, size_t bytes) {
  if (!workspace) return BTQ_ERR_ARG;
  if (bytes < btq_select_workspace_bytes(P, H, k)) return BTQ_ERR_WORKSPACE;
  if (!aligned(workspace, 4)) return BTQ_ERR_ALIGN;
  return BTQ_OK;
}

}  // namespace

int btq_select_outliers(const float* run_min, const float* run_max, int64_t P, int64_t H,
                        int64_t k, float* scale, float* rscale, uint8_t* zero_point,
                        int32_t* outlier_idx, int32_t* fmap, int32_t* cmap, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return btq_select_outliers_rule(run_min, run_max, P, H, k, BTQ_SCORE_SUM, scale, rscale,
                                  zero_point, outlier_idx, fmap, cmap, workspace,
                                  workspace_bytes, stream);
}

int btq_select_outliers_rule(const float* run_min, const float* run_max, int64_t P, int64_t H,
                             int64_t k, int score_rule, float* scale, float* rscale,
                             uint8_t* zero_point, int32_t* outlier_idx, int32_t* fmap,
                             int32_t* cmap, void* workspace, size_t workspace_bytes,
                             void* stream) {
  int st = check_select_outputs(run_min, run_max, P, H, k, scale, rscale, zero_point, outlier_idx,
                                fmap, cmap);
  if (st != BTQ_OK) return st;
  if (score_rule != BTQ_SCORE_SUM && score_rule != BTQ_SCORE_MAX) return BTQ_ERR_ARG;
  st = check_workspace(P, H, k, workspace, workspace_bytes);
  if (st != BTQ_OK) return st;
  return hip_status(btq::launch_select(run_min, run_max, P, H, k, scale, rscale, zero_point,
                                       outlier_idx, fmap, cmap, (float*)workspace,
                                       score_rule == BTQ_SCORE_MAX, (hipStream_t)stream));
}

int btq_select_outliers_per_shard(const float* run_min, const float* run_max, int64_t P,
                                  int64_t H, int64_t k, float* scale, float* rscale,
                                  uint8_t* zero_point, int32_t* outlier_idx, int32_t* fmap,
                                  int32_t* cmap, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  int st = check_select_outputs(run_min, run_max, P, H, k, scale, rscale, zero_point, outlier_idx,
                                fmap, cmap);
  if (st != BTQ_OK) return st;
  st = check_workspace(P, H, k, workspace, workspace_bytes);
  if (st != BTQ_OK) return st;
  return hip_status(btq::launch_select_per_shard(run_min, run_max, P, H, k, scale, rscale,
                                                 zero_point, outlier_idx, fmap, cmap,
                                                 (float*)workspace, (hipStream_t)stream));
}

int btq_select_features(const float* run_min, const float* run_max, int64_t P, int64_t H,
                        int64_t k, const int32_t* features, float* scale, float* rscale,
                        uint8_t* zero_point, int32_t* outlier_idx, int32_t* fmap, int32_t* cmap,
                        void* stream) {
  int st = check_select_outputs(run_min, run_max, P, H, k, scale, rscale, zero_point, outlier_idx,
                                fmap, cmap);
  if (st != BTQ_OK) return st;
  if (k > 0 && !features) return BTQ_ERR_ARG;
  if (!aligned(features, 4)) return BTQ_ERR_ALIGN;
  for (int64_t i = 0; i < k; ++i) {   // distinct, ascending, inside [0, H)
    const int64_t h = features[i];
    if (h < 0 || h >= H || (i > 0 && h <= features[i - 1])) return BTQ_ERR_ARG;
  }
  const hipStream_t s = (hipStream_t)stream;
  if (k > 0) {
    const hipError_t e = hipMemcpyAsync(outlier_idx, features, (size_t)k * sizeof(int32_t),
                                        hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return BTQ_ERR_HIP;
  }
  return hip_status(btq::launch_select_set(run_min, run_max, P, H, k, scale, rscale, zero_point,
                                           outlier_idx, fmap, cmap, s));
}

int btq_compress_pack_ex(const uint16_t* x, int64_t P, int64_t T, int64_t H, int64_t k,
                         const float* rscale, const uint8_t* zero_point,
                         const int32_t* outlier_idx, const int32_t* cmap, int sets,
                         uint8_t* packed, int64_t packed_pitch, uint16_t* outliers,
                         void* stream) {
  int st = check_dims(P, T, H, 0);
  if (st != BTQ_OK) return st;
  st = check_k(H, k);
  if (st != BTQ_OK) return st;
  st = check_pitch(P, T, H, k, packed_pitch);
  if (st != BTQ_OK) return st;
  if (sets != BTQ_SETS_SHARED && sets != BTQ_SETS_PER_SHARD) return BTQ_ERR_ARG;
  if (!rscale || !zero_point || (k > 0 && !outlier_idx) || (k < H && !cmap)) return BTQ_ERR_ARG;
  if (T > 0 && (!x || (k < H && !packed) || (k > 0 && !outliers))) return BTQ_ERR_ARG;
  if (!aligned(x, 2) || !aligned(rscale, 4) || !aligned(outlier_idx, 4) || !aligned(cmap, 4) ||
      !aligned(outliers, 2))
    return BTQ_ERR_ALIGN;
  if (T == 0) return BTQ_OK;
  return hip_status(btq::launch_compress(x, P, T, H, k, rscale, zero_point, outlier_idx, cmap,
                                         packed, packed_pitch, outliers,
                                         sets == BTQ_SETS_PER_SHARD, (hipStream_t)stream));
}

int btq_compress_pack(const uint16_t* x, int64_t P, int64_t T, int64_t H, int64_t k,
                      const float* rscale, const uint8_t* zero_point, const int32_t* outlier_idx,
                      const int32_t* cmap, uint8_t* packed, uint16_t* outliers, void* stream) {
  return btq_compress_pack_ex(x, P, T, H, k, rscale, zero_point, outlier_idx, cmap,
                              BTQ_SETS_SHARED, packed, btq_packed_row_bytes(H, k), outliers,
                              stream);
}

int btq_compress_pack_per_shard(const uint16_t* x, int64_t P, int64_t T, int64_t H, int64_t k,
                                const float* rscale, const uint8_t* zero_point,
                                const int32_t* outlier_idx, const int32_t* cmap, uint8_t* packed,
                                uint16_t* outliers, void* stream) {
  return btq_compress_pack_ex(x, P, T, H, k, rscale, zero_point, outlier_idx, cmap,
                              BTQ_SETS_PER_SHARD, packed, btq_packed_row_bytes(H, k), outliers,
                              stream);
}

int btq_decompress_reduce_ex(const uint8_t* packed, int64_t packed_pitch,
                             const uint16_t* outliers, int64_t P, int64_t T, int64_t H, int64_t k,
                             const float* scale, const uint8_t* zero_point, const int32_t* fmap,
                             int sets, void* y, int y_type, void* stream) {
  int st = check_dims(P, T, H, 0);
  if (st != BTQ_OK) return st;
  st = check_k(H, k);
  if (st != BTQ_OK) return st;
  st = check_pitch(P, T, H, k, packed_pitch);
  if (st != BTQ_OK) return st;
  if (sets != BTQ_SETS_SHARED && sets != BTQ_SETS_PER_SHARD) return BTQ_ERR_ARG;
  if (y_type != BTQ_Y_F32 && y_type != BTQ_Y_BF16) return BTQ_ERR_ARG;
  if (!scale || !zero_point || !fmap) return BTQ_ERR_ARG;
  if (T > 0 && (!y || (k < H && !packed) || (k > 0 && !outliers))) return BTQ_ERR_ARG;
  const bool bf16 = y_type == BTQ_Y_BF16;
  if (!aligned(outliers, 2) || !aligned(scale, 4) || !aligned(fmap, 4) ||
      !aligned(y, bf16 ? 2 : 4))
    return BTQ_ERR_ALIGN;
  if (T == 0) return BTQ_OK;
  return hip_status(btq::launch_decompress(packed, packed_pitch, outliers, P, T, H, k, scale,
                                           zero_point, fmap, sets == BTQ_SETS_PER_SHARD, y, bf16,
                                           (hipStream_t)stream));
}

int btq_decompress_reduce(const uint8_t* packed, const uint16_t* outliers, int64_t P, int64_t T,
                          int64_t H, int64_t k, const float* scale, const uint8_t* zero_point,
                          const int32_t* fmap, float* y, void* stream) {
  return btq_decompress_reduce_ex(packed, btq_packed_row_bytes(H, k), outliers, P, T, H, k, scale,
                                  zero_point, fmap, BTQ_SETS_SHARED, y, BTQ_Y_F32, stream);
}

int btq_decompress_reduce_bf16(const uint8_t* packed, const uint16_t* outliers, int64_t P,
                               int64_t T, int64_t H, int64_t k, const float* scale,
                               const uint8_t* zero_point, const int32_t* fmap, uint16_t* y,
                               void* stream) {
  return btq_decompress_reduce_ex(packed, btq_packed_row_bytes(H, k), outliers, P, T, H, k, scale,
                                  zero_point, fmap, BTQ_SETS_SHARED, y, BTQ_Y_BF16, stream);
}

int btq_decompress_reduce_per_shard(const uint8_t* packed, const uint16_t* outliers, int64_t P,
                                    int64_t T, int64_t H, int64_t k, const float* scale,
                                    const uint8_t* zero_point, const int32_t* fmap, float* y,
                                    void* stream) {
  return btq_decompress_reduce_ex(packed, btq_packed_row_bytes(H, k), outliers, P, T, H, k, scale,
                                  zero_point, fmap, BTQ_SETS_PER_SHARD, y, BTQ_Y_F32, stream);
}

const char* btq_status_str(int status) {
  switch (status) {
    case BTQ_OK: return "ok";
    case BTQ_ERR_ARG: return "invalid argument (null pointer, unknown option, or momentum outside [0,1))";
    case BTQ_ERR_SHAPE: return "invalid shape (P, T, H, k or the packed pitch out of range)";
    case BTQ_ERR_ALIGN: return "pointer not aligned to its element type";
    case BTQ_ERR_WORKSPACE: return "workspace too small";
    case BTQ_ERR_HIP: return "HIP call failed";
    case BTQ_ERR_SCRATCH:
      return "P*H too large for the no-alloc scratch (2*P*H*4 bytes must fit BTQ_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown btq status";
  }
}

const char* btq_version(void) { return "0.3.0"; }

}  // extern "C"
