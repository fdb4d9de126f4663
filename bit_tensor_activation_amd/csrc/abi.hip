// extern "C" entry points of libbtq: host-side argument checks, then the
// launchers in calib.hip, select.hip, compress.hip and decompress.hip.
// The contract of each call is documented in include/btq.h.
#include <math.h>

#include "btq.h"
#include "common.hpp"

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

size_t btq_select_workspace_bytes(int64_t P, int64_t H) {
  if (P < 1 || P > kMaxP || H < 1 || H > kMaxH) return 0;
  return (size_t)(P * H) * sizeof(float);   // per-shard widths; the shared score uses H
}

int64_t btq_enc_table_floats(int64_t P, int64_t H, int64_t k) {
  if (P < 1 || P > kMaxP || H < 1 || H > kMaxH || check_k(H, k) != BTQ_OK) return -1;
  return 2 * P * (H - k);
}

int64_t btq_dec_table_floats(int64_t P, int64_t H, int64_t k) {
  if (P < 1 || P > kMaxP || H < 1 || H > kMaxH || check_k(H, k) != BTQ_OK) return -1;
  return (2 * P + 1) * (H - k);
}

int btq_calib_update(const uint16_t* x, int64_t P, int64_t T, int64_t H, float momentum,
                     int first_batch, float* run_min, float* run_max, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int st = check_dims(P, T, H, 1);
  if (st != BTQ_OK) return st;
  if (!x || !run_min || !run_max) return BTQ_ERR_ARG;
  if (!(momentum >= 0.0f && momentum <= 1.0f)) return BTQ_ERR_ARG;   // also rejects NaN
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

int btq_select_outliers(const float* run_min, const float* run_max, int64_t P, int64_t H,
                        int64_t k, float* scale, float* rscale, uint8_t* zero_point,
                        int32_t* outlier_idx, int32_t* fmap, int32_t* cmap, float* enc_table,
                        float* dec_table, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return btq_select_outliers_rule(run_min, run_max, P, H, k, BTQ_SCORE_SUM, scale, rscale,
                                  zero_point, outlier_idx, fmap, cmap, enc_table, dec_table,
                                  workspace, workspace_bytes, stream);
}

int btq_select_outliers_rule(const float* run_min, const float* run_max, int64_t P, int64_t H,
                             int64_t k, int score_rule, float* scale, float* rscale,
                             uint8_t* zero_point, int32_t* outlier_idx, int32_t* fmap,
                             int32_t* cmap, float* enc_table, float* dec_table, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (P < 1 || P > kMaxP || H < 1 || H > kMaxH) return BTQ_ERR_SHAPE;
  if (score_rule != BTQ_SCORE_SUM && score_rule != BTQ_SCORE_MAX) return BTQ_ERR_ARG;
  int st = check_k(H, k);
  if (st != BTQ_OK) return st;
  if (!run_min || !run_max || !scale || !rscale || !zero_point || !fmap) return BTQ_ERR_ARG;
  if ((k > 0 && !outlier_idx) || (k < H && (!cmap || !enc_table || !dec_table)))
    return BTQ_ERR_ARG;
  if (!aligned(run_min, 4) || !aligned(run_max, 4) || !aligned(scale, 4) ||
      !aligned(rscale, 4) || !aligned(outlier_idx, 4) || !aligned(fmap, 4) || !aligned(cmap, 4) ||
      !aligned(enc_table, 4) || !aligned(dec_table, 4))
    return BTQ_ERR_ALIGN;
  const size_t need = btq_select_workspace_bytes(P, H);
  if (!workspace) return BTQ_ERR_ARG;
  if (workspace_bytes < need) return BTQ_ERR_WORKSPACE;
  if (!aligned(workspace, 4)) return BTQ_ERR_ALIGN;
  return hip_status(btq::launch_select(run_min, run_max, P, H, k, scale, rscale, zero_point,
                                       outlier_idx, fmap, cmap, enc_table, dec_table,
                                       (float*)workspace, score_rule == BTQ_SCORE_MAX,
                                       (hipStream_t)stream));
}

int btq_select_outliers_per_shard(const float* run_min, const float* run_max, int64_t P,
                                  int64_t H, int64_t k, float* scale, float* rscale,
                                  uint8_t* zero_point, int32_t* outlier_idx, int32_t* fmap,
                                  int32_t* cmap, float* enc_table, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (P < 1 || P > kMaxP || H < 1 || H > kMaxH) return BTQ_ERR_SHAPE;
  int st = check_k(H, k);
  if (st != BTQ_OK) return st;
  if (!run_min || !run_max || !scale || !rscale || !zero_point || !fmap) return BTQ_ERR_ARG;
  if ((k > 0 && !outlier_idx) || (k < H && (!cmap || !enc_table))) return BTQ_ERR_ARG;
  if (!aligned(run_min, 4) || !aligned(run_max, 4) || !aligned(scale, 4) ||
      !aligned(rscale, 4) || !aligned(outlier_idx, 4) || !aligned(fmap, 4) || !aligned(cmap, 4) ||
      !aligned(enc_table, 4))
    return BTQ_ERR_ALIGN;
  if (!workspace) return BTQ_ERR_ARG;
  if (workspace_bytes < btq_select_workspace_bytes(P, H)) return BTQ_ERR_WORKSPACE;
  if (!aligned(workspace, 4)) return BTQ_ERR_ALIGN;
  return hip_status(btq::launch_select_per_shard(run_min, run_max, P, H, k, scale, rscale,
                                                 zero_point, outlier_idx, fmap, cmap, enc_table,
                                                 (float*)workspace, (hipStream_t)stream));
}

int btq_select_features(const float* run_min, const float* run_max, int64_t P, int64_t H,
                        int64_t k, const int32_t* features, float* scale, float* rscale,
                        uint8_t* zero_point, int32_t* outlier_idx, int32_t* fmap, int32_t* cmap,
                        float* enc_table, float* dec_table, void* stream) {
  if (P < 1 || P > kMaxP || H < 1 || H > kMaxH) return BTQ_ERR_SHAPE;
  int st = check_k(H, k);
  if (st != BTQ_OK) return st;
  if (!run_min || !run_max || !scale || !rscale || !zero_point || !fmap) return BTQ_ERR_ARG;
  if ((k > 0 && (!outlier_idx || !features)) || (k < H && (!cmap || !enc_table || !dec_table)))
    return BTQ_ERR_ARG;
  if (!aligned(run_min, 4) || !aligned(run_max, 4) || !aligned(scale, 4) ||
      !aligned(rscale, 4) || !aligned(outlier_idx, 4) || !aligned(fmap, 4) || !aligned(cmap, 4) ||
      !aligned(enc_table, 4) || !aligned(dec_table, 4) || !aligned(features, 4))
    return BTQ_ERR_ALIGN;
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
                                           outlier_idx, fmap, cmap, enc_table, dec_table, s));
}

namespace {

int compress_common(const uint16_t* x, int64_t P, int64_t T, int64_t H, int64_t k,
                    const float* enc_table, const int32_t* outlier_idx, const int32_t* cmap,
                    uint8_t* packed, int64_t packed_pitch, uint16_t* outliers, bool per_shard,
                    void* stream) {
  int st = check_dims(P, T, H, 0);
  if (st != BTQ_OK) return st;
  st = check_k(H, k);
  if (st != BTQ_OK) return st;
  st = check_pitch(P, T, H, k, packed_pitch);
  if (st != BTQ_OK) return st;
  if ((k > 0 && !outlier_idx) || (k < H && (!cmap || !enc_table))) return BTQ_ERR_ARG;
  if (T > 0 && (!x || (k < H && !packed) || (k > 0 && !outliers))) return BTQ_ERR_ARG;
  if (!aligned(x, 2) || !aligned(enc_table, 4) || !aligned(outlier_idx, 4) ||
      !aligned(cmap, 4) || !aligned(outliers, 2))
    return BTQ_ERR_ALIGN;
  if (T == 0) return BTQ_OK;
  return hip_status(btq::launch_compress(x, P, T, H, k, enc_table, outlier_idx, cmap, packed,
                                         packed_pitch, outliers, per_shard,
                                         (hipStream_t)stream));
}

}  // namespace

int btq_compress_pack(const uint16_t* x, int64_t P, int64_t T, int64_t H, int64_t k,
                      const float* enc_table, const int32_t* outlier_idx, const int32_t* cmap,
                      uint8_t* packed, int64_t packed_pitch, uint16_t* outliers, void* stream) {
  return compress_common(x, P, T, H, k, enc_table, outlier_idx, cmap, packed, packed_pitch,
                         outliers, false, stream);
}

int btq_compress_pack_per_shard(const uint16_t* x, int64_t P, int64_t T, int64_t H, int64_t k,
                                const float* enc_table, const int32_t* outlier_idx,
                                const int32_t* cmap, uint8_t* packed, int64_t packed_pitch,
                                uint16_t* outliers, void* stream) {
  return compress_common(x, P, T, H, k, enc_table, outlier_idx, cmap, packed, packed_pitch,
                         outliers, true, stream);
}

namespace {

int decompress_common(const uint8_t* packed, int64_t packed_pitch, const uint16_t* outliers,
                      int64_t P, int64_t T, int64_t H, int64_t k, const float* dec_table,
                      const int32_t* outlier_idx, const int32_t* cmap, void* y, bool bf16,
                      void* stream) {
  int st = check_dims(P, T, H, 0);
  if (st != BTQ_OK) return st;
  st = check_k(H, k);
  if (st != BTQ_OK) return st;
  st = check_pitch(P, T, H, k, packed_pitch);
  if (st != BTQ_OK) return st;
  if ((k > 0 && !outlier_idx) || (k < H && (!cmap || !dec_table))) return BTQ_ERR_ARG;
  if (T > 0 && (!y || (k < H && !packed) || (k > 0 && !outliers))) return BTQ_ERR_ARG;
  if (!aligned(outliers, 2) || !aligned(dec_table, 4) || !aligned(outlier_idx, 4) ||
      !aligned(cmap, 4) || !aligned(y, bf16 ? 2 : 4))
    return BTQ_ERR_ALIGN;
  if (T == 0) return BTQ_OK;
  return hip_status(btq::launch_decompress(packed, packed_pitch, outliers, P, T, H, k, dec_table,
                                           outlier_idx, cmap, y, bf16, (hipStream_t)stream));
}

}  // namespace

int btq_decompress_reduce(const uint8_t* packed, int64_t packed_pitch, const uint16_t* outliers,
                          int64_t P, int64_t T, int64_t H, int64_t k, const float* dec_table,
                          const int32_t* outlier_idx, const int32_t* cmap, float* y,
                          void* stream) {
  return decompress_common(packed, packed_pitch, outliers, P, T, H, k, dec_table, outlier_idx,
                           cmap, y, false, stream);
}

int btq_decompress_reduce_bf16(const uint8_t* packed, int64_t packed_pitch,
                               const uint16_t* outliers, int64_t P, int64_t T, int64_t H,
                               int64_t k, const float* dec_table, const int32_t* outlier_idx,
                               const int32_t* cmap, uint16_t* y, void* stream) {
  return decompress_common(packed, packed_pitch, outliers, P, T, H, k, dec_table, outlier_idx,
                           cmap, y, true, stream);
}

int btq_decompress_reduce_per_shard(const uint8_t* packed, int64_t packed_pitch,
                                    const uint16_t* outliers, int64_t P, int64_t T, int64_t H,
                                    int64_t k, const float* scale, const uint8_t* zero_point,
                                    const int32_t* fmap, float* y, void* stream) {
  int st = check_dims(P, T, H, 0);
  if (st != BTQ_OK) return st;
  st = check_k(H, k);
  if (st != BTQ_OK) return st;
  st = check_pitch(P, T, H, k, packed_pitch);
  if (st != BTQ_OK) return st;
  if (!scale || !zero_point || !fmap) return BTQ_ERR_ARG;
  if (T > 0 && (!y || (k < H && !packed) || (k > 0 && !outliers))) return BTQ_ERR_ARG;
  if (!aligned(outliers, 2) || !aligned(scale, 4) || !aligned(fmap, 4) || !aligned(y, 4))
    return BTQ_ERR_ALIGN;
  if (T == 0) return BTQ_OK;
  return hip_status(btq::launch_decompress_sets(packed, packed_pitch, outliers, P, T, H, k, scale,
                                                zero_point, fmap, y, (hipStream_t)stream));
}

const char* btq_status_str(int status) {
  switch (status) {
    case BTQ_OK: return "ok";
    case BTQ_ERR_ARG: return "invalid argument (null pointer or momentum outside [0,1])";
    case BTQ_ERR_SHAPE: return "invalid shape (P, T, H or k out of range)";
    case BTQ_ERR_ALIGN: return "pointer not aligned to its element type";
    case BTQ_ERR_WORKSPACE: return "workspace too small";
    case BTQ_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown btq status";
  }
}

const char* btq_version(void) { return "0.2.0"; }

}  // extern "C"
