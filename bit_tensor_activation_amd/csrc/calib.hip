// Calibration statistics: per-(shard, feature) batch min/max over the token
// axis, then the moving-average update of the running extremes.
//
// Method: "Revolutionizing LLM Inference: The Power of Efficient Low-Bit
// Communication", section "The Hybrid Quantization Algorithm", Calibration
// bullet (moving averages of the minimum and maximum observed on each
// device).
//
// Two kernels. The first reduces column strips of 512 features over a chunk
// of tokens. Each lane streams 16-byte loads of 8 bf16 values and keeps 8
// running min/max pairs, and the 4 waves of a block combine through LDS.
// The result goes to a per-chunk partial array in the workspace. The second
// kernel folds the chunks (4 waves per 64 columns) and applies the EMA.
// min/max are exact and do not depend on order, so the split of the token
// axis cannot change the result.
#include <float.h>

#include "common.hpp"

namespace btq {

constexpr int kCalWaves = 4;
constexpr int kCalCols = kWave * 8;   // 512 features per block

template <bool kVec>
__global__ __launch_bounds__(256) void calib_partial_kernel(
    const uint16_t* __restrict__ x, int64_t T, int64_t H, int64_t rows_per_chunk,
    float* __restrict__ pmin, float* __restrict__ pmax, int64_t P) {
  __shared__ float smin[kCalWaves][kCalCols];
  __shared__ float smax[kCalWaves][kCalCols];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int64_t h0 = (int64_t)blockIdx.x * kCalCols;
  const int64_t p = blockIdx.y;
  const int64_t chunk = blockIdx.z;
  const int64_t t0 = chunk * rows_per_chunk;
  const int64_t t1 = min(T, t0 + rows_per_chunk);
  const uint16_t* __restrict__ xs = x + p * T * H;

  float mn[8], mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mn[e] = INFINITY;
    mx[e] = -INFINITY;
  }
  if (kVec) {
    // lane owns features h0 + 8*lane + e (one 16-byte load per token)
    const int64_t hl = h0 + 8 * lane;
    if (hl < H) {
#pragma unroll 4
      for (int64_t t = t0 + wave; t < t1; t += kCalWaves) {
        const uint4 v = *reinterpret_cast<const uint4*>(xs + t * H + hl);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = __uint_as_float(w[i] << 16);
          const float hi = __uint_as_float(w[i] & 0xFFFF0000u);
          mn[2 * i] = fminf(mn[2 * i], lo);
          mx[2 * i] = fmaxf(mx[2 * i], lo);
          mn[2 * i + 1] = fminf(mn[2 * i + 1], hi);
          mx[2 * i + 1] = fmaxf(mx[2 * i + 1], hi);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      smin[wave][8 * lane + e] = mn[e];
      smax[wave][8 * lane + e] = mx[e];
    }
  } else {
    // lane owns features h0 + lane + 64*e (2-byte loads, any H)
    for (int64_t t = t0 + wave; t < t1; t += kCalWaves) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t h = h0 + lane + kWave * e;
        if (h < H) {
          const float f = bf16_to_f32(xs[t * H + h]);
          mn[e] = fminf(mn[e], f);
          mx[e] = fmaxf(mx[e], f);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      smin[wave][lane + kWave * e] = mn[e];
      smax[wave][lane + kWave * e] = mx[e];
    }
  }
  lds_barrier();
  for (int col = threadIdx.x; col < kCalCols; col += blockDim.x) {
    const int64_t h = h0 + col;
    if (h >= H) continue;
    float a = smin[0][col], b = smax[0][col];
#pragma unroll
    for (int w = 1; w < kCalWaves; ++w) {
      a = fminf(a, smin[w][col]);
      b = fmaxf(b, smax[w][col]);
    }
    const int64_t o = (chunk * P + p) * H + h;
    pmin[o] = a;
    pmax[o] = b;
  }
}

// Fold the chunk partials and apply the moving average:
//   first batch: run = batch;  otherwise run = fl(fl(a*run) + fl(c*batch)).
// A block takes 64 columns of (shard, feature). Its 4 waves fold every 4th
// chunk each (a wave reads 64 consecutive floats per chunk), with several
// chunks in flight per thread, and meet in LDS. min/max are exact and
// order-free, so the grouping cannot change the result.
constexpr int kFoldCols = kWave;
constexpr int kFoldGroups = 4;

__global__ __launch_bounds__(256) void calib_combine_kernel(
    const float* __restrict__ pmin, const float* __restrict__ pmax, int64_t nchunk, int64_t PH,
    float a, float c, int first, float* __restrict__ run_min, float* __restrict__ run_max) {
  __shared__ float smin[kFoldGroups][kFoldCols];
  __shared__ float smax[kFoldGroups][kFoldCols];
  const int col = threadIdx.x & (kFoldCols - 1);
  const int g = threadIdx.x / kFoldCols;
  const int64_t i = (int64_t)blockIdx.x * kFoldCols + col;
  float m = INFINITY, M = -INFINITY;
  if (i < PH) {
#pragma unroll 4
    for (int64_t ch = g; ch < nchunk; ch += kFoldGroups) {
      m = fminf(m, pmin[ch * PH + i]);
      M = fmaxf(M, pmax[ch * PH + i]);
    }
  }
  smin[g][col] = m;
  smax[g][col] = M;
  __syncthreads();
  if (g != 0 || i >= PH) return;
#pragma unroll
  for (int w = 1; w < kFoldGroups; ++w) {
    m = fminf(m, smin[w][col]);
    M = fmaxf(M, smax[w][col]);
  }
  if (first) {
    run_min[i] = m;
    run_max[i] = M;
  } else {
    run_min[i] = __fadd_rn(__fmul_rn(a, run_min[i]), __fmul_rn(c, m));
    run_max[i] = __fadd_rn(__fmul_rn(a, run_max[i]), __fmul_rn(c, M));
  }
}

CalibPlan calib_plan(int64_t P, int64_t T, int64_t H) {
  // Aim for ~2048 blocks in flight (8 per CU on 256 CUs), with at least 16
  // tokens per chunk so that the partial arrays stay small next to x.
  const int64_t colblocks = (H + kCalCols - 1) / kCalCols;
  const int64_t per_chunk = P * colblocks;
  int64_t nchunk = (2048 + per_chunk - 1) / per_chunk;
  const int64_t max_chunks = (T + 15) / 16;
  if (nchunk > max_chunks) nchunk = max_chunks;
  if (nchunk < 1) nchunk = 1;
  CalibPlan plan;
  plan.rows_per_chunk = (T + nchunk - 1) / nchunk;
  plan.nchunk = (T + plan.rows_per_chunk - 1) / plan.rows_per_chunk;
  return plan;
}

CalibPlan calib_plan_capped(int64_t P, int64_t T, int64_t H, int64_t max_ws_floats) {
  CalibPlan plan = calib_plan(P, T, H);
  const int64_t fit = max_ws_floats / (2 * P * H);   // chunks whose partials fit
  if (fit < 1) {
    plan.nchunk = 0;
    plan.rows_per_chunk = 0;
    return plan;
  }
  if (plan.nchunk > fit) {
    plan.rows_per_chunk = (T + fit - 1) / fit;
    plan.nchunk = (T + plan.rows_per_chunk - 1) / plan.rows_per_chunk;
  }
  return plan;
}

hipError_t launch_calib(const uint16_t* x, int64_t P, int64_t T, int64_t H, float a, float c,
                        int first, float* run_min, float* run_max, float* ws, hipStream_t s) {
  return launch_calib_plan(x, P, T, H, a, c, first, run_min, run_max, ws, calib_plan(P, T, H), s);
}

hipError_t launch_calib_plan(const uint16_t* x, int64_t P, int64_t T, int64_t H, float a, float c,
                             int first, float* run_min, float* run_max, float* ws,
                             const CalibPlan& plan, hipStream_t s) {
  float* pmin = ws;
  float* pmax = ws + plan.nchunk * P * H;
  const dim3 grid((unsigned)((H + kCalCols - 1) / kCalCols), (unsigned)P, (unsigned)plan.nchunk);
  const bool vec = (H % 8 == 0) && ((uintptr_t)x % 16 == 0);
  if (vec)
    calib_partial_kernel<true><<<grid, 256, 0, s>>>(x, T, H, plan.rows_per_chunk, pmin, pmax, P);
  else
    calib_partial_kernel<false><<<grid, 256, 0, s>>>(x, T, H, plan.rows_per_chunk, pmin, pmax, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t PH = P * H;
  calib_combine_kernel<<<(unsigned)((PH + kFoldCols - 1) / kFoldCols), 256, 0, s>>>(
      pmin, pmax, plan.nchunk, PH, a, c, first, run_min, run_max);
  return hipGetLastError();
}

}  // namespace btq
