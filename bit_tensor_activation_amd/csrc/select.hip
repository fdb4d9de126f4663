// Selection: per-(shard, feature) 4-bit parameters, the per-feature range
// score, the top-k BF16 feature set and the maps between features and
// message slots.
//
// Method: "Revolutionizing LLM Inference: The Power of Efficient Low-Bit
// Communication", section "The Hybrid Quantization Algorithm": Calibration
// bullet (parameters per feature from the running extremes) and Selection
// bullet (rank features by quantization range, reserve a number for BF16).
//
// It runs once after calibration, on P*H values, so it is built for exact
// determinism, not speed. qparams_kernel uses one thread per feature. Then
// a single 1024-thread block finds the k-th largest 64-bit key
// (score bits << 32 | ~h) by an 8-pass MSB radix select over LDS
// histograms. The keys are unique, so the selected set is exactly
// {key >= k-th key}, with ties in score going to the lower h. A ballot +
// popcount scan over h in ascending order then writes idx, fmap and cmap.
//
// Variants of the ranking (other readings of how per-device ranges rank
// features): the score may be the widest shard's range instead of the sum;
// one set per shard runs the top-k block once per shard on that shard's
// widths (grid P); and a set
// given by the caller skips the ranking, with set_maps_kernel finding
// membership by binary search and sharing the ordered compaction.
#include <float.h>

#include "common.hpp"

namespace btq {

__global__ __launch_bounds__(256) void qparams_kernel(
    const float* __restrict__ run_min, const float* __restrict__ run_max, int64_t P, int64_t H,
    float* __restrict__ scale, float* __restrict__ rscale, uint8_t* __restrict__ zp,
    float* __restrict__ score, bool score_max, float* __restrict__ width) {
  const int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= H) return;
  float sc = 0.0f;
  for (int64_t p = 0; p < P; ++p) {
    const int64_t i = p * H + h;
    const float lo = fminf(run_min[i], 0.0f);   // the grid always holds 0
    const float hi = fmaxf(run_max[i], 0.0f);
    const float w = __fsub_rn(hi, lo);
    float s = __fdiv_rn(w, 15.0f);
    if (s < FLT_MIN) s = 1.0f;                  // zero or subnormal range
    const float r = __fdiv_rn(1.0f, s);
    float z = rintf(__fdiv_rn(-lo, s));
    z = fminf(fmaxf(z, 0.0f), 15.0f);
    scale[i] = s;
    rscale[i] = r;
    zp[i] = (uint8_t)z;
    if (width) width[i] = w;
    sc = score_max ? fmaxf(sc, w) : __fadd_rn(sc, w);   // p ascending, from +0
  }
  if (score) score[h] = sc;
}

// Scores are non-negative widths, their sums or their maxima, so their bit
// patterns order like their values once -0 is made +0 (a width of -0 ranks
// equal to +0, as its value does). The low word ranks lower h higher.
__device__ __forceinline__ unsigned long long rank_key(float s, int64_t h) {
  return ((unsigned long long)__float_as_uint(__fadd_rn(s, 0.0f)) << 32) |
         (unsigned long long)(0xFFFFFFFFu - (uint32_t)h);
}

constexpr int kSelThreads = 1024;

// Ordered compaction in ascending h, one 1024-thread block: i = number of
// selected features below h, j = h - i. Selected h gets fmap = -1 - i (and
// idx[i] = h when idx is given), the others fmap = j and cmap[j] = h. The
// guards keep every write in bounds even if sel() picks a wrong count.
template <class Sel>
__device__ void write_maps(Sel sel, int64_t H, int64_t k, int32_t* __restrict__ idx,
                           int32_t* __restrict__ fmap, int32_t* __restrict__ cmap,
                           unsigned* wave_cnt) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int64_t sel_base = 0;
  for (int64_t base = 0; base < H; base += kSelThreads) {
    const int64_t h = base + tid;
    const bool in = h < H;
    const bool f = in && sel(h);
    const unsigned long long b = __ballot(f);
    if (lane == 0) wave_cnt[wave] = (unsigned)__popcll(b);
    __syncthreads();
    int64_t wp = 0, tot = 0;
    for (int w = 0; w < kSelThreads / kWave; ++w) {
      const unsigned n = wave_cnt[w];
      if (w < wave) wp += n;
      tot += n;
    }
    if (in) {
      const int64_t i = sel_base + wp + __popcll(b & below);
      const int64_t j = h - i;
      if (f) {
        if (i < k) {
          if (idx) idx[i] = (int32_t)h;
          fmap[h] = (int32_t)(-1 - i);
        }
      } else if (j < H - k) {
        cmap[j] = (int32_t)h;
        fmap[h] = (int32_t)j;
      }
    }
    sel_base += tot;
    __syncthreads();
  }
}

// Block b ranks score row b: one block for the shared set, one per shard for
// per-shard sets (rows of score, idx, fmap and cmap are H, k, H and H-k long).
__global__ __launch_bounds__(kSelThreads) void topk_maps_kernel(
    const float* __restrict__ score, int64_t H, int64_t k, int32_t* __restrict__ idx,
    int32_t* __restrict__ fmap, int32_t* __restrict__ cmap) {
  score += (int64_t)blockIdx.x * H;
  idx += (int64_t)blockIdx.x * k;
  fmap += (int64_t)blockIdx.x * H;
  cmap += (int64_t)blockIdx.x * (H - k);
  __shared__ unsigned hist[256];
  __shared__ unsigned long long s_prefix;
  __shared__ unsigned long long s_rem;
  __shared__ unsigned wave_cnt[kSelThreads / kWave];
  const int tid = threadIdx.x;
  const bool none = (k == 0);
  const bool all = (k == H);

  unsigned long long kth = 0;
  if (!none && !all) {
    unsigned long long prefix = 0, mask = 0, rem = (unsigned long long)k;
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      for (int64_t h = tid; h < H; h += kSelThreads) {
        const unsigned long long key = rank_key(score[h], h);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xFF], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        unsigned long long cum = 0;
        for (int d = 255; d >= 0; --d) {
          const unsigned long long n = hist[d];
          if (cum + n >= rem) {
            prefix |= (unsigned long long)d << shift;
            rem -= cum;
            break;
          }
          cum += n;
        }
        s_prefix = prefix;
        s_rem = rem;
      }
      __syncthreads();
      prefix = s_prefix;
      rem = s_rem;
      mask |= 0xFFull << shift;
    }
    kth = prefix;   // the k-th largest key itself
  }

  write_maps(
      [&](int64_t h) { return all || (!none && rank_key(score[h], h) >= kth); }, H, k, idx, fmap,
      cmap, wave_cnt);
}

// Maps for a BF16 set given in ascending h (checked on the host): membership
// by binary search over idx.
__global__ __launch_bounds__(kSelThreads) void set_maps_kernel(const int32_t* __restrict__ idx,
                                                               int64_t H, int64_t k,
                                                               int32_t* __restrict__ fmap,
                                                               int32_t* __restrict__ cmap) {
  __shared__ unsigned wave_cnt[kSelThreads / kWave];
  write_maps(
      [&](int64_t h) {
        int64_t lo = 0, hi = k;   // first i with idx[i] >= h
        while (lo < hi) {
          const int64_t mid = (lo + hi) >> 1;
          if (idx[mid] < h) lo = mid + 1; else hi = mid;
        }
        return lo < k && idx[lo] == h;
      },
      H, k, nullptr, fmap, cmap, wave_cnt);
}

hipError_t launch_select(const float* run_min, const float* run_max, int64_t P, int64_t H,
                         int64_t k, float* scale, float* rscale, uint8_t* zp, int32_t* idx,
                         int32_t* fmap, int32_t* cmap, float* ws_score, bool score_max,
                         hipStream_t s) {
  qparams_kernel<<<(unsigned)((H + 255) / 256), 256, 0, s>>>(run_min, run_max, P, H, scale,
                                                              rscale, zp, ws_score, score_max,
                                                              nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  topk_maps_kernel<<<1, kSelThreads, 0, s>>>(ws_score, H, k, idx, fmap, cmap);
  return hipGetLastError();
}

hipError_t launch_select_per_shard(const float* run_min, const float* run_max, int64_t P,
                                   int64_t H, int64_t k, float* scale, float* rscale, uint8_t* zp,
                                   int32_t* idx, int32_t* fmap, int32_t* cmap, float* ws_width,
                                   hipStream_t s) {
  qparams_kernel<<<(unsigned)((H + 255) / 256), 256, 0, s>>>(run_min, run_max, P, H, scale,
                                                              rscale, zp, nullptr, false,
                                                              ws_width);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  topk_maps_kernel<<<(unsigned)P, kSelThreads, 0, s>>>(ws_width, H, k, idx, fmap, cmap);
  return hipGetLastError();
}

hipError_t launch_select_set(const float* run_min, const float* run_max, int64_t P, int64_t H,
                             int64_t k, float* scale, float* rscale, uint8_t* zp,
                             const int32_t* idx, int32_t* fmap, int32_t* cmap, hipStream_t s) {
  qparams_kernel<<<(unsigned)((H + 255) / 256), 256, 0, s>>>(run_min, run_max, P, H, scale,
                                                              rscale, zp, nullptr, false,
                                                              nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  set_maps_kernel<<<1, kSelThreads, 0, s>>>(idx, H, k, fmap, cmap);
  return hipGetLastError();
}

}  // namespace btq
