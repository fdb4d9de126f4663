// Internal helpers shared by the libbtq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace btq {

constexpr int kWave = 64;

// bf16 bit pattern -> fp32 (exact: the bf16 bits are the high half).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Orders LDS traffic between the lanes of one wavefront. The waves of a
// block work on separate LDS regions and never wait for each other, so a
// block-wide barrier is not needed. The fences keep the compiler from moving
// LDS accesses across this point. The hardware runs one wave's LDS
// instructions in issue order.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Geometry of one wave-tile of the int4 slot axis. A tile owns the slots
// [jstart, jend), 8 per lane, so that no two tiles share a packed byte. It
// also owns every feature h in [hs, he): its int4 features plus the BF16
// features that fall between them. Tile 0 starts at h = 0 and the last
// tile ends at h = H.
constexpr int kLaneSlots = 8;                    // slots per lane = one packed dword
constexpr int kTileSlots = kWave * kLaneSlots;   // 512 slots per wave-tile

struct TileGeom {
  int jstart, jend;   // slot range
  int hs, he;         // feature range
  int ilo, nout;      // BF16 features idx[ilo .. ilo+nout) lie in [hs, he)
};

__device__ __forceinline__ TileGeom tile_geom(const int32_t* __restrict__ cmap, int c,
                                              int ntiles, int Hq, int H) {
  TileGeom g;
  g.jstart = c * kTileSlots;
  g.jend = min(Hq, g.jstart + kTileSlots);
  g.hs = (c == 0) ? 0 : cmap[g.jstart];
  g.he = (c == ntiles - 1) ? H : cmap[g.jend];
  // h0 has exactly h0 - j0 BF16 features below it when cmap[j0] = h0
  g.ilo = g.hs - g.jstart;
  g.nout = (g.he - g.jend) - g.ilo;
  return g;
}

// ---- host-side launchers (one per kernel family), called by abi.hip ----
struct CalibPlan {
  int64_t nchunk;          // token-axis chunks reduced in parallel
  int64_t rows_per_chunk;
};
CalibPlan calib_plan(int64_t P, int64_t T, int64_t H);
hipError_t launch_calib(const uint16_t* x, int64_t P, int64_t T, int64_t H, float a, float c,
                        int first, float* run_min, float* run_max, float* ws, hipStream_t s);

hipError_t launch_select(const float* run_min, const float* run_max, int64_t P, int64_t H,
                         int64_t k, float* scale, float* rscale, uint8_t* zp, int32_t* idx,
                         int32_t* fmap, int32_t* cmap, float* ws_score, hipStream_t s);

hipError_t launch_compress(const uint16_t* x, int64_t P, int64_t T, int64_t H, int64_t k,
                           const float* rscale, const uint8_t* zp, const int32_t* idx,
                           const int32_t* cmap, uint8_t* packed, uint16_t* outl, hipStream_t s);

hipError_t launch_decompress(const uint8_t* packed, const uint16_t* outl, int64_t P, int64_t T,
                             int64_t H, int64_t k, const float* scale, const uint8_t* zp,
                             const int32_t* idx, const int32_t* cmap, float* y, hipStream_t s);

}  // namespace btq
