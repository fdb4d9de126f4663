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
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Block barrier that orders LDS only. __syncthreads() also orders global
// memory, which makes every wave wait for all of its loads in flight
// (vmcnt(0)) before the barrier, also where only LDS needs ordering.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Keeps the scheduler from moving instructions across this point. The fast
// kernels issue their setup loads first and their token-row loads second: the
// vector-memory counter retires in issue order, so a wait for a setup load
// then never includes the row loads behind it.
__device__ __forceinline__ void issue_fence() { __builtin_amdgcn_sched_barrier(0); }

// Marks a register as redefined here (an empty asm that reads and writes it).
// The fast kernels apply it to the per-lane constants that come straight from
// setup loads, once, before their main loop: the completion wait then happens
// there, and the loop body never has to wait for a setup load again.
template <typename V>
__device__ __forceinline__ void settle(V& v) {
  asm volatile("" : "+v"(v));
}

// Hides a value's origin from the optimizer (an empty asm that reads and
// writes it, with no side effects), so it cannot rewrite the computation of
// the value's uses in terms of that origin.
template <typename V>
__device__ __forceinline__ void opaque(V& v) {
  asm("" : "+v"(v));
}

// Raw buffer resources (gfx9 format). A wave builds a descriptor over the
// part of a tensor it touches, so every offset stays 32-bit. The hardware
// range check then handles ragged edges: a load at or past num_records
// returns 0, and a store there is dropped. Lanes that have nothing to do
// point their offset at kOOB instead of branching. That keeps the memory
// instructions out of divergent control flow, where the compiler has to
// wait for all loads in flight at every join. Every descriptor this library
// builds spans fewer than 2^31 bytes, so any offset >= kOOB is out of range.
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // dword3: 32-bit data format, raw (no swizzle)
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}

// Cache policy for streaming (read-once / write-once) buffer accesses:
// the non-temporal hint (bit 1 of the gfx94x/gfx950 cache-policy operand).
constexpr int kStream = 2;

// XCD-aware block order. MI355X deals workgroups round-robin over its 8
// XCDs, and each XCD has its own L2. A unit is a group of `per_unit`
// consecutive logical blocks whose writes share cache lines: all tiles of
// one block of token rows. This mapping runs a whole unit on one XCD, so the
// partial lines its blocks write merge in one L2 before they reach HBM.
// Returns false for the padding blocks of the last round.
constexpr int kXcds = 8;
__device__ __forceinline__ bool xcd_unit_block(int64_t b, int64_t per_unit, int64_t units,
                                               int64_t* unit, int64_t* sub) {
  const int64_t xcd = b % kXcds;
  const int64_t slot = b / kXcds;
  *unit = (slot / per_unit) * kXcds + xcd;
  *sub = slot % per_unit;
  return *unit < units;
}
__host__ __forceinline__ int64_t xcd_grid(int64_t per_unit, int64_t units) {
  return (units + kXcds - 1) / kXcds * kXcds * per_unit;
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
// The same plan with at most as many chunks as fit max_ws_floats floats of
// partials (nchunk 0: not even one chunk fits).
CalibPlan calib_plan_capped(int64_t P, int64_t T, int64_t H, int64_t max_ws_floats);
hipError_t launch_calib(const uint16_t* x, int64_t P, int64_t T, int64_t H, float a, float c,
                        int first, float* run_min, float* run_max, float* ws, hipStream_t s);
// ws holds 2*plan.nchunk*P*H floats.
hipError_t launch_calib_plan(const uint16_t* x, int64_t P, int64_t T, int64_t H, float a, float c,
                             int first, float* run_min, float* run_max, float* ws,
                             const CalibPlan& plan, hipStream_t s);

hipError_t launch_select(const float* run_min, const float* run_max, int64_t P, int64_t H,
                         int64_t k, float* scale, float* rscale, uint8_t* zp, int32_t* idx,
                         int32_t* fmap, int32_t* cmap, float* ws_score, bool score_max,
                         hipStream_t s);
// One BF16 set per shard: idx [P,k], fmap [P,H], cmap [P,H-k]; ws_width
// holds P*H floats.
hipError_t launch_select_per_shard(const float* run_min, const float* run_max, int64_t P,
                                   int64_t H, int64_t k, float* scale, float* rscale, uint8_t* zp,
                                   int32_t* idx, int32_t* fmap, int32_t* cmap, float* ws_width,
                                   hipStream_t s);
// The same outputs for a given BF16 set: idx is a device copy of k distinct
// features in ascending order.
hipError_t launch_select_set(const float* run_min, const float* run_max, int64_t P, int64_t H,
                             int64_t k, float* scale, float* rscale, uint8_t* zp,
                             const int32_t* idx, int32_t* fmap, int32_t* cmap, hipStream_t s);

// rscale [P,H], zp [P,H]; per_shard: idx [P,k] and cmap [P,H-k] hold one
// set per shard, else idx [k] and cmap [H-k].
hipError_t launch_compress(const uint16_t* x, int64_t P, int64_t T, int64_t H, int64_t k,
                           const float* rscale, const uint8_t* zp, const int32_t* idx,
                           const int32_t* cmap, uint8_t* packed, int64_t pitch, uint16_t* outl,
                           bool per_shard, hipStream_t s);

// scale [P,H], zp [P,H]; fmap [P,H] when per_shard, else [H]. y is fp32,
// or bf16 bits when bf16.
hipError_t launch_decompress(const uint8_t* packed, int64_t pitch, const uint16_t* outl, int64_t P,
                             int64_t T, int64_t H, int64_t k, const float* scale,
                             const uint8_t* zp, const int32_t* fmap, bool per_shard, void* y,
                             bool bf16, hipStream_t s);

}  // namespace btq
