// Receiver side: fused dequantize of P shards' messages and fp32 sum.
//
// Method: "Revolutionizing LLM Inference: The Power of Efficient Low-Bit
// Communication", section "The Hybrid Quantization Algorithm", Inference
// bullet (after communication every tensor is converted back and the
// devices' values are summed).
//
// Fast kernel, specialised on the shard count (1..8). One wavefront owns the
// same 512-slot wave-tile as the sender, with 8 slots per lane. Per token
// row, each lane loads one packed dword per shard. Each packed byte is read
// from HBM exactly once, in coalesced 256-byte wave loads. The lane
// accumulates its 8 outputs in registers. A low nibble converts with one
// byte-to-float instruction; a high nibble is masked in place (16*q) and
// meets a scale pre-divided by 16, which is exact. The zero points fold into
// one per-feature constant -sum_p z*s that seeds the accumulator, so each
// term costs one fma. BF16 features are summed in fp32 in shard order from 0.
// The outputs scatter to their feature positions in a wave-private LDS row
// (padded one dword per 8, so the scatter is free of bank conflicts). From
// there the wave writes the tile's contiguous y span with coalesced stores.
//
// General kernel: one thread per (token, slot) and per (token, BF16 feature).
// It evaluates term = fl(q - z) * s and adds the terms in shard order, for
// any P, H, k and alignment.
#include "common.hpp"

namespace btq {

constexpr int kDqWaves = 4;
constexpr int kDqRows = 2;   // token rows per step

__device__ __forceinline__ uint32_t pad_dword(uint32_t i) { return i + (i >> 3); }

template <int NP>
__global__ __launch_bounds__(256) void decompress_kernel(
    const uint32_t* __restrict__ packed32, const uint16_t* __restrict__ outl, int64_t T, int H,
    int Hq, int k, int ntiles, int64_t rows_per_wave, int64_t nrowblk, int64_t nwaves,
    int buf_dwords, const float* __restrict__ scale, const uint8_t* __restrict__ zp,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cmap, float* __restrict__ y) {
  extern __shared__ __align__(16) float ysm[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int64_t gw = (int64_t)blockIdx.x * kDqWaves + wave;
  if (gw >= nwaves) return;   // waves never synchronize with each other
  const int c = (int)(gw % ntiles);
  const int64_t rb = gw / ntiles;
  const TileGeom g = tile_geom(cmap, c, ntiles, Hq, H);
  const int L = g.he - g.hs;
  const int64_t t0 = rb * rows_per_wave;
  const int64_t t1 = min(T, t0 + rows_per_wave);
  float* const buf = ysm + (size_t)wave * kDqRows * buf_dwords;
  const int Bq4 = Hq >> 3;

  const int j0 = g.jstart + kLaneSlots * lane;
  const bool active = j0 < g.jend;
  float sc[NP][8], bias[8];
  uint32_t ya[8];
  if (active) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int h = cmap[j0 + e];
      ya[e] = pad_dword((uint32_t)(h - g.hs));
      float b = 0.0f;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const float s = scale[(int64_t)p * H + h];
        const float z = (float)zp[(int64_t)p * H + h];
        b = __fsub_rn(b, __fmul_rn(z, s));
        sc[p][e] = (e & 1) ? s * 0.0625f : s;   // high nibbles arrive as 16*q
      }
      bias[e] = b;
    }
  }
  uint32_t oa = 0;
  if (lane < g.nout) oa = pad_dword((uint32_t)(idx[g.ilo + lane] - g.hs));

  const int64_t slot_dw = j0 >> 3;
  for (int64_t t = t0; t < t1; t += kDqRows) {
    uint32_t w[kDqRows][NP];
    uint32_t ov[kDqRows][NP];
#pragma unroll
    for (int r = 0; r < kDqRows; ++r) {
      if (t + r < t1) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int64_t row = (int64_t)p * T + t + r;
          if (active) w[r][p] = packed32[row * Bq4 + slot_dw];
          if (lane < g.nout) ov[r][p] = outl[row * k + g.ilo + lane];
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kDqRows; ++r) {
      if (t + r >= t1) break;
      float* b = buf + r * buf_dwords;
      if (active) {
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = bias[e];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const uint32_t lo = w[r][p] & 0x0F0F0F0Fu;
          const uint32_t hi = w[r][p] & 0xF0F0F0F0u;
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            acc[2 * bb] = fmaf((float)((lo >> (8 * bb)) & 0xFFu), sc[p][2 * bb], acc[2 * bb]);
            acc[2 * bb + 1] =
                fmaf((float)((hi >> (8 * bb)) & 0xFFu), sc[p][2 * bb + 1], acc[2 * bb + 1]);
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) b[ya[e]] = acc[e];
      }
      if (lane < g.nout) {
        float o = 0.0f;
#pragma unroll
        for (int p = 0; p < NP; ++p) o = __fadd_rn(o, bf16_to_f32(ov[r][p]));
        b[oa] = o;
      }
      for (int i = kWave + lane; i < g.nout; i += kWave) {   // tiles with > 64 BF16 features
        float o = 0.0f;
        for (int p = 0; p < NP; ++p)
          o = __fadd_rn(o, bf16_to_f32(outl[((int64_t)p * T + t + r) * k + g.ilo + i]));
        b[pad_dword((uint32_t)(idx[g.ilo + i] - g.hs))] = o;
      }
    }
    wave_lds_sync();
#pragma unroll
    for (int r = 0; r < kDqRows; ++r) {
      if (t + r >= t1) break;
      const float* b = buf + r * buf_dwords;
      float* yr = y + (t + r) * (int64_t)H + g.hs;
      for (int i = lane; i < L; i += kWave) yr[i] = b[pad_dword((uint32_t)i)];
    }
    wave_lds_sync();
  }
}

__global__ __launch_bounds__(256) void decompress_general_kernel(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ outl, int64_t P, int64_t T,
    int64_t H, int64_t k, int64_t Hq, int64_t Bq, const float* __restrict__ scale,
    const uint8_t* __restrict__ zp, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ cmap, float* __restrict__ y) {
  const int64_t n1 = T * Hq;
  const int64_t n2 = T * k;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n1 + n2; i += stride) {
    float acc = 0.0f;
    if (i < n1) {
      const int64_t t = i / Hq, j = i % Hq;
      const int64_t h = cmap[j];
      for (int64_t p = 0; p < P; ++p) {
        const uint32_t byte = packed[(p * T + t) * Bq + (j >> 1)];
        const int q = (int)((j & 1) ? (byte >> 4) : (byte & 0xFu));
        const float d = (float)(q - (int)zp[p * H + h]);
        acc = __fadd_rn(acc, __fmul_rn(d, scale[p * H + h]));
      }
      y[t * H + h] = acc;
    } else {
      const int64_t ii = i - n1;
      const int64_t t = ii / k, o = ii % k;
      for (int64_t p = 0; p < P; ++p) acc = __fadd_rn(acc, bf16_to_f32(outl[(p * T + t) * k + o]));
      y[t * H + idx[o]] = acc;
    }
  }
}

template <int NP>
static void launch_fast(const uint8_t* packed, const uint16_t* outl, int64_t T, int64_t H,
                        int64_t k, int64_t Hq, int ntiles, int64_t rpw, int64_t nrowblk,
                        int64_t nwaves, int buf_dwords, size_t lds, const float* scale,
                        const uint8_t* zp, const int32_t* idx, const int32_t* cmap, float* y,
                        hipStream_t s) {
  const unsigned blocks = (unsigned)((nwaves + kDqWaves - 1) / kDqWaves);
  decompress_kernel<NP><<<blocks, 256, lds, s>>>(
      (const uint32_t*)packed, outl, T, (int)H, (int)Hq, (int)k, ntiles, rpw, nrowblk, nwaves,
      buf_dwords, scale, zp, idx, cmap, y);
}

hipError_t launch_decompress(const uint8_t* packed, const uint16_t* outl, int64_t P, int64_t T,
                             int64_t H, int64_t k, const float* scale, const uint8_t* zp,
                             const int32_t* idx, const int32_t* cmap, float* y, hipStream_t s) {
  const int64_t Hq = H - k;
  const int64_t Bq = (Hq + 1) / 2;
  const int64_t span = (H < kTileSlots + k ? H : kTileSlots + k);
  const int buf_dwords = (int)((span + span / 8 + 8 + 3) / 4 * 4);
  const size_t lds = (size_t)kDqWaves * kDqRows * buf_dwords * sizeof(float);
  const bool fast = Hq > 0 && P <= 8 && Hq % 8 == 0 && (uintptr_t)packed % 4 == 0 &&
                    lds <= 65536;
  if (fast) {
    const int ntiles = (int)((Hq + kTileSlots - 1) / kTileSlots);
    // ~4096 waves, 2..32 rows each
    int64_t rpw = (ntiles * T + 4095) / 4096;
    rpw = (rpw + kDqRows - 1) / kDqRows * kDqRows;
    if (rpw < kDqRows) rpw = kDqRows;
    if (rpw > 32) rpw = 32;
    const int64_t nrowblk = (T + rpw - 1) / rpw;
    const int64_t nwaves = nrowblk * ntiles;
    switch (P) {
#define BTQ_DQ_CASE(n)                                                                     \
  case n:                                                                                  \
    launch_fast<n>(packed, outl, T, H, k, Hq, ntiles, rpw, nrowblk, nwaves, buf_dwords, lds, \
                   scale, zp, idx, cmap, y, s);                                            \
    break;
      BTQ_DQ_CASE(1)
      BTQ_DQ_CASE(2)
      BTQ_DQ_CASE(3)
      BTQ_DQ_CASE(4)
      BTQ_DQ_CASE(5)
      BTQ_DQ_CASE(6)
      BTQ_DQ_CASE(7)
      BTQ_DQ_CASE(8)
#undef BTQ_DQ_CASE
    }
    return hipGetLastError();
  }
  const int64_t n = T * H;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  decompress_general_kernel<<<(unsigned)blocks, 256, 0, s>>>(packed, outl, P, T, H, k, Hq, Bq,
                                                             scale, zp, idx, cmap, y);
  return hipGetLastError();
}

}  // namespace btq
