// Sender side: asymmetric 4-bit quantization of the int4 features, nibble
// packing, and the bit copy of the BF16 features.
//
// Method: "Revolutionizing LLM Inference: The Power of Efficient Low-Bit
// Communication", section "The Hybrid Quantization Algorithm", Inference
// bullet (selected features keep BF16, the rest go to 4 bits), and section
// "Combating Quantization Errors with Tensor Parallelism" (each device
// quantizes its partial sum before the sum).
//
// Fast kernel. One wavefront owns a wave-tile of 512 int4 slots, 8 per lane,
// so that each lane writes exactly one packed dword per token row. The wave
// walks a block of token rows of one shard. For each row:
//  1. Coalesced 16-byte loads bring the tile's feature span [hs, he) of the
//     bf16 row (plus alignment slack) into a wave-private LDS buffer. The
//     next rows' loads are issued before the current rows are computed.
//  2. Each lane gathers its 8 features from LDS. Each feature's offset is
//     fixed for the whole tile, and its rscale and zero point sit in
//     registers. The lane quantizes and packs 8 nibbles into one dword, and
//     the 64 dwords of the wave go out as one coalesced 256-byte store.
//  3. The lanes that own the tile's BF16 features copy their bf16 bits out
//     of the same LDS buffer.
// The LDS layout pads 4 bytes after every 16-byte chunk. Lane l's features
// then start at dword 5*l, so the 64 gathers of one instruction spread over
// all banks.
//
// General kernel. One thread per packed byte and per BF16 value, with
// 2-byte loads. It serves any H, k, alignment and LDS size.
#include "common.hpp"

namespace btq {

constexpr int kCpWaves = 4;   // independent waves per 256-thread block
constexpr int kCpRows = 4;    // token rows staged per step

__device__ __forceinline__ uint32_t pad_byte_off(uint32_t e) {   // element offset -> LDS byte
  return (e >> 3) * 20u + (e & 7u) * 2u;
}

__device__ __forceinline__ uint32_t quant4(uint32_t bits16, float r, float z) {
  const float v = __fmul_rn(bf16_to_f32(bits16), r);
  const float q = __builtin_amdgcn_fmed3f(rintf(v) + z, 0.0f, 15.0f);
  return (uint32_t)q;
}

template <int kMaxChunks>
__global__ __launch_bounds__(256) void compress_kernel(
    const uint16_t* __restrict__ x, int64_t T, int H, int Hq, int k, int ntiles,
    int64_t rows_per_wave, int64_t nrowblk, int64_t nwaves, int buf_bytes,
    const float* __restrict__ rscale, const uint8_t* __restrict__ zp,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cmap,
    uint32_t* __restrict__ packed32, uint16_t* __restrict__ outl) {
  extern __shared__ __align__(16) char smem[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int64_t gw = (int64_t)blockIdx.x * kCpWaves + wave;
  if (gw >= nwaves) return;   // waves never synchronize with each other
  const int c = (int)(gw % ntiles);
  const int64_t rest = gw / ntiles;
  const int64_t rb = rest % nrowblk;
  const int64_t p = rest / nrowblk;
  const TileGeom g = tile_geom(cmap, c, ntiles, Hq, H);
  const int a0 = g.hs & ~7;
  const int nch = (((g.he + 7) & ~7) - a0) >> 3;   // 16-byte chunks in the span
  const int64_t t0 = rb * rows_per_wave;
  const int64_t t1 = min(T, t0 + rows_per_wave);
  char* const buf = smem + (size_t)wave * kCpRows * buf_bytes;
  const int Bq4 = Hq >> 3;

  // Per-lane constants for the whole tile.
  const int j0 = g.jstart + kLaneSlots * lane;
  const bool active = j0 < g.jend;
  float rs[8], zf[8];
  uint32_t ad[8];
  if (active) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int h = cmap[j0 + e];
      rs[e] = rscale[p * H + h];
      zf[e] = (float)zp[p * H + h];
      ad[e] = pad_byte_off((uint32_t)(h - a0));
    }
  }
  uint32_t oad = 0;
  if (lane < g.nout) oad = pad_byte_off((uint32_t)(idx[g.ilo + lane] - a0));

  const uint16_t* __restrict__ xs = x + p * T * (int64_t)H + a0;
  uint4 v[kCpRows][kMaxChunks];
  auto load_rows = [&](int64_t t) {
#pragma unroll
    for (int r = 0; r < kCpRows; ++r) {
#pragma unroll
      for (int m = 0; m < kMaxChunks; ++m) {
        const int ci = lane + kWave * m;
        if (t + r < t1 && ci < nch)
          v[r][m] = *reinterpret_cast<const uint4*>(xs + (t + r) * (int64_t)H + 8 * ci);
      }
    }
  };

  load_rows(t0);
  for (int64_t t = t0; t < t1; t += kCpRows) {
#pragma unroll
    for (int r = 0; r < kCpRows; ++r) {
#pragma unroll
      for (int m = 0; m < kMaxChunks; ++m) {
        const int ci = lane + kWave * m;
        if (t + r < t1 && ci < nch) {
          uint32_t* d = reinterpret_cast<uint32_t*>(buf + r * buf_bytes + ci * 20);
          d[0] = v[r][m].x;
          d[1] = v[r][m].y;
          d[2] = v[r][m].z;
          d[3] = v[r][m].w;
        }
      }
    }
    wave_lds_sync();
    if (t + kCpRows < t1) load_rows(t + kCpRows);   // in flight during the compute below
#pragma unroll
    for (int r = 0; r < kCpRows; ++r) {
      const int64_t tt = t + r;
      if (tt >= t1) break;
      const char* b = buf + r * buf_bytes;
      const int64_t row = p * T + tt;
      if (active) {
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t u = *reinterpret_cast<const uint16_t*>(b + ad[e]);
          w |= quant4(u, rs[e], zf[e]) << (4 * e);
        }
        packed32[row * Bq4 + (j0 >> 3)] = w;
      }
      for (int i = lane; i < g.nout; i += kWave) {
        const uint32_t o = (i < kWave) ? oad : pad_byte_off((uint32_t)(idx[g.ilo + i] - a0));
        outl[row * k + g.ilo + i] = *reinterpret_cast<const uint16_t*>(b + o);
      }
    }
    wave_lds_sync();
  }
}

__global__ __launch_bounds__(256) void compress_general_kernel(
    const uint16_t* __restrict__ x, int64_t P, int64_t T, int64_t H, int64_t k, int64_t Hq,
    int64_t Bq, const float* __restrict__ rscale, const uint8_t* __restrict__ zp,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cmap,
    uint8_t* __restrict__ packed, uint16_t* __restrict__ outl) {
  const int64_t n1 = P * T * Bq;
  const int64_t n2 = P * T * k;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n1 + n2; i += stride) {
    if (i < n1) {
      const int64_t row = i / Bq, byte = i % Bq;
      const int64_t p = row / T;
      const int64_t j = 2 * byte;
      const int64_t h0 = cmap[j];
      uint32_t q = quant4(x[row * H + h0], rscale[p * H + h0], (float)zp[p * H + h0]);
      if (j + 1 < Hq) {
        const int64_t h1 = cmap[j + 1];
        q |= quant4(x[row * H + h1], rscale[p * H + h1], (float)zp[p * H + h1]) << 4;
      }
      packed[i] = (uint8_t)q;
    } else {
      const int64_t ii = i - n1;
      const int64_t row = ii / k, o = ii % k;
      outl[ii] = x[row * H + idx[o]];
    }
  }
}

static int64_t pick_rows_per_wave(int64_t slots_waves, int64_t T) {
  // ~8192 waves over the chip, a multiple of the staging depth, 4..64 rows.
  int64_t rpw = (slots_waves * T + 8191) / 8192;
  rpw = (rpw + kCpRows - 1) / kCpRows * kCpRows;
  if (rpw < kCpRows) rpw = kCpRows;
  if (rpw > 64) rpw = 64;
  return rpw;
}

hipError_t launch_compress(const uint16_t* x, int64_t P, int64_t T, int64_t H, int64_t k,
                           const float* rscale, const uint8_t* zp, const int32_t* idx,
                           const int32_t* cmap, uint8_t* packed, uint16_t* outl, hipStream_t s) {
  const int64_t Hq = H - k;
  const int64_t Bq = (Hq + 1) / 2;
  // The span of one tile holds its 512 slots plus the BF16 features between
  // them, at most min(H, 512 + k) features, plus 14 of alignment slack.
  const int64_t span = (H < kTileSlots + k ? H : kTileSlots + k) + 16;
  const int64_t nch_max = (span + 7) / 8;
  const int buf_bytes = (int)((nch_max * 20 + 15) / 16 * 16);
  const size_t lds = (size_t)kCpWaves * kCpRows * buf_bytes;
  const bool fast = Hq > 0 && H % 8 == 0 && Hq % 8 == 0 && (uintptr_t)x % 16 == 0 &&
                    (uintptr_t)packed % 4 == 0 && nch_max <= 4 * kWave && lds <= 65536;
  if (fast) {
    const int ntiles = (int)((Hq + kTileSlots - 1) / kTileSlots);
    const int64_t rpw = pick_rows_per_wave(P * ntiles, T);
    const int64_t nrowblk = (T + rpw - 1) / rpw;
    const int64_t nwaves = P * nrowblk * ntiles;
    const unsigned blocks = (unsigned)((nwaves + kCpWaves - 1) / kCpWaves);
    if (nch_max <= 2 * kWave)
      compress_kernel<2><<<blocks, 256, lds, s>>>(x, T, (int)H, (int)Hq, (int)k, ntiles, rpw,
                                                  nrowblk, nwaves, buf_bytes, rscale, zp, idx,
                                                  cmap, (uint32_t*)packed, outl);
    else
      compress_kernel<4><<<blocks, 256, lds, s>>>(x, T, (int)H, (int)Hq, (int)k, ntiles, rpw,
                                                  nrowblk, nwaves, buf_bytes, rscale, zp, idx,
                                                  cmap, (uint32_t*)packed, outl);
    return hipGetLastError();
  }
  const int64_t n = P * T * (Bq + k);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  compress_general_kernel<<<(unsigned)blocks, 256, 0, s>>>(x, P, T, H, k, Hq, Bq, rscale, zp, idx,
                                                           cmap, packed, outl);
  return hipGetLastError();
}

}  // namespace btq
