// Receiver side: fused dequantize of P shards' messages and fp32 sum.
//
// Method: "Revolutionizing LLM Inference: The Power of Efficient Low-Bit
// Communication", section "The Hybrid Quantization Algorithm", Inference
// bullet (after communication every tensor is converted back and the
// devices' values are summed).
//
// Fast kernel, specialised on the shard count (1..8). A wave-tile is the
// sender's 512 int4 slots, 8 per lane. A 256-thread block takes one tile,
// and its 4 waves walk 4 separate blocks of token rows. All tiles of one row
// group run on one XCD, so the partial cache lines of y written at tile
// boundaries merge in one L2.
//  0. Setup, once per block. The block loads every shard's contiguous
//     parameter span (scale, zero point for features hs..he) into LDS with
//     coalesced loads. Each lane then builds its registers: 8 scales per
//     shard, and one constant per feature, -sum_p z*s, that seeds the
//     accumulator.
//  1. Per token row, each lane loads one packed dword per shard, so each
//     packed byte is read from HBM exactly once, in coalesced 256-byte wave
//     loads. The next rows' words are loaded before this row's math.
//  2. A low nibble converts with one byte-to-float instruction. A high nibble
//     is masked in place (16*q) and meets a scale pre-divided by 16, which is
//     exact. Each term is one fma. BF16 features are summed in fp32 in shard
//     order from 0.
//  3. The outputs scatter to their feature positions in a wave-private LDS
//     row, padded one dword per 8 so the scatter avoids bank conflicts. The
//     wave then writes the tile's contiguous y span with coalesced stores.
//
// General kernel: one thread per (token, slot) and per (token, BF16 feature).
// It evaluates term = fl(q - z) * s and adds the terms in shard order, for
// any P, H, k and alignment.
#include "common.hpp"

namespace btq {

constexpr int kDqWaves = 4;
constexpr int kDqRows = 2;   // token rows per step

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t pad_dword(uint32_t i) { return i + (i >> 3); }

// LDS: [param span: scale fp32 NP x span_max | zero point u8 NP x span_max]
//      [4 waves x kDqRows y rows of buf_dwords]
template <int NP>
__global__ __launch_bounds__(256) void decompress_kernel(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ outl, int64_t T, int H,
    int Hq, int k, int ntiles, int rows_per_wave, int64_t nrowblk, int span_max,
    int buf_dwords, const float* __restrict__ scale, const uint8_t* __restrict__ zp,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cmap, float* __restrict__ y) {
  extern __shared__ __align__(16) char smem[];
  // unit = row group; its ntiles blocks run on one XCD
  int64_t rg, sub;
  if (!xcd_unit_block(blockIdx.x, ntiles, (nrowblk + kDqWaves - 1) / kDqWaves, &rg, &sub)) return;
  const int c = (int)sub;
  const TileGeom g = tile_geom(cmap, c, ntiles, Hq, H);
  const int L = g.he - g.hs;
  const int lane = threadIdx.x & (kWave - 1);
  // wave-uniform by construction; readfirstlane lets the compiler keep
  // everything derived from it (rows, descriptors) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t rb = rg * kDqWaves + wave;
  const int64_t t0 = rb * rows_per_wave;
  // waves past the last row block get no rows: every access of theirs is
  // out of range, and they leave after the block barrier
  const int nrows = (rb < nrowblk) ? (int)min(T - t0, (int64_t)rows_per_wave) : 0;
  const int Bq = Hq >> 1;
  float* const buf = reinterpret_cast<float*>(smem + (size_t)NP * span_max * 5) +
                     (size_t)wave * kDqRows * buf_dwords;
  const uint32_t dummy = (uint32_t)buf_dwords - 1;   // LDS slot for idle lanes

  // Whole message tensors (the launcher checks they span < 2^31 bytes), and
  // this wave's rows of y.
  const rsrc_t rp = make_rsrc(packed, (uint32_t)(NP * T * (int64_t)Bq));
  const rsrc_t ro = make_rsrc(outl, (uint32_t)(NP * T * (int64_t)k * 2));
  const rsrc_t ry = make_rsrc(y + t0 * H, (uint32_t)nrows * (uint32_t)H * 4u);
  const rsrc_t rc = make_rsrc(cmap, (uint32_t)Hq * 4u);

  const int j0 = g.jstart + kLaneSlots * lane;
  const bool active = j0 < g.jend;
  const uint32_t pk_off = (active && nrows > 0) ? (uint32_t)(j0 >> 1) : kOOB;
  const uint32_t o_off = (lane < g.nout && nrows > 0) ? (uint32_t)(g.ilo + lane) * 2u : kOOB;

  uint32_t w[kDqRows][NP], ov[kDqRows][NP];
  // The lane's offsets stay in fixed VGPRs; the (shard, row) offset is
  // uniform and rides in the instruction's SGPR offset.
  auto load_rows = [&](int s) {
#pragma unroll
    for (int r = 0; r < kDqRows; ++r) {
      const int64_t row = t0 + min(s + r, nrows - 1);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int64_t prow = (int64_t)p * T + row;
        w[r][p] = __builtin_amdgcn_raw_buffer_load_b32(rp, pk_off, (uint32_t)(prow * Bq), kStream);
        ov[r][p] = __builtin_amdgcn_raw_buffer_load_b16(ro, o_off, (uint32_t)(prow * k * 2), 0);
      }
    }
  };
  // The first rows' loads go out before the setup below, so that its latency
  // (parameter loads, barrier, map loads) overlaps theirs.
  if (nrows > 0) load_rows(0);

  // 0. every shard's parameter span -> LDS, then one block barrier
  float* const s_l = reinterpret_cast<float*>(smem);
  uint8_t* const z_l = reinterpret_cast<uint8_t*>(smem + (size_t)NP * span_max * 4);
  for (int p = 0; p < NP; ++p) {
    for (int i = threadIdx.x; i < L; i += blockDim.x) {
      s_l[p * span_max + i] = scale[(int64_t)p * H + g.hs + i];
      z_l[p * span_max + i] = zp[(int64_t)p * H + g.hs + i];
    }
  }
  __syncthreads();
  if (nrows <= 0) return;   // no block barrier after this point

  const int jj = active ? j0 : g.jstart;
  const v4u hA = __builtin_amdgcn_raw_buffer_load_b128(rc, (uint32_t)jj * 4u, 0, 0);
  const v4u hB = __builtin_amdgcn_raw_buffer_load_b128(rc, (uint32_t)jj * 4u + 16u, 0, 0);
  const int hh[8] = {(int)hA[0], (int)hA[1], (int)hA[2], (int)hA[3],
                     (int)hB[0], (int)hB[1], (int)hB[2], (int)hB[3]};
  float sc[NP][8], bias[8];
  uint32_t ya[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int o = hh[e] - g.hs;
    ya[e] = active ? pad_dword((uint32_t)o) : dummy;
    float b = 0.0f;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const float s = s_l[p * span_max + o];
      const float z = (float)z_l[p * span_max + o];
      b = __fsub_rn(b, __fmul_rn(z, s));
      sc[p][e] = (e & 1) ? s * 0.0625f : s;   // high nibbles arrive as 16*q
    }
    bias[e] = b;
  }
  const int nout_it = (g.nout + kWave - 1) / kWave;   // uniform
  uint32_t oa = dummy;
  if (g.nout > 0 && lane < g.nout) oa = pad_dword((uint32_t)(idx[g.ilo + lane] - g.hs));
  const int st_it = (L + kWave - 1) / kWave;          // uniform

  for (int s = 0; s < nrows; s += kDqRows) {
#pragma unroll
    for (int r = 0; r < kDqRows; ++r) {
      float* b = buf + r * buf_dwords;
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
      // Idle lanes skip their LDS writes: many lanes storing to one address
      // serialize on its bank.
      if (active) {
#pragma unroll
        for (int e = 0; e < 8; ++e) b[ya[e]] = acc[e];
      }
      float o = 0.0f;
#pragma unroll
      for (int p = 0; p < NP; ++p) o = __fadd_rn(o, bf16_to_f32(ov[r][p]));
      if (lane < g.nout) b[oa] = o;
    }
    // tiles holding more than 64 BF16 features
    for (int it = 1; it < nout_it; ++it) {
      const int i = lane + kWave * it;
      const bool ok = i < g.nout;
      const uint32_t off = ok ? (uint32_t)(g.ilo + i) * 2u : kOOB;
      const uint32_t at = ok ? pad_dword((uint32_t)(idx[g.ilo + i] - g.hs)) : dummy;
#pragma unroll
      for (int r = 0; r < kDqRows; ++r) {
        const int64_t row = t0 + min(s + r, nrows - 1);
        float q = 0.0f;
        for (int p = 0; p < NP; ++p)
          q = __fadd_rn(q, bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(
                               ro, off + (uint32_t)(((int64_t)p * T + row) * k * 2), 0, 0)));
        if (ok) buf[r * buf_dwords + at] = q;
      }
    }
    wave_lds_sync();
    if (s + kDqRows < nrows) load_rows(s + kDqRows);   // in flight during the stores below
#pragma unroll
    for (int r = 0; r < kDqRows; ++r) {
      if (s + r >= nrows) break;
      const float* b = buf + r * buf_dwords;
      const uint32_t rowoff = (uint32_t)(s + r) * (uint32_t)H * 4u;
      // batches of 4: LDS reads first, then the stores
      for (int it0 = 0; it0 < st_it; it0 += 4) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v[q] = b[pad_dword((uint32_t)min(lane + kWave * (it0 + q), L - 1))];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = lane + kWave * (it0 + q);
          const uint32_t off = (i < L) ? (uint32_t)(g.hs + i) * 4u : kOOB;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[q]), ry, off, rowoff, kStream);
        }
      }
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
                        int64_t k, int64_t Hq, int ntiles, int rpw, int64_t nrowblk,
                        int span_max, int buf_dwords, const float* scale, const uint8_t* zp,
                        const int32_t* idx, const int32_t* cmap, float* y, hipStream_t s) {
  const int64_t ngroups = (nrowblk + kDqWaves - 1) / kDqWaves;
  const size_t lds = (size_t)NP * span_max * 5 + (size_t)kDqWaves * kDqRows * buf_dwords * 4;
  decompress_kernel<NP><<<(unsigned)xcd_grid(ntiles, ngroups), 256, lds, s>>>(
      packed, outl, T, (int)H, (int)Hq, (int)k, ntiles, rpw, nrowblk, span_max, buf_dwords,
      scale, zp, idx, cmap, y);
}

hipError_t launch_decompress(const uint8_t* packed, const uint16_t* outl, int64_t P, int64_t T,
                             int64_t H, int64_t k, const float* scale, const uint8_t* zp,
                             const int32_t* idx, const int32_t* cmap, float* y, hipStream_t s) {
  const int64_t Hq = H - k;
  const int64_t Bq = (Hq + 1) / 2;
  const int64_t span = (H < kTileSlots + k ? H : kTileSlots + k);
  const int span_max = (int)((span + 15) / 16 * 16);
  const int buf_dwords = (int)((span + span / 8 + 8 + 3) / 4 * 4);
  const size_t lds = (size_t)P * span_max * 5 + (size_t)kDqWaves * kDqRows * buf_dwords * 4;
  // Buffer resources: the whole message and one wave's rows of y must each
  // span fewer than 2^31 bytes.
  const int64_t lim = int64_t(1) << 31;
  const bool fast = Hq > 0 && P <= 8 && Hq % 8 == 0 && (uintptr_t)packed % 4 == 0 &&
                    lds <= 65536 && P * T * Bq < lim && P * T * k * 2 < lim &&
                    H < (int64_t(1) << 24);
  if (fast) {
    const int ntiles = (int)((Hq + kTileSlots - 1) / kTileSlots);
    // about 2048 waves (8 per CU), 2..32 rows each
    int64_t rpw64 = (ntiles * T + 2047) / 2048;
    rpw64 = (rpw64 + kDqRows - 1) / kDqRows * kDqRows;
    if (rpw64 < kDqRows) rpw64 = kDqRows;
    if (rpw64 > 32) rpw64 = 32;
    const int rpw = (int)rpw64;
    const int64_t nrowblk = (T + rpw - 1) / rpw;
    switch (P) {
#define BTQ_DQ_CASE(n)                                                                         \
  case n:                                                                                      \
    launch_fast<n>(packed, outl, T, H, k, Hq, ntiles, rpw, nrowblk, span_max, buf_dwords, scale, \
                   zp, idx, cmap, y, s);                                                       \
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
