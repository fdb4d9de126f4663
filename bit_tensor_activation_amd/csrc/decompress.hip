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
//  0. Setup, once per wave. Each lane loads its 8 slots' scales for every
//     shard and their constant -sum_p z*s, which seeds the accumulator, from
//     the decoder table that selection wrote in slot order (32 contiguous
//     bytes per row of the table). Then it issues its first kDqRing token
//     rows. No LDS staging and no block barrier.
//  1. Per token row, each lane holds one packed dword per shard, so each
//     packed byte is read from HBM exactly once, in coalesced 256-byte wave
//     loads. The tile's BF16 values of all shards fill one or two registers
//     across the wave, one lane per (shard, feature). A ring of kDqRing rows
//     stays in flight, and consumed slots reload kDqRing rows ahead.
//  2. A low nibble converts with one byte-to-float instruction. A high nibble
//     is masked in place (16*q) and meets a scale pre-divided by 16, which is
//     exact. Each term is one fma. For a BF16 feature, the lane that owns it
//     fetches its shards' values across lanes (ds_bpermute) and adds them in
//     shard order from 0.
//  3. The outputs scatter to their feature positions in a wave-private LDS
//     row, padded one dword per 8 so the scatter avoids bank conflicts. The
//     wave then writes the tile's contiguous y span with coalesced stores.
//
// General kernel: one thread per (token, slot) and per (token, BF16 feature).
// It evaluates term = fl(q - z) * s and adds the terms in shard order, for
// any P, H, k and alignment. Both read the decoder table [2P+1, Hq]: rows
// 0..P-1 scale, rows P..2P-1 zero point, row 2P the per-slot constant.
#include "common.hpp"

namespace btq {

constexpr int kDqWaves = 4;

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t pad_dword(uint32_t i) { return i + (i >> 3); }

constexpr int kDqRing = 8;   // token rows in flight per wave
constexpr int kDqSub = 2;    // token rows per sub-step (LDS y rows)
constexpr int kOutRegs = 2;  // BF16-block registers per row: covers P*nout <= 128

// LDS: 4 waves x kDqSub y rows of buf_dwords
template <int NP>
__global__ __launch_bounds__(256) void decompress_kernel(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ outl, int64_t T, int H,
    int Hq, int k, int ntiles, int rows_per_wave, int64_t nrowblk, int buf_dwords,
    const float* __restrict__ dec, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ cmap, float* __restrict__ y) {
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
  if (rb >= nrowblk) return;   // no rows for this wave (no block barrier below)
  const int64_t t0 = rb * rows_per_wave;
  const int nrows = (int)min(T - t0, (int64_t)rows_per_wave);
  const int Bq = Hq >> 1;
  float* const buf = reinterpret_cast<float*>(smem) + (size_t)wave * kDqSub * buf_dwords;

  // Whole message tensors (the launcher checks they span < 2^31 bytes), and
  // this wave's rows of y.
  const rsrc_t rp = make_rsrc(packed, (uint32_t)(NP * T * (int64_t)Bq));
  const rsrc_t ro = make_rsrc(outl, (uint32_t)(NP * T * (int64_t)k * 2));
  const rsrc_t ry = make_rsrc(y + t0 * H, (uint32_t)nrows * (uint32_t)H * 4u);
  const rsrc_t rc = make_rsrc(cmap, (uint32_t)Hq * 4u);

  const int j0 = g.jstart + kLaneSlots * lane;
  const bool active = j0 < g.jend;
  const uint32_t pk_off = active ? (uint32_t)(j0 >> 1) : kOOB;
  // BF16 block: entry e = r*64 + lane holds shard e / nout, feature e % nout
  const bool compact = NP * g.nout <= kOutRegs * kWave;   // uniform
  uint32_t o_off[kOutRegs];
#pragma unroll
  for (int r = 0; r < kOutRegs; ++r) {
    const int e = r * kWave + lane;
    o_off[r] = kOOB;
    if (g.nout > 0 && compact && e < NP * g.nout) {
      const int sp = e / g.nout, i = e - sp * g.nout;
      o_off[r] = (uint32_t)(((int64_t)sp * T * k + g.ilo + i) * 2);
    }
  }

  uint32_t w[kDqRing][NP], ov[kDqRing][kOutRegs];
  // The lane's offsets stay in fixed VGPRs; the (shard, row) offset is
  // uniform and rides in the instruction's SGPR offset.
  auto load = [&](int q, int row) {
    const bool ok = row < nrows;   // uniform
    const int64_t rowg = t0 + min(row, nrows - 1);
#pragma unroll
    for (int p = 0; p < NP; ++p)
      w[q][p] = __builtin_amdgcn_raw_buffer_load_b32(rp, ok ? pk_off : kOOB,
                                                     (uint32_t)(((int64_t)p * T + rowg) * Bq), kStream);
#pragma unroll
    for (int r = 0; r < kOutRegs; ++r)
      ov[q][r] = __builtin_amdgcn_raw_buffer_load_b16(ro, ok ? o_off[r] : kOOB,
                                                      (uint32_t)(rowg * k * 2), 0);
  };

  // Setup loads first, ring loads second: the vector-memory counter retires
  // in order, so waiting for a setup load never waits for the ring.
  // (a) the lane's 8 slots of every shard's scale row and of the constant
  // row (lanes past the tile read zeros)
  const rsrc_t rd = make_rsrc(dec, (uint32_t)((2 * NP + 1) * (int64_t)Hq * 4));
  const uint32_t d_off = active ? (uint32_t)j0 * 4u : kOOB;
  v4u sv[NP][2], bv[2];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    sv[p][0] = __builtin_amdgcn_raw_buffer_load_b128(rd, d_off, (uint32_t)(p * Hq * 4), 0);
    sv[p][1] = __builtin_amdgcn_raw_buffer_load_b128(rd, d_off + 16u, (uint32_t)(p * Hq * 4), 0);
  }
  bv[0] = __builtin_amdgcn_raw_buffer_load_b128(rd, d_off, (uint32_t)(2 * NP * Hq * 4), 0);
  bv[1] = __builtin_amdgcn_raw_buffer_load_b128(rd, d_off + 16u, (uint32_t)(2 * NP * Hq * 4), 0);
  // (b) the lane's 8 feature indices and its BF16 feature index
  const int jj = active ? j0 : g.jstart;
  const v4u hA = __builtin_amdgcn_raw_buffer_load_b128(rc, (uint32_t)jj * 4u, 0, 0);
  const v4u hB = __builtin_amdgcn_raw_buffer_load_b128(rc, (uint32_t)jj * 4u + 16u, 0, 0);
  const rsrc_t ri_ = make_rsrc(idx, (uint32_t)k * 4u);
  const bool own_out = lane < g.nout;
  const uint32_t oh = __builtin_amdgcn_raw_buffer_load_b32(
      ri_, own_out ? (uint32_t)(g.ilo + lane) * 4u : kOOB, 0, 0);
  // (c) the ring: the first kDqRing rows. Unconditional: a branch around it
  // would make the compiler assume at the join that these loads might not
  // exist, and wait for the ring when it waits for the setup loads.
#pragma unroll
  for (int q = 0; q < kDqRing; ++q) load(q, q);

  const int hh[8] = {(int)hA[0], (int)hA[1], (int)hA[2], (int)hA[3],
                     (int)hB[0], (int)hB[1], (int)hB[2], (int)hB[3]};
  float sc[NP][8], bias[8];
  uint32_t ya[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ya[e] = pad_dword((uint32_t)(hh[e] - g.hs));
    bias[e] = __uint_as_float(bv[e >> 2][e & 3]);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const float s = __uint_as_float(sv[p][e >> 2][e & 3]);
      sc[p][e] = (e & 1) ? s * 0.0625f : s;   // high nibbles arrive as 16*q
    }
  }
  const uint32_t oa = own_out ? pad_dword((uint32_t)((int)oh - g.hs)) : 0u;
  // Lane i < nout owns BF16 feature ilo+i: its shard p value sits in entry
  // p*nout + i, i.e. register (entry / 64) of lane (entry % 64).
  int src_addr[NP];
  bool src_hi[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int e = p * g.nout + (own_out ? lane : 0);
    src_addr[p] = (e & (kWave - 1)) * 4;
    src_hi[p] = e >= kWave;
  }
  const int st_it = (L + kWave - 1) / kWave;   // uniform

  for (int base = 0; base < nrows; base += kDqRing) {
#pragma unroll
    for (int sb = 0; sb < kDqRing / kDqSub; ++sb) {
#pragma unroll
      for (int r = 0; r < kDqSub; ++r) {
        const int q = sb * kDqSub + r;
        float* b = buf + r * buf_dwords;
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = bias[e];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const uint32_t lo = w[q][p] & 0x0F0F0F0Fu;
          const uint32_t hi = w[q][p] & 0xF0F0F0F0u;
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            acc[2 * bb] = fmaf((float)((lo >> (8 * bb)) & 0xFFu), sc[p][2 * bb], acc[2 * bb]);
            acc[2 * bb + 1] =
                fmaf((float)((hi >> (8 * bb)) & 0xFFu), sc[p][2 * bb + 1], acc[2 * bb + 1]);
          }
        }
        // idle lanes skip their LDS writes: many lanes storing to one address
        // serialize on its bank
        if (active) {
#pragma unroll
          for (int e = 0; e < 8; ++e) b[ya[e]] = acc[e];
        }
        if (g.nout > 0) {   // uniform
          const int row = base + q;
          if (compact) {
            float o = 0.0f;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
              const int v0 = __builtin_amdgcn_ds_bpermute(src_addr[p], (int)ov[q][0]);
              const int v1 = __builtin_amdgcn_ds_bpermute(src_addr[p], (int)ov[q][1]);
              o = __fadd_rn(o, bf16_to_f32((uint32_t)(src_hi[p] ? v1 : v0) & 0xFFFFu));
            }
            if (own_out) b[oa] = o;
          } else {
            // many BF16 features in this tile: sum them straight from memory
            const int64_t rowg = t0 + min(row, nrows - 1);
            for (int i = lane; i < g.nout; i += kWave) {
              float o = 0.0f;
              for (int p = 0; p < NP; ++p)
                o = __fadd_rn(o, bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(
                                     ro, (uint32_t)(((int64_t)p * T * k + g.ilo + i) * 2),
                                     (uint32_t)(rowg * k * 2), 0)));
              b[pad_dword((uint32_t)(idx[g.ilo + i] - g.hs))] = o;
            }
          }
        }
      }
      // refill the consumed slots with the rows kDqRing ahead
#pragma unroll
      for (int r = 0; r < kDqSub; ++r) load(sb * kDqSub + r, base + kDqRing + sb * kDqSub + r);
      wave_lds_sync();
#pragma unroll
      for (int r = 0; r < kDqSub; ++r) {
        const int row = base + sb * kDqSub + r;
        const bool ok = row < nrows;   // uniform
        const float* b = buf + r * buf_dwords;
        const uint32_t rowoff = (uint32_t)min(row, nrows - 1) * (uint32_t)H * 4u;
        // batches of 4: LDS reads first, then the stores
        for (int it0 = 0; it0 < st_it; it0 += 4) {
          float v[4];
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            v[qq] = b[pad_dword((uint32_t)min(lane + kWave * (it0 + qq), L - 1))];
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const int i = lane + kWave * (it0 + qq);
            const uint32_t off = (ok && i < L) ? (uint32_t)(g.hs + i) * 4u : kOOB;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[qq]), ry, off, rowoff, kStream);
          }
        }
      }
      wave_lds_sync();
    }
  }
}

__global__ __launch_bounds__(256) void decompress_general_kernel(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ outl, int64_t P, int64_t T,
    int64_t H, int64_t k, int64_t Hq, int64_t Bq, const float* __restrict__ dec,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cmap, float* __restrict__ y) {
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
        const float d = __fsub_rn((float)q, dec[(P + p) * Hq + j]);   // exact
        acc = __fadd_rn(acc, __fmul_rn(d, dec[p * Hq + j]));
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
                        int buf_dwords, const float* dec, const int32_t* idx,
                        const int32_t* cmap, float* y, hipStream_t s) {
  const int64_t ngroups = (nrowblk + kDqWaves - 1) / kDqWaves;
  const size_t lds = (size_t)kDqWaves * kDqSub * buf_dwords * 4;
  decompress_kernel<NP><<<(unsigned)xcd_grid(ntiles, ngroups), 256, lds, s>>>(
      packed, outl, T, (int)H, (int)Hq, (int)k, ntiles, rpw, nrowblk, buf_dwords, dec, idx, cmap,
      y);
}

hipError_t launch_decompress(const uint8_t* packed, const uint16_t* outl, int64_t P, int64_t T,
                             int64_t H, int64_t k, const float* dec, const int32_t* idx,
                             const int32_t* cmap, float* y, hipStream_t s) {
  const int64_t Hq = H - k;
  const int64_t Bq = (Hq + 1) / 2;
  const int64_t span = (H < kTileSlots + k ? H : kTileSlots + k);
  const int buf_dwords = (int)((span + span / 8 + 8 + 3) / 4 * 4);
  const size_t lds = (size_t)kDqWaves * kDqSub * buf_dwords * 4;
  // Buffer resources: the whole message, the decoder table and one wave's
  // rows of y must each span fewer than 2^31 bytes.
  const int64_t lim = int64_t(1) << 31;
  const bool fast = Hq > 0 && P <= 8 && Hq % 8 == 0 && (uintptr_t)packed % 4 == 0 &&
                    (uintptr_t)dec % 16 == 0 && lds <= 65536 && P * T * Bq < lim &&
                    P * T * k * 2 < lim && (2 * P + 1) * Hq * 4 < lim && 64 * H * 4 < lim;
  if (fast) {
    const int ntiles = (int)((Hq + kTileSlots - 1) / kTileSlots);
    // about 2048 waves (8 per CU), a multiple of the ring depth, 8..64 rows
    int64_t rpw64 = (ntiles * T + 2047) / 2048;
    rpw64 = (rpw64 + kDqRing - 1) / kDqRing * kDqRing;
    if (rpw64 < kDqRing) rpw64 = kDqRing;
    if (rpw64 > 64) rpw64 = 64;
    const int rpw = (int)rpw64;
    const int64_t nrowblk = (T + rpw - 1) / rpw;
    switch (P) {
#define BTQ_DQ_CASE(n)                                                                         \
  case n:                                                                                      \
    launch_fast<n>(packed, outl, T, H, k, Hq, ntiles, rpw, nrowblk, buf_dwords, dec, idx, cmap, \
                   y, s);                                                                      \
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
  decompress_general_kernel<<<(unsigned)blocks, 256, 0, s>>>(packed, outl, P, T, H, k, Hq, Bq, dec,
                                                             idx, cmap, y);
  return hipGetLastError();
}

}  // namespace btq
